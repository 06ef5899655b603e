"""HIP graph capture of the decode step and of the fixed-length prefill (both launch kernels
only: no allocation, memset or host copy inside the calls).  Each captured graph is replayed
several times, with eager work and synchronisations between the replays, and every replay is
compared with the same calls run eagerly from the same starting state.  Replays must match the
eager results bit for bit (same kernels, same inputs)."""
import numpy as np
import pytest

import long_context_la_amd as la
import synth

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    return torch


def _tokens(seed, steps, B, H, d, device):
    torch = _torch()
    out = []
    for t in (synth.Q, synth.K, synth.V):
        bits = synth.generate(t, seed, d, nb=B, nh=H, nt=steps, dtype="bf16")  # [B, H, steps, d]
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
        out.append(x.permute(2, 0, 1, 3).contiguous())  # [steps, B, H, d]
    return out


def test_decode_steps_in_a_graph(device):
    torch = _torch()
    B, H, d, steps = 2, 64, 128, 8
    slopes = torch.from_numpy(synth.WORKLOADS["decode"].slopes()[:H].copy()).to(device)
    q, k, v = _tokens(51, steps, B, H, d, device)
    kv0 = torch.randn(B, H, d, d, device=device)
    o = torch.empty(steps, B, H, d, dtype=torch.bfloat16, device=device)
    kv = kv0.clone()

    def run():
        for s in range(steps):
            la.la_decode(q[s], k[s], v[s], slopes, kv, o[s], stream=torch.cuda.current_stream())

    # eager reference
    run()
    torch.cuda.synchronize()
    o_ref, kv_ref = o.clone(), kv.clone()
    # capture (on a side stream, as torch requires), then replay from the same starting state
    kv.copy_(kv0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        kv.copy_(kv0)
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: outputs differ from eager"
        assert torch.equal(kv, kv_ref), f"replay {rep}: states differ from eager"
        # eager work between replays
        torch.matmul(kv0[0, 0], kv0[0, 1]).sum().item()


def test_prefill_in_a_graph(device):
    torch = _torch()
    B, H, N, d = 1, 64, 1000, 128
    raw = [synth.generate(t, 52, d, nb=B, nh=H, nt=N, dtype="bf16") for t in (synth.Q, synth.K, synth.V)]
    q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device) for x in raw)
    slopes = torch.from_numpy(synth.WORKLOADS["full"].slopes().copy()).to(device)
    kv = torch.empty(B, H, d, d, device=device)
    o = torch.empty_like(q)
    ws = torch.empty(max(la.la_prefill_workspace_size(la.LA_BF16, B, H, N, d), 1), dtype=torch.uint8, device=device)

    def run():
        s = torch.cuda.current_stream()
        la.la_state_init(kv, stream=s)
        la.la_prefill(q, k, v, slopes, kv, o=o, workspace=ws, stream=s)

    run()
    torch.cuda.synchronize()
    o_ref, kv_ref = o.clone(), kv.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        o.zero_()
        kv.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: outputs differ from eager"
        assert torch.equal(kv, kv_ref), f"replay {rep}: states differ from eager"
        torch.matmul(kv_ref[0, 0], kv_ref[0, 1]).sum().item()
