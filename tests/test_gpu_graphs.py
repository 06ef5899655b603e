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


def test_backward_and_fused_prefill_in_a_graph(device):
    # la_backward (three prefill passes and the state preparations) and a fused prefill with the
    # norm pass, captured together and replayed three times against the eager results
    torch = _torch()
    B, H, N, d = 1, 8, 3000, 128
    raw = [synth.generate(t, 53, d, nb=B, nh=H, nt=N, dtype="bf16") for t in (synth.Q, synth.K, synth.V, synth.V)]
    q, k, v, do = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device) for x in raw)
    slopes = torch.from_numpy(synth.WORKLOADS["share"].slopes().copy()).to(device)
    kv_in = torch.randn(B, H, d, d, device=device)
    dkv_out = torch.randn(B, H, d, d, device=device)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dkv_in = torch.empty(B, H, d, d, device=device)
    ws_b = torch.empty(la.la_backward_workspace_size(la.LA_BF16, B, H, N, d), dtype=torch.uint8, device=device)
    kv = torch.empty(B, H, d, d, device=device)
    o = torch.empty_like(q)
    gate = torch.randn(B, H, N, d, device=device).to(torch.bfloat16)
    ws_f = torch.empty(max(la.la_prefill_workspace_size(la.LA_BF16, B, H, N, d), 1), dtype=torch.uint8,
                       device=device)

    def run():
        s = torch.cuda.current_stream()
        la.la_backward(q, k, v, do, slopes, kv_in=kv_in, dkv_out=dkv_out, dq=dq, dk=dk, dv=dv, dkv_in=dkv_in,
                       workspace=ws_b, stream=s)
        la.la_state_init(kv, kv_in, stream=s)
        la.la_prefill_fused(q, k, v, slopes, kv, o, silu_q=True, silu_k=True, norm_eps=1e-5, gate=gate,
                            workspace=ws_f, stream=s)

    assert la.la_prefill_chunk_tokens(la.LA_BF16, B, H, N, d) < N  # chunked: summaries and scans too
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dq, dk, dv, dkv_in, o, kv)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for t in (dq, dk, dv, o):
            t.zero_()
        dkv_in.fill_(3.0)
        kv.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("dq", "dk", "dv", "dkv_in", "o", "kv"), (dq, dk, dv, dkv_in, o, kv), ref):
            assert torch.equal(t, r), f"replay {rep}: {name} differs from eager"
        torch.matmul(ref[3][0, 0], ref[3][0, 1]).sum().item()
