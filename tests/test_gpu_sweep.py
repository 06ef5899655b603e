"""Seeded random sweep over the plan space, each case against the oracle at the parity bars:
batch and head counts, ragged lengths, dtype and d, explicit chunk lengths (which also decide
the sub-chunk split of the chunk summaries), incoming states, checkpoints; and the backward
pass over the same kind of shapes.  Sizes stay small enough for the oracle."""
import numpy as np
import pytest

import long_context_la_amd as la
import oracle
from common import assert_close, inputs, to_device, to_host

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    return torch


def _case(i):
    rng = np.random.default_rng(1000 + i)
    dtype, d = [("bf16", 128), ("f32", 128), ("f32", 64), ("bf16", 64)][rng.integers(4)]
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    N = int(rng.integers(1, 2600))
    chunk = int(rng.choice([0, 64, 128, 256, 512, 1024, 1088]))
    slopes = np.exp2(-rng.uniform(1, 9, H)).astype(np.float32)
    kv_in = rng.standard_normal((B, H, d, d)).astype(np.float32) if rng.random() < 0.5 else None
    ckpt = 64 * int(rng.integers(1, 8)) if (rng.random() < 0.4 and N >= 64) else 0
    return dtype, d, B, H, N, chunk, slopes, kv_in, ckpt


@pytest.mark.parametrize("i", range(16))
def test_prefill_sweep(device, i):
    torch = _torch()
    dtype, d, B, H, N, chunk, slopes, kv_in, ckpt = _case(i)
    exact, raw = inputs(2000 + i, B, H, N, d, dtype)
    q, k, v = (to_device(x, dtype, device) for x in raw)
    kv = (torch.zeros(B, H, d, d, device=device) if kv_in is None else torch.from_numpy(kv_in).to(device))
    o = torch.empty_like(q)
    ck = torch.empty(B, H, N // ckpt, d, d, device=device) if ckpt else None
    la.la_prefill(q, k, v, torch.from_numpy(slopes).to(device), kv, o=o, ckpt=ck, ckpt_every=ckpt, chunk_tokens=chunk)
    torch.cuda.synchronize()
    o_ref, kv_ref, ck_ref = oracle.recurrent(*exact, slopes, kv_in=kv_in, ckpt_every=ckpt)
    what = f"case {i}: {dtype} d={d} B={B} H={H} N={N} chunk={chunk} state={kv_in is not None} ckpt={ckpt}"
    assert_close(to_host(o), o_ref, dtype, "O " + what, stored=dtype)
    assert_close(kv.cpu().numpy(), kv_ref, dtype, "KV " + what)
    if ckpt and N // ckpt:
        got = ck.cpu().numpy().reshape(-1, *ck.shape[2:])[:, None]
        assert_close(got, ck_ref.reshape(-1, *ck_ref.shape[2:])[:, None], dtype, "checkpoints " + what)


@pytest.mark.parametrize("i", range(8))
def test_backward_sweep(device, i):
    torch = _torch()
    dtype, d, B, H, N, _, slopes, kv_in, _ = _case(100 + i)
    exact, raw = inputs(3000 + i, B, H, N, d, dtype)
    rng = np.random.default_rng(4000 + i)
    g = rng.standard_normal((B, H, N, d)).astype(np.float32)
    if dtype == "bf16":
        import synth
        g = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(g))
        graw = synth.f32_to_bf16_bits(g)
    else:
        graw = g
    dkv_out = rng.standard_normal((B, H, d, d)).astype(np.float32) if rng.random() < 0.5 else None
    q, k, v, do = (to_device(x, dtype, device) for x in (*raw, graw))
    dq, dk, dv, dkv = la.la_backward(q, k, v, do, torch.from_numpy(slopes).to(device),
                                     kv_in=None if kv_in is None else torch.from_numpy(kv_in).to(device),
                                     dkv_out=None if dkv_out is None else torch.from_numpy(dkv_out).to(device))
    torch.cuda.synchronize()
    want = oracle.backward_recurrent(*exact, g, slopes, kv_in=kv_in, dkv_out=dkv_out)
    what = f"case {i}: {dtype} d={d} B={B} H={H} N={N}"
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want[:3]):
        assert_close(to_host(got), ref, dtype, f"{name} {what}", stored=dtype)
    assert_close(dkv.cpu().numpy(), want[3], dtype, "dKV_in " + what)
