"""GPU parity of la_backward (gradients through the prefill) against the oracle's reverse state
recurrence (oracle.backward_recurrent, float64), element by element per (batch, head) with the
bars of test_gpu_parity.py: dq, dk, dv stored in the input dtype (half an ulp of it allowed),
dL/dKV_in in float32."""
import numpy as np
import pytest

import long_context_la_amd as la
import oracle
import synth
from common import assert_close, inputs, to_device, to_host

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    return torch


def run_backward(B, H, N, d, dtype, device, states=True, seed=71, slopes=None, layout="bhnd", grad_scale=1.0,
                 state_scale=None, zero_grad=False):
    """grad_scale (a power of two, so the scaling is exact) multiplies dL/dO, and state_scale
    (grad_scale if None) dL/dKV_final; zero_grad makes dL/dO all zero."""
    torch = _torch()
    exact, raw = inputs(seed, B, H, N, d, dtype)
    dout_raw = synth.generate(synth.V, seed + 500, d, nb=B, nh=H, nt=N, dtype=dtype)
    dout_exact = synth.bf16_bits_to_f32(dout_raw) if dtype == "bf16" else dout_raw
    if zero_grad:
        grad_scale = 0.0
    if grad_scale != 1.0:
        dout_exact = (dout_exact * np.float32(grad_scale)).astype(np.float32)
        dout_raw = synth.f32_to_bf16_bits(dout_exact) if dtype == "bf16" else dout_exact
        if dtype == "bf16":
            assert np.array_equal(synth.bf16_bits_to_f32(dout_raw), dout_exact)
    if slopes is None:
        slopes = np.array([2.0 ** (-2 - 3 * h) for h in range(H)], dtype=np.float32)
    rng = np.random.default_rng(seed + 1)
    kv_in = rng.standard_normal((B, H, d, d)).astype(np.float32) if states else None
    dkv_out = (rng.standard_normal((B, H, d, d)) * (grad_scale if state_scale is None else state_scale)
               ).astype(np.float32) if states else None

    def dev(x):
        t = to_device(x, dtype, device)
        if layout == "bnhd":  # [B,N,H,d] storage viewed as [B,H,N,d]
            t = t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        return t

    q, k, v, do = (dev(x) for x in (*raw, dout_raw))
    dq, dk, dv, dkv = la.la_backward(
        q, k, v, do, torch.from_numpy(slopes).to(device),
        kv_in=None if kv_in is None else torch.from_numpy(kv_in).to(device),
        dkv_out=None if dkv_out is None else torch.from_numpy(dkv_out).to(device))
    torch.cuda.synchronize()
    want = oracle.backward_recurrent(*exact, dout_exact, slopes, kv_in=kv_in, dkv_out=dkv_out)
    what = f"(B={B}, H={H}, N={N}, d={d}, {dtype}, states={states}, {layout})"
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want[:3]):
        assert_close(to_host(got), ref, dtype, f"{name} {what}", stored=dtype)
    assert_close(dkv.cpu().numpy(), want[3], dtype, f"dkv_in {what}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 128), ("f32", 64), ("bf16", 64)])
@pytest.mark.parametrize("states", [False, True])
def test_backward_small(device, dtype, d, states):
    run_backward(1, 2, 200, d, dtype, device, states=states)


@pytest.mark.parametrize("grad_log2", [-24, -40])
@pytest.mark.parametrize("N,d", [(300, 128), (5000, 128), (700, 64)])
def test_backward_tiny_gradients_bf16(device, grad_log2, N, d):
    # gradients of a mean loss over a large tensor sit far below float16's normal range (2^-14):
    # every backward pass runs on full-range (bf16 hi + lo) operands and keeps the bf16 bar
    run_backward(1, 2, N, d, "bf16", device, states=True, seed=95, grad_scale=2.0 ** grad_log2)


@pytest.mark.parametrize("grad_log2,state_log2", [(-30, 0), (0, -30), (-40, -26)])
def test_backward_gradient_and_state_far_apart_bf16(device, grad_log2, state_log2):
    # dL/dO and dL/dKV_final at scales 2^30 apart either way: the full-range operands keep both
    run_backward(1, 2, 700, 128, "bf16", device, states=True, seed=98, grad_scale=2.0 ** grad_log2,
                 state_scale=2.0 ** state_log2)


@pytest.mark.parametrize("states", [False, True])
def test_backward_zero_gradient_bf16(device, states):
    # an all-zero dL/dO, with and without a dL/dKV_final
    run_backward(1, 2, 300, 128, "bf16", device, states=states, seed=99, zero_grad=True,
                 state_scale=1.0 if states else None)


def test_backward_tiny_gradients_strided_layout_bf16(device):
    # tiny gradients in a [B, N, H, d] layout
    run_backward(2, 2, 200, 128, "bf16", device, states=True, seed=100, layout="bnhd", grad_scale=2.0 ** -30)


@pytest.mark.parametrize("n", [1, 63, 64, 65, 129])
def test_backward_tile_edges_bf16(device, n):
    run_backward(2, 2, n, 128, "bf16", device, states=True, seed=80 + n)


def test_backward_chunked_bf16(device):
    # 2 heads x 4 value slices do not fill the GPU: every pass is cut into chunks, the two reverse
    # walks combine their chunk summaries in reverse order
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, 2, 5000, 128) < 5000
    run_backward(1, 2, 5000, 128, "bf16", device, states=True, seed=90)


def test_backward_chunked_f32(device):
    run_backward(1, 1, 3000, 64, "f32", device, states=True, seed=91)


def test_backward_chunked_bf16_d64(device):
    # bfloat16 at d = 64 (two value slices per head), chunked like the others
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, 2, 3000, 64) < 3000
    run_backward(1, 2, 3000, 64, "bf16", device, states=True, seed=94)


def test_backward_strided_layout(device):
    run_backward(2, 3, 150, 128, "bf16", device, states=True, seed=92, layout="bnhd")


def test_backward_slow_and_fast_decay(device):
    slopes = np.array([2.0 ** -8, 0.9], dtype=np.float32)
    run_backward(1, 2, 700, 128, "bf16", device, states=True, seed=93, slopes=slopes)


def test_backward_empty_sequence(device):
    torch = _torch()
    B, H, d = 1, 2, 128
    q = torch.zeros(B, H, 0, d, dtype=torch.bfloat16, device=device)
    g = torch.randn(B, H, d, d, device=device)
    dq, dk, dv, dkv = la.la_backward(q, q, q, q, torch.full((H,), 0.1, device=device), dkv_out=g)
    torch.cuda.synchronize()
    assert dq.shape == q.shape and torch.equal(dkv, g)


def test_backward_chunked_batch(device):
    # batch of two, chunked: the reverse walks' summaries run per (sequence, head, sub-chunk)
    run_backward(2, 2, 3000, 128, "bf16", device, states=True, seed=94)


def test_backward_is_deterministic(device):
    torch = _torch()
    exact, raw = inputs(95, 1, 2, 2000, 128, "bf16")
    q, k, v = (to_device(x, "bf16", device) for x in raw)
    do = torch.randn_like(q.float()).to(torch.bfloat16)
    slopes = torch.tensor([0.25, 0.01], device=device)
    g = torch.randn(1, 2, 128, 128, device=device)
    a = la.la_backward(q, k, v, do, slopes, dkv_out=g)
    b = la.la_backward(q, k, v, do, slopes, dkv_out=g)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_backward_varlen_packed(device, dtype, d):
    """la_backward_varlen on packed sequences of mixed lengths: empty, short (token by token),
    tiled, and long enough to be cut into chunks, each with its own states; every sequence is
    checked against the oracle on its own tokens."""
    lengths = [300, 0, 5, 1, 2000, 64, 9, 4100]
    cu = [0] + list(np.cumsum(lengths))
    assert la.la_prefill_varlen_chunk_tokens(la.LA_BF16 if dtype == "bf16" else la.LA_F32, cu, 2, d) < 4100
    run_backward_varlen(lengths, 2, d, dtype, device, np.array([2.0 ** -2, 2.0 ** -7], np.float32), seed=96)


def test_backward_varlen_tiny_gradients_bf16(device):
    # packed sequences (token by token, tiled, chunked) with gradients of order 2^-30
    run_backward_varlen([300, 5, 4100], 2, 128, "bf16", device, np.array([2.0 ** -2, 2.0 ** -7], np.float32),
                        seed=97, grad_scale=2.0 ** -30)


@pytest.mark.parametrize("i", range(6))
def test_backward_varlen_sweep(device, i):
    # seeded random packed batches through the backward: lengths (empty, token by token, tiled,
    # chunked), heads, dtype and d, slopes, with or without states
    rng = np.random.default_rng(9000 + i)
    dtype, d = [("bf16", 128), ("f32", 128), ("f32", 64), ("bf16", 64)][rng.integers(4)]
    n_seq = int(rng.integers(1, 7))
    lengths = [int([0, rng.integers(1, 9), rng.integers(9, 300), rng.integers(300, 3000)][k])
               for k in rng.integers(0, 4, n_seq)]
    if sum(lengths) == 0:
        lengths[0] = 1
    H = int(rng.integers(1, 4))
    slopes = np.exp2(-rng.uniform(1, 9, H)).astype(np.float32)
    run_backward_varlen(lengths, H, d, dtype, device, slopes, seed=9100 + 10 * i, states=bool(rng.random() < 0.6))


def run_backward_varlen(lengths, H, d, dtype, device, slopes, seed, states=True, grad_scale=1.0):
    """la_backward_varlen on one packed batch; every sequence against the oracle on its own tokens
    (an empty sequence passes dL/dKV_final through unchanged).  grad_scale (a power of two)
    multiplies dL/dO and dL/dKV_final."""
    torch = _torch()

    cu = [0] + list(np.cumsum(lengths))
    T = cu[-1]
    exact, raw = inputs(seed, 1, H, T, d, dtype)
    graw = synth.generate(synth.V, seed + 1, d, nh=H, nt=T, dtype=dtype)
    gex = synth.bf16_bits_to_f32(graw) if dtype == "bf16" else graw
    if grad_scale != 1.0:
        gex = (gex * np.float32(grad_scale)).astype(np.float32)
        graw = synth.f32_to_bf16_bits(gex) if dtype == "bf16" else gex
    rng = np.random.default_rng(seed + 2)
    kv_in = rng.standard_normal((len(lengths), H, d, d)).astype(np.float32) if states else None
    dkv_out = ((rng.standard_normal((len(lengths), H, d, d)) * grad_scale).astype(np.float32)
               if states else None)

    def packed(x):  # [1, H, T, d] -> device [T, H, d]
        return to_device(np.ascontiguousarray(x[0].transpose(1, 0, 2)), dtype, device)

    def dev_or_none(x):
        return None if x is None else torch.from_numpy(x).to(device)

    q, k, v, do = (packed(x) for x in (*raw, graw))
    dq, dk, dv, dkv = la.la_backward_varlen(q, k, v, do, torch.from_numpy(slopes).to(device), cu,
                                            kv_in=dev_or_none(kv_in), dkv_out=dev_or_none(dkv_out))
    torch.cuda.synchronize()
    got = [to_host(t).transpose(1, 0, 2)[None] for t in (dq, dk, dv)]  # [1, H, T, d]
    dkv_h = dkv.cpu().numpy()
    for s, n in enumerate(lengths):
        a, b = cu[s], cu[s + 1]
        if n == 0:
            passed = dkv_out[s] if states else np.zeros((H, d, d), np.float32)
            np.testing.assert_allclose(dkv_h[s], passed, rtol=1e-6, atol=1e-6)
            continue
        want = oracle.backward_recurrent(*(x[:, :, a:b] for x in exact), gex[:, :, a:b], slopes,
                                         kv_in=kv_in[s:s + 1] if states else None,
                                         dkv_out=dkv_out[s:s + 1] if states else None)
        what = f"sequence {s} ({n} tokens, {dtype}, d={d}, H={H}, states={states})"
        for name, g_, r in zip(("dq", "dk", "dv"), got, want[:3]):
            assert_close(g_[:, :, a:b], r, dtype, f"{name} {what}", stored=dtype)
        assert_close(dkv_h[s:s + 1], want[3], dtype, f"dKV_in {what}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_autograd_function(device, dtype, d):
    # lightning_attention under torch autograd: a loss on both outputs, gradients for q, k, v and
    # the incoming state, against the oracle's reverse recurrence
    torch = _torch()
    B, H, N = 1, 2, 300
    exact, raw = inputs(120, B, H, N, d, dtype)
    q, k, v = (to_device(x, dtype, device).requires_grad_(True) for x in raw)
    slopes = np.array([2.0 ** -2, 2.0 ** -6], np.float32)
    rng = np.random.default_rng(121)
    kv0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    g_o = rng.standard_normal((B, H, N, d)).astype(np.float32)
    g_kv = rng.standard_normal((B, H, d, d)).astype(np.float32)
    if dtype == "bf16":
        g_o = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(g_o))
    kv_in = torch.from_numpy(kv0).to(device).requires_grad_(True)
    o, kv_out = la.lightning_attention(q, k, v, torch.from_numpy(slopes).to(device), kv_in)
    loss = (o.float() * torch.from_numpy(g_o).to(device)).sum() + (kv_out * torch.from_numpy(g_kv).to(device)).sum()
    loss.backward()
    torch.cuda.synchronize()
    want = oracle.backward_recurrent(*exact, g_o, slopes, kv_in=kv0, dkv_out=g_kv)
    for name, t, r in zip(("dq", "dk", "dv"), (q, k, v), want[:3]):
        assert_close(to_host(t.grad), r, dtype, f"autograd {name} ({dtype}, d={d})", stored=dtype)
    assert_close(kv_in.grad.cpu().numpy(), want[3], dtype, f"autograd dKV_in ({dtype}, d={d})")


def test_autograd_function_varlen(device):
    # lightning_attention_varlen under autograd on a packed batch (empty, short, tiled, chunked)
    torch = _torch()
    lengths, H, d, dtype = [200, 0, 3, 2500], 2, 128, "bf16"
    cu = [0] + [int(x) for x in np.cumsum(lengths)]
    T = cu[-1]
    exact, raw = inputs(130, 1, H, T, d, dtype)
    rng = np.random.default_rng(131)
    kv0 = rng.standard_normal((len(lengths), H, d, d)).astype(np.float32)
    g_kv = rng.standard_normal((len(lengths), H, d, d)).astype(np.float32)
    g_o = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((T, H, d)).astype(np.float32)))
    slopes = np.array([2.0 ** -3, 2.0 ** -7], np.float32)
    q, k, v = (to_device(np.ascontiguousarray(x[0].transpose(1, 0, 2)), dtype, device).requires_grad_(True)
               for x in raw)
    kv_in = torch.from_numpy(kv0).to(device).requires_grad_(True)
    o, kv_out = la.lightning_attention_varlen(q, k, v, torch.from_numpy(slopes).to(device), cu, kv_in)
    loss = (o.float() * torch.from_numpy(g_o).to(device)).sum() + (kv_out * torch.from_numpy(g_kv).to(device)).sum()
    loss.backward()
    torch.cuda.synchronize()
    grads = [to_host(t.grad) for t in (q, k, v)]
    dkv = kv_in.grad.cpu().numpy()
    for s, n in enumerate(lengths):
        a, b = cu[s], cu[s + 1]
        if n == 0:
            np.testing.assert_allclose(dkv[s], g_kv[s], rtol=1e-6, atol=1e-6)
            continue
        go = np.ascontiguousarray(g_o[a:b].transpose(1, 0, 2))[None]
        want = oracle.backward_recurrent(*(x[:, :, a:b] for x in exact), go, slopes, kv_in=kv0[s:s + 1],
                                         dkv_out=g_kv[s:s + 1])
        for name, g_, r in zip(("dq", "dk", "dv"), grads, want[:3]):
            assert_close(np.ascontiguousarray(g_[a:b].transpose(1, 0, 2))[None], r, dtype,
                         f"autograd varlen {name} sequence {s}", stored=dtype)
        assert_close(dkv[s:s + 1], want[3], dtype, f"autograd varlen dKV_in sequence {s}")


def test_backward_in_place_state_gradient(device):
    # dkv_in may alias dkv_out: the gradient of the incoming state overwrites dL/dKV_final
    torch = _torch()
    B, H, N, d, dtype = 1, 2, 500, 128, "bf16"
    exact, raw = inputs(140, B, H, N, d, dtype)
    q, k, v = (to_device(x, dtype, device) for x in raw)
    rng = np.random.default_rng(141)
    g_o = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((B, H, N, d)).astype(np.float32)))
    kv0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    g_kv = rng.standard_normal((B, H, d, d)).astype(np.float32)
    do = to_device(synth.f32_to_bf16_bits(g_o), dtype, device)
    slopes = np.array([2.0 ** -3, 2.0 ** -8], np.float32)
    buf = torch.from_numpy(g_kv.copy()).to(device)
    _, _, _, out = la.la_backward(q, k, v, do, torch.from_numpy(slopes).to(device),
                                  kv_in=torch.from_numpy(kv0).to(device), dkv_out=buf, dkv_in=buf)
    torch.cuda.synchronize()
    assert out.data_ptr() == buf.data_ptr()
    want = oracle.backward_recurrent(*exact, g_o, slopes, kv_in=kv0, dkv_out=g_kv)
    assert_close(buf.cpu().numpy(), want[3], dtype, "in-place dKV_in")


def test_backward_state_gradient_over_incoming_state(device):
    # dkv_in may alias kv_in: the incoming state is read before its gradient overwrites it
    torch = _torch()
    B, H, N, d, dtype = 1, 2, 400, 64, "f32"
    exact, raw = inputs(150, B, H, N, d, dtype)
    q, k, v = (to_device(x, dtype, device) for x in raw)
    rng = np.random.default_rng(151)
    g_o = rng.standard_normal((B, H, N, d)).astype(np.float32)
    kv0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    g_kv = rng.standard_normal((B, H, d, d)).astype(np.float32)
    slopes = np.array([2.0 ** -2, 2.0 ** -6], np.float32)
    buf = torch.from_numpy(kv0.copy()).to(device)
    dq, dk, dv, _ = la.la_backward(q, k, v, torch.from_numpy(g_o).to(device), torch.from_numpy(slopes).to(device),
                                   kv_in=buf, dkv_out=torch.from_numpy(g_kv).to(device), dkv_in=buf)
    torch.cuda.synchronize()
    want = oracle.backward_recurrent(*exact, g_o, slopes, kv_in=kv0, dkv_out=g_kv)
    for name, t, r in zip(("dq", "dk", "dv"), (dq, dk, dv), want[:3]):
        assert_close(to_host(t), r, dtype, f"{name} with dkv_in over kv_in", stored=dtype)
    assert_close(buf.cpu().numpy(), want[3], dtype, "dKV_in over kv_in")


def test_backward_maximum_row_stride(device):
    # stride_n at the documented maximum of 2^22 elements through the three runs (two of them
    # walking the tiles backwards, whose rows past a ragged tail wrap above the tile's range)
    torch = _torch()
    B, H, N, d, S, dtype, seed = 1, 2, 130, 128, 1 << 22, "bf16", 97
    exact, raw = inputs(seed, B, H, N, d, dtype)
    dout_raw = synth.generate(synth.V, seed + 500, d, nb=B, nh=H, nt=N, dtype=dtype)
    slopes = np.array([2.0 ** -3, 2.0 ** -7], dtype=np.float32)
    rng = np.random.default_rng(seed + 1)
    kv_in = rng.standard_normal((B, H, d, d)).astype(np.float32)
    dkv_out = rng.standard_normal((B, H, d, d)).astype(np.float32)
    fulls = []

    def strided(t):
        full = torch.zeros((N, S), dtype=t.dtype, device=device)
        view = full[:, :H * d].view(N, H, d).permute(1, 0, 2).unsqueeze(0)
        view.copy_(t)
        fulls.append(full)
        return view

    q, k, v, do = (strided(to_device(x, dtype, device)) for x in (*raw, dout_raw))
    dq, dk, dv = (strided(torch.zeros_like(to_device(raw[0], dtype, device))) for _ in range(3))
    assert q.stride()[1:] == dq.stride()[1:] == (d, S, 1)
    _, _, _, dkv = la.la_backward(q, k, v, do, torch.from_numpy(slopes).to(device),
                                  kv_in=torch.from_numpy(kv_in).to(device),
                                  dkv_out=torch.from_numpy(dkv_out).to(device), dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    want = oracle.backward_recurrent(*exact, synth.bf16_bits_to_f32(dout_raw), slopes, kv_in=kv_in, dkv_out=dkv_out)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), want[:3]):
        assert_close(to_host(got), ref, dtype, f"{name} at stride_n 2^22", stored=dtype)
    assert_close(dkv.cpu().numpy(), want[3], dtype, "dkv_in at stride_n 2^22")
    for full in fulls[4:]:
        assert float(full[:, H * d:].abs().max()) == 0.0  # nothing written outside the heads' features
