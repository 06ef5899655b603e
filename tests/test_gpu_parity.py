"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on seeded inputs.

Bars (per (batch, head) slice, outputs and final states alike): the error beyond half an ulp
of the result's storage format is <= 1e-4 * RMS for float32 inputs and <= 2e-2 * RMS for
bfloat16 inputs with float32 accumulation (tests/common.py states the measure).
Cases cover several tiles with ragged tails, chunked (LASP+-style) runs, no decay, slow
decay, incoming states and continuation, strided views, impulses, checkpoints, the
state-only mode, determinism, and decode steps.
"""
import numpy as np
import pytest

import long_context_la_amd as la
import oracle
from common import TOL, assert_close, inputs, to_device, to_host

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    return torch


def run_prefill(raw, slopes, dtype, device, kv_in=None, chunk_tokens=0, ckpt_every=0, want_o=True):
    torch = _torch()
    q, k, v = (to_device(x, dtype, device) for x in raw)
    B, H, N, d = q.shape
    kv = (torch.zeros(B, H, d, d, dtype=torch.float32, device=device) if kv_in is None
          else torch.from_numpy(np.ascontiguousarray(kv_in, dtype=np.float32)).to(device))
    o = torch.empty_like(q) if want_o else None
    ck = (torch.full((B, H, N // ckpt_every, d, d), float("nan"), dtype=torch.float32, device=device)
          if ckpt_every else None)
    la.la_prefill(q, k, v, torch.from_numpy(np.asarray(slopes, dtype=np.float32)).to(device), kv, o=o,
                  ckpt=ck, ckpt_every=ckpt_every, chunk_tokens=chunk_tokens)
    torch.cuda.synchronize()
    return (to_host(o) if want_o else None), kv.cpu().numpy(), (ck.cpu().numpy() if ck is not None else None)


def check_prefill(seed, B, H, N, d, dtype, slopes, device, kv_in=None, chunk_tokens=0, ckpt_every=0):
    exact, raw = inputs(seed, B, H, N, d, dtype)
    o, kv, ck = run_prefill(raw, slopes, dtype, device, kv_in, chunk_tokens, ckpt_every)
    o_ref, kv_ref, ck_ref = oracle.recurrent(*exact, slopes, kv_in=kv_in, ckpt_every=ckpt_every)
    eo = assert_close(o, o_ref, dtype, f"O (N={N}, d={d}, {dtype}, chunk={chunk_tokens})", stored=dtype)
    ek = assert_close(kv, kv_ref, dtype, f"KV (N={N}, d={d}, {dtype}, chunk={chunk_tokens})")
    if ckpt_every:
        assert_close(ck.reshape(-1, *ck.shape[2:])[:, None], ck_ref.reshape(-1, *ck_ref.shape[2:])[:, None],
                     dtype, "checkpoints")
    return eo, ek


SL2 = np.array([2.0 ** -2, 2.0 ** -8], dtype=np.float32)


def test_tiny_workload_f32(device):
    import synth

    w = synth.WORKLOADS["tiny"]
    check_prefill(w.seed, w.batch, w.heads, w.n, w.d, "f32", w.slopes(), device)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 63, 65, 1000])
def test_f32_ragged(device, d, N):
    check_prefill(21, 1, 2, N, d, "f32", SL2, device)


@pytest.mark.parametrize("chunk", [64, 128, 320])
def test_f32_chunked(device, chunk):
    check_prefill(22, 2, 2, 1000, 64, "f32", SL2, device, chunk_tokens=chunk)


@pytest.mark.parametrize("N", [1, 255, 257, 1000, 4097])
def test_bf16_ragged(device, N):
    check_prefill(23, 1, 2, N, 128, "bf16", SL2, device)


@pytest.mark.parametrize("N", [1, 63, 65, 1000])
def test_bf16_d64_ragged(device, N):
    # bfloat16 at d = 64: the MFMA tile kernel instantiated for the head dimension 64
    check_prefill(35, 2, 3, N, 64, "bf16", np.array([0.5, 2.0 ** -3, 2.0 ** -7], np.float32), device)


@pytest.mark.parametrize("chunk", [64, 1024, 0])
def test_bf16_chunked(device, chunk):
    check_prefill(24, 1, 2, 8192, 128, "bf16", np.array([2.0 ** -4, 2.0 ** -10], np.float32), device,
                  chunk_tokens=chunk)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_decay_cumulative(device, dtype):
    check_prefill(25, 1, 2, 4096, 128, dtype, np.zeros(2, np.float32), device, chunk_tokens=1024)


def test_slow_decay_long_sequence(device):
    check_prefill(26, 1, 1, 32768, 128, "bf16", np.array([2.0 ** -12], np.float32), device)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_incoming_state_and_continuation(device, dtype):
    torch = _torch()
    B, H, N1, N2, d = 1, 2, 700, 1300, 128
    rng = np.random.default_rng(5)
    kv0 = rng.standard_normal((B, H, d, d)) * 10.0
    exact, raw = inputs(27, B, H, N1 + N2, d, dtype)
    o_ref, kv_ref, _ = oracle.recurrent(*exact, SL2, kv_in=kv0.astype(np.float32).astype(np.float64))
    first = [x[:, :, :N1] for x in raw]
    second = [np.ascontiguousarray(x[:, :, N1:]) for x in raw]
    o1, kv1, _ = run_prefill(first, SL2, dtype, device, kv_in=kv0)
    o2, kv2, _ = run_prefill(second, SL2, dtype, device, kv_in=kv1, chunk_tokens=256)
    assert_close(np.concatenate([o1, o2], axis=2), o_ref, dtype, "continued O", stored=dtype)
    assert_close(kv2, kv_ref, dtype, "continued KV")
    # then decode steps from the prefill's state
    kvt = torch.from_numpy(kv2).to(device)
    state = kv_ref.copy()
    ts = torch.from_numpy(SL2).to(device)
    ex_d, raw_d = inputs(27, B, H, 5, d, dtype, t0=N1 + N2)
    for t in range(5):
        q, k, v = (to_device(np.ascontiguousarray(x[:, :, t]), dtype, device) for x in raw_d)
        o = torch.empty_like(q)
        la.la_decode(q, k, v, ts, kvt, o)
        od_ref = oracle.decode_step(*(x[:, :, t] for x in ex_d), SL2, state)
        torch.cuda.synchronize()
        assert_close(to_host(o)[:, :, None], od_ref[:, :, None], dtype, f"decode step {t}", stored=dtype)
    assert_close(kvt.cpu().numpy(), state, dtype, "decode KV")


def test_strided_views(device):
    torch = _torch()
    B, H, N, d = 2, 3, 777, 128
    exact, raw = inputs(28, B, H, N, d, "bf16")
    # store as [B, N, H, d] and hand the kernel [B, H, N, d] views
    dev = [to_device(np.ascontiguousarray(x.transpose(0, 2, 1, 3)), "bf16", device).permute(0, 2, 1, 3)
           for x in raw]
    q, k, v = dev
    assert q.stride() == (N * H * d, d, H * d, 1)
    o = torch.empty_like(q)
    assert o.stride() == q.stride()
    kv = torch.zeros(B, H, d, d, device=device)
    sl = np.array([0.5, 2.0 ** -3, 2.0 ** -7], np.float32)
    la.la_prefill(q, k, v, torch.from_numpy(sl).to(device), kv, o=o)
    torch.cuda.synchronize()
    o_ref, kv_ref, _ = oracle.recurrent(*exact, sl)
    assert_close(to_host(o), o_ref, "bf16", "strided O", stored="bf16")
    assert_close(kv.cpu().numpy(), kv_ref, "bf16", "strided KV")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_padded_row_strides(device, dtype, d):
    # rows of a wider buffer: storage [B, N, H, d + 24], the kernels see the first d features of
    # each (b, n, h) row, so stride_h = d + 24 and stride_n = H (d + 24); chunked and ragged
    torch = _torch()
    B, H, N, pad = 2, 3, 1500, 24
    exact, raw = inputs(39, B, H, N, d, dtype)

    def padded(x):
        full = np.zeros((B, N, H, d + pad), dtype=x.dtype)
        full[..., :d] = x.transpose(0, 2, 1, 3)
        return to_device(full, dtype, device)[..., :d].permute(0, 2, 1, 3)

    q, k, v = (padded(x) for x in raw)
    o_full = torch.zeros((B, N, H, d + pad), dtype=q.dtype, device=device)
    o = o_full[..., :d].permute(0, 2, 1, 3)
    assert q.stride() == o.stride() == (N * H * (d + pad), d + pad, H * (d + pad), 1)
    sl = np.array([0.5, 2.0 ** -4, 2.0 ** -9], np.float32)
    kv = torch.zeros(B, H, d, d, device=device)
    la.la_prefill(q, k, v, torch.from_numpy(sl).to(device), kv, o=o, chunk_tokens=512)
    torch.cuda.synchronize()
    o_ref, kv_ref, _ = oracle.recurrent(*exact, sl)
    assert_close(to_host(o), o_ref, dtype, f"padded O ({dtype}, d={d})", stored=dtype)
    assert_close(kv.cpu().numpy(), kv_ref, dtype, f"padded KV ({dtype}, d={d})")
    assert float(o_full[..., d:].abs().max()) == 0.0  # nothing written outside the d features


@pytest.mark.parametrize("dtype,chunk", [("bf16", 0), ("bf16", 64), ("f32", 0)])
def test_maximum_row_stride(device, dtype, chunk):
    # stride_n at the documented maximum of 2^22 elements: a 64-row tile then spans 512 MiB (bf16)
    # or 1 GiB (f32) of 32-bit buffer offsets; 2 heads side by side in each row, 3 tiles (ragged)
    torch = _torch()
    B, H, N, d, S = 1, 2, 130, 128, 1 << 22
    exact, raw = inputs(41, B, H, N, d, dtype)

    def strided(t):
        full = torch.zeros((N, S), dtype=t.dtype, device=device)
        view = full[:, :H * d].view(N, H, d).permute(1, 0, 2).unsqueeze(0)
        view.copy_(t)
        return full, view

    q, k, v = (strided(to_device(x, dtype, device))[1] for x in raw)
    o_full, o = strided(torch.zeros((B, H, N, d), dtype=q.dtype, device=device))
    assert q.stride()[1:] == o.stride()[1:] == (d, S, 1)
    sl = np.array([2.0 ** -3, 2.0 ** -7], np.float32)
    kv = torch.zeros(B, H, d, d, device=device)
    la.la_prefill(q, k, v, torch.from_numpy(sl).to(device), kv, o=o, chunk_tokens=chunk)
    torch.cuda.synchronize()
    o_ref, kv_ref, _ = oracle.recurrent(*exact, sl)
    assert_close(to_host(o), o_ref, dtype, f"O at stride_n 2^22 ({dtype}, chunk {chunk})", stored=dtype)
    assert_close(kv.cpu().numpy(), kv_ref, dtype, f"KV at stride_n 2^22 ({dtype}, chunk {chunk})")
    assert float(o_full[:, H * d:].abs().max()) == 0.0  # nothing written outside the heads' features


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_impulse(device, dtype):
    B, H, N, d, src = 1, 1, 300, 128, 100
    exact, raw = inputs(29, B, H, N, d, dtype)
    for x in raw[1:]:
        keep = x[:, :, src].copy()
        x[:] = 0
        x[:, :, src] = keep
    import synth

    exact = [synth.bf16_bits_to_f32(x) for x in raw] if dtype == "bf16" else raw
    sl = np.array([0.05], np.float32)
    o, kv, _ = run_prefill(raw, sl, dtype, device)
    o_ref, kv_ref, _ = oracle.recurrent(*exact, sl)
    assert np.all(o[0, 0, :src] == 0.0)  # nothing before the impulse
    assert_close(o, o_ref, dtype, "impulse O", stored=dtype)
    assert_close(kv, kv_ref, dtype, "impulse KV")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 64)])
def test_checkpoints(device, dtype, d):
    check_prefill(30, 1, 2, 1024, d, dtype, SL2, device, ckpt_every=256, chunk_tokens=320 if dtype == "f32" else 0)
    check_prefill(31, 1, 2, 2048, d, dtype, SL2, device, ckpt_every=512, chunk_tokens=1024)


@pytest.mark.parametrize("ckpt_every,chunk", [(64, 320), (192, 1088), (320, 0)])
@pytest.mark.parametrize("slopes", [(2.0 ** -2, 2.0 ** -8), (0.9, 0.3)])
def test_bf16_checkpoints_tile_parities(device, ckpt_every, chunk, slopes):
    # checkpoints after even and odd tiles of chunks that start on odd tiles, ragged last chunk;
    # slow decays (the state waves' paired scaling) and fast ones (per-tile scaling)
    check_prefill(37, 1, 2, 2000, 128, "bf16", np.array(slopes, np.float32), device, ckpt_every=ckpt_every,
                  chunk_tokens=chunk)


@pytest.mark.parametrize("N", [64, 128, 130, 192, 200])
@pytest.mark.parametrize("slopes", [(2.0 ** -2, 2.0 ** -8), (0.9, 0.3)])
def test_bf16_tile_count_parities(device, N, slopes):
    # one to four tiles: the final state after an even or an odd last tile, full or short
    kv0 = np.random.default_rng(N).standard_normal((1, 2, 128, 128)).astype(np.float32)
    check_prefill(38, 1, 2, N, 128, "bf16", np.array(slopes, np.float32), device, kv_in=kv0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_state_only(device, dtype):
    exact, raw = inputs(32, 1, 2, 3000, 128, dtype)
    _, kv, _ = run_prefill(raw, SL2, dtype, device, want_o=False, chunk_tokens=1024)
    _, kv_ref, _ = oracle.recurrent(*exact, SL2, want_o=False)
    assert_close(kv, kv_ref, dtype, "state-only KV")


def test_determinism(device):
    exact, raw = inputs(33, 1, 2, 5000, 128, "bf16")
    r1 = run_prefill(raw, SL2, "bf16", device, chunk_tokens=1024)
    r2 = run_prefill(raw, SL2, "bf16", device, chunk_tokens=1024)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])


def test_state_init(device):
    torch = _torch()
    kv = torch.full((2, 3, 64, 64), 7.0, device=device)
    la.la_state_init(kv)
    src = torch.randn(2, 3, 64, 64, device=device)
    torch.cuda.synchronize()
    assert float(kv.abs().max()) == 0.0
    la.la_state_init(kv, src)
    torch.cuda.synchronize()
    assert torch.equal(kv, src)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 128), ("bf16", 64)])
def test_decode_steps(device, dtype, d):
    torch = _torch()
    B, H, steps = 3, 4, 6
    sl = np.array([2.0 ** -1, 2.0 ** -3, 2.0 ** -6, 0.0], np.float32)
    rng = np.random.default_rng(6)
    kv0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    state = kv0.astype(np.float64)
    kvt = torch.from_numpy(kv0).to(device)
    ts = torch.from_numpy(sl).to(device)
    ex, raw = inputs(34, B, H, steps, d, dtype)
    for t in range(steps):
        q, k, v = (to_device(np.ascontiguousarray(x[:, :, t]), dtype, device) for x in raw)
        o = torch.empty_like(q)
        la.la_decode(q, k, v, ts, kvt, o)
        o_ref = oracle.decode_step(*(x[:, :, t] for x in ex), sl, state)
        torch.cuda.synchronize()
        assert_close(to_host(o)[:, :, None], o_ref[:, :, None], dtype, f"decode o step {t}", stored=dtype)
    assert_close(kvt.cpu().numpy(), state, dtype, "decode KV")


def test_n_zero_is_noop(device):
    torch = _torch()
    q = torch.zeros(1, 2, 0, 128, dtype=torch.bfloat16, device=device)
    kv = torch.randn(1, 2, 128, 128, device=device)
    before = kv.clone()
    la.la_prefill(q, q, q, torch.zeros(2, device=device), kv, o=torch.empty_like(q))
    torch.cuda.synchronize()
    assert torch.equal(kv, before)


def test_bf16_d64_chunked_with_states(device):
    # chunks and sub-chunk summaries through the full-width summary kernel at d = 64
    kv0 = np.random.default_rng(10).standard_normal((1, 2, 64, 64)).astype(np.float32)
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, 2, 9000, 64) < 9000
    check_prefill(36, 1, 2, 9000, 64, "bf16", SL2, device, kv_in=kv0)


def test_bf16_chunked_batch_with_states(device):
    # two sequences of the batch, both cut into chunks and sub-chunk summaries (full-width
    # summary kernel; main pass on 64-column slices), each from its own incoming state
    kv0 = np.random.default_rng(9).standard_normal((2, 2, 128, 128)).astype(np.float32)
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 2, 2, 5000, 128) < 5000
    check_prefill(28, 2, 2, 5000, 128, "bf16", SL2, device, kv_in=kv0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_aliased_inputs(device, dtype):
    # q, k and v may be one tensor (self-similarity attention): the same values as three copies
    torch = _torch()
    B, H, N, d = 1, 2, 700, 128
    exact, raw = inputs(40, B, H, N, d, dtype)
    x = to_device(raw[0], dtype, device)
    kv = torch.zeros(B, H, d, d, device=device)
    o = torch.empty_like(x)
    la.la_prefill(x, x, x, torch.from_numpy(SL2).to(device), kv, o=o, chunk_tokens=256)
    torch.cuda.synchronize()
    o_ref, kv_ref, _ = oracle.recurrent(exact[0], exact[0], exact[0], SL2)
    assert_close(to_host(o), o_ref, dtype, "aliased O", stored=dtype)
    assert_close(kv.cpu().numpy(), kv_ref, dtype, "aliased KV")
