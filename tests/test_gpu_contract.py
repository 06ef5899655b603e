"""GPU tests of boundary behaviour against the fp64 oracle: checkpoints at any positive interval,
the decode workload over all of its 1000 timed steps, NaN / Inf confinement, the packed entry
point's table staging under back-to-back calls, streams other than the current one, and
expanded (stride-0) inputs through the differentiable op.

Bars as everywhere (tests/common.py): per (batch, head) slice, the error beyond half an ulp of
the stored result is <= 2e-2 * RMS for bf16 inputs and <= 1e-4 * RMS for float32."""
import numpy as np
import pytest

import long_context_la_amd as la
import oracle
import synth
from common import assert_close, inputs, to_device, to_host

pytestmark = pytest.mark.gpu

SL2 = np.array([2.0 ** -2, 2.0 ** -8], dtype=np.float32)


def _prefill_ckpt(seed, N, d, dtype, ckpt_every, chunk_tokens, device, kv_in=None):
    import torch

    exact, raw = inputs(seed, 1, 2, N, d, dtype)
    q, k, v = (to_device(x, dtype, device) for x in raw)
    kv = (torch.zeros(1, 2, d, d, device=device) if kv_in is None
          else torch.from_numpy(kv_in).to(device))
    o = torch.empty_like(q)
    ck = torch.full((1, 2, N // ckpt_every, d, d), float("nan"), device=device)
    la.la_prefill(q, k, v, torch.from_numpy(SL2).to(device), kv, o=o, ckpt=ck, ckpt_every=ckpt_every,
                  chunk_tokens=chunk_tokens)
    torch.cuda.synchronize()
    o_ref, kv_ref, ck_ref = oracle.recurrent(*exact, SL2, kv_in=kv_in, ckpt_every=ckpt_every)
    assert_close(to_host(o), o_ref, dtype, f"O (ckpt_every={ckpt_every})", stored=dtype)
    assert_close(kv.cpu().numpy(), kv_ref, dtype, "final KV")
    got = ck.cpu().numpy()
    assert not np.isnan(got).any(), "a checkpoint slot was not written"
    for m in range(N // ckpt_every):
        assert_close(got[:, :, m], ck_ref[:, :, m], dtype, f"checkpoint {m}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ckpt_every,N,chunk", [(100, 1000, 0), (37, 300, 0), (1000, 4097, 0), (999, 3000, 1024),
                                                 (100, 250, 0)])
def test_checkpoints_at_any_interval(device, dtype, ckpt_every, N, chunk):
    # intervals that are not multiples of the 64-token tile: the sequence runs segment by segment
    _prefill_ckpt(50, N, 128 if dtype == "bf16" else 64, dtype, ckpt_every, chunk, device)


def test_checkpoints_any_interval_from_incoming_state(device):
    kv0 = np.random.default_rng(51).standard_normal((1, 2, 128, 128)).astype(np.float32)
    _prefill_ckpt(51, 2500, 128, "bf16", 700, 0, device, kv_in=kv0)


def test_checkpoints_any_interval_long_chunked_segments(device):
    # segments long enough to be chunked (LASP+ summaries) inside each segment
    _prefill_ckpt(52, 20000, 128, "bf16", 9001, 0, device)


def test_decode_workload_all_timed_steps(device):
    """The 128 x 64 decode workload exactly as the benchmark runs it (states from the 4096-token
    prefix, then 1000 consecutive steps), checked on sampled (sequence, head) units against the
    oracle's recurrence over all 4096 + 1000 tokens: every step's output and the final state."""
    import torch

    w = synth.WORKLOADS["decode"]
    B, H, d, P, steps = w.batch, w.heads, w.d, w.n, 1000
    slopes = w.slopes()
    ts = torch.from_numpy(slopes).to(device)
    kv = torch.empty(B, H, d, d, dtype=torch.float32, device=device)
    la.la_state_init(kv)
    for b0 in range(0, B, 16):
        kk = to_device(synth.generate(synth.K, w.seed, d, b0=b0, nb=16, nh=H, nt=P, dtype="bf16"), "bf16", device)
        vv = to_device(synth.generate(synth.V, w.seed, d, b0=b0, nb=16, nh=H, nt=P, dtype="bf16"), "bf16", device)
        la.la_prefill(kk, kk, vv, ts, kv[b0:b0 + 16], o=None)
        del kk, vv
    toks = [to_device(np.ascontiguousarray(
        synth.generate(t, w.seed, d, nb=B, nh=H, t0=P, nt=steps, dtype="bf16").transpose(2, 0, 1, 3)), "bf16", device)
        for t in (synth.Q, synth.K, synth.V)]
    units = [(0, 0), (0, 63), (127, 0), (127, 63), (37, 5), (64, 31), (90, 47), (113, 12)]
    bi = torch.tensor([b for b, _ in units], device=device)
    hi = torch.tensor([h for _, h in units], device=device)
    hist = torch.empty(steps, len(units), d, dtype=torch.bfloat16, device=device)
    o = torch.empty(B, H, d, dtype=torch.bfloat16, device=device)
    for s in range(steps):
        la.la_decode(toks[0][s], toks[1][s], toks[2][s], ts, kv, o)
        hist[s] = o[bi, hi]
    torch.cuda.synchronize()
    got_o = hist.float().cpu().numpy()
    got_kv = kv[bi, hi].cpu().numpy()
    del toks
    for i, (b, h) in enumerate(units):
        ex = [synth.bf16_bits_to_f32(synth.generate(t, w.seed, d, b0=b, h0=h, nt=P + steps, dtype="bf16"))
              for t in (synth.Q, synth.K, synth.V)]
        sl = slopes[h:h + 1]
        _, kv_p, _ = oracle.recurrent(*(x[:, :, :P] for x in ex), sl, want_o=False)
        o_ref, kv_ref, _ = oracle.recurrent(*(x[:, :, P:] for x in ex), sl, kv_in=kv_p)
        assert_close(got_o[:, i][None, None], o_ref, "bf16", f"decode outputs, unit {(b, h)}", stored="bf16")
        assert_close(got_kv[i][None, None], kv_ref, "bf16", f"decode state after {steps} steps, unit {(b, h)}")


@pytest.mark.parametrize("dtype,chunk", [("bf16", 0), ("bf16", 256), ("f32", 0)])
def test_nan_and_inf_stay_confined(device, dtype, chunk):
    """A NaN in one head's q and an Inf in another head's v: the other heads, the other rows of
    the q head and the other value columns of the v head are bit-identical to a clean run; the
    q head's state is untouched; the poisoned row / column are non-finite.  No hang.  (Inside
    the Inf's own 64-token tile, rows before it may turn NaN in that column too: the tile's
    masked product multiplies the Inf by the mask's zero.)"""
    import torch

    d = 128 if dtype == "bf16" else 64
    H, N = 4, 700
    exact, raw = inputs(53, 1, H, N, d, dtype)
    sl = torch.from_numpy(np.array([0.9, 2.0 ** -2, 2.0 ** -8, 0.0], np.float32)).to(device)

    def run(poison):
        q, k, v = (to_device(x, dtype, device) for x in raw)
        if poison:
            q[0, 1, 300, 5] = float("nan")
            v[0, 2, 100, 7] = float("inf")
        kv = torch.zeros(1, H, d, d, device=device)
        o = torch.empty_like(q)
        la.la_prefill(q, k, v, sl, kv, o=o, chunk_tokens=chunk)
        torch.cuda.synchronize()
        return o.float().cpu().numpy(), kv.cpu().numpy()

    o0, kv0 = run(False)
    o1, kv1 = run(True)
    assert np.isfinite(o0).all() and np.isfinite(kv0).all()
    for h in (0, 3):
        assert np.array_equal(o1[0, h], o0[0, h]) and np.array_equal(kv1[0, h], kv0[0, h])
    # q head: only row 300 of the output
    rows = np.arange(N) != 300
    assert np.array_equal(o1[0, 1, rows], o0[0, 1, rows])
    assert not np.isfinite(o1[0, 1, 300]).any()
    assert np.array_equal(kv1[0, 1], kv0[0, 1])
    # v head: value column 7 from token 100 on, in the outputs and the state
    cols = np.arange(d) != 7
    assert np.array_equal(o1[0, 2][:, cols], o0[0, 2][:, cols])
    assert np.array_equal(o1[0, 2, :64], o0[0, 2, :64])      # tiles before the Inf's
    assert not np.isfinite(o1[0, 2, 100:, 7]).any()
    assert np.array_equal(kv1[0, 2][:, cols], kv0[0, 2][:, cols])
    assert not np.isfinite(kv1[0, 2][:, 7]).any()


def test_nan_in_decode_stays_confined(device):
    import torch

    B, H, d = 2, 3, 128
    rng = np.random.default_rng(54)
    kv_init = torch.from_numpy(rng.standard_normal((B, H, d, d)).astype(np.float32)).to(device)
    q, k, v = (torch.from_numpy(rng.standard_normal((B, H, d)).astype(np.float32)).to(device).to(torch.bfloat16)
               for _ in range(3))
    sl = torch.tensor([0.5, 0.1, 0.0], device=device)

    def run(poison):
        kv = kv_init.clone()
        qq, kk = q.clone(), k.clone()
        if poison:
            qq[1, 0, 3] = float("nan")
            kk[0, 2, 9] = float("inf")
        o = torch.empty_like(q)
        la.la_decode(qq, kk, v, sl, kv, o)
        torch.cuda.synchronize()
        return o.float().cpu().numpy(), kv.cpu().numpy()

    o0, kv0 = run(False)
    o1, kv1 = run(True)
    clean = [(0, 0), (0, 1), (1, 1), (1, 2)]
    for b, h in clean:
        assert np.array_equal(o1[b, h], o0[b, h]) and np.array_equal(kv1[b, h], kv0[b, h])
    assert not np.isfinite(o1[1, 0]).any() and np.array_equal(kv1[1, 0], kv0[1, 0])    # NaN q: output only
    rows = np.arange(d) != 9
    assert np.array_equal(kv1[0, 2][rows], kv0[0, 2][rows]) and not np.isfinite(kv1[0, 2][9]).any()


def test_varlen_back_to_back_calls_reuse_staging(device):
    """Twenty packed prefills enqueued without a synchronisation in between, with tables of
    growing size: small ones travel in kernel arguments, larger ones through the page-locked
    staging ring, which wraps and regrows while copies are in flight."""
    import torch

    H, d = 2, 128
    rng = np.random.default_rng(55)
    sl = torch.from_numpy(SL2).to(device)
    runs = []
    for i in range(20):
        if i < 8:
            lengths = [int(x) for x in rng.integers(0, 300, size=4 + 5 * i)]
        else:  # many short sequences: tables past the kernel-argument size, growing
            lengths = [int(x) for x in rng.integers(0, 40, size=120 + 60 * (i - 8))]
        cu = [0] + list(np.cumsum(lengths))
        T = cu[-1]
        exact, raw = inputs(100 + i, 1, H, T, d, "bf16")
        q, k, v = (to_device(np.ascontiguousarray(x[0].transpose(1, 0, 2)), "bf16", device) for x in raw)
        kv = torch.zeros(len(lengths), H, d, d, device=device)
        o = torch.empty_like(q)
        la.la_prefill_varlen(q, k, v, sl, kv, cu, o=o)
        runs.append((exact, cu, o, kv))
    torch.cuda.synchronize()
    for exact, cu, o, kv in runs:
        got_o = o.float().cpu().numpy()
        got_kv = kv.cpu().numpy()
        for s in range(len(cu) - 1):
            a, b = cu[s], cu[s + 1]
            if b == a:
                assert not got_kv[s].any()
                continue
            o_ref, kv_ref, _ = oracle.recurrent(*(x[:, :, a:b] for x in exact), SL2)
            assert_close(got_o[a:b].transpose(1, 0, 2)[None], o_ref, "bf16", f"varlen O, sequence {s}", stored="bf16")
            assert_close(got_kv[s][None], kv_ref, "bf16", f"varlen KV, sequence {s}")


def test_prefill_on_a_side_stream(device):
    # a chunked prefill (workspace allocated by the binding) enqueued on a stream other than the
    # current one; the workspace is recorded on that stream
    import torch

    exact, raw = inputs(56, 1, 2, 6000, 128, "bf16")
    q, k, v = (to_device(x, "bf16", device) for x in raw)
    kv = torch.zeros(1, 2, 128, 128, device=device)
    o = torch.empty_like(q)
    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream(device))
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, 2, 6000, 128) < 6000
    la.la_prefill(q, k, v, torch.from_numpy(SL2).to(device), kv, o=o, stream=side)
    scratch = torch.empty(64 << 20, dtype=torch.uint8, device=device).fill_(0xff)   # reuses freed memory if any
    side.synchronize()
    del scratch
    o_ref, kv_ref, _ = oracle.recurrent(*exact, SL2)
    assert_close(to_host(o), o_ref, "bf16", "side-stream O", stored="bf16")
    assert_close(kv.cpu().numpy(), kv_ref, "bf16", "side-stream KV")


def test_expanded_inputs_through_autograd(device):
    """q shared by all heads as a stride-0 view: the op makes it dense before laying out its
    outputs, and the gradient reaching the shared q is the sum over heads."""
    import torch

    B, H, N, d = 1, 3, 500, 128
    rng = np.random.default_rng(57)
    base = torch.from_numpy(rng.standard_normal((B, 1, N, d)).astype(np.float32)).to(device).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((B, H, N, d)).astype(np.float32)).to(device).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((B, H, N, d)).astype(np.float32)).to(device).to(torch.bfloat16)
    g = torch.from_numpy(rng.standard_normal((B, H, N, d)).astype(np.float32)).to(device)
    sl = torch.tensor([0.5, 0.05, 0.0], device=device)
    grads = []
    for dense in (False, True):
        q0 = base.clone().requires_grad_(True)
        q = q0.expand(B, H, N, d)
        if dense:
            q = q.contiguous()
        o, _ = la.lightning_attention(q, k, v, sl)
        (o.float() * g).sum().backward()
        grads.append((o.detach().float().cpu(), q0.grad.float().cpu()))
    assert torch.equal(grads[0][0], grads[1][0])
    assert torch.equal(grads[0][1], grads[1][1])
    assert torch.isfinite(grads[0][1]).all()



@pytest.mark.parametrize("chunk", [0, 512])
@pytest.mark.parametrize("scale,kv_scale", [((40.0, 40.0, 500.0), 1e6), ((2.0 ** -4,) * 3, 1e-2)])
def test_bf16_products_far_from_unit_scale(device, chunk, scale, kv_scale):
    """The bf16 path's products take float16 operands (inputs converted exactly; scores, weighted
    values and the state scaled by 2^-8).  Inputs up to a few thousand with states of order 1e6,
    and inputs of order 2^-4 with states of order 1e-2, stay inside that format's normal range
    where it matters and meet the bf16 bar."""
    import torch

    B, H, N, d = 1, 2, 2000, 128
    exact, _ = inputs(58, B, H, N, d, "bf16")
    scaled = [synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x * c)) for x, c in zip(exact, scale)]
    q, k, v = (to_device(synth.f32_to_bf16_bits(x), "bf16", device) for x in scaled)
    kv0 = (np.random.default_rng(59).standard_normal((B, H, d, d)) * kv_scale).astype(np.float32)
    kv = torch.from_numpy(kv0).to(device)
    o = torch.empty_like(q)
    slopes = np.array([2.0 ** -2, 2.0 ** -12], dtype=np.float32)    # the second head keeps kv0
    la.la_prefill(q, k, v, torch.from_numpy(slopes).to(device), kv, o=o, chunk_tokens=chunk)
    torch.cuda.synchronize()
    o_ref, kv_ref, _ = oracle.recurrent(*scaled, slopes, kv_in=kv0)
    if kv_scale > 1:
        assert max(float(np.abs(x).max()) for x in scaled) > 2000 and np.abs(kv_ref).max() > 1e6
    assert_close(to_host(o), o_ref, "bf16", "O", stored="bf16")
    assert_close(kv.cpu().numpy(), kv_ref, "bf16", "KV")


@pytest.mark.parametrize("n_tiled,n_short", [(52, 4), (55, 0)])
def test_varlen_tables_at_the_kernel_argument_limit(device, n_tiled, n_short):
    """Chunk tables of 384 int64 words (5 per tiled chunk, 2 per sequence, 3 more per sequence
    of at most 8 tokens) travel in kernel arguments, 385 words through page-locked staging; both
    sides of that boundary against the oracle, sequence by sequence."""
    import torch

    words = 7 * n_tiled + 5 * n_short
    assert words in (384, 385)
    H, d = 2, 128
    rng = np.random.default_rng(60 + words)
    lengths = [int(x) for x in rng.integers(9, 200, size=n_tiled)] + [int(x) for x in rng.integers(1, 9, size=n_short)]
    lengths = [lengths[i] for i in rng.permutation(len(lengths))]
    cu = [0] + list(np.cumsum(lengths))
    exact, raw = inputs(61, 1, H, cu[-1], d, "bf16")
    q, k, v = (to_device(np.ascontiguousarray(x[0].transpose(1, 0, 2)), "bf16", device) for x in raw)
    kv = torch.zeros(len(lengths), H, d, d, device=device)
    o = torch.empty_like(q)
    la.la_prefill_varlen(q, k, v, torch.from_numpy(SL2).to(device), kv, cu, o=o)
    torch.cuda.synchronize()
    got_o, got_kv = o.float().cpu().numpy(), kv.cpu().numpy()
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        o_ref, kv_ref, _ = oracle.recurrent(*(x[:, :, a:b] for x in exact), SL2)
        assert_close(got_o[a:b].transpose(1, 0, 2)[None], o_ref, "bf16", f"varlen O, sequence {s} ({b - a} tokens)",
                     stored="bf16")
        assert_close(got_kv[s][None], kv_ref, "bf16", f"varlen KV, sequence {s}")
