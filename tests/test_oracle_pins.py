"""Pins for the fp64 oracle: each check ties it to something other than itself.

Sources: page "MiniMax-01: Scaling Foundation Models with Lightning Attention |
Summary", section 2.2 (reordered Q(K^T V) form, causal cumulative state,
tiles = intra masked term + inter state term, no normalisation/SiLU/gating)
and section 3.2 (LASP+: local prefix summaries combined into global
prefixes).  The pages print no worked numbers, so the pins are a hand-worked
example, closed forms, textbook routines (cumulative sum, a first-order IIR
filter), identities and brute force -- chosen so that a dropped term, a wrong
exponent, a transposed state or a read-before-update fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny():
    w = synth.WORKLOADS["tiny"]
    q = synth.generate(synth.Q, w.seed, w.d, nh=w.heads, nt=w.n)
    k = synth.generate(synth.K, w.seed, w.d, nh=w.heads, nt=w.n)
    v = synth.generate(synth.V, w.seed, w.d, nh=w.heads, nt=w.n)
    return q, k, v, w.slopes().astype(np.float64)


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


# ---------------------------------------------------------------- generator

def test_splitmix64_published_sequence():
    # SplitMix64 seeded with 0 (Steele, Lea & Flood 2014) -- its first four outputs, as published
    # with the reference xoshiro seeding code.
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    gamma = 0x9E3779B97F4A7C15
    got = [synth.splitmix64_next((i * gamma) % 2**64) for i in range(4)]
    assert got == want


def test_generator_moments_and_slices():
    z = synth.generate(synth.V, 11, 128, nh=4, nt=4096)
    x = synth.generate(synth.Q, 11, 128, nh=4, nt=4096)
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1.0) < 0.01
    # E[SiLU(z)] = 0.2066, E[SiLU(z)^2] = 0.3558 for z ~ N(0,1) (numerical integration below)
    t = np.linspace(-12, 12, 200001)
    pdf = np.exp(-t * t / 2) / math.sqrt(2 * math.pi)
    silu = t / (1 + np.exp(-t))
    m1 = np.trapezoid(silu * pdf, t)
    m2 = np.trapezoid(silu * silu * pdf, t)
    assert abs(x.mean() - m1) < 0.005 and abs((x.astype(np.float64) ** 2).mean() - m2) < 0.005
    # counter-based: any slice regenerates exactly
    part = synth.generate(synth.Q, 11, 128, h0=2, nh=1, t0=1000, nt=77)
    assert np.array_equal(part[0, 0], x[0, 2, 1000:1077])
    # bf16 bits are the RNE rounding of the float32 values
    xb = synth.generate(synth.Q, 11, 128, nh=4, nt=64, dtype="bf16")
    assert np.array_equal(xb, synth.f32_to_bf16_bits(x[:, :, :64]))


def test_bf16_rounding_rule():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 0.0], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(vals)
    back = synth.bf16_bits_to_f32(bits)
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1); 1+3*2^-8 ties to 1+2^-6 (even mantissa)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2**-6, 1.0, -2.5, 0.0]


# ---------------------------------------------------------------- hand-worked example

def test_hand_worked_example_all_forms():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_d2_n3.json")))
    q = np.array(g["q"], dtype=np.float32)[None, None]
    k = np.array(g["k"], dtype=np.float32)[None, None]
    v = np.array(g["v"], dtype=np.float32)[None, None]
    s = np.array([g["slope"]])
    kv_in = np.array(g["kv_in"], dtype=np.float64)[None, None]
    for kin, o_want, kv_want in ((None, g["o_zero_state"], g["kv_zero_state"]),
                                 (kv_in, g["o_with_state"], g["kv_with_state"])):
        o_r, kv_r, _ = oracle.recurrent(q, k, v, s, kv_in=kin)
        o_q, kv_q = oracle.quadratic(q, k, v, s, kv_in=kin)
        np.testing.assert_allclose(o_r[0, 0], o_want, atol=1e-12)
        np.testing.assert_allclose(kv_r[0, 0], kv_want, atol=1e-12)
        np.testing.assert_allclose(o_q[0, 0], o_want, atol=1e-12)
        np.testing.assert_allclose(kv_q[0, 0], kv_want, atol=1e-12)
        for blk in (1, 2, 3, 5):
            o_b, kv_b = oracle.blocked(q, k, v, s, blk, kv_in=kin)
            np.testing.assert_allclose(o_b[0, 0], o_want, atol=1e-12)
            np.testing.assert_allclose(kv_b[0, 0], kv_want, atol=1e-12)
        kv = np.zeros((1, 1, 2, 2)) if kin is None else kin.copy()
        for t in range(3):
            o_t = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], s, kv)
            np.testing.assert_allclose(o_t[0, 0], o_want[t], atol=1e-12)
        np.testing.assert_allclose(kv[0, 0], kv_want, atol=1e-12)


# ---------------------------------------------------------------- P1: forms agree

@pytest.mark.parametrize("block", [1, 7, 64, 256, 512])
def test_p1_recurrent_quadratic_blocked_agree(block):
    q, k, v, s = _tiny()
    o_r, kv_r, _ = oracle.recurrent(q, k, v, s)
    o_q, kv_q = oracle.quadratic(q, k, v, s)
    o_b, kv_b = oracle.blocked(q, k, v, s, block)
    assert _rel(o_q, o_r) < 1e-12 and _rel(kv_q, kv_r) < 1e-12
    assert _rel(o_b, o_r) < 1e-12 and _rel(kv_b, kv_r) < 1e-12


def test_p1_with_incoming_state_and_ragged_tail():
    q, k, v, s = _tiny()
    N = 301  # not a multiple of any block below
    q, k, v = q[:, :, :N], k[:, :, :N], v[:, :, :N]
    rng = np.random.default_rng(7)
    kv_in = rng.standard_normal((1, 2, 64, 64))
    o_r, kv_r, _ = oracle.recurrent(q, k, v, s, kv_in=kv_in)
    o_q, kv_q = oracle.quadratic(q, k, v, s, kv_in=kv_in)
    assert _rel(o_q, o_r) < 1e-12 and _rel(kv_q, kv_r) < 1e-12
    for block in (7, 64, 256):
        o_b, kv_b = oracle.blocked(q, k, v, s, block, kv_in=kv_in)
        assert _rel(o_b, o_r) < 1e-12 and _rel(kv_b, kv_r) < 1e-12


# ---------------------------------------------------------------- P2: no decay = cumulative sum

def test_p2_no_decay_is_cumulative_sum_attention():
    q, k, v, _ = _tiny()
    q, k, v = q[:, :1, :200], k[:, :1, :200], v[:, :1, :200]
    s = np.array([0.0])
    o, kv, _ = oracle.recurrent(q, k, v, s)
    outer = np.einsum("ti,tj->tij", k[0, 0].astype(np.float64), v[0, 0].astype(np.float64))
    states = np.cumsum(outer, axis=0)
    want = np.einsum("ti,tij->tj", q[0, 0].astype(np.float64), states)
    assert _rel(o[0, 0], want) < 1e-12
    assert _rel(kv[0, 0], states[-1]) < 1e-12


# ---------------------------------------------------------------- P3: d = 1 is a first-order IIR filter

def test_p3_scalar_case_is_first_order_filter():
    rng = np.random.default_rng(3)
    N = 1000
    q = rng.standard_normal((1, 1, N, 1)).astype(np.float32)
    k = rng.standard_normal((1, 1, N, 1)).astype(np.float32)
    v = rng.standard_normal((1, 1, N, 1)).astype(np.float32)
    s = 0.01
    lam = math.exp(-s)
    o, kv, _ = oracle.recurrent(q, k, v, np.array([s]))
    y = scipy.signal.lfilter([1.0], [1.0, -lam], (k.astype(np.float64) * v.astype(np.float64)).ravel())
    want = q.astype(np.float64).ravel() * y
    assert _rel(o.ravel(), want) < 1e-12
    assert abs(kv.ravel()[0] - y[-1]) <= 1e-12 * abs(y[-1])


# ---------------------------------------------------------------- P4: impulse

def test_p4_impulse_response():
    rng = np.random.default_rng(4)
    N, d, src = 300, 16, 37
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    k = np.zeros((1, 1, N, d), dtype=np.float32)
    v = np.zeros((1, 1, N, d), dtype=np.float32)
    k[0, 0, src] = rng.standard_normal(d)
    v[0, 0, src] = rng.standard_normal(d)
    s = 0.05
    o, kv, _ = oracle.recurrent(q, k, v, np.array([s]))
    t = np.arange(N)
    qk = q[0, 0].astype(np.float64) @ k[0, 0, src].astype(np.float64)
    want = np.where(t >= src, np.exp(-s * np.maximum(t - src, 0)), 0.0)[:, None] * qk[:, None] \
        * v[0, 0, src].astype(np.float64)[None, :]
    np.testing.assert_allclose(o[0, 0], want, rtol=1e-12, atol=1e-300)
    kv_want = math.exp(-s * (N - 1 - src)) * np.outer(k[0, 0, src].astype(np.float64), v[0, 0, src].astype(np.float64))
    np.testing.assert_allclose(kv[0, 0], kv_want, rtol=1e-12)


# ---------------------------------------------------------------- P5: single token

def test_p5_single_token_closed_form():
    rng = np.random.default_rng(5)
    d = 32
    q, k, v = (rng.standard_normal((1, 1, 1, d)).astype(np.float32) for _ in range(3))
    kv_in = rng.standard_normal((1, 1, d, d))
    s = 0.3
    o, kv, _ = oracle.recurrent(q, k, v, np.array([s]), kv_in=kv_in)
    q64, k64, v64 = (x.astype(np.float64)[0, 0, 0] for x in (q, k, v))
    kv_want = math.exp(-s) * kv_in[0, 0] + np.outer(k64, v64)
    np.testing.assert_allclose(kv[0, 0], kv_want, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 0], q64 @ kv_want, rtol=1e-13)
    o0, kv0, _ = oracle.recurrent(q, k, v, np.array([s]))
    np.testing.assert_allclose(o0[0, 0, 0], (q64 @ k64) * v64, rtol=1e-14)


# ---------------------------------------------------------------- P6: continuation, checkpoints, decode

def test_p6_continuation_and_checkpoints_and_decode():
    q, k, v, s = _tiny()
    N1 = 200
    o, kv, ck = oracle.recurrent(q, k, v, s, ckpt_every=100)
    o1, kv1, _ = oracle.recurrent(q[:, :, :N1], k[:, :, :N1], v[:, :, :N1], s)
    o2, kv2, _ = oracle.recurrent(q[:, :, N1:], k[:, :, N1:], v[:, :, N1:], s, kv_in=kv1)
    assert _rel(np.concatenate([o1, o2], axis=2), o) < 1e-12 and _rel(kv2, kv) < 1e-12
    assert ck.shape[2] == 5
    assert _rel(ck[:, :, 1], kv1) < 1e-12
    assert _rel(ck[:, :, 4], oracle.recurrent(q[:, :, :500], k[:, :, :500], v[:, :, :500], s, want_o=False)[1]) < 1e-12
    state = kv1.copy()
    for t in range(N1, N1 + 40):
        ot = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], s, state)
        assert _rel(ot, o[:, :, t]) < 1e-12
    ref = oracle.recurrent(q[:, :, :N1 + 40], k[:, :, :N1 + 40], v[:, :, :N1 + 40], s, want_o=False)[1]
    assert _rel(state, ref) < 1e-12


# ---------------------------------------------------------------- P7: LASP+ prefixes

@pytest.mark.parametrize("chunks", [[512], [256, 256], [100, 200, 212], [64] * 8, [1, 510, 1]])
def test_p7_lasp_plus_combine_equals_serial(chunks):
    q, k, v, s = _tiny()
    rng = np.random.default_rng(8)
    kv_in = rng.standard_normal((1, 2, 64, 64))
    o, kv, _ = oracle.recurrent(q, k, v, s, kv_in=kv_in)
    S = oracle.chunk_local_states(k, v, s, chunks)
    P = oracle.lasp_plus_prefixes(S, s, chunks, kv_in=kv_in)
    assert _rel(P[:, :, -1], kv) < 1e-12
    start = 0
    for j, C in enumerate(chunks):
        oj, kvj, _ = oracle.recurrent(q[:, :, start:start + C], k[:, :, start:start + C],
                                      v[:, :, start:start + C], s, kv_in=P[:, :, j])
        assert _rel(oj, o[:, :, start:start + C]) < 1e-11
        assert _rel(kvj, P[:, :, j + 1]) < 1e-12
        start += C


# ---------------------------------------------------------------- P8: linearity (no hidden normalisation)

def test_p8_linearity():
    q, k, v, s = _tiny()
    q, k, v = q[:, :, :128], k[:, :, :128], v[:, :, :128]
    rng = np.random.default_rng(9)
    v2 = rng.standard_normal(v.shape).astype(np.float32)
    a, b = 0.75, -2.0
    o1 = oracle.recurrent(q, k, v, s)[0]
    o2 = oracle.recurrent(q, k, v2, s)[0]
    o12 = oracle.recurrent(q, k, (a * v.astype(np.float64) + b * v2).astype(np.float32), s)[0]
    # a*v + b*v2 rounded to float32 -> compare against the same rounded input via linearity on exact parts
    vmix = (a * v.astype(np.float64) + b * v2).astype(np.float32)
    o_lin = oracle.recurrent(q, k, vmix, s)[0]
    assert _rel(o12, o_lin) == 0.0
    assert _rel(o12, a * o1 + b * o2) < 1e-6  # the only gap is the float32 rounding of vmix
    o_scaled = oracle.recurrent((4.0 * q).astype(np.float32), k, v, s)[0]  # power of two: exact
    assert _rel(o_scaled, 4.0 * o1) < 1e-13


# ---------------------------------------------------------------- P9: windowing (long-context spot checks)

def test_p9_window_restart_bound():
    rng = np.random.default_rng(10)
    N, d, W = 12000, 8, 8192
    s = 2.0 ** -8
    q, k, v = (rng.standard_normal((1, 1, N, d)).astype(np.float32) for _ in range(3))
    o, kv, _ = oracle.recurrent(q, k, v, np.array([s]))
    t0 = N - 500
    ow, kvw, _ = oracle.recurrent(q[:, :, t0 - W:], k[:, :, t0 - W:], v[:, :, t0 - W:], np.array([s]))
    bound = math.exp(-s * W)  # relative size of everything before the window
    assert bound < 2e-14
    assert _rel(ow[:, :, W:], o[:, :, t0:]) < 50 * bound
    assert _rel(kvw, kv) < 50 * bound


# ---------------------------------------------------------------- the pins catch planted mistakes

def _mutant_recurrent(q, k, v, s, kind):
    """Deliberately wrong variants, to show each is caught by the hand-worked example."""
    q, k, v = (np.asarray(x, dtype=np.float64)[0, 0] for x in (q, k, v))
    lam = math.exp(-s)
    KV = np.zeros((q.shape[1], q.shape[1]))
    out = []
    for t in range(q.shape[0]):
        prev = KV.copy()
        if kind == "no_decay":
            KV = KV + np.outer(k[t], v[t])
        elif kind == "transposed_state":
            KV = lam * KV + np.outer(v[t], k[t])
        else:
            KV = lam * KV + np.outer(k[t], v[t])
        if kind == "read_before_update":
            out.append(q[t] @ prev)
        elif kind == "double_decay_on_read":
            out.append(lam * (q[t] @ KV))
        else:
            out.append(q[t] @ KV)
    return np.array(out)


@pytest.mark.parametrize("kind", ["no_decay", "transposed_state", "read_before_update", "double_decay_on_read"])
def test_planted_mistakes_are_caught(kind):
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_d2_n3.json")))
    q = np.array(g["q"], dtype=np.float32)[None, None]
    k = np.array(g["k"], dtype=np.float32)[None, None]
    v = np.array(g["v"], dtype=np.float32)[None, None]
    got = _mutant_recurrent(q, k, v, g["slope"], kind)
    assert np.abs(got - np.array(g["o_zero_state"])).max() > 0.1
    ok = _mutant_recurrent(q, k, v, g["slope"], "correct")
    np.testing.assert_allclose(ok, g["o_zero_state"], atol=1e-12)


# ---------------------------------------------------------------- prologue / epilogue pins
def test_p10_sigmoid_and_silu_values():
    # sigmoid(1) = 1 / (1 + e^-1); SiLU(x) - SiLU(-x) = x; limits; SiLU(0) = 0
    assert oracle.sigmoid(0.0) == 0.5
    assert abs(float(oracle.sigmoid(1.0)) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(float(oracle.sigmoid(1.0)) - 0.7310585786300049) < 1e-15
    x = np.linspace(-30.0, 30.0, 121)
    np.testing.assert_allclose(oracle.sigmoid(x) + oracle.sigmoid(-x), 1.0, atol=1e-15)
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, atol=1e-12)
    assert float(oracle.silu(0.0)) == 0.0
    assert abs(float(oracle.silu(40.0)) - 40.0) < 1e-12
    assert abs(float(oracle.silu(-40.0))) < 1e-14
    assert abs(float(oracle.silu(-1.0)) + 0.2689414213699951) < 1e-15


def test_p11_rms_norm_values_and_invariants():
    # [3, 4]: mean square 12.5, so the normalised row is [3, 4] / sqrt(12.5)
    np.testing.assert_allclose(oracle.rms_norm(np.array([3.0, 4.0]), 0.0), [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)],
                               rtol=1e-15)
    rng = np.random.default_rng(0)
    o = rng.standard_normal((3, 5, 128))
    r = oracle.rms_norm(o, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(r * r, axis=-1)), 1.0, rtol=1e-12)   # unit RMS per row
    np.testing.assert_allclose(oracle.rms_norm(7.5 * o, 0.0), r, rtol=1e-12)          # scale invariant
    w = rng.standard_normal(128)
    np.testing.assert_allclose(oracle.rms_norm(o, 0.0, w), r * w, rtol=1e-12)          # per-feature weight
    # eps only matters for small rows: a zero row stays zero
    assert np.all(oracle.rms_norm(np.zeros(8), 1e-6) == 0.0)
    # the axis is the feature axis: normalising over tokens instead changes the result
    assert np.abs(oracle.rms_norm(o, 0.0) - np.swapaxes(oracle.rms_norm(np.swapaxes(o, -1, -2), 0.0), -1, -2)).max() > 0.1


def test_p12_fused_hand_worked_example():
    # d = 2, one token: k = [1, 0], v = [3, 4], q = [1, 0] -> o = q . (k^T v) = [3, 4];
    # RMS normalisation -> [3, 4] / sqrt(12.5); gate g = [0, 60] -> times [1/2, ~1]
    q = np.array([1.0, 0.0], dtype=np.float32)[None, None, None]
    k = np.array([1.0, 0.0], dtype=np.float32)[None, None, None]
    v = np.array([3.0, 4.0], dtype=np.float32)[None, None, None]
    g = np.array([0.0, 60.0])[None, None, None]
    o, kv = oracle.fused(q, k, v, [0.5], norm_eps=0.0, gate=g)
    r = math.sqrt(12.5)
    np.testing.assert_allclose(o[0, 0, 0], [3 / r * 0.5, 4 / r], rtol=1e-12)
    np.testing.assert_allclose(kv[0, 0], [[3.0, 4.0], [0.0, 0.0]], rtol=0, atol=0)
    # SiLU on v only: v -> [3 sigmoid(3), 4 sigmoid(4)]
    o, _ = oracle.fused(q, k, v, [0.5], silu_v=True)
    np.testing.assert_allclose(o[0, 0, 0], [3 / (1 + math.exp(-3)), 4 / (1 + math.exp(-4))], rtol=1e-7)


def test_p13_fused_without_options_is_the_recurrence():
    exact, _ = (lambda r: (r, None))([synth.generate(t, 9, 64, nb=1, nh=2, nt=70) for t in (synth.Q, synth.K, synth.V)])
    slopes = np.array([0.1, 0.01])
    o, kv = oracle.fused(*exact, slopes)
    o_r, kv_r, _ = oracle.recurrent(*exact, slopes)
    assert np.array_equal(o, o_r) and np.array_equal(kv, kv_r)
    # each option is the plain composition of its piece with the recurrence
    o, _ = oracle.fused(*exact, slopes, silu_q=True, silu_k=True)
    o_r, _, _ = oracle.recurrent(oracle.silu(exact[0]), oracle.silu(exact[1]), exact[2], slopes)
    np.testing.assert_allclose(o, o_r, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- backward pins
# The backward oracle (reverse state recurrence and n x n form) is tied to the forward definition by
# automatic differentiation (torch, float64, CPU, of the token recurrence written out below) and by
# central finite differences of the oracle's own forward; mutants show the pins bite.

def _bwd_inputs(seed, B, H, N, d, with_state=True):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    kv = rng.standard_normal((B, H, d, d)) if with_state else None
    g = rng.standard_normal((B, H, d, d)) if with_state else None
    slopes = np.array([0.05 + 0.6 * h for h in range(H)])
    return q, k, v, do, kv, g, slopes


def _loss(q, k, v, do, slopes, kv, g):
    """L = sum(dO . O) + sum(G_out . KV_final) through the oracle's forward (quadratic form)."""
    o, kv_out = oracle.quadratic(q, k, v, slopes, kv_in=kv)
    return float(np.sum(do * o) + (0.0 if g is None else np.sum(g * kv_out)))


@pytest.mark.parametrize("form", ["recurrent", "quadratic"])
def test_p14_backward_matches_autograd(form):
    torch = pytest.importorskip("torch")
    q, k, v, do, kv, g, slopes = _bwd_inputs(5, 1, 2, 23, 6)
    want = getattr(oracle, "backward_" + form)(q, k, v, do, slopes, kv_in=kv, dkv_out=g)
    T = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, kv)]
    tq, tk, tv, tkv = T
    loss = torch.zeros((), dtype=torch.float64)
    for h in range(2):
        lam = math.exp(-slopes[h])
        S = tkv[0, h]
        for t in range(q.shape[2]):
            S = lam * S + torch.outer(tk[0, h, t], tv[0, h, t])
            loss = loss + torch.dot(tq[0, h, t] @ S, torch.tensor(do[0, h, t]))
        loss = loss + torch.sum(S * torch.tensor(g[0, h]))
    grads = torch.autograd.grad(loss, T)
    for name, got, ref in zip(("dq", "dk", "dv", "dkv_in"), want, grads):
        assert _rel(got, ref.numpy()) < 1e-12, name


def test_p15_backward_matches_finite_differences():
    q, k, v, do, kv, g, slopes = _bwd_inputs(6, 1, 2, 7, 3)
    grads = oracle.backward_recurrent(q, k, v, do, slopes, kv_in=kv, dkv_out=g)
    rng = np.random.default_rng(11)
    eps = 1e-5
    for which in range(4):
        for _ in range(3):
            x = [q, k, v, kv]
            u = rng.standard_normal(x[which].shape)
            xp, xm = list(x), list(x)
            xp[which] = x[which] + eps * u
            xm[which] = x[which] - eps * u
            fd = (_loss(xp[0], xp[1], xp[2], do, slopes, xp[3], g) -
                  _loss(xm[0], xm[1], xm[2], do, slopes, xm[3], g)) / (2 * eps)
            an = float(np.sum(grads[which] * u))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("shape", [(1, 1, 1, 4), (2, 2, 65, 8), (1, 3, 130, 5)])
@pytest.mark.parametrize("with_state", [False, True])
def test_p16_backward_forms_agree(shape, with_state):
    q, k, v, do, kv, g, slopes = _bwd_inputs(7, *shape, with_state=with_state)
    a = oracle.backward_recurrent(q, k, v, do, slopes, kv_in=kv, dkv_out=g)
    b = oracle.backward_quadratic(q, k, v, do, slopes, kv_in=kv, dkv_out=g)
    for x, y in zip(a, b):
        assert _rel(x, y) < 1e-12


def test_p17_backward_empty_sequence_and_no_decay():
    # N = 0: the incoming state's gradient is the outgoing one, untouched
    q, k, v, do, kv, g, slopes = _bwd_inputs(8, 1, 2, 0, 4)
    dq, dk, dv, dkv = oracle.backward_recurrent(q, k, v, do, slopes, kv_in=kv, dkv_out=g)
    assert dq.shape == (1, 2, 0, 4) and np.array_equal(dkv, g)
    # lambda = 1: dV_s = sum_{t >= s} (q_t . k_s) do_t + k_s G_out -- reverse cumulative sums
    q, k, v, do, kv, g, _ = _bwd_inputs(9, 1, 1, 12, 3)
    _, _, dv, dkv = oracle.backward_recurrent(q, k, v, do, np.zeros(1), kv_in=kv, dkv_out=g)
    Q, K, dO = q[0, 0], k[0, 0], do[0, 0]
    rev = np.cumsum((Q[:, :, None] * dO[:, None, :])[::-1], axis=0)[::-1]  # sum_{t >= s} q_t^T do_t
    want = np.einsum("si,sij->sj", K, rev) + K @ g[0, 0]
    assert _rel(dv[0, 0], want) < 1e-12
    assert _rel(dkv[0, 0], Q.T @ dO + g[0, 0]) < 1e-12


def _mutant_backward(q, k, v, do, slopes, kv, g, kind):
    """Deliberately wrong variants of the reverse recurrence (one (b, h) of index 0 only)."""
    lam = math.exp(-float(slopes[0]))
    Q, K, Vm, dO = (x[0, 0] for x in (q, k, v, do))
    N, d = Q.shape
    arriving = g[0, 0].copy() if kind != "drop_g_out" else np.zeros((d, d))
    dk, dv = np.empty_like(Q), np.empty_like(Q)
    for t in range(N - 1, -1, -1):
        if kind == "decay_before_add":
            G = lam * (np.outer(Q[t], dO[t]) + arriving)
        else:
            G = np.outer(Q[t], dO[t]) + arriving
        dk[t] = Vm[t] @ (G if kind == "untransposed_dk" else G.T)
        dv[t] = K[t] @ G
        arriving = lam * G
    return dk, dv


@pytest.mark.parametrize("kind", ["drop_g_out", "decay_before_add", "untransposed_dk"])
def test_backward_planted_mistakes_are_caught(kind):
    q, k, v, do, kv, g, slopes = _bwd_inputs(10, 1, 1, 6, 3)
    rng = np.random.default_rng(12)
    eps = 1e-5

    def fd(which):
        u = rng.standard_normal(q.shape)
        x = [q, k, v]
        xp, xm = list(x), list(x)
        xp[which] = x[which] + eps * u
        xm[which] = x[which] - eps * u
        return u, (_loss(*xp, do, slopes, kv, g) - _loss(*xm, do, slopes, kv, g)) / (2 * eps)

    def caught(dk, dv):
        bad = False
        for which, grad in ((1, dk), (2, dv)):
            u, f = fd(which)
            bad |= abs(f - float(np.sum(grad * u[0, 0]))) > 1e-3 * max(1.0, abs(f))
        return bad

    assert caught(*_mutant_backward(q, k, v, do, slopes, kv, g, kind))
    assert not caught(*_mutant_backward(q, k, v, do, slopes, kv, g, "correct"))


def test_p18_nan_and_inf_stay_in_their_head_row_and_column():
    """The recurrence's own confinement, which the GPU test mirrors: a NaN in one head's q
    reaches only that head's output row (q is not part of the state); an Inf in another head's v
    reaches only that head's value column, from its token on, in outputs and state; every other
    head, row and column is unchanged bit for bit."""
    rng = np.random.default_rng(80)
    H, N, d = 4, 40, 8
    q, k, v = (rng.standard_normal((1, H, N, d)).astype(np.float32) for _ in range(3))
    s = np.array([0.9, 0.25, 2.0 ** -8, 0.0])
    o0, kv0, _ = oracle.recurrent(q, k, v, s)
    q1, v1 = q.copy(), v.copy()
    q1[0, 1, 17, 2] = np.nan
    v1[0, 2, 9, 5] = np.inf
    with np.errstate(invalid="ignore"):
        o1, kv1, _ = oracle.recurrent(q1, k, v1, s)
    for h in (0, 3):
        assert np.array_equal(o1[0, h], o0[0, h]) and np.array_equal(kv1[0, h], kv0[0, h])
    rows = np.arange(N) != 17
    assert np.array_equal(o1[0, 1, rows], o0[0, 1, rows]) and np.isnan(o1[0, 1, 17]).all()
    assert np.array_equal(kv1[0, 1], kv0[0, 1])
    cols = np.arange(d) != 5
    assert np.array_equal(o1[0, 2][:, cols], o0[0, 2][:, cols])
    assert np.array_equal(o1[0, 2, :9], o0[0, 2, :9])
    assert not np.isfinite(o1[0, 2, 9:, 5]).any()
    assert np.array_equal(kv1[0, 2][:, cols], kv0[0, 2][:, cols]) and not np.isfinite(kv1[0, 2][:, 5]).any()
