"""GPU parity of the fused prologue/epilogue (SiLU on q/k/v, RMS normalisation over d, sigmoid
gate) in la_prefill_fused and la_decode_fused, against the oracle's step-by-step composition
(oracle.fused: SiLU in float64 on the stored inputs, the recurrence, the norm, the gate).

The bf16 paths round the activated inputs to bf16 before the matrix products (2^-9 relative),
well inside the bf16 bar.

Bars: the parity bars of test_gpu_parity.py hold for the attention output before the epilogue.
The epilogue maps an error e of a pre-epilogue element to about e * scale, with
scale = sigmoid(g) * |weight| / rms_row (rms_row: the row's RMS over d before the norm, the norm's
condition number) with the norm and scale = sigmoid(g) with the gate alone.  The check therefore
divides each element's excess error by its scale and compares it with TOL * RMS of the head's
pre-epilogue output.  With the norm, the tile prefill stores the pre-norm output in the output's
format and a second pass normalises it, so half an ulp of that intermediate value (times scale)
is allowed too, besides half an ulp of the stored result.
"""
import numpy as np
import pytest

import long_context_la_amd as la
import oracle
import synth
from common import TOL, assert_close, half_ulp, inputs, to_device, to_host

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    return torch


def gate_and_weight(seed, shape, d, dtype):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(shape).astype(np.float32) * 2.0
    if dtype == "bf16":
        g = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(g))
    w = (1.0 + 0.5 * rng.standard_normal(d)).astype(np.float32)
    return g, w


def dev(x, dtype, device):
    return to_device(synth.f32_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32), dtype,
                     device)


def activated(exact, silu, dtype):
    """Inputs and SiLU flags for the oracle.  In bf16 the activation's output is a bf16 tensor, as
    the separate activation op of a bf16 model would store it, so the oracle takes SiLU (float64)
    rounded to bf16; in float32 the oracle applies SiLU itself."""
    if dtype != "bf16":
        return list(exact), tuple(silu)
    x = [synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(oracle.silu(e.astype(np.float64)).astype(np.float32)))
         if f else e for e, f in zip(exact, silu)]
    return x, (False, False, False)


def run_prefill_fused(B, H, N, d, dtype, device, silu=(False, False, False), norm=False, weight=False, gate=False,
                      kv_in=None, seed=41):
    torch = _torch()
    exact, raw = inputs(seed, B, H, N, d, dtype)
    slopes = np.array([2.0 ** (-2 - 3 * h) for h in range(H)], dtype=np.float32)
    g, w = gate_and_weight(seed + 1, (B, H, N, d), d, dtype)
    q, k, v = (to_device(x, dtype, device) for x in raw)
    kv = (torch.zeros(B, H, d, d, dtype=torch.float32, device=device) if kv_in is None
          else torch.from_numpy(np.ascontiguousarray(kv_in, np.float32)).to(device))
    o = torch.empty_like(q)
    la.la_prefill_fused(q, k, v, torch.from_numpy(slopes).to(device), kv, o,
                        silu_q=silu[0], silu_k=silu[1], silu_v=silu[2],
                        norm_eps=1e-5 if norm else None,
                        norm_weight=torch.from_numpy(w).to(device) if (norm and weight) else None,
                        gate=dev(g, dtype, device) if gate else None)
    torch.cuda.synchronize()
    x, act = activated(exact, silu, dtype)
    o_ref, kv_ref = oracle.fused(*x, slopes, kv_in=kv_in, silu_q=act[0], silu_k=act[1], silu_v=act[2],
                                 norm_eps=1e-5 if norm else None, norm_weight=w if (norm and weight) else None,
                                 gate=g if gate else None)
    o_pre, _ = oracle.fused(*x, slopes, kv_in=kv_in, silu_q=act[0], silu_k=act[1], silu_v=act[2])
    what = f"(N={N}, d={d}, {dtype}, silu={silu}, norm={norm}, weight={weight}, gate={gate})"
    assert_close_epilogue(to_host(o), o_ref, o_pre, dtype, "O " + what, norm, 1e-5, w if (norm and weight) else None,
                          g if gate else None, intermediate=norm)
    assert_close(kv.cpu().numpy(), kv_ref, dtype, "KV " + what)


def assert_close_epilogue(got, want, o_pre, dtype, what, norm, eps, weight, gate, intermediate):
    """Parity of an output after the epilogue, measured in the pre-epilogue domain (module doc)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    o_pre = np.asarray(o_pre, np.float64)
    scale = np.ones_like(o_pre)
    if norm:
        rrow = np.sqrt(np.mean(o_pre ** 2, axis=-1, keepdims=True) + eps)
        scale = scale / rrow * (np.abs(np.asarray(weight, np.float64)) if weight is not None else 1.0)
    if gate is not None:
        scale = scale * oracle.sigmoid(np.asarray(gate, np.float64))
    allow = half_ulp(got, dtype)
    if intermediate:
        allow = allow + half_ulp(o_pre, dtype) * scale
    excess = np.maximum(np.abs(got - want) - allow, 0.0) / scale
    worst = 0.0
    for b in range(want.shape[0]):
        for h in range(want.shape[1]):
            rms = float(np.sqrt(np.mean(o_pre[b, h] ** 2)))
            worst = max(worst, float(excess[b, h].max()) / max(rms, 1e-30))
    assert worst <= TOL[dtype], f"{what}: max excess error / RMS (pre-epilogue) = {worst:.3e} > {TOL[dtype]:.0e}"
    return worst


CASES = [("bf16", 128), ("f32", 128), ("f32", 64), ("bf16", 64)]


@pytest.mark.parametrize("dtype,d", CASES)
@pytest.mark.parametrize("norm,weight,gate", [(True, True, True), (True, False, False), (False, False, True)])
def test_epilogue_on_the_kernels_own_output(device, dtype, d, norm, weight, gate):
    """The epilogue alone, held to its definition element by element: the fused call's output
    against the oracle's RMS norm and sigmoid gate applied in float64 to the same kernels' output
    without the epilogue (the kernels are deterministic, so that output is exactly what the
    epilogue received, or for the gate in the store its rounding).  Bar: one ulp of the result,
    plus for float32 2^-14 relative (the epilogue's float32 sum of squares, square root and
    exponential), plus, for the gate in the store, half an ulp of the pre-epilogue value times
    the gate (that value is rounded in the run without the epilogue, not in the fused one)."""
    torch = _torch()
    B, H, N = 1, 2, 333
    exact, raw = inputs(47, B, H, N, d, dtype)
    slopes = torch.from_numpy(np.array([2.0 ** -2, 2.0 ** -8], dtype=np.float32)).to(device)
    g, w = gate_and_weight(48, (B, H, N, d), d, dtype)
    q, k, v = (to_device(x, dtype, device) for x in raw)

    def run(**kw):
        kv = torch.zeros(B, H, d, d, dtype=torch.float32, device=device)
        o = torch.empty_like(q)
        la.la_prefill_fused(q, k, v, slopes, kv, o, silu_q=True, silu_k=True, silu_v=True, **kw)
        torch.cuda.synchronize()
        return to_host(o).astype(np.float64)

    pre = run()
    got = run(norm_eps=1e-5 if norm else None, norm_weight=torch.from_numpy(w).to(device) if weight else None,
              gate=dev(g, dtype, device) if gate else None)
    want = oracle.rms_norm(pre, 1e-5, w if weight else None) if norm else pre
    sig = oracle.sigmoid(g) if gate else 1.0
    want = want * sig
    allow = 2.0 * half_ulp(got, dtype) + (2.0 ** -14 * np.abs(want) if dtype == "f32" else 0.0)
    if gate and not norm:
        allow = allow + half_ulp(pre, dtype) * sig
    excess = np.abs(got - want) - allow
    i = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess.max() <= 0.0, (f"epilogue (norm={norm}, weight={weight}, gate={gate}, {dtype}, d={d}) at {i}: "
                                 f"got {got[i]:.8g}, want {want[i]:.8g}, allowed {allow[i]:.3g}")


@pytest.mark.parametrize("dtype,d", CASES)
def test_prologue_silu_qk(device, dtype, d):
    run_prefill_fused(1, 2, 200, d, dtype, device, silu=(True, True, False))


@pytest.mark.parametrize("dtype,d", CASES)
def test_prologue_and_epilogue_all(device, dtype, d):
    run_prefill_fused(2, 2, 333, d, dtype, device, silu=(True, True, True), norm=True, weight=True, gate=True)


@pytest.mark.parametrize("dtype,d", CASES)
def test_gate_only_in_the_store(device, dtype, d):
    run_prefill_fused(1, 3, 130, d, dtype, device, gate=True)


def test_norm_only_without_weight(device):
    run_prefill_fused(1, 2, 257, 128, "bf16", device, norm=True)


def test_fused_chunked_with_incoming_state(device):
    # 2 heads x 4 slices do not fill the GPU, so the 5000 tokens are cut into chunks
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, 2, 5000, 128) < 5000
    kv_in = np.random.default_rng(3).standard_normal((1, 2, 128, 128)).astype(np.float32)
    run_prefill_fused(1, 2, 5000, 128, "bf16", device, silu=(True, False, True), norm=True, weight=True, gate=True,
                      kv_in=kv_in)


@pytest.mark.parametrize("i", range(10))
def test_prefill_fused_sweep(device, i):
    # seeded random fused prefills: SiLU on any subset of q, k, v, norm with or without a weight,
    # gate, dtype and d, batch/heads/length (chunked when long), incoming states
    rng = np.random.default_rng(7000 + i)
    dtype, d = [("bf16", 128), ("f32", 128), ("f32", 64), ("bf16", 64)][rng.integers(4)]
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    N = int(rng.integers(1, 3000))
    silu = tuple(bool(x) for x in rng.random(3) < 0.5)
    norm = bool(rng.random() < 0.5)
    weight = norm and bool(rng.random() < 0.5)
    gate = bool(rng.random() < 0.5)
    kv_in = rng.standard_normal((B, H, d, d)).astype(np.float32) if rng.random() < 0.5 else None
    run_prefill_fused(B, H, N, d, dtype, device, silu=silu, norm=norm, weight=weight, gate=gate, kv_in=kv_in,
                      seed=7100 + i)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_decode_fused(device, dtype, d):
    torch = _torch()
    B, H, steps = 3, 4, 5
    slopes = np.array([2.0 ** (-1 - h) for h in range(H)], dtype=np.float32)
    ts = torch.from_numpy(slopes).to(device)
    kv0 = np.random.default_rng(7).standard_normal((B, H, d, d)).astype(np.float32)
    kv = torch.from_numpy(kv0.copy()).to(device)
    kv_ref = kv0.astype(np.float64)
    w = (1.0 + 0.3 * np.random.default_rng(8).standard_normal(d)).astype(np.float32)
    for s in range(steps):
        exact, raw = inputs(50 + s, B, H, 1, d, dtype)
        g, _ = gate_and_weight(60 + s, (B, H, d), d, dtype)
        q, k, v = (to_device(np.ascontiguousarray(x[:, :, 0]), dtype, device) for x in raw)
        o = torch.empty_like(q)
        la.la_decode_fused(q, k, v, ts, kv, o, silu_q=True, silu_k=True, silu_v=(s % 2 == 0), norm_eps=1e-6,
                           norm_weight=torch.from_numpy(w).to(device), gate=dev(g, dtype, device))
        torch.cuda.synchronize()
        x, act = activated([e[:, :, 0] for e in exact], (True, True, s % 2 == 0), dtype)
        qa, ka, va = (oracle.silu(e) if f else e for e, f in zip(x, act))
        o_pre = oracle.decode_step(qa, ka, va, slopes, kv_ref)
        o_ref = oracle.rms_norm(o_pre, 1e-6, w) * oracle.sigmoid(g)
        # decode normalises in registers: no intermediate rounding
        assert_close_epilogue(to_host(o), o_ref, o_pre, dtype, f"decode fused O step {s}", True, 1e-6, w, g,
                              intermediate=False)
    assert_close(kv.cpu().numpy(), kv_ref, dtype, "decode fused KV")


@pytest.mark.parametrize("i", range(8))
def test_decode_sweep(device, i):
    # seeded random decode runs: batch, heads, dtype and d, steps, and per step a random choice of
    # the plain step or the fused one (SiLU subset, norm with or without a weight, gate)
    torch = _torch()
    rng = np.random.default_rng(8000 + i)
    dtype, d = [("bf16", 128), ("f32", 128), ("f32", 64), ("bf16", 64)][rng.integers(4)]
    B, H, steps = int(rng.integers(1, 5)), int(rng.integers(1, 6)), int(rng.integers(1, 6))
    slopes = np.exp2(-rng.uniform(0.5, 9, H)).astype(np.float32)
    ts = torch.from_numpy(slopes).to(device)
    kv0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    kv = torch.from_numpy(kv0.copy()).to(device)
    kv_ref = kv0.astype(np.float64)
    w = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    for s in range(steps):
        exact, raw = inputs(8100 + 10 * i + s, B, H, 1, d, dtype)
        q, k, v = (to_device(np.ascontiguousarray(x[:, :, 0]), dtype, device) for x in raw)
        o = torch.empty_like(q)
        what = f"case {i} step {s} ({dtype}, d={d}, B={B}, H={H})"
        if rng.random() < 0.3:
            la.la_decode(q, k, v, ts, kv, o)
            torch.cuda.synchronize()
            o_ref = oracle.decode_step(*(e[:, :, 0] for e in exact), slopes, kv_ref)
            assert_close(to_host(o)[:, :, None], o_ref[:, :, None], dtype, "decode O " + what, stored=dtype)
            continue
        silu = tuple(bool(x) for x in rng.random(3) < 0.5)
        norm = bool(rng.random() < 0.5)
        weight = norm and bool(rng.random() < 0.5)
        gate = bool(rng.random() < 0.5)
        g, _ = gate_and_weight(8200 + 10 * i + s, (B, H, d), d, dtype)
        la.la_decode_fused(q, k, v, ts, kv, o, silu_q=silu[0], silu_k=silu[1], silu_v=silu[2],
                           norm_eps=1e-6 if norm else None,
                           norm_weight=torch.from_numpy(w).to(device) if weight else None,
                           gate=dev(g, dtype, device) if gate else None)
        torch.cuda.synchronize()
        x, act = activated([e[:, :, 0] for e in exact], silu, dtype)
        qa, ka, va = (oracle.silu(e) if f else e for e, f in zip(x, act))
        o_pre = oracle.decode_step(qa, ka, va, slopes, kv_ref)
        o_ref = o_pre
        if norm:
            o_ref = oracle.rms_norm(o_ref, 1e-6, w if weight else None)
        if gate:
            o_ref = o_ref * oracle.sigmoid(g)
        assert_close_epilogue(to_host(o), o_ref, o_pre, dtype, "decode fused O " + what, norm, 1e-6,
                              w if weight else None, g if gate else None, intermediate=False)
    assert_close(kv.cpu().numpy(), kv_ref, dtype, f"decode KV case {i}")
