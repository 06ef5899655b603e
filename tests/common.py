"""Shared helpers for the GPU tests: seeded inputs as numpy (exact values) and as device
tensors, the per-(batch, head) error measure, and thin calls into the oracle."""
from __future__ import annotations

import numpy as np

import synth

# Parity bars, per (batch, head) slice, for outputs and states alike:
#     max over elements of max(|gpu - oracle| - half_ulp(gpu), 0)  <=  TOL * RMS(oracle)
# TOL bounds the computation (float32 accumulation of float32 or bfloat16 inputs); half an
# ulp of the storage format of the GPU's result is allowed on top, because the oracle's
# exact value has to be rounded to be stored at all (for bf16 outputs that rounding alone
# reaches ~2.7e-2 of a fast-decaying head's RMS, so no bf16 result could meet a bar without it).
TOL = {"f32": 1e-4, "bf16": 2e-2}
MANTISSA_BITS = {"f32": 24, "bf16": 8}


def inputs(seed, B, H, N, d, dtype, t0=0):
    """Q, K, V for batches 0..B-1, heads 0..H-1, tokens t0..t0+N-1.

    Returns (exact float32 values, raw arrays as stored on the device: float32 or bf16 bits)."""
    raw = [synth.generate(t, seed, d, nb=B, nh=H, t0=t0, nt=N, dtype=dtype) for t in (synth.Q, synth.K, synth.V)]
    exact = [synth.bf16_bits_to_f32(x) if dtype == "bf16" else x for x in raw]
    return exact, raw


def to_device(raw, dtype, device):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(raw)).to(device)


def to_host(t):
    import torch

    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def half_ulp(x, stored):
    """Half a unit in the last place of |x| in the storage format ``stored`` ("f32" or "bf16")."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - MANTISSA_BITS[stored]), 0.0)


def head_err(got, want, stored="f32"):
    """max over leading (b, h) slices of max(|got - want| - half_ulp(got), 0) / RMS(want)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    B, H = want.shape[:2]
    worst = 0.0
    for b in range(B):
        for h in range(H):
            if want[b, h].size == 0:
                continue
            rms = float(np.sqrt(np.mean(want[b, h] ** 2)))
            excess = np.maximum(np.abs(got[b, h] - want[b, h]) - half_ulp(got[b, h], stored), 0.0)
            worst = max(worst, float(excess.max()) / max(rms, 1e-30))
    return worst


def assert_close(got, want, dtype, what, stored="f32"):
    """Parity bar of ``dtype`` ("f32"/"bf16" inputs) for a result stored as ``stored``."""
    e = head_err(got, want, stored)
    assert e <= TOL[dtype], f"{what}: max excess error / RMS = {e:.3e} > {TOL[dtype]:.0e}"
    return e
