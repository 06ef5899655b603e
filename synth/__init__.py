"""Seeded synthetic inputs for Lightning Attention runs (shared by tests, bench and the oracle's callers).

This module holds no attention arithmetic.  It generates Q, K, V activations
from a counter-based generator (SplitMix64 + Box-Muller, see ``synth.c``),
so any (batch, head, token-range) slice can be regenerated independently,
and it names the workload configurations (shapes, seeds, per-head decay
slopes).  Both the oracle side and the GPU side take their inputs from here;
neither imports the other.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

Q, K, V = 0, 1, 2


def build(verbose: bool = False) -> str:
    """Compile ``synth.c`` into ``libsynth.so`` (host code, gcc + OpenMP)."""
    import subprocess

    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           os.path.join(_HERE, "synth.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_int,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        lib.synth_draw.restype = ctypes.c_uint64
        lib.synth_draw.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_uint64]
        lib.synth_mix64_next.restype = ctypes.c_uint64
        lib.synth_mix64_next.argtypes = [ctypes.c_uint64]
        _lib = lib
    return _lib


def generate(tensor: int, seed: int, d: int, *, b0: int = 0, nb: int = 1, h0: int = 0, nh: int = 1,
             t0: int = 0, nt: int = 1, dtype: str = "f32", out: np.ndarray | None = None) -> np.ndarray:
    """Values of ``tensor`` (Q, K or V) for batches b0.., heads h0.., tokens t0.., as [nb, nh, nt, d].

    ``dtype`` "f32" gives float32 values; "bf16" gives the raw bf16 bits as uint16
    (round-to-nearest-even of the float32 value).
    """
    lib = _load()
    np_dtype = np.uint16 if dtype == "bf16" else np.float32
    if out is None:
        out = np.empty((nb, nh, nt, d), dtype=np_dtype)
    if out.dtype != np_dtype or not out.flags.c_contiguous or out.size != nb * nh * nt * d:
        raise ValueError("out must be a contiguous array of the requested dtype and size")
    rc = lib.synth_fill(out.ctypes.data, 1 if dtype == "bf16" else 0, seed, tensor,
                        b0, nb, h0, nh, t0, nt, d)
    if rc != 0:
        raise ValueError("synth_fill rejected its arguments")
    return out


def raw_draw(seed: int, tensor: int, b: int, h: int, n: int) -> int:
    """The n-th raw 64-bit draw of the (seed, tensor, b, h) stream."""
    return int(_load().synth_draw(seed, tensor, b, h, n))


def splitmix64_next(state: int) -> int:
    """SplitMix64 output for generator state ``state`` (the step adds the golden gamma first)."""
    return int(_load().synth_mix64_next(state))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits with round-to-nearest-even (NaN kept quiet)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7F800000) == 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    quiet = np.where((u[nan] & np.uint64(0x7FFFFF)) != 0, np.uint64(0x40), np.uint64(0))
    r[nan] = ((u[nan] >> np.uint64(16)) | quiet).astype(np.uint16)
    return r


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, element type, seed and per-head decay slopes."""

    name: str
    batch: int
    heads: int
    n: int
    d: int
    dtype: str
    seed: int
    slope_rule: str
    ckpt_every: int = 0
    decode_steps: int = 0
    extra: dict = field(default_factory=dict)

    def slopes(self, heads: int | None = None) -> np.ndarray:
        """Per-head decay slopes s_h (float32); lambda_h = exp(-s_h)."""
        H = self.heads if heads is None else heads
        h = np.arange(H, dtype=np.float64)
        if self.slope_rule == "alibi_heads":      # 2^(-8(h+1)/H) over the heads present
            s = 2.0 ** (-8.0 * (h + 1) / H)
        elif self.slope_rule == "alibi_64":       # 2^(-8(h+1)/64), the 64-head layer
            s = 2.0 ** (-8.0 * (h + 1) / 64.0)
        else:
            raise ValueError(self.slope_rule)
        return s.astype(np.float32)


# The shapes follow the pages' lightning layer (64 heads, head dim 128, contexts up to 1M tokens);
# the values are synthetic stand-ins for that layer's activations.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 512, 64, "f32", 1, "alibi_heads", extra={"block": 64}),
    "share": Workload("share", 1, 8, 32768, 128, "bf16", 2, "alibi_heads", extra={"block": 256}),
    "full": Workload("full", 1, 64, 131072, 128, "bf16", 3, "alibi_64"),
    "full_d64": Workload("full_d64", 1, 64, 131072, 64, "bf16", 3, "alibi_64"),  # the same at d = 64
    "long": Workload("long", 1, 8, 1048576, 128, "bf16", 4, "alibi_heads", ckpt_every=65536),
    "decode": Workload("decode", 128, 64, 4096, 128, "bf16", 5, "alibi_64", decode_steps=1000),
}
