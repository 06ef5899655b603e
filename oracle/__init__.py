"""Plain, slow, fp64 reference for Lightning Attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the GPU path (no
kernels, headers, helpers or constants) and never imports it.

Source of the method: the page "MiniMax-01: Scaling Foundation Models with
Lightning Attention | Summary" --
  * section 2.2 (Linear Attention): attention is evaluated in the reordered
    form Q(K^T V) so no n x n matrix is built; causal prediction makes the
    key-value summary cumulative; the sequence is split into tiles, each tile
    takes a masked-attention term from inside the tile plus a term from the
    accumulated key-value state of all earlier tiles, and the state is then
    updated (their Algorithm 1, whose listing is not on the page); the
    derivation leaves out normalisation, SiLU and gating; work is
    O(n d^2 + n B d).
  * section 3.2 (Long Context Optimization): LASP+ turns the serial passing of
    the state between sequence partitions into local prefix summaries that
    are gathered and combined into the global prefixes.
The decay mask M[t][s] = lambda^(t-s) (s <= t), lambda_h = exp(-s_h), is our
reading of "masked attention" (with s_h = 0 it is the plain causal mask).

Forms provided (each a separate, literal transcription of one definition):
  recurrent  -- token-by-token state recurrence (C, ``la_oracle.c``)
  quadratic  -- the n x n masked form O = [(Q K^T) . M] V (+ incoming state term)
  blocked    -- tile-by-tile: intra-tile masked term + inter-tile state term,
                then the state update (the page's Algorithm 1 as described)
  decode     -- one step of the recurrence
  chunk states / LASP+ combine -- local summaries from a zero state, then
                prefixes P_{j+1} = lambda^{C_j} P_j + S_j.
  backward   -- gradients of a scalar loss through the recurrence (dq, dk, dv and the
                incoming state's gradient, given dL/dO and optionally dL/dKV_final), as the
                reverse-order state recurrence and as the n x n masked form; LASP+'s
                training side (section 3.2) runs this reverse recurrence across partitions.
  prologue / epilogue -- the pieces the derivation leaves out (section 2.2
                names normalisation, SiLU and gating; section 3.3 fuses such
                memory-bound steps into the attention kernels): SiLU on q, k, v
                before attention, and after it an RMS normalisation over the
                head dimension followed by an elementwise sigmoid gate.
Every power of lambda is exp(-s*k) with k >= 0.  No part is "parity unpinned":
the pins live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_la.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle (gcc, OpenMP, no fast-math)."""
    import subprocess

    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           os.path.join(_HERE, "la_oracle.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
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
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_recurrent.restype = None
        lib.oracle_recurrent.argtypes = [p, p, p, i64, i64, i64, p, p, p, p, p, i64]
        lib.oracle_decode_step.restype = None
        lib.oracle_decode_step.argtypes = [p, p, p, i64, i64, p, p, p]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _rows(slopes, B, H):
    """Per-(batch, head) slope rows from a per-head vector."""
    s = np.asarray(slopes, dtype=np.float64).reshape(-1)
    if s.size != H:
        raise ValueError("one slope per head expected")
    return np.ascontiguousarray(np.tile(s, B))


def recurrent(q, k, v, slopes, kv_in=None, want_o=True, ckpt_every=0):
    """Token-by-token recurrence.  q, k, v: [B, H, N, d] (values exact in float32).

    Returns (o [B,H,N,d] float64 or None, kv_out [B,H,d,d] float64, ckpt or None), where
    ckpt[b,h,m] is the state after token (m+1)*ckpt_every - 1.
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, N, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one shape")
    s = _rows(slopes, B, H)
    kin = None if kv_in is None else np.ascontiguousarray(kv_in, dtype=np.float64).reshape(B * H, d, d)
    o = np.empty((B, H, N, d), dtype=np.float64) if want_o else None
    kv_out = np.empty((B, H, d, d), dtype=np.float64)
    n_ck = N // ckpt_every if ckpt_every > 0 else 0
    ck = np.empty((B, H, n_ck, d, d), dtype=np.float64) if n_ck > 0 else None
    _load().oracle_recurrent(_ptr(q), _ptr(k), _ptr(v), B * H, N, d, _ptr(s), _ptr(kin), _ptr(o),
                             _ptr(kv_out), _ptr(ck), ckpt_every if n_ck > 0 else 0)
    return o, kv_out, ck


def decode_step(q, k, v, slopes, kv):
    """One decode step, in place on ``kv`` ([B,H,d,d] float64).  q,k,v: [B,H,d].  Returns o [B,H,d]."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, d = q.shape
    if kv.dtype != np.float64 or not kv.flags.c_contiguous or kv.shape != (B, H, d, d):
        raise ValueError("kv must be a contiguous float64 [B,H,d,d] array")
    s = _rows(slopes, B, H)
    o = np.empty((B, H, d), dtype=np.float64)
    _load().oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), B * H, d, _ptr(s), _ptr(kv), _ptr(o))
    return o


def decay_powers(s, exps):
    """lambda^e = exp(-s*e) for integer e >= 0 (never a negative power)."""
    e = np.asarray(exps, dtype=np.float64)
    if np.any(e < 0):
        raise ValueError("negative decay exponent")
    return np.exp(-float(s) * e)


def quadratic(q, k, v, slopes, kv_in=None):
    """The n x n form: O = [(Q K^T) . M] V + diag(lambda^(t+1)) Q KV_in, M[t][s] = lambda^(t-s) for s <= t.

    Final state: lambda^N KV_in + K^T diag(lambda^(N-1-s)) V.  Returns (o, kv_out), float64.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, d = q.shape
    t = np.arange(N)
    diff = t[:, None] - t[None, :]
    o = np.empty((B, H, N, d))
    kv_out = np.empty((B, H, d, d))
    for b in range(B):
        for h in range(H):
            s = float(slopes[h])
            M = np.where(diff >= 0, np.exp(-s * np.maximum(diff, 0)), 0.0)
            Q, K, Vm = q[b, h], k[b, h], v[b, h]
            o[b, h] = ((Q @ K.T) * M) @ Vm
            w = decay_powers(s, N - 1 - t)
            kv_out[b, h] = (K * w[:, None]).T @ Vm
            if kv_in is not None:
                KV0 = np.asarray(kv_in[b, h], dtype=np.float64)
                o[b, h] += decay_powers(s, t + 1)[:, None] * (Q @ KV0)
                kv_out[b, h] += decay_powers(s, N) * KV0
    return o, kv_out


def blocked(q, k, v, slopes, block, kv_in=None):
    """Tile-by-tile evaluation (section 2.2's Algorithm 1 as the page describes it).

    For tile i holding tokens iB..iB+L-1 (L = B except a short last tile) with
    incoming state KV:
        o_{iB+r} = lambda^(r+1) q_r KV + sum_{c<=r} lambda^(r-c) (q_r . k_c) v_c
        KV      <- lambda^L KV + sum_{c<L} lambda^(L-1-c) k_c^T v_c
    Returns (o, kv_out), float64.
    """
    if block < 1:
        raise ValueError("block must be >= 1")
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, d = q.shape
    o = np.empty((B, H, N, d))
    kv_out = np.empty((B, H, d, d))
    for b in range(B):
        for h in range(H):
            s = float(slopes[h])
            KV = np.zeros((d, d)) if kv_in is None else np.array(kv_in[b, h], dtype=np.float64)
            for start in range(0, N, block):
                L = min(block, N - start)
                Qi, Ki, Vi = q[b, h, start:start + L], k[b, h, start:start + L], v[b, h, start:start + L]
                r = np.arange(L)
                diff = r[:, None] - r[None, :]
                Mi = np.where(diff >= 0, np.exp(-s * np.maximum(diff, 0)), 0.0)
                intra = ((Qi @ Ki.T) * Mi) @ Vi
                inter = decay_powers(s, r + 1)[:, None] * (Qi @ KV)
                o[b, h, start:start + L] = intra + inter
                KV = decay_powers(s, L) * KV + (Ki * decay_powers(s, L - 1 - r)[:, None]).T @ Vi
            kv_out[b, h] = KV
    return o, kv_out


def chunk_local_states(k, v, slopes, chunk_lens):
    """LASP+ local summaries: for each chunk j the state of its tokens alone from a zero state.

    chunk_lens: lengths C_j summing to N.  Returns [B, H, n_chunks, d, d] float64.
    """
    k, v = np.asarray(k, dtype=np.float64), np.asarray(v, dtype=np.float64)
    B, H, N, d = k.shape
    if sum(chunk_lens) != N:
        raise ValueError("chunk lengths must sum to N")
    S = np.empty((B, H, len(chunk_lens), d, d))
    for b in range(B):
        for h in range(H):
            s = float(slopes[h])
            start = 0
            for j, C in enumerate(chunk_lens):
                c = np.arange(C)
                Kc, Vc = k[b, h, start:start + C], v[b, h, start:start + C]
                S[b, h, j] = (Kc * decay_powers(s, C - 1 - c)[:, None]).T @ Vc
                start += C
    return S


def lasp_plus_prefixes(local_states, slopes, chunk_lens, kv_in=None):
    """Combine local summaries into global prefixes: P_0 = KV_in, P_{j+1} = lambda^{C_j} P_j + S_j.

    Returns [B, H, n_chunks + 1, d, d]; entry j is the state entering chunk j, the last is the final state.
    """
    S = np.asarray(local_states, dtype=np.float64)
    B, H, n, d, _ = S.shape
    P = np.empty((B, H, n + 1, d, d))
    for b in range(B):
        for h in range(H):
            s = float(slopes[h])
            P[b, h, 0] = 0.0 if kv_in is None else kv_in[b, h]
            for j in range(n):
                P[b, h, j + 1] = decay_powers(s, chunk_lens[j]) * P[b, h, j] + S[b, h, j]
    return P


# ---------------------------------------------------------------- prologue / epilogue
# Our reading of the pieces the derivation omits (section 2.2 lists them without formulas):
#   SiLU(x) = x * sigmoid(x), elementwise, applied to q, k and/or v before attention;
#   Norm(o) = o / sqrt(mean_e(o_e^2) + eps) * w_e, over the d features of one (token, head),
#             the plain RMS normalisation, with an optional per-feature weight w (default 1);
#   gate:     o * sigmoid(g) for a gate tensor g of the output's shape.

def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    """x * sigmoid(x) in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def rms_norm(o, eps, weight=None):
    """RMS normalisation over the last axis (the head dimension) in float64."""
    o = np.asarray(o, dtype=np.float64)
    r = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return r if weight is None else r * np.asarray(weight, dtype=np.float64)


def fused(q, k, v, slopes, kv_in=None, silu_q=False, silu_k=False, silu_v=False, norm_eps=None,
          norm_weight=None, gate=None):
    """The attention of ``recurrent`` wrapped in the optional prologue and epilogue, step by step:
    SiLU on the selected inputs, the recurrence, RMS normalisation (when norm_eps is given), then
    the sigmoid gate (when gate is given).  Returns (o, final state)."""
    q = silu(q) if silu_q else np.asarray(q, dtype=np.float64)
    k = silu(k) if silu_k else np.asarray(k, dtype=np.float64)
    v = silu(v) if silu_v else np.asarray(v, dtype=np.float64)
    o, kv, _ = recurrent(q, k, v, slopes, kv_in=kv_in)
    if norm_eps is not None:
        o = rms_norm(o, norm_eps, norm_weight)
    if gate is not None:
        o = o * sigmoid(gate)
    return o, kv



# ---------------------------------------------------------------- backward (training)
# For a scalar loss L with dO = dL/dO and G_out = dL/dKV_final (zero when not given), differentiate
#     KV_t = lambda KV_{t-1} + k_t^T v_t,   o_t = q_t KV_t,   KV_{-1} = KV_in.
# The gradient reaching the state after token t, G_t = dL/dKV_t (all paths), obeys the reverse
# recurrence
#     G_{N-1} = q_{N-1}^T do_{N-1} + G_out,   G_t = q_t^T do_t + lambda G_{t+1},
# and then  dq_t = do_t KV_t^T,  dk_t = v_t G_t^T,  dv_t = k_t G_t,  dL/dKV_in = lambda G_0
# (= G_out for N = 0).  The slopes are constants (not differentiated).

def backward_recurrent(q, k, v, do, slopes, kv_in=None, dkv_out=None):
    """Token-by-token form: a forward pass for the states KV_t, then the reverse pass for G_t.

    q, k, v, do: [B, H, N, d]; kv_in, dkv_out: [B, H, d, d] or None.
    Returns (dq, dk, dv, dkv_in), float64."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, N, d = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    dkv_in = np.empty((B, H, d, d))
    for b in range(B):
        for h in range(H):
            lam = math.exp(-float(slopes[h]))
            KV = np.zeros((d, d)) if kv_in is None else np.array(kv_in[b, h], dtype=np.float64)
            for t in range(N):
                KV = lam * KV + np.outer(k[b, h, t], v[b, h, t])
                dq[b, h, t] = do[b, h, t] @ KV.T
            # `arriving` is what later tokens (or G_out, for the last one) pass back to G_t
            arriving = np.zeros((d, d)) if dkv_out is None else np.array(dkv_out[b, h], dtype=np.float64)
            for t in range(N - 1, -1, -1):
                G = np.outer(q[b, h, t], do[b, h, t]) + arriving
                dk[b, h, t] = v[b, h, t] @ G.T
                dv[b, h, t] = k[b, h, t] @ G
                arriving = lam * G
            dkv_in[b, h] = arriving
    return dq, dk, dv, dkv_in


def backward_quadratic(q, k, v, do, slopes, kv_in=None, dkv_out=None):
    """The n x n form of the same gradients, with A = (dO V^T) . M and P = (Q K^T) . M:
        dQ = A K + diag(lambda^(t+1)) dO KV_in^T
        dK = A^T Q + diag(lambda^(N-1-s)) V G_out^T
        dV = P^T dO + diag(lambda^(N-1-s)) K G_out
        dKV_in = Q^T diag(lambda^(t+1)) dO + lambda^N G_out.
    Returns (dq, dk, dv, dkv_in), float64."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, N, d = q.shape
    t = np.arange(N)
    diff = t[:, None] - t[None, :]
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    dkv_in = np.empty((B, H, d, d))
    for b in range(B):
        for h in range(H):
            s = float(slopes[h])
            M = np.where(diff >= 0, np.exp(-s * np.maximum(diff, 0)), 0.0)
            Q, K, Vm, dO = q[b, h], k[b, h], v[b, h], do[b, h]
            A = (dO @ Vm.T) * M
            P = (Q @ K.T) * M
            dq[b, h] = A @ K
            dk[b, h] = A.T @ Q
            dv[b, h] = P.T @ dO
            dkv_in[b, h] = (Q * decay_powers(s, t + 1)[:, None]).T @ dO
            if kv_in is not None:
                dq[b, h] += decay_powers(s, t + 1)[:, None] * (dO @ np.asarray(kv_in[b, h], dtype=np.float64).T)
            if dkv_out is not None:
                Gout = np.asarray(dkv_out[b, h], dtype=np.float64)
                w = decay_powers(s, N - 1 - t)[:, None]
                dk[b, h] += w * (Vm @ Gout.T)
                dv[b, h] += w * (K @ Gout)
                dkv_in[b, h] += decay_powers(s, N) * Gout
    return dq, dk, dv, dkv_in
