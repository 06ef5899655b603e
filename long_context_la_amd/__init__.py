"""Lightning Attention on MI355X: thin Python binding over liblightning_la.so.

The C ABI (include/la.h) is the product boundary; this module only marshals
arguments: it takes torch tensors on the GPU, passes their device pointers,
strides and torch's current HIP stream, and raises on a non-OK status.  Every
step of the computation runs in the library's gfx950 kernels -- there is no
fallback: if the library is missing, every call raises.

Names follow the C entry points: la_state_init, la_prefill (with checkpoints and
chunk_tokens), la_prefill_noalloc, la_prefill_workspace_size,
la_prefill_chunk_tokens, la_prefill_varlen, la_prefill_varlen_workspace_size,
la_prefill_varlen_chunk_tokens, la_decode, la_prefill_fused, la_decode_fused,
la_backward, la_backward_varlen and their workspace sizes, la_status_string,
la_last_error.  Every wrapper checks shapes, dtypes, strides and the state,
checkpoint and slope buffers before anything is launched, since the C ABI sees
raw pointers only.  mixed_step issues a decode group and a varlen prefill group
(two library calls, nothing else) on the current stream or on two streams;
lightning_attention and lightning_attention_varlen wrap the prefill and its
backward as differentiable ops.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblightning_la.so")

LA_OK = 0
LA_ERR_INVALID_ARGUMENT = 1
LA_ERR_UNSUPPORTED = 2
LA_ERR_WORKSPACE = 3
LA_ERR_DEVICE = 4
LA_ERR_INTERNAL = 5
LA_F32 = 0
LA_BF16 = 1
LA_NOALLOC_SCRATCH_BYTES = 96 << 20  # include/la.h: the allocation-free prefill's per-GPU array

EXPORTED = ["la_state_init", "la_prefill_chunk_tokens", "la_prefill_workspace_size",
            "la_prefill_workspace_size_ex", "la_prefill", "la_prefill_ex",
            "la_prefill_varlen_workspace_size", "la_prefill_varlen_workspace_size_ex",
            "la_prefill_varlen_chunk_tokens", "la_prefill_varlen", "la_prefill_varlen_ex", "la_decode",
            "la_prefill_fused", "la_decode_fused", "la_backward_workspace_size", "la_backward",
            "la_backward_varlen_workspace_size", "la_backward_varlen",
            "la_prefill_noalloc", "la_status_string", "la_last_error"]

LA_SILU_Q = 1
LA_SILU_K = 2
LA_SILU_V = 4
LA_NORM = 8
LA_GATE = 16


class la_fusion(ctypes.Structure):
    """The C struct la_fusion (include/la.h)."""
    _fields_ = [("flags", ctypes.c_uint32), ("gate", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float)]

_lib = None


class LAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {detail} (status {status})")
        self.status = status


def lib():
    """The loaded library with ctypes signatures set (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(there is no non-HIP fallback)")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    L.la_state_init.restype = i32
    L.la_state_init.argtypes = [p, p, i64, i64, i64, p]
    L.la_prefill_chunk_tokens.restype = i64
    L.la_prefill_chunk_tokens.argtypes = [i32, i64, i64, i64, i64]
    L.la_prefill_workspace_size.restype = sz
    L.la_prefill_workspace_size.argtypes = [i32, i64, i64, i64, i64]
    L.la_prefill_workspace_size_ex.restype = sz
    L.la_prefill_workspace_size_ex.argtypes = [i32, i64, i64, i64, i64, i64]
    L.la_prefill.restype = i32
    L.la_prefill.argtypes = [i32, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p, p, i64, p, sz, p]
    L.la_prefill_noalloc.restype = i32
    L.la_prefill_noalloc.argtypes = [i32, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p, p, i64, p]
    L.la_prefill_ex.restype = i32
    L.la_prefill_ex.argtypes = [i32, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p, p, i64, i64, p, sz, p]
    L.la_prefill_varlen_workspace_size.restype = sz
    L.la_prefill_varlen_workspace_size.argtypes = [i32, i64, p, i64, i64]
    L.la_prefill_varlen_workspace_size_ex.restype = sz
    L.la_prefill_varlen_workspace_size_ex.argtypes = [i32, i64, p, i64, i64, i64]
    L.la_prefill_varlen_chunk_tokens.restype = i64
    L.la_prefill_varlen_chunk_tokens.argtypes = [i32, i64, p, i64, i64]
    L.la_prefill_varlen.restype = i32
    L.la_prefill_varlen.argtypes = [i32, p, p, p, p, i64, p, i64, i64, i64, i64, p, p, p, sz, p]
    L.la_prefill_varlen_ex.restype = i32
    L.la_prefill_varlen_ex.argtypes = [i32, p, p, p, p, i64, p, i64, i64, i64, i64, p, p, i64, p, sz, p]
    L.la_prefill_fused.restype = i32
    L.la_prefill_fused.argtypes = [i32, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p,
                                   ctypes.POINTER(la_fusion), p, sz, p]
    L.la_decode_fused.restype = i32
    L.la_decode_fused.argtypes = [i32, p, p, p, p, i64, i64, i64, p, p, ctypes.POINTER(la_fusion), p]
    L.la_backward_workspace_size.restype = sz
    L.la_backward_workspace_size.argtypes = [i32, i64, i64, i64, i64]
    L.la_backward.restype = i32
    L.la_backward.argtypes = [i32, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, p, p, p, p, p, p, p, p, sz, p]
    L.la_backward_varlen_workspace_size.restype = sz
    L.la_backward_varlen_workspace_size.argtypes = [i32, i64, p, i64, i64]
    L.la_backward_varlen.restype = i32
    L.la_backward_varlen.argtypes = [i32, p, p, p, p, i64, p, i64, i64, i64, i64, p, p, p, p, p, p, p, p, sz, p]
    L.la_decode.restype = i32
    L.la_decode.argtypes = [i32, p, p, p, p, i64, i64, i64, p, p, p]
    L.la_status_string.restype = ctypes.c_char_p
    L.la_status_string.argtypes = [i32]
    L.la_last_error.restype = ctypes.c_char_p
    L.la_last_error.argtypes = []
    _lib = L
    return L


def _rows_disjoint(t) -> bool:
    """True when no two rows (all indices but the last, which is contiguous) of the strided tensor
    t share an element: with the dimensions longer than one sorted by stride, each stride is at
    least the span of the faster ones (the same rule the library applies to its outputs)."""
    if t.is_contiguous():
        return True
    span = t.shape[-1]
    for st, n in sorted((st, n) for st, n in zip(t.stride()[:-1], t.shape[:-1]) if n > 1):
        if st < span:
            return False
        span += st * (n - 1)
    return True


def _check_f32(t, shape, name):
    """t is None or a contiguous float32 tensor of exactly this shape (states, checkpoints)."""
    import torch

    if t is None:
        return
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)} "
                         f"(got {t.dtype}, {tuple(t.shape)}, contiguous={t.is_contiguous()})")


def _check_slopes(slopes, heads):
    import torch

    if (slopes.dtype != torch.float32 or slopes.dim() != 1 or slopes.numel() != heads
            or not slopes.is_contiguous()):
        raise ValueError(f"slopes must be a contiguous 1-D float32 tensor of {heads} elements "
                         f"(got {slopes.dtype}, {tuple(slopes.shape)})")


def _check_qkv(q, k, v, ndim):
    shape, dtype = q.shape, q.dtype
    if len(shape) != ndim:
        raise ValueError(f"q, k, v must be {ndim}-D")
    if k.shape != shape or v.shape != shape or k.dtype != dtype or v.dtype != dtype:
        raise ValueError("q, k, v must share shape and dtype")
    if not _same_strides(k, q) or not _same_strides(v, q) or q.stride(-1) != 1:
        raise ValueError("q, k, v must share strides with a contiguous last dimension")


def _check_out(t, q, name):
    """An output (or gate) tensor laid out like q; outputs must also have disjoint rows."""
    if t is None:
        return
    if t.shape != q.shape or not _same_strides(t, q) or t.dtype != q.dtype:
        raise ValueError(f"{name} must match q in shape, strides and dtype")
    if not _rows_disjoint(t):
        raise ValueError(f"the rows of {name} overlap (a zero stride on a dimension longer than one, or "
                         "strides that map two rows onto shared elements)")


def _dense_layout(*ts):
    """The inputs as they are when their rows are disjoint, else contiguous copies (an expanded
    view has stride 0, and outputs allocated with its strides would overlap)."""
    if all(_rows_disjoint(t) for t in ts):
        return ts
    return tuple(t.contiguous() for t in ts)


def _on_stream(stream, *ts):
    """Temporaries used by work enqueued on a stream other than the current one are recorded on
    it, so the caching allocator does not hand their memory out again before that work is done."""
    import torch

    if stream is None:
        return
    cur = torch.cuda.current_stream(stream.device)
    if stream == cur:
        return
    for t in ts:
        if t is not None:
            t.record_stream(stream)


def _same_strides(t, ref) -> bool:
    """Same element strides as ref on every dimension longer than 1 (a dimension of size 1 is
    never stepped over, so its stride does not matter; the library takes ref's)."""
    ts, rs = t.stride(), ref.stride()
    return ts == rs or all(a == b for a, b, n in zip(ts, rs, ref.shape) if n > 1)


def la_status_string(status: int) -> str:
    return lib().la_status_string(status).decode()


def la_last_error() -> str:
    return lib().la_last_error().decode()


def _check(status: int, where: str):
    if status != LA_OK:
        raise LAError(status, where, la_last_error() or la_status_string(status))


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return LA_F32
    if t.dtype == torch.bfloat16:
        return LA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _stream_ptr(stream, device):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def la_state_init(kv, kv0=None, stream=None) -> None:
    """kv[B,H,d,d] (float32) := 0, or a copy of kv0."""
    if kv.dim() != 4 or kv.shape[2] != kv.shape[3]:
        raise ValueError("kv must be [B, H, d, d]")
    B, H, d, _ = kv.shape
    _check_f32(kv, (B, H, d, d), "kv")
    _check_f32(kv0, (B, H, d, d), "kv0")
    _require_cuda(kv, kv0)
    _check(lib().la_state_init(_ptr(kv), _ptr(kv0), B, H, d, _stream_ptr(stream, kv.device)), "la_state_init")


def la_prefill_chunk_tokens(dtype: int, batch: int, heads: int, n: int, d: int) -> int:
    return int(lib().la_prefill_chunk_tokens(dtype, batch, heads, n, d))


def la_prefill_workspace_size(dtype: int, batch: int, heads: int, n: int, d: int, chunk_tokens: int = 0) -> int:
    return int(lib().la_prefill_workspace_size_ex(dtype, batch, heads, n, d, chunk_tokens))


def la_prefill(q, k, v, slopes, kv, o=None, ckpt=None, ckpt_every: int = 0, workspace=None,
               chunk_tokens: int = 0, stream=None) -> None:
    """Prefill over q, k, v [B,H,N,d] (views allowed if the last dim is contiguous and the
    three share strides).  Updates kv [B,H,d,d] in place; writes o (same shape/strides as q)
    unless it is None; fills ckpt [B,H,N//ckpt_every,d,d] when given.  A workspace of
    la_prefill_workspace_size() bytes is allocated here when not supplied."""
    import torch

    _check_qkv(q, k, v, 4)
    dt = _dtype_code(q)
    B, H, N, d = q.shape
    _check_out(o, q, "o")
    _check_slopes(slopes, H)
    _check_f32(kv, (B, H, d, d), "kv")
    if ckpt is not None:
        if ckpt_every <= 0:
            raise ValueError("ckpt_every must be positive when ckpt is given")
        _check_f32(ckpt, (B, H, N // ckpt_every, d, d), "ckpt")
    _require_cuda(q, k, v, slopes, kv, o, ckpt, workspace)
    need = la_prefill_workspace_size(dt, B, H, N, d, chunk_tokens)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _on_stream(stream, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sb, sh, sn, _ = q.stride()
    st = lib().la_prefill_ex(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, d, sb, sh, sn,
                             _ptr(slopes), _ptr(kv), _ptr(ckpt), ckpt_every, chunk_tokens,
                             _ptr(workspace), ws_bytes, _stream_ptr(stream, q.device))
    _check(st, "la_prefill")


def la_prefill_noalloc(q, k, v, slopes, kv, o=None, ckpt=None, ckpt_every: int = 0, stream=None) -> None:
    """la_prefill without a workspace argument, for callers that cannot allocate: the chunk
    states live in the library's per-GPU scratch array (LA_NOALLOC_SCRATCH_BYTES), so calls
    that overlap on one GPU race.  Allocates nothing."""
    _check_qkv(q, k, v, 4)
    dt = _dtype_code(q)
    B, H, N, d = q.shape
    _check_out(o, q, "o")
    _check_slopes(slopes, H)
    _check_f32(kv, (B, H, d, d), "kv")
    if ckpt is not None:
        if ckpt_every <= 0:
            raise ValueError("ckpt_every must be positive when ckpt is given")
        _check_f32(ckpt, (B, H, N // ckpt_every, d, d), "ckpt")
    _require_cuda(q, k, v, slopes, kv, o, ckpt)
    sb, sh, sn, _ = q.stride()
    st = lib().la_prefill_noalloc(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, d, sb, sh, sn,
                                  _ptr(slopes), _ptr(kv), _ptr(ckpt), ckpt_every, _stream_ptr(stream, q.device))
    _check(st, "la_prefill_noalloc")


def la_decode(q, k, v, slopes, kv, o, stream=None) -> None:
    """One decode step: kv <- lambda*kv + k^T v ; o = q . kv.  q,k,v,o contiguous [B,H,d]."""
    if q.dim() != 3:
        raise ValueError("q, k, v, o must be [B,H,d]")
    dt = _dtype_code(q)
    B, H, d = q.shape
    for t in (q, k, v, o):
        if not t.is_contiguous() or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, o must be contiguous [B,H,d] tensors of one dtype")
    _check_slopes(slopes, H)
    _check_f32(kv, (B, H, d, d), "kv")
    _require_cuda(q, k, v, slopes, kv, o)
    st = lib().la_decode(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, d, _ptr(slopes), _ptr(kv),
                         _stream_ptr(stream, q.device))
    _check(st, "la_decode")


def _cu_array(cu_seqlens):
    """cu_seqlens (list / numpy / CPU tensor) as a ctypes int64 array (host memory)."""
    vals = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    return (ctypes.c_int64 * len(vals))(*vals), len(vals) - 1


def la_prefill_varlen_workspace_size(dtype: int, cu_seqlens, heads: int, d: int, chunk_tokens: int = 0) -> int:
    cu, n_seq = _cu_array(cu_seqlens)
    return int(lib().la_prefill_varlen_workspace_size_ex(dtype, n_seq, cu, heads, d, chunk_tokens))


def la_prefill_varlen_chunk_tokens(dtype: int, cu_seqlens, heads: int, d: int) -> int:
    cu, n_seq = _cu_array(cu_seqlens)
    return int(lib().la_prefill_varlen_chunk_tokens(dtype, n_seq, cu, heads, d))


def la_prefill_varlen(q, k, v, slopes, kv, cu_seqlens, o=None, workspace=None, chunk_tokens: int = 0,
                      stream=None) -> None:
    """Packed variable-length prefill over q, k, v [total, H, d] (or any view with strides
    (stride_n, stride_h, 1)); sequence s is rows cu_seqlens[s]:cu_seqlens[s+1].  Updates
    kv [n_seq, H, d, d] in place and writes o (same shape/strides as q) unless it is None.
    The workspace (la_prefill_varlen_workspace_size bytes) is allocated here if not given."""
    import torch

    _check_qkv(q, k, v, 3)
    dt = _dtype_code(q)
    T, H, d = q.shape
    _check_out(o, q, "o")
    _check_slopes(slopes, H)
    cu, n_seq = _cu_array(cu_seqlens)
    if cu[n_seq] != T:
        raise ValueError("cu_seqlens[-1] must equal the packed token count")
    _check_f32(kv, (n_seq, H, d, d), "kv")
    _require_cuda(q, k, v, slopes, kv, o, workspace)
    if workspace is None:
        need = int(lib().la_prefill_varlen_workspace_size_ex(dt, n_seq, cu, H, d, chunk_tokens))
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            _on_stream(stream, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sn, sh, _ = q.stride()
    st = lib().la_prefill_varlen_ex(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(o), n_seq, cu, H, d, sh, sn,
                                    _ptr(slopes), _ptr(kv), chunk_tokens, _ptr(workspace), ws_bytes,
                                    _stream_ptr(stream, q.device))
    _check(st, "la_prefill_varlen")


def mixed_step(slopes, decode=None, prefill=None, streams=None) -> None:
    """One step of a mixed batch, separated as section 3.3 of the MiniMax-01 summary page does:
    the single-token sequences go to la_decode and the multi-token ones to la_prefill_varlen.
    decode = (q, k, v, o, kv) with [B,H,d] tensors; prefill = (q, k, v, o, kv, cu_seqlens,
    workspace or None).  With streams = (s0, s1) the two calls are issued on two streams that
    first wait for, and are then joined back into, the current stream; with streams = None both
    run on the current stream, one after the other (for small batches the cross-stream
    synchronisation costs more than the overlap gains)."""
    import torch

    cur = torch.cuda.current_stream()
    if streams is not None:
        for s in streams:
            s.wait_stream(cur)
    sd, sp = (None, None) if streams is None else streams
    if decode is not None:
        q, k, v, o, kv = decode
        la_decode(q, k, v, slopes, kv, o, stream=sd)
    if prefill is not None:
        q, k, v, o, kv, cu, ws = prefill
        la_prefill_varlen(q, k, v, slopes, kv, cu, o=o, workspace=ws, stream=sp)
    if streams is not None:
        for s in streams:
            cur.wait_stream(s)


def _fusion(silu_q=False, silu_k=False, silu_v=False, norm_eps=None, norm_weight=None, gate=None):
    flags = (LA_SILU_Q if silu_q else 0) | (LA_SILU_K if silu_k else 0) | (LA_SILU_V if silu_v else 0)
    if norm_eps is not None:
        flags |= LA_NORM
    if gate is not None:
        flags |= LA_GATE
    return la_fusion(flags, None if gate is None else gate.data_ptr(),
                     None if norm_weight is None else norm_weight.data_ptr(),
                     0.0 if norm_eps is None else float(norm_eps))


def la_prefill_fused(q, k, v, slopes, kv, o, silu_q=False, silu_k=False, silu_v=False, norm_eps=None,
                     norm_weight=None, gate=None, workspace=None, stream=None) -> None:
    """la_prefill with the fused prologue/epilogue: SiLU on the selected inputs, then (optionally)
    RMS normalisation over d with weight norm_weight [d] (float32) and eps norm_eps, then the gate
    o * sigmoid(gate) (gate: q's shape, strides and dtype).  o is required."""
    import torch

    _check_qkv(q, k, v, 4)
    dt = _dtype_code(q)
    B, H, N, d = q.shape
    if o is None:
        raise ValueError("la_prefill_fused needs an output tensor o")
    _check_out(o, q, "o")
    if gate is not None and (gate.shape != q.shape or not _same_strides(gate, q) or gate.dtype != q.dtype):
        raise ValueError("gate must match q in shape, strides and dtype")
    if norm_weight is not None and (norm_weight.dtype != torch.float32 or norm_weight.numel() != d
                                    or not norm_weight.is_contiguous()):
        raise ValueError("norm_weight must be a contiguous float32 tensor of d elements")
    _check_slopes(slopes, H)
    _check_f32(kv, (B, H, d, d), "kv")
    _require_cuda(q, k, v, slopes, kv, o, workspace, norm_weight, gate)
    need = la_prefill_workspace_size(dt, B, H, N, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _on_stream(stream, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sb, sh, sn, _ = q.stride()
    fu = _fusion(silu_q, silu_k, silu_v, norm_eps, norm_weight, gate)
    st = lib().la_prefill_fused(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, d, sb, sh, sn, _ptr(slopes),
                                _ptr(kv), ctypes.byref(fu), _ptr(workspace), ws_bytes, _stream_ptr(stream, q.device))
    _check(st, "la_prefill_fused")


def la_decode_fused(q, k, v, slopes, kv, o, silu_q=False, silu_k=False, silu_v=False, norm_eps=None,
                    norm_weight=None, gate=None, stream=None) -> None:
    """la_decode with the fused prologue/epilogue (see la_prefill_fused); gate is [B,H,d]."""
    import torch

    if q.dim() != 3:
        raise ValueError("q, k, v, o must be [B,H,d]")
    dt = _dtype_code(q)
    B, H, d = q.shape
    for t in (q, k, v, o) + ((gate,) if gate is not None else ()):
        if not t.is_contiguous() or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, o (and gate) must be contiguous [B,H,d] tensors of one dtype")
    if norm_weight is not None and (norm_weight.dtype != torch.float32 or norm_weight.numel() != d
                                    or not norm_weight.is_contiguous()):
        raise ValueError("norm_weight must be a contiguous float32 tensor of d elements")
    _check_slopes(slopes, H)
    _check_f32(kv, (B, H, d, d), "kv")
    _require_cuda(q, k, v, slopes, kv, o, norm_weight, gate)
    fu = _fusion(silu_q, silu_k, silu_v, norm_eps, norm_weight, gate)
    st = lib().la_decode_fused(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, d, _ptr(slopes), _ptr(kv),
                               ctypes.byref(fu), _stream_ptr(stream, q.device))
    _check(st, "la_decode_fused")



def la_backward_workspace_size(dtype: int, batch: int, heads: int, n: int, d: int) -> int:
    return int(lib().la_backward_workspace_size(dtype, batch, heads, n, d))


def la_backward(q, k, v, dout, slopes, kv_in=None, dkv_out=None, dq=None, dk=None, dv=None, dkv_in=None,
                workspace=None, stream=None):
    """Gradients of a loss through la_prefill: given dout = dL/dO (q's shape, strides, dtype) and
    optionally dkv_out = dL/dKV_final [B,H,d,d] float32, returns (dq, dk, dv, dkv_in) with
    dkv_in = dL/dKV_in [B,H,d,d] float32.  kv_in is the forward pass's incoming state (None:
    zero).  Outputs are allocated when not given (dq, dk, dv like q)."""
    import torch

    if q.dim() != 4:
        raise ValueError("q, k, v, dout must be [B,H,N,d]")
    for t in (k, v, dout):
        if t.shape != q.shape or t.dtype != q.dtype or not _same_strides(t, q):
            raise ValueError("q, k, v, dout must share shape, strides and dtype")
    if q.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    dt = _dtype_code(q)
    B, H, N, d = q.shape
    _check_slopes(slopes, H)
    for t, name in ((kv_in, "kv_in"), (dkv_out, "dkv_out"), (dkv_in, "dkv_in")):
        _check_f32(t, (B, H, d, d), name)
    if all(t is None for t in (dq, dk, dv)):
        q, k, v, dout = _dense_layout(q, k, v, dout)   # gradients are allocated with q's strides
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_out(t, q, name)
    _require_cuda(q, k, v, dout, slopes, kv_in, dkv_out, dq, dk, dv, dkv_in, workspace)
    outs = [torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) if t is None else t
            for t in (dq, dk, dv)]
    if dkv_in is None:
        dkv_in = torch.empty(B, H, d, d, dtype=torch.float32, device=q.device)
    need = la_backward_workspace_size(dt, B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _on_stream(stream, workspace)
    _on_stream(stream, *(o for o, given in zip(outs, (dq, dk, dv)) if given is None))
    ws_bytes = workspace.numel() * workspace.element_size()
    sb, sh, sn, _ = q.stride()
    st = lib().la_backward(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, H, N, d, sb, sh, sn, _ptr(slopes),
                           _ptr(kv_in), _ptr(dkv_out), _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _ptr(dkv_in),
                           _ptr(workspace), ws_bytes, _stream_ptr(stream, q.device))
    _check(st, "la_backward")
    return outs[0], outs[1], outs[2], dkv_in


def la_backward_varlen_workspace_size(dtype: int, cu_seqlens, heads: int, d: int) -> int:
    cu, n_seq = _cu_array(cu_seqlens)
    return int(lib().la_backward_varlen_workspace_size(dtype, n_seq, cu, heads, d))


def la_backward_varlen(q, k, v, dout, slopes, cu_seqlens, kv_in=None, dkv_out=None, dq=None, dk=None, dv=None,
                       dkv_in=None, workspace=None, stream=None):
    """la_backward for packed sequences: q, k, v, dout are [T, H, d] (or any [T, H, d] view with a
    contiguous last dimension and shared strides) and cu_seqlens holds n_seq + 1 offsets (host);
    states are [n_seq, H, d, d] float32.  Returns (dq, dk, dv, dkv_in)."""
    import torch

    if q.dim() != 3:
        raise ValueError("q, k, v, dout must be [T,H,d]")
    for t in (k, v, dout):
        if t.shape != q.shape or t.dtype != q.dtype or not _same_strides(t, q):
            raise ValueError("q, k, v, dout must share shape, strides and dtype")
    if q.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    dt = _dtype_code(q)
    T, H, d = q.shape
    _check_slopes(slopes, H)
    cu, n_seq = _cu_array(cu_seqlens)
    if cu[n_seq] != T:
        raise ValueError("cu_seqlens[-1] must equal the number of packed tokens")
    for t, name in ((kv_in, "kv_in"), (dkv_out, "dkv_out"), (dkv_in, "dkv_in")):
        _check_f32(t, (n_seq, H, d, d), name)
    if all(t is None for t in (dq, dk, dv)):
        q, k, v, dout = _dense_layout(q, k, v, dout)
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_out(t, q, name)
    _require_cuda(q, k, v, dout, slopes, kv_in, dkv_out, dq, dk, dv, dkv_in, workspace)
    outs = [torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device) if t is None else t
            for t in (dq, dk, dv)]
    if dkv_in is None:
        dkv_in = torch.empty(n_seq, H, d, d, dtype=torch.float32, device=q.device)
    need = int(lib().la_backward_varlen_workspace_size(dt, n_seq, cu, H, d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        _on_stream(stream, workspace)
    _on_stream(stream, *(o for o, given in zip(outs, (dq, dk, dv)) if given is None))
    ws_bytes = workspace.numel() * workspace.element_size()
    sn, sh, _ = q.stride()
    st = lib().la_backward_varlen(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), n_seq, cu, H, d, sh, sn, _ptr(slopes),
                                  _ptr(kv_in), _ptr(dkv_out), _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]),
                                  _ptr(dkv_in), _ptr(workspace), ws_bytes, _stream_ptr(stream, q.device))
    _check(st, "la_backward_varlen")
    return outs[0], outs[1], outs[2], dkv_in


_autograd_cls = None


def _autograd():
    """torch.autograd.Function over la_prefill (forward) and la_backward (backward), built once."""
    global _autograd_cls
    if _autograd_cls is not None:
        return _autograd_cls
    import torch

    class LightningAttention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, slopes, kv_in):
            B, H, N, d = q.shape
            kv = (torch.zeros(B, H, d, d, dtype=torch.float32, device=q.device) if kv_in is None
                  else kv_in.detach().clone().contiguous())
            q, k, v = _dense_layout(q, k, v)
            o = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
            la_prefill(q, k, v, slopes, kv, o=o)
            ctx.save_for_backward(q, k, v, slopes, kv_in)
            ctx.mark_non_differentiable(slopes)
            return o, kv

        @staticmethod
        def backward(ctx, do, dkv):
            q, k, v, slopes, kv_in = ctx.saved_tensors
            if do is None:
                do = torch.zeros_like(q)
            if not (_same_strides(do, q) and do.dtype == q.dtype):
                # la_backward takes one set of strides for q, k, v and dL/dO
                q, k, v = (t.contiguous() for t in (q, k, v))
                do = do.to(q.dtype).contiguous()
            dkv_out = None if dkv is None else dkv.to(torch.float32).contiguous()
            dq, dk, dv, dkv_in = la_backward(q, k, v, do, slopes,
                                             kv_in=None if kv_in is None else kv_in.detach().contiguous(),
                                             dkv_out=dkv_out)
            return dq, dk, dv, None, (dkv_in if kv_in is not None else None)

    class LightningAttentionVarlen(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, slopes, kv_in, cu_seqlens):
            T, H, d = q.shape
            n_seq = len(cu_seqlens) - 1
            kv = (torch.zeros(n_seq, H, d, d, dtype=torch.float32, device=q.device) if kv_in is None
                  else kv_in.detach().clone().contiguous())
            q, k, v = _dense_layout(q, k, v)
            o = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
            la_prefill_varlen(q, k, v, slopes, kv, cu_seqlens, o=o)
            ctx.save_for_backward(q, k, v, slopes, kv_in)
            ctx.cu_seqlens = list(cu_seqlens)
            ctx.mark_non_differentiable(slopes)
            return o, kv

        @staticmethod
        def backward(ctx, do, dkv):
            q, k, v, slopes, kv_in = ctx.saved_tensors
            if do is None:
                do = torch.zeros_like(q)
            if not (_same_strides(do, q) and do.dtype == q.dtype):
                q, k, v = (t.contiguous() for t in (q, k, v))
                do = do.to(q.dtype).contiguous()
            dkv_out = None if dkv is None else dkv.to(torch.float32).contiguous()
            dq, dk, dv, dkv_in = la_backward_varlen(q, k, v, do, slopes, ctx.cu_seqlens,
                                                    kv_in=None if kv_in is None else kv_in.detach().contiguous(),
                                                    dkv_out=dkv_out)
            return dq, dk, dv, None, (dkv_in if kv_in is not None else None), None

    _autograd_cls = (LightningAttention, LightningAttentionVarlen)
    return _autograd_cls


def lightning_attention(q, k, v, slopes, kv_in=None):
    """Differentiable prefill for training: (o, kv_out) = the prefill of q, k, v [B,H,N,d] from
    kv_in [B,H,d,d] float32 (None: zero).  Gradients reach q, k, v and kv_in through la_backward;
    the decay slopes are constants.  Both passes run in the library's kernels."""
    return _autograd()[0].apply(q, k, v, slopes, kv_in)


def lightning_attention_varlen(q, k, v, slopes, cu_seqlens, kv_in=None):
    """Differentiable packed prefill: (o, kv_out) for q, k, v [T,H,d] holding the sequences
    cu_seqlens[s]:cu_seqlens[s+1] (host offsets), each from its own state kv_in[s] (None: zero).
    Gradients reach q, k, v and kv_in through la_backward_varlen."""
    return _autograd()[1].apply(q, k, v, slopes, kv_in, list(cu_seqlens))
