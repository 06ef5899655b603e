"""C-ABI checks that need no GPU: the library loads, exports every declared entry point,
validates arguments before touching HIP, and reports a missing device as LA_ERR_DEVICE."""
import ctypes
import os
import re

import numpy as np
import pytest

import long_context_la_amd as la
from conftest import gpu_available

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "la.h")
FAKE = ctypes.c_void_p(1 << 20)  # aligned non-null address, never dereferenced by validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = la.lib()
    names = declared_functions()
    assert set(names) == set(la.EXPORTED)
    for name in names:
        assert hasattr(L, name), name


def test_status_strings():
    for s in range(6):
        assert la.la_status_string(s).startswith("LA_")
    assert "unknown" in la.la_status_string(99)


def _prefill(**kw):
    args = dict(dt=la.LA_BF16, q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, H=8, N=4096, d=128,
                sb=8 * 4096 * 128, sh=4096 * 128, sn=128, slopes=FAKE, kv=FAKE, ckpt=None,
                ckpt_every=0, chunk=0, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    a = args
    return la.lib().la_prefill_ex(a["dt"], a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["N"], a["d"],
                                  a["sb"], a["sh"], a["sn"], a["slopes"], a["kv"], a["ckpt"], a["ckpt_every"],
                                  a["chunk"], a["ws"], a["ws_bytes"], None)


def test_prefill_validation_codes():
    assert _prefill(q=None) == la.LA_ERR_INVALID_ARGUMENT
    assert _prefill(kv=None) == la.LA_ERR_INVALID_ARGUMENT
    assert _prefill(slopes=None) == la.LA_ERR_INVALID_ARGUMENT
    assert _prefill(dt=7) == la.LA_ERR_INVALID_ARGUMENT
    assert _prefill(B=0) == la.LA_ERR_INVALID_ARGUMENT
    assert _prefill(N=-1) == la.LA_ERR_INVALID_ARGUMENT
    assert _prefill(d=96, sn=96) == la.LA_ERR_UNSUPPORTED
    # bf16 at d = 64 is a supported shape: it gets as far as the workspace check
    assert _prefill(d=64, sn=64, ws=None, ws_bytes=0) == la.LA_ERR_WORKSPACE
    assert _prefill(sn=100) == la.LA_ERR_INVALID_ARGUMENT           # not a 16-byte multiple
    assert _prefill(sn=64) == la.LA_ERR_INVALID_ARGUMENT            # stride_n < d
    assert _prefill(sn=(1 << 22) + 8) == la.LA_ERR_UNSUPPORTED      # 32-bit tile offsets
    assert _prefill(B=1 << 10, H=(1 << 10) + 1) == la.LA_ERR_UNSUPPORTED   # > 2^20 (batch, head) pairs
    assert _prefill(N=1 << 30, sh=128 << 30, sb=8 * (128 << 30), chunk=64) == la.LA_ERR_UNSUPPORTED  # > 2^20 items
    assert _prefill(q=ctypes.c_void_p((1 << 20) + 2)) == la.LA_ERR_INVALID_ARGUMENT  # misaligned
    assert _prefill(ckpt=FAKE, ckpt_every=0) == la.LA_ERR_INVALID_ARGUMENT
    assert _prefill(ckpt=FAKE, ckpt_every=-64) == la.LA_ERR_INVALID_ARGUMENT
    # output rows must be pairwise disjoint: stride 0 over heads, or heads closer than d
    assert _prefill(sh=0) == la.LA_ERR_INVALID_ARGUMENT
    assert _prefill(sh=64, sb=1 << 24) == la.LA_ERR_INVALID_ARGUMENT
    assert _prefill(B=2, sb=0) == la.LA_ERR_INVALID_ARGUMENT
    assert "overlap" in la.la_last_error()
    # ... which inputs may break when there is no output (state only)
    if not gpu_available():
        assert _prefill(sh=0, o=None) == la.LA_ERR_DEVICE
        assert _prefill(ckpt=FAKE, ckpt_every=100) == la.LA_ERR_DEVICE   # any positive interval is valid
    assert _prefill(chunk=100) == la.LA_ERR_INVALID_ARGUMENT
    assert "64" in la.la_last_error()
    # chunked plan without (enough) workspace
    assert _prefill(ws=None, ws_bytes=0) == la.LA_ERR_WORKSPACE
    assert _prefill(ws_bytes=10) == la.LA_ERR_WORKSPACE
    # n == 0 is a no-op and never touches the device
    assert _prefill(N=0, q=None, k=None, v=None, ws=None, ws_bytes=0) == la.LA_OK


@pytest.mark.skipif(gpu_available(), reason="checks the no-device path")
def test_no_device_is_reported_not_fatal():
    assert _prefill() == la.LA_ERR_DEVICE
    assert "GPU" in la.la_last_error()
    L = la.lib()
    assert L.la_decode(la.LA_BF16, FAKE, FAKE, FAKE, FAKE, 2, 2, 128, FAKE, FAKE, None) == la.LA_ERR_DEVICE
    assert L.la_state_init(FAKE, None, 2, 2, 128, None) == la.LA_ERR_DEVICE


def test_decode_and_state_init_validation():
    L = la.lib()
    assert L.la_decode(la.LA_BF16, None, FAKE, FAKE, FAKE, 2, 2, 128, FAKE, FAKE, None) == la.LA_ERR_INVALID_ARGUMENT
    assert L.la_decode(la.LA_BF16, FAKE, FAKE, FAKE, FAKE, 2, 2, 96, FAKE, FAKE, None) == la.LA_ERR_UNSUPPORTED
    assert L.la_decode(la.LA_F32, FAKE, FAKE, FAKE, FAKE, 0, 2, 64, FAKE, FAKE, None) == la.LA_ERR_INVALID_ARGUMENT
    # one launch covers at most 2^20 (batch, head) pairs
    assert L.la_decode(la.LA_F32, FAKE, FAKE, FAKE, FAKE, (1 << 19) + 1, 2, 64, FAKE, FAKE, None) == la.LA_ERR_UNSUPPORTED
    assert L.la_state_init(None, None, 1, 1, 128, None) == la.LA_ERR_INVALID_ARGUMENT
    assert L.la_state_init(FAKE, None, 1, 1, 32, None) == la.LA_ERR_UNSUPPORTED


def test_plan_and_workspace_sizes():
    # 64 heads x 131072 tokens: 64-column slices in two chunks (64 x 2 x 2 = 256 workgroups); the
    # summaries of chunk 0 in 16 sub-chunks of 4096 tokens: 2 prefix + 1 + 16 summary slots per head
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, 64, 131072, 128) == 65536
    assert la.la_prefill_workspace_size(la.LA_BF16, 1, 64, 131072, 128) == 64 * (2 + 1 + 16) * 128 * 128 * 4
    # every default plan's chunk states fit the allocation-free entry point's array
    assert max(la.la_prefill_workspace_size(la.LA_BF16, 1, h, n, 128) for h in (1, 8, 26, 64)
               for n in (65536, 262144, 1 << 20, 1 << 22)) <= la.LA_NOALLOC_SCRATCH_BYTES
    # shorter: 32-column slices fill the GPU once, unchunked
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, 64, 32768, 128) == 32768
    assert la.la_prefill_workspace_size(la.LA_BF16, 1, 64, 32768, 128) == 0
    # 2 x 64 heads: one round of 256 workgroups of 64 columns, no chunks
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 2, 64, 131072, 128) == 131072
    assert la.la_prefill_workspace_size(la.LA_BF16, 2, 64, 131072, 128) == 0
    # 8 heads: the 32-column plan would cut 8 chunks, so the 64-column plan runs: 16 chunks per
    # sequence (8 x 2 slices x 16 = 256 workgroups)
    c = la.la_prefill_chunk_tokens(la.LA_BF16, 1, 8, 32768, 128)
    assert c == 2048
    # the size query covers both widths' plans (it does not know whether outputs are asked for):
    # 64 columns: prefix slots (16 per head) + summary slots: 15 chunks x 2 sub-chunks + 1, so that the
    # summary pass has 8 x 30 = 240 >= 128 full-width workgroups; 32 columns: 8 + 1 + 7 x 4
    assert la.la_prefill_workspace_size(la.LA_BF16, 1, 8, 32768, 128) == 8 * (16 + 1 + 15 * 2) * 128 * 128 * 4
    # 1M tokens: 16 chunks of 65536; their sub-chunks go finer (the summaries skip decayed tokens):
    # 15 x 8 sub-chunks of 8192, 8 x 120 = 960 summary workgroups
    c = la.la_prefill_chunk_tokens(la.LA_BF16, 1, 8, 1048576, 128)
    assert c == 65536
    assert la.la_prefill_workspace_size(la.LA_BF16, 1, 8, 1048576, 128) == 8 * (16 + 1 + 15 * 8) * 128 * 128 * 4
    # float32 keeps 32-column slices (4 per head at d = 128), and so does d = 64 (2 per head)
    assert la.la_prefill_chunk_tokens(la.LA_F32, 1, 8, 32768, 128) == 4096
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, 8, 32768, 64) == 2048
    # sub-chunks stay >= 256 tokens and multiples of 64: a 1024-token chunk splits at most 4 ways
    assert la.la_prefill_workspace_size(la.LA_BF16, 1, 1, 4096, 128, chunk_tokens=1024) == (4 + 1 + 3 * 4) * 128 * 128 * 4
    # short sequences are not chunked
    assert la.la_prefill_chunk_tokens(la.LA_F32, 1, 2, 512, 64) == 512
    # explicit chunking
    assert la.la_prefill_workspace_size(la.LA_F32, 1, 2, 512, 64, chunk_tokens=128) == 2 * 4 * 64 * 64 * 4
    assert la.la_prefill_workspace_size(la.LA_F32, 1, 2, 512, 64, chunk_tokens=1024) == 0
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, 8, 100, 96) == -1


def _cu(lengths):
    return [0] + list(np.cumsum(lengths).astype(int))


def _varlen(lengths, **kw):
    cu, n_seq = la._cu_array(kw.pop("cu", _cu(lengths)))
    a = dict(dt=la.LA_BF16, q=FAKE, k=FAKE, v=FAKE, o=FAKE, H=8, d=128, sh=128, sn=8 * 128, slopes=FAKE, kv=FAKE,
             chunk=0, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return la.lib().la_prefill_varlen_ex(a["dt"], a["q"], a["k"], a["v"], a["o"], n_seq, cu, a["H"], a["d"],
                                         a["sh"], a["sn"], a["slopes"], a["kv"], a["chunk"], a["ws"],
                                         a["ws_bytes"], None)


def test_varlen_plan_and_workspace_sizes():
    def table(n_chunks, n_seq, n_short=0):
        return ((5 * n_chunks + 2 * n_seq + 3 * n_short) * 8 + 255) // 256 * 256
    # the pages' mixed batch: two 50-token inputs run in tiles (one chunk each, 64 heads fill the
    # GPU), the 18 single-token inputs token by token; tables only
    lengths = [50, 50] + [1] * 18
    assert la.la_prefill_varlen_chunk_tokens(la.LA_BF16, _cu(lengths), 64, 128) == 50
    assert la.la_prefill_varlen_workspace_size(la.LA_BF16, _cu(lengths), 64, 128) == table(2, 20, 18)
    # one long, one medium and one short sequence on 8 heads: the long one is chunked
    lengths = [32768, 100, 7]
    c = la.la_prefill_varlen_chunk_tokens(la.LA_BF16, _cu(lengths), 8, 128)
    assert c % 64 == 0 and 1024 <= c < 32768
    n_chunks = (32768 + c - 1) // c + 1
    assert la.la_prefill_varlen_workspace_size(la.LA_BF16, _cu(lengths), 8, 128) == \
        table(n_chunks, 3, 1) + n_chunks * 8 * 128 * 128 * 4
    # explicit chunking; empty sequences take no chunk, 9+ token ones run in tiles
    lengths = [300, 0, 64, 9]
    n_chunks = 3 + 0 + 1 + 1
    assert la.la_prefill_varlen_workspace_size(la.LA_F32, _cu(lengths), 2, 64, chunk_tokens=128) == \
        table(n_chunks, 4) + n_chunks * 2 * 64 * 64 * 4
    # only short sequences: no tiles, no state slots
    assert la.la_prefill_varlen_workspace_size(la.LA_F32, _cu([8, 1, 3]), 2, 64, chunk_tokens=128) == table(0, 3, 3)
    # invalid inputs
    assert la.la_prefill_varlen_workspace_size(la.LA_BF16, [1, 5], 8, 128) == 0      # cu[0] != 0
    assert la.la_prefill_varlen_workspace_size(la.LA_BF16, [0, 5, 3], 8, 128) == 0   # decreasing
    assert la.la_prefill_varlen_chunk_tokens(la.LA_BF16, [0, 5], 8, 96) == -1


def test_varlen_validation_codes():
    assert _varlen([10, 20], q=None) == la.LA_ERR_INVALID_ARGUMENT
    assert _varlen([10, 20], kv=None) == la.LA_ERR_INVALID_ARGUMENT
    assert _varlen([10, 20], cu=[3, 10, 20]) == la.LA_ERR_INVALID_ARGUMENT
    assert _varlen([10, 20], cu=[0, 10, 5]) == la.LA_ERR_INVALID_ARGUMENT
    assert _varlen([10, 20], d=96, sh=96, sn=768) == la.LA_ERR_UNSUPPORTED
    assert _varlen([10, 20], d=64, sh=64, sn=512, ws=None, ws_bytes=0) == la.LA_ERR_WORKSPACE  # bf16 d = 64: valid
    assert _varlen([10, 20], sn=100) == la.LA_ERR_INVALID_ARGUMENT
    assert _varlen([10, 20], sn=(1 << 22) + 8) == la.LA_ERR_UNSUPPORTED
    assert _varlen([10, 20], sh=0) == la.LA_ERR_INVALID_ARGUMENT                   # output heads overlap
    assert _varlen([1 << 30, 20], chunk=64) == la.LA_ERR_UNSUPPORTED        # > 2^20 (chunk, head) items
    assert _varlen([10, 20], chunk=100) == la.LA_ERR_INVALID_ARGUMENT
    assert _varlen([10, 20], ws=None, ws_bytes=0) == la.LA_ERR_WORKSPACE
    assert _varlen([10, 20], ws_bytes=8) == la.LA_ERR_WORKSPACE
    # every sequence empty: a no-op that touches nothing
    assert _varlen([0, 0], q=None, k=None, v=None, ws=None, ws_bytes=0) == la.LA_OK


@pytest.mark.skipif(gpu_available(), reason="checks the no-device path")
def test_varlen_no_device_is_reported_not_fatal():
    assert _varlen([10, 20]) == la.LA_ERR_DEVICE


def _fusion(flags, gate=None, weight=None, eps=0.0):
    return la.la_fusion(flags, None if gate is None else gate.value, None if weight is None else weight.value, eps)


def test_fused_validation_codes():
    L = la.lib()

    def prefill(fu, o=FAKE):
        return L.la_prefill_fused(la.LA_BF16, FAKE, FAKE, FAKE, o, 1, 8, 4096, 128, 8 * 4096 * 128, 4096 * 128, 128,
                                  FAKE, FAKE, ctypes.byref(fu), FAKE, 1 << 30, None)

    def decode(fu, o=FAKE):
        return L.la_decode_fused(la.LA_BF16, FAKE, FAKE, FAKE, o, 2, 2, 128, FAKE, FAKE, ctypes.byref(fu), None)

    for call in (prefill, decode):
        assert call(_fusion(1 << 10)) == la.LA_ERR_INVALID_ARGUMENT                      # unknown flag
        assert call(_fusion(la.LA_GATE)) == la.LA_ERR_INVALID_ARGUMENT                   # gate tensor missing
        assert call(_fusion(la.LA_GATE, gate=ctypes.c_void_p((1 << 20) + 4))) == la.LA_ERR_INVALID_ARGUMENT
        assert call(_fusion(la.LA_NORM, eps=0.0)) == la.LA_ERR_INVALID_ARGUMENT          # eps must be > 0
        assert call(_fusion(la.LA_NORM, weight=ctypes.c_void_p((1 << 20) + 4), eps=1e-5)) == la.LA_ERR_INVALID_ARGUMENT
        assert call(_fusion(la.LA_NORM, eps=1e-5), o=None) == la.LA_ERR_INVALID_ARGUMENT  # the epilogue needs o
    # SiLU alone without an output is a state-only prefill: valid
    if not gpu_available():
        assert prefill(_fusion(la.LA_SILU_K | la.LA_SILU_V), o=None) == la.LA_ERR_DEVICE


def _backward(**kw):
    a = dict(dt=la.LA_BF16, q=FAKE, k=FAKE, v=FAKE, do=FAKE, B=1, H=8, N=4096, d=128, sb=8 * 4096 * 128,
             sh=4096 * 128, sn=128, slopes=FAKE, kv_in=None, dkv_out=None, dq=FAKE, dk=FAKE, dv=FAKE, dkv_in=None,
             ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return la.lib().la_backward(a["dt"], a["q"], a["k"], a["v"], a["do"], a["B"], a["H"], a["N"], a["d"], a["sb"],
                                a["sh"], a["sn"], a["slopes"], a["kv_in"], a["dkv_out"], a["dq"], a["dk"], a["dv"],
                                a["dkv_in"], a["ws"], a["ws_bytes"], None)


def test_backward_validation_codes():
    # the workspace holds one state per (batch, head) plus the prefill's chunk workspace
    need = la.la_backward_workspace_size(la.LA_BF16, 1, 8, 4096, 128)
    assert need == 8 * 128 * 128 * 4 + la.la_prefill_workspace_size(la.LA_BF16, 1, 8, 4096, 128)
    assert la.la_backward_workspace_size(la.LA_BF16, 1, 64, 131072, 128) == 64 * 128 * 128 * 4
    assert la.la_backward_workspace_size(la.LA_BF16, 1, 8, 100, 96) == 0                 # invalid shape
    assert _backward(do=None) == la.LA_ERR_INVALID_ARGUMENT
    assert _backward(dk=None) == la.LA_ERR_INVALID_ARGUMENT
    assert _backward(slopes=None) == la.LA_ERR_INVALID_ARGUMENT
    assert _backward(d=64, sn=64, ws=None, ws_bytes=0) == la.LA_ERR_WORKSPACE              # bf16 d = 64 is valid
    assert _backward(dkv_out=ctypes.c_void_p((1 << 20) + 4)) == la.LA_ERR_INVALID_ARGUMENT  # misaligned state
    assert _backward(ws=None, ws_bytes=0) == la.LA_ERR_WORKSPACE
    assert _backward(ws_bytes=need - 16) == la.LA_ERR_WORKSPACE
    assert _backward(sh=0) == la.LA_ERR_INVALID_ARGUMENT                          # gradient rows overlap
    if not gpu_available():
        assert _backward(ws_bytes=need) == la.LA_ERR_DEVICE
        assert _backward(N=0, q=None, k=None, v=None, do=None, dq=None, dk=None, dv=None) == la.LA_ERR_DEVICE


def test_backward_varlen_workspace_and_validation():
    lengths = [300, 0, 5, 1, 2000]
    cu = _cu(lengths)
    ws = la.la_backward_varlen_workspace_size(la.LA_BF16, cu, 2, 128)
    assert ws == len(lengths) * 2 * 128 * 128 * 4 + la.la_prefill_varlen_workspace_size(la.LA_BF16, cu, 2, 128)
    assert la.la_backward_varlen_workspace_size(la.LA_BF16, [1, 5], 2, 128) == 0     # cu[0] != 0
    c, n_seq = la._cu_array(cu)
    L = la.lib()

    def call(**kw):
        a = dict(q=FAKE, do=FAKE, dk=FAKE, slopes=FAKE, dkv_out=None, ws=FAKE, ws_bytes=ws)
        a.update(kw)
        return L.la_backward_varlen(la.LA_BF16, a["q"], FAKE, FAKE, a["do"], n_seq, c, 2, 128, 128, 256,
                                    a["slopes"], None, a["dkv_out"], FAKE, a["dk"], FAKE, None, a["ws"],
                                    a["ws_bytes"], None)
    assert call(do=None) == la.LA_ERR_INVALID_ARGUMENT
    assert call(dk=None) == la.LA_ERR_INVALID_ARGUMENT
    assert call(slopes=None) == la.LA_ERR_INVALID_ARGUMENT
    assert call(dkv_out=ctypes.c_void_p((1 << 20) + 4)) == la.LA_ERR_INVALID_ARGUMENT
    assert call(ws_bytes=ws - 16) == la.LA_ERR_WORKSPACE
    if not gpu_available():
        assert call() == la.LA_ERR_DEVICE


def test_binding_stride_match_ignores_size_one_dims():
    import torch

    # numpy gives a size-1 leading dimension the stride of the next one
    q = torch.from_numpy(np.ascontiguousarray(np.zeros((3, 1, 128), np.float32).transpose(1, 0, 2))).permute(1, 0, 2)
    o = torch.empty((1, 3, 128)).permute(1, 0, 2)                           # [3, 1, 128], stride_h 384
    assert q.stride() != o.stride()
    assert la._same_strides(o, q) and la._same_strides(q, o)
    assert not la._same_strides(torch.empty(3, 2, 128).permute(1, 0, 2), torch.empty(2, 3, 128))


def test_noalloc_array_size_matches_the_header():
    import os
    import re

    h = open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "..", "include", "la.h")).read()
    m = re.search(r"#define LA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << 20\)", h)
    assert m and int(m.group(1)) << 20 == la.LA_NOALLOC_SCRATCH_BYTES


@pytest.mark.skipif(gpu_available(), reason="relies on the device check coming after the workspace check")
def test_workspace_query_covers_every_plan():
    # with exactly the queried bytes no prefill fails its workspace check, with or without outputs,
    # whichever slice width and chunking the call takes; one byte less fails for plans that chunk
    for dt, d in ((la.LA_BF16, 128), (la.LA_BF16, 64), (la.LA_F32, 128)):
        for B, H in ((1, 1), (1, 8), (1, 26), (2, 32), (1, 48), (1, 64), (2, 64), (3, 48)):
            for N in (1000, 1025, 5000, 40000, 65536, 131072, 1 << 20):
                need = la.la_prefill_workspace_size(dt, B, H, N, d)
                sh, sb = N * d, H * N * d
                for o in (FAKE, None):
                    r = _prefill(dt=dt, B=B, H=H, N=N, d=d, sh=sh, sb=sb, sn=d, o=o,
                                 ws=FAKE if need else None, ws_bytes=need)
                    assert r == la.LA_ERR_DEVICE, (dt, B, H, N, d, o is None, need, la.la_status_string(r))
                if need and la.la_prefill_chunk_tokens(dt, B, H, N, d) < N:
                    r = _prefill(dt=dt, B=B, H=H, N=N, d=d, sh=sh, sb=sb, sn=d, ws=FAKE, ws_bytes=need - 1)
                    assert r == la.LA_ERR_WORKSPACE, (dt, B, H, N, d)
