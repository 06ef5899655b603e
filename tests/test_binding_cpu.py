"""Argument checks of the Python binding that need no GPU.

The C ABI receives raw device pointers and cannot see buffer sizes, so the binding checks every
state, checkpoint and slope tensor against the shape the call implies before anything is
launched.  The tensors here live on the CPU: each rejection must fire before the binding looks
at the device at all."""
import pytest
import torch

import long_context_la_amd as la

B, H, N, D = 1, 4, 256, 64


def qkv(n=N, dtype=torch.bfloat16):
    return [torch.zeros(B, H, n, D, dtype=dtype) for _ in range(3)]


def good():
    q, k, v = qkv()
    return dict(q=q, k=k, v=v, slopes=torch.ones(H), kv=torch.zeros(B, H, D, D))


def test_rows_disjoint_rule():
    assert la._rows_disjoint(torch.empty(2, 3, 5, 64))
    assert la._rows_disjoint(torch.empty(2, 5, 3, 64).permute(0, 2, 1, 3))      # [B,N,H,d] view
    assert la._rows_disjoint(torch.empty(2, 3, 5, 128)[..., :64])              # padded rows
    assert la._rows_disjoint(torch.empty(1, 1, 7, 64).expand(1, 1, 7, 64))     # size-1 dims are free
    assert not la._rows_disjoint(torch.empty(1, 1, 5, 64).expand(1, 3, 5, 64))  # stride 0 over heads
    assert not la._rows_disjoint(torch.empty(4096).as_strided((3, 5, 64), (32, 320, 1)))  # heads 32 apart < d


def test_prefill_rejects_bad_states_and_slopes():
    a = good()
    call = lambda **kw: la.la_prefill(**{**a, **kw})
    with pytest.raises(ValueError, match="kv"):
        call(kv=torch.zeros(B, H, D, D - 1))
    with pytest.raises(ValueError, match="kv"):
        call(kv=torch.zeros(B, H + 1, D, D))
    with pytest.raises(ValueError, match="kv"):
        call(kv=torch.zeros(B, H, D, D, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="kv"):
        call(kv=torch.zeros(B, H, D, D).transpose(2, 3))                        # transposed view
    with pytest.raises(ValueError, match="slopes"):
        call(slopes=torch.ones(H - 1))
    with pytest.raises(ValueError, match="slopes"):
        call(slopes=torch.ones(H, dtype=torch.float64))
    with pytest.raises(ValueError, match="slopes"):
        call(slopes=torch.ones(2 * H)[::2])
    with pytest.raises(ValueError, match="ckpt"):
        call(ckpt=torch.zeros(B, H, 3, D, D), ckpt_every=64)                   # 256 / 64 = 4 slots
    with pytest.raises(ValueError, match="ckpt_every"):
        call(ckpt=torch.zeros(B, H, 4, D, D), ckpt_every=0)
    with pytest.raises(ValueError, match="o"):
        call(o=torch.zeros(B, H, N, D, dtype=torch.float32))
    with pytest.raises(ValueError, match="overlap"):
        q = torch.zeros(B, 1, N, D, dtype=torch.bfloat16).expand(B, H, N, D)
        la.la_prefill(q, q, q, a["slopes"], a["kv"], o=torch.zeros(B, 1, N, D, dtype=torch.bfloat16).expand(B, H, N, D))
    # a valid call gets past every check and stops only at the device
    with pytest.raises(ValueError, match="GPU"):
        call(ckpt=torch.zeros(B, H, 2, D, D), ckpt_every=100)


def test_noalloc_prefill_rejects_bad_states():
    a = good()
    call = lambda **kw: la.la_prefill_noalloc(**{**a, **kw})
    with pytest.raises(ValueError, match="kv"):
        call(kv=torch.zeros(B, H, D, D + 1))
    with pytest.raises(ValueError, match="slopes"):
        call(slopes=torch.ones(H + 1))
    with pytest.raises(ValueError, match="ckpt"):
        call(ckpt=torch.zeros(B, H, 1, D, D), ckpt_every=64)
    with pytest.raises(ValueError, match="GPU"):
        call()


def test_state_init_and_decode_reject_bad_states():
    with pytest.raises(ValueError, match="kv0"):
        la.la_state_init(torch.zeros(B, H, D, D), torch.zeros(B, H, D, D, dtype=torch.float64))
    with pytest.raises(ValueError, match="kv"):
        la.la_state_init(torch.zeros(B, H, D, D).transpose(2, 3))
    q = torch.zeros(2, H, D, dtype=torch.bfloat16)
    ok = dict(q=q, k=q.clone(), v=q.clone(), slopes=torch.ones(H), kv=torch.zeros(2, H, D, D), o=q.clone())
    dec = lambda **kw: la.la_decode(**{**ok, **kw})
    with pytest.raises(ValueError, match="kv"):
        dec(kv=torch.zeros(1, H, D, D))
    with pytest.raises(ValueError, match="kv"):
        dec(kv=torch.zeros(2, H, D, D, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="slopes"):
        dec(slopes=torch.ones(H + 2))
    fused = lambda **kw: la.la_decode_fused(**{**ok, **kw})
    with pytest.raises(ValueError, match="kv"):
        fused(kv=torch.zeros(2, H, D, 2 * D))
    with pytest.raises(ValueError, match="norm_weight"):
        fused(norm_eps=1e-5, norm_weight=torch.ones(D + 1))
    with pytest.raises(ValueError, match="GPU"):
        dec()


def test_varlen_rejects_bad_states():
    lengths = [100, 0, 7, 149]
    cu = [0, 100, 100, 107, 256]
    q = torch.zeros(256, H, D, dtype=torch.bfloat16)
    ok = dict(q=q, k=q.clone(), v=q.clone(), slopes=torch.ones(H), kv=torch.zeros(len(lengths), H, D, D), cu_seqlens=cu)
    call = lambda **kw: la.la_prefill_varlen(**{**ok, **kw})
    with pytest.raises(ValueError, match="kv"):
        call(kv=torch.zeros(len(lengths) - 1, H, D, D))
    with pytest.raises(ValueError, match="slopes"):
        call(slopes=torch.ones(1))
    with pytest.raises(ValueError, match="cu_seqlens"):
        call(cu_seqlens=[0, 100, 100, 107, 255])
    with pytest.raises(ValueError, match="GPU"):
        call()


def test_fused_prefill_rejects_bad_arguments():
    a = good()
    o = torch.zeros_like(a["q"])
    call = lambda **kw: la.la_prefill_fused(**{**a, "o": o, **kw})
    with pytest.raises(ValueError, match="kv"):
        call(kv=torch.zeros(B, H, D, D)[:, :, :, :D - 1])
    with pytest.raises(ValueError, match="gate"):
        call(gate=torch.zeros(B, H, N, D))                                    # float32 gate for bf16 inputs
    with pytest.raises(ValueError, match="output"):
        call(o=None)
    with pytest.raises(ValueError, match="GPU"):
        call(silu_q=True, gate=torch.zeros_like(o))


def test_backward_rejects_bad_states_and_allocates_dense_gradients():
    a = good()
    g = torch.zeros_like(a["q"])
    call = lambda **kw: la.la_backward(a["q"], a["k"], a["v"], g, a["slopes"], **kw)
    with pytest.raises(ValueError, match="dkv_out"):
        call(dkv_out=torch.zeros(B, H, D, D, dtype=torch.float64))
    with pytest.raises(ValueError, match="kv_in"):
        call(kv_in=torch.zeros(B, H + 1, D, D))
    with pytest.raises(ValueError, match="dq"):
        call(dq=torch.zeros(B, 1, N, D, dtype=torch.bfloat16).expand(B, H, N, D))
    with pytest.raises(ValueError, match="slopes"):
        la.la_backward(a["q"], a["k"], a["v"], g, torch.ones(H + 1))
    # expanded inputs are made dense before gradients are laid out like them
    q = torch.zeros(B, 1, N, D, dtype=torch.bfloat16).expand(B, H, N, D)
    assert la._dense_layout(q, q)[0].is_contiguous()
    with pytest.raises(ValueError, match="GPU"):
        la.la_backward(q, q, q, q, a["slopes"])
