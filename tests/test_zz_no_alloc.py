"""la_prefill_noalloc (no workspace argument; the chunk states live in the library's device array)
against la_prefill with a caller workspace, through the C ABI: two calls in a row on one GPU, the
second with a smaller input, both equal to the workspace entry point's results, which in turn
meet the bf16 parity bar against the fp64 oracle."""
import ctypes

import numpy as np
import pytest

import long_context_la_amd as la
import oracle
from common import assert_close, inputs, to_device, to_host

pytestmark = pytest.mark.gpu

SL2 = np.array([2.0 ** -2, 2.0 ** -8], dtype=np.float32)


def _call(entry, q, k, v, o, slopes, kv, ckpt=None, ckpt_every=0, ws=None):
    import torch

    B, H, N, d = q.shape
    sb, sh, sn, _ = q.stride()
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    L = la.lib()
    ck = None if ckpt is None else ctypes.c_void_p(ckpt.data_ptr())
    if entry == "noalloc":
        st = L.la_prefill_noalloc(la.LA_BF16, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, d,
                                  sb, sh, sn, slopes.data_ptr(), kv.data_ptr(), ck, ckpt_every, stream)
    else:
        st = L.la_prefill(la.LA_BF16, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, d, sb, sh, sn,
                          slopes.data_ptr(), kv.data_ptr(), ck, ckpt_every,
                          None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(), stream)
    assert st == la.LA_OK, la.la_last_error()


@pytest.mark.parametrize("shapes", [((1, 2, 9000), (1, 2, 3000)), ((2, 3, 20000), (1, 1, 1500))])
def test_noalloc_matches_workspace_prefill_twice(device, shapes):
    import torch

    for i, (B, H, N) in enumerate(shapes):
        d = 128
        assert la.la_prefill_workspace_size(la.LA_BF16, B, H, N, d) > 0      # the plan uses chunk states
        exact, raw = inputs(70 + i, B, H, N, d, "bf16")
        q, k, v = (to_device(x, "bf16", device) for x in raw)
        sl = torch.from_numpy(np.tile(SL2, (H + 1) // 2)[:H].copy()).to(device)
        kv0 = np.random.default_rng(71 + i).standard_normal((B, H, d, d)).astype(np.float32)
        results = {}
        for entry in ("noalloc", "workspace"):
            kv = torch.from_numpy(kv0).to(device)
            o = torch.empty_like(q)
            ws = None
            if entry == "workspace":
                ws = torch.empty(la.la_prefill_workspace_size(la.LA_BF16, B, H, N, d), dtype=torch.uint8,
                                 device=device)
            _call(entry, q, k, v, o, sl, kv, ws=ws)
            torch.cuda.synchronize()
            results[entry] = (to_host(o), kv.cpu().numpy())
        o_n, kv_n = results["noalloc"]
        o_w, kv_w = results["workspace"]
        assert np.array_equal(o_n, o_w) and np.array_equal(kv_n, kv_w), f"call {i}: entry points differ"
        o_ref, kv_ref, _ = oracle.recurrent(*exact, sl.cpu().numpy(), kv_in=kv0)
        assert_close(o_n, o_ref, "bf16", f"call {i} O", stored="bf16")
        assert_close(kv_n, kv_ref, "bf16", f"call {i} KV")


def test_noalloc_checkpoints_between_tiles(device):
    # checkpoints at an interval that is not a tile multiple: segments chunked inside the array
    import torch

    B, H, N, d, every = 1, 2, 5000, 128, 1700
    exact, raw = inputs(72, B, H, N, d, "bf16")
    q, k, v = (to_device(x, "bf16", device) for x in raw)
    sl = torch.from_numpy(SL2).to(device)
    kv = torch.zeros(B, H, d, d, device=device)
    o = torch.empty_like(q)
    ck = torch.full((B, H, N // every, d, d), float("nan"), device=device)
    _call("noalloc", q, k, v, o, sl, kv, ckpt=ck, ckpt_every=every)
    torch.cuda.synchronize()
    o_ref, kv_ref, ck_ref = oracle.recurrent(*exact, SL2, ckpt_every=every)
    assert_close(to_host(o), o_ref, "bf16", "O", stored="bf16")
    assert_close(kv.cpu().numpy(), kv_ref, "bf16", "KV")
    for m in range(N // every):
        assert_close(ck.cpu().numpy()[:, :, m], ck_ref[:, :, m], "bf16", f"checkpoint {m}")


def test_noalloc_through_the_binding(device):
    """The binding's la_prefill_noalloc against la_prefill with a workspace, bit for bit, on a
    chunked shape with checkpoints."""
    import torch

    B, H, N, d = 1, 2, 6000, 128
    exact, raw = inputs(75, B, H, N, d, "bf16")
    q, k, v = (to_device(x, "bf16", device) for x in raw)
    sl = torch.from_numpy(SL2).to(device)
    out = {}
    for name, fn in (("noalloc", la.la_prefill_noalloc), ("workspace", la.la_prefill)):
        kv = torch.zeros(B, H, d, d, device=device)
        o = torch.empty_like(q)
        ck = torch.zeros(B, H, N // 1024, d, d, device=device)
        fn(q, k, v, sl, kv, o=o, ckpt=ck, ckpt_every=1024)
        torch.cuda.synchronize()
        out[name] = (o.cpu(), kv.cpu(), ck.cpu())
    for x, y in zip(out["noalloc"], out["workspace"]):
        assert torch.equal(x, y)


def test_noalloc_at_the_layer_shape(device):
    """The 64-head layer (1 x 64 x 131072, d = 128), whose plan fills most of the array (two chunks
    of 64-column slices, sixteen summary sub-chunks: 76 MiB), against la_prefill with a caller
    workspace bit for bit, then a smaller call through the same array; the oracle checks windows of
    the layer in tests/test_gpu_workloads.py."""
    import torch

    import bench
    import synth

    w = synth.WORKLOADS["full"]
    need = la.la_prefill_workspace_size(la.LA_BF16, w.batch, w.heads, w.n, w.d)
    assert 32 << 20 < need <= la.LA_NOALLOC_SCRATCH_BYTES
    q, k, v = bench.make_prefill_inputs(w, device)
    sl = torch.from_numpy(w.slopes()).to(device)
    out = {}
    for entry in ("noalloc", "workspace"):
        kv = torch.zeros(w.batch, w.heads, w.d, w.d, device=device)
        o = torch.empty_like(q)
        ws = torch.empty(need, dtype=torch.uint8, device=device) if entry == "workspace" else None
        _call(entry, q, k, v, o, sl, kv, ws=ws)
        torch.cuda.synchronize()
        out[entry] = (o, kv)
    assert torch.equal(out["noalloc"][0], out["workspace"][0]) and torch.equal(out["noalloc"][1], out["workspace"][1])
    del out, q, k, v
    torch.cuda.empty_cache()
    # a smaller chunked call after it, through the same array
    B, H, N, d = 1, 2, 9000, 128
    exact, raw = inputs(76, B, H, N, d, "bf16")
    q, k, v = (to_device(x, "bf16", device) for x in raw)
    kv = torch.zeros(B, H, d, d, device=device)
    o = torch.empty_like(q)
    _call("noalloc", q, k, v, o, torch.from_numpy(SL2).to(device), kv)
    torch.cuda.synchronize()
    o_ref, kv_ref, _ = oracle.recurrent(*exact, SL2)
    assert_close(to_host(o), o_ref, "bf16", "O after the layer", stored="bf16")
    assert_close(kv.cpu().numpy(), kv_ref, "bf16", "KV after the layer")
