"""GPU parity of the plans that give each bf16 workgroup 64 value columns (d = 128, float16
products, no SiLU prologue), against the fp64 oracle, with the bars of tests/common.py:

* one unchunked round of 64-column slices, where 32-column slices would need more than one
  round of workgroups (more than 64 (batch, head) pairs): incoming states, checkpoints inside
  and at the end of the tiles, the gate epilogue, determinism;
* chunked plans with summaries (few heads, where the 32-column plan would chunk the sequence);
* packed batches whose work spreads well beyond one round (and chunked packed batches);
* the same plan shapes at d = 64, which keeps 32-column slices.
Other bf16 d = 128 tests with outputs, few (batch, head) pairs and sequences long enough to be
chunked (over 1024 tokens) run these slices too.
"""
import numpy as np
import pytest

import long_context_la_amd as la
import oracle
from common import TOL, assert_close, half_ulp, inputs, to_device, to_host

pytestmark = pytest.mark.gpu


def layer_slopes(H):
    # the 64-head layer's decay rates 2^(-8(h+1)/H)
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)


def run(B, H, N, seed, device, kv_in=None, ckpt_every=0, gate=None, d=128):
    import torch

    exact, raw = inputs(seed, B, H, N, d, "bf16")
    q, k, v = (to_device(x, "bf16", device) for x in raw)
    slopes = layer_slopes(H)
    ts = torch.from_numpy(slopes).to(device)
    kv = (torch.zeros(B, H, d, d, dtype=torch.float32, device=device) if kv_in is None
          else torch.from_numpy(np.ascontiguousarray(kv_in, np.float32)).to(device))
    o = torch.empty_like(q)
    ck = (torch.full((B, H, N // ckpt_every, d, d), float("nan"), dtype=torch.float32, device=device)
          if ckpt_every else None)
    if gate is None:
        la.la_prefill(q, k, v, ts, kv, o=o, ckpt=ck, ckpt_every=ckpt_every)
    else:
        import synth

        g = to_device(synth.f32_to_bf16_bits(gate), "bf16", device)
        la.la_prefill_fused(q, k, v, ts, kv, o, gate=g)
    torch.cuda.synchronize()
    return exact, slopes, to_host(o), kv.cpu().numpy(), (ck.cpu().numpy() if ck is not None else None)


@pytest.mark.parametrize("every", [256, 1000])
def test_one_round_checkpoints(device, every):
    B, H, N = 2, 64, 2000
    assert la.la_prefill_chunk_tokens(la.LA_BF16, B, H, N, 128) == N
    rng = np.random.default_rng(5)
    kv_in = (rng.standard_normal((B, H, 128, 128)) * 0.5).astype(np.float32)
    exact, slopes, o, kv, ck = run(B, H, N, 62, device, kv_in=kv_in, ckpt_every=every)
    o_ref, kv_ref, ck_ref = oracle.recurrent(*exact, slopes, kv_in=kv_in, ckpt_every=every)
    assert_close(o, o_ref, "bf16", "O with checkpoints", stored="bf16")
    assert_close(kv, kv_ref, "bf16", "KV with checkpoints")
    assert not np.isnan(ck).any(), "a checkpoint slot was left unwritten"
    assert_close(ck.reshape(-1, *ck.shape[2:])[:, None], ck_ref.reshape(-1, *ck_ref.shape[2:])[:, None], "bf16",
                 "checkpoints")


def test_one_round_gate(device):
    B, H, N = 2, 64, 700
    rng = np.random.default_rng(7)
    import synth

    g = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits((rng.standard_normal((B, H, N, 128)) * 2.0).astype(np.float32)))
    exact, slopes, o, kv, _ = run(B, H, N, 63, device, gate=g)
    o_pre, kv_ref, _ = oracle.recurrent(*exact, slopes)
    sg = oracle.sigmoid(g.astype(np.float64))
    want = o_pre * sg
    # measured in the pre-gate domain: the gate multiplies the float32 result before the one rounding
    excess = np.maximum(np.abs(o - want) - half_ulp(o, "bf16"), 0.0) / sg
    worst = max(float(excess[b, h].max()) / float(np.sqrt(np.mean(o_pre[b, h] ** 2)))
                for b in range(B) for h in range(H))
    assert worst <= TOL["bf16"], f"gated: {worst:.3e}"
    assert_close(kv, kv_ref, "bf16", "KV gated")


def test_one_round_deterministic(device):
    a = run(2, 64, 1000, 64, device)
    b = run(2, 64, 1000, 64, device)
    assert np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3])


def test_one_round_of_wide_slices(device):
    B, H, N = 3, 32, 1500  # 96 pairs: 192 workgroups of 64 columns, no chunks
    assert la.la_prefill_chunk_tokens(la.LA_BF16, B, H, N, 128) == N
    exact, slopes, o, kv, _ = run(B, H, N, 65, device)
    o_ref, kv_ref, _ = oracle.recurrent(*exact, slopes)
    assert_close(o, o_ref, "bf16", "O one round", stored="bf16")
    assert_close(kv, kv_ref, "bf16", "KV one round")


@pytest.mark.parametrize("H,N", [(8, 5000), (16, 4097)])
def test_wide_slices_with_summaries(device, H, N):
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, H, N, 128) < N
    rng = np.random.default_rng(9)
    kv_in = (rng.standard_normal((1, H, 128, 128)) * 0.5).astype(np.float32)
    exact, slopes, o, kv, _ = run(1, H, N, 66, device, kv_in=kv_in)
    o_ref, kv_ref, _ = oracle.recurrent(*exact, slopes, kv_in=kv_in)
    assert_close(o, o_ref, "bf16", f"O summaries ({H}x{N})", stored="bf16")
    assert_close(kv, kv_ref, "bf16", f"KV summaries ({H}x{N})")


@pytest.mark.parametrize("head_major", [False, True])
def test_packed_batch_on_wide_slices(device, head_major):
    # 64 heads over many tiles: the packed plan takes 64-column slices (its 32-column work spread
    # over the GPU exceeds 1.55x the longest tile chain), next to token-by-token and empty sequences
    from test_gpu_varlen import run_varlen

    run_varlen([1500, 700, 300, 65, 64, 9, 8, 1, 0, 2000], 64, 128, "bf16", device, head_major=head_major, seed=71)


def test_packed_chunked_on_wide_slices(device):
    # few heads, one long sequence: chunked (summaries on 32-column slices, main pass on 64)
    from test_gpu_varlen import run_varlen

    lengths = [6000, 2500, 40]
    assert la.la_prefill_varlen_chunk_tokens(la.LA_BF16, [0] + list(np.cumsum(lengths)), 3, 128) < 6000
    run_varlen(lengths, 3, 128, "bf16", device, seed=72)


# d = 64 keeps 32-column slices (two per head) in every plan; the same shapes as above


def test_d64_two_rounds_checkpoints_and_gate(device):
    B, H, N, d = 3, 48, 700, 64  # 144 pairs: 288 workgroups of 32 columns, more than one round
    assert la.la_prefill_chunk_tokens(la.LA_BF16, B, H, N, d) == N
    rng = np.random.default_rng(11)
    kv_in = (rng.standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    exact, slopes, o, kv, ck = run(B, H, N, 81, device, kv_in=kv_in, ckpt_every=128, d=d)
    o_ref, kv_ref, ck_ref = oracle.recurrent(*exact, slopes, kv_in=kv_in, ckpt_every=128)
    assert_close(o, o_ref, "bf16", "O d=64 one round", stored="bf16")
    assert_close(kv, kv_ref, "bf16", "KV d=64 one round")
    assert not np.isnan(ck).any()
    assert_close(ck.reshape(-1, *ck.shape[2:])[:, None], ck_ref.reshape(-1, *ck_ref.shape[2:])[:, None], "bf16",
                 "checkpoints d=64")
    import synth

    g = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits((rng.standard_normal((B, H, N, d)) * 2.0).astype(np.float32)))
    exact, slopes, o, kv, _ = run(B, H, N, 82, device, gate=g, d=d)
    o_pre, kv_ref, _ = oracle.recurrent(*exact, slopes)
    sg = oracle.sigmoid(g.astype(np.float64))
    excess = np.maximum(np.abs(o - o_pre * sg) - half_ulp(o, "bf16"), 0.0) / sg
    worst = max(float(excess[b, h].max()) / float(np.sqrt(np.mean(o_pre[b, h] ** 2)))
                for b in range(B) for h in range(H))
    assert worst <= TOL["bf16"], f"gated d=64: {worst:.3e}"
    assert_close(kv, kv_ref, "bf16", "KV gated d=64")


@pytest.mark.parametrize("H,N", [(64, 3000), (2, 9000)])
def test_d64_chunked(device, H, N):
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, H, N, 64) < N
    rng = np.random.default_rng(12)
    kv_in = (rng.standard_normal((1, H, 64, 64)) * 0.5).astype(np.float32)
    exact, slopes, o, kv, _ = run(1, H, N, 83, device, kv_in=kv_in, d=64)
    o_ref, kv_ref, _ = oracle.recurrent(*exact, slopes, kv_in=kv_in)
    assert_close(o, o_ref, "bf16", f"O d=64 chunked ({H}x{N})", stored="bf16")
    assert_close(kv, kv_ref, "bf16", f"KV d=64 chunked ({H}x{N})")


# Chunk summaries skip the tokens whose weight at their chunk's end, times the largest state the
# float16 input range allows, is below the smallest float32 denormal (fast-decaying heads skip most
# of every chunk); sub-chunks of 4096 tokens or more sit end to end over each head's window before
# its chunk's end, where the summary kernel and the prefix combine must agree.  The results must not
# change; the boosted cases put large values in the first half of every 1024-token block (the
# skipped tokens, for the fast heads) and small ones after them.


def _skip_case(device, H, N, slopes, boost, seed, what):
    import torch

    B, d = 1, 128
    exact, raw = inputs(seed, B, H, N, d, "bf16")
    if boost:
        # the first half of each 1024-token block scaled by 8, the rest by 1/8 (exact in bf16, and
        # within the float16 products' range)
        scale = np.where((np.arange(N) % 1024) < 512, 8.0, 1.0 / 8.0).astype(np.float32)[None, None, :, None]
        exact = [x * scale for x in exact]
        import synth

        raw = [synth.f32_to_bf16_bits(x) for x in exact]
    q, k, v = (to_device(x, "bf16", device) for x in raw)
    kv = torch.zeros(B, H, d, d, device=device)
    o = torch.empty_like(q)
    la.la_prefill(q, k, v, torch.from_numpy(slopes).to(device), kv, o=o)
    torch.cuda.synchronize()
    o_ref, kv_ref, _ = oracle.recurrent(*exact, slopes)
    assert_close(to_host(o), o_ref, "bf16", f"O {what} (boost={boost})", stored="bf16")
    assert_close(kv.cpu().numpy(), kv_ref, "bf16", f"KV {what} (boost={boost})")


@pytest.mark.parametrize("boost", [False, True])
def test_summaries_skip_decayed_tokens(device, boost):
    # 1280-token chunks in two sub-chunks each, split evenly
    H, N = 4, 40000
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, H, N, 128) < N
    _skip_case(device, H, N, np.array([0.5, 0.05, 2.0 ** -6, 2.0 ** -9], dtype=np.float32), boost, 67,
               "skipped summaries")


@pytest.mark.parametrize("boost", [False, True])
def test_summaries_over_decay_windows(device, boost):
    # 8192-token chunks in two 4096-token sub-chunks: long enough that each head's two sub-chunks
    # sit over its window before the chunk's end (for the 0.5 and 0.05 heads a few hundred and
    # ~2600 tokens, for 2^-6 and 2^-9 the whole chunk), and the prefix combine places them alike
    H, N = 16, 65536
    assert la.la_prefill_chunk_tokens(la.LA_BF16, 1, H, N, 128) == 8192
    assert la.la_prefill_workspace_size(la.LA_BF16, 1, H, N, 128) == H * (8 + 1 + 7 * 2) * 128 * 128 * 4
    slopes = np.tile(np.array([0.5, 0.05, 2.0 ** -6, 2.0 ** -9], dtype=np.float32), 4)
    _skip_case(device, H, N, slopes, boost, 68, "summaries over windows")
