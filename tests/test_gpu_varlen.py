"""GPU parity of the packed variable-length prefill and of the two-stream mixed step against
the fp64 oracle, run sequence by sequence.

The page "MiniMax-01: Scaling Foundation Models with Lightning Attention | Summary" packs
variable-length samples back to back (section 3.2) and, in section 3.3, runs single-token
generation and longer inputs as separate kernels on separate streams.  Each packed sequence
must equal the recurrence run on that sequence alone, from its own incoming state; empty
sequences leave their state unchanged.  Bars as in test_gpu_parity.py.
"""
import numpy as np
import pytest

import long_context_la_amd as la
import oracle
import synth
from common import TOL, assert_close, to_host

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    return torch


def packed_inputs(seed, lengths, H, d, dtype):
    """Sequence s = generator batch index s, tokens 0..n_s-1.  Returns per-sequence exact
    [1,H,n,d] arrays and the packed device-layout arrays [T,H,d] (float32 or bf16 bits)."""
    exact, packed = [], [[], [], []]
    for s, n in enumerate(lengths):
        parts = []
        for i, t in enumerate((synth.Q, synth.K, synth.V)):
            raw = synth.generate(t, seed, d, b0=s, nb=1, nh=H, t0=0, nt=n, dtype=dtype)
            packed[i].append(np.transpose(raw[0], (1, 0, 2)))
            parts.append(synth.bf16_bits_to_f32(raw) if dtype == "bf16" else raw)
        exact.append(parts)
    return exact, [np.ascontiguousarray(np.concatenate(p, axis=0)) for p in packed]


def to_dev(arr, dtype, device):
    torch = _torch()
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(arr).to(device)


def slopes_for(H):
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)


def initial_states(lengths, H, d, seed):
    rng = np.random.default_rng(seed)
    kv = np.zeros((len(lengths), H, d, d), dtype=np.float32)
    for s in range(len(lengths)):
        if s % 2 == 1:
            kv[s] = rng.standard_normal((H, d, d)).astype(np.float32) * 4.0
    return kv


def run_varlen(lengths, H, d, dtype, device, chunk_tokens=0, head_major=False, want_o=True, seed=11):
    torch = _torch()
    exact, packed = packed_inputs(seed, lengths, H, d, dtype)
    T = sum(lengths)
    if head_major:  # storage [H, T, d]; the call sees a [T, H, d] view with stride_h = T*d
        q, k, v = (to_dev(np.ascontiguousarray(np.transpose(p, (1, 0, 2))), dtype, device).permute(1, 0, 2)
                   for p in packed)
    else:
        q, k, v = (to_dev(p, dtype, device) for p in packed)
    kv0 = initial_states(lengths, H, d, seed + 1)
    kv = torch.from_numpy(kv0.copy()).to(device)
    o = (torch.empty_like(q) if not head_major else torch.empty((H, T, d), dtype=q.dtype, device=device).permute(1, 0, 2)) \
        if want_o else None
    slopes = slopes_for(H)
    cu = [0] + list(np.cumsum(lengths))
    la.la_prefill_varlen(q, k, v, torch.from_numpy(slopes).to(device), kv, cu, o=o, chunk_tokens=chunk_tokens)
    torch.cuda.synchronize()
    o_h = to_host(o) if want_o else None
    kv_h = kv.cpu().numpy()
    for s, n in enumerate(lengths):
        if n == 0:
            assert np.array_equal(kv_h[s], kv0[s]), f"empty sequence {s} changed its state"
            continue
        o_ref, kv_ref, _ = oracle.recurrent(*exact[s], slopes, kv_in=kv0[s:s + 1])
        what = f"seq {s} (n={n}, d={d}, {dtype}, chunk={chunk_tokens}, head_major={head_major})"
        if want_o:
            got = np.transpose(o_h[cu[s]:cu[s + 1]], (1, 0, 2))[None]
            assert_close(got, o_ref, dtype, "O " + what, stored=dtype)
        assert_close(kv_h[s:s + 1], kv_ref, dtype, "KV " + what)


LENGTHS = [0, 1, 5, 64, 65, 200, 1000, 1500]


@pytest.mark.parametrize("i", range(10))
def test_varlen_sweep(device, i):
    # seeded random packed batches: sequence count and lengths (empty, token by token, tiled, cut
    # into chunks), heads, dtype and d, explicit chunk lengths, layout, with and without outputs
    rng = np.random.default_rng(5000 + i)
    dtype, d = [("bf16", 128), ("f32", 128), ("f32", 64), ("bf16", 64)][rng.integers(4)]
    n_seq = int(rng.integers(1, 9))
    lengths = [int([0, rng.integers(1, 9), rng.integers(9, 300), rng.integers(300, 3000)][k])
               for k in rng.integers(0, 4, n_seq)]
    if sum(lengths) == 0:
        lengths[0] = 1
    H = int(rng.integers(1, 4))
    chunk = int(rng.choice([0, 64, 256, 1024]))
    run_varlen(lengths, H, d, dtype, device, chunk_tokens=chunk, head_major=bool(rng.random() < 0.5),
               want_o=bool(rng.random() < 0.8), seed=6000 + i)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 128), ("f32", 64), ("bf16", 64)])
def test_varlen_mixed_lengths(device, dtype, d):
    run_varlen(LENGTHS, 4, d, dtype, device)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_forced_chunks(device, dtype):
    run_varlen([700, 3, 129, 0, 1024, 64], 3, 128 if dtype == "bf16" else 64, dtype, device, chunk_tokens=128)


def test_varlen_long_sequence_default_chunks(device):
    # one sequence long enough to be chunked by the default plan next to short ones
    lengths = [9000, 17, 300]
    assert la.la_prefill_varlen_chunk_tokens(la.LA_BF16, [0] + list(np.cumsum(lengths)), 2, 128) < 9000
    run_varlen(lengths, 2, 128, "bf16", device)


def test_varlen_head_major_layout(device):
    run_varlen([130, 70, 1], 4, 128, "bf16", device, chunk_tokens=64, head_major=True)


def test_varlen_state_only(device):
    run_varlen([256, 33, 0, 500], 2, 128, "bf16", device, chunk_tokens=128, want_o=False)


def test_mixed_step_two_streams(device):
    """The page's example shape: a batch of 20 cached inputs, two of them 50-token inputs and
    the rest single-token; decode and varlen prefill run on two streams."""
    torch = _torch()
    H, d, dtype = 8, 128, "bf16"
    slopes = slopes_for(H)
    ts = torch.from_numpy(slopes).to(device)
    # decode group: 18 sequences with cached states, one token each
    nd = 18
    kv0_d = initial_states([1] * nd, H, d, 5) + 0.5
    raw = [synth.generate(t, 21, d, nb=nd, nh=H, t0=0, nt=1, dtype=dtype)[:, :, 0] for t in (synth.Q, synth.K, synth.V)]
    ex = [synth.bf16_bits_to_f32(r) for r in raw]
    qd, kd, vd = (to_dev(np.ascontiguousarray(r), dtype, device) for r in raw)
    od = torch.empty_like(qd)
    kvd = torch.from_numpy(kv0_d.copy()).to(device)
    # prefill group: two 50-token inputs continuing cached states
    lengths = [50, 50]
    exact, packed = packed_inputs(22, lengths, H, d, dtype)
    qp, kp, vp = (to_dev(p, dtype, device) for p in packed)
    op = torch.empty_like(qp)
    kv0_p = initial_states(lengths, H, d, 23) + 0.25
    kvp = torch.from_numpy(kv0_p.copy()).to(device)
    cu = [0, 50, 100]
    ws = torch.empty(la.la_prefill_varlen_workspace_size(la.LA_BF16, cu, H, d), dtype=torch.uint8, device=device)
    la.mixed_step(ts, decode=(qd, kd, vd, od, kvd), prefill=(qp, kp, vp, op, kvp, cu, ws),
                  streams=(torch.cuda.Stream(), torch.cuda.Stream()))
    torch.cuda.synchronize()
    # decode group against the oracle's decode step
    kv_ref = kv0_d.astype(np.float64)
    o_ref = oracle.decode_step(ex[0], ex[1], ex[2], slopes, kv_ref)
    assert_close(to_host(od)[:, :, None], o_ref[:, :, None], dtype, "mixed step decode O", stored=dtype)
    assert_close(kvd.cpu().numpy(), kv_ref, dtype, "mixed step decode KV")
    # prefill group against the recurrence
    o_h = to_host(op)
    for s in range(2):
        o_r, kv_r, _ = oracle.recurrent(*exact[s], slopes, kv_in=kv0_p[s:s + 1])
        assert_close(np.transpose(o_h[cu[s]:cu[s + 1]], (1, 0, 2))[None], o_r, dtype, f"mixed step prefill O {s}",
                     stored=dtype)
        assert_close(kvp.cpu().numpy()[s:s + 1], kv_r, dtype, f"mixed step prefill KV {s}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_varlen_short_sequences(device, dtype, d):
    # 1..8 tokens run token by token, 9 and more in 64-token tiles; the boundary on both sides
    run_varlen([1, 8, 9, 2, 0, 7, 3], 3, d, dtype, device)


def test_varlen_short_sequences_state_only(device):
    run_varlen([4, 1, 8], 2, 128, "bf16", device, want_o=False)
