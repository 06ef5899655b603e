"""Parity at the full workload sizes, in the launch configuration the benchmark times.

* share  (1 x 8 heads x 32768 tokens, bf16): every output and final state against the oracle.
* full   (1 x 64 heads x 131072 tokens, bf16): sampled windows and every final state; the same
  shape at head dimension 64 too.
* long   (1 x 8 heads x 1,048,576 tokens, bf16, checkpoints every 65536): checkpoints, final
  states and output windows (including the chunk boundaries of the LASP+-style split).
* decode (128 sequences x 64 heads, 4096-token prefix then decode steps): sampled (seq, head).
* varlen (the full layer's tokens cut into 18 packed sequences of 65536, 32768, ..., 1, 1 tokens,
  as the benchmark times them): every final state and sampled output windows of every sequence.
* backward of the full layer: dq on forward windows, dk and dv on reverse windows (G_t depends on
  the next W tokens), dL/dKV_in on the first W tokens.

Windows use the oracle's windowing pin: for slopes s >= 2^-8 the state is fixed by the last
W = 8192 tokens up to lambda^W <= e^-32 (relative), far below the bars, so a window's outputs are
recomputed from a zero state W tokens earlier.
"""
import numpy as np
import pytest

import long_context_la_amd as la
import oracle
import synth
from common import assert_close, to_host

pytestmark = pytest.mark.gpu

WINDOW = 8192


def _torch():
    import torch

    return torch


def upload(w, device, head_group=8, t0=0, nt=None):
    torch = _torch()
    nt = w.n if nt is None else nt
    out = []
    for t in (synth.Q, synth.K, synth.V):
        dev = torch.empty((w.batch, w.heads, nt, w.d), dtype=torch.bfloat16, device=device)
        for h0 in range(0, w.heads, head_group):
            nh = min(head_group, w.heads - h0)
            bits = synth.generate(t, w.seed, w.d, nb=w.batch, h0=h0, nh=nh, t0=t0, nt=nt, dtype="bf16")
            dev[:, h0:h0 + nh] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
        out.append(dev)
    return out


def exact(w, b, h, t0, nt):
    """Exact (float32) Q, K, V of one (batch, head) for tokens t0..t0+nt-1, shaped [1,1,nt,d]."""
    return [synth.bf16_bits_to_f32(synth.generate(t, w.seed, w.d, b0=b, nb=1, h0=h, nh=1, t0=t0, nt=nt,
                                                  dtype="bf16")) for t in (synth.Q, synth.K, synth.V)]


def window_reference(w, b, h, end, length, slopes):
    """Oracle outputs for tokens end-length..end-1 and the state after token end-1, from a zero
    state at max(0, end-length-WINDOW)."""
    return windows_reference(w, [(b, h, end)], length, slopes)[0]


def windows_reference(w, items, length, slopes):
    """window_reference for many (b, h, end) at once (one oracle call, threaded over the rows)."""
    span = length + WINDOW
    rows = [[], [], []]
    row_slopes = []
    for b, h, end in items:
        start = max(0, end - span)
        parts = exact(w, b, h, start, end - start)
        for i in range(3):
            x = parts[i][0, 0]
            if x.shape[0] < span:  # sequence start: zero-pad in front (zero tokens leave the state at 0)
                x = np.concatenate([np.zeros((span - x.shape[0], w.d), np.float32), x])
            rows[i].append(x)
        row_slopes.append(slopes[h])
    q, k, v = (np.stack(r)[None] for r in rows)
    o, kv, _ = oracle.recurrent(q, k, v, np.array(row_slopes, dtype=np.float64))
    return [(o[0, r, -length:], kv[0, r]) for r in range(len(items))]


def run_prefill(w, q, k, v, device, ckpt_every=0):
    torch = _torch()
    slopes = torch.from_numpy(w.slopes()).to(device)
    kv = torch.zeros(w.batch, w.heads, w.d, w.d, dtype=torch.float32, device=device)
    o = torch.empty_like(q)
    ck = None
    if ckpt_every:
        ck = torch.empty((w.batch, w.heads, w.n // ckpt_every, w.d, w.d), dtype=torch.float32, device=device)
    la.la_prefill(q, k, v, slopes, kv, o=o, ckpt=ck, ckpt_every=ckpt_every)
    torch.cuda.synchronize()
    return o, kv, ck


def test_share_workload_all_outputs(device):
    w = synth.WORKLOADS["share"]
    q, k, v = upload(w, device)
    o, kv, _ = run_prefill(w, q, k, v, device)
    assert la.la_prefill_chunk_tokens(la.LA_BF16, w.batch, w.heads, w.n, w.d) < w.n  # chunked path
    ex = [synth.bf16_bits_to_f32(synth.generate(t, w.seed, w.d, nh=w.heads, nt=w.n, dtype="bf16"))
          for t in (synth.Q, synth.K, synth.V)]
    o_ref, kv_ref, _ = oracle.recurrent(*ex, w.slopes())
    assert_close(to_host(o), o_ref, "bf16", "share O", stored="bf16")
    assert_close(kv.cpu().numpy(), kv_ref, "bf16", "share KV")


def test_full_layer_windows_and_states(device):
    w = synth.WORKLOADS["full"]
    slopes = w.slopes()
    q, k, v = upload(w, device)
    o, kv, _ = run_prefill(w, q, k, v, device)
    del q, k, v
    kv_h = kv.cpu().numpy()
    length = 256
    items = [(0, h, end) for h in (0, 21, 42, 63) for end in (256, 4096 + 37, 65536, w.n)]
    for (b, h, end), (o_ref, _) in zip(items, windows_reference(w, items, length, slopes)):
        got = to_host(o[0:1, h:h + 1, end - length:end])
        assert_close(got, o_ref[None, None], "bf16", f"full O head {h} tokens ..{end}", stored="bf16")
    items = [(0, h, w.n) for h in range(w.heads)]
    for (b, h, end), (_, kv_ref) in zip(items, windows_reference(w, items, 1, slopes)):
        assert_close(kv_h[0:1, h:h + 1], kv_ref[None, None], "bf16", f"full KV head {h}")


def test_full_layer_d64_windows_and_states(device):
    # the full layer's shape at head dimension 64 (2 value slices per head, so the sequences are
    # cut into chunks to fill the GPU): sampled windows across the chunk boundary, every state
    w = synth.WORKLOADS["full_d64"]
    slopes = w.slopes()
    chunk = la.la_prefill_chunk_tokens(la.LA_BF16, w.batch, w.heads, w.n, w.d)
    assert chunk < w.n
    q, k, v = upload(w, device)
    o, kv, _ = run_prefill(w, q, k, v, device)
    del q, k, v
    kv_h = kv.cpu().numpy()
    length = 256
    items = [(0, h, end) for h in (0, 37, 63) for end in (256, chunk, chunk + 256, w.n)]
    for (b, h, end), (o_ref, _) in zip(items, windows_reference(w, items, length, slopes)):
        got = to_host(o[0:1, h:h + 1, end - length:end])
        assert_close(got, o_ref[None, None], "bf16", f"d=64 O head {h} tokens ..{end}", stored="bf16")
    items = [(0, h, w.n) for h in range(w.heads)]
    for (b, h, end), (_, kv_ref) in zip(items, windows_reference(w, items, 1, slopes)):
        assert_close(kv_h[0:1, h:h + 1], kv_ref[None, None], "bf16", f"d=64 KV head {h}")


def test_long_context_checkpoints_and_boundaries(device):
    w = synth.WORKLOADS["long"]
    slopes = w.slopes()
    q, k, v = upload(w, device, head_group=2)
    o, kv, ck = run_prefill(w, q, k, v, device, ckpt_every=w.ckpt_every)
    del q, k, v
    chunk = la.la_prefill_chunk_tokens(la.LA_BF16, w.batch, w.heads, w.n, w.d)
    assert chunk < w.n
    ck_h = ck.cpu().numpy()
    kv_h = kv.cpu().numpy()
    cks = [(h, m) for h in range(w.heads) for m in ((0, 1, 7, 8, 15) if h in (0, 7) else (5,))]
    items = [(0, h, (m + 1) * w.ckpt_every) for h, m in cks]
    for (h, m), (_, kv_ref) in zip(cks, windows_reference(w, items, 1, slopes)):
        assert_close(ck_h[0:1, h:h + 1, m], kv_ref[None, None], "bf16", f"long ckpt {m} head {h}")
    items = [(0, h, w.n) for h in range(w.heads)]
    for (b, h, end), (_, kv_ref) in zip(items, windows_reference(w, items, 1, slopes)):
        assert_close(kv_h[0:1, h:h + 1], kv_ref[None, None], "bf16", f"long KV head {h}")
    length = 128
    items = [(0, h, end) for h in (0, 3, 7) for end in (chunk + 64, 3 * chunk + 1, 5 * chunk - 7, w.n)]
    for (b, h, end), (o_ref, _) in zip(items, windows_reference(w, items, length, slopes)):
        got = to_host(o[0:1, h:h + 1, end - length:end])
        assert_close(got, o_ref[None, None], "bf16", f"long O head {h} tokens ..{end}", stored="bf16")


def test_decode_workload_sampled_units(device):
    torch = _torch()
    w = synth.WORKLOADS["decode"]
    B, H, d, P, steps = w.batch, w.heads, w.d, w.n, 12
    slopes = w.slopes()
    ts = torch.from_numpy(slopes).to(device)
    kv = torch.empty(B, H, d, d, dtype=torch.float32, device=device)
    la.la_state_init(kv)
    for b0 in range(0, B, 16):
        kk = torch.from_numpy(synth.generate(synth.K, w.seed, d, b0=b0, nb=16, nh=H, nt=P, dtype="bf16")
                              .view(np.int16)).view(torch.bfloat16).to(device)
        vv = torch.from_numpy(synth.generate(synth.V, w.seed, d, b0=b0, nb=16, nh=H, nt=P, dtype="bf16")
                              .view(np.int16)).view(torch.bfloat16).to(device)
        la.la_prefill(kk, kk, vv, ts, kv[b0:b0 + 16], o=None)
        del kk, vv
    outs = []
    for s in range(steps):
        qkv = [torch.from_numpy(synth.generate(t, w.seed, d, nb=B, nh=H, t0=P + s, nt=1, dtype="bf16")[:, :, 0]
                                .view(np.int16).copy()).view(torch.bfloat16).to(device)
               for t in (synth.Q, synth.K, synth.V)]
        o = torch.empty_like(qkv[0])
        la.la_decode(*qkv, ts, kv, o)
        outs.append(o)
    torch.cuda.synchronize()
    o_all = torch.stack(outs, dim=2).float().cpu().numpy()  # [B,H,steps,d]
    kv_h = kv.cpu().numpy()
    units = ((0, 0), (0, 63), (17, 5), (64, 31), (101, 47), (127, 12), (127, 63), (55, 0))
    parts = [exact(w, b, h, 0, P + steps) for b, h in units]
    q, k, v = (np.concatenate([p[i] for p in parts], axis=1) for i in range(3))
    o_ref, kv_ref, _ = oracle.recurrent(q, k, v, np.array([slopes[h] for _, h in units], dtype=np.float64))
    for r, (b, h) in enumerate(units):
        assert_close(o_all[b:b + 1, h:h + 1], o_ref[:, r:r + 1, P:], "bf16", f"decode o ({b},{h})", stored="bf16")
        assert_close(kv_h[b:b + 1, h:h + 1], kv_ref[:, r:r + 1], "bf16", f"decode KV ({b},{h})")


def seq_windows_reference(w, items, length, slopes):
    """Like windows_reference for sequences packed inside the workload's token axis: item
    (h, seq_start, end) restarts the recurrence from zero at seq_start, so a window's reference
    runs from max(seq_start, end - length - WINDOW); zero tokens pad the front of short ones."""
    span = length + WINDOW
    rows = [[], [], []]
    row_slopes = []
    for h, seq_start, end in items:
        start = max(seq_start, end - span)
        parts = exact(w, 0, h, start, end - start)
        for i in range(3):
            x = parts[i][0, 0]
            if x.shape[0] < span:
                x = np.concatenate([np.zeros((span - x.shape[0], w.d), np.float32), x])
            rows[i].append(x)
        row_slopes.append(slopes[h])
    q, k, v = (np.stack(r)[None] for r in rows)
    o, kv, _ = oracle.recurrent(q, k, v, np.array(row_slopes, dtype=np.float64))
    return [(o[0, r, -length:], kv[0, r]) for r in range(len(items))]


def test_varlen_packed_full_layer(device):
    import bench

    torch = _torch()
    w = synth.WORKLOADS["full"]
    slopes = w.slopes()
    q, k, v = upload(w, device)
    o = torch.empty_like(q)
    lengths = bench.VARLEN_LENGTHS
    cu = [0] + list(np.cumsum(lengths))
    n_seq = len(lengths)
    kv = torch.zeros(n_seq, w.heads, w.d, w.d, dtype=torch.float32, device=device)
    la.la_prefill_varlen(q[0].permute(1, 0, 2), k[0].permute(1, 0, 2), v[0].permute(1, 0, 2),
                         torch.from_numpy(slopes).to(device), kv, cu, o=o[0].permute(1, 0, 2))
    torch.cuda.synchronize()
    del q, k, v
    kv_h = kv.cpu().numpy()
    heads = (0, 9, 33, 63)
    # final states of every sequence (four heads each)
    items = [(h, cu[s], cu[s + 1]) for s in range(n_seq) for h in heads]
    for (h, s0, end), (_, kv_ref) in zip(items, seq_windows_reference(w, items, 1, slopes)):
        s = cu.index(s0)
        assert_close(kv_h[s:s + 1, h:h + 1], kv_ref[None, None], "bf16", f"varlen KV seq {s} head {h}")
    # the last (up to) 64 outputs of every sequence, and a window inside the longest
    items = [(h, cu[s], cu[s + 1]) for s in range(n_seq) for h in heads[:2]] + [(21, 0, 40000)]
    for (h, s0, end), (o_ref, _) in zip(items, seq_windows_reference(w, items, 64, slopes)):
        n = min(64, end - s0)
        got = to_host(o[0:1, h:h + 1, end - n:end])
        assert_close(got, o_ref[None, None, 64 - n:], "bf16", f"varlen O head {h} tokens ..{end}", stored="bf16")



def test_backward_full_layer_windows(device):
    """la_backward on the full layer as the benchmark times it (64 heads x 131072 tokens, bf16,
    dL/dO from the generator).  dq at token t depends on the forward state (the last W tokens), dk
    and dv on G_t (the next W tokens), dL/dKV_in on G_0 (the first W tokens), so each is checked
    on windows: forward windows for dq, reverse windows for dk and dv."""
    torch = _torch()
    w = synth.WORKLOADS["full"]
    slopes = w.slopes()
    q, k, v = upload(w, device)
    seed_do = w.seed + 1000
    do = torch.empty_like(q)
    for h0 in range(0, w.heads, 8):
        bits = synth.generate(synth.V, seed_do, w.d, h0=h0, nh=8, nt=w.n, dtype="bf16")
        do[:, h0:h0 + 8] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    dq, dk, dv, dkv = la.la_backward(q, k, v, do, torch.from_numpy(slopes).to(device))
    torch.cuda.synchronize()
    del q, k, v, do

    def inputs_of(h, t0, nt):
        x = exact(w, 0, h, t0, nt)
        g = synth.bf16_bits_to_f32(synth.generate(synth.V, seed_do, w.d, h0=h, nh=1, t0=t0, nt=nt, dtype="bf16"))
        return x + [g]

    length = 128
    sl = lambda h: np.array([slopes[h]])
    for h in (0, 31, 63):
        for end in (length, 70000, w.n):
            start = max(0, end - length - WINDOW)
            ref = oracle.backward_recurrent(*inputs_of(h, start, end - start), sl(h))
            got = to_host(dq[0:1, h:h + 1, end - length:end])
            assert_close(got, ref[0][:, :, -length:], "bf16", f"full dq head {h} tokens ..{end}", stored="bf16")
        for begin in (0, 70000, w.n - length):
            stop = min(w.n, begin + length + WINDOW)
            ref = oracle.backward_recurrent(*inputs_of(h, begin, stop - begin), sl(h))
            for name, t, r in (("dk", dk, ref[1]), ("dv", dv, ref[2])):
                got = to_host(t[0:1, h:h + 1, begin:begin + length])
                assert_close(got, r[:, :, :length], "bf16", f"full {name} head {h} tokens {begin}..", stored="bf16")
            if begin == 0:
                assert_close(dkv[0:1, h:h + 1].cpu().numpy(), ref[3], "bf16", f"full dKV_in head {h}")


def test_maximum_units_prefill_then_decode(device):
    # batch * heads at the documented maximum of 2^20 units (16384 sequences x 64 heads, d = 64):
    # a 3-token prefill (one ragged tile per unit) and then one decode step, checked against the
    # oracle's 4-token recurrence on sampled units, the first and the last among them
    import torch

    B, H, N, d, seed = 16384, 64, 3, 64, 23
    slopes = np.array([2.0 ** (-(h + 1) / 8) for h in range(H)], dtype=np.float32)
    pre = [synth.generate(t, seed, d, nb=B, nh=H, nt=N, dtype="bf16") for t in (synth.Q, synth.K, synth.V)]
    step = [synth.generate(t, seed, d, nb=B, nh=H, t0=N, nt=1, dtype="bf16")[:, :, 0] for t in (synth.Q, synth.K, synth.V)]

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)

    q, k, v = (up(x) for x in pre)
    o = torch.empty_like(q)
    kv = torch.empty(B, H, d, d, dtype=torch.float32, device=device)
    sl = torch.from_numpy(slopes).to(device)
    la.la_state_init(kv)
    la.la_prefill(q, k, v, sl, kv, o=o)
    del q, k, v
    qd, kd, vd = (up(x) for x in step)
    od = torch.empty_like(qd)
    la.la_decode(qd, kd, vd, sl, kv, od)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    units = [0, 1, H - 1, 4097, (1 << 19) + 13, (1 << 20) - 1] + [int(u) for u in rng.integers(0, B * H, 10)]
    for u in units:
        b, h = divmod(u, H)
        ex = [synth.bf16_bits_to_f32(np.concatenate([p[b, h], s[b, h][None]])[None, None]) for p, s in zip(pre, step)]
        o_ref, kv_ref, _ = oracle.recurrent(*ex, slopes[h:h + 1])
        what = f"unit {u} (b={b}, h={h})"
        assert_close(to_host(o[b:b + 1, h:h + 1]), o_ref[:, :, :N], "bf16", f"prefill O {what}", stored="bf16")
        assert_close(to_host(od[b:b + 1, h:h + 1])[:, :, None], o_ref[:, :, N:], "bf16", f"decode o {what}",
                     stored="bf16")
        assert_close(kv[b:b + 1, h:h + 1].cpu().numpy(), kv_ref, "bf16", f"KV {what}")


def test_maximum_units_packed_short_sequences(device):
    # n_seq * heads at the documented maximum of 2^20 (16384 packed sequences x 64 heads, d = 64),
    # every sequence 1..8 tokens long (the token-by-token launch, one workgroup per unit, plus a
    # few empty ones), from random incoming states; sampled sequences against the oracle
    import torch

    S, H, d, seed = 16384, 64, 64, 29
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 9, S)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    slopes = np.array([2.0 ** (-(h + 1) / 8) for h in range(H)], dtype=np.float32)
    raw = [synth.generate(t, seed, d, nh=H, nt=T, dtype="bf16")[0].transpose(1, 0, 2) for t in (synth.Q, synth.K, synth.V)]

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)

    q, k, v = (up(x) for x in raw)  # [T, H, d]
    o = torch.zeros_like(q)
    kv = torch.randn(S, H, d, d, generator=torch.Generator(device=device).manual_seed(seed), device=device)
    picks = [0, 1, S // 2, S - 1] + [int(s) for s in rng.integers(0, S, 12)] + [int(np.argmin(lens))]
    kv0 = {s: kv[s].cpu().numpy() for s in picks}
    la.la_prefill_varlen(q, k, v, torch.from_numpy(slopes).to(device), kv, cu, o=o)
    torch.cuda.synchronize()
    for s in picks:
        a, b = int(cu[s]), int(cu[s + 1])
        what = f"sequence {s} ({b - a} tokens)"
        if b == a:
            assert np.array_equal(kv[s].cpu().numpy(), kv0[s]), f"{what}: an empty sequence changed its state"
            continue
        ex = [synth.bf16_bits_to_f32(np.ascontiguousarray(x[a:b].transpose(1, 0, 2))[None]) for x in raw]
        o_ref, kv_ref, _ = oracle.recurrent(*ex, slopes, kv_in=kv0[s][None])
        assert_close(np.ascontiguousarray(to_host(o[a:b]).transpose(1, 0, 2))[None], o_ref, "bf16", f"O {what}",
                     stored="bf16")
        assert_close(kv[s].cpu().numpy()[None], kv_ref, "bf16", f"KV {what}")
