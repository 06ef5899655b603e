"""Benchmark: Lightning Attention prefill and decode on one MI355X.

Workload of the headline number: full-layer prefill, batch 1, 64 heads, head dim 128,
131072 tokens, bf16 Q/K/V/O, fp32 state (the 64-head d=128 lightning layer of the
MiniMax-01 pages at 128K context), seeded synthetic activations.  One step = one
la_prefill over that batch (tile scores, masking, intra/inter terms, state
recurrence, output write, final state).  The decode leg times 1000 consecutive
la_decode steps on 128 sequences x 64 heads whose states were preloaded from a
4096-token seeded prefix; it is reported as "decode" in the same JSON line.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (datasheet); the run's peaks come from device_peaks()
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (datasheet), replaced at run time
MODEL_TILE = 256               # the pages' tile: flop model 4*B*d + 4*d^2 per token-head
BYTES_PER_TOKEN_HEAD = 4 * 128 * 2   # q, k, v read + o write, bf16, d = 128
BWD_BYTES_PER_TOKEN_HEAD = 7 * 128 * 2  # backward: q, k, v, dO read + dq, dk, dv write, bf16
DECODE_BYTES_PER_UNIT = 2 * 128 * 128 * 4 + 4 * 128 * 2   # state read + write, q/k/v/o


# Packed variable-length leg: the full layer's 131072-token budget split into 18 sequences of
# halving lengths (65536 ... 1, plus one more single token), packed back to back in one launch.
VARLEN_LENGTHS = [65536 >> i for i in range(17)] + [1]
# Mixed batch of the pages' example: 20 cached inputs, two of them 50 tokens, the rest one token.
MIXED_LENGTHS = [50, 50] + [1] * 18

PROFILES = os.path.join(ROOT, "profiles")
PREFILL_SOURCE = os.path.join(ROOT, "long_context_la_amd", "csrc", "la_prefill_bf16.hip")
FLUSH_BYTES = 512 << 20   # read between timed steps of the cache-sized legs (256 MB Infinity Cache)


def source_digest(path=PREFILL_SOURCE):
    from long_context_la_amd import profiling

    return profiling.source_digest(path)


def measured_traffic(workload):
    """HBM bytes per prefill launch from the committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE per dispatch, each scaled by the same counter's reading for a plain copy of known
    size), or None when there is none for this workload or the kernel source changed since."""
    from long_context_la_amd import profiling

    return profiling.current_value(os.path.join(PROFILES, f"prefill_{workload}_hbm_traffic.txt"), "traffic_bytes")


def measured_mfma():
    """Counter-based MFMA utilisation and cycles per tile of the full-layer prefill kernel from the
    committed rocprofv3 summary, or None when the kernel source changed since it was taken."""
    from long_context_la_amd import profiling

    path = os.path.join(PROFILES, "prefill_full_mfma_util.txt")
    util = profiling.current_value(path, "mfma_utilisation")
    if util is None:
        return None
    return {"mfma_utilisation": util, "cycles_per_tile": profiling.current_value(path, "cycles_per_tile"),
            "source": "profiles/prefill_full_mfma_util.txt"}


def copy_probe(device, gib=4, reps=3):
    """A plain device copy of known size, for calibrating the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device=device).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "reps": reps}), flush=True)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


SETTLE_S = 0.2  # seconds of untimed steps before each leg's warm-up (--settle-s)


def set_settle(seconds):
    global SETTLE_S
    SETTLE_S = max(0.0, float(seconds))


def settle(fn, seconds=None, batch=4):
    """Runs `fn` (one untimed step) for about `seconds` of wall time before a leg's warm-up.
    After the GPU idles (input generation on the host), its clock climbs over the first ~15
    launches of the full-layer prefill (~5.6 ms for the first step, ~2.6 ms from about the 15th);
    the timed steps should see the clock that a continuous workload runs at."""
    import torch

    seconds = SETTLE_S if seconds is None else seconds
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
        n += batch
    return n


def model_flops_per_token_head(d=128, B=MODEL_TILE):
    return 4 * B * d + 4 * d * d


def upload_bf16(bits, device):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def make_prefill_inputs(w, device, head_group=8):
    import torch

    import synth

    shape = (w.batch, w.heads, w.n, w.d)
    out = []
    for t in (synth.Q, synth.K, synth.V):
        dev = torch.empty(shape, dtype=torch.bfloat16, device=device)
        for h0 in range(0, w.heads, head_group):
            nh = min(head_group, w.heads - h0)
            bits = synth.generate(t, w.seed, w.d, nb=w.batch, h0=h0, nh=nh, nt=w.n, dtype="bf16")
            dev[:, h0:h0 + nh] = upload_bf16(bits, device)
        out.append(dev)
    return out


def time_prefill(w, steps, warmup, device, with_backward=True, with_varlen=True, flush=False):
    import torch

    import long_context_la_amd as la

    log(f"generating {w.name} inputs {w.batch}x{w.heads}x{w.n}x{w.d} bf16")
    t0 = time.time()
    q, k, v = make_prefill_inputs(w, device)
    log(f"inputs ready in {time.time() - t0:.1f} s")
    slopes = torch.from_numpy(w.slopes()).to(device)
    kv = torch.zeros(w.batch, w.heads, w.d, w.d, dtype=torch.float32, device=device)
    o = torch.empty_like(q)
    ws_bytes = la.la_prefill_workspace_size(la.LA_BF16, w.batch, w.heads, w.n, w.d)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream(device)
    # the long-context workload keeps a state checkpoint every ckpt_every tokens
    ck = (torch.empty(w.batch, w.heads, w.n // w.ckpt_every, w.d, w.d, dtype=torch.float32, device=device)
          if w.ckpt_every else None)

    def step():
        la.la_state_init(kv)
        la.la_prefill(q, k, v, slopes, kv, o=o, ckpt=ck, ckpt_every=w.ckpt_every, workspace=ws)

    settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # flush: before each timed step (outside its events) a 512 MB buffer is read, so a workload
    # about the size of the 256 MB Infinity Cache starts every step from HBM, and the write-back of
    # the previous step's dirty lines happens before the step.  A flush that writes the buffer
    # instead leaves ~256 MB of dirty lines whose write-back then falls inside the next step; that
    # figure is reported beside it.
    junk = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device=device) if flush else None
    flush_write = None

    def flushed_steps(flush_op):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            flush_op()
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    if flush:
        ms = flushed_steps(lambda: junk.max())
        flush_write = flushed_steps(lambda: junk.fill_(1))
    else:
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
    # the prefill kernel(s) alone (state init excluded), timed on the same stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        la.la_state_init(kv)
        if flush:
            junk.max()
        a.record(stream)
        la.la_prefill(q, k, v, slopes, kv, o=o, ckpt=ck, ckpt_every=w.ckpt_every, workspace=ws)
        b.record(stream)
    torch.cuda.synchronize()
    kernel_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    del junk
    n_chunks = -(-w.n // la.la_prefill_chunk_tokens(la.LA_BF16, w.batch, w.heads, w.n, w.d))
    varlen = None
    if with_varlen and w.batch == 1 and sum(VARLEN_LENGTHS) == w.n:
        varlen = time_varlen_packed(q, k, v, o, slopes, w, steps, warmup, device)
    backward = time_backward(q, k, v, o, slopes, w, steps, warmup, device) if with_backward else None
    del q, k, v, o, ws
    return ms, kernel_ms, n_chunks, varlen, backward, flush_write


def time_backward(q, k, v, dout, slopes, w, steps, warmup, device):
    """la_backward over the same layer (the prefill's output stands in for dL/dO), with a
    dL/dKV_final, timed per call on the launch stream."""
    import torch

    import long_context_la_amd as la

    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    g = torch.ones(w.batch, w.heads, w.d, w.d, dtype=torch.float32, device=device)
    dkv = torch.empty_like(g)
    ws = torch.empty(la.la_backward_workspace_size(la.LA_BF16, w.batch, w.heads, w.n, w.d), dtype=torch.uint8,
                     device=device)
    stream = torch.cuda.current_stream(device)

    def call():
        la.la_backward(q, k, v, dout, slopes, dkv_out=g, dq=dq, dk=dk, dv=dv, dkv_in=dkv, workspace=ws)

    settle(call)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    th = w.batch * w.heads * w.n
    log(f"backward: {ms:.3f} ms ({th * BWD_BYTES_PER_TOKEN_HEAD / (ms * 1e-3) / 1e9:.0f} GB/s algorithmic)")
    del dq, dk, dv, ws
    return {"workload": f"backward of the {w.name} prefill: dq, dk, dv (bf16) and dL/dKV_in from dL/dO and "
                        f"dL/dKV_final",
            "ms_per_step": ms, "tokens_per_s": w.batch * w.n / (ms * 1e-3),
            "hbm_GBs": th * BWD_BYTES_PER_TOKEN_HEAD / (ms * 1e-3) / 1e9,
            "hbm_frac": th * BWD_BYTES_PER_TOKEN_HEAD / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "bytes_per_token_head": BWD_BYTES_PER_TOKEN_HEAD,
            "passes": 3, "pass_bytes_per_token_head": 3 * BYTES_PER_TOKEN_HEAD}


def time_varlen_packed(q, k, v, o, slopes, w, steps, warmup, device):
    """The same tokens cut into VARLEN_LENGTHS sequences: la_prefill_varlen on head-major views
    ([T,H,d] with stride_h = T*d), every sequence from a zero state."""
    import torch

    import long_context_la_amd as la

    qv, kv_, vv, ov = (t[0].permute(1, 0, 2) for t in (q, k, v, o))
    cu = [0] + list(np.cumsum(VARLEN_LENGTHS))
    n_seq = len(VARLEN_LENGTHS)
    kv = torch.zeros(n_seq, w.heads, w.d, w.d, dtype=torch.float32, device=device)
    ws = torch.empty(la.la_prefill_varlen_workspace_size(la.LA_BF16, cu, w.heads, w.d), dtype=torch.uint8,
                     device=device)
    stream = torch.cuda.current_stream(device)
    settle(lambda: la.la_prefill_varlen(qv, kv_, vv, slopes, kv, cu, o=ov, workspace=ws))
    for _ in range(warmup):
        la.la_prefill_varlen(qv, kv_, vv, slopes, kv, cu, o=ov, workspace=ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        la.la_state_init(kv)
        a.record(stream)
        la.la_prefill_varlen(qv, kv_, vv, slopes, kv, cu, o=ov, workspace=ws)
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    chunk = la.la_prefill_varlen_chunk_tokens(la.LA_BF16, cu, w.heads, w.d)
    log(f"varlen packed: {n_seq} sequences, {w.n} tokens: {ms:.3f} ms (chunk {chunk})")
    return {"workload": f"{n_seq} packed sequences ({VARLEN_LENGTHS[0]}..1 tokens, halving) = {w.n} tokens, "
                        f"{w.heads} heads, d={w.d}, bf16, zero incoming states",
            "ms_per_step": ms, "tokens_per_s": w.n / (ms * 1e-3),
            "hbm_GBs": BYTES_PER_TOKEN_HEAD * w.heads * w.n / (ms * 1e-3) / 1e9,
            "hbm_frac": BYTES_PER_TOKEN_HEAD * w.heads * w.n / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "chunk_tokens": chunk}


def time_mixed(device, heads=64, d=128, iters=200):
    """MIXED_LENGTHS for one layer: (a) all 20 sequences through one varlen prefill launch, (b) the
    18 single-token ones through la_decode and the two 50-token ones through la_prefill_varlen on
    two streams (mixed_step with two streams), (c) the same two calls one after the other on one
    stream (mixed_step's default)."""
    import torch

    import long_context_la_amd as la
    import synth

    def packed(lengths, seed):
        cu = [0] + list(np.cumsum(lengths))
        arrs = []
        for t in (synth.Q, synth.K, synth.V):
            parts = [synth.generate(t, seed, d, b0=s, nb=1, nh=heads, nt=n, dtype="bf16")[0].transpose(1, 0, 2)
                     for s, n in enumerate(lengths)]
            arrs.append(upload_bf16(np.ascontiguousarray(np.concatenate(parts, axis=0)), device))
        return arrs, cu

    slopes = torch.from_numpy(np.array([2.0 ** (-(h + 1) / 8) for h in range(heads)], dtype=np.float32)).to(device)
    long_n = [n for n in MIXED_LENGTHS if n > 1]
    n_short = len(MIXED_LENGTHS) - len(long_n)
    (qa, ka, va), cu_all = packed(MIXED_LENGTHS, 31)
    oa = torch.empty_like(qa)
    kv_all = torch.zeros(len(MIXED_LENGTHS), heads, d, d, dtype=torch.float32, device=device)
    ws_all = torch.empty(la.la_prefill_varlen_workspace_size(la.LA_BF16, cu_all, heads, d), dtype=torch.uint8,
                         device=device)
    (qp, kp, vp), cu_p = packed(long_n, 32)
    op = torch.empty_like(qp)
    kv_p = torch.zeros(len(long_n), heads, d, d, dtype=torch.float32, device=device)
    ws_p = torch.empty(la.la_prefill_varlen_workspace_size(la.LA_BF16, cu_p, heads, d), dtype=torch.uint8,
                       device=device)
    qd, kd, vd = (upload_bf16(synth.generate(t, 33, d, nb=n_short, nh=heads, nt=1, dtype="bf16")[:, :, 0], device)
                  for t in (synth.Q, synth.K, synth.V))
    od = torch.empty_like(qd)
    kv_d = torch.zeros(n_short, heads, d, d, dtype=torch.float32, device=device)
    streams = (torch.cuda.Stream(device), torch.cuda.Stream(device))
    variants = {
        "us_one_varlen_launch": lambda: la.la_prefill_varlen(qa, ka, va, slopes, kv_all, cu_all, o=oa, workspace=ws_all),
        "us_separate_streams": lambda: la.mixed_step(slopes, decode=(qd, kd, vd, od, kv_d),
                                                     prefill=(qp, kp, vp, op, kv_p, cu_p, ws_p), streams=streams),
        "us_separate_kernels_one_stream": lambda: la.mixed_step(slopes, decode=(qd, kd, vd, od, kv_d),
                                                                prefill=(qp, kp, vp, op, kv_p, cu_p, ws_p)),
    }
    res = {"workload": f"{len(MIXED_LENGTHS)} cached inputs: {len(long_n)} x {long_n[0]} tokens + {n_short} x 1 token, "
                       f"{heads} heads, d={d}, bf16 (one layer)"}
    stream = torch.cuda.current_stream(device)
    for name, fn in variants.items():
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) * 1e3 / iters
    log("mixed batch: " + ", ".join(f"{k} {v:.1f}" for k, v in res.items() if k.startswith("us")))
    return res


def time_decode_small(device, heads=64, d=128, steps=64, reps=20):
    """One sequence x 64 heads: a launch-bound decode.  Eager calls versus the same 64 steps
    captured once in a HIP graph (torch.cuda.CUDAGraph) and replayed."""
    import torch

    import long_context_la_amd as la

    gen = torch.Generator(device="cpu").manual_seed(61)
    q, k, v = (torch.randn(steps, 1, heads, d, generator=gen).to(torch.bfloat16).to(device) for _ in range(3))
    slopes = torch.from_numpy(np.exp2(-(np.arange(heads) + 1) / 8.0).astype(np.float32)).to(device)
    kv = torch.zeros(1, heads, d, d, dtype=torch.float32, device=device)
    o = torch.empty(steps, 1, heads, d, dtype=torch.bfloat16, device=device)

    def run():
        for t in range(steps):
            la.la_decode(q[t], k[t], v[t], slopes, kv, o[t])

    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    eager = (time.perf_counter() - t0) / (reps * steps) * 1e6
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    graph = (time.perf_counter() - t0) / (reps * steps) * 1e6
    log(f"small decode (1 x {heads} heads): eager {eager:.1f} us/step, graph {graph:.1f} us/step")
    return {"workload": f"1 seq x {heads} heads, d={d}, bf16; {steps} steps per graph", "us_per_step_eager": eager,
            "us_per_step_graph": graph}


def time_decode(w, steps, device, prefix_slab=16):
    import torch

    import long_context_la_amd as la
    import synth

    B, H, d, P = w.batch, w.heads, w.d, w.n
    slopes = torch.from_numpy(w.slopes()).to(device)
    kv = torch.empty(B, H, d, d, dtype=torch.float32, device=device)
    la.la_state_init(kv)
    log(f"decode: preloading {B}x{H} states from a {P}-token prefix")
    t0 = time.time()
    for b0 in range(0, B, prefix_slab):
        nb = min(prefix_slab, B - b0)
        kk = upload_bf16(synth.generate(synth.K, w.seed, d, b0=b0, nb=nb, nh=H, nt=P, dtype="bf16"), device)
        vv = upload_bf16(synth.generate(synth.V, w.seed, d, b0=b0, nb=nb, nh=H, nt=P, dtype="bf16"), device)
        la.la_prefill(kk, kk, vv, slopes, kv[b0:b0 + nb], o=None)  # state only: q is not read
        del kk, vv
    torch.cuda.synchronize()
    log(f"decode: prefix done in {time.time() - t0:.1f} s; generating {steps} step tokens")
    toks = []
    for t in (synth.Q, synth.K, synth.V):
        bits = synth.generate(t, w.seed, d, nb=B, nh=H, t0=P, nt=steps, dtype="bf16")  # [B,H,steps,d]
        toks.append(upload_bf16(np.ascontiguousarray(bits.transpose(2, 0, 1, 3)), device))  # [steps,B,H,d]
    o = torch.empty(B, H, d, dtype=torch.bfloat16, device=device)
    stream = torch.cuda.current_stream(device)
    # warm-up on a scratch copy of the state so the timed run starts from the preloaded one
    scratch = kv.clone()
    settle(lambda: la.la_decode(toks[0][0], toks[1][0], toks[2][0], slopes, scratch, o))
    for s in range(3):
        la.la_decode(toks[0][s], toks[1][s], toks[2][s], slopes, scratch, o)
    del scratch
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(steps):
        la.la_decode(toks[0][s], toks[1][s], toks[2][s], slopes, kv, o)
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / steps
    return us


def cpu_baseline_decode(wd, steps=10):
    """The oracle's decode step (fp64, OpenMP over the units) on all 128 x 64 units of the decode
    workload for `steps` steps from a random state, extrapolated to the 1000 timed steps.  The cost
    of a step does not depend on the state's values, so the 4096-token prefix is not replayed."""
    import oracle
    import synth

    B, H, d = wd.batch, wd.heads, wd.d
    rng = np.random.default_rng(0)
    state = rng.standard_normal((B, H, d, d))
    toks = [synth.bf16_bits_to_f32(synth.generate(t, wd.seed, d, nb=B, nh=H, t0=wd.n, nt=steps, dtype="bf16"))
            for t in (synth.Q, synth.K, synth.V)]
    slopes = wd.slopes()
    t0 = time.perf_counter()
    for s in range(steps):
        oracle.decode_step(*(np.ascontiguousarray(x[:, :, s]) for x in toks), slopes, state)
    dt = (time.perf_counter() - t0) / steps
    return {"us_per_step": dt * 1e6, "GB/s": B * H * DECODE_BYTES_PER_UNIT / dt / 1e9,
            "seconds_for_1000_steps": dt * 1000,
            "sample": f"{steps} steps of all {B * H} units (fp64), extrapolated to 1000"}


def cpu_baseline(w, target_s=15.0):
    """The fp64 oracle (token recurrence, OpenMP over heads) on the host cores, on a bounded
    sample of the workload: all heads, the first T tokens, T sized to ~target_s of CPU work."""
    import oracle
    import synth

    from long_context_la_amd import profiling

    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()

    def run(T):
        ex = [synth.bf16_bits_to_f32(synth.generate(t, w.seed, w.d, nb=w.batch, nh=w.heads, nt=T, dtype="bf16"))
              for t in (synth.Q, synth.K, synth.V)]
        t0 = time.perf_counter()
        oracle.recurrent(*ex, w.slopes())
        return time.perf_counter() - t0

    T = 256
    dt = run(T)
    T = int(min(w.n, max(256, T * target_s / max(dt, 1e-3))) // 256 * 256)
    dt = run(T)
    cpu = profiling.cpu_description()
    return {"value": w.batch * T / dt, "unit": "tokens/s", "cores": min(cores, w.batch * w.heads),
            "kind": "oracle", "cpu_model": cpu["model"], "logical_cpus": cpu["logical_cpus"],
            "sample": f"all {w.heads} heads x first {T} tokens of the {w.n}-token workload "
                      f"(fp64 recurrence, {dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="seconds of untimed steps before each leg's warm-up (lets the clock settle)")
    ap.add_argument("--workload", default="full", choices=["full", "share", "long", "full_d64"])
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the informational share (8 x 32K), long (8 x 1M) and d = 64 full-layer prefill legs")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 4 GiB device copy (counter calibration for the traffic figure)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only run the 128 x 64 decode leg (for its counter passes)")
    args = ap.parse_args()
    set_settle(args.settle_s)
    if args.gpus != 1:
        print("bench.py measures one GPU; runs on several GPUs are not supported (heads and sequences "
              "would shard across GPUs with no exchange or one small all-gather).", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_la_amd as la
    import synth

    device = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(device)
        return
    la.lib()
    from long_context_la_amd import profiling

    global PEAK_HBM_GBS, PEAK_BF16_TFLOPS
    peaks = profiling.device_peaks()
    PEAK_HBM_GBS, PEAK_BF16_TFLOPS = peaks["hbm_gbs"], peaks["bf16_tflops"]
    if args.decode_only:
        wd = synth.WORKLOADS["decode"]
        us = time_decode(wd, args.decode_steps, device)
        gbs = wd.batch * wd.heads * DECODE_BYTES_PER_UNIT / (us * 1e-6) / 1e9
        print(json.dumps({"decode_only": True, "us_per_step": us, "GB/s": gbs, "frac": gbs / PEAK_HBM_GBS}),
              flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    ms, kernel_ms, n_chunks, varlen, backward, _ = time_prefill(w, args.steps, args.warmup, device,
                                                             with_backward=not args.no_backward,
                                                             with_varlen=not args.no_varlen)
    token_heads = w.batch * w.heads * w.n
    tokens_s = w.batch * w.n / (ms * 1e-3)
    flops = model_flops_per_token_head(w.d) * token_heads
    alg_bytes = BYTES_PER_TOKEN_HEAD * token_heads
    log(f"prefill {w.name}: {ms:.3f} ms/step, kernel(s) {kernel_ms:.3f} ms, {n_chunks} chunk(s)")
    result = {
        "metric": "prefill tokens/s (all heads, d=128) + % MFMA roofline; decode GB/s",
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle_s,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64/Box-Muller activations, SiLU on Q/K)",
        "config": {"workload": f"{w.name} prefill: batch {w.batch}, {w.heads} heads, d={w.d}, N={w.n}, "
                               f"bf16 q/k/v/o, fp32 state, per-head decay",
                   "global_batch": w.batch, "seq_len": w.n, "heads": w.heads, "head_dim": w.d},
        "model_tflops": flops / (ms * 1e-3) / 1e12,
        "mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "hbm", "achieved": alg_bytes / (kernel_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": alg_bytes / (kernel_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": measured_traffic(w.name)},
        "peaks": peaks,
        "counters": measured_mfma() if w.name == "full" else None,
    }
    if varlen is not None:
        result["varlen"] = varlen
    if backward is not None:
        result["backward"] = backward
    if args.workload == "full" and not args.no_other_workloads:
        others = {}
        for name, steps in (("share", 20), ("long", 3), ("full_d64", 20)):
            wo = synth.WORKLOADS[name]
            # the share workload (268 MB moved) is about the size of the Infinity Cache: each of its
            # timed steps starts from a flushed cache
            flush = name == "share"
            ms_o, kms_o, nch_o, _, _, ms_wr = time_prefill(wo, steps, 1, device, with_backward=False,
                                                           with_varlen=False, flush=flush)
            th = wo.batch * wo.heads * wo.n
            log(f"prefill {name}: {ms_o:.3f} ms/step, kernel(s) {kms_o:.3f} ms, {nch_o} chunk(s)"
                + (" (cache flushed before each step)" if flush else ""))
            others[name] = {"workload": f"batch {wo.batch}, {wo.heads} heads, d={wo.d}, N={wo.n}, bf16, "
                                        f"{nch_o} chunks (LASP+ summaries + prefix combine)",
                            "ms_per_step": ms_o, "kernel_ms": kms_o, "tokens_per_s": wo.batch * wo.n / (ms_o * 1e-3),
                            "hbm_frac": 4 * wo.d * 2 * th / (kms_o * 1e-3) / 1e9 / PEAK_HBM_GBS,
                            "mfma_frac": model_flops_per_token_head(wo.d) * th / (ms_o * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                            "cache_flushed_between_steps": "by reading 512 MiB" if flush else False,
                            "traffic": measured_traffic(name) if wo.d == 128 else None}
            if ms_wr is not None:
                others[name]["ms_per_step_flushed_by_writing_512MiB"] = ms_wr
        result["other_workloads"] = others
    if not args.no_decode:
        result["mixed_batch"] = time_mixed(device)
        result["decode_small_batch"] = time_decode_small(device)
        wd = synth.WORKLOADS["decode"]
        us = time_decode(wd, args.decode_steps, device)
        gbs = wd.batch * wd.heads * DECODE_BYTES_PER_UNIT / (us * 1e-6) / 1e9
        log(f"decode: {us:.1f} us/step, {gbs:.0f} GB/s")
        result["decode"] = {"workload": f"{wd.batch} seqs x {wd.heads} heads, d={wd.d}, prefix {wd.n}, "
                                        f"{args.decode_steps} steps", "us_per_step": us, "GB/s": gbs,
                            "frac": gbs / PEAK_HBM_GBS}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w)
        if not args.no_decode:
            result["cpu_baseline"]["decode"] = cpu_baseline_decode(synth.WORKLOADS["decode"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
