// C ABI of liblightning_la.so: argument validation, work planning and
// dispatch to the gfx950 kernels.  See include/la.h for the contract.
#include <string.h>

#include <exception>
#include <mutex>
#include <string>
#include <vector>

#include "la_common.h"

namespace la {
namespace {

thread_local std::string g_last_error;

la_status fail(la_status s, const std::string& msg)
{
    g_last_error = msg;
    return s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

la_status device_check()
{
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return fail(LA_ERR_DEVICE, std::string("no usable GPU: ") + hipGetErrorString(e));
    }
    return LA_OK;
}

la_status launch_status(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(LA_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
    return LA_OK;
}

}  // namespace

Plan make_plan(int64_t batch, int64_t heads, int64_t n, int64_t d, int64_t chunk_override, int slice_w)
{
    Plan p;
    p.slices = (int)(d / slice_w);
    const int64_t units = batch * heads * p.slices;
    int64_t chunk = n;
    if (chunk_override > 0) {
        chunk = chunk_override;
    } else if (2 * units <= kTargetGroups && n > kMinChunk) {
        // chunks per sequence: as many as keep the workgroups within one round (rounded up, more
        // than half a round of unchunked workgroups would turn into two rounds plus a summary pass)
        const int64_t want = kTargetGroups / units;
        int64_t c = (n + want - 1) / want;
        c = ((c + kBlock - 1) / kBlock) * kBlock;
        if (c < kMinChunk) c = kMinChunk;
        chunk = c;
    }
    p.sub = 1;
    if (chunk >= n) {
        p.chunk = n > 0 ? n : 1;
        p.n_chunks = 1;
    } else {
        p.chunk = chunk;
        p.n_chunks = (n + chunk - 1) / chunk;
        const int64_t local_groups = batch * heads * (p.n_chunks - 1);  // full-width summary workgroups
        // (a d = 64 summary holds a quarter of a d = 128 state: twice the workgroups fill the GPU;
        // measured on the 64-head d = 64 layer, 1.35 -> 1.21 ms, and four times gains nothing more)
        const int64_t target = d == 64 ? 2 * kLocalTargetGroups : kLocalTargetGroups;
        while (local_groups * p.sub < target && p.chunk % (2 * p.sub * kBlock) == 0 &&
               p.chunk / (2 * p.sub) >= kMinSubChunk)
            p.sub *= 2;
        // Long sub-chunks go finer, up to eight times the target (two summary workgroups fit one CU)
        // while the chunk states stay within the allocation-free entry point's array: the summary
        // kernel skips the tokens too far before their chunk's end to matter, so the pass takes as
        // long as the longest window a sub-chunk must still cover (measured on 8 heads x 1M tokens:
        // 2.23 -> 2.01 ms; the 64-head d = 64 layer: 1.094 -> 1.028 ms; short sub-chunks, as at 8
        // heads x 32K, lose by it).
        auto state_bytes_at = [&](int64_t sub) {
            return (size_t)(batch * heads * (p.n_chunks + 1 + (p.n_chunks - 1) * sub)) * (size_t)(d * d) *
                   sizeof(float);
        };
        while (local_groups * p.sub < 8 * target && p.chunk % (2 * p.sub * kBlock) == 0 &&
               p.chunk / (2 * p.sub) >= kLongSubChunk && state_bytes_at(2 * p.sub) <= LA_NOALLOC_SCRATCH_BYTES)
            p.sub *= 2;
    }
    return p;
}

}  // namespace la

using namespace la;

namespace {

// Tile kernels address a 64-row tile with 32-bit buffer offsets (rows past a ragged tail wrap to
// offsets above the tile's range): a row stride of at most 2^22 elements keeps that within reach.
constexpr int64_t kMaxRowStride = int64_t(1) << 22;
// Work items of one launch: (batch, head) pairs, or (sequence or batch, head, chunk) triples.  At
// most 2^20 keeps every grid (4 value slices x 512 threads per item) at or below 2^31 work-items,
// within the dispatch's 32-bit grid size.
constexpr int64_t kMaxUnits = int64_t(1) << 20;

// Rows of a strided output (d contiguous elements per (batch, head, token)) are pairwise disjoint:
// with the dimensions of more than one element sorted by stride, each stride is at least the span
// of the faster ones.  A zero stride or rows of different heads that overlap would make several
// workgroups write different values to one element.
bool rows_disjoint(int64_t d, int64_t s0, int64_t n0, int64_t s1, int64_t n1, int64_t s2, int64_t n2)
{
    int64_t st[3] = {s0, s1, s2}, sz[3] = {n0, n1, n2};
    for (int i = 0; i < 3; ++i)  // insertion sort by stride
        for (int j = i; j > 0 && st[j] < st[j - 1]; --j) {
            const int64_t a = st[j], b = sz[j];
            st[j] = st[j - 1];
            sz[j] = sz[j - 1];
            st[j - 1] = a;
            sz[j - 1] = b;
        }
    int64_t span = d;
    for (int i = 0; i < 3; ++i) {
        if (sz[i] <= 1) continue;
        if (st[i] < span) return false;
        span += st[i] * (sz[i] - 1);
    }
    return true;
}

la_status check_shape(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d)
{
    if (dt != LA_F32 && dt != LA_BF16) return fail(LA_ERR_INVALID_ARGUMENT, "dtype must be LA_F32 or LA_BF16");
    if (batch < 1 || heads < 1 || n < 0 || d < 1)
        return fail(LA_ERR_INVALID_ARGUMENT, "batch, heads, d must be >= 1 and n >= 0");
    if (d != 64 && d != 128) return fail(LA_ERR_UNSUPPORTED, "d must be 64 or 128");
    if (batch > (int64_t(1) << 24) || heads > (int64_t(1) << 24) || n > (int64_t(1) << 40))
        return fail(LA_ERR_INVALID_ARGUMENT, "size out of range");
    if (batch * heads > kMaxUnits) return fail(LA_ERR_UNSUPPORTED, "more than 2^20 (batch, head) pairs in one call");
    return LA_OK;
}

// Prefix slots [B*H][n_chunks][d][d], then (with sub-chunks) summary slots [B*H][1 + n_sub][d][d].
size_t workspace_bytes_for(const Plan& p, int64_t batch, int64_t heads, int64_t d)
{
    if (p.n_chunks <= 1) return 0;
    const int64_t slots = p.n_chunks + (p.sub > 1 ? 1 + (p.n_chunks - 1) * p.sub : 0);
    return (size_t)batch * (size_t)heads * (size_t)slots * (size_t)d * (size_t)d * sizeof(float);
}

// Workspace of a prefill of this shape whatever it computes: the plans of both slice widths (the
// size queries do not know whether outputs are asked for).
size_t prefill_workspace_any(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d, int64_t chunk_tokens)
{
    const size_t a = workspace_bytes_for(make_plan(batch, heads, n, d, chunk_tokens), batch, heads, d);
    const size_t b = workspace_bytes_for(
        make_plan(batch, heads, n, d, chunk_tokens, fwd_slice_w(dt, batch, heads, n, d, true, false, 0)), batch, heads,
        d);
    return a > b ? a : b;
}

la_status check_fusion(const la_fusion* fu, const void* o)
{
    if (!fu) return LA_OK;
    if (fu->flags & ~(uint32_t)(LA_SILU_Q | LA_SILU_K | LA_SILU_V | LA_NORM | LA_GATE))
        return fail(LA_ERR_INVALID_ARGUMENT, "unknown fusion flag");
    if ((fu->flags & (LA_NORM | LA_GATE)) && !o)
        return fail(LA_ERR_INVALID_ARGUMENT, "LA_NORM and LA_GATE need an output tensor");
    if ((fu->flags & LA_GATE) && (!fu->gate || !aligned16(fu->gate)))
        return fail(LA_ERR_INVALID_ARGUMENT, "LA_GATE needs a 16-byte aligned gate tensor");
    if ((fu->flags & LA_NORM) && !(fu->norm_eps > 0.f))
        return fail(LA_ERR_INVALID_ARGUMENT, "LA_NORM needs norm_eps > 0");
    if ((fu->flags & LA_NORM) && fu->norm_weight && !aligned16(fu->norm_weight))
        return fail(LA_ERR_INVALID_ARGUMENT, "norm_weight must be 16-byte aligned");
    return LA_OK;
}

// Host-side argument checks of a prefill (everything but the workspace and the device).
la_status prefill_checks(la_dtype dt, const void* q, const void* k, const void* v, const void* o,
                         int64_t batch, int64_t heads, int64_t n, int64_t d,
                         int64_t sb, int64_t sh, int64_t sn, const float* slopes, const float* kv,
                         const float* ckpt, int64_t ckpt_every, int64_t chunk_tokens, const la_fusion* fu)
{
    la_status s = check_shape(dt, batch, heads, n, d);
    if (s != LA_OK) return s;
    s = check_fusion(fu, o);
    if (s != LA_OK) return s;
    if (!kv || !slopes) return fail(LA_ERR_INVALID_ARGUMENT, "kv and slopes must not be NULL");
    if (chunk_tokens < 0 || (chunk_tokens > 0 && chunk_tokens % kBlock != 0))
        return fail(LA_ERR_INVALID_ARGUMENT, "chunk_tokens must be 0 or a positive multiple of 64");
    if (ckpt && ckpt_every <= 0) return fail(LA_ERR_INVALID_ARGUMENT, "ckpt_every must be positive");
    if (n == 0) return LA_OK;
    if (!q || !k || !v) return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v must not be NULL");
    const int64_t align = (dt == LA_BF16) ? 8 : 4;
    if (sn < d || sb < 0 || sh < 0 || sb % align || sh % align || sn % align)
        return fail(LA_ERR_INVALID_ARGUMENT, "strides must be >= 0, multiples of 16 bytes, stride_n >= d");
    if (sn > kMaxRowStride) return fail(LA_ERR_UNSUPPORTED, "stride_n above 2^22 elements");
    if (o && !rows_disjoint(d, sn, n, sh, heads, sb, batch))
        return fail(LA_ERR_INVALID_ARGUMENT, "output rows overlap: the strides map two (batch, head, token) rows onto "
                                             "shared elements");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (o && !aligned16(o)) || !aligned16(kv) ||
        (ckpt && !aligned16(ckpt)))
        return fail(LA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
    return LA_OK;
}

la_status prefill_impl(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                       int64_t batch, int64_t heads, int64_t n, int64_t d,
                       int64_t sb, int64_t sh, int64_t sn, const float* slopes, float* kv,
                       float* ckpt, int64_t ckpt_every, int64_t chunk_tokens,
                       void* workspace, size_t workspace_bytes, void* stream, const la_fusion* fu = nullptr,
                       bool rev = false, bool wide = false)
{
    la_status s = prefill_checks(dt, q, k, v, o, batch, heads, n, d, sb, sh, sn, slopes, kv, ckpt, ckpt_every,
                                 chunk_tokens, fu);
    if (s != LA_OK || n == 0) return s;
    const int slice_w = fwd_slice_w(dt, batch, heads, n, d, o != nullptr, rev || wide,
                                    (fu ? fu->flags : 0u) & (LA_SILU_Q | LA_SILU_K | LA_SILU_V));

    if (ckpt && ckpt_every % kBlock != 0) {
        // Checkpoints inside a tile: the sequence runs as one prefill per checkpoint segment of
        // ckpt_every tokens (the state carried in kv), each followed by a copy of the state into
        // its slot.  Multiples of the tile are stored by the tile kernels themselves.
        s = device_check();
        if (s != LA_OK) return s;
        const int64_t n_ck = n / ckpt_every;
        const size_t esz = dt == LA_BF16 ? 2 : 4;
        auto at = [&](const void* base, int64_t t) -> const char* {
            return static_cast<const char*>(base) + (size_t)t * (size_t)sn * esz;
        };
        for (int64_t m = 0, t0 = 0; t0 < n; ++m) {
            const int64_t len = m < n_ck ? ckpt_every : n - t0;
            // a segment is chunked only when its own chunk workspace fits in the caller's
            int64_t ct = chunk_tokens;
            const int seg_w = fwd_slice_w(dt, batch, heads, len, d, o != nullptr, rev || wide,
                                          (fu ? fu->flags : 0u) & (LA_SILU_Q | LA_SILU_K | LA_SILU_V));
            if (ct == 0 && workspace_bytes_for(make_plan(batch, heads, len, d, 0, seg_w), batch, heads, d) >
                               (workspace ? workspace_bytes : 0))
                ct = ((len + kBlock - 1) / kBlock) * kBlock;
            s = prefill_impl(dt, at(q, t0), at(k, t0), at(v, t0), o ? (void*)at(o, t0) : nullptr, batch, heads, len, d,
                             sb, sh, sn, slopes, kv, nullptr, 0, ct, workspace, workspace_bytes, stream, fu, rev, wide);
            if (s != LA_OK) return s;
            if (m < n_ck) {
                s = launch_status(launch_state_to_slot(ckpt, kv, batch * heads, (int)d, n_ck, m,
                                                       static_cast<hipStream_t>(stream)),
                                  "checkpoint copy");
                if (s != LA_OK) return s;
            }
            t0 += len;
        }
        return LA_OK;
    }
    const Plan p = make_plan(batch, heads, n, d, chunk_tokens, slice_w);
    const int64_t n_sub = p.n_chunks > 1 ? (p.n_chunks - 1) * p.sub : 0;
    if (batch * heads * (p.n_chunks > n_sub ? p.n_chunks : n_sub) > kMaxUnits)
        return fail(LA_ERR_UNSUPPORTED, "more than 2^20 (batch, head, chunk) work items: use a larger chunk_tokens");
    const size_t need = workspace_bytes_for(p, batch, heads, d);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return fail(LA_ERR_WORKSPACE, "workspace missing, misaligned or smaller than la_prefill_workspace_size");

    s = device_check();
    if (s != LA_OK) return s;

    FwdArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.sb = sb;
    a.sh = sh;
    a.sn = sn;
    a.heads = heads;
    a.n = n;
    a.chunk = p.chunk;
    a.n_chunks = p.n_chunks;
    a.slices = p.slices;
    a.slopes = slopes;
    a.kv = kv;
    a.ws = static_cast<float*>(workspace);
    a.ckpt = ckpt;
    a.ckpt_every = ckpt ? ckpt_every : 0;
    a.n_ckpt = ckpt ? n / ckpt_every : 0;
    const uint32_t ff = fu ? fu->flags : 0u;
    a.act = ff & (LA_SILU_Q | LA_SILU_K | LA_SILU_V);
    a.gate = ((ff & LA_GATE) && !(ff & LA_NORM)) ? fu->gate : nullptr;  // gate alone: in the store
    a.rev = rev ? 1 : 0;
    a.wide = (rev || wide) ? 1 : 0;
    const int64_t bh = batch * heads;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool mfma = dt == LA_BF16;  // the bf16 MFMA kernels; float32 runs on the VALU tile kernel

    auto run = [&](int mode, int64_t chunks) -> hipError_t {
        FwdArgs b = a;
        b.chunks_launched = chunks;
        b.groups = bh * chunks;
        return mfma ? launch_fwd_bf16(b, (int)d, mode, st) : launch_fwd_f32(b, (int)d, mode, st);
    };

    // chunk summaries: full width (one workgroup per chunk-head) for plain bf16, else the sliced
    // tile kernel in its summary mode
    const bool full_width = mfma && a.act == 0;
    if (p.n_chunks > 1 && p.sub == 1) {
        FwdArgs b = a;
        b.span = p.chunk;
        b.chunks_launched = p.n_chunks - 1;
        b.groups = bh * (p.n_chunks - 1);
        s = launch_status(full_width ? launch_summary_bf16(b, (int)d, st) : run(kModeLocal, p.n_chunks - 1),
                          "chunk-summary launch");
        if (s != LA_OK) return s;
        s = launch_status(launch_scan(a.ws, kv, slopes, bh, heads, p.n_chunks, p.chunk, (int)d, st),
                          "prefix-combine launch");
        if (s != LA_OK) return s;
    } else if (p.n_chunks > 1) {
        // summaries per sub-chunk of every chunk but the last (all full length), into their own
        // slots; the scan folds them into the chunk prefixes
        const int64_t n_sub = (p.n_chunks - 1) * p.sub;
        FwdArgs b = a;
        b.ws = a.ws + bh * p.n_chunks * d * d;
        b.chunk = p.chunk / p.sub;
        b.span = p.chunk;
        b.n_chunks = n_sub + 1;  // the summary pass skips a sequence's last (sub-)chunk
        b.chunks_launched = n_sub;
        b.groups = bh * n_sub;
        s = launch_status(full_width ? launch_summary_bf16(b, (int)d, st)
                                     : mfma ? launch_fwd_bf16(b, (int)d, kModeLocal, st)
                                            : launch_fwd_f32(b, (int)d, kModeLocal, st),
                          "chunk-summary launch");
        if (s != LA_OK) return s;
        // the full-width forward summaries place their sub-chunks over each head's window
        const int window = full_width && !a.rev && summary_windowed(b.chunk) ? (a.o && !a.wide ? 1 : 2) : 0;
        s = launch_status(launch_scan_sub(a.ws, b.ws, kv, slopes, bh, heads, p.n_chunks, p.sub, b.chunk, window,
                                          (int)d, st),
                          "prefix-combine launch");
        if (s != LA_OK) return s;
    }
    s = launch_status(run(o ? kModeOut : kModeState, p.n_chunks), "prefill launch");
    if (s != LA_OK || !(ff & LA_NORM)) return s;
    // the normalisation needs all d features of a row: one more pass over o (gate included)
    return launch_status(launch_norm_gate(dt, o, (ff & LA_GATE) ? fu->gate : nullptr, fu->norm_weight, fu->norm_eps,
                                          true, batch, heads, n, (int)d, sb, sh, sn, st),
                         "normalisation launch");
}

// ---------------------------------------------------------------- prefill without allocation
// Device scratch for la_prefill_noalloc: the chunk states of a prefill live in this file-scope
// array instead of a caller-supplied workspace.  Every GPU the library runs on holds its own copy
// (until the process ends); host code reaches it only through the device address taken once per
// device with hipGetSymbolAddress -- in host code the array's name is not a device address.
constexpr size_t kScratchBytes = LA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kScratchDevices = 16;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];

la_status scratch_for_current_device(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) {
        (void)hipGetLastError();
        return fail(LA_ERR_DEVICE, "no current device (or more than 16 devices) for the scratch array");
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(LA_ERR_DEVICE, std::string("scratch array address: ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LA_OK;
}

la_status prefill_noalloc_impl(la_dtype dt, const void* q, const void* k, const void* v, void* o, int64_t batch,
                               int64_t heads, int64_t n, int64_t d, int64_t sb, int64_t sh, int64_t sn,
                               const float* slopes, float* kv, float* ckpt, int64_t ckpt_every, void* stream)
{
    la_status s = prefill_checks(dt, q, k, v, o, batch, heads, n, d, sb, sh, sn, slopes, kv, ckpt, ckpt_every, 0,
                                 nullptr);
    if (s != LA_OK || n == 0) return s;
    const size_t need = prefill_workspace_any(dt, batch, heads, n, d, 0);
    if (need > kScratchBytes)
        return fail(LA_ERR_UNSUPPORTED, "this shape needs " + std::to_string(need) +
                                            " bytes of chunk states; la_prefill_noalloc holds " +
                                            std::to_string(kScratchBytes));
    s = device_check();
    if (s != LA_OK) return s;
    void* ws = nullptr;
    s = scratch_for_current_device(&ws);
    if (s != LA_OK) return s;
    // the chunk states are written before they are read within one call, so nothing needs clearing
    return prefill_impl(dt, q, k, v, o, batch, heads, n, d, sb, sh, sn, slopes, kv, ckpt, ckpt_every, 0, ws,
                        kScratchBytes, stream);
}

// ---------------------------------------------------------------- backward pass
// Gradients of a loss through the recurrence (the reverse state recurrence that the training side
// of LASP+, page "MiniMax-01: Scaling Foundation Models with Lightning Attention | Summary",
// section 3.2, passes between partitions).  With G_t = dL/dKV_t:
//   dq_t = do_t KV_t^T                          -- the forward recurrence of (dO, V, K) from KV_in^T
//   dv_t = k_t G_t,  G_t = q_t^T do_t + l G_{t+1} -- the recurrence of (K, Q, dO) walked backwards,
//   dk_t = v_t G_t^T                            -- and of (V, dO, Q) backwards for G^T,
// each started from dL/dKV_final / lambda (the first reversed token adds it undecayed), and
// dL/dKV_in = lambda G_0.  So the three gradients are three runs of the prefill kernels.
size_t state_bytes(int64_t batch, int64_t heads, int64_t d)
{
    return (size_t)batch * (size_t)heads * (size_t)d * (size_t)d * sizeof(float);
}

la_status backward_impl(la_dtype dt, const void* q, const void* k, const void* v, const void* dout,
                        int64_t batch, int64_t heads, int64_t n, int64_t d, int64_t sb, int64_t sh, int64_t sn,
                        const float* slopes, const float* kv_in, const float* dkv_out, void* dq, void* dk, void* dv,
                        float* dkv_in, void* workspace, size_t workspace_bytes, void* stream)
{
    la_status s = check_shape(dt, batch, heads, n, d);
    if (s != LA_OK) return s;
    if (!slopes) return fail(LA_ERR_INVALID_ARGUMENT, "slopes must not be NULL");
    if (n > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv))
        return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v, dout, dq, dk, dv must not be NULL");
    if ((kv_in && !aligned16(kv_in)) || (dkv_out && !aligned16(dkv_out)) || (dkv_in && !aligned16(dkv_in)))
        return fail(LA_ERR_INVALID_ARGUMENT, "state pointers must be 16-byte aligned");
    if (n > 0 && !rows_disjoint(d, sn, n, sh, heads, sb, batch))
        return fail(LA_ERR_INVALID_ARGUMENT, "gradient rows overlap: the strides map two (batch, head, token) rows onto "
                                             "shared elements");
    const Plan p = make_plan(batch, heads, n, d, 0);
    const size_t sbytes = state_bytes(batch, heads, d);
    const size_t need = sbytes + workspace_bytes_for(p, batch, heads, d);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(LA_ERR_WORKSPACE, "workspace missing, misaligned or smaller than la_backward_workspace_size");
    s = device_check();
    if (s != LA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    float* S = static_cast<float*>(workspace);
    void* chunk_ws = static_cast<char*>(workspace) + sbytes;
    const size_t chunk_bytes = workspace_bytes - sbytes;
    const int64_t bh = batch * heads;
    auto prep = [&](float* dst, const float* src, bool tr, int power) {
        return launch_status(launch_state_prep(dst, src, slopes, bh, heads, (int)d, tr, power, st), "state set-up launch");
    };
    if (n == 0) return dkv_in ? prep(dkv_in, dkv_out, false, 0) : LA_OK;
    // dQ: (dO, V, K) forward from KV_in^T.  Every pass runs on full-range operands: dO can be
    // far smaller than activations.
    s = prep(S, kv_in, true, 0);
    if (s == LA_OK)
        s = prefill_impl(dt, dout, v, k, dq, batch, heads, n, d, sb, sh, sn, slopes, S, nullptr, 0, 0, chunk_ws,
                         chunk_bytes, stream, nullptr, false, true);
    // dK: (V, dO, Q) backwards from (dL/dKV_final / lambda)^T
    if (s == LA_OK) s = prep(S, dkv_out, true, dkv_out ? 1 : 0);
    if (s == LA_OK)
        s = prefill_impl(dt, v, dout, q, dk, batch, heads, n, d, sb, sh, sn, slopes, S, nullptr, 0, 0, chunk_ws,
                         chunk_bytes, stream, nullptr, true);
    // dV: (K, Q, dO) backwards from dL/dKV_final / lambda; the final state is G_0
    if (s == LA_OK) s = prep(S, dkv_out, false, dkv_out ? 1 : 0);
    if (s == LA_OK)
        s = prefill_impl(dt, k, q, dout, dv, batch, heads, n, d, sb, sh, sn, slopes, S, nullptr, 0, 0, chunk_ws,
                         chunk_bytes, stream, nullptr, true);
    if (s == LA_OK && dkv_in) s = prep(dkv_in, S, false, -1);
    return s;
}

// ---------------------------------------------------------------- packed variable-length batches
// Page "MiniMax-01: Scaling Foundation Models with Lightning Attention | Summary", section 3.2
// (data packing: samples concatenated without padding, each with its own offsets) and section
// 3.3 (separate handling of long and short inputs): one launch covers every sequence; long
// sequences are cut into chunks (the LASP+ combine of section 3.2), short ones run whole.
struct VarPlan {
    int64_t chunk = 0;         // chunk length (tokens) of every chunk but a sequence's last
    int64_t total_chunks = 0;  // over the sequences that run in 64-token tiles
    int64_t n_short = 0;       // sequences of 1..kShortTokens tokens, run token by token
    bool chunked = false;      // some sequence has more than one chunk
    int slices = 0;
    std::vector<int64_t> tab;  // ctab (5 per chunk), stab (2 per sequence), rtab (3 per short sequence)
};

size_t varlen_table_bytes(const VarPlan& p) { return ((p.tab.size() * sizeof(int64_t) + 255) / 256) * 256; }

size_t varlen_workspace_bytes(const VarPlan& p, int64_t heads, int64_t d)
{
    size_t b = varlen_table_bytes(p);
    if (p.chunked) b += (size_t)p.total_chunks * (size_t)heads * (size_t)d * (size_t)d * sizeof(float);
    return b;
}

la_status make_varlen_plan(la_dtype dt, int64_t n_seq, const int64_t* cu, int64_t heads, int64_t d,
                           int64_t chunk_override, VarPlan& p, int slice_w = kSliceW, bool tables = true)
{
    if (n_seq < 1 || n_seq > (int64_t(1) << 24)) return fail(LA_ERR_INVALID_ARGUMENT, "n_seq must be in [1, 2^24]");
    if (!cu) return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens must not be NULL");
    if (cu[0] != 0) return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens[0] must be 0");
    int64_t longest = 0, nonempty = 0;
    for (int64_t s = 0; s < n_seq; ++s) {
        const int64_t n = cu[s + 1] - cu[s];
        if (n < 0) return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens must be nondecreasing");
        longest = n > longest ? n : longest;
        nonempty += n > 0;
    }
    la_status st = check_shape(dt, n_seq, heads, longest, d);
    if (st != LA_OK) return st;
    if (chunk_override < 0 || (chunk_override > 0 && chunk_override % kBlock != 0))
        return fail(LA_ERR_INVALID_ARGUMENT, "chunk_tokens must be 0 or a positive multiple of 64");
    p.slices = (int)(d / slice_w);
    const int64_t total = cu[n_seq];
    int64_t chunk = longest;
    if (chunk_override > 0) {
        chunk = chunk_override;
    } else if (nonempty * heads * p.slices < kTargetGroups && longest > kMinChunk) {
        // about kTargetGroups workgroups over the whole batch, chunks no shorter than kMinChunk
        int64_t c = (total * heads * p.slices + kTargetGroups - 1) / kTargetGroups;
        c = ((c + kBlock - 1) / kBlock) * kBlock;
        if (c < kMinChunk) c = kMinChunk;
        chunk = c;
    }
    p.chunk = chunk > 0 ? chunk : kBlock;
    int64_t n_tiled_chunks = 0;
    for (int64_t s = 0; s < n_seq; ++s) {
        const int64_t n = cu[s + 1] - cu[s];
        if (n > kShortTokens) n_tiled_chunks += (n + p.chunk - 1) / p.chunk;
    }
    if (n_tiled_chunks * heads > kMaxUnits)
        return fail(LA_ERR_UNSUPPORTED, "more than 2^20 (chunk, head) work items: use a larger chunk_tokens");
    p.tab.clear();
    if (!tables) {  // the plan's shape only: chunk counts, no tables
        for (int64_t s = 0; s < n_seq; ++s) {
            const int64_t n = cu[s + 1] - cu[s];
            if (n >= 1 && n <= kShortTokens) {
                ++p.n_short;
                continue;
            }
            const int64_t nc = n == 0 ? 0 : (n <= p.chunk ? 1 : (n + p.chunk - 1) / p.chunk);
            p.total_chunks += nc;
            if (nc > 1) p.chunked = true;
        }
        return LA_OK;
    }
    std::vector<int64_t> stab((size_t)(2 * n_seq)), rtab;
    for (int64_t s = 0; s < n_seq; ++s) {
        const int64_t n = cu[s + 1] - cu[s];
        if (n >= 1 && n <= kShortTokens) {  // short: token by token, no tile
            rtab.insert(rtab.end(), {cu[s], n, s});
            ++p.n_short;
            stab[2 * s] = p.total_chunks;
            stab[2 * s + 1] = 0;
            continue;
        }
        const int64_t nc = n == 0 ? 0 : (n <= p.chunk ? 1 : (n + p.chunk - 1) / p.chunk);
        stab[2 * s] = p.total_chunks;
        stab[2 * s + 1] = nc;
        for (int64_t jj = 0; jj < nc; ++jj) {
            const int64_t b = cu[s] + jj * p.chunk;
            const int64_t e = (jj == nc - 1) ? cu[s + 1] : b + p.chunk;
            p.tab.insert(p.tab.end(), {b, e, s, jj, stab[2 * s]});
        }
        p.total_chunks += nc;
        if (nc > 1) p.chunked = true;
    }
    p.tab.insert(p.tab.end(), stab.begin(), stab.end());
    p.tab.insert(p.tab.end(), rtab.begin(), rtab.end());
    return LA_OK;
}

// Value columns per workgroup of a packed prefill (see fwd_slice_w): 64 when the 32-column plan
// chunks, or when the 32-column work spread over the GPU (the tiles of every (chunk, head,
// slice) over kTargetGroups workgroup slots) exceeds 1.55x the longest sequence's tile chain --
// 1.55 being the measured time per tile of a 64-column workgroup against a 32-column one, so
// that the longer chains of the 64-column plan stay off the critical path.  Arguments as for
// make_varlen_plan; an invalid batch gets kSliceW (make_varlen_plan then reports it).
int varlen_slice_w(la_dtype dt, int64_t n_seq, const int64_t* cu, int64_t heads, int64_t d, bool out, bool wide)
{
    if (!(dt == LA_BF16 && d == 128 && out && !wide) || !cu || n_seq < 1) return kSliceW;
    VarPlan p32;
    if (make_varlen_plan(dt, n_seq, cu, heads, d, 0, p32, kSliceW, false) != LA_OK) return kSliceW;
    if (p32.chunked) return kWideSliceW;
    int64_t tiles = 0, longest = 0;
    for (int64_t s = 0; s < n_seq; ++s) {
        const int64_t n = cu[s + 1] - cu[s];
        if (n <= kShortTokens) continue;  // token by token, no tile kernel
        const int64_t t = (n + kBlock - 1) / kBlock;
        tiles += t;
        longest = t > longest ? t : longest;
    }
    const int64_t spread = tiles * heads * (d / kSliceW);  // 32-column tiles over all workgroups
    return 100 * spread > 155 * longest * kTargetGroups ? kWideSliceW : kSliceW;
}

// Small tables travel by value in the arguments of a one-block kernel that writes them to the
// workspace: no copy call, nothing on the host to keep alive, and a captured graph replays the
// same values.  kTableArgWords * 8 bytes stays well inside the 4 KiB kernel-argument limit.
constexpr int kTableArgWords = 384;
struct TableArg {
    int64_t n;
    int64_t v[kTableArgWords];
};
__global__ __launch_bounds__(128) void k_write_table(int64_t* dst, TableArg t)
{
    for (int64_t i = threadIdx.x; i < t.n; i += blockDim.x) dst[i] = t.v[i];
}

// Larger tables go through page-locked staging: a ring of host buffers per device, each reused
// only after the event recorded behind its last copy has completed.  The copy is then
// asynchronous and never reads host memory that has been released.
struct Staging {
    void* host = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
};
constexpr int kStageDevices = 16, kStageRing = 8;
std::mutex g_stage_mu;
Staging g_stage[kStageDevices][kStageRing];
unsigned g_stage_next[kStageDevices];

la_status upload_tables(void* dst, const std::vector<int64_t>& tab, hipStream_t st)
{
    if (tab.size() <= (size_t)kTableArgWords) {
        TableArg t;
        t.n = (int64_t)tab.size();
        memcpy(t.v, tab.data(), tab.size() * sizeof(int64_t));
        hipLaunchKernelGGL(k_write_table, dim3(1), dim3(128), 0, st, static_cast<int64_t*>(dst), t);
        return launch_status(hipGetLastError(), "table upload");
    }
    const size_t bytes = tab.size() * sizeof(int64_t);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kStageDevices)
        return fail(LA_ERR_DEVICE, "table upload: no current device (or more than 16 devices)");
    std::lock_guard<std::mutex> lock(g_stage_mu);
    Staging& b = g_stage[dev][g_stage_next[dev]++ % kStageRing];
    if (b.pending) {
        const hipError_t e = hipEventSynchronize(b.ev);
        if (e != hipSuccess) return fail(LA_ERR_DEVICE, std::string("table upload: ") + hipGetErrorString(e));
        b.pending = false;
    }
    if (b.cap < bytes) {
        if (b.host) (void)hipHostFree(b.host);
        b.host = nullptr;
        b.cap = 0;
        size_t cap = 4096;
        while (cap < bytes) cap *= 2;
        if (hipHostMalloc(&b.host, cap, hipHostMallocDefault) != hipSuccess) {
            b.host = nullptr;
            return fail(LA_ERR_DEVICE, "table upload: page-locked host allocation failed");
        }
        b.cap = cap;
    }
    if (!b.ev && hipEventCreateWithFlags(&b.ev, hipEventDisableTiming) != hipSuccess) {
        b.ev = nullptr;
        return fail(LA_ERR_DEVICE, "table upload: event creation failed");
    }
    memcpy(b.host, tab.data(), bytes);
    hipError_t e = hipMemcpyAsync(dst, b.host, bytes, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipEventRecord(b.ev, st);
    if (e != hipSuccess) return fail(LA_ERR_DEVICE, std::string("table upload: ") + hipGetErrorString(e));
    b.pending = true;
    return LA_OK;
}

la_status prefill_varlen_impl(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                              int64_t n_seq, const int64_t* cu, int64_t heads, int64_t d,
                              int64_t sh, int64_t sn, const float* slopes, float* kv, int64_t chunk_tokens,
                              void* workspace, size_t workspace_bytes, void* stream, bool rev = false,
                              bool wide = false)
{
    VarPlan p;
    la_status s = make_varlen_plan(dt, n_seq, cu, heads, d, chunk_tokens, p,
                                   varlen_slice_w(dt, n_seq, cu, heads, d, o != nullptr, rev || wide));
    if (s != LA_OK) return s;
    if (!kv || !slopes) return fail(LA_ERR_INVALID_ARGUMENT, "kv and slopes must not be NULL");
    if (p.total_chunks == 0 && p.n_short == 0) return LA_OK;  // every sequence empty
    if (!q || !k || !v) return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v must not be NULL");
    const int64_t align = (dt == LA_BF16) ? 8 : 4;
    if (sn < d || sh < 0 || sh % align || sn % align)
        return fail(LA_ERR_INVALID_ARGUMENT, "strides must be >= 0, multiples of 16 bytes, stride_n >= d");
    if (sn > kMaxRowStride) return fail(LA_ERR_UNSUPPORTED, "stride_n above 2^22 elements");
    if (o && !rows_disjoint(d, sn, cu[n_seq], sh, heads, 0, 1))
        return fail(LA_ERR_INVALID_ARGUMENT, "output rows overlap: the strides map two (token, head) rows onto shared "
                                             "elements");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (o && !aligned16(o)) || !aligned16(kv))
        return fail(LA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
    const size_t need = varlen_workspace_bytes(p, heads, d);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
        return fail(LA_ERR_WORKSPACE, "workspace missing, misaligned or smaller than la_prefill_varlen_workspace_size");
    s = device_check();
    if (s != LA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the chunk and sequence tables go to the front of the workspace (kernel arguments or
    // page-locked staging, by size)
    s = upload_tables(workspace, p.tab, st);
    if (s != LA_OK) return s;
    const int64_t* ctab = static_cast<const int64_t*>(workspace);
    FwdArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.sh = sh;
    a.sn = sn;
    a.heads = heads;
    a.chunk = p.chunk;
    a.slices = p.slices;
    a.slopes = slopes;
    a.kv = kv;
    a.ws = p.chunked ? reinterpret_cast<float*>(static_cast<char*>(workspace) + varlen_table_bytes(p)) : nullptr;
    a.ctab = ctab;
    a.stab = ctab + 5 * p.total_chunks;
    a.groups = p.total_chunks * heads;
    a.rev = rev ? 1 : 0;
    a.wide = (rev || wide) ? 1 : 0;
    auto run = [&](int mode) -> hipError_t {
        return dt == LA_BF16 ? launch_fwd_bf16(a, (int)d, mode, st) : launch_fwd_f32(a, (int)d, mode, st);
    };
    if (p.n_short > 0) {
        const int64_t* rtab = a.stab + 2 * n_seq;
        s = launch_status(launch_recur_short(dt, q, k, v, o, p.n_short, heads, (int)d, sn, sh, slopes, kv, rtab, rev, st),
                          "short-sequence launch");
        if (s != LA_OK) return s;
    }
    if (p.total_chunks == 0) return LA_OK;
    if (p.chunked) {
        // local summaries on 32-column slices whatever the main pass uses (each slice writes its
        // columns of the d x d slots)
        FwdArgs b = a;
        b.slices = (int)(d / kSliceW);
        s = launch_status(dt == LA_BF16 ? launch_fwd_bf16(b, (int)d, kModeLocal, st)
                                        : launch_fwd_f32(b, (int)d, kModeLocal, st),
                          "chunk-summary launch");
        if (s != LA_OK) return s;
        s = launch_status(launch_scan_varlen(a.ws, kv, slopes, a.stab, n_seq, heads, p.chunk, (int)d, st),
                          "prefix-combine launch");
        if (s != LA_OK) return s;
    }
    return launch_status(run(o ? kModeOut : kModeState), "prefill launch");
}

// The backward pass for packed sequences: the three runs of backward_impl, each over the packed
// layout (the reverse runs walk every sequence from its last token to its first).
size_t backward_varlen_bytes(const VarPlan& p, int64_t n_seq, int64_t heads, int64_t d)
{
    return state_bytes(n_seq, heads, d) + varlen_workspace_bytes(p, heads, d);
}

la_status backward_varlen_impl(la_dtype dt, const void* q, const void* k, const void* v, const void* dout,
                               int64_t n_seq, const int64_t* cu, int64_t heads, int64_t d, int64_t sh, int64_t sn,
                               const float* slopes, const float* kv_in, const float* dkv_out, void* dq, void* dk,
                               void* dv, float* dkv_in, void* workspace, size_t workspace_bytes, void* stream)
{
    VarPlan p;
    la_status s = make_varlen_plan(dt, n_seq, cu, heads, d, 0, p);
    if (s != LA_OK) return s;
    if (!slopes) return fail(LA_ERR_INVALID_ARGUMENT, "slopes must not be NULL");
    if (cu[n_seq] > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv))
        return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v, dout, dq, dk, dv must not be NULL");
    if ((kv_in && !aligned16(kv_in)) || (dkv_out && !aligned16(dkv_out)) || (dkv_in && !aligned16(dkv_in)))
        return fail(LA_ERR_INVALID_ARGUMENT, "state pointers must be 16-byte aligned");
    if (cu[n_seq] > 0 && !rows_disjoint(d, sn, cu[n_seq], sh, heads, 0, 1))
        return fail(LA_ERR_INVALID_ARGUMENT, "gradient rows overlap: the strides map two (token, head) rows onto shared "
                                             "elements");
    const size_t sbytes = state_bytes(n_seq, heads, d);
    if (!workspace || workspace_bytes < backward_varlen_bytes(p, n_seq, heads, d) || !aligned16(workspace))
        return fail(LA_ERR_WORKSPACE, "workspace missing, misaligned or smaller than la_backward_varlen_workspace_size");
    s = device_check();
    if (s != LA_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    float* S = static_cast<float*>(workspace);
    void* vws = static_cast<char*>(workspace) + sbytes;
    const size_t vbytes = workspace_bytes - sbytes;
    const int64_t bh = n_seq * heads;
    auto prep = [&](float* dst, const float* src, bool tr, int power) {
        return launch_status(launch_state_prep(dst, src, slopes, bh, heads, (int)d, tr, power, st), "state set-up launch");
    };
    s = prep(S, kv_in, true, 0);
    if (s == LA_OK)
        s = prefill_varlen_impl(dt, dout, v, k, dq, n_seq, cu, heads, d, sh, sn, slopes, S, 0, vws, vbytes, stream,
                                false, true);
    if (s == LA_OK) s = prep(S, dkv_out, true, dkv_out ? 1 : 0);
    if (s == LA_OK)
        s = prefill_varlen_impl(dt, v, dout, q, dk, n_seq, cu, heads, d, sh, sn, slopes, S, 0, vws, vbytes, stream, true);
    if (s == LA_OK) s = prep(S, dkv_out, false, dkv_out ? 1 : 0);
    if (s == LA_OK)
        s = prefill_varlen_impl(dt, k, q, dout, dv, n_seq, cu, heads, d, sh, sn, slopes, S, 0, vws, vbytes, stream, true);
    if (s == LA_OK && dkv_in) s = prep(dkv_in, S, false, -1);
    return s;
}

}  // namespace

extern "C" {

size_t la_prefill_varlen_workspace_size_ex(la_dtype dt, int64_t n_seq, const int64_t* cu_seqlens, int64_t heads,
                                           int64_t d, int64_t chunk_tokens)
{
    try {
        // the plans of both slice widths (the query does not know whether outputs are asked for)
        VarPlan p, p64;
        if (make_varlen_plan(dt, n_seq, cu_seqlens, heads, d, chunk_tokens, p) != LA_OK) return 0;
        const size_t a = varlen_workspace_bytes(p, heads, d);
        const int w = varlen_slice_w(dt, n_seq, cu_seqlens, heads, d, true, false);
        if (w == kSliceW || make_varlen_plan(dt, n_seq, cu_seqlens, heads, d, chunk_tokens, p64, w) != LA_OK) return a;
        const size_t b = varlen_workspace_bytes(p64, heads, d);
        return a > b ? a : b;
    } catch (...) {
        return 0;
    }
}

size_t la_prefill_varlen_workspace_size(la_dtype dt, int64_t n_seq, const int64_t* cu_seqlens, int64_t heads,
                                        int64_t d)
{
    return la_prefill_varlen_workspace_size_ex(dt, n_seq, cu_seqlens, heads, d, 0);
}

int64_t la_prefill_varlen_chunk_tokens(la_dtype dt, int64_t n_seq, const int64_t* cu_seqlens, int64_t heads,
                                       int64_t d)
{
    try {
        VarPlan p;
        if (make_varlen_plan(dt, n_seq, cu_seqlens, heads, d, 0, p,
                             varlen_slice_w(dt, n_seq, cu_seqlens, heads, d, true, false)) != LA_OK)
            return -1;
        return p.chunk;
    } catch (...) {
        return -1;
    }
}

la_status la_prefill_varlen_ex(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                               int64_t n_seq, const int64_t* cu_seqlens, int64_t heads, int64_t d,
                               int64_t stride_h, int64_t stride_n, const float* slopes, float* kv,
                               int64_t chunk_tokens, void* workspace, size_t workspace_bytes, void* stream)
{
    try {
        return prefill_varlen_impl(dt, q, k, v, o, n_seq, cu_seqlens, heads, d, stride_h, stride_n, slopes, kv,
                                   chunk_tokens, workspace, workspace_bytes, stream);
    } catch (const std::exception& e) {
        return fail(LA_ERR_INTERNAL, e.what());
    } catch (...) {
        return fail(LA_ERR_INTERNAL, "unknown error");
    }
}

la_status la_prefill_varlen(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                            int64_t n_seq, const int64_t* cu_seqlens, int64_t heads, int64_t d,
                            int64_t stride_h, int64_t stride_n, const float* slopes, float* kv,
                            void* workspace, size_t workspace_bytes, void* stream)
{
    return la_prefill_varlen_ex(dt, q, k, v, o, n_seq, cu_seqlens, heads, d, stride_h, stride_n, slopes, kv, 0,
                                workspace, workspace_bytes, stream);
}


la_status la_state_init(float* kv, const float* kv0, int64_t batch, int64_t heads, int64_t d, void* stream)
{
    try {
        if (!kv) return fail(LA_ERR_INVALID_ARGUMENT, "kv must not be NULL");
        if (batch < 1 || heads < 1) return fail(LA_ERR_INVALID_ARGUMENT, "batch and heads must be >= 1");
        if (d != 64 && d != 128) return fail(LA_ERR_UNSUPPORTED, "d must be 64 or 128");
        if (!aligned16(kv) || (kv0 && !aligned16(kv0)))
            return fail(LA_ERR_INVALID_ARGUMENT, "kv pointers must be 16-byte aligned");
        la_status s = device_check();
        if (s != LA_OK) return s;
        return launch_status(launch_state_init(kv, kv0, batch * heads * d * d, static_cast<hipStream_t>(stream)),
                             "state-init launch");
    } catch (const std::exception& e) {
        return fail(LA_ERR_INTERNAL, e.what());
    } catch (...) {
        return fail(LA_ERR_INTERNAL, "unknown error");
    }
}

int64_t la_prefill_chunk_tokens(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d)
{
    if (check_shape(dt, batch, heads, n, d) != LA_OK) return -1;
    const Plan p = make_plan(batch, heads, n, d, 0, fwd_slice_w(dt, batch, heads, n, d, true, false, 0));
    return p.n_chunks > 1 ? p.chunk : n;
}

size_t la_prefill_workspace_size_ex(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d,
                                    int64_t chunk_tokens)
{
    if (check_shape(dt, batch, heads, n, d) != LA_OK) return 0;
    if (chunk_tokens < 0 || (chunk_tokens > 0 && chunk_tokens % kBlock != 0)) return 0;
    return prefill_workspace_any(dt, batch, heads, n, d, chunk_tokens);
}

size_t la_prefill_workspace_size(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d)
{
    return la_prefill_workspace_size_ex(dt, batch, heads, n, d, 0);
}

la_status la_prefill_ex(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                        int64_t batch, int64_t heads, int64_t n, int64_t d,
                        int64_t stride_b, int64_t stride_h, int64_t stride_n,
                        const float* slopes, float* kv, float* ckpt, int64_t ckpt_every,
                        int64_t chunk_tokens, void* workspace, size_t workspace_bytes, void* stream)
{
    try {
        return prefill_impl(dt, q, k, v, o, batch, heads, n, d, stride_b, stride_h, stride_n, slopes, kv,
                            ckpt, ckpt_every, chunk_tokens, workspace, workspace_bytes, stream);
    } catch (const std::exception& e) {
        return fail(LA_ERR_INTERNAL, e.what());
    } catch (...) {
        return fail(LA_ERR_INTERNAL, "unknown error");
    }
}

la_status la_prefill(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                     int64_t batch, int64_t heads, int64_t n, int64_t d,
                     int64_t stride_b, int64_t stride_h, int64_t stride_n,
                     const float* slopes, float* kv, float* ckpt, int64_t ckpt_every,
                     void* workspace, size_t workspace_bytes, void* stream)
{
    return la_prefill_ex(dt, q, k, v, o, batch, heads, n, d, stride_b, stride_h, stride_n, slopes, kv, ckpt,
                         ckpt_every, 0, workspace, workspace_bytes, stream);
}

la_status la_prefill_noalloc(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                             int64_t batch, int64_t heads, int64_t n, int64_t d,
                             int64_t stride_b, int64_t stride_h, int64_t stride_n,
                             const float* slopes, float* kv, float* ckpt, int64_t ckpt_every, void* stream)
{
    try {
        return prefill_noalloc_impl(dt, q, k, v, o, batch, heads, n, d, stride_b, stride_h, stride_n, slopes, kv,
                                    ckpt, ckpt_every, stream);
    } catch (const std::exception& e) {
        return fail(LA_ERR_INTERNAL, e.what());
    } catch (...) {
        return fail(LA_ERR_INTERNAL, "unknown error");
    }
}

la_status la_decode_fused(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                          int64_t batch, int64_t heads, int64_t d, const float* slopes, float* kv,
                          const la_fusion* fusion, void* stream)
{
    try {
        la_status s = check_fusion(fusion, o);
        if (s != LA_OK) return s;
        if (dt != LA_F32 && dt != LA_BF16) return fail(LA_ERR_INVALID_ARGUMENT, "dtype must be LA_F32 or LA_BF16");
        if (!q || !k || !v || !o || !slopes || !kv)
            return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v, o, slopes and kv must not be NULL");
        if (batch < 1 || heads < 1) return fail(LA_ERR_INVALID_ARGUMENT, "batch and heads must be >= 1");
        if (d != 64 && d != 128) return fail(LA_ERR_UNSUPPORTED, "d must be 64 or 128");
        if (batch * heads > kMaxUnits) return fail(LA_ERR_UNSUPPORTED, "more than 2^20 (batch, head) pairs in one call");
        if (!aligned16(kv)) return fail(LA_ERR_INVALID_ARGUMENT, "kv must be 16-byte aligned");
        s = device_check();
        if (s != LA_OK) return s;
        return launch_status(launch_decode(dt, q, k, v, o, batch * heads, heads, (int)d, slopes, kv, fusion,
                                           static_cast<hipStream_t>(stream)),
                             "decode launch");
    } catch (const std::exception& e) {
        return fail(LA_ERR_INTERNAL, e.what());
    } catch (...) {
        return fail(LA_ERR_INTERNAL, "unknown error");
    }
}

la_status la_decode(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                    int64_t batch, int64_t heads, int64_t d, const float* slopes, float* kv, void* stream)
{
    return la_decode_fused(dt, q, k, v, o, batch, heads, d, slopes, kv, nullptr, stream);
}

la_status la_prefill_fused(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                           int64_t batch, int64_t heads, int64_t n, int64_t d,
                           int64_t stride_b, int64_t stride_h, int64_t stride_n,
                           const float* slopes, float* kv, const la_fusion* fusion,
                           void* workspace, size_t workspace_bytes, void* stream)
{
    try {
        return prefill_impl(dt, q, k, v, o, batch, heads, n, d, stride_b, stride_h, stride_n, slopes, kv,
                            nullptr, 0, 0, workspace, workspace_bytes, stream, fusion);
    } catch (const std::exception& e) {
        return fail(LA_ERR_INTERNAL, e.what());
    } catch (...) {
        return fail(LA_ERR_INTERNAL, "unknown error");
    }
}

size_t la_backward_workspace_size(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d)
{
    if (check_shape(dt, batch, heads, n, d) != LA_OK) return 0;
    return state_bytes(batch, heads, d) + workspace_bytes_for(make_plan(batch, heads, n, d, 0), batch, heads, d);
}

la_status la_backward(la_dtype dt, const void* q, const void* k, const void* v, const void* dout,
                      int64_t batch, int64_t heads, int64_t n, int64_t d,
                      int64_t stride_b, int64_t stride_h, int64_t stride_n, const float* slopes,
                      const float* kv_in, const float* dkv_out, void* dq, void* dk, void* dv, float* dkv_in,
                      void* workspace, size_t workspace_bytes, void* stream)
{
    try {
        return backward_impl(dt, q, k, v, dout, batch, heads, n, d, stride_b, stride_h, stride_n, slopes, kv_in,
                             dkv_out, dq, dk, dv, dkv_in, workspace, workspace_bytes, stream);
    } catch (const std::exception& e) {
        return fail(LA_ERR_INTERNAL, e.what());
    } catch (...) {
        return fail(LA_ERR_INTERNAL, "unknown error");
    }
}

size_t la_backward_varlen_workspace_size(la_dtype dt, int64_t n_seq, const int64_t* cu_seqlens, int64_t heads,
                                         int64_t d)
{
    try {
        VarPlan p;
        if (make_varlen_plan(dt, n_seq, cu_seqlens, heads, d, 0, p) != LA_OK) return 0;
        return backward_varlen_bytes(p, n_seq, heads, d);
    } catch (...) {
        return 0;
    }
}

la_status la_backward_varlen(la_dtype dt, const void* q, const void* k, const void* v, const void* dout,
                             int64_t n_seq, const int64_t* cu_seqlens, int64_t heads, int64_t d,
                             int64_t stride_h, int64_t stride_n, const float* slopes, const float* kv_in,
                             const float* dkv_out, void* dq, void* dk, void* dv, float* dkv_in,
                             void* workspace, size_t workspace_bytes, void* stream)
{
    try {
        return backward_varlen_impl(dt, q, k, v, dout, n_seq, cu_seqlens, heads, d, stride_h, stride_n, slopes, kv_in,
                                    dkv_out, dq, dk, dv, dkv_in, workspace, workspace_bytes, stream);
    } catch (const std::exception& e) {
        return fail(LA_ERR_INTERNAL, e.what());
    } catch (...) {
        return fail(LA_ERR_INTERNAL, "unknown error");
    }
}

const char* la_status_string(la_status s)
{
    switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARGUMENT: return "LA_ERR_INVALID_ARGUMENT: invalid argument";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: outside the supported configurations";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace missing or too small";
    case LA_ERR_DEVICE: return "LA_ERR_DEVICE: GPU unavailable or HIP error";
    case LA_ERR_INTERNAL: return "LA_ERR_INTERNAL: internal error";
    }
    return "unknown la_status";
}

const char* la_last_error(void)
{
    return g_last_error.c_str();
}

}  // extern "C"
