// C ABI of liblightning_la.so: argument validation, work planning and
// dispatch to the gfx950 kernels.  See include/la.h for the contract.
#include <string.h>

#include <exception>
#include <string>

#include "la_common.h"

namespace la {
namespace {

thread_local std::string g_last_error;

la_status fail(la_status s, const std::string& msg)
{
    g_last_error = msg;
    return s;
}

la_status ok()
{
    return LA_OK;
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

Plan make_plan(int64_t batch, int64_t heads, int64_t n, int64_t d, int64_t chunk_override)
{
    Plan p;
    p.slices = (int)(d / kSliceW);
    const int64_t units = batch * heads * p.slices;
    int64_t chunk = n;
    if (chunk_override > 0) {
        chunk = chunk_override;
    } else if (units < kTargetGroups && n > kMinChunk) {
        const int64_t want = (kTargetGroups + units - 1) / units;  // chunks per sequence
        int64_t c = (n + want - 1) / want;
        c = ((c + kBlock - 1) / kBlock) * kBlock;
        if (c < kMinChunk) c = kMinChunk;
        chunk = c;
    }
    if (chunk >= n) {
        p.chunk = n > 0 ? n : 1;
        p.n_chunks = 1;
    } else {
        p.chunk = chunk;
        p.n_chunks = (n + chunk - 1) / chunk;
    }
    return p;
}

}  // namespace la

using namespace la;

namespace {

la_status check_shape(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d)
{
    if (dt != LA_F32 && dt != LA_BF16) return fail(LA_ERR_INVALID_ARGUMENT, "dtype must be LA_F32 or LA_BF16");
    if (batch < 1 || heads < 1 || n < 0 || d < 1)
        return fail(LA_ERR_INVALID_ARGUMENT, "batch, heads, d must be >= 1 and n >= 0");
    if (d != 64 && d != 128) return fail(LA_ERR_UNSUPPORTED, "d must be 64 or 128");
    if (dt == LA_BF16 && d != 128) return fail(LA_ERR_UNSUPPORTED, "bf16 prefill supports d = 128 only");
    if (batch > (int64_t(1) << 24) || heads > (int64_t(1) << 24) || n > (int64_t(1) << 40))
        return fail(LA_ERR_INVALID_ARGUMENT, "size out of range");
    return LA_OK;
}

size_t workspace_bytes_for(const Plan& p, int64_t batch, int64_t heads, int64_t d)
{
    if (p.n_chunks <= 1) return 0;
    return (size_t)batch * (size_t)heads * (size_t)p.n_chunks * (size_t)d * (size_t)d * sizeof(float);
}

la_status prefill_impl(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                       int64_t batch, int64_t heads, int64_t n, int64_t d,
                       int64_t sb, int64_t sh, int64_t sn, const float* slopes, float* kv,
                       float* ckpt, int64_t ckpt_every, int64_t chunk_tokens,
                       void* workspace, size_t workspace_bytes, void* stream)
{
    la_status s = check_shape(dt, batch, heads, n, d);
    if (s != LA_OK) return s;
    if (!kv || !slopes) return fail(LA_ERR_INVALID_ARGUMENT, "kv and slopes must not be NULL");
    if (chunk_tokens < 0 || (chunk_tokens > 0 && chunk_tokens % kBlock != 0))
        return fail(LA_ERR_INVALID_ARGUMENT, "chunk_tokens must be 0 or a positive multiple of 64");
    if (ckpt && (ckpt_every <= 0 || ckpt_every % kBlock != 0))
        return fail(LA_ERR_UNSUPPORTED, "ckpt_every must be a positive multiple of 64");
    if (n == 0) return LA_OK;
    if (!q || !k || !v) return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v must not be NULL");
    const int64_t align = (dt == LA_BF16) ? 8 : 4;
    if (sn < d || sb < 0 || sh < 0 || sb % align || sh % align || sn % align)
        return fail(LA_ERR_INVALID_ARGUMENT, "strides must be >= 0, multiples of 16 bytes, stride_n >= d");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (o && !aligned16(o)) || !aligned16(kv) ||
        (ckpt && !aligned16(ckpt)))
        return fail(LA_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");

    const Plan p = make_plan(batch, heads, n, d, chunk_tokens);
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
    const int64_t bh = batch * heads;
    hipStream_t st = static_cast<hipStream_t>(stream);

    auto run = [&](int mode, int64_t chunks) -> hipError_t {
        FwdArgs b = a;
        b.chunks_launched = chunks;
        b.groups = bh * chunks;
        return dt == LA_BF16 ? launch_fwd_bf16(b, mode, st) : launch_fwd_f32(b, (int)d, mode, st);
    };

    if (p.n_chunks > 1) {
        s = launch_status(run(kModeLocal, p.n_chunks - 1), "chunk-summary launch");
        if (s != LA_OK) return s;
        s = launch_status(launch_scan(a.ws, kv, slopes, bh, heads, p.n_chunks, p.chunk, (int)d, st),
                          "prefix-combine launch");
        if (s != LA_OK) return s;
    }
    return launch_status(run(o ? kModeOut : kModeState, p.n_chunks), "prefill launch");
}

}  // namespace

extern "C" {

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
    const Plan p = make_plan(batch, heads, n, d, 0);
    return p.n_chunks > 1 ? p.chunk : n;
}

size_t la_prefill_workspace_size_ex(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d,
                                    int64_t chunk_tokens)
{
    if (check_shape(dt, batch, heads, n, d) != LA_OK) return 0;
    if (chunk_tokens < 0 || (chunk_tokens > 0 && chunk_tokens % kBlock != 0)) return 0;
    return workspace_bytes_for(make_plan(batch, heads, n, d, chunk_tokens), batch, heads, d);
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

la_status la_decode(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                    int64_t batch, int64_t heads, int64_t d, const float* slopes, float* kv, void* stream)
{
    try {
        if (dt != LA_F32 && dt != LA_BF16) return fail(LA_ERR_INVALID_ARGUMENT, "dtype must be LA_F32 or LA_BF16");
        if (!q || !k || !v || !o || !slopes || !kv)
            return fail(LA_ERR_INVALID_ARGUMENT, "q, k, v, o, slopes and kv must not be NULL");
        if (batch < 1 || heads < 1) return fail(LA_ERR_INVALID_ARGUMENT, "batch and heads must be >= 1");
        if (d != 64 && d != 128) return fail(LA_ERR_UNSUPPORTED, "d must be 64 or 128");
        if (batch * heads > (int64_t(1) << 31) - 1) return fail(LA_ERR_INVALID_ARGUMENT, "too many (batch, head) pairs");
        if (!aligned16(kv)) return fail(LA_ERR_INVALID_ARGUMENT, "kv must be 16-byte aligned");
        la_status s = device_check();
        if (s != LA_OK) return s;
        return launch_status(launch_decode(dt, q, k, v, o, batch * heads, heads, (int)d, slopes, kv,
                                           static_cast<hipStream_t>(stream)),
                             "decode launch");
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
