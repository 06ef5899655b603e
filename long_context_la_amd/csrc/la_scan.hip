// Chunk-prefix combine and state initialisation.
//
// Page "MiniMax-01: Scaling Foundation Models with Lightning Attention |
// Summary", section 3.2 (LASP+): each sequence partition first computes a
// local summary, the summaries are gathered, and the global prefixes are
// built from them.  On one GPU the partitions are chunks of the sequence:
// slot j+1 of the workspace holds the local state S_j of chunk j (from a zero
// state); this kernel turns the slots into prefixes in place,
//     P_0 = KV_in,   P_{j+1} = lambda^C * P_j + S_j,
// so that slot j is the state entering chunk j.  Every state element is an
// independent scalar recurrence over the chunks, so threads own float4s of the
// state and walk the chunks; all loads of a thread are independent of the
// running value and are issued ahead of the multiply-adds.
#include "la_common.h"

namespace la {
namespace {

__global__ __launch_bounds__(256) void k_scan(float* __restrict__ ws, const float* __restrict__ kv,
                                              const float* __restrict__ slopes, int64_t bh,
                                              int64_t heads, int64_t n_chunks, int64_t chunk, int d2)
{
    const int64_t per = d2 / 4;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < bh * per; idx += (int64_t)gridDim.x * 256) {
        const int64_t u = idx / per;
        const int64_t e = idx % per;
        const float nsl = neg_slope_log2e(slopes, u % heads);
        const float lc = decay_pow(nsl, (float)chunk);
        float4* base = reinterpret_cast<float4*>(ws + u * n_chunks * (int64_t)d2) + e;
        float4 p = reinterpret_cast<const float4*>(kv + u * (int64_t)d2)[e];
        base[0] = p;
#pragma unroll 4
        for (int64_t j = 1; j < n_chunks; ++j) {
            const float4 s = base[j * per];
            p.x = lc * p.x + s.x;
            p.y = lc * p.y + s.y;
            p.z = lc * p.z + s.z;
            p.w = lc * p.w + s.w;
            base[j * per] = p;
        }
    }
}

// Chunk prefixes from sub-chunk summaries (the summary pass runs on sub-chunks to fill the GPU):
// the recurrence P <- lambda^sub_len P + S runs over the sub-chunks in order and P is stored at
// every chunk boundary.
template <bool WIN>
__global__ __launch_bounds__(256) void k_scan_sub(float* __restrict__ pref, const float* __restrict__ sub,
                                                  const float* __restrict__ kv, const float* __restrict__ slopes,
                                                  int64_t bh, int64_t heads, int64_t n_chunks, int64_t n_sub_per,
                                                  int64_t sub_len, bool f16, int d2)
{
    const int64_t per = d2 / 4;
    const int64_t n_sub = (n_chunks - 1) * n_sub_per;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < bh * per; idx += (int64_t)gridDim.x * 256) {
        const int64_t u = idx / per;
        const int64_t e = idx % per;
        const float nsl = neg_slope_log2e(slopes, u % heads);
        // WIN: sub-chunks over the head's window, whose chunk's first `gap` tokens are in none of
        // them; the prefix entering the chunk decays across those in two factors (each underflows
        // only where the product is below float32's range anyway)
        int64_t len = sub_len, gap = 0;
        float g1 = 1.f, g2 = 1.f;
        if constexpr (WIN) {
            len = summary_sub_len(summary_window(slopes[u % heads], f16), n_sub_per * sub_len, n_sub_per);
            gap = n_sub_per * (sub_len - len);
            g1 = decay_pow(nsl, (float)(gap / 2));
            g2 = decay_pow(nsl, (float)(gap - gap / 2));
        }
        const float ls = decay_pow(nsl, (float)len);
        const float4* S = reinterpret_cast<const float4*>(sub + u * (n_sub + 1) * (int64_t)d2) + e;
        float4* P = reinterpret_cast<float4*>(pref + u * n_chunks * (int64_t)d2) + e;
        float4 p = reinterpret_cast<const float4*>(kv + u * (int64_t)d2)[e];
        P[0] = p;
        // The sub-chunk states are loaded kGroup at a time before they are folded, so a group costs
        // one memory round trip instead of one per chunk.  After sub-chunk i (0-based) the fold has
        // covered (i + 1) / n_sub_per whole chunks; at each chunk boundary that prefix is stored.
        constexpr int kGroup = 16;
        int64_t j = 1;     // next chunk prefix to store
        int64_t f = 0;     // sub-chunks folded into the current chunk
        for (int64_t base = 0; base < n_sub; base += kGroup) {
            float4 s[kGroup];
#pragma unroll
            for (int q = 0; q < kGroup; ++q)
                s[q] = base + q < n_sub ? S[(base + q + 1) * per] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int q = 0; q < kGroup; ++q) {
                if (base + q < n_sub) {
                    if (WIN && gap > 0 && f == 0) {
                        p.x = p.x * g1 * g2;
                        p.y = p.y * g1 * g2;
                        p.z = p.z * g1 * g2;
                        p.w = p.w * g1 * g2;
                    }
                    p.x = ls * p.x + s[q].x;
                    p.y = ls * p.y + s[q].y;
                    p.z = ls * p.z + s[q].z;
                    p.w = ls * p.w + s[q].w;
                    if (++f == n_sub_per) {
                        P[j * per] = p;
                        ++j;
                        f = 0;
                    }
                }
            }
        }
    }
}

// Packed variable-length batches: the chunks of sequence s are global chunks c0..c0+nc-1 (stab)
// and slot (c, h) = c*heads + h; slot (c0+j+1, h) holds the local state of chunk j.
__global__ __launch_bounds__(256) void k_scan_varlen(float* __restrict__ ws, const float* __restrict__ kv,
                                                     const float* __restrict__ slopes,
                                                     const int64_t* __restrict__ stab, int64_t n_seq,
                                                     int64_t heads, int64_t chunk, int d2)
{
    const int64_t per = d2 / 4;
    const int64_t step = heads * per;  // float4s between slots (c, h) and (c+1, h)
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n_seq * heads * per;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t u = idx / per;
        const int64_t e = idx % per;
        const int64_t sq = u / heads, h = u % heads;
        const int64_t c0 = stab[2 * sq], nc = stab[2 * sq + 1];
        if (nc <= 1) continue;
        const float nsl = neg_slope_log2e(slopes, h);
        const float lc = decay_pow(nsl, (float)chunk);
        float4* base = reinterpret_cast<float4*>(ws + (c0 * heads + h) * (int64_t)d2) + e;
        float4 p = reinterpret_cast<const float4*>(kv + u * (int64_t)d2)[e];
        base[0] = p;
#pragma unroll 4
        for (int64_t j = 1; j < nc; ++j) {
            const float4 s = base[j * step];
            p.x = lc * p.x + s.x;
            p.y = lc * p.y + s.y;
            p.z = lc * p.z + s.z;
            p.w = lc * p.w + s.w;
            base[j * step] = p;
        }
    }
}

__global__ __launch_bounds__(256) void k_state_init(float* __restrict__ kv, const float* __restrict__ kv0,
                                                    int64_t count4)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count4; i += (int64_t)gridDim.x * 256)
        reinterpret_cast<float4*>(kv)[i] =
            kv0 ? reinterpret_cast<const float4*>(kv0)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

// Backward-pass state set-up: a state (or its transpose) scaled by exp(power * s_h).
__global__ __launch_bounds__(256) void k_state_prep(float* __restrict__ dst, const float* __restrict__ src,
                                                    const float* __restrict__ slopes, int64_t bh, int64_t heads,
                                                    int d, int transpose, int power)
{
    const int64_t d2 = (int64_t)d * d;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < bh * d2; idx += (int64_t)gridDim.x * 256) {
        const int64_t u = idx / d2, e = idx % d2;
        float x = 0.f;
        if (src) {
            const int64_t r = e / d, c = e % d;
            x = src[u * d2 + (transpose ? c * d + r : e)];
            if (power != 0) x *= exp2f(-(float)power * neg_slope_log2e(slopes, u % heads));
        }
        dst[idx] = x;
    }
}

// Checkpoint slot m of every (batch, head): ckpt[u][m] := kv[u] for the bh states u (d2 floats each,
// n_ckpt slots per state in ckpt).
__global__ __launch_bounds__(256) void k_state_to_slot(float* __restrict__ ckpt, const float* __restrict__ kv,
                                                       int64_t bh, int64_t d2, int64_t n_ckpt, int64_t m)
{
    const int64_t per4 = d2 / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < bh * per4; i += (int64_t)gridDim.x * 256) {
        const int64_t u = i / per4, e = i % per4;
        reinterpret_cast<float4*>(ckpt + (u * n_ckpt + m) * d2)[e] = reinterpret_cast<const float4*>(kv + u * d2)[e];
    }
}

// Grid of a grid-stride kernel over `items` threads' worth of work (256 per block), capped so the
// launch stays far inside the 32-bit work-item count of a dispatch.
dim3 stride_grid(int64_t items)
{
    const int64_t blocks = (items + 255) / 256;
    return dim3((unsigned)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536));
}

}  // namespace

hipError_t launch_state_prep(float* dst, const float* src, const float* slopes, int64_t bh, int64_t heads,
                             int d, bool transpose, int power, hipStream_t stream)
{
    const int64_t count = bh * (int64_t)d * d;
    const dim3 grid = stride_grid(count), block(256);
    hipLaunchKernelGGL(k_state_prep, grid, block, 0, stream, dst, src, slopes, bh, heads, d, transpose ? 1 : 0,
                       power);
    return hipGetLastError();
}

hipError_t launch_scan(float* ws, const float* kv, const float* slopes, int64_t bh, int64_t heads,
                       int64_t n_chunks, int64_t chunk, int d, hipStream_t stream)
{
    const int d2 = d * d;
    const int64_t threads = bh * (d2 / 4);
    const dim3 grid = stride_grid(threads), block(256);
    hipLaunchKernelGGL(k_scan, grid, block, 0, stream, ws, kv, slopes, bh, heads, n_chunks, chunk, d2);
    return hipGetLastError();
}

hipError_t launch_scan_sub(float* pref, const float* sub, const float* kv, const float* slopes, int64_t bh,
                           int64_t heads, int64_t n_chunks, int64_t n_sub_per, int64_t sub_len, int window,
                           int d, hipStream_t stream)
{
    const int d2 = d * d;
    const int64_t threads = bh * (d2 / 4);
    const dim3 grid = stride_grid(threads), block(256);
    if (window)
        hipLaunchKernelGGL(k_scan_sub<true>, grid, block, 0, stream, pref, sub, kv, slopes, bh, heads, n_chunks,
                           n_sub_per, sub_len, window == 1, d2);
    else
        hipLaunchKernelGGL(k_scan_sub<false>, grid, block, 0, stream, pref, sub, kv, slopes, bh, heads, n_chunks,
                           n_sub_per, sub_len, false, d2);
    return hipGetLastError();
}

hipError_t launch_scan_varlen(float* ws, const float* kv, const float* slopes, const int64_t* stab,
                              int64_t n_seq, int64_t heads, int64_t chunk, int d, hipStream_t stream)
{
    const int d2 = d * d;
    const int64_t threads = n_seq * heads * (d2 / 4);
    const dim3 grid = stride_grid(threads), block(256);
    hipLaunchKernelGGL(k_scan_varlen, grid, block, 0, stream, ws, kv, slopes, stab, n_seq, heads, chunk, d2);
    return hipGetLastError();
}

hipError_t launch_state_to_slot(float* ckpt, const float* kv, int64_t bh, int d, int64_t n_ckpt, int64_t m,
                                hipStream_t stream)
{
    const int64_t d2 = (int64_t)d * d;
    const dim3 grid = stride_grid(bh * (d2 / 4)), block(256);
    hipLaunchKernelGGL(k_state_to_slot, grid, block, 0, stream, ckpt, kv, bh, d2, n_ckpt, m);
    return hipGetLastError();
}

hipError_t launch_state_init(float* kv, const float* kv0, int64_t count, hipStream_t stream)
{
    const int64_t count4 = count / 4;  // count = B*H*d*d, a multiple of 4096
    const dim3 grid = stride_grid(count4), block(256);
    hipLaunchKernelGGL(k_state_init, grid, block, 0, stream, kv, kv0, count4);
    return hipGetLastError();
}

}  // namespace la
