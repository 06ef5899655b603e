// Float32 prefill (the exact-arithmetic path, d = 64 or 128) on gfx950.
//
// Page "MiniMax-01: Scaling Foundation Models with Lightning Attention |
// Summary", section 2.2: the sequence is split into tiles; tile i of L tokens
// with incoming state KV gets
//     o_r = lambda^(r+1) q_r KV + sum_{c<=r} lambda^(r-c) (q_r . k_c) v_c     (inter + intra)
// and then KV <- lambda^L KV + sum_c lambda^(L-1-c) k_c^T v_c.
// Work is O(n d^2 + n B d) with B the tile length.
//
// One 256-thread workgroup owns one (batch, head, chunk, 32-column value
// slice): the state's columns and the outputs' columns split cleanly by value
// column, so slices need no communication.  Everything is float32 FMAs on
// LDS tiles; this path favours plain, checkable arithmetic over speed (the
// bfloat16 path is the fast one).
#include "la_common.h"

namespace la {
namespace {

template <int D, int MODE>
__global__ __launch_bounds__(256) void k_fwd_f32(FwdArgs a)
{
    constexpr int BK = kBlock, SW = kSliceW;
    constexpr int RPT = D / 8;  // state rows per thread (thread owns column tid%32, rows tid/32 + 8m)
    __shared__ float sQ[BK][D + 1];
    __shared__ float sK[BK][D + 1];
    __shared__ float sV[BK][SW];
    __shared__ float sP[BK][BK + 1];
    __shared__ float sKV[D][SW];
    __shared__ float sW[BK];

    int64_t group;
    int slice;
    xcd_decode(blockIdx.x, a.slices, group, slice);
    if (group >= a.groups) return;
    const Work wk = decode_work(a, group);
    if (MODE == kModeLocal && wk.j == wk.nck - 1) return;  // last chunks need no summary
    const int64_t u = wk.u, j = wk.j, h = wk.h;
    const int64_t t_begin = wk.t_begin, t_end = wk.t_end;
    const int tid = threadIdx.x;
    const int col = tid % SW;
    const int row0 = tid / SW;
    const float nsl = neg_slope_log2e(a.slopes, h);
    const int64_t base = wk.base;
    const float* Q = static_cast<const float*>(a.q) + base;
    const float* K = static_cast<const float*>(a.k) + base;
    const float* V = static_cast<const float*>(a.v) + base;
    float* O = static_cast<float*>(a.o) + base;
    const int64_t d2 = (int64_t)D * D;
    // memory row of token t of the recurrence: t, or n-1-t when the sequence is walked backwards
    // (the reverse state recurrence of the backward pass)
    auto mrow = [&](int64_t t) { return a.rev ? wk.rev_end - 1 - t : t; };

    // incoming state slice
    float st[RPT];
    const float* src = nullptr;
    if (MODE != kModeLocal) src = (wk.nck > 1) ? a.ws + wk.slot_in * d2 : a.kv + u * d2;
#pragma unroll
    for (int m = 0; m < RPT; ++m) st[m] = src ? src[(row0 + 8 * m) * D + slice * SW + col] : 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) sKV[row0 + 8 * m][col] = st[m];

    for (int64_t t0 = t_begin; t0 < t_end; t0 += BK) {
        const int L = (int)((t_end - t0 < BK) ? t_end - t0 : BK);
        __syncthreads();  // previous tile's readers are done
        for (int e = tid; e < BK * (D / 4); e += 256) {
            const int r = e / (D / 4), c4 = e % (D / 4);
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), qx = kx;
            if (r < L) {
                kx = *reinterpret_cast<const float4*>(K + mrow(t0 + r) * a.sn + 4 * c4);
                if (MODE == kModeOut) qx = *reinterpret_cast<const float4*>(Q + mrow(t0 + r) * a.sn + 4 * c4);
                if (a.act & LA_SILU_K) kx = make_float4(silu_f32(kx.x), silu_f32(kx.y), silu_f32(kx.z), silu_f32(kx.w));
                if (a.act & LA_SILU_Q) qx = make_float4(silu_f32(qx.x), silu_f32(qx.y), silu_f32(qx.z), silu_f32(qx.w));
            }
            sK[r][4 * c4] = kx.x; sK[r][4 * c4 + 1] = kx.y; sK[r][4 * c4 + 2] = kx.z; sK[r][4 * c4 + 3] = kx.w;
            sQ[r][4 * c4] = qx.x; sQ[r][4 * c4 + 1] = qx.y; sQ[r][4 * c4 + 2] = qx.z; sQ[r][4 * c4 + 3] = qx.w;
        }
        for (int e = tid; e < BK * SW; e += 256) {
            const int r = e / SW, c = e % SW;
            const float x = (r < L) ? V[mrow(t0 + r) * a.sn + slice * SW + c] : 0.f;
            sV[r][c] = (a.act & LA_SILU_V) ? silu_f32(x) : x;
        }
        if (tid < BK) sW[tid] = (tid < L) ? decay_pow(nsl, (float)(L - 1 - tid)) : 0.f;
        __syncthreads();

        if (MODE == kModeOut) {
            // masked, decayed scores P[r][c] = lambda^(r-c) q_r . k_c  (c <= r)
            for (int e = tid; e < BK * BK; e += 256) {
                const int r = e / BK, c = e % BK;
                float p = 0.f;
                if (c <= r) {
                    float dot = 0.f;
#pragma unroll 8
                    for (int i = 0; i < D; ++i) dot += sQ[r][i] * sK[c][i];
                    p = dot * decay_pow(nsl, (float)(r - c));
                }
                sP[r][c] = p;
            }
            __syncthreads();
            for (int r = row0; r < L; r += 8) {
                float inter = 0.f;
#pragma unroll 8
                for (int i = 0; i < D; ++i) inter += sQ[r][i] * sKV[i][col];
                float acc = decay_pow(nsl, (float)(r + 1)) * inter;
                for (int c = 0; c <= r; ++c) acc += sP[r][c] * sV[c][col];
                if (a.gate) acc *= sigmoid_f32(static_cast<const float*>(a.gate)[base + mrow(t0 + r) * a.sn + slice * SW + col]);
                O[mrow(t0 + r) * a.sn + slice * SW + col] = acc;
            }
        }

        // state update
        const float dl = decay_pow(nsl, (float)L);
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = row0 + 8 * m;
            float acc = 0.f;
            for (int c = 0; c < L; ++c) acc += sW[c] * sK[c][i] * sV[c][col];
            st[m] = dl * st[m] + acc;
        }
        __syncthreads();  // all inter-term reads of sKV are done
#pragma unroll
        for (int m = 0; m < RPT; ++m) sKV[row0 + 8 * m][col] = st[m];

        if (MODE != kModeLocal && a.ckpt) {
            const int64_t end = t0 + L;
            if (end % a.ckpt_every == 0) {
                float* dst = a.ckpt + (u * a.n_ckpt + (end / a.ckpt_every - 1)) * d2;
#pragma unroll
                for (int m = 0; m < RPT; ++m) dst[(row0 + 8 * m) * D + slice * SW + col] = st[m];
            }
        }
    }

    float* dst = nullptr;
    if (MODE == kModeLocal) dst = a.ws + wk.slot_out * d2;
    else if (j == wk.nck - 1) dst = a.kv + u * d2;
    if (dst) {
#pragma unroll
        for (int m = 0; m < RPT; ++m) dst[(row0 + 8 * m) * D + slice * SW + col] = st[m];
    }
}

template <int D>
hipError_t launch_d(const FwdArgs& a, int mode, hipStream_t stream)
{
    const dim3 grid((unsigned)xcd_grid_size(a.groups, a.slices)), block(256);
    if (mode == kModeOut) hipLaunchKernelGGL((k_fwd_f32<D, kModeOut>), grid, block, 0, stream, a);
    else if (mode == kModeState) hipLaunchKernelGGL((k_fwd_f32<D, kModeState>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_fwd_f32<D, kModeLocal>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, int d, int mode, hipStream_t stream)
{
    return d == 128 ? launch_d<128>(a, mode, stream) : launch_d<64>(a, mode, stream);
}

}  // namespace la
