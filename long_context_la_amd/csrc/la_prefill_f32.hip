// Float32 prefill (the exact-arithmetic path, d = 64 or 128) on gfx950.
//
// Page "MiniMax-01: Scaling Foundation Models with Lightning Attention |
// Summary", section 2.2: the sequence is split into tiles; tile i of L tokens
// with incoming state KV gets
//     o_r = lambda^(r+1) q_r KV + sum_{c<=r} lambda^(r-c) (q_r . k_c) v_c     (inter + intra)
// and then KV <- lambda^L KV + sum_c lambda^(L-1-c) k_c^T v_c.
// Work is O(n d^2 + n B d) with B the tile length.
//
// One 512-thread workgroup (two waves per SIMD) owns one (batch, head, chunk,
// 32-column value slice): the state's columns and the outputs' columns split
// cleanly by value column, so slices need no communication.  Everything is
// float32 FMAs on LDS tiles (the bfloat16 path is the matrix-core one).  Each
// thread keeps a block of results in registers and reads its operands as 8- or
// 16-byte runs, so one LDS read feeds 2 to 8 FMAs:
//   scores  P[r][c]     rows 8w + 4x (x = (t%64)/32, wave w), keys t%32 + 32b
//                       for the key blocks b that reach the wave's 8 rows
//   outputs O[r][col]   rows 2(t/16)..+1, columns 2(t%16), 2(t%16)+1
//   state   KV[i][col]  key rows R(t/8)..+R-1 (R = d/64), columns 4(t%8)..+3
// Row paddings of 4 floats put consecutive rows on distinct banks for these
// reads.
#include "la_common.h"

namespace la {
namespace {

template <int N> struct IntC { static constexpr int value = N; };

__device__ inline float dot4(float4 x, float4 y, float acc)
{
    acc = fmaf(x.x, y.x, acc);
    acc = fmaf(x.y, y.y, acc);
    acc = fmaf(x.z, y.z, acc);
    return fmaf(x.w, y.w, acc);
}
__device__ inline float4 silu4(float4 x)
{
    return make_float4(silu_f32(x.x), silu_f32(x.y), silu_f32(x.z), silu_f32(x.w));
}

constexpr int kThreads = 512;

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) void k_fwd_f32(FwdArgs a)
{
    constexpr int BK = kBlock, SW = kSliceW;
    constexpr int DP = D + 4, SP = SW + 4, PP = BK + 4;  // padded rows (floats)
    constexpr int RI = D / 64;                           // state rows per thread
    constexpr bool OUT = MODE == kModeOut;
    __shared__ __attribute__((aligned(16))) float sQ[OUT ? BK : 1][DP];
    __shared__ __attribute__((aligned(16))) float sK[BK][DP];
    __shared__ __attribute__((aligned(16))) float sV[OUT ? BK : 1][SP];
    __shared__ __attribute__((aligned(16))) float sVW[BK][SP];
    __shared__ __attribute__((aligned(16))) float sP[OUT ? BK : 1][PP];
    __shared__ __attribute__((aligned(16))) float sKV[OUT ? D : 1][SP];
    __shared__ float sDec[BK + 1];  // lambda^k, k = 0..BK

    int64_t group;
    int slice;
    xcd_decode(blockIdx.x, a.slices, group, slice);
    if (group >= a.groups) return;
    const Work wk = decode_work(a, group);
    if (MODE == kModeLocal && wk.j == wk.nck - 1) return;  // last chunks need no summary
    const int64_t u = wk.u, j = wk.j, h = wk.h;
    const int64_t t_begin = wk.t_begin, t_end = wk.t_end;
    const int tid = threadIdx.x;
    const int wv = tid >> 6;                                  // wave: score rows 8wv..8wv+7
    const int sr = 8 * wv + 4 * ((tid & 63) >> 5), sc = tid & 31;  // score block: rows sr..+3, keys sc + 32b
    const int rb = tid >> 4, cb = tid & 15;                   // output block: rows 2rb..+1, columns 2cb..+1
    const int ib = tid >> 3, jb = tid & 7;                    // state block
    const float nsl = neg_slope_log2e(a.slopes, h);
    const int64_t base = wk.base;
    const float* Q = static_cast<const float*>(a.q) + base;
    const float* K = static_cast<const float*>(a.k) + base;
    const float* V = static_cast<const float*>(a.v) + base + slice * SW;
    float* O = static_cast<float*>(a.o) + base + slice * SW;
    const float* G = a.gate ? static_cast<const float*>(a.gate) + base + slice * SW : nullptr;
    const int64_t d2 = (int64_t)D * D;
    // memory row of token t of the recurrence: t, or rev_end-1-t when the sequence is walked
    // backwards (the reverse state recurrence of the backward pass)
    auto mrow = [&](int64_t t) { return a.rev ? wk.rev_end - 1 - t : t; };
    if (tid <= BK) sDec[tid] = decay_pow(nsl, (float)tid);

    // this thread's block of the incoming state slice, also published to LDS for the inter term
    float st[RI][4];
    const float* src = nullptr;
    if (MODE != kModeLocal) src = (wk.nck > 1) ? a.ws + wk.slot_in * d2 : a.kv + u * d2;
    auto state_at = [&](int r, int e) { return (RI * ib + r) * D + slice * SW + 4 * jb + e; };
#pragma unroll
    for (int r = 0; r < RI; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[r][e] = src ? src[state_at(r, e)] : 0.f;
    auto publish = [&]() {
        if constexpr (OUT)
#pragma unroll
            for (int r = 0; r < RI; ++r)
                *reinterpret_cast<float4*>(&sKV[RI * ib + r][4 * jb]) =
                    make_float4(st[r][0], st[r][1], st[r][2], st[r][3]);
    };
    publish();

    // masked, decayed scores of this thread's 4 rows against key blocks 0..NB-1 (a later block
    // lies wholly above the wave's rows)
    auto scores = [&](auto nbc) __attribute__((always_inline)) {
        constexpr int NB = decltype(nbc)::value;
        float s[4][NB];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int b = 0; b < NB; ++b) s[x][b] = 0.f;
#pragma unroll 2
        for (int i = 0; i < D; i += 4) {
            float4 q[4], k[NB];
#pragma unroll
            for (int x = 0; x < 4; ++x) q[x] = *reinterpret_cast<const float4*>(&sQ[sr + x][i]);
#pragma unroll
            for (int b = 0; b < NB; ++b) k[b] = *reinterpret_cast<const float4*>(&sK[sc + 32 * b][i]);
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int b = 0; b < NB; ++b) s[x][b] = dot4(q[x], k[b], s[x][b]);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int r = sr + x, c = sc + 32 * b;
                sP[r][c] = (b < NB && c <= r) ? s[x][b < NB ? b : 0] * sDec[r - c] : 0.f;
            }
    };

    for (int64_t t0 = t_begin; t0 < t_end; t0 += BK) {
        const int L = (int)((t_end - t0 < BK) ? t_end - t0 : BK);
        __syncthreads();  // the previous tile's readers are done; the published state is visible
        for (int e = tid; e < BK * (D / 4); e += kThreads) {
            const int r = e / (D / 4), c4 = e % (D / 4);
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), qx = kx;
            if (r < L) {
                kx = *reinterpret_cast<const float4*>(K + mrow(t0 + r) * a.sn + 4 * c4);
                if (a.act & LA_SILU_K) kx = silu4(kx);
                if (OUT) {
                    qx = *reinterpret_cast<const float4*>(Q + mrow(t0 + r) * a.sn + 4 * c4);
                    if (a.act & LA_SILU_Q) qx = silu4(qx);
                }
            }
            *reinterpret_cast<float4*>(&sK[r][4 * c4]) = kx;
            if constexpr (OUT) *reinterpret_cast<float4*>(&sQ[r][4 * c4]) = qx;
        }
        for (int e = tid; e < BK * (SW / 4); e += kThreads) {
            const int r = e / (SW / 4), c4 = e % (SW / 4);
            float4 vx = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < L) {
                vx = *reinterpret_cast<const float4*>(V + mrow(t0 + r) * a.sn + 4 * c4);
                if (a.act & LA_SILU_V) vx = silu4(vx);
            }
            if constexpr (OUT) *reinterpret_cast<float4*>(&sV[r][4 * c4]) = vx;
            const float w = (r < L) ? sDec[L - 1 - r] : 0.f;  // W = lambda^(L-1-r)
            *reinterpret_cast<float4*>(&sVW[r][4 * c4]) = make_float4(w * vx.x, w * vx.y, w * vx.z, w * vx.w);
        }
        __syncthreads();

        if constexpr (OUT) {
            if (wv < 4) scores(IntC<1>{});  // rows below 32 meet keys 0..31 only
            else scores(IntC<2>{});
            __syncthreads();
            // o = lambda^(r+1) q_r KV + sum_{c <= r} P[r][c] v_c  (P is zero above the diagonal)
            float o[2][2];
#pragma unroll
            for (int x = 0; x < 2; ++x) o[x][0] = o[x][1] = 0.f;
#pragma unroll 2
            for (int i = 0; i < D; i += 4) {
                float4 q[2];
                float2 kv[4];
#pragma unroll
                for (int x = 0; x < 2; ++x) q[x] = *reinterpret_cast<const float4*>(&sQ[2 * rb + x][i]);
#pragma unroll
                for (int e = 0; e < 4; ++e) kv[e] = *reinterpret_cast<const float2*>(&sKV[i + e][2 * cb]);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    o[x][0] = dot4(q[x], make_float4(kv[0].x, kv[1].x, kv[2].x, kv[3].x), o[x][0]);
                    o[x][1] = dot4(q[x], make_float4(kv[0].y, kv[1].y, kv[2].y, kv[3].y), o[x][1]);
                }
            }
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const float dr = sDec[2 * rb + x + 1];
                o[x][0] *= dr;
                o[x][1] *= dr;
            }
            const int c_end = 8 * wv + 8;  // keys at or before this wave's last row (rows 8wv..8wv+7)
            for (int c = 0; c < c_end; c += 4) {
                float4 p[2];
                float2 v[4];
#pragma unroll
                for (int x = 0; x < 2; ++x) p[x] = *reinterpret_cast<const float4*>(&sP[2 * rb + x][c]);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = *reinterpret_cast<const float2*>(&sV[c + e][2 * cb]);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    o[x][0] = dot4(p[x], make_float4(v[0].x, v[1].x, v[2].x, v[3].x), o[x][0]);
                    o[x][1] = dot4(p[x], make_float4(v[0].y, v[1].y, v[2].y, v[3].y), o[x][1]);
                }
            }
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int r = 2 * rb + x;
                if (r >= L) continue;
                const int64_t at = mrow(t0 + r) * a.sn + 2 * cb;
                float2 y = make_float2(o[x][0], o[x][1]);
                if (G) {
                    const float2 g = *reinterpret_cast<const float2*>(G + at);
                    y.x *= sigmoid_f32(g.x);
                    y.y *= sigmoid_f32(g.y);
                }
                *reinterpret_cast<float2*>(O + at) = y;
            }
        }

        // state update on this thread's block: KV <- lambda^L KV + K^T (W V)
        const float dl = sDec[L];
        float acc[RI][4];
#pragma unroll
        for (int r = 0; r < RI; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[r][e] = 0.f;
        for (int c = 0; c < L; ++c) {
            const float4 w4 = *reinterpret_cast<const float4*>(&sVW[c][4 * jb]);
            float kk[RI];
            if constexpr (RI == 2) {
                const float2 k2 = *reinterpret_cast<const float2*>(&sK[c][2 * ib]);
                kk[0] = k2.x; kk[1] = k2.y;
            } else {
                kk[0] = sK[c][ib];
            }
#pragma unroll
            for (int r = 0; r < RI; ++r) {
                acc[r][0] = fmaf(kk[r], w4.x, acc[r][0]);
                acc[r][1] = fmaf(kk[r], w4.y, acc[r][1]);
                acc[r][2] = fmaf(kk[r], w4.z, acc[r][2]);
                acc[r][3] = fmaf(kk[r], w4.w, acc[r][3]);
            }
        }
#pragma unroll
        for (int r = 0; r < RI; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) st[r][e] = fmaf(dl, st[r][e], acc[r][e]);
        __syncthreads();  // all inter-term reads of the published state are done
        publish();

        if (MODE != kModeLocal && a.ckpt) {
            const int64_t end = t0 + L;
            if (end % a.ckpt_every == 0) {
                float* dst = a.ckpt + (u * a.n_ckpt + (end / a.ckpt_every - 1)) * d2;
#pragma unroll
                for (int r = 0; r < RI; ++r)
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[state_at(r, e)] = st[r][e];
            }
        }
    }

    float* dst = nullptr;
    if (MODE == kModeLocal) dst = a.ws + wk.slot_out * d2;
    else if (j == wk.nck - 1) dst = a.kv + u * d2;
    if (dst) {
#pragma unroll
        for (int r = 0; r < RI; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[state_at(r, e)] = st[r][e];
    }
}

template <int D>
hipError_t launch_d(const FwdArgs& a, int mode, hipStream_t stream)
{
    const dim3 grid((unsigned)xcd_grid_size(a.groups, a.slices)), block(kThreads);
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
