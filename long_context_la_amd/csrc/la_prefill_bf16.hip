// bfloat16 prefill on gfx950 matrix cores (d = 128).
//
// Page "MiniMax-01: Scaling Foundation Models with Lightning Attention |
// Summary", section 2.2: tiles of the sequence get an intra-tile masked term
// and an inter-tile term from the accumulated key-value state, after which the
// state is updated.  For a tile of L tokens with incoming state KV and decay
// lambda = exp(-s):
//     S^T[c][r] = k_c . q_r                       (MFMA, k = feature dim)
//     P[r][c]   = lambda^(r-c) S[r][c]  (c <= r), 0 otherwise
//     O         = diag(lambda^(r+1)) Q KV + P V    (MFMA, k = feature dim, then k = token)
//     KV       <- lambda^L KV + K^T (W V),  W = diag(lambda^(L-1-c))   (MFMA, k = token)
// Inputs are bfloat16.  P, W V and the operand copy of the state are carried
// as bfloat16 hi + lo pairs (x = hi + lo, both parts bf16, two MFMAs per
// product), which keeps them to about float32 precision: rounding them to a
// single bf16 costs about 2e-2 of the output RMS on fast-decaying heads (P),
// 1.6e-2 of the state RMS (W V), and up to 2.5e-2 of the output RMS right
// after a large incoming state (KV).  Every product accumulates in float32 and
// the state itself stays float32 in accumulators.
//
// Decomposition.  A workgroup (4 waves) owns one (batch, head, chunk, slice of
// 32 value columns): both the state's columns and the outputs' columns split
// by value column with no communication, which gives 4 workgroups per head
// without a second pass over K and V.  Q and K rows are read by the four
// slices of a head; their workgroups sit on one XCD so the re-reads hit L2.
// Sequences with too few heads to fill the GPU are also cut into chunks
// (la_scan.hip combines the chunk summaries).
//
// Per 64-token tile, wave w owns query rows 16w..16w+15 (scores, masking,
// outputs) and state rows 32w..32w+31.  MFMA used: v_mfma_f32_16x16x32_bf16
// (A 16x32, B 32x16, C 16x16 fp32; lane l holds A row l%16 / B column l%16 and
// 8 consecutive k of group l/16; C column l%16, rows 4(l/16)..+3).  Any
// permutation of k works as long as A and B use the same one; this is used
// twice:
//   * S is computed transposed (S^T = K Q^T), so a lane's accumulator holds
//     one query row r and the key columns {4g..4g+3} and {16+4g..16+4g+3} of
//     two adjacent 16-key tiles -- exactly an A operand of P.V over a 32-key
//     step with that k order, with no data movement;
//   * V^T and K^T are stored in LDS with tokens in that same order (tok_pos),
//     so the B operand of P.V and both operands of the state update are plain
//     16-byte LDS reads.
// Q goes straight from global memory into registers in operand layout (it is
// the B operand of S^T and the A operand of Q.KV for the same rows).  K is
// staged twice: row-major for S^T and transposed for the state update; V is
// staged transposed, plain for P.V and decay-weighted (hi + lo) for the state
// update.  Staging of tile b+1 overlaps tile b (global
// loads issued before the tile's MFMAs, LDS double-buffered), one barrier per
// tile.
#include "la_common.h"

namespace la {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr int D = 128, BK = kBlock, SW = kSliceW;
constexpr int KS = D + 8;   // row stride (elements) of row-major K tiles
constexpr int TS = BK + 8;  // row stride of transposed K / V tiles
constexpr int SS = D + 8;   // row stride of the bf16 state copies (stored KV^T: [value col][key row])
constexpr int OS = SW + 8;  // row stride of the output staging tile

// Position of token c (0..63) inside a transposed tile row; see the header comment.
__device__ __forceinline__ int tok_pos(int c)
{
    const int u = c & 31;
    return (c & 32) + 8 * ((u & 15) >> 2) + 4 * (u >> 4) + (u & 3);
}

__device__ __forceinline__ uint32_t elem_bits(const uint4& x, int e)
{
    const uint32_t w = (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

__device__ __forceinline__ float bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ uint32_t f32_to_bits(float f)
{
    return (uint32_t)__builtin_bit_cast(u16, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

__device__ __forceinline__ bf16x8 lds8(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int MODE>
__global__ __launch_bounds__(256, 1) void k_fwd_bf16(FwdArgs a)
{
    constexpr bool OUT = MODE == kModeOut;
    __shared__ __attribute__((aligned(16))) u16 sK[2][BK * KS];
    __shared__ __attribute__((aligned(16))) u16 sKT[2][D * TS];
    __shared__ __attribute__((aligned(16))) u16 sVT[2][SW * TS];
    __shared__ __attribute__((aligned(16))) u16 sVWh[2][SW * TS];
    __shared__ __attribute__((aligned(16))) u16 sVWl[2][SW * TS];
    __shared__ __attribute__((aligned(16))) u16 sSh[2][SW * SS];
    __shared__ __attribute__((aligned(16))) u16 sSl[2][SW * SS];
    __shared__ __attribute__((aligned(16))) u16 sO[BK * OS];

    int64_t group;
    int slice;
    xcd_decode(blockIdx.x, a.slices, group, slice);
    if (group >= a.groups) return;
    const int64_t u = group / a.chunks_launched;
    const int64_t j = group % a.chunks_launched;
    const int64_t bb = u / a.heads, h = u % a.heads;
    const int64_t t_begin = j * a.chunk;
    const int64_t t_end = (t_begin + a.chunk < a.n) ? t_begin + a.chunk : a.n;
    const int64_t d2 = (int64_t)D * D;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, g = l >> 4;
    const float nsl = neg_slope_log2e(a.slopes, h);
    const int64_t base = bb * a.sb + h * a.sh;
    const u16* Qg = static_cast<const u16*>(a.q) + base;
    const u16* Kg = static_cast<const u16*>(a.k) + base;
    const u16* Vg = static_cast<const u16*>(a.v) + base + slice * SW;
    u16* Og = OUT ? static_cast<u16*>(a.o) + base + slice * SW : nullptr;
    const int64_t sn = a.sn;

    // staging roles: threads 0..127 carry an 8x8 K tile, 128..159 an 8x8 V tile
    const bool k_role = tid < 128;
    const bool v_role = tid >= 128 && tid < 160;
    const int ktg = tid >> 4, kdg = tid & 15;                 // K: token group, feature group
    const int vtg = (tid - 128) >> 2, vcg = (tid - 128) & 3;  // V: token group, column group

    uint4 qn[4];   // next tile's Q operand fragments (rows 16w+lr, features 32ks+8g..)
    uint4 tn[8];   // next tile's 8x8 K or V block (8 token rows x 16 bytes)

    auto load_tile = [&](int64_t t0, int L) {
        if (OUT) {
            const int r = 16 * w + lr;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qn[ks] = (r < L) ? *reinterpret_cast<const uint4*>(Qg + (t0 + r) * sn + 32 * ks + 8 * g)
                                 : make_uint4(0, 0, 0, 0);
        }
        if (k_role) {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int r = 8 * ktg + m;
                tn[m] = (r < L) ? *reinterpret_cast<const uint4*>(Kg + (t0 + r) * sn + 8 * kdg)
                                : make_uint4(0, 0, 0, 0);
            }
        } else if (v_role) {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int r = 8 * vtg + m;
                tn[m] = (r < L) ? *reinterpret_cast<const uint4*>(Vg + (t0 + r) * sn + 8 * vcg)
                                : make_uint4(0, 0, 0, 0);
            }
        }
    };

    auto stage_tile = [&](int buf, int L) {
        if (k_role) {
            if (OUT) {
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    *reinterpret_cast<uint4*>(&sK[buf][(8 * ktg + m) * KS + 8 * kdg]) = tn[m];
            }
            const int p0 = tok_pos(8 * ktg), p1 = tok_pos(8 * ktg + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t x[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) x[m] = elem_bits(tn[m], e);
                u16* row = &sKT[buf][(8 * kdg + e) * TS];
                *reinterpret_cast<uint2*>(row + p0) = make_uint2(pack2(x[0], x[1]), pack2(x[2], x[3]));
                *reinterpret_cast<uint2*>(row + p1) = make_uint2(pack2(x[4], x[5]), pack2(x[6], x[7]));
            }
        } else if (v_role) {
            float wt[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int c = 8 * vtg + m;
                wt[m] = (c < L) ? decay_pow(nsl, (float)(L - 1 - c)) : 0.f;
            }
            const int p0 = tok_pos(8 * vtg), p1 = tok_pos(8 * vtg + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t x[8], hi[8], lo[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    x[m] = elem_bits(tn[m], e);
                    const float y = bits_to_f32(x[m]) * wt[m];
                    hi[m] = f32_to_bits(y);
                    lo[m] = f32_to_bits(y - bits_to_f32(hi[m]));
                }
                const int ro = (8 * vcg + e) * TS;
                *reinterpret_cast<uint2*>(&sVT[buf][ro + p0]) = make_uint2(pack2(x[0], x[1]), pack2(x[2], x[3]));
                *reinterpret_cast<uint2*>(&sVT[buf][ro + p1]) = make_uint2(pack2(x[4], x[5]), pack2(x[6], x[7]));
                *reinterpret_cast<uint2*>(&sVWh[buf][ro + p0]) = make_uint2(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
                *reinterpret_cast<uint2*>(&sVWh[buf][ro + p1]) = make_uint2(pack2(hi[4], hi[5]), pack2(hi[6], hi[7]));
                *reinterpret_cast<uint2*>(&sVWl[buf][ro + p0]) = make_uint2(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
                *reinterpret_cast<uint2*>(&sVWl[buf][ro + p1]) = make_uint2(pack2(lo[4], lo[5]), pack2(lo[6], lo[7]));
            }
        }
    };

    // incoming state: rows i = 32w + 16it + 4g + t, value columns 16jt + lr of this slice
    f32x4 st[2][2];
    {
        const float* src = nullptr;
        if (MODE != kModeLocal) src = (a.n_chunks > 1) ? a.ws + (u * a.n_chunks + j) * d2 : a.kv + u * d2;
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    st[it][jt][t] = src ? src[(32 * w + 16 * it + 4 * g + t) * D + slice * SW + 16 * jt + lr] : 0.f;
    }
    auto write_state_copy = [&](int buf) {
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    hi[t] = f32_to_bits(st[it][jt][t]);
                    lo[t] = f32_to_bits(st[it][jt][t] - bits_to_f32(hi[t]));
                }
                const int off = (16 * jt + lr) * SS + 32 * w + 16 * it + 4 * g;
                *reinterpret_cast<uint2*>(&sSh[buf][off]) = make_uint2(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
                *reinterpret_cast<uint2*>(&sSl[buf][off]) = make_uint2(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
            }
    };
    auto store_state = [&](float* dst) {
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    dst[(32 * w + 16 * it + 4 * g + t) * D + slice * SW + 16 * jt + lr] = st[it][jt][t];
    };

    {
        const int L0 = (int)((t_end - t_begin < BK) ? t_end - t_begin : BK);
        load_tile(t_begin, L0);
        stage_tile(0, L0);
        if (OUT) write_state_copy(0);
        __syncthreads();
    }

    int cur = 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += BK, cur ^= 1) {
        const int L = (int)((t_end - t0 < BK) ? t_end - t0 : BK);
        const bool has_next = t0 + BK < t_end;
        const int Ln = has_next ? (int)((t_end - t0 - BK < BK) ? t_end - t0 - BK : BK) : 0;
        bf16x8 qf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, qn[ks]);
        if (has_next) load_tile(t0 + BK, Ln);

        if (OUT) {
            // inter-tile term: Q KV, rows scaled by lambda^(r+1)
            f32x4 acc[2];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int off = (16 * jt + lr) * SS + 32 * ks + 8 * g;
                    acc[jt] = mfma(qf[ks], lds8(&sSh[cur][off]), acc[jt]);
                    acc[jt] = mfma(qf[ks], lds8(&sSl[cur][off]), acc[jt]);
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float rs = decay_pow(nsl, (float)(16 * w + 4 * g + t + 1));
                acc[0][t] *= rs;
                acc[1][t] *= rs;
            }
            // intra-tile scores S^T for key tiles 0..w (later key tiles are fully masked)
            const int r = 16 * w + lr;
            float p[4][4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                if (ct <= w) {
                    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        s = mfma(lds8(&sK[cur][(16 * ct + lr) * KS + 32 * ks + 8 * g]), qf[ks], s);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int c = 16 * ct + 4 * g + t;
                        p[ct][t] = (c <= r) ? s[t] * decay_pow(nsl, (float)(r - c)) : 0.f;
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) p[ct][t] = 0.f;
                }
            }
            // intra-tile output P V
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                if (2 * k2 <= w) {
                    bf16x8 ph, pl;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        ph[t] = (__bf16)p[2 * k2][t];
                        ph[4 + t] = (__bf16)p[2 * k2 + 1][t];
                        pl[t] = (__bf16)(p[2 * k2][t] - (float)ph[t]);
                        pl[4 + t] = (__bf16)(p[2 * k2 + 1][t] - (float)ph[4 + t]);
                    }
#pragma unroll
                    for (int jt = 0; jt < 2; ++jt) {
                        const bf16x8 vb = lds8(&sVT[cur][(16 * jt + lr) * TS + 32 * k2 + 8 * g]);
                        acc[jt] = mfma(ph, vb, acc[jt]);
                        acc[jt] = mfma(pl, vb, acc[jt]);
                    }
                }
            }
            // output tile: stage this wave's 16 rows, then 16-byte stores
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    sO[(16 * w + 4 * g + t) * OS + 16 * jt + lr] = (u16)f32_to_bits(acc[jt][t]);
            wave_lds_sync();
            {
                const int rr = 16 * w + (l >> 2), cc = 8 * (l & 3);
                const uint4 x = *reinterpret_cast<const uint4*>(&sO[rr * OS + cc]);
                if (rr < L) *reinterpret_cast<uint4*>(Og + (t0 + rr) * sn + cc) = x;
            }
        }

        // state update: KV <- lambda^L KV + K^T (W V) for this wave's 32 key rows
        {
            const float dl = decay_pow(nsl, (float)L);
#pragma unroll
            for (int it = 0; it < 2; ++it)
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) st[it][jt] *= dl;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 vh[2], vl[2];
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    vh[jt] = lds8(&sVWh[cur][(16 * jt + lr) * TS + 32 * ks + 8 * g]);
                    vl[jt] = lds8(&sVWl[cur][(16 * jt + lr) * TS + 32 * ks + 8 * g]);
                }
#pragma unroll
                for (int it = 0; it < 2; ++it) {
                    const bf16x8 ka = lds8(&sKT[cur][(32 * w + 16 * it + lr) * TS + 32 * ks + 8 * g]);
#pragma unroll
                    for (int jt = 0; jt < 2; ++jt) {
                        st[it][jt] = mfma(ka, vh[jt], st[it][jt]);
                        st[it][jt] = mfma(ka, vl[jt], st[it][jt]);
                    }
                }
            }
        }
        if (OUT && has_next) write_state_copy(cur ^ 1);
        if (MODE != kModeLocal && a.ckpt) {
            const int64_t end = t0 + L;
            if (end % a.ckpt_every == 0) store_state(a.ckpt + (u * a.n_ckpt + (end / a.ckpt_every - 1)) * d2);
        }
        if (has_next) stage_tile(cur ^ 1, Ln);
        __syncthreads();
    }

    if (MODE == kModeLocal) store_state(a.ws + (u * a.n_chunks + j + 1) * d2);
    else if (j == a.n_chunks - 1) store_state(a.kv + u * d2);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int mode, hipStream_t stream)
{
    const dim3 grid((unsigned)xcd_grid_size(a.groups, a.slices)), block(256);
    if (mode == kModeOut) hipLaunchKernelGGL(k_fwd_bf16<kModeOut>, grid, block, 0, stream, a);
    else if (mode == kModeState) hipLaunchKernelGGL(k_fwd_bf16<kModeState>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(k_fwd_bf16<kModeLocal>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace la
