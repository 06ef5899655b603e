// Single-token decode step on gfx950: kv <- lambda*kv + k^T v, then o = q . kv.
//
// Page "MiniMax-01: Scaling Foundation Models with Lightning Attention |
// Summary", section 3.3: single-token generation runs as its own kernel and
// is limited by memory traffic.  Per (batch, head) the step streams the
// 64 KiB float32 state once in and once out; everything else is 4*d values.
//
// One 256-thread workgroup per (batch, head).  Thread t owns four adjacent
// value columns (a float4) and every (256/(d/4))-th key row, so each wave's
// load/store covers whole contiguous state rows (1 KiB per instruction at
// d = 128).  The readout o[j] = sum_i q_i KV[i][j] is reduced across the row
// groups through LDS.
#include "la_common.h"

namespace la {
namespace {

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(__bf16 x) { return (float)x; }
template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }
// An activated input rounded to the input dtype, as the prefill kernels hold it.
template <typename T> __device__ inline float act_round(float x) { return to_f32(from_f32<T>(x)); }

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Fused prologue/epilogue of la_decode_fused (all-zero Fu: none).
struct Fu {
    uint32_t flags;
    const void* gate;
    const float* weight;
    float eps;
};

// FUSED compiles the prologue/epilogue in; the plain step carries none of it.
template <typename T, int D, bool FUSED>
__global__ __launch_bounds__(256) void k_decode(const T* __restrict__ q, const T* __restrict__ k,
                                                const T* __restrict__ v, T* __restrict__ o,
                                                const float* __restrict__ slopes,
                                                float* __restrict__ kv, int64_t heads, Fu fu)
{
    const uint32_t flags = FUSED ? fu.flags : 0u;
    constexpr int CG = D / 4;       // float4 column groups per row
    constexpr int RG = 256 / CG;    // row groups
    constexpr int RPT = D / RG;     // rows per thread
    const int64_t u = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;

    __shared__ float sq[D];
    __shared__ float sk[D];
    __shared__ f32x4 red[RG][CG];

    float* S = kv + u * (int64_t)(D * D);
    f32x4 st[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        st[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (rg + RG * m) * D) + cg);

    if (tid < D) {
        const float xq = to_f32(q[u * D + tid]), xk = to_f32(k[u * D + tid]);
        sq[tid] = (flags & LA_SILU_Q) ? act_round<T>(silu_f32(xq)) : xq;
        sk[tid] = (flags & LA_SILU_K) ? act_round<T>(silu_f32(xk)) : xk;
    }
    const T* vu = v + u * D + 4 * cg;
    f32x4 vv = {to_f32(vu[0]), to_f32(vu[1]), to_f32(vu[2]), to_f32(vu[3])};
    if (flags & LA_SILU_V)
        vv = f32x4{act_round<T>(silu_f32(vv[0])), act_round<T>(silu_f32(vv[1])), act_round<T>(silu_f32(vv[2])),
                   act_round<T>(silu_f32(vv[3]))};
    const float lam = (float)exp(-(double)slopes[u % heads]);
    __syncthreads();

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        const f32x4 s = lam * st[m] + sk[i] * vv;
        __builtin_nontemporal_store(s, reinterpret_cast<f32x4*>(S + i * D) + cg);
        acc += sq[i] * s;
    }
    red[rg][cg] = acc;
    __syncthreads();
    if (tid < CG) {
        f32x4 r = red[0][tid];
        for (int g = 1; g < RG; ++g) r += red[g][tid];
        if (flags & LA_NORM) {
            // mean square over the d features: the CG threads of this row are lanes 0..CG-1
            float ss = r[0] * r[0] + r[1] * r[1] + r[2] * r[2] + r[3] * r[3];
#pragma unroll
            for (int m = CG / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, CG);
            const float sc = rsqrtf(ss / (float)D + fu.eps);
            const f32x4 wv = fu.weight ? reinterpret_cast<const f32x4*>(fu.weight)[tid] : f32x4{1.f, 1.f, 1.f, 1.f};
            r = r * sc * wv;
        }
        if (flags & LA_GATE) {
            const T* gu = static_cast<const T*>(fu.gate) + u * D + 4 * tid;
            r = r * f32x4{sigmoid_f32(to_f32(gu[0])), sigmoid_f32(to_f32(gu[1])), sigmoid_f32(to_f32(gu[2])),
                          sigmoid_f32(to_f32(gu[3]))};
        }
        T* ou = o + u * D + 4 * tid;
        ou[0] = from_f32<T>(r[0]);
        ou[1] = from_f32<T>(r[1]);
        ou[2] = from_f32<T>(r[2]);
        ou[3] = from_f32<T>(r[3]);
    }
}

// RMS normalisation and/or sigmoid gate in place over rows of d values (one wave per row,
// rows taken in turn by the waves of the grid).  Row r = (b, h, t) at b*sb + h*sh + t*sn.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_norm_gate(T* __restrict__ o, const T* __restrict__ gate,
                                                   const float* __restrict__ weight, float eps, bool norm,
                                                   int64_t rows, int64_t heads, int64_t n,
                                                   int64_t sb, int64_t sh, int64_t sn)
{
    constexpr int PER = D / 64;  // values per lane
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t waves = ((int64_t)gridDim.x * 256) >> 6;
    float w[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) w[e] = (norm && weight) ? weight[lane * PER + e] : 1.f;
    for (int64_t r = wave; r < rows; r += waves) {
        const int64_t b = r / (heads * n), h = (r / n) % heads, t = r % n;
        const int64_t off = b * sb + h * sh + t * sn + lane * PER;
        float x[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) x[e] = to_f32(o[off + e]);
        if (norm) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < PER; ++e) ss += x[e] * x[e];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
            const float sc = rsqrtf(ss / (float)D + eps);
#pragma unroll
            for (int e = 0; e < PER; ++e) x[e] *= sc * w[e];
        }
        if (gate) {
#pragma unroll
            for (int e = 0; e < PER; ++e) x[e] *= sigmoid_f32(to_f32(gate[off + e]));
        }
#pragma unroll
        for (int e = 0; e < PER; ++e) o[off + e] = from_f32<T>(x[e]);
    }
}

// Short packed sequences, token by token (the smallest of the work sizes that section 3.3 of the
// page above uses for short inputs; longer sequences go through the 64-token tile kernels).  One
// workgroup per (short sequence, head): the state stays in registers across the sequence's
// tokens, each token updates it and reads o_t = q_t . KV_t out through an LDS reduction; the
// state is read and written once.  tab[3e..3e+2] = first packed token, token count and sequence
// index of short sequence e; q, k, v, o rows at t*sn + h*sh (o may be null: state only).
template <typename T, int D>
__global__ __launch_bounds__(256) void k_recur_short(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, T* __restrict__ o,
                                                     const float* __restrict__ slopes, float* __restrict__ kv,
                                                     int64_t heads, int64_t sn, int64_t sh,
                                                     const int64_t* __restrict__ tab, int rev)
{
    constexpr int CG = D / 4;
    constexpr int RG = 256 / CG;
    constexpr int RPT = D / RG;
    const int64_t e = blockIdx.x / heads, h = blockIdx.x % heads;
    const int64_t tok0 = tab[3 * e], n = tab[3 * e + 1], sq_idx = tab[3 * e + 2];
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;

    __shared__ float sq[D];
    __shared__ float sk[D];
    __shared__ f32x4 red[RG][CG];

    float* S = kv + (sq_idx * heads + h) * (int64_t)(D * D);
    f32x4 st[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) st[m] = reinterpret_cast<const f32x4*>(S + (rg + RG * m) * D)[cg];
    const float lam = (float)exp(-(double)slopes[h]);
    for (int64_t i = 0; i < n; ++i) {
        const int64_t row = (rev ? tok0 + n - 1 - i : tok0 + i) * sn + h * sh;
        if (tid < D) {
            sq[tid] = to_f32(q[row + tid]);
            sk[tid] = to_f32(k[row + tid]);
        }
        const T* vu = v + row + 4 * cg;
        const f32x4 vv = {to_f32(vu[0]), to_f32(vu[1]), to_f32(vu[2]), to_f32(vu[3])};
        __syncthreads();
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int r = rg + RG * m;
            st[m] = lam * st[m] + sk[r] * vv;
            acc += sq[r] * st[m];
        }
        red[rg][cg] = acc;
        __syncthreads();
        if (tid < CG && o) {
            f32x4 rr = red[0][tid];
            for (int g = 1; g < RG; ++g) rr += red[g][tid];
            T* ou = o + row + 4 * tid;
            ou[0] = from_f32<T>(rr[0]);
            ou[1] = from_f32<T>(rr[1]);
            ou[2] = from_f32<T>(rr[2]);
            ou[3] = from_f32<T>(rr[3]);
        }
        __syncthreads();  // sq, sk and red are rewritten by the next token
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) reinterpret_cast<f32x4*>(S + (rg + RG * m) * D)[cg] = st[m];
}

}  // namespace

hipError_t launch_recur_short(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                              int64_t n_short, int64_t heads, int d, int64_t sn, int64_t sh,
                              const float* slopes, float* kv, const int64_t* tab, bool rev, hipStream_t stream)
{
    const dim3 grid((unsigned)(n_short * heads)), block(256);
    if (dt == LA_BF16) {
        auto qq = static_cast<const __bf16*>(q), kk = static_cast<const __bf16*>(k),
             vv = static_cast<const __bf16*>(v);
        auto oo = static_cast<__bf16*>(o);
        if (d == 128)
            hipLaunchKernelGGL((k_recur_short<__bf16, 128>), grid, block, 0, stream, qq, kk, vv, oo, slopes, kv, heads, sn, sh, tab, rev ? 1 : 0);
        else
            hipLaunchKernelGGL((k_recur_short<__bf16, 64>), grid, block, 0, stream, qq, kk, vv, oo, slopes, kv, heads, sn, sh, tab, rev ? 1 : 0);
    } else {
        auto qq = static_cast<const float*>(q), kk = static_cast<const float*>(k),
             vv = static_cast<const float*>(v);
        auto oo = static_cast<float*>(o);
        if (d == 128)
            hipLaunchKernelGGL((k_recur_short<float, 128>), grid, block, 0, stream, qq, kk, vv, oo, slopes, kv, heads, sn, sh, tab, rev ? 1 : 0);
        else
            hipLaunchKernelGGL((k_recur_short<float, 64>), grid, block, 0, stream, qq, kk, vv, oo, slopes, kv, heads, sn, sh, tab, rev ? 1 : 0);
    }
    return hipGetLastError();
}

hipError_t launch_norm_gate(la_dtype dt, void* o, const void* gate, const float* weight, float eps, bool norm,
                            int64_t batch, int64_t heads, int64_t n, int d, int64_t sb, int64_t sh, int64_t sn,
                            hipStream_t stream)
{
    const int64_t rows = batch * heads * n;
    const int64_t blocks = (rows + 3) / 4 < 8192 ? (rows + 3) / 4 : 8192;
    const dim3 grid((unsigned)blocks), block(256);
    if (dt == LA_BF16) {
        auto oo = static_cast<__bf16*>(o);
        auto gg = static_cast<const __bf16*>(gate);
        if (d == 128) hipLaunchKernelGGL((k_norm_gate<__bf16, 128>), grid, block, 0, stream, oo, gg, weight, eps, norm, rows, heads, n, sb, sh, sn);
        else hipLaunchKernelGGL((k_norm_gate<__bf16, 64>), grid, block, 0, stream, oo, gg, weight, eps, norm, rows, heads, n, sb, sh, sn);
    } else {
        auto oo = static_cast<float*>(o);
        auto gg = static_cast<const float*>(gate);
        if (d == 128) hipLaunchKernelGGL((k_norm_gate<float, 128>), grid, block, 0, stream, oo, gg, weight, eps, norm, rows, heads, n, sb, sh, sn);
        else hipLaunchKernelGGL((k_norm_gate<float, 64>), grid, block, 0, stream, oo, gg, weight, eps, norm, rows, heads, n, sb, sh, sn);
    }
    return hipGetLastError();
}

template <typename T>
void launch_decode_t(const T* q, const T* k, const T* v, T* o, int64_t bh, int64_t heads, int d, const float* slopes,
                     float* kv, Fu fu, dim3 grid, dim3 block, hipStream_t stream)
{
    (void)bh;
    if (fu.flags && d == 128) hipLaunchKernelGGL((k_decode<T, 128, true>), grid, block, 0, stream, q, k, v, o, slopes, kv, heads, fu);
    else if (fu.flags) hipLaunchKernelGGL((k_decode<T, 64, true>), grid, block, 0, stream, q, k, v, o, slopes, kv, heads, fu);
    else if (d == 128) hipLaunchKernelGGL((k_decode<T, 128, false>), grid, block, 0, stream, q, k, v, o, slopes, kv, heads, fu);
    else hipLaunchKernelGGL((k_decode<T, 64, false>), grid, block, 0, stream, q, k, v, o, slopes, kv, heads, fu);
}

hipError_t launch_decode(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                         int64_t bh, int64_t heads, int d, const float* slopes, float* kv,
                         const la_fusion* fusion, hipStream_t stream)
{
    const dim3 grid((unsigned)bh), block(256);
    Fu fu{0u, nullptr, nullptr, 0.f};
    if (fusion) fu = Fu{fusion->flags, fusion->gate, fusion->norm_weight, fusion->norm_eps};
    if (dt == LA_BF16)
        launch_decode_t<__bf16>(static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                                static_cast<const __bf16*>(v), static_cast<__bf16*>(o), bh, heads, d, slopes, kv, fu,
                                grid, block, stream);
    else
        launch_decode_t<float>(static_cast<const float*>(q), static_cast<const float*>(k),
                               static_cast<const float*>(v), static_cast<float*>(o), bh, heads, d, slopes, kv, fu,
                               grid, block, stream);
    return hipGetLastError();
}

}  // namespace la
