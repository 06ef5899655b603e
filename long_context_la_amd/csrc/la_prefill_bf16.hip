// bfloat16 prefill on gfx950 matrix cores (d = 128 and d = 64).
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
// Inputs are bfloat16; every product accumulates in float32 and the state itself
// stays float32 in accumulators.  The operands that are not inputs -- P, W V and
// the operand copy of the state -- need more than bf16's 8 mantissa bits:
// rounded to one bf16 they cost about 2e-2 of the output RMS on fast-decaying
// heads (P), 1.6e-2 of the state RMS (W V) and up to 2.5e-2 of the output RMS
// after a large incoming state (KV).  With outputs, every product therefore runs
// on float16 operands (v_mfma_f32_16x16x32_f16): 11 mantissa bits keep each of
// those roundings near 2.4e-4 relative, with one MFMA per product, and the bf16
// inputs convert to float16 exactly.  Float16's range is met by scaling: P, W V
// and the state (held scaled in its accumulators) carry a factor 2^-8 that the
// output and the stored states take back.  Inputs must stay below 65504 in
// magnitude, scores and state elements below 65504 * 2^8 (bf16 activations of
// a working model are far below both).  Gradients are not: the backward's
// passes, whose inputs include dL/dO, run a full-range instantiation (WIDE)
// with bf16 inputs as they are and P, W V and the state copy as bf16 hi + lo
// pairs (x = hi + lo, two MFMAs per product), which covers float32's range.
// Without outputs (state-only and chunk-summary modes) the state update keeps
// bfloat16 operands, with W V as a hi + lo pair.
//
// Decomposition.  A workgroup owns one (batch, head, chunk, slice of 32 or 64
// value columns): both the state's columns and the outputs' columns split by
// value column with no communication, which gives 4 (or 2) workgroups per head
// without a second pass over K and V.  Q and K rows are read by every slice of
// a head; their workgroups sit on one XCD so the re-reads hit L2.  Sequences
// with too few heads to fill the GPU are also cut into chunks (la_scan.hip
// combines the chunk summaries).  The 64-column instantiation (float16
// outputs at d = 128) does the score products and the Q and K conversions
// once for twice the columns: a tile takes about 1.55x as long, so a head
// costs ~23% less GPU time.  The host uses it where the work is split
// anyway (chunked sequences, or more (batch, head) pairs than one round of
// 32-column workgroups holds); 64 heads of one sequence keep 32 columns,
// which fill the GPU without the summary pass that two chunks would need.
//
// Wave roles (8 waves, two per SIMD, so one wave's latencies hide behind the
// other's work).  Output waves 0..3: wave w owns query rows 16w..16w+15 of
// each 64-token tile -- scores, masking, P V, the inter-tile term and the
// output store.  Q is the B operand of S^T and of the transposed inter
// product.  With float16 products each output wave loads its own 16 rows of Q
// as 8 rows x 128 bytes per instruction (a load straight into operand layout
// touches 16 rows and 16 cache lines per instruction; whole 256-byte rows
// raised the L2 misses of the sibling slices' re-reads), converts them and
// stages them in its own part of an LDS tile, from which it reads the operand.
// WIDE operands load Q straight into operand layout (the staging's LDS traffic
// made the backward's passes 7% slower).  The outputs
// are accumulated transposed, O^T = KV^T Q^T + V^T P^T, so a lane holds four
// consecutive value columns of one row and stages them with one 8-byte LDS
// write before the 16-byte global stores.  State waves 4..7: the global
// loads and LDS staging of K and V, the decay-weighted W V, and the state
// update, with the state's 16 tiles of 16x16 split 6/5/3/2 (32 tiles split
// 12/10/6/4 with 64 columns: more state work on the SIMDs whose output waves
// own the earlier, lighter query rows, so that each SIMD issues about the same
// number of MFMAs).  The state waves publish
// the state after tile b (a float16 copy in LDS, or a bf16 hi + lo pair) for
// the output waves' inter term of tile b+1.  Without outputs (state-only
// modes) the kernel runs the four state waves alone.
//
// MFMA: v_mfma_f32_16x16x32_f16 / _bf16 (A 16x32, B 32x16, C 16x16 fp32; lane l holds
// A row l%16 / B column l%16 and 8 k-values of group g = l/16; C column l%16,
// rows 4g..4g+3).  The sum over k does not care which k a slot holds as long
// as A and B agree, which is used twice:
//   * S is computed transposed (S^T = K Q^T), so a lane's accumulators hold
//     one query row r and keys {4g..4g+3} and {16+4g..16+4g+3} of two
//     adjacent 16-key tiles -- the B operand of V^T P^T over a 32-key step in
//     that k order, with no data movement;
//   * the k = token operands (V for P.V; K^T and W V for the state update) are
//     read from row-major LDS tiles with the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16): within each 16-lane group, the lane that supplies
//     the address of row k0 + a/4, columns c0 + 4(a%4)..+3 makes lane i
//     receive rows k0..k0+3 of column c0 + i, i.e. four consecutive k of one
//     MFMA row/column.  Two such reads fill an 8-value operand, so tiles are
//     staged as plain row copies and any k order is available.
// Global traffic uses buffer loads/stores on a per-tile resource whose size
// ends at the tile's last valid row, so the rows of a ragged last tile read as
// zero without branches.  Loads run two tiles ahead (two register sets) and are
// issued every step, also past the end of the chunk (zero-size resource), so the
// compiler's waits cover exactly the loads a step consumes; tiles are double-
// buffered in LDS, one barrier per tile.  Per-element decay factors come from
// per-lane tables computed once per workgroup.
#include "la_common.h"

namespace la {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BK = kBlock, SW = kSliceW;
// Row stride (elements) of the row-major K tile of head dimension D: 288 B at d = 128 and 160 B at
// d = 64, so the 4 rows of a transposing read fall in disjoint banks.
template <int D> constexpr int kKS = D + 16;
constexpr int VS = SW + 16;  // row stride of the V, W V tiles: 96 B (same reason)
constexpr int OS = SW + 16;  // row stride of the output staging tile: 96 B, so that 16 rows x 32 B of
                             // 8-byte writes and 16 rows x 64 B of 16-byte reads spread evenly over
                             // the banks
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9-family raw buffer descriptor word 3

__device__ __forceinline__ float bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ bf16x8 lds8(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Element offset of (row, col) in a state copy (stored KV^T: [value col][key row]): unpadded rows of
// D elements whose 16-byte chunks are permuted by the row index (modulo the D/8 chunks of a row), so
// that 16 lanes reading one chunk position of 16 rows (operand reads) or writing 8-byte halves of
// 16 rows (state publication) spread over the bank space.
template <int D>
__device__ __forceinline__ int ss_off(int row, int col)
{
    return row * D + ((((col >> 3) ^ row) & (D / 8 - 1)) << 3) + (col & 7);
}

// Two floats -> packed bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t cvt2(float a, float b)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
// (a, b) -> bf16 pairs hi and lo with x = hi + lo to about 16 bits.  The low half of hi goes back
// to float32 through a byte permute (bytes 1, 0 of hi on top of two zero bytes): written as a
// shift, the compiler recognises a bf16 round trip of a and converts a a second time.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo)
{
    hi = cvt2(a, b);
    const float ha = __uint_as_float(__builtin_amdgcn_perm(hi, hi, 0x01000c0cu));
    lo = cvt2(a - ha, b - hi_to_f32(hi));
}

// SiLU of 8 packed bf16 values (float32 arithmetic, rounded back to bf16).
__device__ __forceinline__ uint4 silu8(uint4 x)
{
    const uint32_t in[4] = {x.x, x.y, x.z, x.w};
    uint32_t out[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = cvt2(silu_f32(bits_to_f32(in[e] & 0xffffu)), silu_f32(hi_to_f32(in[e])));
    return make_uint4(out[0], out[1], out[2], out[3]);
}
// acc[e] * sigmoid(g_e) for 4 float32 outputs and their 4 packed bf16 gate values.
__device__ __forceinline__ void gate4(f32x4& acc, uint2 g)
{
    acc[0] *= sigmoid_f32(bits_to_f32(g.x & 0xffffu));
    acc[1] *= sigmoid_f32(hi_to_f32(g.x));
    acc[2] *= sigmoid_f32(bits_to_f32(g.y & 0xffffu));
    acc[3] *= sigmoid_f32(hi_to_f32(g.y));
}

// Transposing LDS read (see the header comment): returns rows k0..k0+3 of column c0 + (lane % 16)
// when this lane passes the address of row k0 + (lane%16)/4, column c0 + 4*(lane%4).
__device__ __forceinline__ s16x4 lds_tr(const u16* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) char*)p));
}

__device__ __forceinline__ bf16x8 join(s16x4 a, s16x4 b)
{
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Float16 operands: 8 values per lane, the same lane layout as the bf16 products.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x4 mfma_h(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                   0);
}
// Two floats -> packed float16 pair (round to nearest even).
__device__ __forceinline__ uint32_t cvt2h(float a, float b)
{
    const f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}
// 8 packed bf16 values -> 8 packed float16 values (exact for |x| < 65504; the bit patterns are
// returned in a bf16x8 so they travel through the same registers and LDS tiles).
__device__ __forceinline__ uint4 bf16x8_to_f16(uint4 x)
{
    const uint32_t in[4] = {x.x, x.y, x.z, x.w};
    uint32_t out[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = cvt2h(__uint_as_float(in[e] << 16), __uint_as_float(in[e] & 0xffff0000u));
    return make_uint4(out[0], out[1], out[2], out[3]);
}
// Scale of the float16 operands that are not inputs (P, W V, the state).
constexpr float kHalfScale = 0.00390625f;  // 2^-8

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Raw buffer covering `bytes` bytes from p (reads past the end return 0, writes there are dropped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, (int)kRsrcWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

template <int N> struct IntC { static constexpr int value = N; };

// The four value slices of a head read the same Q and K rows at nearly the same time; each slice
// walks its blocks of Q (8 rows x 128 bytes when staged, 64-byte column blocks in operand layout)
// and of K (16-row blocks) starting at its own index, so that the simultaneous requests of sibling
// slices fall on different cache lines.
// Q as loaded: 16 bytes per piece of one of the wave's 16 rows (see load_q)
template <int D> struct QRegs { uint4 q[D / 32]; };
// K chunks st_id + 256m of the 64 x D tile; V slice row st_id/4
template <int D, int NV> struct KVRegs { uint4 k[D / 32]; uint4 v[NV]; };

// REV walks each sequence from its last token to its first (token index t of the recurrence is
// memory row n-1-t), the order of the reverse state recurrence of the backward pass.  ACT enables
// the SiLU prologue (which of q, k, v is chosen at run time); without it no activation code is
// compiled in, since untaken branches inside the tile loops still cost about 10% here.
template <int MODE, bool GATE, bool REV, bool ACT, int D, bool WIDE, int SWT>
__global__ __launch_bounds__(MODE == kModeOut ? 512 : 256, 1) void k_fwd_bf16(FwdArgs a)
{
    static_assert(SWT == 32 || (SWT == 64 && D == 128 && MODE == kModeOut && !WIDE),
                  "64-column slices only for float16 outputs at d = 128");
    // value columns of this workgroup's slice, and the row strides that depend on it: V and W V
    // rows of 96 B (32 columns) or 160 B (64 columns), so the 4 rows of a transposing read fall in
    // disjoint banks; output staging rows likewise
    constexpr int SW = SWT, VS = SWT + 16, OS = SWT + 16;
    constexpr int NJ = SW / 16;         // 16-column tiles of the slice
    constexpr int PPR = SW / 8;         // 16-byte pieces of a slice row
    constexpr int NV = SW / 32;         // V pieces per state lane (64 rows x PPR pieces over 256 lanes)
    static_assert(!(GATE && REV), "the reverse walk has no epilogue");
    static_assert(D == 64 || D == 128, "head dimension 64 or 128");
    static_assert(!WIDE || MODE == kModeOut, "full-range operands matter only with outputs");
    constexpr bool OUT = MODE == kModeOut;
    // float16 products with outputs; bf16 (P, W V and the state copy as hi + lo pairs) with WIDE
    // outputs and in the state-only and summary modes
    constexpr bool F16 = OUT && !WIDE;
    constexpr float kPSc = F16 ? kHalfScale : 1.f;  // scale of P
    constexpr float kSc = F16 ? kHalfScale : 1.f, kScInv = F16 ? 1.f / kHalfScale : 1.f;
    constexpr int KS = kKS<D>;
    constexpr int NQ = D / 32;   // 32-feature steps of a score or inter product; also Q, K loads per lane
    constexpr int CPR = D / 8, CPR_LOG = D == 128 ? 4 : 3;  // 16-byte chunks per row of Q or K
    using QR = QRegs<D>;
    using KR = KVRegs<D, NV>;
    constexpr int SW0 = OUT ? 4 : 0;  // first state wave
    __shared__ __attribute__((aligned(16))) u16 sK[2][BK * KS];
    __shared__ __attribute__((aligned(16))) u16 sV[2][BK * VS];
    __shared__ __attribute__((aligned(16))) u16 sVWh[2][BK * VS];
    __shared__ __attribute__((aligned(16))) u16 sVWl[F16 ? 1 : 2][F16 ? 8 : BK * VS];
    __shared__ __attribute__((aligned(16))) u16 sS[2][SW * D];
    __shared__ __attribute__((aligned(16))) u16 sSl[OUT && !F16 ? 2 : 1][OUT && !F16 ? SW * D : 8];
    __shared__ __attribute__((aligned(16))) u16 sO[BK * OS];
    constexpr bool QLDS = F16;  // Q staged in LDS (see the header comment)
    __shared__ __attribute__((aligned(16))) u16 sQ[QLDS ? 2 : 1][QLDS ? BK * KS : 8];  // Q tile, K's row stride

    int64_t group;
    int slice;
    xcd_decode(blockIdx.x, a.slices, group, slice);
    if (group >= a.groups) return;
    const Work wk = decode_work(a, group);
    if (MODE == kModeLocal && wk.j == wk.nck - 1) return;  // last chunks need no summary
    const int64_t u = wk.u, j = wk.j, h = wk.h;
    const int64_t t_begin = wk.t_begin, t_end = wk.t_end;
    const int64_t d2 = (int64_t)D * D;
    const int n_tiles = (int)((t_end - t_begin + BK - 1) / BK);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_state = w >= SW0;
    const int l = tid & 63, lr = l & 15, g = l >> 4;
    const float nsl = neg_slope_log2e(a.slopes, h);
    const int64_t base = wk.base;
    const u16* Qg = static_cast<const u16*>(a.q) + base;
    const u16* Kg = static_cast<const u16*>(a.k) + base;
    const u16* Vg = static_cast<const u16*>(a.v) + base + slice * SW;
    u16* Og = OUT ? static_cast<u16*>(a.o) + base + slice * SW : nullptr;
    const u16* Gg = GATE ? static_cast<const u16*>(a.gate) + base + slice * SW : nullptr;
    const bool silu_q = ACT && (a.act & LA_SILU_Q), silu_k = ACT && (a.act & LA_SILU_K),
               silu_v = ACT && (a.act & LA_SILU_V);
    const int64_t sn = a.sn;
    const uint32_t row_bytes = (uint32_t)(sn * 2);
    // transposing-read address pieces: row k0 + lr/4, column c0 + 4*(lr%4)
    const int tr_row = lr >> 2, tr_col = 4 * (lr & 3);

    auto tile_start = [&](int tile) __attribute__((always_inline)) { return t_begin + (int64_t)tile * BK; };
    auto tile_len = [&](int tile) __attribute__((always_inline)) {
        const int64_t t0 = t_begin + (int64_t)tile * BK;
        return (int)((t_end - t0 < BK) ? t_end - t0 : BK);
    };
    // Bytes of a tile's rows that lie inside the chunk: 0 for tiles past its end, whose loads
    // then return zeros without touching memory.  Prefetches are therefore issued every step,
    // unconditionally, which lets the compiler wait for exactly the loads a step consumes rather
    // than for every outstanding load and store.
    auto tile_bytes = [&](int tile) __attribute__((always_inline)) {
        const int L = tile_len(tile);
        return (int64_t)(L > 0 ? L : 0) * row_bytes;
    };
    // Memory row of a tile's first byte, and the byte offset of its row r.  In the reverse walk
    // the tile's L rows lie backwards from memory row n - t0 - 1, so row r sits at L-1-r from
    // memory row n - t0 - L; rows r >= L wrap to offsets far above the tile's byte count, which
    // the buffer range check turns into zero loads and dropped stores, as for forward rows >= L.
    auto tile_row0 = [&](int tile) __attribute__((always_inline)) {
        const int64_t t0 = tile_start(tile);
        if constexpr (!REV) return t0;
        const int L = tile_len(tile);
        const int64_t r0 = wk.rev_end - t0 - (L > 0 ? L : 0);
        return r0 > 0 ? r0 : (int64_t)0;
    };
    auto row_off = [&](int tile, int r) __attribute__((always_inline)) {
        if constexpr (!REV) return (uint32_t)r * row_bytes;
        return (uint32_t)(tile_len(tile) - 1 - r) * row_bytes;
    };

    // ------------------------------------------------------------------ state waves
    const int st_id = tid - SW0 * 64;  // 0..255 within the state waves
    // State tiles q = NJ*it + jt (it: key rows 16it.., jt: value columns 16jt..), D*SW/256 of them, of
    // state wave sw: [first, first + count).  With outputs the split moves state work off the SIMDs
    // whose output waves own the later query rows (more score blocks): at d = 128, 6/5/3/2 of 16 (which
    // evens out the MFMA counts per SIMD; measured against 8/5/2/1, 7/6/2/1, 8/4/3/1, 5/5/3/3,
    // 6/4/3/3 and 7/5/2/2), 12/10/6/4 of 32 with 64 columns (48 MFMAs per SIMD and tile on each),
    // 3/3/1/1 of 8 at d = 64; equal shares without outputs.
    auto st_first = [](int sw) constexpr {
        if (!OUT) return (D * SW / 1024) * sw;
        if (D == 64) return sw == 0 ? 0 : sw == 1 ? 3 : sw == 2 ? 6 : 7;
        if (SW == 64) return sw == 0 ? 0 : sw == 1 ? 12 : sw == 2 ? 22 : 28;
        return sw == 0 ? 0 : sw == 1 ? 6 : sw == 2 ? 11 : 14;
    };
    auto st_count = [](int sw) constexpr {
        if (!OUT) return D * SW / 1024;
        if (D == 64) return sw <= 1 ? 3 : 1;
        if (SW == 64) return sw == 0 ? 12 : sw == 1 ? 10 : sw == 2 ? 6 : 4;
        return sw == 0 ? 6 : sw == 1 ? 5 : sw == 2 ? 3 : 2;
    };

    auto load_kv = [&](KR& R, int tile) __attribute__((always_inline)) {
        const int64_t t0 = tile_row0(tile);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + t0 * sn, tile_bytes(tile));
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + t0 * sn, tile_bytes(tile));
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int c = st_id + 256 * ((m + slice) & (NQ - 1));
            R.k[m] = buf_load16(rk, row_off(tile, c >> CPR_LOG) + 16u * (c & (CPR - 1)));
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
            const int c = st_id + 256 * m;
            R.v[m] = buf_load16(rv, row_off(tile, c / PPR) + 16u * (c % PPR));
        }
    };
    // Decay weights, computed once: lambda^(L-1-r) for the V row r this lane stages (0 past the
    // tile's end) and lambda^L for the state, for a full tile and for the last tile, the only one
    // that can be shorter.
    const int L_last = tile_len(n_tiles - 1);
    float wt_full[NV], wt_last[NV];
#pragma unroll
    for (int m = 0; m < NV; ++m) {
        const int r = (st_id + 256 * m) / PPR;
        wt_full[m] = decay_pow(nsl, (float)(BK - 1 - r)) * kSc;
        wt_last[m] = (r < L_last) ? decay_pow(nsl, (float)(L_last - 1 - r)) * kSc : 0.f;
    }
    const float dl_full = decay_pow(nsl, (float)BK);
    const float dl_last = decay_pow(nsl, (float)L_last);
    // K and V rows into LDS buffer `buf` with the decay-weighted V: float16 (and W V scaled by 2^-8)
    // with float16 outputs, else bf16 with W V as a hi + lo pair (WIDE outputs, state-only and
    // summary modes).
    auto stage_tile = [&](const KR& R, int buf, int tile) __attribute__((always_inline)) {
        const int L = tile_len(tile);
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            const int c = st_id + 256 * ((m + slice) & (NQ - 1));
            const uint4 kx = silu_k ? silu8(R.k[m]) : R.k[m];
            *reinterpret_cast<uint4*>(&sK[buf][(c >> CPR_LOG) * KS + 8 * (c & (CPR - 1))]) = F16 ? bf16x8_to_f16(kx) : kx;
        }
#pragma unroll
        for (int m = 0; m < NV; ++m) {
        const int c = st_id + 256 * m;
        const int off = (c / PPR) * VS + 8 * (c % PPR);
        const uint4 vx = silu_v ? silu8(R.v[m]) : R.v[m];
        const float wt = (L == BK) ? wt_full[m] : wt_last[m];
        const uint32_t in[4] = {vx.x, vx.y, vx.z, vx.w};
        if constexpr (F16) {
            uint32_t hv[4], hw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = bits_to_f32(in[e] & 0xffffu), b = hi_to_f32(in[e]);
                hv[e] = cvt2h(a, b);
                hw[e] = cvt2h(a * wt, b * wt);
            }
            *reinterpret_cast<uint4*>(&sV[buf][off]) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
            *reinterpret_cast<uint4*>(&sVWh[buf][off]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        } else {
            *reinterpret_cast<uint4*>(&sV[buf][off]) = vx;
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) split2(bits_to_f32(in[e] & 0xffffu) * wt, hi_to_f32(in[e]) * wt, hi[e], lo[e]);
            *reinterpret_cast<uint4*>(&sVWh[buf][off]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint4*>(&sVWl[buf][off]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
        }
    };
    // state copy for the inter term, KV^T[value col][key row], 4 consecutive key rows per lane:
    // float16 (the accumulators hold the state scaled by 2^-8), or a bf16 hi + lo pair when WIDE
    auto write_state_copy = [&](auto swc, const f32x4* st, int buf) __attribute__((always_inline)) {
        constexpr int F = st_first(decltype(swc)::value), C = st_count(decltype(swc)::value);
#pragma unroll
        for (int k = 0; k < C; ++k) {
            const int q = F + k;
            const int off = ss_off<D>(16 * (q % NJ) + lr, 16 * (q / NJ) + 4 * g);
            if constexpr (F16) {
                *reinterpret_cast<uint2*>(&sS[buf][off]) = make_uint2(cvt2h(st[k][0], st[k][1]), cvt2h(st[k][2], st[k][3]));
            } else {
                uint32_t h01, l01, h23, l23;
                split2(st[k][0], st[k][1], h01, l01);
                split2(st[k][2], st[k][3], h23, l23);
                *reinterpret_cast<uint2*>(&sS[buf][off]) = make_uint2(h01, h23);
                *reinterpret_cast<uint2*>(&sSl[buf][off]) = make_uint2(l01, l23);
            }
        }
    };
    auto store_state = [&](auto swc, const f32x4* st, float* dst) __attribute__((always_inline)) {
        constexpr int F = st_first(decltype(swc)::value), C = st_count(decltype(swc)::value);
#pragma unroll
        for (int k = 0; k < C; ++k) {
            const int q = F + k;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                dst[(16 * (q / NJ) + 4 * g + t) * D + slice * SW + 16 * (q % NJ) + lr] = st[k][t] * kScInv;
        }
    };
    auto load_state = [&](auto swc, f32x4* st, const float* src) __attribute__((always_inline)) {
        constexpr int F = st_first(decltype(swc)::value), C = st_count(decltype(swc)::value);
#pragma unroll
        for (int k = 0; k < C; ++k) {
            const int q = F + k;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                st[k][t] = src ? src[(16 * (q / NJ) + 4 * g + t) * D + slice * SW + 16 * (q % NJ) + lr] * kSc : 0.f;
        }
    };
    // KV <- lambda^L KV + K^T (W V) on this wave's state tiles
    auto update_state = [&](auto swc, f32x4* st, int buf, int tile) __attribute__((always_inline)) {
        constexpr int F = st_first(decltype(swc)::value), C = st_count(decltype(swc)::value);
        const float dl = (tile_len(tile) == BK) ? dl_full : dl_last;
#pragma unroll
        for (int k = 0; k < C; ++k) st[k] *= dl;
        // key-row tiles it0..it1 cover this wave's state tiles; the two value-column tiles of one
        // key-row tile share its K^T operand
        constexpr int IT0 = F / NJ, NIT = (F + C - 1) / NJ - IT0 + 1;
        bf16x8 vh[2][NJ], vl[2][NJ], ka[2][NIT];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int k0 = 32 * ks + 8 * g;
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
                const int o = (k0 + tr_row) * VS + 16 * jt + tr_col;
                vh[ks][jt] = join(lds_tr(&sVWh[buf][o]), lds_tr(&sVWh[buf][o + 4 * VS]));
                if constexpr (!F16) vl[ks][jt] = join(lds_tr(&sVWl[buf][o]), lds_tr(&sVWl[buf][o + 4 * VS]));
            }
#pragma unroll
            for (int n = 0; n < NIT; ++n) {
                const int o = (k0 + tr_row) * KS + 16 * (IT0 + n) + tr_col;
                ka[ks][n] = join(lds_tr(&sK[buf][o]), lds_tr(&sK[buf][o + 4 * KS]));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int k = 0; k < C; ++k) {
                const int q = F + k;
                if constexpr (F16) {
                    st[k] = mfma_h(ka[ks][q / NJ - IT0], vh[ks][q % NJ], st[k]);
                } else {
                    st[k] = mfma(ka[ks][q / NJ - IT0], vh[ks][q % NJ], st[k]);
                    st[k] = mfma(ka[ks][q / NJ - IT0], vl[ks][q % NJ], st[k]);
                }
            }
    };

    // ------------------------------------------------------------------ output waves
    // dmask[ct][t] = 2^-8 lambda^(r - c) (lambda^(r - c) when WIDE) for query r = 16w + lr and key
    // c = 16ct + 4g + t (0 if c > r); drow = lambda^(r+1) for this lane's output row r = 16w + lr.
    // With float16 operands P and the state copy both carry the factor 2^-8, which the output takes
    // back once before it is stored.
    float dmask[4][4], drow = 0.f;
    if (OUT && !is_state) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int e = 16 * (w - ct) + lr - 4 * g - t;
                dmask[ct][t] = (e >= 0) ? decay_pow(nsl, (float)e) * kPSc : 0.f;
            }
        drow = decay_pow(nsl, (float)(16 * w + lr + 1));
    }
    // Q of this wave.  Staged (QLDS): load i covers 8 rows x 128 bytes, 8 lanes of 16 bytes per row:
    // row half (b & 1) of the wave's 16 rows, byte half (b >> 1) of each row (d = 128).  In operand
    // layout: piece i is row 16w + lr, features 32b + 8g .. +7.  Either way b is i rotated by the
    // slice, so that sibling slices start on different blocks.
    auto q_row = [&](int i) __attribute__((always_inline)) {
        if constexpr (!QLDS) return 16 * w + lr;
        return 16 * w + 8 * (((i + slice) & (NQ - 1)) & 1) + (l >> 3);
    };
    auto q_piece = [&](int i) __attribute__((always_inline)) {  // 16-byte piece within the row
        if constexpr (!QLDS) return 4 * ((i + slice) & (NQ - 1)) + g;
        return 8 * (((i + slice) & (NQ - 1)) >> 1) + (l & 7);
    };
    auto load_q = [&](QR& R, int tile) __attribute__((always_inline)) {
        const int64_t t0 = tile_row0(tile);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qg + t0 * sn, tile_bytes(tile));
#pragma unroll
        for (int i = 0; i < NQ; ++i) R.q[i] = buf_load16(rq, row_off(tile, q_row(i)) + 16u * q_piece(i));
    };
    // loaded rows -> LDS buffer `buf` (float16 with float16 products, else bf16), SiLU first if asked
    auto stage_q = [&](const QR& R, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const uint4 qx = silu_q ? silu8(R.q[i]) : R.q[i];
            *reinterpret_cast<uint4*>(&sQ[buf][q_row(i) * KS + 8 * q_piece(i)]) = F16 ? bf16x8_to_f16(qx) : qx;
        }
    };
    // Outputs of tile `tile` from LDS buffers `buf`.  Staged Q: R holds the loaded rows of tile + 1,
    // which are staged into the other Q buffer once the products are issued.  Otherwise R holds the
    // operands of this tile.  Either way R then loads tile + 2.
    auto compute_out = [&](auto wc, QR& R, int buf, int tile) __attribute__((always_inline)) {
        constexpr int W = decltype(wc)::value;
        const int64_t t0 = tile_row0(tile);
        // Q operand: row 16W + lr, features 32((ks + slice) % NQ) + 8g .. +7 (the order of kop below)
        bf16x8 qf[NQ];
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks) {
            if constexpr (QLDS) {
                qf[ks] = lds8(&sQ[buf][(16 * W + lr) * KS + 32 * ((ks + slice) & (NQ - 1)) + 8 * g]);
            } else {
                const uint4 qx = silu_q ? silu8(R.q[ks]) : R.q[ks];
                qf[ks] = __builtin_bit_cast(bf16x8, F16 ? bf16x8_to_f16(qx) : qx);
            }
        }
        // the gate values of this lane's outputs (row 16W + lr, columns 16jt + 4g..+3), read early
        // so the loads are long done when the products are
        uint2 gx[NJ];
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) gx[jt] = make_uint2(0u, 0u);
        if constexpr (GATE) {
            const __amdgpu_buffer_rsrc_t rg = make_rsrc(Gg + t0 * sn, tile_bytes(tile));
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
                gx[jt] = buf_load8(rg, (uint32_t)(16 * W + lr) * row_bytes + 2u * (16 * jt + 4 * g));
        }
        // Issue every LDS operand read of the inter and score products up front (the fence keeps
        // the scheduler from sinking them next to their MFMAs, which would expose each read's
        // latency in turn).
        bf16x8 sh[NJ][NQ], sl[NJ][NQ], kop[W + 1][NQ];
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
            for (int ks = 0; ks < NQ; ++ks) {
                const int off = ss_off<D>(16 * jt + lr, 32 * ((ks + slice) & (NQ - 1)) + 8 * g);
                sh[jt][ks] = lds8(&sS[buf][off]);
                if constexpr (!F16) sl[jt][ks] = lds8(&sSl[buf][off]);
            }
#pragma unroll
        for (int ct = 0; ct <= W; ++ct)
#pragma unroll
            for (int ks = 0; ks < NQ; ++ks)
                kop[ct][ks] = lds8(&sK[buf][(16 * ct + lr) * KS + 32 * ((ks + slice) & (NQ - 1)) + 8 * g]);
        __builtin_amdgcn_sched_barrier(0);
        // inter-tile term, transposed: (Q KV)^T = KV^T Q^T, so a lane's accumulators hold one output
        // row (query lr) and four consecutive value columns 16jt + 4g..+3; rows scaled by lambda^(r+1)
        f32x4 acc[NJ];
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NQ; ++ks) {
                if constexpr (F16) {
                    acc[jt] = mfma_h(sh[jt][ks], qf[ks], acc[jt]);
                } else {
                    acc[jt] = mfma(sh[jt][ks], qf[ks], acc[jt]);
                    acc[jt] = mfma(sl[jt][ks], qf[ks], acc[jt]);
                }
            }
        }
        // intra-tile scores S^T for key tiles 0..W (later key tiles are fully masked)
        float p[4][4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            if (ct <= W) {
                f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NQ; ++ks) s = F16 ? mfma_h(kop[ct][ks], qf[ks], s) : mfma(kop[ct][ks], qf[ks], s);
#pragma unroll
                for (int t = 0; t < 4; ++t) p[ct][t] = s[t] * dmask[ct][t];
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) p[ct][t] = 0.f;
            }
        }
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) acc[jt] *= drow;
        // (the fences keep the staging and refill at this point, measured best: at the start of the
        // tile they delay the products, at its end the next tile's Q)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (QLDS)
            if (tile + 1 < n_tiles) stage_q(R, buf ^ 1);
        load_q(R, tile + 2);
        __builtin_amdgcn_sched_barrier(0);
        // intra-tile output, transposed like the inter term: (P V)^T = V^T P^T (keys 32k2 +
        // {4g..4g+3, 16+4g..16+4g+3} in each 32-key step; the S^T accumulators are P^T's operand)
        constexpr int NK2 = W / 2 + 1;
        bf16x8 vop[NK2][NJ];
#pragma unroll
        for (int k2 = 0; k2 < NK2; ++k2)
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
                const u16* vb = &sV[buf][tr_row * VS + 16 * jt + tr_col];
                vop[k2][jt] = join(lds_tr(vb + (32 * k2 + 4 * g) * VS), lds_tr(vb + (32 * k2 + 16 + 4 * g) * VS));
            }
#pragma unroll
        for (int k2 = 0; k2 < NK2; ++k2) {
            if constexpr (F16) {
                const bf16x8 ph = __builtin_bit_cast(
                    bf16x8, make_uint4(cvt2h(p[2 * k2][0], p[2 * k2][1]), cvt2h(p[2 * k2][2], p[2 * k2][3]),
                                       cvt2h(p[2 * k2 + 1][0], p[2 * k2 + 1][1]),
                                       cvt2h(p[2 * k2 + 1][2], p[2 * k2 + 1][3])));
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt) acc[jt] = mfma_h(vop[k2][jt], ph, acc[jt]);
            } else {
                uint32_t hh[4], ll[4];
                split2(p[2 * k2][0], p[2 * k2][1], hh[0], ll[0]);
                split2(p[2 * k2][2], p[2 * k2][3], hh[1], ll[1]);
                split2(p[2 * k2 + 1][0], p[2 * k2 + 1][1], hh[2], ll[2]);
                split2(p[2 * k2 + 1][2], p[2 * k2 + 1][3], hh[3], ll[3]);
                const bf16x8 ph = __builtin_bit_cast(bf16x8, make_uint4(hh[0], hh[1], hh[2], hh[3]));
                const bf16x8 pl = __builtin_bit_cast(bf16x8, make_uint4(ll[0], ll[1], ll[2], ll[3]));
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt) {
                    acc[jt] = mfma(vop[k2][jt], ph, acc[jt]);
                    acc[jt] = mfma(vop[k2][jt], pl, acc[jt]);
                }
            }
        }
        // undo the 2^-8 of P and of the state copy
        if constexpr (F16)
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) acc[jt] *= 1.f / kHalfScale;
        // gate in float32, so the output is rounded to bf16 once
        if constexpr (GATE)
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) gate4(acc[jt], gx[jt]);
        // output tile: stage this wave's 16 rows (8-byte runs of 4 columns), then 16-byte stores
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
            *reinterpret_cast<uint2*>(&sO[(16 * W + lr) * OS + 16 * jt + 4 * g]) =
                make_uint2(cvt2(acc[jt][0], acc[jt][1]), cvt2(acc[jt][2], acc[jt][3]));
        wave_lds_sync();
        {
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(Og + t0 * sn, tile_bytes(tile));
#pragma unroll
            for (int m = 0; m < NV; ++m) {
                const int c = l + 64 * m, rr = 16 * W + c / PPR, cc = 8 * (c % PPR);
                const uint4 x = *reinterpret_cast<const uint4*>(&sO[rr * OS + cc]);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), ro,
                                                       (int)(row_off(tile, rr) + 2u * cc), 0, 0);
            }
        }
    };

    // ------------------------------------------------------------------ tile loops
    // Each role runs its own loop (so their registers do not overlap); both pass the same
    // barriers: one after the prologue and one between consecutive tiles.  Tiles alternate
    // between LDS buffers 0 and 1 and between register sets A and B.
    auto state_loop = [&](auto swc) __attribute__((always_inline)) {
        f32x4 st[st_count(decltype(swc)::value)];
        const float* src = nullptr;
        if (MODE != kModeLocal) src = (wk.nck > 1) ? a.ws + wk.slot_in * d2 : a.kv + u * d2;
        load_state(swc, st, src);
        KR RA, RB;
        load_kv(RA, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_kv(RB, 1);
        __builtin_amdgcn_sched_barrier(0);
        stage_tile(RA, 0, 0);
        if (OUT) write_state_copy(swc, st, 0);
        // Both roles issue at the same priority.  (Raising the state waves' priority, as they carry
        // the chain from one tile's state to the next tile's inter term, paid before Q was staged
        // in LDS and has cost 0.6-2.5% since.)
        // Checkpoints fall on tile ends (ckpt_every is a multiple of the tile and chunks start on
        // tile boundaries), so a per-tile counter replaces a 64-bit division per tile: ck_phase
        // counts the tiles since the last checkpoint, ck_slot is the next checkpoint's slot.
        const int ck_tiles = a.ckpt ? (int)(a.ckpt_every / BK) : 1;
        int ck_phase = a.ckpt ? (int)((t_begin / BK) % ck_tiles) : 0;
        int64_t ck_slot = a.ckpt ? t_begin / a.ckpt_every : 0;
        __syncthreads();
        auto step = [&](KR& R, KR& Rn, int buf, int tile) __attribute__((always_inline)) {
            __builtin_amdgcn_sched_barrier(0);
            load_kv(R, tile + 2);
            __builtin_amdgcn_sched_barrier(0);
            update_state(swc, st, buf, tile);
            if (OUT && tile + 1 < n_tiles) write_state_copy(swc, st, buf ^ 1);
            if (MODE != kModeLocal && a.ckpt) {
                if (++ck_phase == ck_tiles) {
                    ck_phase = 0;
                    // a short last tile never ends on a checkpoint (its end is not a tile multiple)
                    if (tile_len(tile) == BK) store_state(swc, st, a.ckpt + (u * a.n_ckpt + ck_slot) * d2);
                    ++ck_slot;
                }
            }
            if (tile + 1 < n_tiles) stage_tile(Rn, buf ^ 1, tile + 1);
        };
        int tile = 0;
        for (; tile + 2 <= n_tiles; tile += 2) {
            step(RA, RB, 0, tile);
            __syncthreads();
            step(RB, RA, 1, tile + 1);
            __syncthreads();
        }
        if (tile < n_tiles) step(RA, RB, 0, tile);
        if (MODE == kModeLocal) store_state(swc, st, a.ws + wk.slot_out * d2);
        else if (j == wk.nck - 1) store_state(swc, st, a.kv + u * d2);
    };
    auto out_loop = [&](auto wc) __attribute__((always_inline)) {
        // Staged Q: Q of tile t is loaded during tile t - 2 and staged during tile t - 1, a tile of
        // latency in one register set (measured as fast as two sets loaded a tile earlier); tile 0 is
        // staged here.  Otherwise two register sets alternate, each loaded two tiles ahead.
        QR QA, QB;
        load_q(QA, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (QLDS) {
            stage_q(QA, 0);
            load_q(QA, 1);
        } else {
            load_q(QB, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        QR& Q1 = QLDS ? QA : QB;
        int tile = 0;
        for (; tile + 2 <= n_tiles; tile += 2) {
            compute_out(wc, QA, 0, tile);
            __syncthreads();
            compute_out(wc, Q1, 1, tile + 1);
            __syncthreads();
        }
        if (tile < n_tiles) compute_out(wc, QA, 0, tile);
    };
    // Each wave runs a loop specialised to its role and index (static work lists, no per-tile
    // branches); all loops pass the same barriers: one after the prologue and one between tiles.
    switch (w) {
    case 0: if constexpr (OUT) out_loop(IntC<0>{}); else state_loop(IntC<0>{}); break;
    case 1: if constexpr (OUT) out_loop(IntC<1>{}); else state_loop(IntC<1>{}); break;
    case 2: if constexpr (OUT) out_loop(IntC<2>{}); else state_loop(IntC<2>{}); break;
    case 3: if constexpr (OUT) out_loop(IntC<3>{}); else state_loop(IntC<3>{}); break;
    case 4: state_loop(IntC<0>{}); break;
    case 5: state_loop(IntC<1>{}); break;
    case 6: state_loop(IntC<2>{}); break;
    default: state_loop(IntC<3>{}); break;
    }
}

// ------------------------------------------------------------------ chunk summaries at full width
// Page "MiniMax-01: Scaling Foundation Models with Lightning Attention | Summary", section 3.2
// (LASP+): each partition's local summary S = sum_t lambda^(C-1-t) k_t^T v_t, from a zero state.
// The tile kernel above slices the value columns over four workgroups, which suits the outputs,
// but for a summary alone it makes each slice re-read all of K.  Here one workgroup owns a whole
// (sequence, head, sub-chunk) and its full d x d state: K and V are read once.  Per 64-token tile
// the state is decayed by lambda^L and K^T (W V) is added.  F16 (summaries for a prefill with
// float16 outputs, which bounds the inputs the same way): K and W V as float16, one MFMA per
// product; W V needs no scale here, as no copy of the state enters a product.  Otherwise (state-only
// prefills and the backward) bf16 K and W V as a bf16 hi + lo pair, over float32's range.  Eight
// waves split the (D/16)^2 state tiles of 16 x 16 into 8 / (D/32) key-row groups x D/32
// value-column groups: 2 x 4 groups of 4 x 2 tiles at d = 128, 4 x 2 groups of 1 x 2 tiles at
// d = 64.  No SiLU prologue (the fused path keeps the sliced summaries).  Forward summaries skip
// the tokens whose weight at their chunk's end is too small to reach float32 (see tile0 below).
template <int D> struct SumRegs { uint4 k[D / 64]; uint4 v[D / 64]; };  // 16-byte chunks tid + 512m of K and V

template <bool REV, bool F16, int D>
__global__ __launch_bounds__(512, 1) void k_summary_bf16(FwdArgs a)
{
    static_assert(D == 64 || D == 128, "head dimension 64 or 128");
    constexpr int KS = kKS<D>;
    constexpr int CPR = D / 8, CPR_LOG = D == 128 ? 4 : 3;    // 16-byte chunks per row of K or V
    constexpr int M = D / 64;                                  // chunks per thread and tile
    constexpr int WJ = D / 32, WI = 8 / WJ;                    // wave groups over value, key tiles
    constexpr int NI = (D / 16) / WI, NJ = (D / 16) / WJ;      // a wave's key-row, value-col tiles
    using SR = SumRegs<D>;
    __shared__ __attribute__((aligned(16))) u16 sK[2][BK * KS];
    __shared__ __attribute__((aligned(16))) u16 sWh[2][BK * KS];
    __shared__ __attribute__((aligned(16))) u16 sWl[F16 ? 1 : 2][F16 ? 8 : BK * KS];

    if ((int64_t)blockIdx.x >= a.groups) return;
    // Workgroup order (fixed-length batches, evenly split sub-chunks): by a sub-chunk's position
    // from its chunk's end first, then (sequence, head), then chunk.  The sub-chunks nearest their
    // chunk's end are the ones that keep the most tiles once the decayed tokens are skipped, so
    // they are dispatched first, ahead of the ones that finish at once; consecutive ids (which go
    // round-robin over the XCDs) keep walking a head's chunks, as in the plain order.
    int64_t group = blockIdx.x;
    if (!a.ctab && a.span > 0) {
        const int64_t ns = a.chunks_launched, per = a.span / a.chunk, nc = ns / per, bh = a.groups / ns;
        if (per > 1 && summary_windowed(a.chunk)) {
            // sub-chunks over the decay windows: all of a head's sub-chunks keep the same number of
            // tiles, which grows with the head's window; the model's decay rates fall with the head
            // index, so the last (sequence, head) comes first and the longest windows start on
            // CUs of their own
            group = (bh - 1 - group / ns) * ns + group % ns;
        } else {
            const int64_t rank = group / (bh * nc), rem = group % (bh * nc);
            group = (rem / nc) * ns + (rem % nc) * per + (per - 1 - rank);
        }
    }
    const Work wk = decode_work(a, group);
    if (wk.j == wk.nck - 1) return;  // a sequence's last (sub-)chunk needs no summary
    // Tokens too far before their chunk's end to matter (summary_window: the tokens before e - W
    // change a chunk ending at e by less than the smallest float32 denormal).  Forward summaries
    // start their tiles at the first one that holds a token from e - W on, all of them with no
    // decay; long fixed-length sub-chunks are moreover placed end to end over the window alone
    // (summary_sub_len, as the prefix combine expects), so a head whose window is shorter than its
    // chunk splits the window, not the chunk, over its workgroups.
    int64_t t_begin = wk.t_begin, t_end = wk.t_end;
    double win = 0.0;
    int64_t e = 0;
    if (!REV && a.span > 0) {
        win = summary_window(a.slopes[wk.h], F16);
        e = ((t_begin / a.span) + 1) * a.span;
        const int64_t per = a.span / a.chunk;
        if (!a.ctab && per > 1 && summary_windowed(a.chunk)) {
            const int64_t len = summary_sub_len(win, a.span, per);
            const int64_t i = (t_begin % a.span) / a.chunk;  // position within the chunk
            t_begin = e - (per - i) * len;
            t_end = t_begin + len;
        }
    }
    const int n_tiles = (int)((t_end - t_begin + BK - 1) / BK);
    int tile0 = 0;
    if (!REV && a.span > 0) {
        const double first = (double)(e - t_begin) - win;  // tokens of the sub-chunk before e - W
        if (first > 0.0) tile0 = first >= (double)n_tiles * BK ? n_tiles : (int)(first / BK);
    }
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, g = l >> 4;
    // this wave's state tiles: key rows 16(it0..it0+NI-1), value columns 16(jt0..jt0+NJ-1)
    const int it0 = NI * (w / WJ), jt0 = NJ * (w % WJ);
    const int tr_row = lr >> 2, tr_col = 4 * (lr & 3);
    const float nsl = neg_slope_log2e(a.slopes, wk.h);
    const u16* Kg = static_cast<const u16*>(a.k) + wk.base;
    const u16* Vg = static_cast<const u16*>(a.v) + wk.base;
    const int64_t sn = a.sn;
    const uint32_t row_bytes = (uint32_t)(sn * 2);

    auto tile_len = [&](int tile) __attribute__((always_inline)) {
        const int64_t t0 = t_begin + (int64_t)tile * BK;
        return (int)((t_end - t0 < BK) ? t_end - t0 : BK);
    };
    auto tile_bytes = [&](int tile) __attribute__((always_inline)) {
        const int L = tile_len(tile);
        return (int64_t)(L > 0 ? L : 0) * row_bytes;
    };
    // memory row of the tile's first byte and byte offset of its row r (reverse walk: row r is
    // memory row L-1-r of the span; rows past the span fall outside the buffer and read zero)
    auto tile_row0 = [&](int tile) __attribute__((always_inline)) {
        const int64_t t0 = t_begin + (int64_t)tile * BK;
        if constexpr (!REV) return t0;
        const int L = tile_len(tile);
        const int64_t r0 = wk.rev_end - t0 - (L > 0 ? L : 0);
        return r0 > 0 ? r0 : (int64_t)0;
    };
    auto row_off = [&](int tile, int r) __attribute__((always_inline)) {
        if constexpr (!REV) return (uint32_t)r * row_bytes;
        return (uint32_t)(tile_len(tile) - 1 - r) * row_bytes;
    };
    auto load = [&](SR& R, int tile) __attribute__((always_inline)) {
        const int64_t t0 = tile_row0(tile);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + t0 * sn, tile_bytes(tile));
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + t0 * sn, tile_bytes(tile));
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int c = tid + 512 * m;
            R.k[m] = buf_load16(rk, row_off(tile, c >> CPR_LOG) + 16u * (c & (CPR - 1)));
            R.v[m] = buf_load16(rv, row_off(tile, c >> CPR_LOG) + 16u * (c & (CPR - 1)));
        }
    };
    // decay weights of a full tile and of the last tile (the only one that can be shorter),
    // computed once: rows (tid + 512m) / CPR of W, and lambda^L
    const int L_last = tile_len(n_tiles - 1);
    float wt_full[M], wt_last[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int r = (tid + 512 * m) >> CPR_LOG;
        wt_full[m] = decay_pow(nsl, (float)(BK - 1 - r));
        wt_last[m] = (r < L_last) ? decay_pow(nsl, (float)(L_last - 1 - r)) : 0.f;
    }
    const float dl_full = decay_pow(nsl, (float)BK);
    const float dl_last = decay_pow(nsl, (float)L_last);
    auto stage = [&](const SR& R, int buf, int tile) __attribute__((always_inline)) {
        const int L = tile_len(tile);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int c = tid + 512 * m, r = c >> CPR_LOG, off = r * KS + 8 * (c & (CPR - 1));
            *reinterpret_cast<uint4*>(&sK[buf][off]) = F16 ? bf16x8_to_f16(R.k[m]) : R.k[m];
            const float wt = (L == BK) ? wt_full[m] : wt_last[m];
            const uint32_t in[4] = {R.v[m].x, R.v[m].y, R.v[m].z, R.v[m].w};
            if constexpr (F16) {
                uint32_t hw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) hw[e] = cvt2h(bits_to_f32(in[e] & 0xffffu) * wt, hi_to_f32(in[e]) * wt);
                *reinterpret_cast<uint4*>(&sWh[buf][off]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            } else {
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    split2(bits_to_f32(in[e] & 0xffffu) * wt, hi_to_f32(in[e]) * wt, hi[e], lo[e]);
                *reinterpret_cast<uint4*>(&sWh[buf][off]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                *reinterpret_cast<uint4*>(&sWl[buf][off]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            }
        }
    };
    f32x4 st[NI * NJ];
#pragma unroll
    for (int k = 0; k < NI * NJ; ++k) st[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    // S <- lambda^L S + K^T (W V) on this wave's 4 x 2 state tiles (k = token within the tile)
    auto update = [&](int buf, int tile) __attribute__((always_inline)) {
        const float dl = (tile_len(tile) == BK) ? dl_full : dl_last;
#pragma unroll
        for (int k = 0; k < NI * NJ; ++k) st[k] *= dl;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int k0 = 32 * ks + 8 * g;
            bf16x8 ka[NI], vh[NJ], vl[NJ];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int o = (k0 + tr_row) * KS + 16 * (it0 + i) + tr_col;
                ka[i] = join(lds_tr(&sK[buf][o]), lds_tr(&sK[buf][o + 4 * KS]));
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int o = (k0 + tr_row) * KS + 16 * (jt0 + j) + tr_col;
                vh[j] = join(lds_tr(&sWh[buf][o]), lds_tr(&sWh[buf][o + 4 * KS]));
                if constexpr (!F16) vl[j] = join(lds_tr(&sWl[buf][o]), lds_tr(&sWl[buf][o + 4 * KS]));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if constexpr (F16) {
                        st[NJ * i + j] = mfma_h(ka[i], vh[j], st[NJ * i + j]);
                    } else {
                        st[NJ * i + j] = mfma(ka[i], vh[j], st[NJ * i + j]);
                        st[NJ * i + j] = mfma(ka[i], vl[j], st[NJ * i + j]);
                    }
                }
        }
    };
    SR RA, RB;
    load(RA, tile0);
    __builtin_amdgcn_sched_barrier(0);
    load(RB, tile0 + 1);
    __builtin_amdgcn_sched_barrier(0);
    if (tile0 < n_tiles) stage(RA, 0, tile0);
    __syncthreads();
    auto step = [&](SR& R, SR& Rn, int buf, int tile) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        load(R, tile + 2);
        __builtin_amdgcn_sched_barrier(0);
        update(buf, tile);
        if (tile + 1 < n_tiles) stage(Rn, buf ^ 1, tile + 1);
    };
    int tile = tile0;
    for (; tile + 2 <= n_tiles; tile += 2) {
        step(RA, RB, 0, tile);
        __syncthreads();
        step(RB, RA, 1, tile + 1);
        __syncthreads();
    }
    if (tile < n_tiles) step(RA, RB, 0, tile);
    // C layout: lane (g, lr) holds rows 4g..4g+3 (key) of column lr (value) of each tile
    float* dst = a.ws + wk.slot_out * (int64_t)(D * D);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                dst[(16 * (it0 + i) + 4 * g + t) * D + 16 * (jt0 + j) + lr] = st[NJ * i + j][t];
}

template <bool GATE, bool REV, bool ACT, int D, bool WIDE>
void launch_mode(const FwdArgs& a, int mode, dim3 grid, hipStream_t stream)
{
    if (mode == kModeOut)
        hipLaunchKernelGGL((k_fwd_bf16<kModeOut, GATE, REV, ACT, D, WIDE, 32>), grid, dim3(512), 0, stream, a);
    else if (mode == kModeState)
        hipLaunchKernelGGL((k_fwd_bf16<kModeState, false, REV, ACT, D, false, 32>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((k_fwd_bf16<kModeLocal, false, REV, ACT, D, false, 32>), grid, dim3(256), 0, stream, a);
}

template <int D>
bool launch_d(const FwdArgs& a, int mode, hipStream_t stream)
{
    const dim3 grid((unsigned)xcd_grid_size(a.groups, a.slices));
    const bool gate = a.gate && mode == kModeOut, act = a.act != 0;
    if (a.slices * 64 == D) {
        // 64-column slices (two per head): plans choose them only for float16 outputs at d = 128
        // without a prologue; anything else is refused rather than run on the wrong columns
        if (D != 128 || mode != kModeOut || a.wide || a.rev || act) return false;
        if (gate) hipLaunchKernelGGL((k_fwd_bf16<kModeOut, true, false, false, 128, false, 64>), grid, dim3(512), 0, stream, a);
        else hipLaunchKernelGGL((k_fwd_bf16<kModeOut, false, false, false, 128, false, 64>), grid, dim3(512), 0, stream, a);
        return true;
    }
    // the backward's passes: plain inputs, full-range operands
    if (a.rev) launch_mode<false, true, false, D, true>(a, mode, grid, stream);
    else if (a.wide) launch_mode<false, false, false, D, true>(a, mode, grid, stream);
    else if (gate && act) launch_mode<true, false, true, D, false>(a, mode, grid, stream);
    else if (gate) launch_mode<true, false, false, D, false>(a, mode, grid, stream);
    else if (act) launch_mode<false, false, true, D, false>(a, mode, grid, stream);
    else launch_mode<false, false, false, D, false>(a, mode, grid, stream);
    return true;
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, int mode, hipStream_t stream)
{
    if (!(d == 128 ? launch_d<128>(a, mode, stream) : launch_d<64>(a, mode, stream))) return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int D>
void launch_summary_d(const FwdArgs& a, hipStream_t stream)
{
    const dim3 grid((unsigned)a.groups), block(512);
    // float16 operands only for a prefill with float16 outputs (whose inputs are bounded alike)
    if (a.rev) hipLaunchKernelGGL((k_summary_bf16<true, false, D>), grid, block, 0, stream, a);
    else if (a.o && !a.wide) hipLaunchKernelGGL((k_summary_bf16<false, true, D>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_summary_bf16<false, false, D>), grid, block, 0, stream, a);
}

hipError_t launch_summary_bf16(const FwdArgs& a, int d, hipStream_t stream)
{
    if (d == 128) launch_summary_d<128>(a, stream);
    else launch_summary_d<64>(a, stream);
    return hipGetLastError();
}

}  // namespace la
