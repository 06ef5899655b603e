// Internal declarations shared by the gfx950 kernels and the C-ABI layer of
// liblightning_la.so.  Not installed; the public interface is include/la.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la.h"

namespace la {

constexpr int kBlock = 64;       // tokens per kernel tile (the model's tile of 256 is a flop-count
                                 // convention only; results do not depend on the tile)
constexpr int kSliceW = 32;      // value columns per workgroup (value-dim slicing)
constexpr int kTargetGroups = 256;  // workgroups that fill one MI355X (256 CUs, one resident each)
constexpr int kMinChunk = 1024;  // shortest chunk worth a 64 KiB state exchange
constexpr int kShortTokens = 8;  // packed sequences this short run token by token (no 64-token tile)
#ifndef LA_LOCAL_TARGET_GROUPS
#define LA_LOCAL_TARGET_GROUPS 128
#endif
// Chunk summaries are computed per sub-chunk (halving) until the summary pass has at least this
// many full-width workgroups at d = 128, twice as many at d = 64 (one per chunk-head; the sliced
// summaries of the fused path get a workgroup per value slice).  Measured on 8 heads at d = 128:
// 256 is 1.1% faster at 1M tokens and 5% slower at 32K (more summary slots to fold); 512 is slower
// at both.
constexpr int kLocalTargetGroups = LA_LOCAL_TARGET_GROUPS;
constexpr int kMinSubChunk = 256;  // shortest sub-chunk worth a 64 KiB summary
constexpr int kLongSubChunk = 4096;  // sub-chunks this long may be split further (la_abi.hip, make_plan)

// How a prefill is split: value-column slices x sequence chunks per (batch, head).
struct Plan {
    int64_t chunk;     // tokens per chunk (multiple of kBlock unless a single chunk)
    int64_t n_chunks;  // >= 1
    int slices;        // d / kSliceW
    int64_t sub;       // sub-chunks per chunk in the summary pass (power of two, chunk / sub a multiple of kBlock)
};

Plan make_plan(int64_t batch, int64_t heads, int64_t n, int64_t d, int64_t chunk_override,
               int slice_w = kSliceW);
constexpr int kWideSliceW = 64;  // value columns per workgroup of the wide-slice plans
constexpr int64_t kWideMinTokens = 65536;  // sequences this long take the wide slices in any case
// Value columns per workgroup of a forward prefill.  bf16 at d = 128 with float16 outputs and no
// SiLU prologue has a 64-column instantiation, whose workgroups take 1.55x the time per tile of
// the 32-column ones for twice the columns (the score products and the Q and K conversions serve
// twice the columns).  It pays where the work is split anyway: when the 32-column plan chunks the
// sequence (the wide plan's summaries then cover a few more tokens: 3/4 instead of 1/2 of them,
// 15/16 instead of 7/8), or needs more than one round of workgroups.  Where 32-column slices fill
// the GPU once without chunks (33 to 64 (batch, head) pairs), the wide plan adds a summary pass
// over about half the tokens; from kWideMinTokens on it still pays (64 heads x 131072 tokens:
// 2.19 -> 2.00 ms; the summaries skip the tokens whose decay cannot reach float32, and with no
// decay to skip it measured 2.145 ms), while shorter sequences keep the 32-column tile chains.
inline int fwd_slice_w(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d, bool out, bool wide,
                       uint32_t act)
{
    if (!(dt == LA_BF16 && d == 128 && out && !wide && act == 0)) return kSliceW;
    if (batch * heads * (d / kSliceW) > kTargetGroups || n >= kWideMinTokens) return kWideSliceW;
    return make_plan(batch, heads, n, d, 0, kSliceW).n_chunks > 1 ? kWideSliceW : kSliceW;
}

// What a forward kernel launch does with each (batch, head, chunk, slice) it owns.
enum FwdMode : int {
    kModeOut = 0,    // outputs + state, starting from the chunk's prefix state
    kModeState = 1,  // state (and checkpoints) only, starting from the chunk's prefix state
    kModeLocal = 2,  // local chunk summary from a zero state, written to the workspace
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int64_t sb, sh, sn;      // element strides of q/k/v/o
    int64_t heads;
    int64_t n;               // tokens per sequence
    int64_t chunk;           // tokens per chunk
    int64_t n_chunks;        // chunks per sequence
    int64_t chunks_launched; // chunks per sequence covered by this launch (n_chunks or n_chunks-1)
    int64_t groups;          // batch*heads*chunks_launched
    int slices;
    const float* slopes;
    float* kv;               // [B*H][d][d]
    float* ws;               // [B*H][n_chunks][d][d] (slot j = state entering chunk j) or null
    float* ckpt;             // [B*H][n_ckpt][d][d] or null
    int64_t ckpt_every;
    int64_t n_ckpt;
    // Packed variable-length batches (null for the fixed-length batch): ctab[5c..5c+4] = token
    // range begin and end (packed indices), sequence, chunk index within the sequence and first
    // chunk of that sequence, for global chunk c; stab[2s..2s+1] = first chunk and chunk count of
    // sequence s.  Workspace slot (c, h) = c*heads + h.
    const int64_t* ctab;
    const int64_t* stab;
    // Fused prologue/epilogue (la_fusion): act = LA_SILU_Q | LA_SILU_K | LA_SILU_V applied to the
    // inputs as they are loaded; gate (same layout as o, or null) multiplies each output by
    // sigmoid(gate) before it is stored.
    uint32_t act;
    const void* gate;
    // Reverse walk: token t of the recurrence is memory row rev_end-1-t of its sequence (see
    // Work); outputs are written to the same rows.  Used by the backward pass.
    int rev;
    // Full-range products for the outputs (bf16 hi + lo operands instead of float16): the
    // backward's passes, whose gradient inputs can lie far below float16's normal range.
    int wide;
    // Full-width chunk summaries of sub-chunks: tokens per chunk of the plan (the fold weighs a
    // sub-chunk's state by the decay to its chunk's end), or 0 when the launch's chunks are whole.
    int64_t span;
};

// SiLU(x) = x * sigmoid(x) = x / (1 + exp(-x)), in float32.
__device__ inline float silu_f32(float x)
{
    return x / (1.f + __expf(-x));
}
__device__ inline float sigmoid_f32(float x)
{
    return 1.f / (1.f + __expf(-x));
}

// What one workgroup processes: a chunk of one (sequence, head).
struct Work {
    int64_t u;         // state index: sequence * heads + head
    int64_t h;
    int64_t j;         // chunk index within the sequence
    int64_t nck;       // chunks of this sequence
    int64_t base;      // element offset of the (sequence, head) rows in q/k/v/o (t indexes rows)
    int64_t t_begin;   // token range of the chunk, [t_begin, t_end)
    int64_t t_end;
    int64_t slot_in;   // workspace slot with the chunk's incoming prefix (chunked sequences)
    int64_t slot_out;  // workspace slot that receives the chunk's local state (kModeLocal)
    int64_t rev_end;   // reverse walk: token u of the recurrence is memory row rev_end - 1 - u
                       // (n for a fixed-length batch, s0 + s1 for packed sequence [s0, s1))
};

__device__ inline Work decode_work(const FwdArgs& a, int64_t group)
{
    Work w;
    if (a.ctab) {
        const int64_t c = group / a.heads;
        w.h = group % a.heads;
        const int64_t* e = a.ctab + 5 * c;
        w.t_begin = e[0];
        w.t_end = e[1];
        const int64_t s = e[2];
        w.j = e[3];
        w.nck = a.stab[2 * s + 1];
        w.u = s * a.heads + w.h;
        w.base = w.h * a.sh;
        w.slot_in = c * a.heads + w.h;
        w.slot_out = (c + 1) * a.heads + w.h;
        // the sequence's first chunk begins at s0 and its last chunk ends at s1
        const int64_t c0 = e[4];
        w.rev_end = a.rev ? a.ctab[5 * c0] + a.ctab[5 * (c0 + w.nck - 1) + 1] : 0;
    } else {
        w.u = group / a.chunks_launched;
        w.j = group % a.chunks_launched;
        const int64_t bb = w.u / a.heads;
        w.h = w.u % a.heads;
        w.t_begin = w.j * a.chunk;
        w.t_end = (w.t_begin + a.chunk < a.n) ? w.t_begin + a.chunk : a.n;
        w.nck = a.n_chunks;
        w.base = bb * a.sb + w.h * a.sh;
        w.slot_in = w.u * a.n_chunks + w.j;
        w.slot_out = w.slot_in + 1;
        w.rev_end = a.n;
    }
    return w;
}

// Launchers (each returns the hipError_t of its launch).
// The float32 tile kernel (VALU arithmetic, d = 64 or 128).
hipError_t launch_fwd_f32(const FwdArgs& a, int d, int mode, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdArgs& a, int d, int mode, hipStream_t stream);
// Chunk summaries (kModeLocal semantics) at full width, one workgroup per group of `a` (no value
// slices); bf16 without the SiLU prologue, d = 64 or 128.
hipError_t launch_summary_bf16(const FwdArgs& a, int d, hipStream_t stream);
hipError_t launch_scan(float* ws, const float* kv, const float* slopes, int64_t bh, int64_t heads,
                       int64_t n_chunks, int64_t chunk, int d, hipStream_t stream);
// Prefixes from sub-chunk summaries: pref[u][0] = kv[u]; pref[u][j] = the state after chunks
// 0..j-1, folding sub[u][1 + (j-1)*n_sub_per + f] (sub-chunks of sub_len tokens) in order.
// window 0: the sub-chunks split each chunk evenly; 1 (float16 summaries) or 2 (bf16): they sit
// over each head's window before the chunk's end (summary_sub_len), as the summary kernel places
// them, and the tokens before it only decay the incoming prefix.
hipError_t launch_scan_sub(float* pref, const float* sub, const float* kv, const float* slopes, int64_t bh,
                           int64_t heads, int64_t n_chunks, int64_t n_sub_per, int64_t sub_len, int window,
                           int d, hipStream_t stream);
hipError_t launch_scan_varlen(float* ws, const float* kv, const float* slopes, const int64_t* stab,
                              int64_t n_seq, int64_t heads, int64_t chunk, int d, hipStream_t stream);
hipError_t launch_state_init(float* kv, const float* kv0, int64_t count, hipStream_t stream);
// ckpt[u][m] := kv[u] for the bh states u of d x d floats; ckpt holds n_ckpt slots per state.
hipError_t launch_state_to_slot(float* ckpt, const float* kv, int64_t bh, int d, int64_t n_ckpt, int64_t m,
                                hipStream_t stream);
// dst[u] := scale_u * src[u] (or its transpose), for the bh d x d states u; src == NULL gives
// zeros.  scale_u = exp(power * s_h), h = u % heads, power in {-1, 0, 1}.  dst may equal src
// only without the transpose.
hipError_t launch_state_prep(float* dst, const float* src, const float* slopes, int64_t bh, int64_t heads,
                             int d, bool transpose, int power, hipStream_t stream);
// Sequences of <= kShortTokens tokens, token by token (rev: from the last token to the first).
hipError_t launch_recur_short(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                              int64_t n_short, int64_t heads, int d, int64_t sn, int64_t sh,
                              const float* slopes, float* kv, const int64_t* tab, bool rev, hipStream_t stream);
// Decode step; `fu` (optional) adds the SiLU prologue, RMS normalisation and gate epilogue.
hipError_t launch_decode(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                         int64_t bh, int64_t heads, int d, const float* slopes, float* kv,
                         const la_fusion* fu, hipStream_t stream);
// RMS normalisation over d (optional weight) and/or sigmoid gate, in place on o, for the rows
// (b, h, t) of a [batch][heads][n] prefill output with o's strides (gate shares them).
hipError_t launch_norm_gate(la_dtype dt, void* o, const void* gate, const float* weight, float eps, bool norm,
                            int64_t batch, int64_t heads, int64_t n, int d, int64_t sb, int64_t sh, int64_t sn,
                            hipStream_t stream);

// Workgroup index -> (group, slice) with the slices of one group on one XCD.  Consecutive
// workgroup ids are dispatched round-robin over the 8 XCDs, so slices that share Q/K rows
// land on the same XCD and share its L2.
__host__ __device__ inline int64_t xcd_grid_size(int64_t groups, int slices)
{
    return ((groups + 7) / 8) * 8 * slices;
}

__device__ inline void xcd_decode(int64_t x, int slices, int64_t& group, int& slice)
{
    const int64_t xcd = x & 7;
    const int64_t loc = x >> 3;
    slice = (int)(loc % slices);
    group = (loc / slices) * 8 + xcd;
}

// lambda^k = exp(-s*k) for k >= 0, as exp2(nsl*k) with nsl = -s*log2(e).
__device__ inline float decay_pow(float nsl, float k)
{
    return exp2f(nsl * k);
}

__device__ inline float neg_slope_log2e(const float* slopes, int64_t h)
{
    return (float)(-(double)slopes[h] * 1.4426950408889634);
}

// Tokens before a chunk's end that can still reach its float32 state, for decay rate s: a token t
// of a chunk ending at e enters the state with weight lambda^(e-1-t), and every element of a local
// state is bounded by max|k v| / (1 - lambda) <= max|k v| (1 + 1/s), so the tokens before e - W with
// s W >= ln(max|k v|) + 150 ln 2 + ln(1 + 1/s) change it by less than the smallest float32 denormal.
// max|k v| < 65504^2 with float16 operands (f16: the range their prefill requires), else bf16's
// largest value squared; ln 2 of margin each.  No decay (or a rate that is not a positive finite
// number) returns a window longer than any sequence.
__device__ inline double summary_window(float slope, bool f16)
{
    const double sl = (double)slope;
    if (!(sl > 0.0 && sl < 1e30)) return 1e300;
    const double c = f16 ? 2.0 * 11.09 + 151.0 * 0.6931471805599453 : 2.0 * 88.72 + 151.0 * 0.6931471805599453;
    return (c + log1p(1.0 / sl)) / sl;
}

// Forward sub-chunks of at least kLongSubChunk tokens (even split) are placed over their head's
// window; shorter ones split their chunk evenly (at 1024-token sub-chunks the window placement
// measured 2-4% slower: the sub-chunks it fills had ended at once).
__host__ __device__ inline bool summary_windowed(int64_t even_sub_len)
{
    return even_sub_len >= kLongSubChunk;
}

// Sub-chunk length when the `per` sub-chunks of a chunk of `span` tokens sit end to end over the
// last tokens of the chunk only: the shortest tile multiple whose `per` copies cover the window,
// and at most span / per (the even split, whenever the window spans the chunk).  The summary
// kernel and the prefix combine both take it from here, so they place the sub-chunks alike.
__device__ inline int64_t summary_sub_len(double win, int64_t span, int64_t per)
{
    const int64_t even = span / per;
    const double tiles = ceil(win / (double)(per * kBlock));
    if (!(tiles * kBlock < (double)even)) return even;
    return (tiles >= 1.0 ? (int64_t)tiles : 1) * kBlock;
}

}  // namespace la
