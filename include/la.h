/*
 * la.h -- C ABI of the MI355X (gfx950) Lightning Attention library
 * (liblightning_la.so).
 *
 * The operation: causal linear attention with a per-head exponential decay,
 * evaluated tile by tile with a d x d key-value state carried across tiles --
 * the "lightning attention" of the page "MiniMax-01: Scaling Foundation Models
 * with Lightning Attention | Summary", section 2.2 (Linear Attention): the
 * product is reordered to Q(K^T V) so no n x n matrix is formed, each tile
 * takes a masked intra-tile term plus a term from the accumulated state of
 * earlier tiles, then the state is updated; normalisation, SiLU and gating
 * are not part of it.  With lambda_h = exp(-slopes[h]) and, per (batch,
 * head), KV_{-1} = the incoming state:
 *
 *     KV_t = lambda_h * KV_{t-1} + k_t^T v_t        KV[i][j]: i = key dim, j = value dim
 *     o_t  = q_t . KV_t
 *
 * equivalently O = [(Q K^T) (.) M] V + diag(lambda^(t+1)) Q KV_{-1} with
 * M[t][s] = lambda^(t-s) for s <= t and 0 otherwise.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates no device memory.  Between calls it keeps a thread-local error
 *     string and, for the packed (varlen) entry points, a small ring of
 *     page-locked host buffers per device that stage their chunk tables.
 *   - Every call only enqueues work on `stream` (a hipStream_t passed as void*,
 *     NULL = the default stream) and returns; device-side faults appear at the
 *     caller's next synchronisation.
 *   - The return value reports argument validation and launch errors.  Invalid
 *     arguments are rejected before any HIP call.  With no usable GPU the call
 *     returns LA_ERR_DEVICE (it never aborts).  No C++ exception crosses the ABI.
 *   - The KV state is always float32, [batch][heads][d][d], row i = key dim.
 *   - Results are deterministic: the same inputs on the same device give the
 *     same bits (no floating-point atomics).
 *   - HIP graphs: la_state_init, la_prefill(_ex, _fused), la_decode(_fused)
 *     and la_backward enqueue kernels only (no allocation, memset or host
 *     copy), so a sequence of them can be captured into a graph and replayed;
 *     the replay reads the tensors at the captured addresses.
 *     la_prefill_varlen and la_backward_varlen pass chunk tables of up to 384
 *     int64 words (5 per chunk, 2 per sequence, 3 more per sequence of at most
 *     8 tokens) by value in kernel arguments, which a captured graph replays;
 *     larger tables are copied from a page-locked staging buffer that later
 *     calls reuse, so such calls must not be captured.
 */
#ifndef LIGHTNING_LA_H
#define LIGHTNING_LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad stride/alignment */
    LA_ERR_UNSUPPORTED = 2,      /* valid request outside the supported matrix (d, dtype, ckpt_every) */
    LA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than the queried size */
    LA_ERR_DEVICE = 4,           /* no GPU, or a HIP runtime error */
    LA_ERR_INTERNAL = 5
} la_status;

typedef enum {
    LA_F32 = 0,  /* q, k, v, o are float32 */
    LA_BF16 = 1  /* q, k, v, o are bfloat16; accumulation and state are float32 */
} la_dtype;
/*
 * Value range of LA_BF16 prefills with outputs.  Their products run on float16
 * matrix-core operands.  q, k and v are converted exactly for magnitudes in
 * [2^-14, 65504) (larger ones overflow to Inf).  The decay-weighted score block
 * q k^T, v weighted by its decay, and the float32 state enter their products
 * scaled by 2^-8, so each score and each state element must stay below
 * 65504 * 2^8 (about 1.7e7) in magnitude.  Operands round to 2^-11 relative
 * down to 2^-14 (inputs) and 2^-6 (scaled quantities); below that float16 keeps
 * fewer bits, which costs nothing where a small operand sits beside large ones
 * but loses relative precision for a head whose inputs are all far below unit
 * scale (the operation is linear in q and in v: scale them up and the outputs
 * down).  The float32 state itself is accumulated and stored at full precision.
 * State-only prefills (o == NULL), chunk summaries and the backward pass keep
 * bfloat16 operands with a hi + lo split of the float32 ones, over float32's
 * whole range.
 */

/*
 * Optional prologue and epilogue fused into the attention kernels.  Section 2.2
 * of the page above leaves normalisation, SiLU and gating out of the
 * derivation; section 3.3 fuses memory-bound steps into the attention kernels
 * ("batched kernel fusion").  Our reading of the three pieces:
 *   LA_SILU_Q/K/V : x -> x * sigmoid(x), elementwise, on q, k and/or v as they
 *                   are loaded (the bf16 paths round the activated value to
 *                   bf16 before the matrix products);
 *   LA_NORM       : o -> o / sqrt(mean_e(o_e^2) + norm_eps) * w_e over the d
 *                   features of one (token, head), w = norm_weight (NULL = 1);
 *   LA_GATE       : o -> o * sigmoid(g), g = gate, after the normalisation.
 */
enum {
    LA_SILU_Q = 1,
    LA_SILU_K = 2,
    LA_SILU_V = 4,
    LA_NORM = 8,
    LA_GATE = 16
};
typedef struct {
    uint32_t flags;           /* OR of the LA_SILU_* / LA_NORM / LA_GATE bits above */
    const void* gate;         /* LA_GATE: device tensor of o's dtype, shape and strides */
    const float* norm_weight; /* LA_NORM: [d] float32 device array, or NULL for all ones */
    float norm_eps;           /* LA_NORM: > 0 */
} la_fusion;

/*
 * kv[batch][heads][d][d] (float32) := 0 when kv0 == NULL, else a copy of kv0
 * (same layout; kv0 may not overlap kv).  The state a prefill or decode
 * starts from, e.g. a cached prefix (section 3 of the page above reuses the
 * computation of earlier input segments).  d in {64, 128}.
 */
la_status la_state_init(float* kv, const float* kv0, int64_t batch, int64_t heads, int64_t d,
                        void* stream);

/*
 * Tokens per sequence chunk that la_prefill uses for this shape.  Chunks are
 * the single-GPU form of LASP+ (section 3.2 of the page above: local prefix
 * summaries, combined into global prefixes): each chunk's local state is
 * computed from a zero state, the prefixes are combined, and every chunk then
 * runs from its own prefix, so a long sequence fills all compute units.  The
 * result equals the serial recurrence.  Returns n when one chunk is used, a
 * positive multiple of 64 otherwise, or -1 for invalid shapes.  For LA_BF16 at
 * d = 128 it describes a prefill with outputs (those may split the value
 * columns 64 instead of 32 per workgroup, which changes the chunking).
 */
int64_t la_prefill_chunk_tokens(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d);

/* Bytes of device workspace la_prefill needs for this shape (0 when it needs none),
 * with or without outputs. */
size_t la_prefill_workspace_size(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d);

/*
 * Prefill: for every (b, h), run tokens 0..n-1 starting from the state in
 * kv[b][h], write o (unless o == NULL: state only) and leave in kv[b][h] the
 * state after token n-1.
 *   q, k, v, o : element (b, h, t, e) at base + b*stride_b + h*stride_h +
 *                t*stride_n + e (strides in elements, shared by all four;
 *                the last dimension is contiguous).  q, k, v are read-only and
 *                may alias each other; o must not overlap q, k, v or kv, and
 *                its rows must be pairwise disjoint (no stride 0 on a
 *                dimension longer than one, no two (b, h, t) rows sharing an
 *                element), else LA_ERR_INVALID_ARGUMENT.
 *                Pointers 16-byte aligned; strides multiples of 8 elements
 *                (bf16) or 4 (f32); d <= stride_n <= 2^22 (a 64-row tile
 *                then spans under 2 GiB, the reach of a 32-bit buffer
 *                offset), else LA_ERR_UNSUPPORTED.
 *   slopes     : [heads] float32 device array, s_h >= 0 and finite
 *                (documented, not checked: reading it would need a sync);
 *                lambda_h = exp(-s_h).
 *   kv         : [batch][heads][d][d] float32, read then overwritten.
 *   ckpt       : NULL, or [batch][heads][n / ckpt_every][d][d] float32 that
 *                receives the state after token (m+1)*ckpt_every - 1 in slot m.
 *                ckpt_every must be positive (else LA_ERR_INVALID_ARGUMENT).
 *                Multiples of 64 (the kernel tile) are stored by the prefill
 *                kernels at tile ends at no extra cost; any other value runs
 *                the sequence as one prefill per ckpt_every tokens, each
 *                followed by a copy of the state into its slot.
 *   workspace  : device scratch of at least la_prefill_workspace_size() bytes
 *                (may be NULL when that size is 0); contents are clobbered.
 * Supported: d in {64, 128} for both dtypes (bfloat16 runs on the MFMA
 * kernels, float32 on the float32-arithmetic tile kernel);
 * batch*heads <= 2^20, and batch*heads*chunks <= 2^20 for the chunk count the
 * plan (or chunk_tokens) gives, else LA_ERR_UNSUPPORTED.
 * n == 0 is a no-op that leaves kv unchanged.
 */
la_status la_prefill(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                     int64_t batch, int64_t heads, int64_t n, int64_t d,
                     int64_t stride_b, int64_t stride_h, int64_t stride_n,
                     const float* slopes, float* kv, float* ckpt, int64_t ckpt_every,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * la_prefill for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument.  The chunk states live in a device array inside the
 * library of LA_NOALLOC_SCRATCH_BYTES (96 MiB), one per GPU, held until the
 * process ends; every shape the default plan chunks fits (the plan keeps its
 * chunk and sub-chunk states within 96 MiB; 15 heads of 1M tokens at d = 128
 * need 94.7 MiB), and a shape needing more returns LA_ERR_UNSUPPORTED.  The call allocates nothing and frees nothing.
 * All calls on one GPU share that array: calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race and
 * give wrong results; calls ordered on one stream are safe.  Arguments,
 * results and errors otherwise as la_prefill.
 */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
la_status la_prefill_noalloc(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                             int64_t batch, int64_t heads, int64_t n, int64_t d,
                             int64_t stride_b, int64_t stride_h, int64_t stride_n,
                             const float* slopes, float* kv, float* ckpt, int64_t ckpt_every, void* stream);

/*
 * As la_prefill with an explicit chunk length: chunk_tokens == 0 picks the
 * default (la_prefill_chunk_tokens), otherwise it must be a positive multiple
 * of 64 (values >= n mean one chunk).  The workspace must hold
 * la_prefill_workspace_size_ex() bytes for the same chunk_tokens.
 */
size_t la_prefill_workspace_size_ex(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d,
                                    int64_t chunk_tokens);
la_status la_prefill_ex(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                        int64_t batch, int64_t heads, int64_t n, int64_t d,
                        int64_t stride_b, int64_t stride_h, int64_t stride_n,
                        const float* slopes, float* kv, float* ckpt, int64_t ckpt_every,
                        int64_t chunk_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Packed variable-length prefill: n_seq sequences concatenated along the token
 * axis without padding (section 3.2 of the page above packs variable-length
 * samples back to back and tracks each one's offsets; section 3.3 runs long
 * and short inputs with separate work sizes).  Sequence s owns packed tokens
 * cu_seqlens[s] .. cu_seqlens[s+1]-1; each sequence starts from its own state
 * kv[s][h] and leaves its final state there.  One launch of the 64-token tile
 * kernel (plus, when a long sequence is cut into chunks, a chunk-summary launch
 * and a prefix combine) covers every sequence longer than 8 tokens; sequences
 * of 1..8 tokens run token by token in one more launch that reads and writes
 * their states once (the smallest of the work sizes section 3.3 uses for short
 * inputs), so short and long sequences share the GPU without padding.
 *   q, k, v, o : element (t, h, e) at base + t*stride_n + h*stride_h + e, t =
 *                packed token index (e.g. [total][heads][d] has stride_n =
 *                heads*d, stride_h = d); rules as for la_prefill (o's rows
 *                pairwise disjoint).
 *   cu_seqlens : HOST array of n_seq + 1 int64, cu_seqlens[0] = 0,
 *                nondecreasing (empty sequences allowed: their state is left
 *                unchanged).  Read during the call only.
 *   kv         : [n_seq][heads][d][d] float32, read then overwritten.
 *   workspace  : device scratch of at least la_prefill_varlen_workspace_size()
 *                bytes (never 0 bytes: it also receives the chunk tables);
 *                the call writes those tables into it asynchronously on
 *                `stream`: up to 384 words through a kernel's arguments, more
 *                by a copy from page-locked staging buffers that the library
 *                reuses only once the copy has completed.  Either way
 *                cu_seqlens may be released as soon as the call returns.  The
 *                workspace must not be in use by other work on other streams.
 * No checkpoints.  Supported dtypes and d as for la_prefill; n_seq*heads and
 * (chunks of the sequences longer than 8 tokens)*heads at most 2^20, else
 * LA_ERR_UNSUPPORTED.
 */
size_t la_prefill_varlen_workspace_size(la_dtype dt, int64_t n_seq, const int64_t* cu_seqlens, int64_t heads,
                                        int64_t d);
/* Chunk length the varlen prefill uses (sequences longer than it are chunked), -1 if invalid. */
int64_t la_prefill_varlen_chunk_tokens(la_dtype dt, int64_t n_seq, const int64_t* cu_seqlens, int64_t heads,
                                       int64_t d);
la_status la_prefill_varlen(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                            int64_t n_seq, const int64_t* cu_seqlens, int64_t heads, int64_t d,
                            int64_t stride_h, int64_t stride_n, const float* slopes, float* kv,
                            void* workspace, size_t workspace_bytes, void* stream);
/* As la_prefill_varlen with an explicit chunk length (0 = default, else a positive multiple of 64). */
size_t la_prefill_varlen_workspace_size_ex(la_dtype dt, int64_t n_seq, const int64_t* cu_seqlens, int64_t heads,
                                           int64_t d, int64_t chunk_tokens);
la_status la_prefill_varlen_ex(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                               int64_t n_seq, const int64_t* cu_seqlens, int64_t heads, int64_t d,
                               int64_t stride_h, int64_t stride_n, const float* slopes, float* kv,
                               int64_t chunk_tokens, void* workspace, size_t workspace_bytes, void* stream);
/*
 * la_prefill with the prologue/epilogue of `fusion` (NULL = none; then it is
 * la_prefill without checkpoints).  The SiLU flags act inside the prefill
 * kernels.  LA_GATE alone is applied in the prefill kernel's output store.
 * With LA_NORM, whose mean runs over all d features while each prefill
 * workgroup owns a slice of 32 or 64 value columns, the prefill writes o and one
 * more memory-bound pass normalises (and gates) it in place.  o must not be
 * NULL when LA_NORM or LA_GATE is set; gate must not overlap o.  Workspace as
 * for la_prefill.
 */
la_status la_prefill_fused(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                           int64_t batch, int64_t heads, int64_t n, int64_t d,
                           int64_t stride_b, int64_t stride_h, int64_t stride_n,
                           const float* slopes, float* kv, const la_fusion* fusion,
                           void* workspace, size_t workspace_bytes, void* stream);
/*
 * la_decode with the prologue/epilogue of `fusion` (NULL = none), all of it in
 * the decode kernel (one workgroup holds a whole output row).  gate is a
 * contiguous [batch][heads][d] tensor of dtype dt.
 */
la_status la_decode_fused(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                          int64_t batch, int64_t heads, int64_t d,
                          const float* slopes, float* kv, const la_fusion* fusion, void* stream);
/*
 * One decode step per (b, h) (section 3.3 of the page above runs single-token
 * generation as its own kernel): kv <- lambda_h * kv + k^T v, then o = q . kv.
 *   q, k, v, o : contiguous [batch][heads][d] of dtype dt (o must not overlap
 *                q, k, v or kv); slopes [heads] float32; kv [batch][heads][d][d]
 *                float32 updated in place.  d in {64, 128}; both dtypes;
 *                batch*heads <= 2^20 (else LA_ERR_UNSUPPORTED).
 */
la_status la_decode(la_dtype dt, const void* q, const void* k, const void* v, void* o,
                    int64_t batch, int64_t heads, int64_t d,
                    const float* slopes, float* kv, void* stream);

/*
 * Backward pass (training): gradients of a scalar loss L through la_prefill's
 * computation, given dout = dL/dO and optionally dkv_out = dL/dKV_final.  The
 * training side of LASP+ (section 3.2 of the page above) passes the state's
 * gradient backwards between partitions; here dkv_out is what a later
 * partition passes back and dkv_in what this one passes on.  With
 * G_t = dL/dKV_t (G_t = q_t^T do_t + lambda G_{t+1}, G_{n-1} = q^T do + dkv_out):
 *   dq_t = do_t KV_t^T,  dk_t = v_t G_t^T,  dv_t = k_t G_t,  dkv_in = lambda G_0.
 * The slopes are constants (no gradient).  Computed as three runs of the
 * prefill kernels (one forward, two walking the sequence backwards), so it
 * costs about three prefills.  With LA_BF16 the runs use full-range operands
 * (bfloat16 hi + lo pairs, not the forward's float16): gradients of a loss over
 * many elements are often far below float16's normal range, and every
 * magnitude bfloat16 holds is computed to the same relative precision.
 *   q, k, v, dout       : inputs of the forward pass and dL/dO, layout and
 *                         strides as for la_prefill (read-only, may alias).
 *   kv_in               : the forward pass's incoming state, or NULL (zero).
 *   dkv_out             : dL/dKV_final [batch][heads][d][d] float32, or NULL (zero).
 *                         Requires s_h < 80 (lambda > e^-80): it is scaled by 1/lambda.
 *   dq, dk, dv          : outputs, same layout and dtype; must not overlap the
 *                         inputs or each other, and their rows must be pairwise
 *                         disjoint as for la_prefill's o (else
 *                         LA_ERR_INVALID_ARGUMENT).
 *   dkv_in              : output dL/dKV_in [batch][heads][d][d] float32, or NULL
 *                         (not wanted); may alias kv_in or dkv_out.
 *   workspace           : at least la_backward_workspace_size() bytes (never 0).
 * No fused prologue/epilogue.  Supported dtypes and d as for la_prefill.
 * n == 0 gives dkv_in = dkv_out.  Asynchronous on `stream`.
 */
size_t la_backward_workspace_size(la_dtype dt, int64_t batch, int64_t heads, int64_t n, int64_t d);
la_status la_backward(la_dtype dt, const void* q, const void* k, const void* v, const void* dout,
                      int64_t batch, int64_t heads, int64_t n, int64_t d,
                      int64_t stride_b, int64_t stride_h, int64_t stride_n, const float* slopes,
                      const float* kv_in, const float* dkv_out, void* dq, void* dk, void* dv, float* dkv_in,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * la_backward for packed variable-length sequences (layout, cu_seqlens and
 * short-sequence handling as la_prefill_varlen): kv_in, dkv_out and dkv_in
 * are [n_seq][heads][d][d] float32 (NULL as for la_backward).  Each sequence's
 * gradients use only its own tokens and states; an empty sequence gives
 * dkv_in = dkv_out.  Like la_prefill_varlen it uploads chunk tables (three
 * times: one per run) and must not be captured into a graph.
 */
size_t la_backward_varlen_workspace_size(la_dtype dt, int64_t n_seq, const int64_t* cu_seqlens, int64_t heads,
                                         int64_t d);
la_status la_backward_varlen(la_dtype dt, const void* q, const void* k, const void* v, const void* dout,
                             int64_t n_seq, const int64_t* cu_seqlens, int64_t heads, int64_t d,
                             int64_t stride_h, int64_t stride_n, const float* slopes, const float* kv_in,
                             const float* dkv_out, void* dq, void* dk, void* dv, float* dkv_in,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* la_status_string(la_status s);

/* Thread-local detail of the last non-OK status returned on this thread ("" if none). */
const char* la_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_LA_H */
