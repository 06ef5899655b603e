/*
 * la_oracle.c -- plain, slow, obviously-correct fp64 reference for Lightning
 * Attention.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the product library never does.  It
 * shares no code with the GPU path.
 *
 * What is computed (page "MiniMax-01: Scaling Foundation Models with
 * Lightning Attention | Summary", section 2.2 Linear Attention): causal
 * linear attention evaluated in the reordered form Q(K^T V), i.e. with a
 * d x d key-value state carried along the sequence, with no normalisation,
 * no SiLU and no gating inside the operation.  The per-head exponential
 * decay lambda_h = exp(-s_h) of the mask is our reading of "masked
 * attention" within a tile; with s_h = 0 it is the plain causal case.
 *
 * For one (batch, head) with incoming state KV_{-1} (zero unless given):
 *     KV_t = lambda * KV_{t-1} + k_t^T v_t         (KV[i][j]: i key dim, j value dim)
 *     o_t  = q_t . KV_t                            (update first, then read out)
 * Every power of lambda is exp(-s*k) with k >= 0.
 *
 * Inputs are float32 (bf16 inputs are widened exactly by the caller); all
 * arithmetic is double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/*
 * Token-by-token recurrence over a whole prefill.
 *   q, k, v : [BH][N][d] float32, contiguous
 *   slopes  : [BH] double (s for each (batch, head) row)
 *   kv_in   : [BH][d][d] double or NULL (zero state)
 *   o       : [BH][N][d] double or NULL (state only)
 *   kv_out  : [BH][d][d] double or NULL
 *   ckpt    : [BH][N / ckpt_every][d][d] double or NULL; slot m holds KV after
 *             token (m+1)*ckpt_every - 1
 * kv_out may alias kv_in.
 */
void oracle_recurrent(const float* q, const float* k, const float* v,
                      int64_t BH, int64_t N, int64_t d, const double* slopes,
                      const double* kv_in, double* o, double* kv_out,
                      double* ckpt, int64_t ckpt_every)
{
    const int64_t n_ckpt = (ckpt && ckpt_every > 0) ? N / ckpt_every : 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < BH; ++u) {
        const double lam = exp(-slopes[u]);
        double* KV = (double*)malloc((size_t)(d * d) * sizeof(double));
        if (kv_in) memcpy(KV, kv_in + u * d * d, (size_t)(d * d) * sizeof(double));
        else memset(KV, 0, (size_t)(d * d) * sizeof(double));
        for (int64_t t = 0; t < N; ++t) {
            const float* qt = q + (u * N + t) * d;
            const float* kt = k + (u * N + t) * d;
            const float* vt = v + (u * N + t) * d;
            for (int64_t i = 0; i < d; ++i)
                for (int64_t j = 0; j < d; ++j)
                    KV[i * d + j] = lam * KV[i * d + j] + (double)kt[i] * (double)vt[j];
            if (o) {
                double* ot = o + (u * N + t) * d;
                for (int64_t j = 0; j < d; ++j) ot[j] = 0.0;
                for (int64_t i = 0; i < d; ++i) {
                    const double qi = (double)qt[i];
                    for (int64_t j = 0; j < d; ++j) ot[j] += qi * KV[i * d + j];
                }
            }
            if (n_ckpt && (t + 1) % ckpt_every == 0) {
                const int64_t m = (t + 1) / ckpt_every - 1;
                memcpy(ckpt + (u * n_ckpt + m) * d * d, KV, (size_t)(d * d) * sizeof(double));
            }
        }
        if (kv_out) memcpy(kv_out + u * d * d, KV, (size_t)(d * d) * sizeof(double));
        free(KV);
    }
}

/*
 * One decode step (section 3.3 of the same page keeps single-token
 * generation as its own kernel): for each row u,
 *     KV <- lambda * KV + k^T v ;   o = q . KV
 *   q, k, v : [BH][d] float32;  kv : [BH][d][d] double, updated in place;
 *   o : [BH][d] double.
 */
void oracle_decode_step(const float* q, const float* k, const float* v,
                        int64_t BH, int64_t d, const double* slopes,
                        double* kv, double* o)
{
#pragma omp parallel for schedule(static)
    for (int64_t u = 0; u < BH; ++u) {
        const double lam = exp(-slopes[u]);
        double* KV = kv + u * d * d;
        const float* qu = q + u * d;
        const float* ku = k + u * d;
        const float* vu = v + u * d;
        double* ou = o + u * d;
        for (int64_t i = 0; i < d; ++i)
            for (int64_t j = 0; j < d; ++j)
                KV[i * d + j] = lam * KV[i * d + j] + (double)ku[i] * (double)vu[j];
        for (int64_t j = 0; j < d; ++j) ou[j] = 0.0;
        for (int64_t i = 0; i < d; ++i)
            for (int64_t j = 0; j < d; ++j) ou[j] += (double)qu[i] * KV[i * d + j];
    }
}
