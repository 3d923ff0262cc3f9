/*
 * gla_oracle.c -- fp64 reference for the causal gated linear attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or call
 * this file.  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the GPU library.
 *
 * What it computes (the definition, not an optimisation of it):
 *
 *   Linear attention with the softmax removed is a linear recurrence whose hidden state
 *   is a Dk x Dv matrix; each step is a rank-1 outer-product write followed by a
 *   vector-matrix read.  [Hardware-Efficient Training of Linear Attention Models, talk
 *   summary, sections 4:04 "Introduction to Linear Attention" and 7:36 "Challenges in
 *   Training Linear Attention".]
 *
 *   Gated linear attention makes the recurrence data dependent.  [Gated Linear Attention
 *   Transformers with Hardware-Efficient Training, abstract.]  The pages print no
 *   formula; the plainest reading, used here, is that a gate alpha_t in (0,1]^Dk decays
 *   the rows (the key channels) of the state before the current token is written, and an
 *   optional scalar input gate i_t scales the write (the sigmoid-input-gate mLSTM
 *   variant of the Tiled Flash Linear Attention abstract):
 *
 *       S_t = diag(alpha_t) S_{t-1} + i_t k_t^T v_t ,     o_t = q_t S_t ,
 *
 *   with S_{-1} = S0 (zero unless an initial state is given).  Gates arrive in log
 *   space (log_alpha, log_ig); the factor applied at step t is exp() of the given value,
 *   evaluated in fp64 from the exact input value.  No scale factor or normaliser is
 *   applied.
 *
 * Precision: every input is converted to double by the caller (bf16 and fp32 convert
 * exactly); all arithmetic is fp64.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC -o liboracle.so gla_oracle.c -lm
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Token-by-token recurrence for every (b, h) pair.
 *
 *   q, k        [B, H, L, Dk]
 *   v           [B, H, L, Dv]
 *   log_alpha   [B, H, L, Dk]  (the caller broadcasts scalar gate kinds; zeros = ungated)
 *   log_ig      [B, H, L]      or NULL (input gate factor 1)
 *   S0          [B, H, Dk, Dv] or NULL (zero initial state)
 *   out         [B, H, L, Dv]
 *   final_state [B, H, Dk, Dv] or NULL
 *
 * Returns 0, or -1 when a size is not positive or a required pointer is NULL.
 * The (b, h) pairs are independent and are spread over OpenMP threads. */
int gla_oracle_recurrent(const double *q, const double *k, const double *v,
                         const double *log_alpha, const double *log_ig,
                         const double *S0, double *out, double *final_state,
                         long B, long H, long L, long Dk, long Dv)
{
    if (!q || !k || !v || !log_alpha || !out) return -1;
    if (B <= 0 || H <= 0 || L <= 0 || Dk <= 0 || Dv <= 0) return -1;
    const long BH = B * H;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        double *S = (double *)malloc(sizeof(double) * (size_t)(Dk * Dv));
        double *alpha = (double *)malloc(sizeof(double) * (size_t)Dk);
        if (!S || !alpha) {
            free(S);
            free(alpha);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        if (S0)
            memcpy(S, S0 + bh * Dk * Dv, sizeof(double) * (size_t)(Dk * Dv));
        else
            memset(S, 0, sizeof(double) * (size_t)(Dk * Dv));

        for (long t = 0; t < L; ++t) {
            const double *qt = q + (bh * L + t) * Dk;
            const double *kt = k + (bh * L + t) * Dk;
            const double *vt = v + (bh * L + t) * Dv;
            const double *lat = log_alpha + (bh * L + t) * Dk;
            const double ig = log_ig ? exp(log_ig[bh * L + t]) : 1.0;
            double *ot = out + (bh * L + t) * Dv;

            for (long d = 0; d < Dk; ++d) alpha[d] = exp(lat[d]);

            /* write: S <- diag(alpha_t) S + i_t k_t^T v_t */
            for (long d = 0; d < Dk; ++d) {
                double *Sd = S + d * Dv;
                const double a = alpha[d];
                const double w = ig * kt[d];
                for (long c = 0; c < Dv; ++c) Sd[c] = a * Sd[c] + w * vt[c];
            }
            /* read: o_t = q_t S_t */
            for (long c = 0; c < Dv; ++c) ot[c] = 0.0;
            for (long d = 0; d < Dk; ++d) {
                const double *Sd = S + d * Dv;
                const double qd = qt[d];
                for (long c = 0; c < Dv; ++c) ot[c] += qd * Sd[c];
            }
        }
        if (final_state)
            memcpy(final_state + bh * Dk * Dv, S, sizeof(double) * (size_t)(Dk * Dv));
        free(S);
        free(alpha);
    }
    return failed ? -1 : 0;
}

/* Number of OpenMP threads the recurrence uses (1 without OpenMP). */
int gla_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
