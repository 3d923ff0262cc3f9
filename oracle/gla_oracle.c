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

/* Gradients of the recurrence (reverse-mode differentiation of each step, in fp64).
 *
 * Given the forward inputs and the gradients of a scalar loss with respect to the outputs,
 *   dO          [B, H, L, Dv]   d loss / d out
 *   dS_fin      [B, H, Dk, Dv]  d loss / d final_state, or NULL (zero)
 * it returns
 *   dq, dk      [B, H, L, Dk]
 *   dv          [B, H, L, Dv]
 *   dlog_alpha  [B, H, L, Dk]   with respect to the per-channel log decay (the caller sums
 *                               it over the broadcast axes of a scalar gate kind)
 *   dlog_ig     [B, H, L]       or NULL
 *   dS0         [B, H, Dk, Dv]  with respect to the initial state, or NULL
 *
 * Each step t is S_t = diag(a_t) S_{t-1} + i_t k_t^T v_t, o_t = q_t S_t, with
 * a_t = exp(log_alpha_t), i_t = exp(log_ig_t).  Walking t from L-1 down to 0 with
 * G = d loss / d S_t (starting from dS_fin):
 *   G += q_t^T dO_t                       (the read o_t = q_t S_t)
 *   dq_t = dO_t S_t^T
 *   dk_t = i_t G v_t^T,   dv_t = i_t k_t G
 *   dlog_ig_t = i_t k_t G v_t^T
 *   dlog_alpha_t[d] = a_t[d] sum_c G[d, c] S_{t-1}[d, c]
 *   G <- diag(a_t) G                      (d loss / d S_{t-1})
 * and dS0 is the final G.  The states S_{t-1} are recomputed from checkpoints every 64
 * tokens (the same forward recurrence), so memory stays O((L/64 + 64) Dk Dv) per pair.
 * Returns 0, or -1 on a bad size, a NULL required pointer or an allocation failure. */
int gla_oracle_backward(const double *q, const double *k, const double *v, const double *log_alpha,
                        const double *log_ig, const double *S0, const double *dO, const double *dS_fin,
                        double *dq, double *dk, double *dv, double *dlog_alpha, double *dlog_ig,
                        double *dS0, long B, long H, long L, long Dk, long Dv)
{
    if (!q || !k || !v || !log_alpha || !dO || !dq || !dk || !dv || !dlog_alpha) return -1;
    if (B <= 0 || H <= 0 || L <= 0 || Dk <= 0 || Dv <= 0) return -1;
    const long BH = B * H, M = Dk * Dv, CK = 64;
    const long ncp = (L + CK - 1) / CK;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        /* cp[j] = state before token j*CK (j = 0..ncp-1); blk[u] = state after token j*CK+u */
        double *cp = (double *)malloc(sizeof(double) * (size_t)(ncp * M));
        double *blk = (double *)malloc(sizeof(double) * (size_t)(CK * M));
        double *G = (double *)malloc(sizeof(double) * (size_t)M);
        if (!cp || !blk || !G) {
            free(cp);
            free(blk);
            free(G);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        const double *la = log_alpha + bh * L * Dk;
        const double *li = log_ig ? log_ig + bh * L : NULL;
        /* one forward step from Sp (state before t) into Sn */
#define GLA_STEP(Sp, Sn, t)                                                                  \
        do {                                                                                 \
            const double *kt_ = k + (bh * L + (t)) * Dk, *vt_ = v + (bh * L + (t)) * Dv;     \
            const double ig_ = li ? exp(li[(t)]) : 1.0;                                      \
            for (long d = 0; d < Dk; ++d) {                                                  \
                const double a_ = exp(la[(t) * Dk + d]), w_ = ig_ * kt_[d];                  \
                for (long c = 0; c < Dv; ++c) (Sn)[d * Dv + c] = a_ * (Sp)[d * Dv + c] + w_ * vt_[c]; \
            }                                                                                \
        } while (0)
        /* forward: checkpoints */
        if (S0)
            memcpy(cp, S0 + bh * M, sizeof(double) * (size_t)M);
        else
            memset(cp, 0, sizeof(double) * (size_t)M);
        for (long j = 0; j < ncp; ++j) {
            const long t0 = j * CK, t1 = t0 + CK < L ? t0 + CK : L;
            const double *Sp = cp + j * M;
            for (long t = t0; t < t1; ++t) {
                double *Sn = blk + (t - t0) * M;
                GLA_STEP(Sp, Sn, t);
                Sp = Sn;
            }
            if (j + 1 < ncp) memcpy(cp + (j + 1) * M, Sp, sizeof(double) * (size_t)M);
        }
        /* reverse */
        if (dS_fin)
            memcpy(G, dS_fin + bh * M, sizeof(double) * (size_t)M);
        else
            memset(G, 0, sizeof(double) * (size_t)M);
        for (long j = ncp - 1; j >= 0; --j) {
            const long t0 = j * CK, t1 = t0 + CK < L ? t0 + CK : L;
            {   /* states of this block, recomputed from its checkpoint */
                const double *Sp = cp + j * M;
                for (long t = t0; t < t1; ++t) {
                    double *Sn = blk + (t - t0) * M;
                    GLA_STEP(Sp, Sn, t);
                    Sp = Sn;
                }
            }
            for (long t = t1 - 1; t >= t0; --t) {
                const double *St = blk + (t - t0) * M;
                const double *Sprev = t > t0 ? blk + (t - 1 - t0) * M : cp + j * M;
                const double *qt = q + (bh * L + t) * Dk, *kt = k + (bh * L + t) * Dk;
                const double *vt = v + (bh * L + t) * Dv, *dOt = dO + (bh * L + t) * Dv;
                const double ig = li ? exp(li[t]) : 1.0;
                double *dqt = dq + (bh * L + t) * Dk, *dkt = dk + (bh * L + t) * Dk;
                double *dvt = dv + (bh * L + t) * Dv, *dlat = dlog_alpha + (bh * L + t) * Dk;
                for (long d = 0; d < Dk; ++d)
                    for (long c = 0; c < Dv; ++c) G[d * Dv + c] += qt[d] * dOt[c];
                double dli = 0.0;
                for (long c = 0; c < Dv; ++c) dvt[c] = 0.0;
                for (long d = 0; d < Dk; ++d) {
                    double sq = 0.0, sk = 0.0, sa = 0.0;
                    for (long c = 0; c < Dv; ++c) {
                        sq += dOt[c] * St[d * Dv + c];
                        sk += G[d * Dv + c] * vt[c];
                        sa += G[d * Dv + c] * Sprev[d * Dv + c];
                        dvt[c] += kt[d] * G[d * Dv + c];
                    }
                    const double a = exp(la[t * Dk + d]);
                    dqt[d] = sq;
                    dkt[d] = ig * sk;
                    dli += kt[d] * sk;
                    dlat[d] = a * sa;
                }
                for (long c = 0; c < Dv; ++c) dvt[c] *= ig;
                if (dlog_ig) dlog_ig[bh * L + t] = ig * dli;
                for (long d = 0; d < Dk; ++d) {
                    const double a = exp(la[t * Dk + d]);
                    for (long c = 0; c < Dv; ++c) G[d * Dv + c] *= a;
                }
            }
        }
#undef GLA_STEP
        if (dS0) memcpy(dS0 + bh * M, G, sizeof(double) * (size_t)M);
        free(cp);
        free(blk);
        free(G);
    }
    return failed ? -1 : 0;
}

/* The delta rule (DeltaNet) and its gated form, token by token, for every (b, h) pair.
 *
 * DeltaNet gives each token a writing strength beta_t that decides how much of the value
 * the state already associates with k_t is replaced by v_t [Hardware-Efficient Training of
 * Linear Attention Models, talk summary, 22:36].  Its update is one step of stochastic
 * gradient descent, with step size beta_t, on the squared error of predicting v_t from
 * k_t with the state as a fast weight [same talk, 31:16]: with the loss
 * 1/2 |k_t S - v_t|^2, whose gradient in S is k_t^T (k_t S - v_t),
 *
 *     S_t = S' - beta_t k_t^T (k_t S' - v_t) = (I - beta_t k_t^T k_t) S' + beta_t k_t^T v_t ,
 *
 * an identity-plus-rank-one transition [same talk, 31:16].  Gated DeltaNet adds a scalar
 * per-token decay alpha_t in the manner of Mamba-2 [same talk, 31:16]; read plainly, as
 * for the gated linear recurrence above, the decay applies to the previous state before
 * the token is written: S' = alpha_t S_{t-1} (alpha_t = 1 for DeltaNet).  The read is
 * o_t = q_t S_t, as in linear attention [same talk, 4:04].
 *
 *   q, k        [B, H, L, Dk]
 *   v           [B, H, L, Dv]
 *   beta        [B, H, L]      writing strength, used as given
 *   log_alpha   [B, H, L]      natural log of the decay, or NULL (alpha = 1)
 *   S0          [B, H, Dk, Dv] or NULL (zero initial state)
 *   out         [B, H, L, Dv]
 *   final_state [B, H, Dk, Dv] or NULL
 *
 * Returns 0, or -1 when a size is not positive, a required pointer is NULL or an
 * allocation fails. */
int gla_oracle_delta(const double *q, const double *k, const double *v, const double *beta,
                     const double *log_alpha, const double *S0, double *out, double *final_state,
                     long B, long H, long L, long Dk, long Dv)
{
    if (!q || !k || !v || !beta || !out) return -1;
    if (B <= 0 || H <= 0 || L <= 0 || Dk <= 0 || Dv <= 0) return -1;
    const long BH = B * H;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        double *S = (double *)malloc(sizeof(double) * (size_t)(Dk * Dv));
        double *pred = (double *)malloc(sizeof(double) * (size_t)Dv);
        if (!S || !pred) {
            free(S);
            free(pred);
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
            const double bt = beta[bh * L + t];
            const double at = log_alpha ? exp(log_alpha[bh * L + t]) : 1.0;
            double *ot = out + (bh * L + t) * Dv;

            /* decay: S' = alpha_t S_{t-1} */
            for (long i = 0; i < Dk * Dv; ++i) S[i] *= at;
            /* prediction of v_t from the decayed state: k_t S' */
            for (long c = 0; c < Dv; ++c) pred[c] = 0.0;
            for (long d = 0; d < Dk; ++d) {
                const double *Sd = S + d * Dv;
                for (long c = 0; c < Dv; ++c) pred[c] += kt[d] * Sd[c];
            }
            /* gradient step: S_t = S' + beta_t k_t^T (v_t - k_t S') */
            for (long d = 0; d < Dk; ++d) {
                double *Sd = S + d * Dv;
                const double w = bt * kt[d];
                for (long c = 0; c < Dv; ++c) Sd[c] += w * (vt[c] - pred[c]);
            }
            /* read: o_t = q_t S_t */
            for (long c = 0; c < Dv; ++c) ot[c] = 0.0;
            for (long d = 0; d < Dk; ++d) {
                const double *Sd = S + d * Dv;
                for (long c = 0; c < Dv; ++c) ot[c] += qt[d] * Sd[c];
            }
        }
        if (final_state)
            memcpy(final_state + bh * Dk * Dv, S, sizeof(double) * (size_t)(Dk * Dv));
        free(S);
        free(pred);
    }
    return failed ? -1 : 0;
}

/* The mLSTM cell (the xLSTM's matrix memory), token by token in fp64: the memory and its
 * normaliser decay by the forget gate f_t = exp(log_f_t) and take the token's write with the
 * exponential input gate i_t = exp(log_i_t),
 *     C_t = f_t C_{t-1} + i_t k_t^T v_t ,    n_t = f_t n_{t-1} + i_t k_t ,
 * and the token reads h_t = q_t C_t / max(|q_t . n_t|, 1)
 * [Tiled Flash Linear Attention, abstract: the mLSTM of Beck et al. (2024), with its
 * exponential input gate and normaliser; the sigmoid-gated variant drops both].
 * C is Dk x Dv (row d, column c), n has Dk entries.  An initial state (C0, n0) is taken in
 * the unstabilised scale; NULL starts from zero.  final_C / final_n may be NULL. */
int gla_oracle_mlstm(const double *q, const double *k, const double *v, const double *log_f,
                     const double *log_i, const double *C0, const double *n0, double *out, double *final_C,
                     double *final_n, long B, long H, long L, long Dk, long Dv)
{
    if (!q || !k || !v || !log_f || !log_i || !out) return -1;
    if (B <= 0 || H <= 0 || L <= 0 || Dk <= 0 || Dv <= 0) return -1;
    const long BH = B * H;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        double *C = (double *)malloc(sizeof(double) * (size_t)(Dk * Dv));
        double *n = (double *)malloc(sizeof(double) * (size_t)Dk);
        if (!C || !n) {
            free(C);
            free(n);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        if (C0)
            memcpy(C, C0 + bh * Dk * Dv, sizeof(double) * (size_t)(Dk * Dv));
        else
            memset(C, 0, sizeof(double) * (size_t)(Dk * Dv));
        if (n0)
            memcpy(n, n0 + bh * Dk, sizeof(double) * (size_t)Dk);
        else
            memset(n, 0, sizeof(double) * (size_t)Dk);

        for (long t = 0; t < L; ++t) {
            const double *qt = q + (bh * L + t) * Dk;
            const double *kt = k + (bh * L + t) * Dk;
            const double *vt = v + (bh * L + t) * Dv;
            const double ft = exp(log_f[bh * L + t]);
            const double it = exp(log_i[bh * L + t]);
            double *ht = out + (bh * L + t) * Dv;

            /* memory and normaliser: decay, then the token's write */
            for (long d = 0; d < Dk; ++d) {
                double *Cd = C + d * Dv;
                const double w = it * kt[d];
                for (long c = 0; c < Dv; ++c) Cd[c] = ft * Cd[c] + w * vt[c];
                n[d] = ft * n[d] + w;
            }
            /* read: q_t C_t over max(|q_t . n_t|, 1) */
            double qn = 0.0;
            for (long d = 0; d < Dk; ++d) qn += qt[d] * n[d];
            const double den = fabs(qn) > 1.0 ? fabs(qn) : 1.0;
            for (long c = 0; c < Dv; ++c) ht[c] = 0.0;
            for (long d = 0; d < Dk; ++d) {
                const double *Cd = C + d * Dv;
                for (long c = 0; c < Dv; ++c) ht[c] += qt[d] * Cd[c];
            }
            for (long c = 0; c < Dv; ++c) ht[c] /= den;
        }
        if (final_C) memcpy(final_C + bh * Dk * Dv, C, sizeof(double) * (size_t)(Dk * Dv));
        if (final_n) memcpy(final_n + bh * Dk, n, sizeof(double) * (size_t)Dk);
        free(C);
        free(n);
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
