// delta_kernels.hip -- gfx950 kernel of the chunkwise delta rule (DeltaNet and Gated DeltaNet).
//
// The update.  Each token takes one gradient step of size beta_t on the squared error of
// predicting v_t from k_t, with the state as a fast weight, after the previous state is
// decayed by a scalar gate alpha_t (1 for DeltaNet) [Hardware-Efficient Training of Linear
// Attention Models, talk summary, 22:36 and 31:16]:
//
//     S_t = alpha_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t ,     o_t = q_t S_t .
//
// Chunkwise form.  The transition is identity plus rank one; its product over a chunk is
// carried by the WY representation, which turns it into sums so that the chunkwise
// algorithm runs on matrix products [same talk, 31:16 and 11:58].  For a chunk of 64 tokens
// entering with state S0, with b the running log decay inside the chunk and g = 2^b:
//
//     A   = strictly lower part of  diag(beta) [g_t / g_s] (K K^T)
//     U   = (I + A)^-1 diag(beta) (V - diag(g) K S0)     (the tokens' corrections u_t)
//     O   = diag(g) Q S0  +  ((Q K^T) * [g_t / g_s]_{s<=t}) U
//     S1  = g_63 S0  +  K^T diag(g_63 / g) U .
//
// u_t = beta_t (v_t - alpha_t k_t S_{t-1}) is the step each token takes; unrolled over the
// chunk the u_t satisfy (I + A) U = diag(beta) (V - diag(g) K S0), which is where the
// triangular system comes from.  Every decay ratio that appears is g_t / g_s with s <= t,
// at most 1.
//
// Work split.  One workgroup (4 waves) owns one (batch, head) and one 64-column slice of
// the value dimension, and walks the sequence chunk by chunk with its Dk x 64 slice of the
// state in registers (wave w: columns 16w..16w+15, in matrix-core accumulator layout).  Per
// chunk:
//   1. the chunk's q, k (rows, and k transposed), v (transposed), beta and gates into LDS;
//   2. K K^T -> A and Q K^T -> P (masked, decayed), and Q S0 (the state's share of O);
//   3. the diagonal 16x16 blocks D_i of I + A inverted (fp32, vector ALU);
//   4. U = (I + A)^-1 R with R = diag(beta) (V - diag(g) K S0), by block forward
//      substitution over the four 16-token blocks, U_i = D_i (R_i - sum_{k<i} A_ik U_k), on
//      the matrix cores for the wave's own 16 columns (N is never formed);
//   5. O += P U, S1 = g_63 S0 + K^T diag(g_63 / g) U.
// The accumulator layout of the state (lane (g, c) holds rows 4g+e of each 16-row block,
// column c) doubles as the B operand of the products that contract over the state's rows,
// once the contraction index is ordered so that k-slot 8g+j of a 32-deep step is row
// 4g+j (j < 4) or 16+4g+j-4 (j >= 4) of the step's 32 rows; the same order is used for
// tokens, so U feeds P U and K^T U straight from registers.  Channel rows (q, k, W) and
// token rows (P, N, K^T, V^T) are stored in LDS in that order.
//
// Numbers.  bf16 inputs: matrix operands fp16 (q, k, v converted; computed operands rounded
// once), fp32 accumulation; the triangular solve of the diagonal blocks is fp32.  The
// corrections U enter the output product (and the right-hand side of each substitution step
// its product) as an fp16 value plus an fp16 rounding residual: the output is a small
// difference of terms of the size of U, so one rounding of U would dominate its error.  The
// state update takes U rounded once.  fp32 inputs: fp32 operands
// throughout.  States, decays and outputs are fp32.
//
// Rows past the sequence end read as zero through buffer resources (k = v = beta = 0 and
// no decay: such a token changes nothing) and their output stores are dropped.
#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include <atomic>

#include "gla.h"
#include "gla_delta.h"
#include "gla_rows.h"

namespace gla_delta {

using namespace gla_rows;

constexpr int kAR = 68;                  // fp32 row stride of the A / N matrix in LDS

// LDS layout (bytes).
struct Plan {
    uint32_t q, k, kt, vt, p, a, b, be, total;
};
__host__ __device__ inline Plan make_plan(bool f32, int dk) {
    const uint32_t ob = f32 ? 4u : 2u;
    const uint32_t rq = (uint32_t)dk + 16u / ob, rt = (uint32_t)kC + 16u / ob;
    auto al = [](uint32_t x) { return (x + 255u) & ~255u; };
    Plan p{};
    uint32_t off = 0;
    p.q = off;
    off += al(kC * rq * ob);
    p.k = off;
    off += al(kC * rq * ob);
    p.kt = off;
    off += al((uint32_t)dk * rt * ob);
    p.vt = off;
    off += al(64u * rt * ob);
    p.p = off;
    off += al(kC * rt * ob);
    p.a = off;
    off += al(kC * kAR * 4u);
    p.b = off;
    off += al(kC * 4u);
    p.be = off;
    off += al(kC * 4u);
    p.total = off;
    return p;
}

uint32_t lds_bytes(bool f32, int dk) { return make_plan(f32, dk).total; }

// The next chunk's raw pieces plus the beta and gate of token tid & 63.  Its loads are
// issued in three groups (q rows, k rows, then v, beta and the gate) at different points of
// the current chunk, so that their issue overlaps the work in between instead of stalling
// the waves in one block.
template <class C>
struct Pref : Pieces<C> {
    float beta, la;
};

template <class C>
__device__ __forceinline__ void prefetch_rest(Pref<C> &pf, rsrc_t rv, rsrc_t rb, rsrc_t rla, uint32_t gstride,
                                              int T0, int tid, int dv0, int Dv) {
    prefetch_v<C>(pf.v, rv, T0, tid, dv0, Dv);
    pf.beta = bld_f32(rb, (uint32_t)(T0 + (tid & 63)) * 4u);
    pf.la = bld_f32(rla, (uint32_t)(T0 + (tid & 63)) * gstride);
}

// The prefetched chunk into LDS: q, k, k^T and v^T rows, then beta and the running log2
// decay (wave 0).
template <class C>
__device__ __forceinline__ void stage(const Pref<C> &pf, unsigned char *smem, const Plan &lp, int tid, int lane,
                                      int w, bool row_valid_lane) {
    using OpT = typename C::OpT;
    stage_rows<C>(pf, reinterpret_cast<OpT *>(smem + lp.q), reinterpret_cast<OpT *>(smem + lp.k),
                  reinterpret_cast<OpT *>(smem + lp.kt), reinterpret_cast<OpT *>(smem + lp.vt), tid);
    if (w == 0) {
        float *sB = reinterpret_cast<float *>(smem + lp.b);
        float *sBe = reinterpret_cast<float *>(smem + lp.be);
        const float x = row_valid_lane ? log2_decay(pf.la) : 0.f;
        sB[lane] = scan_incl(x, lane);
        sBe[lane] = row_valid_lane ? pf.beta : 0.f;
    }
}

// Score blocks of wave W: row block W of A and row block 3-W of P, blocks on or below the
// diagonal only.  Each product has a key block as its A operand and the row block (keys for
// A, queries for P) as its B operand, so the accumulator of lane (g, c) holds four
// consecutive key positions s = 16j + 4g + e of one row t = 16 W' + c: a row segment of A
// or P, written with one vector store.  A: t = 16 W + c, A[t][s] = beta_t 2^(b_t - b_s)
// (K K^T)[t][s] for s < t.  P: t = 16 (3 - W) + c, P[t][s] = 2^(b_t - b_s) (Q K^T)[t][s] for
// s <= t, with the key positions in slot order; the zero blocks of P that the output
// product reads (P[0][1] and P[2][3]) are written too.
template <class C, int W>
__device__ __forceinline__ void scores(const typename C::OpT *sQ, const typename C::OpT *sK, typename C::OpT *sP,
                                       float *sA, const float *sB, const float *sBe, int g, int c16) {
    using Frag = typename C::Frag;
    using OpT = typename C::OpT;
    constexpr int IQ = 3 - W;
    constexpr int NK = W + 1, NQ = IQ + 1;
    constexpr int NJ = NK > NQ ? NK : NQ;
    f32x4 kk[NK], qk[NQ];
#pragma unroll
    for (int j = 0; j < NK; ++j) kk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NQ; ++j) qk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < C::NM; ++m) {
        Frag ka[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) ka[j] = ld_frag<C>(sK + (16 * j + c16) * C::RQ + 32 * m + 8 * g);
        const Frag bq = ld_frag<C>(sQ + (16 * IQ + c16) * C::RQ + 32 * m + 8 * g);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (j < NK) kk[j] = mma(ka[j], ka[W], kk[j]);
            if (j < NQ) qk[j] = mma(ka[j], bq, qk[j]);
        }
    }
    {
        const int t = 16 * W + c16;
        const float bt = sB[t], bet = sBe[t];
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const f32x4 bs = *reinterpret_cast<const f32x4 *>(sB + 16 * j + 4 * g);
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = 16 * j + 4 * g + e < t ? bet * fexp2(bt - bs[e]) * kk[j][e] : 0.f;
            *reinterpret_cast<f32x4 *>(sA + t * kAR + 16 * j + 4 * g) = x;
        }
    }
    {
        const int t = 16 * IQ + c16;
        const float bt = sB[t];
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const f32x4 bs = *reinterpret_cast<const f32x4 *>(sB + 16 * j + 4 * g);
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = 16 * j + 4 * g + e <= t ? fexp2(bt - bs[e]) * qk[j][e] : 0.f;
            store_quad<C>(sP + t * C::RT + perm(16 * j + 4 * g), x[0], x[1], x[2], x[3]);
        }
        if constexpr (IQ == 0 || IQ == 2) store_quad<C>(sP + t * C::RT + perm(16 * (IQ + 1) + 4 * g), 0.f, 0.f, 0.f, 0.f);
    }
}

template <class C>
__global__ __launch_bounds__(256, 1) void delta_chunk_kernel(DeltaArgs a) {
    using OpT = typename C::OpT;
    using Frag = typename C::Frag;
    using Quad = typename C::Quad;
    extern __shared__ __align__(256) unsigned char smem[];
    const Plan lp = make_plan(C::F32, C::DK);
    const OpT *sQ = reinterpret_cast<const OpT *>(smem + lp.q);
    const OpT *sK = reinterpret_cast<const OpT *>(smem + lp.k);
    const OpT *sKt = reinterpret_cast<const OpT *>(smem + lp.kt);
    const OpT *sVt = reinterpret_cast<const OpT *>(smem + lp.vt);
    OpT *sP = reinterpret_cast<OpT *>(smem + lp.p);
    float *sA = reinterpret_cast<float *>(smem + lp.a);
    const float *sB = reinterpret_cast<const float *>(smem + lp.b);
    const float *sBe = reinterpret_cast<const float *>(smem + lp.be);

    const int id = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int dvt = id % a.ndv;
    const int bh = id / a.ndv;
    const int h = bh % a.H;
    const int dv0 = dvt * 64;
    const int tid = (int)threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int L = a.L, Dv = a.Dv;
    const size_t bhL = (size_t)bh * L;

    const rsrc_t rq = make_rsrc(reinterpret_cast<const char *>(a.q) + bhL * C::DK * C::IB, (uint64_t)L * C::DK * C::IB);
    const rsrc_t rk = make_rsrc(reinterpret_cast<const char *>(a.k) + bhL * C::DK * C::IB, (uint64_t)L * C::DK * C::IB);
    const rsrc_t rv = make_rsrc(reinterpret_cast<const char *>(a.v) + bhL * Dv * C::IB, (uint64_t)L * Dv * C::IB);
    const rsrc_t rb = make_rsrc(a.beta + bhL, (uint64_t)L * 4);
    rsrc_t rla;
    uint32_t gstride = 4u;
    if (a.gate == GLA_GATE_HEAD) {
        rla = make_rsrc(a.la + bhL, (uint64_t)L * 4);
    } else if (a.gate == GLA_GATE_HEAD_CONST) {
        rla = make_rsrc(a.la + h, 4);
        gstride = 0u;
    } else {
        rla = make_rsrc(a.out, 0);  // reads return zero: no decay
    }
    const rsrc_t rout = make_rsrc(a.out + bhL * Dv, (uint64_t)L * Dv * 4);

    // this wave's slice of the state: rows 16r+4g+e, column dv0 + 16w + c16
    f32x4 S[C::NB];
    const int col = dv0 + 16 * w + c16;
#pragma unroll
    for (int r = 0; r < C::NB; ++r) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[r][e] = a.s0 ? a.s0[((size_t)bh * C::DK + 16 * r + 4 * g + e) * Dv + col] : 0.f;
    }

    Pref<C> pf;
    prefetch_rows<C>(pf.q, rq, 0, tid);
    prefetch_rows<C>(pf.k, rk, 0, tid);
    prefetch_rest<C>(pf, rv, rb, rla, gstride, 0, tid, dv0, Dv);
    const int nc = (L + kC - 1) / kC;
    for (int ci = 0; ci < nc; ++ci) {
        const int T0 = ci * kC;
        stage<C>(pf, smem, lp, tid, lane, w, T0 + lane < L);
        barrier();  // B1: chunk staged
        prefetch_rows<C>(pf.q, rq, T0 + kC, tid);

        // ---- products that do not need the triangular solve: A (row block w) and P (row
        // block 3-w), only their blocks on or below the diagonal (five per wave)
        switch (w) {
            case 0: scores<C, 0>(sQ, sK, sP, sA, sB, sBe, g, c16); break;
            case 1: scores<C, 1>(sQ, sK, sP, sA, sB, sBe, g, c16); break;
            case 2: scores<C, 2>(sQ, sK, sP, sA, sB, sBe, g, c16); break;
            default: scores<C, 3>(sQ, sK, sP, sA, sB, sBe, g, c16); break;
        }
        prefetch_rows<C>(pf.k, rk, T0 + kC, tid);
        // the state's share of the output, diag(g) Q S0, and the right-hand side of the
        // triangular system, R = diag(beta) (V - diag(g) K S0), for this wave's 16 columns
        f32x4 O[4], R[4];
        {
            Frag sf[C::NM];
#pragma unroll
            for (int m = 0; m < C::NM; ++m) sf[m] = acc_frag<C>(S[2 * m], S[2 * m + 1]);
            f32x4 ks[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) O[i] = ks[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < C::NM; ++m) {
                Frag qa[4], ka[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qa[i] = ld_frag<C>(sQ + (16 * i + c16) * C::RQ + 32 * m + 8 * g);
                    ka[i] = ld_frag<C>(sK + (16 * i + c16) * C::RQ + 32 * m + 8 * g);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    O[i] = mma(qa[i], sf[m], O[i]);
                    ks[i] = mma(ka[i], sf[m], ks[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const Quad vq = *reinterpret_cast<const Quad *>(sVt + (16 * w + c16) * C::RT + perm(16 * i + 4 * g));
                const f32x4 bt = *reinterpret_cast<const f32x4 *>(sB + 16 * i + 4 * g);
                const f32x4 be = *reinterpret_cast<const f32x4 *>(sBe + 16 * i + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float gt = fexp2(bt[e]);
                    O[i][e] *= gt;
                    R[i][e] = be[e] * ((float)vq[e] - gt * ks[i][e]);
                }
            }
        }
        barrier();  // B2: A and P complete

        // ---- diagonal blocks of I + A inverted (wave w: block w), right-looking over four
        // 4-row groups: lane (g, c16) holds rows 4g..4g+3 of column c16; group bg solves its
        // 4x4 diagonal piece, hands its rows to the groups below (cross-lane reads) and they
        // subtract their A entries times those rows.
        {
            float *blk = sA + (16 * w) * kAR + 16 * w;
            f32x4 ar[4][4];  // ar[bg][e] = A[4g+e][4bg..4bg+3] of this block
#pragma unroll
            for (int bg = 0; bg < 4; ++bg)
#pragma unroll
                for (int e = 0; e < 4; ++e) ar[bg][e] = *reinterpret_cast<const f32x4 *>(blk + (4 * g + e) * kAR + 4 * bg);
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (4 * g + e == c16) ? 1.f : 0.f;
            const auto step = [&](auto bgc) {
                constexpr int bg = decltype(bgc)::value;
                if (g == bg) {
#pragma unroll
                    for (int e = 1; e < 4; ++e)
#pragma unroll
                        for (int j = 0; j < e; ++j) x[e] -= ar[bg][e][j] * x[j];
                }
                float xb[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) xb[j] = row_to_all<bg>(x[j]);
                if (g > bg) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int j = 0; j < 4; ++j) x[e] -= ar[bg][e][j] * xb[j];
                }
            };
            step(std::integral_constant<int, 0>{});
            step(std::integral_constant<int, 1>{});
            step(std::integral_constant<int, 2>{});
            step(std::integral_constant<int, 3>{});
#pragma unroll
            for (int e = 0; e < 4; ++e) blk[(4 * g + e) * kAR + c16] = x[e];
        }
        barrier();  // B3: diagonal inverses D_i in place
        prefetch_rest<C>(pf, rv, rb, rla, gstride, T0 + kC, tid, dv0, Dv);

        // ---- U = (I + A)^-1 R by block forward substitution over the four 16-token blocks:
        // U_i = D_i (R_i - sum_{k<i} A_ik U_k); accumulators serve as B operands directly
        f32x4 U[4];
        {
            f32x4 ab[4][4];  // ab[i][k] = row c16 of block (i, k), columns 4g..4g+3 (k < i: -A_ik; k = i: D_i)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int k = 0; k <= i; ++k) {
                    const f32x4 x = *reinterpret_cast<const f32x4 *>(sA + (16 * i + c16) * kAR + 16 * k + 4 * g);
                    ab[i][k] = k < i ? -x : x;
                }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 acc = R[i];
#pragma unroll
                for (int k = 0; k < i; ++k) acc = mma16<C::F32>(ab[i][k], U[k], acc);
                U[i] = mma16<C::F32>(ab[i][i], acc, f32x4{0.f, 0.f, 0.f, 0.f});
                if constexpr (!C::F32) {
                    // the right-hand side enters as fp16 twice: its value and its rounding
                    // residual (an independent product, added after)
                    f32x4 res;
#pragma unroll
                    for (int e = 0; e < 4; ++e) res[e] = acc[e] - (float)(f16)acc[e];
                    U[i] += mma16<C::F32>(ab[i][i], res, f32x4{0.f, 0.f, 0.f, 0.f});
                }
            }
        }
        // ---- O += P U, stored
        {
            // U enters as its fp16 value plus the rounding residual (the output is a small
            // difference of terms of the size of U)
            const f32x4 one = {1.f, 1.f, 1.f, 1.f};
            Frag uf[2], ur[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                uf[m] = acc_frag<C>(U[2 * m], U[2 * m + 1]);
                ur[m] = residual<C>(U[2 * m], U[2 * m + 1], uf[m], one, one);
            }
            Frag pa[4][2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    if (i >= 2 * m) pa[i][m] = ld_frag<C>(sP + (16 * i + c16) * C::RT + 32 * m + 8 * g);
            // token blocks 2 and 3 (m = 1) do not reach query blocks 0 and 1
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int i = 2 * m; i < 4; ++i) O[i] = mma(pa[i][m], uf[m], O[i]);
            if constexpr (!C::F32) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int i = 2 * m; i < 4; ++i) O[i] = mma(pa[i][m], ur[m], O[i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    bst_f32(O[i][e], rout, ((uint32_t)(T0 + 16 * i + 4 * g + e) * Dv + col) * 4u);
        }
        // ---- S1 = g_63 S0 + K^T diag(g_63 / g) U
        {
            const float bC = sB[kC - 1];
            const float gC = fexp2(bC);
            f32x4 f[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) f[i][e] = fexp2(bC - sB[16 * i + 4 * g + e]);
            // the state's increment takes U rounded once: unlike the output, it is not a
            // small difference of larger terms
            Frag ub[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) ub[m] = acc_frag_rows<C>(U[2 * m], U[2 * m + 1], f[2 * m], f[2 * m + 1]);
#pragma unroll
            for (int r = 0; r < C::NB; ++r) S[r] *= gC;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                Frag ka[C::NB];
#pragma unroll
                for (int r = 0; r < C::NB; ++r)
                    ka[r] = ld_frag<C>(sKt + (16 * r + c16) * C::RT + kt_col(16 * r + c16, 32 * m + 8 * g));
#pragma unroll
                for (int r = 0; r < C::NB; ++r) S[r] = mma(ka[r], ub[m], S[r]);
            }
        }
        barrier();  // B4: the chunk's LDS may be overwritten
    }

    if (a.fin) {
#pragma unroll
        for (int r = 0; r < C::NB; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.fin[((size_t)bh * C::DK + 16 * r + 4 * g + e) * Dv + col] = S[r][e];
    }
}

template <class C>
static hipError_t launch_cfg(const DeltaArgs &a, hipStream_t st) {
    static std::atomic<uint64_t> done{0};
    const uint32_t lds = lds_bytes(C::F32, C::DK);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = 1ull << (dev & 63);
    if (!(done.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&delta_chunk_kernel<C>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        done.fetch_or(bit, std::memory_order_acq_rel);
    }
    hipLaunchKernelGGL(delta_chunk_kernel<C>, dim3((unsigned)a.nwg), dim3(256), lds, st, a);
    return hipGetLastError();
}

hipError_t launch(const DeltaArgs &a, bool f32, int dk, hipStream_t st) {
    if (f32) {
        if (dk == 64) return launch_cfg<Cfg<true, 64>>(a, st);
        return hipErrorInvalidValue;
    }
    if (dk == 64) return launch_cfg<Cfg<false, 64>>(a, st);
    if (dk == 128) return launch_cfg<Cfg<false, 128>>(a, st);
    if (dk == 256) return launch_cfg<Cfg<false, 256>>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace gla_delta
