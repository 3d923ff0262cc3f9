// mlstm_kernels.hip -- gfx950 kernel of the mLSTM with exponential input gate and normaliser.
//
// The cell.  The xLSTM's matrix memory (the mLSTM of Beck et al. (2024), to which the Tiled
// Flash Linear Attention abstract applies its kernels; the abstract's sigmoid-gated variant
// drops the normaliser): with f_t = exp(log_f_t) and i_t = exp(log_i_t),
//
//     C_t = f_t C_{t-1} + i_t k_t^T v_t ,   n_t = f_t n_{t-1} + i_t k_t ,
//     h_t = q_t C_t / max(|q_t . n_t|, 1) .
//
// The input gate is unbounded, so memory and normaliser are kept scaled by a running
// maximum m of the log weights: (C', n', m) with C = e^m C' and n = e^m n'; the read is then
// q C' / max(|q . n'|, e^-m), the same value.
//
// Chunkwise form (64 tokens).  A chunk enters with (C', n', m).  In log2 units, with b the
// running sum of the log forget gates inside the chunk and a_s = log_i_s - b_s, token s
// reaches row t >= s with log weight b_t + a_s and the entering state reaches it with
// b_t + m; the row's maximum is m_t = b_t + M_t with M_t = max(m, max_{s<=t} a_s), so every
// factor below is at most 1:
//
//     num_t = 2^(m - M_t) q_t C' + sum_{s<=t} 2^(a_s - M_t) (q_t . k_s) v_s
//     den_t = 2^(m - M_t) q_t . n' + sum_{s<=t} 2^(a_s - M_t) (q_t . k_s)
//     h_t   = num_t / max(|den_t|, 2^(-m_t)) ,
//
// and at the chunk end, with M_e the last row's maximum,
//
//     C' <- 2^(m - M_e) C' + K^T diag(2^(a - M_e)) V ,   n' <- 2^(m - M_e) n' + K^T 2^(a - M_e) ,
//     m  <- b_63 + M_e .
//
// Work split.  One workgroup (4 waves) owns one (batch, head) and one 64-column slice of the
// value dimension and walks the sequence with its Dk x 64 slice of C' in registers (wave w:
// columns 16w..16w+15, in matrix-core accumulator layout) and n' (Dk fp32) in LDS.  Per chunk:
//   1. q, k, k^T, v^T into LDS; wave 0 scans the gates (b, a, M, m_t and the end weights);
//   2. wave w: score row block w, P_ts = 2^(a_s - M_t) q_t . k_s (causal), its row sums and
//      q_t . n', hence den_t; every wave: 2^(m - M_t) q_t C' for its columns;
//   3. O += P V, the division by max(|den|, 2^(-m_t)) and the stores;
//   4. C' on the matrix cores; n' with one channel per thread.
// Row and slot orders of LDS and accumulators are those of gla_rows.h.
//
// Numbers.  bf16 inputs: matrix operands fp16 (q, k, v converted), fp32 accumulation;
// normaliser, maxima and gate arithmetic in fp32.  The state C', the scores P and the
// weighted values of the state update enter their products as an fp16 value plus an fp16
// rounding residual: the read divides by the normaliser, which magnifies a single rounding of
// any of them past 1e-2 of the output's RMS (C' and P at Dk = 256, the weighted values with
// input gates spread over e^(+-12)).  fp32 inputs: fp32 operands.  Outputs and states are fp32.
//
// Rows past the sequence end read as zero through buffer resources; they write nothing (log
// input gate taken as -inf) and do not decay, and their output stores are dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gla.h"
#include "gla_mlstm.h"
#include "gla_rows.h"

namespace gla_mlstm {

using namespace gla_rows;

constexpr float kNone = -1.0e30f;       // log2 weight of nothing (no write, no entering state)
constexpr float kLn2 = 0.6931471805599453f;

// LDS layout (bytes).
struct Plan {
    uint32_t q, k, kt, vt, p, pl, a, mx, mt, wp, den, n, total;
};
__host__ __device__ inline Plan make_plan(bool f32, int dk, int cols) {
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
    off += al((uint32_t)cols * rt * ob);
    p.p = off;  // scores (fp16 value)
    off += al(kC * rt * ob);
    p.pl = off;  // their fp16 rounding residual (fp16 operands only)
    off += f32 ? 0u : al(kC * rt * ob);
    p.a = off;  // a_s by token
    off += al(kC * 4u);
    p.mx = off;  // M_t by token
    off += al(kC * 4u);
    p.mt = off;  // m_t = b_t + M_t by token
    off += al(kC * 4u);
    p.wp = off;  // 2^(a_s - M_e) by slot
    off += al(kC * 4u);
    p.den = off;  // den_t by token
    off += al(kC * 4u);
    p.n = off;  // n' by channel slot
    off += al((uint32_t)dk * 4u);
    p.total = off;
    return p;
}

int wg_cols(bool f32, int dk, int dv) { return !f32 && dk == 256 && dv % 128 == 0 ? 128 : 64; }
uint32_t lds_bytes(bool f32, int dk, int cols) { return make_plan(f32, dk, cols).total; }

__device__ __forceinline__ float scan_max(float x, [[maybe_unused]] int lane) {
    return scan_dpp(x, -__builtin_inff(), [](float u, float v) { return fmaxf(u, v); });
}

// The next chunk's raw pieces plus the two gates of token tid & 63.
template <class C>
struct Pref : Pieces<C> {
    float lf, li;
};

template <class C>
__device__ __forceinline__ void prefetch_rest(Pref<C> &pf, rsrc_t rv, rsrc_t rlf, rsrc_t rli, int T0, int tid, int dv0,
                                              int Dv) {
    prefetch_v<C>(pf.v, rv, T0, tid, dv0, Dv);
    pf.lf = bld_f32(rlf, (uint32_t)(T0 + (tid & 63)) * 4u);
    pf.li = bld_f32(rli, (uint32_t)(T0 + (tid & 63)) * 4u);
}

// The prefetched chunk into LDS, and the gate scans (wave 0, lane = token).
template <class C>
__device__ __forceinline__ void stage(const Pref<C> &pf, unsigned char *smem, const Plan &lp, int tid, int lane,
                                      int w, bool row_valid_lane, float m_in) {
    using OpT = typename C::OpT;
    stage_rows<C>(pf, reinterpret_cast<OpT *>(smem + lp.q), reinterpret_cast<OpT *>(smem + lp.k),
                  reinterpret_cast<OpT *>(smem + lp.kt), reinterpret_cast<OpT *>(smem + lp.vt), tid);
    if (w == 0) {
        const float x = row_valid_lane ? log2_decay(pf.lf) : 0.f;
        const float b = scan_incl(x, lane);
        const float a = row_valid_lane ? pf.li * kLog2e - b : kNone;
        const float M = fmaxf(scan_max(a, lane), m_in);
        const float Me = lane_bcast(M, 63);
        reinterpret_cast<float *>(smem + lp.a)[lane] = a;
        reinterpret_cast<float *>(smem + lp.mx)[lane] = M;
        reinterpret_cast<float *>(smem + lp.mt)[lane] = b + M;
        reinterpret_cast<float *>(smem + lp.wp)[perm(lane)] = fexp2(a - Me);
    }
}

// Score row block W: P_ts = 2^(a_s - M_t) (q_t . k_s) for s <= t (t = 16 W + c), written in
// slot order (fp16 operands: its fp16 value and, in a second array, the rounding residual);
// the products take a key block as A operand and the query block as B operand, so lane
// (g, c) holds four consecutive keys of row t.  Also the row sums of P and
// q_t . n' (lanes of a row split the channels in four), hence den_t.  The zero blocks of P
// that the value product reads (P[0][1] and P[2][3]) are written too.
template <class C, int W>
__device__ __forceinline__ void scores(const typename C::OpT *sQ, const typename C::OpT *sK, typename C::OpT *sP,
                                       typename C::OpT *sPl, const float *sA, const float *sMx, const float *sN,
                                       float *sDen, float m_in, int g, int c16) {
    using Frag = typename C::Frag;
    constexpr int NJ = W + 1;
    f32x4 qk[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) qk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < C::NM; ++m) {
        Frag ka[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) ka[j] = ld_frag<C>(sK + (16 * j + c16) * C::RQ + 32 * m + 8 * g);
        const Frag bq = ld_frag<C>(sQ + (16 * W + c16) * C::RQ + 32 * m + 8 * g);
#pragma unroll
        for (int j = 0; j < NJ; ++j) qk[j] = mma(ka[j], bq, qk[j]);
    }
    const int t = 16 * W + c16;
    const float Mt = sMx[t];
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const f32x4 as = *reinterpret_cast<const f32x4 *>(sA + 16 * j + 4 * g);
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = 16 * j + 4 * g + e <= t ? fexp2(as[e] - Mt) * qk[j][e] : 0.f;
            rs += x[e];
        }
        store_quad<C>(sP + t * C::RT + perm(16 * j + 4 * g), x[0], x[1], x[2], x[3]);
        if constexpr (!C::F32) {
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = x[e] - (float)(f16)x[e];
            store_quad<C>(sPl + t * C::RT + perm(16 * j + 4 * g), r[0], r[1], r[2], r[3]);
        }
    }
    if constexpr (W == 0 || W == 2) {
        store_quad<C>(sP + t * C::RT + perm(16 * (W + 1) + 4 * g), 0.f, 0.f, 0.f, 0.f);
        if constexpr (!C::F32) store_quad<C>(sPl + t * C::RT + perm(16 * (W + 1) + 4 * g), 0.f, 0.f, 0.f, 0.f);
    }
    // q_t . n' over the channel slots [g DK/4, (g + 1) DK/4)
    float qn = 0.f;
#pragma unroll
    for (int u = 0; u < C::DK / 32; ++u) {
        const int c0 = g * (C::DK / 4) + 8 * u;
        const Frag qf = ld_frag<C>(sQ + t * C::RQ + c0);
        const f32x4 n0 = *reinterpret_cast<const f32x4 *>(sN + c0);
        const f32x4 n1 = *reinterpret_cast<const f32x4 *>(sN + c0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) qn += (float)qf[e] * n0[e] + (float)qf[e + 4] * n1[e];
    }
    rs = add_xor32(add_xor16(rs));
    qn = add_xor32(add_xor16(qn));
    if (g == 0) sDen[t] = fexp2(m_in - Mt) * qn + rs;
}

template <class C>
__global__ __launch_bounds__(C::NT, 1) void mlstm_chunk_kernel(MlstmArgs a) {
    using OpT = typename C::OpT;
    using Frag = typename C::Frag;
    extern __shared__ __align__(256) unsigned char smem[];
    constexpr int NCOL = C::NT / 4;  // value columns of the workgroup, 16 per wave
    const Plan lp = make_plan(C::F32, C::DK, NCOL);
    const OpT *sQ = reinterpret_cast<const OpT *>(smem + lp.q);
    const OpT *sK = reinterpret_cast<const OpT *>(smem + lp.k);
    const OpT *sKt = reinterpret_cast<const OpT *>(smem + lp.kt);
    const OpT *sVt = reinterpret_cast<const OpT *>(smem + lp.vt);
    OpT *sP = reinterpret_cast<OpT *>(smem + lp.p);
    OpT *sPl = reinterpret_cast<OpT *>(smem + lp.pl);
    const float *sA = reinterpret_cast<const float *>(smem + lp.a);
    const float *sMx = reinterpret_cast<const float *>(smem + lp.mx);
    const float *sMt = reinterpret_cast<const float *>(smem + lp.mt);
    const float *sWp = reinterpret_cast<const float *>(smem + lp.wp);
    float *sDen = reinterpret_cast<float *>(smem + lp.den);
    float *sN = reinterpret_cast<float *>(smem + lp.n);

    const int id = xcd_remap((int)blockIdx.x, (int)gridDim.x);
    const int dvt = id % a.ndv;
    const int bh = id / a.ndv;
    const int dv0 = dvt * NCOL;
    // the wave index in a scalar register: the score products below run on some waves only,
    // and a matrix-core instruction does not look at the execution mask
    const int tid = (int)threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4,
              c16 = lane & 15;
    const int L = a.L, Dv = a.Dv;
    const size_t bhL = (size_t)bh * L;

    const rsrc_t rq = make_rsrc(reinterpret_cast<const char *>(a.q) + bhL * C::DK * C::IB, (uint64_t)L * C::DK * C::IB);
    const rsrc_t rk = make_rsrc(reinterpret_cast<const char *>(a.k) + bhL * C::DK * C::IB, (uint64_t)L * C::DK * C::IB);
    const rsrc_t rv = make_rsrc(reinterpret_cast<const char *>(a.v) + bhL * Dv * C::IB, (uint64_t)L * Dv * C::IB);
    const rsrc_t rlf = make_rsrc(a.lf + bhL, (uint64_t)L * 4);
    const rsrc_t rli = make_rsrc(a.li + bhL, (uint64_t)L * 4);
    const rsrc_t rout = make_rsrc(a.out + bhL * Dv, (uint64_t)L * Dv * 4);

    // this wave's slice of C': rows 16r+4g+e, column dv0 + 16w + c16; n' in LDS by slot
    f32x4 S[C::NB];
    const int col = dv0 + 16 * w + c16;
#pragma unroll
    for (int r = 0; r < C::NB; ++r) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[r][e] = a.c0 ? a.c0[((size_t)bh * C::DK + 16 * r + 4 * g + e) * Dv + col] : 0.f;
    }
    if (tid < C::DK) sN[perm(tid)] = a.n0 ? a.n0[(size_t)bh * C::DK + tid] : 0.f;
    float m_in = a.m0 ? a.m0[bh] * kLog2e : kNone;  // log2 maximum of the entering state

    Pref<C> pf;
    prefetch_rows<C>(pf.q, rq, 0, tid);
    prefetch_rows<C>(pf.k, rk, 0, tid);
    prefetch_rest<C>(pf, rv, rlf, rli, 0, tid, dv0, Dv);
    const int nc = (L + kC - 1) / kC;
    for (int ci = 0; ci < nc; ++ci) {
        const int T0 = ci * kC;
        stage<C>(pf, smem, lp, tid, lane, w, T0 + lane < L, m_in);
        barrier();  // B1: chunk staged, gates scanned
        prefetch_rows<C>(pf.q, rq, T0 + kC, tid);

        switch (w) {
            case 0: scores<C, 0>(sQ, sK, sP, sPl, sA, sMx, sN, sDen, m_in, g, c16); break;
            case 1: scores<C, 1>(sQ, sK, sP, sPl, sA, sMx, sN, sDen, m_in, g, c16); break;
            case 2: scores<C, 2>(sQ, sK, sP, sPl, sA, sMx, sN, sDen, m_in, g, c16); break;
            case 3: scores<C, 3>(sQ, sK, sP, sPl, sA, sMx, sN, sDen, m_in, g, c16); break;
            default: break;  // waves 4..7 of an eight-wave workgroup
        }
        prefetch_rows<C>(pf.k, rk, T0 + kC, tid);

        // the entering state's share of the output, 2^(m - M_t) q_t C', for this wave's columns;
        // C' enters as its fp16 value plus the rounding residual (the read divides by the
        // normaliser, which magnifies one rounding of the state past the bar)
        f32x4 O[4];
        {
            const f32x4 one = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < C::NM; ++m) {
                const Frag sf = acc_frag<C>(S[2 * m], S[2 * m + 1]);
                Frag qa[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) qa[i] = ld_frag<C>(sQ + (16 * i + c16) * C::RQ + 32 * m + 8 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) O[i] = mma(qa[i], sf, O[i]);
                if constexpr (!C::F32) {
                    const Frag sr = residual<C>(S[2 * m], S[2 * m + 1], sf, one, one);
#pragma unroll
                    for (int i = 0; i < 4; ++i) O[i] = mma(qa[i], sr, O[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 mx = *reinterpret_cast<const f32x4 *>(sMx + 16 * i + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) O[i][e] *= fexp2(m_in - mx[e]);
            }
        }
        barrier();  // B2: P and den complete
        prefetch_rest<C>(pf, rv, rlf, rli, T0 + kC, tid, dv0, Dv);

        // ---- O += P V, divided by max(|den|, 2^(-m_t)), stored
        Frag vb[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) vb[m] = ld_frag<C>(sVt + (16 * w + c16) * C::RT + 32 * m + 8 * g);
        {
            // token blocks 2 and 3 (m = 1) do not reach query blocks 0 and 1
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int i = 2 * m; i < 4; ++i) {
                    const Frag pa = ld_frag<C>(sP + (16 * i + c16) * C::RT + 32 * m + 8 * g);
                    O[i] = mma(pa, vb[m], O[i]);
                    if constexpr (!C::F32) {
                        const Frag pr = ld_frag<C>(sPl + (16 * i + c16) * C::RT + 32 * m + 8 * g);
                        O[i] = mma(pr, vb[m], O[i]);
                    }
                }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 dn = *reinterpret_cast<const f32x4 *>(sDen + 16 * i + 4 * g);
                const f32x4 mt = *reinterpret_cast<const f32x4 *>(sMt + 16 * i + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float h = O[i][e] / fmaxf(fabsf(dn[e]), fexp2(-mt[e]));
                    bst_f32(h, rout, ((uint32_t)(T0 + 16 * i + 4 * g + e) * Dv + col) * 4u);
                }
            }
        }
        // ---- C' <- 2^(m - M_e) C' + K^T diag(2^(a - M_e)) V ;  n' likewise
        const float esc = fexp2(m_in - sMx[kC - 1]);
        {
#pragma unroll
            for (int r = 0; r < C::NB; ++r) S[r] *= esc;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const f32x4 w0 = *reinterpret_cast<const f32x4 *>(sWp + 32 * m + 8 * g);
                const f32x4 w1 = *reinterpret_cast<const f32x4 *>(sWp + 32 * m + 8 * g + 4);
                Frag wv, wr;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = (float)vb[m][e] * w0[e], x1 = (float)vb[m][e + 4] * w1[e];
                    wv[e] = (OpT)x0;
                    wv[e + 4] = (OpT)x1;
                    wr[e] = (OpT)(x0 - (float)wv[e]);
                    wr[e + 4] = (OpT)(x1 - (float)wv[e + 4]);
                }
                // k^T fragments four state blocks at a time (bounds the live registers)
#pragma unroll
                for (int r0 = 0; r0 < C::NB; r0 += 4) {
                    Frag ka[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        ka[r] = ld_frag<C>(sKt + (16 * (r0 + r) + c16) * C::RT + kt_col(16 * (r0 + r) + c16, 32 * m + 8 * g));
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[r0 + r] = mma(ka[r], wv, S[r0 + r]);
                    if constexpr (!C::F32) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) S[r0 + r] = mma(ka[r], wr, S[r0 + r]);
                    }
                }
            }
        }
        if (tid < C::DK) {
            float acc = 0.f;
#pragma unroll
            for (int G = 0; G < 8; ++G) {
                const Frag kf = ld_frag<C>(sKt + tid * C::RT + kt_col(tid, 8 * G));
                const f32x4 w0 = *reinterpret_cast<const f32x4 *>(sWp + 8 * G);
                const f32x4 w1 = *reinterpret_cast<const f32x4 *>(sWp + 8 * G + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc += (float)kf[e] * w0[e] + (float)kf[e + 4] * w1[e];
            }
            const int pd = perm(tid);
            sN[pd] = esc * sN[pd] + acc;
        }
        m_in = sMt[kC - 1];
        barrier();  // B3: the chunk's LDS may be overwritten
    }

    if (a.fin_c) {
#pragma unroll
        for (int r = 0; r < C::NB; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.fin_c[((size_t)bh * C::DK + 16 * r + 4 * g + e) * Dv + col] = S[r][e];
    }
    if (dvt == 0) {
        if (a.fin_n && tid < C::DK) a.fin_n[(size_t)bh * C::DK + tid] = sN[perm(tid)];
        if (a.fin_m && tid == 0) a.fin_m[bh] = m_in * kLn2;
    }
}

template <class C>
static hipError_t launch_cfg(const MlstmArgs &a, hipStream_t st) {
    static std::atomic<uint64_t> done{0};
    const uint32_t lds = lds_bytes(C::F32, C::DK, C::NT / 4);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = 1ull << (dev & 63);
    if (!(done.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&mlstm_chunk_kernel<C>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        done.fetch_or(bit, std::memory_order_acq_rel);
    }
    hipLaunchKernelGGL(mlstm_chunk_kernel<C>, dim3((unsigned)a.nwg), dim3(C::NT), lds, st, a);
    return hipGetLastError();
}

hipError_t launch(const MlstmArgs &a, bool f32, int dk, hipStream_t st) {
    if (f32) {
        if (dk == 64) return launch_cfg<Cfg<true, 64>>(a, st);
        return hipErrorInvalidValue;
    }
    if (dk == 64) return launch_cfg<Cfg<false, 64>>(a, st);
    if (dk == 128) return launch_cfg<Cfg<false, 128>>(a, st);
    if (dk == 256)
        return a.Dv / a.ndv == 128 ? launch_cfg<Cfg<false, 256, 512>>(a, st) : launch_cfg<Cfg<false, 256>>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace gla_mlstm
