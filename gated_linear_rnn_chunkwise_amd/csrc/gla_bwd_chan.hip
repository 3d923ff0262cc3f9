// gla_bwd_chan.hip -- the backward pass (gla_bwd) with per-channel gates.
//
// The three passes of the scalar-gate backward (gla_bwd.hip) carry over: with R the
// reversal of token order and a' the reversed gate (a'_u = log alpha_{L-u}, a'_0 = 0),
//
//   dv = i . R(F_key(q = R(k), k = R(q), v = R(dout), gate a', S0 = dfinal))
//   dk = i . R(F_val(q = R(v), k = R(dout), v = R(q), gate a', S0 = dfinal^T))
//   dq =        F_val(q = dout, k = v, v = i k, gate alpha, S0 = initial^T)
//
// but with a per-channel gate the last two need the decay on the value dimension of their
// state: F_val runs S_t = S_{t-1} diag(gamma_t) + k_t^T v_t, o_t = q_t S_t, where F_key is
// the forward recurrence S_t = diag(gamma_t) S_{t-1} + k_t^T v_t.  chan_pass_kernel computes
// both in fp32 over 16-token blocks from running log2 decays b_t: every decay factor
// 2^(b_t - b_s) <= 1 is either split into two factors bounded by 2^60 (while the block's
// decay stays above 2^-60) or formed exactly, and the state is carried from block to block
// and across sequence segments.  Reversal, the input gate of the values and the output row
// mapping are index arithmetic on the caller's tensors, so the passes need no operand copies.
//
// With bf16 inputs the value-gated passes run on fp16 operands (chan_vg16_kernel), and fp32
// inputs keep them in chan_pass_kernel.
//
// The per-channel log-gate gradient is the reverse running sum over tokens of
// q_t,d dq_t,d - k_t,d dk_t,d, plus sum_j dfinal[d][j] S_fin[d][j] at the last token.  On the
// fp16 path the reversed dk pass forms it in pass order (after the dq pass), and
// chan_gfix_kernel adds the earlier segments' totals; on the fp32 path chan_g_kernel and
// chan_scan_kernel form it afterwards (64-token segments, then carries).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gla.h"
#include "gla_layout.h"

namespace gla {

// One pass: token u of the pass reads row L-1-u of a reversed operand.
struct ChanPass {
    const void *q, *k, *v;
    int qdt, kdt, vdt;     // GLA_DTYPE_* of each operand
    int qrev, krev, vrev;
    const float *vli;      // value row weight exp(vli[bh][source row]), or null
    const float *la;       // [BH][L][Dg] log gate, Dg = Dq (key gate) or Dn (value gate)
    int grev;              // gate of token u: 0 for u = 0, la[L-u] for u >= 1
    const float *s0;       // [BH][Dq][Dn] or null
    float *out;            // [BH][L][Dn]
    int orev;              // row u stored at row L-1-u
    const float *oli;      // output row weight exp(oli[bh][destination row]), or null
    float *fin;            // [BH][Dq][Dn] or null
    int L, Dn;
    // Sequence segments run in parallel: segment s covers pass tokens [s seg_len, (s+1) seg_len).
    // ws_state [BH][nseg-1][Dq][Dn]: a segment's own state (state kernel), then the state
    // entering segment s+1 (scan); ws_decay [BH][nseg-1][Dg]: the segment's decay.
    int seg_len, nseg;
    float *ws_state, *ws_decay;
    // fp16 passes (chan_vg16_kernel): per (batch, head) output-gradient scale bits; outputs are
    // divided by the scale s, and the initial state multiplied by s when s0_scaled
    const uint32_t *mx;
    int s0_scaled;
    // The per-channel log-gate gradient, formed by the reversed dk pass on fp16 operands
    // (chan_vg16_kernel, g_out non-null): pass token u is sequence row t = L-1-u, so the
    // running sum over the pass of g_t = q_t dq_t - k_t dk_t (the pass's v operand is q) is the
    // sum over s >= t.  g_dq: dq [BH][L][Dn] fp32 (from the dq pass), g_k: k [BH][L][Dn] bf16;
    // g_out: dlog_alpha, complete in the first segment (which starts from g_fterm, the
    // final-state term, or zero), the segment's own sum elsewhere; g_part [BH][nseg][Dn]: the
    // segments' totals, for chan_gfix_kernel.
    const float *g_dq;
    const void *g_k;
    float *g_out, *g_part;
    const float *g_fterm;
};

namespace {

constexpr float kLog2eC = 1.4426950408889634f;
constexpr int kBlk = 16;  // tokens per block


// Buffer resources over one (batch, head) slice: 32-bit element offsets, and an offset past
// the range (kOff) reads zero, so masked elements need no branch.
typedef __amdgpu_buffer_rsrc_t rsrc_c;
constexpr uint32_t kOff = 0xffffffffu;
__device__ __forceinline__ rsrc_c mk_rsrc(const void *p, uint64_t bytes) {
    const uint32_t n = bytes > 0xfffffff0ull ? 0xfffffff0u : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n, 0x00020000);
}
// Raw input bits (fp32, or bf16 in the low half) of element i; the dtype is a template
// argument so that a load's result is not consumed on the path that issues it.
template <bool F32>
__device__ __forceinline__ uint32_t ld_raw(rsrc_c r, uint32_t i) {
    const uint32_t off = i == kOff ? kOff : i * (F32 ? 4u : 2u);
    if constexpr (F32) return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    else return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ float ld_f32(rsrc_c r, uint32_t i) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)(i == kOff ? kOff : i * 4u), 0, 0));
}
template <bool F32>
__device__ __forceinline__ float raw_val(uint32_t x) {
    return F32 ? __uint_as_float(x) : __uint_as_float(x << 16);
}

__device__ __forceinline__ float fexp2c(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier over LDS only: global loads in flight (the next block's operands) are
// not waited for.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float log2_gate(float la) {
    const float x = la * kLog2eC;
    return x < -150.f ? -150.f : x;
}

typedef float f32x4c __attribute__((ext_vector_type(4)));

// LDS plan of a pass (floats): q and k rows padded to DQ + 4, transposed tiles with rows of
// 16 tokens padded to 20.
template <bool KG, int DQ>
struct ChanLds {
    static constexpr int QP = DQ + 4, TP = 20;
    static constexpr int Q = 0;                           // [16][QP] q, then the decayed q (key gate)
    static constexpr int KX = Q + kBlk * QP;              // [16][QP] k (value gate) or k 2^(-b_s) (key gate)
    static constexpr int KT = KX + kBlk * QP;             // [DQ][TP] decayed k, transposed
    static constexpr int B = KT + DQ * TP;                // key gate [16][QP] / value gate [64][TP]: log2 decays
    static constexpr int VT = B + (KG ? kBlk * QP : 64 * TP);  // [64][TP] v, transposed
    static constexpr int VF = VT + 64 * TP;               // [64][TP] decayed v, transposed (value gate)
    static constexpr int VX = VF + (KG ? 0 : 64 * TP);    // [64][TP] v 2^(-b_s), transposed (value gate)
    static constexpr int P = VX + (KG ? 0 : 64 * TP);     // [16][TP] scores; value gate: [4][16][TP], one
                                                          // partial sum per wave
    static constexpr int TOT = P + (KG ? 1 : 4) * kBlk * TP;  // [4][64] value gate: each wave's log2 decay
    static constexpr int FLAG = TOT + (KG ? 0 : 4 * 64);  // strong-decay flag of the block
    static constexpr int TOTAL = FLAG + 4;
};

__device__ __forceinline__ f32x4c mfma4(float a, float b, f32x4c c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// A block whose running log2 decay reaches below this (in any key channel) forms its
// key-gated scores exactly instead of as a product of q 2^(b_t) and k 2^(-b_s).
constexpr float kFactorFloor = -60.f;

// grid = BH * (Dn / 64) * segments workgroups of 256 threads (segment index fastest).  Wave w
// owns value columns 16 w .. 16 w + 15
// of the workgroup's 64; lane l (c16 = l & 15, g = l >> 4) holds the state in matrix-core
// accumulator layout: rows 16 j + 4 g + e (j < DQ / 16, e < 4) of column 16 w + c16.  Both
// block products run on the fp32 matrix cores (16x16x4):
//   output  O[t][n] += sum_d q'[t][d] S[d][n], with the contraction index of step (j, e) and
//           lane group g being d = 16 j + 4 g + e, so that each lane's own state registers
//           are its B operand;
//   state   S[d][n] = dec S[d][n] + sum_s k'[s][d] v'[s][n], token index s = 4 g + m.
// The operands of the next block are fetched into registers (raw bits) while the current one
// is computed.  FM: which of q, k, v (bits 0, 1, 2) are fp32; the others are bf16.
// ST: the state kernel of the segments before the last (no outputs; the segment's own state
// from zero and its decay into the workspace).
template <bool KG, int DQ, int FM, bool ST>
__global__ __launch_bounds__(256, 2) void chan_pass_kernel(ChanPass a) {
    constexpr bool QF = FM & 1, KF = (FM >> 1) & 1, VF = (FM >> 2) & 1;
    using Lp = ChanLds<KG, DQ>;
    constexpr int QP = Lp::QP, TP = Lp::TP, NJ = DQ / 16;
    constexpr int GW = KG ? DQ : 64;
    constexpr int NQ = kBlk * DQ / 256;   // q (and k) elements fetched per thread
    constexpr int NG = kBlk * GW / 256;   // gate elements fetched per thread
    constexpr int NV = kBlk * 64 / 256;   // value elements fetched per thread
    extern __shared__ __align__(16) float lds[];
    float *sQ = lds + Lp::Q, *sKX = lds + Lp::KX, *sKT = lds + Lp::KT, *sB = lds + Lp::B;
    float *sVT = lds + Lp::VT, *sVF = lds + Lp::VF, *sVX = lds + Lp::VX, *sP = lds + Lp::P, *sTot = lds + Lp::TOT;
    int *sFlag = reinterpret_cast<int *>(lds + Lp::FLAG);

    const int ndt = a.Dn / 64;
    const int nsb = ST ? a.nseg - 1 : a.nseg;
    size_t id = blockIdx.x;
    const int seg = (int)(id % (unsigned)nsb);
    id /= (unsigned)nsb;
    const int n0 = (int)(id % (unsigned)ndt) * 64;
    const size_t bh = id / (unsigned)ndt;
    const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6, c16 = lane & 15, g = lane >> 4;
    const int ncol = 16 * w + c16;        // this lane's column within the workgroup's 64
    const int L = a.L, Dn = a.Dn;
    const int Dg = KG ? DQ : Dn;
    const int ub = seg * a.seg_len, ue = min(L, ub + a.seg_len);
    const size_t nsm = (size_t)(a.nseg - 1);

    // the state entering the segment: the initial state, the scanned boundary state, or zero
    const float *s_in = (ST || seg == 0) ? nullptr : a.ws_state + (bh * nsm + seg - 1) * (size_t)DQ * Dn;
    f32x4c S[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[j][e] = s_in ? s_in[(size_t)(16 * j + 4 * g + e) * Dn + n0 + ncol] : 0.f;
    if (!ST && seg == 0 && a.s0) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[j][e] = a.s0[(bh * DQ + 16 * j + 4 * g + e) * Dn + n0 + ncol];
    }
    float gtot = 0.f;  // state kernel: the segment's log2 decay of column tid (tid < GW)

    // next block: raw q, k, v bits, value-row and output-row log weights, log gates
    const uint64_t Lu = (uint64_t)L;
    const rsrc_c rq = mk_rsrc(reinterpret_cast<const char *>(a.q) + bh * Lu * DQ * (QF ? 4 : 2), Lu * DQ * (QF ? 4 : 2));
    const rsrc_c rk = mk_rsrc(reinterpret_cast<const char *>(a.k) + bh * Lu * DQ * (KF ? 4 : 2), Lu * DQ * (KF ? 4 : 2));
    const rsrc_c rv = mk_rsrc(reinterpret_cast<const char *>(a.v) + bh * Lu * Dn * (VF ? 4 : 2), Lu * Dn * (VF ? 4 : 2));
    const rsrc_c rg = mk_rsrc(a.la + bh * Lu * Dg, Lu * Dg * 4);
    const rsrc_c rvl = mk_rsrc(a.vli ? a.vli + bh * Lu : a.la, a.vli ? Lu * 4 : 0);
    const rsrc_c rol = mk_rsrc(a.oli ? a.oli + bh * Lu : a.la, a.oli ? Lu * 4 : 0);
    uint32_t fq[NQ], fk[NQ], fv[NV];
    float fvl[NV], fg[NG], fol[4], ol[4];
    // Element i of a thread's share sits RS = 256 / DQ rows (q, k, key-side gates) or one row
    // (v, value-side gates: tokens 4 tv .. 4 tv + 3 of column cv) after element i - 1, so its
    // offset is a fixed step from the first.
    constexpr int RS = 256 / DQ;
    const int tq = tid / DQ, dq = tid % DQ, tv = tid >> 6, cv = tid & 63;
    auto row_of = [&](int rev, int u) { return rev ? L - 1 - u : u; };
    auto fetch = [&](int u0) {
        const int uq = u0 + tq, uv = u0 + 4 * tv;
        {
            const int bq = row_of(a.qrev, uq) * DQ + dq, bk = row_of(a.krev, uq) * DQ + dq;
            const int sq = a.qrev ? -RS * DQ : RS * DQ, sk = a.krev ? -RS * DQ : RS * DQ;
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const bool ok = uq + i * RS < ue;
                if constexpr (!ST) fq[i] = ld_raw<QF>(rq, ok ? (uint32_t)(bq + i * sq) : kOff);  // no q: states only
                fk[i] = ld_raw<KF>(rk, ok ? (uint32_t)(bk + i * sk) : kOff);
            }
        }
        {
            const int rv0 = row_of(a.vrev, uv), sr = a.vrev ? -1 : 1;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const bool ok = uv + i < ue;
                const int row = rv0 + i * sr;
                fv[i] = ld_raw<VF>(rv, ok ? (uint32_t)(row * Dn + n0 + cv) : kOff);
                fvl[i] = ld_f32(rvl, ok ? (uint32_t)row : kOff);
            }
        }
        {
            // gate rows: token u reads row L - u when reversed (zero for u = 0), else row u
            const int ug = KG ? uq : uv, cg = KG ? dq : n0 + cv, step = KG ? RS : 1;
            const int r0 = a.grev ? L - ug : ug, sr = a.grev ? -step : step;
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int u = ug + i * step;
                const bool ok = u < ue && !(a.grev && u == 0);
                fg[i] = ld_f32(rg, ok ? (uint32_t)((r0 + i * sr) * Dg + cg) : kOff);
            }
        }
        {
            const int u = u0 + 4 * g, r0 = row_of(a.orev, u), sr = a.orev ? -1 : 1;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                fol[e] = ld_f32(rol, (!ST && u + e < ue) ? (uint32_t)(r0 + e * sr) : kOff);
        }
    };
    fetch(ub);

    for (int u0 = ub; u0 < ue; u0 += kBlk) {
        // ---- raw operands into LDS: q, k by rows (value gate: k also transposed), v
        // transposed, key-gate logs by token rows; the value gate's running log2 decays over
        // each thread's four tokens stay in registers, with the wave's total in LDS
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int idx = tid + i * 256, t = idx / DQ, d = idx % DQ;
            if constexpr (!ST) sQ[t * QP + d] = raw_val<QF>(fq[i]);
            const float kv = raw_val<KF>(fk[i]);
            if constexpr (KG || !ST) sKX[t * QP + d] = kv;  // value-gate states use k^T only
            if constexpr (!KG) sKT[d * TP + t] = kv;
        }
        f32x4c vr;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float v = raw_val<VF>(fv[i]);
            if (a.vli) v *= fexp2c(fvl[i] * kLog2eC);
            vr[i] = v;
        }
        f32x4c loc;
        if constexpr (KG) {
            *reinterpret_cast<f32x4c *>(sVT + cv * TP + 4 * tv) = vr;
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int idx = tid + i * 256, t = idx / GW, c = idx % GW;
                sB[t * QP + c] = fg[i] == 0.f ? 0.f : log2_gate(fg[i]);
            }
        } else {
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                run += fg[i] == 0.f ? 0.f : log2_gate(fg[i]);
                loc[i] = run;
            }
            sTot[tv * 64 + cv] = run;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) ol[e] = fol[e];
        if (tid == 0) *sFlag = 0;
        lds_sync();
        if (u0 + kBlk < ue) fetch(u0 + kBlk);
        if constexpr (KG) {
            // ---- running log2 decays inside the block, inclusive
            if (tid < GW) {
                float b[kBlk];
#pragma unroll
                for (int t = 0; t < kBlk; ++t) b[t] = sB[t * QP + tid];
                float run = 0.f;
#pragma unroll
                for (int t = 0; t < kBlk; ++t) {
                    run += b[t];
                    sB[t * QP + tid] = run;
                }
                if (run < kFactorFloor) *sFlag = 1;
                gtot += run;
            }
            lds_sync();
            const bool exact = !ST && *sFlag != 0;
            if (exact) {
                // strong decay in this block: key-gated scores with every factor formed exactly
                const int t = tid >> 4, s = tid & 15;
                float p = 0.f;
                if (s <= t)
                    for (int d = 0; d < DQ; ++d)
                        p += sQ[t * QP + d] * sKX[s * QP + d] * fexp2c(sB[t * QP + d] - sB[s * QP + d]);
                sP[t * TP + s] = p;
                lds_sync();
            }
            // ---- decay-weighted operands
            for (int idx = tid; idx < kBlk * DQ; idx += 256) {
                const int t = idx / DQ, d = idx % DQ;
                const float bt = sB[t * QP + d], b15 = sB[(kBlk - 1) * QP + d];
                const float kv = sKX[t * QP + d];
                if constexpr (!ST) sQ[t * QP + d] *= fexp2c(bt);  // q_t 2^(b_t)
                sKT[d * TP + t] = kv * fexp2c(b15 - bt);  // k_t 2^(b_15 - b_t)
                sKX[t * QP + d] = kv * fexp2c(-bt);       // k_t 2^(-b_t), for the scores
            }
            lds_sync();
            // ---- scores P[t][s] = sum_d q[t][d] k[s][d] on the matrix cores (wave 0), s <= t
            if (!ST && !exact && w == 0) {
                // four independent accumulators (one per e) so that the products do not wait on
                // each other
                f32x4c pe[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const f32x4c qa = *reinterpret_cast<const f32x4c *>(sQ + c16 * QP + 16 * j + 4 * g);
                    const f32x4c kb = *reinterpret_cast<const f32x4c *>(sKX + c16 * QP + 16 * j + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) pe[e] = mfma4(qa[e], kb[e], pe[e]);
                }
                const f32x4c pc = (pe[0] + pe[1]) + (pe[2] + pe[3]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 4 * g + e;
                    sP[t * TP + c16] = c16 <= t ? pc[e] : 0.f;
                }
            }
            if constexpr (!ST) lds_sync();
        } else {
            // ---- value gate: the running log2 decays of column cv, tokens 4 tv .. 4 tv + 3,
            // from the waves' totals; the decay-weighted values
            float pre = 0.f, tot = 0.f;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float y = sTot[x * 64 + cv];
                tot += y;
                pre += x < tv ? y : 0.f;
            }
            f32x4c b4, vf4, vx4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                b4[i] = pre + loc[i];
                vf4[i] = vr[i] * fexp2c(tot - b4[i]);
                vx4[i] = vr[i] * fexp2c(-b4[i]);  // bounded by 2^60 unless strong
            }
            *reinterpret_cast<f32x4c *>(sB + cv * TP + 4 * tv) = b4;
            *reinterpret_cast<f32x4c *>(sVF + cv * TP + 4 * tv) = vf4;
            if constexpr (!ST) {
                *reinterpret_cast<f32x4c *>(sVT + cv * TP + 4 * tv) = vr;
                *reinterpret_cast<f32x4c *>(sVX + cv * TP + 4 * tv) = vx4;
                if (tot < kFactorFloor) *sFlag = 1;
                // ---- scores P[t][s] = sum_d q[t][d] k[s][d] on the matrix cores, the
                // contraction split over the four waves (wave w: channels of steps j in its
                // quarter), one partial per wave
                constexpr int JW = NJ / 4;
                f32x4c pe[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int jj = 0; jj < JW; ++jj) {
                    const int j = w * JW + jj;
                    const f32x4c qa = *reinterpret_cast<const f32x4c *>(sQ + c16 * QP + 16 * j + 4 * g);
                    const f32x4c kb = *reinterpret_cast<const f32x4c *>(sKX + c16 * QP + 16 * j + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) pe[e] = mfma4(qa[e], kb[e], pe[e]);
                }
                const f32x4c pc = (pe[0] + pe[1]) + (pe[2] + pe[3]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 4 * g + e;
                    sP[(w * kBlk + t) * TP + c16] = c16 <= t ? pc[e] : 0.f;
                }
            }
            if (tid < 64) gtot += tot;
            lds_sync();
        }
        // scores, 4 consecutive columns of row t (value gate: the sum of the waves' partials)
        auto p4 = [&](int t, int s0) {
            f32x4c r = *reinterpret_cast<const f32x4c *>(sP + t * TP + s0);
            if constexpr (!KG) {
#pragma unroll
                for (int x = 1; x < 4; ++x) r += *reinterpret_cast<const f32x4c *>(sP + (x * kBlk + t) * TP + s0);
            }
            return r;
        };
        // strong decay in this block: key gate: scores with exact factors (above); value gate:
        // the block's own tokens with exact factors
        const bool strong = !ST && *sFlag != 0;
        // ---- outputs of the block's 16 tokens for this lane's column
        if constexpr (!ST) {
        f32x4c Oe[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const f32x4c qa = *reinterpret_cast<const f32x4c *>(sQ + c16 * QP + 16 * j + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) Oe[e] = mfma4(qa[e], S[j][e], Oe[e]);
        }
        f32x4c O = (Oe[0] + Oe[1]) + (Oe[2] + Oe[3]);
        if constexpr (KG) {
            // the block's own tokens: P (decays included) times v
            const f32x4c pa = *reinterpret_cast<const f32x4c *>(sP + c16 * TP + 4 * g);
            const f32x4c vb = *reinterpret_cast<const f32x4c *>(sVT + ncol * TP + 4 * g);
#pragma unroll
            for (int m = 0; m < 4; ++m) O = mfma4(pa[m], vb[m], O);
        } else if (!strong) {
            // value gate: (q S + P v 2^(-b_s)) 2^(b_t) per column, all factors bounded
            const f32x4c pa = p4(c16, 4 * g);
            const f32x4c vb = *reinterpret_cast<const f32x4c *>(sVX + ncol * TP + 4 * g);
#pragma unroll
            for (int m = 0; m < 4; ++m) O = mfma4(pa[m], vb[m], O);
            const f32x4c b4 = *reinterpret_cast<const f32x4c *>(sB + ncol * TP + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) O[e] *= fexp2c(b4[e]);
        } else {
            // value gate, strong decay: the entering state's term decays with the column; the
            // block's own tokens with exact factors 2^(b_t - b_s), s <= t
            float vc[kBlk], bc[kBlk];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4c v4 = *reinterpret_cast<const f32x4c *>(sVT + ncol * TP + 4 * m);
                const f32x4c b4 = *reinterpret_cast<const f32x4c *>(sB + ncol * TP + 4 * m);
#pragma unroll
                for (int e = 0; e < 4; ++e) vc[4 * m + e] = v4[e], bc[4 * m + e] = b4[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float bt = bc[0];
#pragma unroll
                for (int m = 1; m < kBlk; ++m) bt = (4 * g + e == m) ? bc[m] : bt;
                float o = O[e] * fexp2c(bt);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const f32x4c pr = p4(4 * g + e, 4 * m);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int s2 = 4 * m + x;
                        const float f = s2 <= 4 * g + e ? fexp2c(bt - bc[s2]) : 0.f;
                        o += pr[x] * vc[s2] * f;
                    }
                }
                O[e] = o;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int u = u0 + 4 * g + e;
            if (u < ue) {
                const size_t dst = bh * L + (a.orev ? L - 1 - u : u);
                float o = O[e];
                if (a.oli) o *= fexp2c(ol[e] * kLog2eC);
                a.out[dst * Dn + n0 + ncol] = o;
            }
        }
        }
        // ---- state to the block end
        if constexpr (KG) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const f32x4c d4 = *reinterpret_cast<const f32x4c *>(sB + (kBlk - 1) * QP + 16 * j + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) S[j][e] *= fexp2c(d4[e]);
            }
        } else {
            const float dec = fexp2c(sB[ncol * TP + kBlk - 1]);
#pragma unroll
            for (int j = 0; j < NJ; ++j) S[j] *= dec;
        }
        const float *vsrc = KG ? sVT : sVF;
        const f32x4c vb = *reinterpret_cast<const f32x4c *>(vsrc + ncol * TP + 4 * g);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const f32x4c ka = *reinterpret_cast<const f32x4c *>(sKT + (16 * j + c16) * TP + 4 * g);
#pragma unroll
            for (int m = 0; m < 4; ++m) S[j] = mfma4(ka[m], vb[m], S[j]);
        }
        lds_sync();
    }
    if constexpr (ST) {
        float *st = a.ws_state + (bh * nsm + seg) * (size_t)DQ * Dn;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) st[(size_t)(16 * j + 4 * g + e) * Dn + n0 + ncol] = S[j][e];
        // the segment's decay: per key channel (written by the first value tile) or per value column
        if (tid < GW && (!KG || n0 == 0))
            a.ws_decay[(bh * nsm + seg) * Dg + (KG ? tid : n0 + tid)] = fexp2c(gtot);
    } else if (a.fin && seg == a.nseg - 1) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.fin[(bh * DQ + 16 * j + 4 * g + e) * Dn + n0 + ncol] = S[j][e];
    }
}

// ---------------------------------------------------------------------------------------
// Value-gated pass with fp16 operands (bf16 inputs; the scaled fp16 output gradient as one
// operand).  The same blocks, decays and state layout as chan_pass_kernel<false, ...>, with
// the products on the fp16 matrix cores: scores and q S as 16x16x32 steps whose 32-slot
// contraction of lane group g holds channels 32 m + 4 g + x and 32 m + 16 + 4 g + x (x < 4),
// the lane's own state rows of blocks 2 m and 2 m + 1; the block's own tokens and the state
// update as 16x16x16 steps over the 16 tokens.  Factors applied to fp16 operands are bounded
// by 2^8: a block whose decay reaches below 2^-8 forms its own tokens' factors exactly.
// Accumulation, decays and the state are fp32; the state is rounded to fp16 as the B operand
// of q S, as in the forward kernel.  Outputs are scaled by 1/s (mx) and, when s0_scaled, the
// initial state by s.
typedef _Float16 h16c;
typedef h16c h16x4c __attribute__((ext_vector_type(4)));
typedef h16c h16x8c __attribute__((ext_vector_type(8)));
typedef h16c h16x2c __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2c __attribute__((ext_vector_type(2)));

constexpr float kFactorFloor16 = -8.f;

// LDS plan (bytes): fp16 q and k rows padded by 48 B (the fragment reads of a half-wave then
// fall on distinct banks), fp16 transposed rows of 16 tokens
// padded to 20 halves, fp32 transposed rows padded to 20 floats.
template <int DQ>
struct VgLds {
    static constexpr int QH = DQ + 24, TH = 20, TP = 20;
    static constexpr int Q = 0;                       // [16][QH] h  q
    static constexpr int K = Q + kBlk * QH * 2;       // [16][QH] h  k
    static constexpr int KT = K + kBlk * QH * 2;      // [DQ][TH] h  k, transposed
    static constexpr int VF = KT + DQ * TH * 2;       // [64][TH] h  v 2^(b_15 - b_s), transposed
    static constexpr int VX = VF + 64 * TH * 2;       // [64][TH] h  v 2^(-b_s), transposed
    static constexpr int B = VX + 64 * TH * 2;        // [64][TP] f  running log2 decays
    static constexpr int VT = B + 64 * TP * 4;        // [64][TP] f  v (strong blocks)
    static constexpr int P = VT + 64 * TP * 4;        // [4][16][TP] f  score partials, one per wave
    static constexpr int TOT = P + 4 * kBlk * TP * 4; // [4][64] f  each wave's log2 decay
    static constexpr int FLAG = TOT + 4 * 64 * 4;
    static constexpr int BYTES = FLAG + 16;
};

__device__ __forceinline__ f32x4c mfma16x16(h16x4c a, h16x4c b, f32x4c c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4c mfma16x32(h16x8c a, h16x8c b, f32x4c c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// Four operands (two dwords) as fp16: fp16 bits as they are, bf16 converted.
template <bool H16>
__device__ __forceinline__ h16x4c to_h4(u32x2c r) {
    if constexpr (H16) {
        return __builtin_bit_cast(h16x4c, r);
    } else {
        const f32x4c f = {__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                          __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
        return __builtin_convertvector(f, h16x4c);
    }
}
template <bool H16>
__device__ __forceinline__ float h_val(uint32_t x) {
    if constexpr (H16) return (float)__builtin_bit_cast(h16c, (uint16_t)x);
    else return __uint_as_float(x << 16);
}
// Eight fp16 operands of a 16x16x32 step: channels c .. c + 3 and c + 16 .. c + 19.
__device__ __forceinline__ h16x8c frag8(const h16c *row, int c) {
    const h16x4c lo = *reinterpret_cast<const h16x4c *>(row + c);
    const h16x4c hi = *reinterpret_cast<const h16x4c *>(row + c + 16);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// grid and work split as chan_pass_kernel.  FH: which of q, k, v (bits 0, 1, 2) are fp16;
// the others are bf16.  GG: the pass forms the log-gate gradient (g_out).
template <int DQ, int FH, bool ST, bool GG = false>
__global__ __launch_bounds__(256, 2) void chan_vg16_kernel(ChanPass a) {
    constexpr bool QH16 = FH & 1, KH16 = (FH >> 1) & 1, VH16 = (FH >> 2) & 1;
    using Lp = VgLds<DQ>;
    constexpr int QH = Lp::QH, TH = Lp::TH, TP = Lp::TP, NJ = DQ / 16, NM = DQ / 32;
    constexpr int GR = DQ / 4;   // four-channel groups per row
    constexpr int NR = DQ / 64;  // q and k rows per thread
    constexpr int NV = 4;        // v: tokens 4 tv .. 4 tv + 3 of column cv
    extern __shared__ __align__(16) char smem[];
    h16c *sQ = reinterpret_cast<h16c *>(smem + Lp::Q), *sK = reinterpret_cast<h16c *>(smem + Lp::K);
    h16c *sKT = reinterpret_cast<h16c *>(smem + Lp::KT), *sVF = reinterpret_cast<h16c *>(smem + Lp::VF);
    h16c *sVX = reinterpret_cast<h16c *>(smem + Lp::VX);
    float *sB = reinterpret_cast<float *>(smem + Lp::B), *sVT = reinterpret_cast<float *>(smem + Lp::VT);
    float *sP = reinterpret_cast<float *>(smem + Lp::P), *sTot = reinterpret_cast<float *>(smem + Lp::TOT);
    int *sFlag = reinterpret_cast<int *>(smem + Lp::FLAG);

    const int ndt = a.Dn / 64;
    const int nsb = ST ? a.nseg - 1 : a.nseg;
    size_t id = blockIdx.x;
    const int seg = (int)(id % (unsigned)nsb);
    id /= (unsigned)nsb;
    const int n0 = (int)(id % (unsigned)ndt) * 64;
    const size_t bh = id / (unsigned)ndt;
    const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6, c16 = lane & 15, g = lane >> 4;
    const int ncol = 16 * w + c16;
    const int L = a.L, Dn = a.Dn;
    const int ub = seg * a.seg_len, ue = min(L, ub + a.seg_len);
    const size_t nsm = (size_t)(a.nseg - 1);
    const float sc = grad_scale_of(a.mx[bh]);
    const float osc = 1.f / sc;

    const float *s_in = (ST || seg == 0) ? nullptr : a.ws_state + (bh * nsm + seg - 1) * (size_t)DQ * Dn;
    f32x4c S[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[j][e] = s_in ? s_in[(size_t)(16 * j + 4 * g + e) * Dn + n0 + ncol] : 0.f;
    if (!ST && seg == 0 && a.s0) {
        const float is = a.s0_scaled ? sc : 1.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[j][e] = a.s0[(bh * DQ + 16 * j + 4 * g + e) * Dn + n0 + ncol] * is;
    }
    float gtot = 0.f;
    // gate gradient: running sum of the segment's terms before the current block (every lane
    // group g of a column holds it), and the final-state term that the first segment starts from
    float grun = 0.f;
    const float gf = (GG && !ST && seg == 0 && a.g_fterm) ? a.g_fterm[bh * Dn + n0 + ncol] : 0.f;

    const uint64_t Lu = (uint64_t)L;
    const rsrc_c rq = mk_rsrc(reinterpret_cast<const char *>(a.q) + bh * Lu * DQ * 2, Lu * DQ * 2);
    const rsrc_c rk = mk_rsrc(reinterpret_cast<const char *>(a.k) + bh * Lu * DQ * 2, Lu * DQ * 2);
    const rsrc_c rv = mk_rsrc(reinterpret_cast<const char *>(a.v) + bh * Lu * Dn * 2, Lu * Dn * 2);
    // The gate of a reversed pass is token u's row L - u: row L - 1 - u of a view that starts
    // one row later.
    const uint64_t g1 = a.grev ? 1 : 0;
    const rsrc_c rg = mk_rsrc(a.la + (bh * Lu + g1) * Dn, (Lu - g1) * Dn * 4);
    const rsrc_c rvl = mk_rsrc(a.vli ? a.vli + bh * Lu : a.la, a.vli ? Lu * 4 : 0);
    const rsrc_c rol = mk_rsrc(a.oli ? a.oli + bh * Lu : a.la, a.oli ? Lu * 4 : 0);
    constexpr bool gg = GG && !ST;
    const rsrc_c rgd = mk_rsrc(gg ? a.g_dq + bh * Lu * Dn : a.la, gg ? Lu * Dn * 4 : 0);
    const rsrc_c rgk = mk_rsrc(gg ? reinterpret_cast<const char *>(a.g_k) + bh * Lu * Dn * 2 : nullptr, gg ? Lu * Dn * 2 : 0);
    u32x2c fq[NR], fk[NR];
    uint32_t fv[NV];
    float fvl[NV], fg[NV], fol[4], ol[4];
    // q, k: thread (rq0, gq) holds rows NR rq0 + i, channels 4 gq .. 4 gq + 3
    const int rq0 = tid / GR, gq = tid % GR, tv = tid >> 6, cv = tid & 63;
    // Token u reads row L - 1 - u of a reversed operand, else row u, with no masks: segments
    // end on block boundaries, so only the sequence end cuts a block, and rows past either end
    // lie outside the slice (a negative row wraps to a 32-bit offset past it) and read zero.
    auto row_of = [&](int rev, int u) { return (uint32_t)(rev ? L - 1 - u : u); };
    auto fetch = [&](int u0) {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int u = u0 + NR * rq0 + i;
            const uint32_t oq = (row_of(a.qrev, u) * (uint32_t)DQ + 4u * gq) * 2u;
            const uint32_t ok_ = (row_of(a.krev, u) * (uint32_t)DQ + 4u * gq) * 2u;
            if constexpr (!ST) fq[i] = __builtin_amdgcn_raw_buffer_load_b64(rq, (int)oq, 0, 0);  // no q: states only
            fk[i] = __builtin_amdgcn_raw_buffer_load_b64(rk, (int)ok_, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int u = u0 + 4 * tv + i;
            const uint32_t rv_ = row_of(a.vrev, u), rg_ = row_of(a.grev, u);
            fv[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rv, (int)((rv_ * (uint32_t)Dn + n0 + cv) * 2u), 0, 0);
            fvl[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvl, (int)(rv_ * 4u), 0, 0));
            fg[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, (int)((rg_ * (uint32_t)Dn + n0 + cv) * 4u), 0, 0));
        }
        if constexpr (!ST) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                fol[e] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(rol, (int)(row_of(a.orev, u0 + 4 * g + e) * 4u), 0, 0));
        }
    };
    fetch(ub);

    for (int u0 = ub; u0 < ue; u0 += kBlk) {
        // ---- q, k rows and k transposed as fp16; v and the running log2 decays of its four
        // tokens in registers, the wave's decay total in LDS
        h16x4c kh[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int t = NR * rq0 + i;
            if constexpr (!ST) *reinterpret_cast<h16x4c *>(sQ + t * QH + 4 * gq) = to_h4<QH16>(fq[i]);
            kh[i] = to_h4<KH16>(fk[i]);
            if constexpr (!ST) *reinterpret_cast<h16x4c *>(sK + t * QH + 4 * gq) = kh[i];  // states use k^T only
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            h16c *dst = sKT + (4 * gq + x) * TH + NR * rq0;
            if constexpr (NR == 1) {
                dst[0] = kh[0][x];
            } else if constexpr (NR == 2) {
                *reinterpret_cast<h16x2c *>(dst) = h16x2c{kh[0][x], kh[1][x]};
            } else {
                *reinterpret_cast<h16x4c *>(dst) = h16x4c{kh[0][x], kh[1][x], kh[2][x], kh[3][x]};
            }
        }
        f32x4c vr, loc;
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float v = h_val<VH16>(fv[i]);
            if (a.vli) v *= fexp2c(fvl[i] * kLog2eC);
            vr[i] = v;
            run += log2_gate(fg[i]);
            loc[i] = run;
        }
        sTot[tv * 64 + cv] = run;
        if constexpr (!ST) {
#pragma unroll
            for (int e = 0; e < 4; ++e) ol[e] = fol[e];
        }
        if (tid == 0) *sFlag = 0;
        lds_sync();
        if (u0 + kBlk < ue) fetch(u0 + kBlk);
        // gate gradient: dq and k of this lane's output elements, needed after the block's
        // products (loaded here rather than a block ahead, to keep registers for occupancy)
        float gd[4], gk[4];
        if constexpr (gg) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t oe = row_of(a.orev, u0 + 4 * g + e) * (uint32_t)Dn + n0 + ncol;
                gd[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rgd, (int)(oe * 4u), 0, 0));
                gk[e] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rgk, (int)(oe * 2u), 0, 0) << 16);
            }
        }
        // ---- running log2 decays of column cv, tokens 4 tv .. 4 tv + 3; decay-weighted values
        {
            float pre = 0.f, tot = 0.f;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float y = sTot[x * 64 + cv];
                tot += y;
                pre += x < tv ? y : 0.f;
            }
            f32x4c b4, vf4, vx4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                b4[i] = pre + loc[i];
                vf4[i] = vr[i] * fexp2c(tot - b4[i]);
                vx4[i] = vr[i] * fexp2c(-b4[i]);  // bounded by 2^8 unless strong
            }
            *reinterpret_cast<f32x4c *>(sB + cv * TP + 4 * tv) = b4;
            *reinterpret_cast<h16x4c *>(sVF + cv * TH + 4 * tv) = __builtin_convertvector(vf4, h16x4c);
            if constexpr (!ST) {
                *reinterpret_cast<f32x4c *>(sVT + cv * TP + 4 * tv) = vr;
                *reinterpret_cast<h16x4c *>(sVX + cv * TH + 4 * tv) = __builtin_convertvector(vx4, h16x4c);
                if (tot < kFactorFloor16) *sFlag = 1;
            }
            if (tid < 64) gtot += tot;
        }
        if constexpr (!ST) {
            // ---- scores P[t][s] = q_t . k_s, the 32-channel steps split over the waves, one
            // partial per wave (zero for a wave without steps)
            constexpr int MW = NM >= 4 ? NM / 4 : 1;
            f32x4c pc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mm = 0; mm < MW; ++mm) {
                const int m = w * MW + mm;
                if (m < NM) {
                    const h16x8c qa = frag8(sQ + c16 * QH, 32 * m + 4 * g);
                    const h16x8c kb = frag8(sK + c16 * QH, 32 * m + 4 * g);
                    pc = mfma16x32(qa, kb, pc);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * g + e;
                sP[(w * kBlk + t) * TP + c16] = c16 <= t ? pc[e] : 0.f;
            }
        }
        lds_sync();
        if constexpr (!ST) {
            const bool strong = *sFlag != 0;
            auto p4 = [&](int t, int s0) {
                f32x4c r = *reinterpret_cast<const f32x4c *>(sP + t * TP + s0);
#pragma unroll
                for (int x = 1; x < 4; ++x) r += *reinterpret_cast<const f32x4c *>(sP + (x * kBlk + t) * TP + s0);
                return r;
            };
            // ---- outputs of the block's 16 tokens for this lane's column: q S
            f32x4c O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const h16x8c qa = frag8(sQ + c16 * QH, 32 * m + 4 * g);
                const h16x4c s0 = __builtin_convertvector(S[2 * m], h16x4c);
                const h16x4c s1 = __builtin_convertvector(S[2 * m + 1], h16x4c);
                O = mfma16x32(qa, __builtin_shufflevector(s0, s1, 0, 1, 2, 3, 4, 5, 6, 7), O);
            }
            if (!strong) {
                // (q S + P v 2^(-b_s)) 2^(b_t)
                const h16x4c pa = __builtin_convertvector(p4(c16, 4 * g), h16x4c);
                const h16x4c vb = *reinterpret_cast<const h16x4c *>(sVX + ncol * TH + 4 * g);
                O = mfma16x16(pa, vb, O);
                const f32x4c b4 = *reinterpret_cast<const f32x4c *>(sB + ncol * TP + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) O[e] *= fexp2c(b4[e]);
            } else {
                // strong decay: the entering state's term decays with the column; the block's
                // own tokens with exact factors 2^(b_t - b_s), s <= t, in fp32
                float vc[kBlk], bc[kBlk];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const f32x4c v4 = *reinterpret_cast<const f32x4c *>(sVT + ncol * TP + 4 * m);
                    const f32x4c b4 = *reinterpret_cast<const f32x4c *>(sB + ncol * TP + 4 * m);
#pragma unroll
                    for (int e = 0; e < 4; ++e) vc[4 * m + e] = v4[e], bc[4 * m + e] = b4[e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float bt = bc[0];
#pragma unroll
                    for (int m = 1; m < kBlk; ++m) bt = (4 * g + e == m) ? bc[m] : bt;
                    float o = O[e] * fexp2c(bt);
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const f32x4c pr = p4(4 * g + e, 4 * m);
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            const int s2 = 4 * m + x;
                            const float f = s2 <= 4 * g + e ? fexp2c(bt - bc[s2]) : 0.f;
                            o += pr[x] * vc[s2] * f;
                        }
                    }
                    O[e] = o;
                }
            }
            f32x4c gt;  // gate-gradient terms q dq - k dk of this lane's four tokens
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int u = u0 + 4 * g + e;
                float o = O[e] * osc;
                if (a.oli) o *= fexp2c(ol[e] * kLog2eC);
                if constexpr (gg) gt[e] = sVT[ncol * TP + 4 * g + e] * gd[e] - gk[e] * o;
                if (u < ue) a.out[(bh * L + (a.orev ? L - 1 - u : u)) * Dn + n0 + ncol] = o;
            }
            if constexpr (gg) {
                // running sum over the block's 16 tokens (token 4 g + e): within the lane, then
                // over the lane groups g of the column (lanes c16 + 16 g)
                // by gfx950 lane-swap moves: p0 / p1 hold rows (0, 0, 2, 2) / (1, 1, 3, 3) of c3,
                // their sum the pair sums; h0 / h1 the pair sums of rows 0-1 / 2-3 in every row
                const float c1 = gt[0] + gt[1], c2 = c1 + gt[2], c3 = c2 + gt[3];
                const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(c3), __float_as_uint(c3), false, false);
                const float pair = __uint_as_float(p[0]) + __uint_as_float(p[1]);
                const auto hq = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
                const float h0 = __uint_as_float(hq[0]), h1 = __uint_as_float(hq[1]);
                const float inc = g == 0 ? c3 : (g == 1 ? pair : (g == 2 ? h0 + c3 : h0 + pair));
                const float base = gf + grun + (inc - c3);
                const float cs[4] = {gt[0], c1, c2, c3};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int u = u0 + 4 * g + e;
                    if (u < ue) a.g_out[(bh * L + (a.orev ? L - 1 - u : u)) * Dn + n0 + ncol] = base + cs[e];
                }
                grun += h0 + h1;  // the column's total over the block (row 3's inc)
            }
        }
        // ---- state to the block end: S diag(2^(b_15)) + k^T (v 2^(b_15 - b_s))
        const float dec = fexp2c(sB[ncol * TP + kBlk - 1]);
        const h16x4c vb = *reinterpret_cast<const h16x4c *>(sVF + ncol * TH + 4 * g);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const h16x4c ka = *reinterpret_cast<const h16x4c *>(sKT + (16 * j + c16) * TH + 4 * g);
            S[j] = mfma16x16(ka, vb, S[j] * dec);
        }
        lds_sync();
    }
    if constexpr (ST) {
        float *st = a.ws_state + (bh * nsm + seg) * (size_t)DQ * Dn;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) st[(size_t)(16 * j + 4 * g + e) * Dn + n0 + ncol] = S[j][e];
        if (tid < 64) a.ws_decay[(bh * nsm + seg) * Dn + n0 + tid] = fexp2c(gtot);
    } else if (a.fin && seg == a.nseg - 1) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.fin[(bh * DQ + 16 * j + 4 * g + e) * Dn + n0 + ncol] = S[j][e];
    }
    if (gg && g == 0) a.g_part[(bh * a.nseg + seg) * Dn + n0 + ncol] = grun;
}

// dlog_alpha rows of segments 1 .. nseg-1 of the reversed dk pass: add the final-state term
// and the totals of the segments before (later rows of the sequence).  Workgroup = up to 64
// pass tokens of one segment of one (batch, head); thread = 4 channels of a row.
__global__ __launch_bounds__(256) void chan_gfix_kernel(float *gout, const float *part, const float *fterm, int L,
                                                        int Dk, int seg_len, int nseg, int chunks) {
    size_t id = blockIdx.x;
    const int ch = (int)(id % (unsigned)chunks);
    id /= (unsigned)chunks;
    const int seg = 1 + (int)(id % (unsigned)(nseg - 1));
    const size_t bh = id / (unsigned)(nseg - 1);
    const int G = Dk / 4, R = 256 / G;  // channel groups per row, rows in flight
    const int c = 4 * ((int)threadIdx.x % G), r = (int)threadIdx.x / G;
    float4 add = fterm ? *reinterpret_cast<const float4 *>(fterm + bh * Dk + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s2 = 0; s2 < seg; ++s2) {
        const float4 p = *reinterpret_cast<const float4 *>(part + (bh * nseg + s2) * Dk + c);
        add.x += p.x, add.y += p.y, add.z += p.z, add.w += p.w;
    }
    const int u0 = seg * seg_len + ch * 64, u1 = min(min(L, (seg + 1) * seg_len), u0 + 64);
    for (int u = u0 + r; u < u1; u += R) {
        float4 *x = reinterpret_cast<float4 *>(gout + (bh * L + (L - 1 - u)) * Dk + c);
        float4 v = *x;
        v.x += add.x, v.y += add.y, v.z += add.z, v.w += add.w;
        *x = v;
    }
}

// The states entering segments 1 .. nseg-1: S <- decay_s S + own_s from the initial state
// (or zero), one thread per state element, written over the segments' own states.
template <bool KG>
__global__ __launch_bounds__(256) void chan_seg_scan_kernel(ChanPass a, int Dq, size_t total) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const size_t m = (size_t)Dq * a.Dn;
    const size_t bh = i / m, e = i % m;
    const int d = (int)(e / (size_t)a.Dn), n = (int)(e % (size_t)a.Dn);
    const int Dg = KG ? Dq : a.Dn;
    const size_t nsm = (size_t)(a.nseg - 1);
    float x = a.s0 ? a.s0[i] * (a.s0_scaled ? grad_scale_of(a.mx[bh]) : 1.f) : 0.f;
    for (size_t s = 0; s < nsm; ++s) {
        float *st = a.ws_state + (bh * nsm + s) * m + e;
        x = a.ws_decay[(bh * nsm + s) * Dg + (KG ? d : n)] * x + *st;
        *st = x;
    }
}

// fterm[bh][d] = sum_j dfT[bh][j][d] finC[bh][j][d] (both [Dv][Dk]): the final-state term
// of channel d's log-gate gradient.  Workgroup = 64 channels of one (bh); its four waves
// take every fourth j and are summed through LDS.
__global__ __launch_bounds__(256) void chan_fterm_kernel(const float *dfT, const float *finC, float *fterm, int Dk,
                                                        int Dv) {
    __shared__ float part[4][64];
    const int ndt = Dk / 64;
    const size_t bh = blockIdx.x / (unsigned)ndt;
    const int d = (int)(blockIdx.x % (unsigned)ndt) * 64 + ((int)threadIdx.x & 63);
    const int w = (int)threadIdx.x >> 6;
    const size_t base = bh * (size_t)Dv * Dk + d;
    float s = 0.f;
#pragma unroll 4
    for (int j = w; j < Dv; j += 4) s += dfT[base + (size_t)j * Dk] * finC[base + (size_t)j * Dk];
    part[w][threadIdx.x & 63] = s;
    __syncthreads();
    if (w == 0) fterm[bh * Dk + d] = (part[0][threadIdx.x] + part[1][threadIdx.x]) + (part[2][threadIdx.x] + part[3][threadIdx.x]);
}

constexpr int kSeg = 64;  // tokens per segment of the log-gate scan

// Four consecutive channels of an input row as fp32 (16-byte fp32 or 8-byte bf16 loads).
__device__ __forceinline__ float4 ld4_in(const void *p, int dt, size_t i) {
    if (dt == GLA_DTYPE_F32) return *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(p) + i);
    const uint2 x = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(p) + i);
    return make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u), __uint_as_float(x.y << 16),
                       __uint_as_float(x.y & 0xffff0000u));
}

// g[bh][t][d] = q dq - k dk (+ fterm at the last token) and the segment totals
// part[bh][seg][d].  Workgroup = 64 channels of one (bh) and four segments: lane l of wave w
// takes channels 4 (l & 15) .. + 3 and rows t = 4 i + (l >> 4) of segment 4 * block + w.
__global__ __launch_bounds__(256) void chan_g_kernel(gla_bwd_desc d, const float *fterm, float *g, float *part,
                                                    int nseg) {
    __shared__ float4 red[4][4][16];
    const int ndt = d.Dk / 64, nsb = (nseg + 3) / 4;
    size_t id = blockIdx.x;
    const int sb = (int)(id % (unsigned)nsb);
    id /= (unsigned)nsb;
    const int dt = (int)(id % (unsigned)ndt);
    const size_t bh = id / (unsigned)ndt;
    const int w = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63, q4 = lane & 15, r4 = lane >> 4;
    const int seg = sb * 4 + w;
    const int c = dt * 64 + 4 * q4;
    const int L = d.L, Dk = d.Dk;
    const int t0 = seg * kSeg, t1 = min(L, t0 + kSeg);
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    if (seg < nseg) {
        for (int t = t0 + r4; t < t1; t += 4) {
            const size_t i = (bh * L + t) * Dk + c;
            const float4 q = ld4_in(d.q, d.in_dtype, i), k = ld4_in(d.k, d.in_dtype, i);
            const float4 dq = *reinterpret_cast<const float4 *>(d.dq + i), dk = *reinterpret_cast<const float4 *>(d.dk + i);
            float4 x = make_float4(q.x * dq.x - k.x * dk.x, q.y * dq.y - k.y * dk.y, q.z * dq.z - k.z * dk.z,
                                   q.w * dq.w - k.w * dk.w);
            if (t == L - 1 && fterm) {
                const float4 f = *reinterpret_cast<const float4 *>(fterm + bh * Dk + c);
                x.x += f.x, x.y += f.y, x.z += f.z, x.w += f.w;
            }
            *reinterpret_cast<float4 *>(g + i) = x;
            sum.x += x.x, sum.y += x.y, sum.z += x.z, sum.w += x.w;
        }
    }
    red[w][r4][q4] = sum;
    __syncthreads();
    if (seg < nseg && r4 == 0) {
        float4 s = red[w][0][q4];
#pragma unroll
        for (int j = 1; j < 4; ++j) {
            const float4 y = red[w][j][q4];
            s.x += y.x, s.y += y.y, s.z += y.z, s.w += y.w;
        }
        *reinterpret_cast<float4 *>(part + (bh * nseg + seg) * Dk + c) = s;
    }
}

// dlog_alpha[bh][t][d] = sum over s >= t of g[bh][s][d]: the carry from the later segments,
// then the segment's tokens from its end.
__global__ __launch_bounds__(64) void chan_scan_kernel(gla_bwd_desc d, const float *g, const float *part, int nseg) {
    const int ndt = d.Dk / 64;
    size_t id = blockIdx.x;
    const int seg = (int)(id % (unsigned)nseg);
    id /= (unsigned)nseg;
    const int dt = (int)(id % (unsigned)ndt);
    const size_t bh = id / (unsigned)ndt;
    const int c = dt * 64 + (int)threadIdx.x;
    const int L = d.L, Dk = d.Dk;
    float run = 0.f;
    for (int s = seg + 1; s < nseg; ++s) run += part[(bh * nseg + s) * Dk + c];
    const int t0 = seg * kSeg, t1 = min(L, t0 + kSeg);
    for (int t = t1 - 1; t >= t0; --t) {
        const size_t i = (bh * L + t) * Dk + c;
        run += g[i];
        d.dlog_alpha[i] = run;
    }
}


// Raise the kernel's dynamic-LDS limit once per device (one bit per device ordinal).
hipError_t lds_limit(const void *fn, std::atomic<uint64_t> &done, int bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

template <bool KG, int DQ, int FM>
hipError_t launch_dq(const ChanPass &p, int BH, hipStream_t st) {
    static std::atomic<uint64_t> done[2] = {{0}, {0}};
    const int bytes = ChanLds<KG, DQ>::TOTAL * 4;
    hipError_t e;
    if (p.nseg > 1) {
        const void *fs = reinterpret_cast<const void *>(&chan_pass_kernel<KG, DQ, FM, true>);
        if ((e = lds_limit(fs, done[1], bytes)) != hipSuccess) return e;
        const dim3 gs((unsigned)((size_t)BH * (p.Dn / 64) * (p.nseg - 1)));
        hipLaunchKernelGGL((chan_pass_kernel<KG, DQ, FM, true>), gs, dim3(256), bytes, st, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const size_t total = (size_t)BH * DQ * p.Dn;
        hipLaunchKernelGGL((chan_seg_scan_kernel<KG>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, p,
                           DQ, total);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const void *fn = reinterpret_cast<const void *>(&chan_pass_kernel<KG, DQ, FM, false>);
    if ((e = lds_limit(fn, done[0], bytes)) != hipSuccess) return e;
    const dim3 grid((unsigned)((size_t)BH * (p.Dn / 64) * p.nseg));
    hipLaunchKernelGGL((chan_pass_kernel<KG, DQ, FM, false>), grid, dim3(256), bytes, st, p);
    return hipGetLastError();
}

template <int DQ, int FH, bool GG>
hipError_t launch_vg16_dq(const ChanPass &p, int BH, hipStream_t st) {
    static std::atomic<uint64_t> done[2] = {{0}, {0}};
    const int bytes = VgLds<DQ>::BYTES;
    hipError_t e;
    if (p.nseg > 1) {
        const void *fs = reinterpret_cast<const void *>(&chan_vg16_kernel<DQ, FH, true>);
        if ((e = lds_limit(fs, done[1], bytes)) != hipSuccess) return e;
        const dim3 gs((unsigned)((size_t)BH * (p.Dn / 64) * (p.nseg - 1)));
        hipLaunchKernelGGL((chan_vg16_kernel<DQ, FH, true>), gs, dim3(256), bytes, st, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const size_t total = (size_t)BH * DQ * p.Dn;
        hipLaunchKernelGGL((chan_seg_scan_kernel<false>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, p,
                           DQ, total);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const void *fn = reinterpret_cast<const void *>(&chan_vg16_kernel<DQ, FH, false, GG>);
    if ((e = lds_limit(fn, done[0], bytes)) != hipSuccess) return e;
    const dim3 grid((unsigned)((size_t)BH * (p.Dn / 64) * p.nseg));
    hipLaunchKernelGGL((chan_vg16_kernel<DQ, FH, false, GG>), grid, dim3(256), bytes, st, p);
    return hipGetLastError();
}

// A value-gated pass on fp16 operands: FH = 2 (k is the fp16 output gradient) or 1 (q is);
// GG: the pass also forms the log-gate gradient (p.g_out).
template <int FH, bool GG>
hipError_t launch_vg16(const ChanPass &p, int BH, int Dq, hipStream_t st) {
    if (Dq == 64) return launch_vg16_dq<64, FH, GG>(p, BH, st);
    if (Dq == 128) return launch_vg16_dq<128, FH, GG>(p, BH, st);
    return launch_vg16_dq<256, FH, GG>(p, BH, st);
}

template <bool KG, int FM>
hipError_t launch_fm(const ChanPass &p, int BH, int Dq, hipStream_t st) {
    if (Dq == 64) return launch_dq<KG, 64, FM>(p, BH, st);
    if (Dq == 128) return launch_dq<KG, 128, FM>(p, BH, st);
    return launch_dq<KG, 256, FM>(p, BH, st);
}

// The operand dtypes the three passes use: every operand fp32 (fp32 inputs), or bf16 inputs
// with the fp32 output gradient as v (key-gated pass), k or q (value-gated passes).
template <bool KG>
hipError_t launch_pass(const ChanPass &p, int BH, int Dq, hipStream_t st) {
    const int fm = (p.qdt == GLA_DTYPE_F32 ? 1 : 0) | (p.kdt == GLA_DTYPE_F32 ? 2 : 0) |
                   (p.vdt == GLA_DTYPE_F32 ? 4 : 0);
    if (fm == 7) return launch_fm<KG, 7>(p, BH, Dq, st);
    if constexpr (KG) {
        if (fm == 4) return launch_fm<KG, 4>(p, BH, Dq, st);
    } else {
        if (fm == 2) return launch_fm<KG, 2>(p, BH, Dq, st);
        if (fm == 1) return launch_fm<KG, 1>(p, BH, Dq, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// Sequence segments of the passes: about `target` workgroups (value tiles x segments),
// segments of at least 64 tokens, lengths a multiple of 16.  On 256 compute units: the fp32
// pass kernel holds two workgroups per unit (two rounds of 512), the fp16 value-gated kernel
// three (one round of 768; 512, 1024, 1536 and 2048 measured slower).
constexpr int kChanTargetWorkgroups = 1024;
constexpr int kVg16TargetWorkgroups = 768;
// The dk pass that also forms the log-gate gradient holds two workgroups per unit (its
// registers): one round of 512 (768 and 1,024 measured slower).
constexpr int kVg16GateTargetWorkgroups = 512;
void chan_segments(int BH, int L, int Dn, int target, int *nseg, int *seg_len) {
    const long long tiles = (long long)BH * (Dn / 64);
    long long want = (target + tiles - 1) / tiles;
    const long long most = ((long long)L + 63) / 64;
    if (want > most) want = most;
    if (want < 1) want = 1;
    int len = (int)((((long long)L + want - 1) / want + kBlk - 1) / kBlk * kBlk);
    *seg_len = len;
    *nseg = (int)(((long long)L + len - 1) / len);
}

// Scratch floats of the per-channel path beyond the transposed states: the g rows (g_rows:
// fp32 inputs) and the segment totals of the log-gate gradient, the final-state term, and the
// segment states and decays of the passes.
size_t chan_scratch_floats(int BH, int L, int Dk, int Dv, bool g_rows) {
    const size_t ns = ((size_t)L + kSeg - 1) / kSeg;
    size_t n = (g_rows ? (size_t)BH * L * Dk : 0) + (size_t)BH * ns * Dk + (size_t)BH * Dk;
    int s1, l1, s2, l2;
    chan_segments(BH, L, Dv, kChanTargetWorkgroups, &s1, &l1);  // the key-gated pass (value dimension Dv)
    chan_segments(BH, L, Dk, kChanTargetWorkgroups, &s2, &l2);  // the value-gated passes (value dimension Dk)
    int s3 = 0;
    chan_segments(BH, L, Dk, kVg16TargetWorkgroups, &s3, &l2);  // the same on fp16 operands
    s2 = s2 > s3 ? s2 : s3;
    const size_t nsm = (size_t)((s1 > s2 ? s1 : s2) - 1);
    n += (size_t)BH * nsm * Dk * Dv + (size_t)BH * nsm * (Dk > Dv ? Dk : Dv);
    return n;
}

// The three passes and the per-channel log-gate gradient.  s0T = initial^T and dfT =
// dfinal^T ([Dv][Dk], or null), finA [Dk][Dv] and finC [Dv][Dk] receive the first and third
// passes' final states, scratch holds chan_scratch_floats(...) floats.
// skip_dv: the dv pass ran elsewhere (bf16 inputs with Dk <= 128 take it on the forward
// kernel's fp16 path).  fdo, mx (bf16 inputs, else null): the output gradient times s as fp16
// ([BH][L][Dv]) and the scale bits of s per (batch, head); with them the dk and dq passes run
// on fp16 operands (chan_vg16_kernel).
hipError_t chan_backward(const gla_bwd_desc &d, const float *s0T, const float *dfT, float *finA, float *finC,
                         float *scratch, bool skip_dv, const _Float16 *fdo, const uint32_t *mx, hipStream_t st) {
    const int BH = d.B * d.H, L = d.L, Dk = d.Dk, Dv = d.Dv, dt = d.in_dtype;
    hipError_t e;
    const int nsg = (L + kSeg - 1) / kSeg;
    // the log-gate rows exist only where chan_g_kernel forms them (fp32 inputs)
    float *g_rows = scratch;
    float *part = g_rows + (mx ? 0 : (size_t)BH * L * Dk);
    float *fterm = part + (size_t)BH * nsg * Dk;
    float *seg_ws = fterm + (size_t)BH * Dk;
    ChanPass p{};
    p.L = L;
    p.ws_state = seg_ws;
    auto segs = [&](int Dn, int Dq, int target) {
        chan_segments(BH, L, Dn, target, &p.nseg, &p.seg_len);
        p.ws_decay = seg_ws + (size_t)BH * (p.nseg - 1) * Dq * Dn;
    };
    // dv: key-gated, reversed
    p.q = d.k, p.qdt = dt, p.qrev = 1;
    p.k = d.q, p.kdt = dt, p.krev = 1;
    p.v = d.dout, p.vdt = GLA_DTYPE_F32, p.vrev = 1;
    p.vli = nullptr;
    p.la = d.log_alpha, p.grev = 1;
    p.s0 = d.dfinal_state;
    p.out = d.dv, p.orev = 1, p.oli = d.log_ig;
    p.fin = finA;
    p.Dn = Dv;
    segs(Dv, Dk, kChanTargetWorkgroups);
    if (!skip_dv && (e = launch_pass<true>(p, BH, Dk, st)) != hipSuccess) return e;
    const bool h16 = mx != nullptr;
    p.mx = mx;
    p.la = d.log_alpha;
    p.Dn = Dk;
    segs(Dk, Dv, h16 ? kVg16TargetWorkgroups : kChanTargetWorkgroups);
    // dk: value-gated, reversed, keys and values exchanged
    auto dk_pass = [&](bool with_g) {
        p.q = d.v, p.qdt = dt, p.qrev = 1;
        p.k = h16 ? static_cast<const void *>(fdo) : d.dout, p.kdt = GLA_DTYPE_F32, p.krev = 1;
        p.v = d.q, p.vdt = dt, p.vrev = 1;
        p.vli = nullptr;
        p.grev = 1;
        p.s0 = dfT, p.s0_scaled = h16 ? 1 : 0;
        p.out = d.dk, p.orev = 1, p.oli = d.log_ig;
        p.fin = nullptr;
        p.g_dq = with_g ? d.dq : nullptr;
        p.g_k = with_g ? d.k : nullptr;
        p.g_out = with_g ? d.dlog_alpha : nullptr;
        p.g_part = with_g ? part : nullptr;
        p.g_fterm = with_g && dfT ? fterm : nullptr;
        if (!h16) return launch_pass<false>(p, BH, Dv, st);
        return with_g ? launch_vg16<2, true>(p, BH, Dv, st) : launch_vg16<2, false>(p, BH, Dv, st);
    };
    // dq: value-gated, keys and values exchanged, input gate on the values
    auto dq_pass = [&]() {
        p.q = h16 ? static_cast<const void *>(fdo) : d.dout, p.qdt = GLA_DTYPE_F32, p.qrev = 0;
        p.k = d.v, p.kdt = dt, p.krev = 0;
        p.v = d.k, p.vdt = dt, p.vrev = 0;
        p.vli = d.log_ig;
        p.grev = 0;
        p.s0 = s0T, p.s0_scaled = 0;
        p.out = d.dq, p.orev = 0, p.oli = nullptr;
        p.fin = finC;
        p.g_dq = nullptr, p.g_k = nullptr, p.g_out = nullptr, p.g_part = nullptr, p.g_fterm = nullptr;
        return h16 ? launch_vg16<1, false>(p, BH, Dv, st) : launch_pass<false>(p, BH, Dv, st);
    };
    auto fterm_of = [&]() {
        hipLaunchKernelGGL(chan_fterm_kernel, dim3((unsigned)((size_t)BH * (Dk / 64))), dim3(256), 0, st, dfT, finC,
                           fterm, Dk, Dv);
        return hipGetLastError();
    };
    if (h16 && d.dlog_alpha) {
        // the reversed dk pass forms the log-gate gradient: dq and the final-state term first
        if ((e = dq_pass()) != hipSuccess) return e;
        if (dfT && (e = fterm_of()) != hipSuccess) return e;
        segs(Dk, Dv, kVg16GateTargetWorkgroups);
        if ((e = dk_pass(true)) != hipSuccess) return e;
        if (p.nseg > 1) {
            const int chunks = (p.seg_len + 63) / 64;
            const dim3 grid((unsigned)((size_t)BH * (p.nseg - 1) * chunks));
            hipLaunchKernelGGL(chan_gfix_kernel, grid, dim3(256), 0, st, d.dlog_alpha, part, dfT ? fterm : nullptr, L,
                               Dk, p.seg_len, p.nseg, chunks);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if ((e = dk_pass(false)) != hipSuccess) return e;
    if ((e = dq_pass()) != hipSuccess) return e;
    if (d.dlog_alpha) {
        const int nseg = nsg;
        float *g = g_rows;
        if (dfT && (e = fterm_of()) != hipSuccess) return e;
        const dim3 grid_g((unsigned)((size_t)BH * (Dk / 64) * ((nseg + 3) / 4)));
        hipLaunchKernelGGL(chan_g_kernel, grid_g, dim3(256), 0, st, d, dfT ? fterm : nullptr, g, part, nseg);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const dim3 grid((unsigned)((size_t)BH * (Dk / 64) * nseg));
        hipLaunchKernelGGL(chan_scan_kernel, grid, dim3(64), 0, st, d, g, part, nseg);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gla
