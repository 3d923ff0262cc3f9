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
// both in fp32 over 16-token blocks: inside a block every decay factor is formed exactly as
// 2^(b_t - b_s) <= 1 from running log2 decays, and the state is carried from block to block.
// Reversal, the input gate of the values and the output row mapping are index arithmetic on
// the caller's tensors, so the passes need no operand copies.
//
// The per-channel log-gate gradient is the reverse running sum over tokens of
// q_t,d dq_t,d - k_t,d dk_t,d, plus sum_j dfinal[d][j] S_fin[d][j] at the last token
// (chan_g_kernel and chan_scan_kernel: 64-token segments, then carries).

#include <hip/hip_runtime.h>
#include <stdint.h>

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
};

namespace {

constexpr float kLog2eC = 1.4426950408889634f;
constexpr int kBlk = 16;  // tokens per block

__device__ __forceinline__ float ld_in(const void *p, int dt, size_t i) {
    if (dt == GLA_DTYPE_F32) return reinterpret_cast<const float *>(p)[i];
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p)[i] << 16);
}

__device__ __forceinline__ float fexp2c(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier over LDS only: global loads in flight (the next block's operands) are
// not waited for.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum over the 8 consecutive lanes of a row group: quad swaps, then the half-row mirror
// (lane i and 7 - i of each group of eight).
__device__ __forceinline__ float sum8(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
    return x;
}

__device__ __forceinline__ float log2_gate(float la) {
    const float x = la * kLog2eC;
    return x < -150.f ? -150.f : x;
}

// grid = BH * (Dn / 64) workgroups of 512 threads.  Thread tid owns value column
// n = tid >> 3 of the workgroup's 64 and the RD consecutive state rows from r RD, r = tid & 7.
// The operands of the next block are fetched into registers while the current one is
// computed.
constexpr int kThr = 512;
template <bool KG, int DQ>
__global__ __launch_bounds__(kThr) void chan_pass_kernel(ChanPass a) {
    constexpr int RD = DQ / 8;
    constexpr int QP = DQ + 4;            // padded row of q, k and key-side decays (16-byte aligned)
    constexpr int GW = KG ? DQ : 64;      // gate columns of a block
    constexpr int GP = GW + 4;
    constexpr int NQ = kBlk * DQ / kThr;  // q (and k) elements fetched per thread
    constexpr int NG = kBlk * GW / kThr;  // gate elements fetched per thread
    constexpr int NV = kBlk * 64 / kThr;  // value elements fetched per thread
    __shared__ __align__(16) float sQ[kBlk * QP];
    __shared__ __align__(16) float sK[kBlk * QP];
    __shared__ __align__(16) float sB[kBlk * GP];
    __shared__ __align__(16) float sV[kBlk * 64];
    __shared__ __align__(16) float sVf[kBlk * 64];
    __shared__ __align__(16) float sP[kBlk * kBlk];

    const int ndt = a.Dn / 64;
    const size_t bh = blockIdx.x / (unsigned)ndt;
    const int n0 = (int)(blockIdx.x % (unsigned)ndt) * 64;
    const int tid = (int)threadIdx.x, n = tid >> 3, r = tid & 7;
    const int L = a.L, Dn = a.Dn;
    const int Dg = KG ? DQ : Dn;
    const int d0 = r * RD;

    float S[RD];
#pragma unroll
    for (int i = 0; i < RD; ++i) S[i] = a.s0 ? a.s0[(bh * DQ + d0 + i) * Dn + n0 + n] : 0.f;

    float fq[NQ], fk[NQ], fg[NG], fv[NV];
    // operands of the block at u0 (zero past the sequence end) and per-token log2 gates
    auto fetch = [&](int u0) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int idx = tid + j * kThr, t = idx / DQ, d = idx % DQ, u = u0 + t;
            fq[j] = fk[j] = 0.f;
            if (u < L) {
                const size_t rq = bh * L + (a.qrev ? L - 1 - u : u), rk = bh * L + (a.krev ? L - 1 - u : u);
                fq[j] = ld_in(a.q, a.qdt, rq * DQ + d);
                fk[j] = ld_in(a.k, a.kdt, rk * DQ + d);
            }
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int idx = tid + j * kThr, t = idx >> 6, c = idx & 63, u = u0 + t;
            fv[j] = 0.f;
            if (u < L) {
                const size_t rv = bh * L + (a.vrev ? L - 1 - u : u);
                fv[j] = ld_in(a.v, a.vdt, rv * Dn + n0 + c);
                if (a.vli) fv[j] *= fexp2c(a.vli[rv] * kLog2eC);
            }
        }
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const int idx = tid + j * kThr, t = idx / GW, c = idx % GW, u = u0 + t;
            fg[j] = 0.f;
            if (u < L && !(a.grev && u == 0)) {
                const size_t rg = bh * L + (a.grev ? L - u : u);
                fg[j] = log2_gate(a.la[rg * Dg + (KG ? c : n0 + c)]);
            }
        }
    };
    fetch(0);

    for (int u0 = 0; u0 < L; u0 += kBlk) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int idx = tid + j * kThr, t = idx / DQ, d = idx % DQ;
            sQ[t * QP + d] = fq[j];
            sK[t * QP + d] = fk[j];
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) sV[tid + j * kThr] = fv[j];
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const int idx = tid + j * kThr;
            sB[(idx / GW) * GP + idx % GW] = fg[j];
        }
        lds_sync();
        if (u0 + kBlk < L) fetch(u0 + kBlk);
        // running log2 decay inside the block, inclusive
        if (tid < GW) {
            float b[kBlk];
#pragma unroll
            for (int t = 0; t < kBlk; ++t) b[t] = sB[t * GP + tid];
            float run = 0.f;
#pragma unroll
            for (int t = 0; t < kBlk; ++t) {
                run += b[t];
                sB[t * GP + tid] = run;
            }
        }
        lds_sync();
        // ---- scores P[t][s] (s <= t); the key gate enters them exactly
        if (tid < kBlk * kBlk) {
            const int t = tid >> 4, s = tid & 15;
            float p = 0.f;
            if (s <= t) {
#pragma unroll 4
                for (int d = 0; d < DQ; d += 4) {
                    const float4 x = *reinterpret_cast<const float4 *>(sQ + t * QP + d);
                    const float4 y = *reinterpret_cast<const float4 *>(sK + s * QP + d);
                    if constexpr (KG) {
                        const float4 bt = *reinterpret_cast<const float4 *>(sB + t * GP + d);
                        const float4 bs = *reinterpret_cast<const float4 *>(sB + s * GP + d);
                        p += x.x * y.x * fexp2c(bt.x - bs.x) + x.y * y.y * fexp2c(bt.y - bs.y) +
                             x.z * y.z * fexp2c(bt.z - bs.z) + x.w * y.w * fexp2c(bt.w - bs.w);
                    } else {
                        p += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
                    }
                }
            }
            sP[t * kBlk + s] = p;
        }
        lds_sync();
        // ---- decay-weighted operands: key gate: q_t 2^(b_t), k_s 2^(b_15 - b_s); value gate:
        // v_s 2^(b_15 - b_s)
        if constexpr (KG) {
            for (int idx = tid; idx < kBlk * DQ; idx += kThr) {
                const int t = idx / DQ, d = idx % DQ;
                sQ[t * QP + d] *= fexp2c(sB[t * GP + d]);
                sK[t * QP + d] *= fexp2c(sB[(kBlk - 1) * GP + d] - sB[t * GP + d]);
            }
        } else {
            for (int idx = tid; idx < kBlk * 64; idx += kThr) {
                const int t = idx >> 6, c = idx & 63;
                sVf[idx] = sV[idx] * fexp2c(sB[(kBlk - 1) * GP + c] - sB[t * GP + c]);
            }
        }
        lds_sync();
        // ---- outputs: the entering state's term, reduced over the eight row groups, plus the
        // block's own tokens
        float acc[kBlk];
#pragma unroll
        for (int t = 0; t < kBlk; ++t) {
            float x = 0.f;
#pragma unroll
            for (int i = 0; i < RD; i += 4) {
                const float4 q4 = *reinterpret_cast<const float4 *>(sQ + t * QP + d0 + i);
                x += q4.x * S[i] + q4.y * S[i + 1] + q4.z * S[i + 2] + q4.w * S[i + 3];
            }
            acc[t] = x;
        }
#pragma unroll
        for (int t = 0; t < kBlk; ++t) acc[t] = sum8(acc[t]);
        float vcol[kBlk];
#pragma unroll
        for (int s = 0; s < kBlk; ++s) vcol[s] = sV[s * 64 + n];
        // lane r of the group finishes tokens r and r + 8 (no divergence: selects, and a fixed
        // loop over the block's tokens with the causal mask as a select)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int t = r + 8 * h;
            float o = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) o = (r == j) ? acc[j + 8 * h] : o;
            const float4 *prow = reinterpret_cast<const float4 *>(sP + t * kBlk);
            float pr[kBlk];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 p4 = prow[j];
                pr[4 * j] = p4.x, pr[4 * j + 1] = p4.y, pr[4 * j + 2] = p4.z, pr[4 * j + 3] = p4.w;
            }
            if constexpr (KG) {
#pragma unroll
                for (int s2 = 0; s2 < kBlk; ++s2) o += pr[s2] * vcol[s2];  // P is zero above the diagonal
            } else {
                const float bt = sB[t * GP + n];
                o *= fexp2c(bt);
#pragma unroll
                for (int s2 = 0; s2 < kBlk; ++s2) {
                    const float f = s2 <= t ? fexp2c(bt - sB[s2 * GP + n]) : 0.f;
                    o += pr[s2] * vcol[s2] * f;
                }
            }
            const int u = u0 + t;
            if (u < L) {
                const size_t dst = bh * L + (a.orev ? L - 1 - u : u);
                if (a.oli) o *= fexp2c(a.oli[dst] * kLog2eC);
                a.out[dst * Dn + n0 + n] = o;
            }
        }
        // ---- state to the block end
        if constexpr (KG) {
#pragma unroll
            for (int i = 0; i < RD; i += 4) {
                const float4 dec = *reinterpret_cast<const float4 *>(sB + (kBlk - 1) * GP + d0 + i);
                float x0 = S[i] * fexp2c(dec.x), x1 = S[i + 1] * fexp2c(dec.y);
                float x2 = S[i + 2] * fexp2c(dec.z), x3 = S[i + 3] * fexp2c(dec.w);
#pragma unroll
                for (int s = 0; s < kBlk; ++s) {
                    const float4 k4 = *reinterpret_cast<const float4 *>(sK + s * QP + d0 + i);
                    x0 += k4.x * vcol[s];
                    x1 += k4.y * vcol[s];
                    x2 += k4.z * vcol[s];
                    x3 += k4.w * vcol[s];
                }
                S[i] = x0, S[i + 1] = x1, S[i + 2] = x2, S[i + 3] = x3;
            }
        } else {
            const float dec = fexp2c(sB[(kBlk - 1) * GP + n]);
            float vf[kBlk];
#pragma unroll
            for (int s = 0; s < kBlk; ++s) vf[s] = sVf[s * 64 + n];
#pragma unroll
            for (int i = 0; i < RD; i += 4) {
                float x0 = S[i] * dec, x1 = S[i + 1] * dec, x2 = S[i + 2] * dec, x3 = S[i + 3] * dec;
#pragma unroll
                for (int s = 0; s < kBlk; ++s) {
                    const float4 k4 = *reinterpret_cast<const float4 *>(sK + s * QP + d0 + i);
                    x0 += k4.x * vf[s];
                    x1 += k4.y * vf[s];
                    x2 += k4.z * vf[s];
                    x3 += k4.w * vf[s];
                }
                S[i] = x0, S[i + 1] = x1, S[i + 2] = x2, S[i + 3] = x3;
            }
        }
        lds_sync();
    }
    if (a.fin) {
#pragma unroll
        for (int i = 0; i < RD; ++i) a.fin[(bh * DQ + d0 + i) * Dn + n0 + n] = S[i];
    }
}

// fterm[bh][d] = sum_j dfT[bh][j][d] finC[bh][j][d] (both [Dv][Dk]): the final-state term
// of channel d's log-gate gradient.  One thread per (bh, d).
__global__ __launch_bounds__(256) void chan_fterm_kernel(const float *dfT, const float *finC, float *fterm, int Dk,
                                                        int Dv, size_t total) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const size_t bh = i / (size_t)Dk;
    const int d = (int)(i % (size_t)Dk);
    const size_t base = bh * (size_t)Dv * Dk + d;
    float s = 0.f;
    for (int j = 0; j < Dv; ++j) s += dfT[base + (size_t)j * Dk] * finC[base + (size_t)j * Dk];
    fterm[i] = s;
}

constexpr int kSeg = 64;  // tokens per segment of the log-gate scan

// g[bh][t][d] = q dq - k dk (+ fterm at the last token) and the segment totals
// part[bh][seg][d].  Workgroup = 64 channels of one (bh, segment).
__global__ __launch_bounds__(64) void chan_g_kernel(gla_bwd_desc d, const float *fterm, float *g, float *part,
                                                   int nseg) {
    const int ndt = d.Dk / 64;
    size_t id = blockIdx.x;
    const int seg = (int)(id % (unsigned)nseg);
    id /= (unsigned)nseg;
    const int dt = (int)(id % (unsigned)ndt);
    const size_t bh = id / (unsigned)ndt;
    const int c = dt * 64 + (int)threadIdx.x;
    const int L = d.L, Dk = d.Dk;
    const int t0 = seg * kSeg, t1 = min(L, t0 + kSeg);
    float sum = 0.f;
    for (int t = t0; t < t1; ++t) {
        const size_t i = (bh * L + t) * Dk + c;
        float x = ld_in(d.q, d.in_dtype, i) * d.dq[i] - ld_in(d.k, d.in_dtype, i) * d.dk[i];
        if (t == L - 1 && fterm) x += fterm[bh * Dk + c];
        g[i] = x;
        sum += x;
    }
    part[(bh * nseg + seg) * Dk + c] = sum;
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

inline unsigned nblkc(size_t n, unsigned per) { return (unsigned)((n + per - 1) / per); }

template <bool KG>
hipError_t launch_pass(const ChanPass &p, int BH, int Dq, hipStream_t st) {
    const dim3 grid((unsigned)((size_t)BH * (p.Dn / 64)));
    if (Dq == 64) hipLaunchKernelGGL((chan_pass_kernel<KG, 64>), grid, dim3(kThr), 0, st, p);
    else if (Dq == 128) hipLaunchKernelGGL((chan_pass_kernel<KG, 128>), grid, dim3(kThr), 0, st, p);
    else hipLaunchKernelGGL((chan_pass_kernel<KG, 256>), grid, dim3(kThr), 0, st, p);
    return hipGetLastError();
}

}  // namespace

// Scratch floats of the per-channel path beyond the transposed states: the g rows and the
// segment totals.
size_t chan_scratch_floats(int BH, int L, int Dk) {
    const size_t nseg = ((size_t)L + kSeg - 1) / kSeg;
    return (size_t)BH * L * Dk + (size_t)BH * nseg * Dk + (size_t)BH * Dk;
}

// The three passes and the per-channel log-gate gradient.  s0T = initial^T and dfT =
// dfinal^T ([Dv][Dk], or null), finA [Dk][Dv] and finC [Dv][Dk] receive the first and third
// passes' final states, scratch holds chan_scratch_floats(...) floats.
hipError_t chan_backward(const gla_bwd_desc &d, const float *s0T, const float *dfT, float *finA, float *finC,
                         float *scratch, hipStream_t st) {
    const int BH = d.B * d.H, L = d.L, Dk = d.Dk, Dv = d.Dv, dt = d.in_dtype;
    hipError_t e;
    ChanPass p{};
    p.L = L;
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
    if ((e = launch_pass<true>(p, BH, Dk, st)) != hipSuccess) return e;
    // dk: value-gated, reversed, keys and values exchanged
    p.q = d.v, p.qdt = dt, p.qrev = 1;
    p.k = d.dout, p.kdt = GLA_DTYPE_F32, p.krev = 1;
    p.v = d.q, p.vdt = dt, p.vrev = 1;
    p.s0 = dfT;
    p.out = d.dk;
    p.fin = nullptr;
    p.Dn = Dk;
    if ((e = launch_pass<false>(p, BH, Dv, st)) != hipSuccess) return e;
    // dq: value-gated, keys and values exchanged, input gate on the values
    p.q = d.dout, p.qdt = GLA_DTYPE_F32, p.qrev = 0;
    p.k = d.v, p.kdt = dt, p.krev = 0;
    p.v = d.k, p.vdt = dt, p.vrev = 0;
    p.vli = d.log_ig;
    p.grev = 0;
    p.s0 = s0T;
    p.out = d.dq, p.orev = 0, p.oli = nullptr;
    p.fin = finC;
    if ((e = launch_pass<false>(p, BH, Dv, st)) != hipSuccess) return e;
    if (d.dlog_alpha) {
        const int nseg = (L + kSeg - 1) / kSeg;
        float *g = scratch;
        float *part = g + (size_t)BH * L * Dk;
        float *fterm = part + (size_t)BH * nseg * Dk;
        if (dfT) {
            const size_t total = (size_t)BH * Dk;
            hipLaunchKernelGGL(chan_fterm_kernel, dim3(nblkc(total, 256)), dim3(256), 0, st, dfT, finC, fterm, Dk, Dv,
                               total);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        const dim3 grid((unsigned)((size_t)BH * (Dk / 64) * nseg));
        hipLaunchKernelGGL(chan_g_kernel, grid, dim3(64), 0, st, d, dfT ? fterm : nullptr, g, part, nseg);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(chan_scan_kernel, grid, dim3(64), 0, st, d, g, part, nseg);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gla
