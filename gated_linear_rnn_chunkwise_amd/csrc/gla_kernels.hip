// gla_kernels.hip -- gfx950 kernels of the chunkwise gated linear attention forward pass.
//
// The chunkwise algorithm [Hardware-Efficient Training of Linear Attention Models, talk
// summary, 11:58]: tokens are grouped into chunks; within a chunk the causal pairwise term
// is a masked product of score and value matrices, and the state from earlier chunks
// enters through one product with the chunk's queries; the state itself is only formed at
// chunk boundaries, where the sum of key-value outer products is one matrix product.
// Chunks larger than 64 tokens are split again into 64-token query and key tiles
// [Tiled Flash Linear Attention, abstract].
//
// Three kernels:
//  * segment_state_kernel -- for each sequence segment but the last, the state the
//    segment alone produces from a zero state (chunk states summed with their decay), and
//    the segment's total decay.
//  * segment_scan_kernel  -- carries the state across segments (sequential over segments,
//    parallel over state elements), giving every segment its incoming state.
//  * chunk_output_kernel  -- per segment, walks its chunks in order with the state held in
//    registers: output of each chunk (intra-chunk masked term plus the incoming state),
//    then the state update.  The last segment also writes the final state.
// With one segment (enough (batch, head, value-tile) work to fill the GPU) only the last
// kernel runs and no state ever goes to memory.
//
// Numerics.  Gates are applied in the product domain: per-step decays alpha = 2^(log2e *
// log_alpha) are multiplied into running products, so every factor that multiplies an
// operand is <= 1, except the key factor of a diagonal 16x16 block, which is bounded by
// the block's own decay span (checked; a block whose span is too large is computed exactly
// on the vector ALU instead).  Scalar gates (none / per head) keep q and k raw in the
// score product and multiply each score by its exact decay afterwards.  Operands computed
// from bf16 inputs are fp16 (range-checked by construction); fp32 inputs keep fp32
// operands.  Accumulation, states and outputs are fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gla.h"
#include "gla_layout.h"

namespace gla {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------------------------
// Instance configuration.
template <bool F32_, int DK_, bool CH_, bool MT_>
struct Cfg {
    static constexpr bool F32 = F32_;  // fp32 inputs and operands (else bf16 inputs, fp16 operands)
    static constexpr int DK = DK_;
    static constexpr bool CH = CH_;    // per-channel gate
    static constexpr bool MT = MT_;    // chunk of several 64-token tiles
    using OpT = typename std::conditional<F32, float, f16>::type;
    using Frag = typename std::conditional<F32, f32x8, f16x8>::type;
    using Half = typename std::conditional<F32, f32x4, f16x4>::type;
    using InT = typename std::conditional<F32, float, uint16_t>::type;
    static constexpr int OPB = F32 ? 4 : 2;
    static constexpr int CPL = (!F32 && DK >= 128) ? 2 : 1;
    static constexpr int SLAB = 64 * CPL;
    static constexpr int NSLAB = DK / SLAB;
    static constexpr int RP = SLAB + 16 / OPB;  // +16 B per row against LDS bank conflicts
    static constexpr int KTP = 64 + 16 / OPB;
    static constexpr int NBD = DK / 16;         // 16-row blocks of the state
    static constexpr int KSTEP = SLAB / 32;     // 32-deep MFMA steps per slab
    static constexpr int NBS = SLAB / 16;       // 16-row state blocks per slab
    // Smallest decay of a 16-token sub-block whose diagonal block still uses the matrix
    // cores: the key operand there is scaled by up to 1/decay (2^8 for fp16 operands).
    static constexpr float kMinDiagDecay = F32 ? 1e-30f : 0.00390625f;
};

// ------------------------------------------------------------------------------------
// Small device helpers.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}
__device__ __forceinline__ float scan_incl(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// Hardware dispatches workgroup i to XCD i % 8; give consecutive logical workgroups (which
// share q, k and gate reads through L2) the same XCD.
__device__ __forceinline__ int xcd_remap(int i, int n) {
    if ((n & 7) != 0) return i;
    return (i & 7) * (n >> 3) + (i >> 3);
}

__device__ __forceinline__ f32x4 mma(const f16x8 &a, const f16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// Same contraction with fp32 operands: element e of every lane's 8 values forms one
// 16x16x4 product, so the eight products cover the 32 slots in the same pairing.
__device__ __forceinline__ f32x4 mma(const f32x8 &a, const f32x8 &b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}

template <class T>
__device__ __forceinline__ T lds_ld(const void *p) {
    return *reinterpret_cast<const T *>(p);
}

// 8 consecutive operands (16 B fp16, 32 B fp32) from LDS.
template <class C>
__device__ __forceinline__ typename C::Frag ld8(const typename C::OpT *p) {
    if constexpr (C::F32) {
        const f32x4 a = lds_ld<f32x4>(p), b = lds_ld<f32x4>(p + 4);
        return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
        return lds_ld<f16x8>(p);
    }
}
// Two groups of 4 consecutive operands.
template <class C>
__device__ __forceinline__ typename C::Frag ld4x2(const typename C::OpT *p0, const typename C::OpT *p1) {
    using H = typename C::Half;
    const H a = lds_ld<H>(p0), b = lds_ld<H>(p1);
    return typename C::Frag{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <class C>
__device__ __forceinline__ typename C::Frag scale8(const typename C::Frag &f, const f32x4 &s0, const f32x4 &s1) {
    using OpT = typename C::OpT;
    typename C::Frag r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (OpT)((float)f[e] * s0[e]);
        r[e + 4] = (OpT)((float)f[e + 4] * s1[e]);
    }
    return r;
}

// ------------------------------------------------------------------------------------
// Raw input of one unit (64-token tile x one slab of key channels), prefetched into
// registers.  Thread (wave w, lane) holds rows 16w..16w+15 of the tile for its CPL key
// channels; value pieces are rows 4*(tid>>4)+e, columns 4*(tid&15)..+3 of the 64x64 tile.
template <bool F32, int CPL>
struct InPack;
template <>
struct InPack<false, 2> {
    uint32_t x;
    __device__ float get(int c) const { return c == 0 ? __uint_as_float(x << 16) : __uint_as_float(x & 0xffff0000u); }
};
template <>
struct InPack<false, 1> {
    uint16_t x;
    __device__ float get(int) const { return bf16_to_f32(x); }
};
template <>
struct InPack<true, 1> {
    float x;
    __device__ float get(int) const { return x; }
};

template <bool F32>
struct VPiece;
template <>
struct VPiece<false> {
    uint2 x;
    __device__ float get(int j) const {
        const uint32_t w = (j < 2) ? x.x : x.y;
        return (j & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    }
};
template <>
struct VPiece<true> {
    float4 x;
    __device__ float get(int j) const { return j == 0 ? x.x : j == 1 ? x.y : j == 2 ? x.z : x.w; }
};

template <class C>
struct Raw {
    InPack<C::F32, C::CPL> q[16], k[16];
    float la[C::CH ? 16 : 1][C::CPL];
    float las, lis;  // scalar log gate / log input gate of row (tile start + lane)
    VPiece<C::F32> v[4];
};

// Per-(batch, head) base pointers and gate addressing.
template <class C>
struct Base {
    const typename C::InT *q, *k, *v;
    const float *la;  // per-channel: [L][Dk]; head: [L]; head_const: one value; none: null
    const float *li;  // [L] or null
    int L, Dv, gate;
};

template <class C, bool WQ>
__device__ __forceinline__ void load_unit(Raw<C> &r, const Base<C> &b, int T0, int sl, bool with_v, int w,
                                          int lane, int tid, int dv0) {
    using P = InPack<C::F32, C::CPL>;
    const int ch0 = sl * C::SLAB + C::CPL * lane;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const int t = T0 + 16 * w + rr;
        const bool ok = t < b.L;
        const size_t off = (size_t)t * C::DK + ch0;
        if constexpr (WQ) r.q[rr].x = ok ? *reinterpret_cast<const decltype(P::x) *>(b.q + off) : decltype(P::x)(0);
        r.k[rr].x = ok ? *reinterpret_cast<const decltype(P::x) *>(b.k + off) : decltype(P::x)(0);
        if constexpr (C::CH) {
            if constexpr (C::CPL == 2) {
                const float2 g2 = ok ? *reinterpret_cast<const float2 *>(b.la + off) : make_float2(0.f, 0.f);
                r.la[rr][0] = g2.x;
                r.la[rr][1] = g2.y;
            } else {
                r.la[rr][0] = ok ? b.la[off] : 0.f;
            }
        }
    }
    {
        const int t = T0 + lane;
        const bool ok = t < b.L;
        float x = 0.f;
        if constexpr (!C::CH) {
            if (ok && b.gate == GLA_GATE_HEAD) x = b.la[t];
            if (ok && b.gate == GLA_GATE_HEAD_CONST) x = b.la[0];
        }
        r.las = x;
        r.lis = (ok && b.li) ? b.li[t] : 0.f;
    }
    if (with_v) {
        const int c0 = dv0 + 4 * (tid & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = T0 + 4 * (tid >> 4) + e;
            const bool ok = t < b.L;
            const typename C::InT *p = b.v + (size_t)t * b.Dv + c0;
            if constexpr (C::F32)
                r.v[e].x = ok ? *reinterpret_cast<const float4 *>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
            else
                r.v[e].x = ok ? *reinterpret_cast<const uint2 *>(p) : make_uint2(0u, 0u);
        }
    }
}

// Value tile into LDS in MFMA operand order: [p][g][c][8], element (hh*4+e) of slot
// (p, g, c) is row 32p + 16hh + 4g + e, column c.  Thread tid holds rows 4*(tid>>4)+e.
template <class C>
__device__ __forceinline__ void v_to_lds(const Raw<C> &r, typename C::OpT *sV, int tid) {
    using OpT = typename C::OpT;
    using H = typename C::Half;
    const int quad = tid >> 4;  // rows 4*quad .. 4*quad+3
    const int p = quad >> 3, hh = (quad >> 2) & 1, g = quad & 3;
    const int c0 = 4 * (tid & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        H h4;
#pragma unroll
        for (int e = 0; e < 4; ++e) h4[e] = (OpT)r.v[e].get(j);
        *reinterpret_cast<H *>(sV + ((p * 4 + g) * 64 + c0 + j) * 8 + hh * 4) = h4;
    }
}

// Slot of token s (0..63 in the tile) in the k-slot order of the value and key^T operands.
__device__ __forceinline__ int kslot(int s) { return (((s >> 5) * 4 + ((s >> 2) & 3)) * 8) + ((s >> 4) & 1) * 4 + (s & 3); }

// ------------------------------------------------------------------------------------
// Gate preparation for one unit, per-channel gate.  Thread rows r of sub-block w.
// Outputs (all factors <= 1 except 1/ablk):
//   eq[r] = decay from the sub-block start through row r (inclusive), ek[r] = decay after
//   row r to the sub-block end; ablk/ainv in LDS; pre = decay of the sub-blocks before w,
//   post = after w; at = decay of the whole tile.
template <class C>
struct ChGate {
    float eq[16][C::CPL], ek[16][C::CPL];
    float pre[C::CPL], post[C::CPL], at[C::CPL];
    bool harsh;
};

template <class C>
__device__ __forceinline__ void ch_gate(ChGate<C> &G, const Raw<C> &r, float *sAb, float *sAi, int w, int lane) {
    float al[16][C::CPL];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
#pragma unroll
        for (int c = 0; c < C::CPL; ++c) al[rr][c] = fexp2(r.la[rr][c] * kLog2e);
#pragma unroll
    for (int c = 0; c < C::CPL; ++c) {
        float run = 1.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            run *= al[rr][c];
            G.eq[rr][c] = run;
        }
        run = 1.f;
#pragma unroll
        for (int rr = 15; rr >= 0; --rr) {
            G.ek[rr][c] = run;
            run *= al[rr][c];
        }
    }
    bool small = false;
#pragma unroll
    for (int c = 0; c < C::CPL; ++c) {
        const float aw = G.eq[15][c];
        sAb[w * C::SLAB + C::CPL * lane + c] = aw;
        sAi[w * C::SLAB + C::CPL * lane + c] = frcp(aw);
        small |= !(aw >= C::kMinDiagDecay);
    }
    G.harsh = __ballot(small) != 0ull;
    lds_barrier();
#pragma unroll
    for (int c = 0; c < C::CPL; ++c) {
        float pre = 1.f, post = 1.f, all = 1.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float au = sAb[u * C::SLAB + C::CPL * lane + c];
            all *= au;
            if (u < w) pre *= au;
            if (u > w) post *= au;
        }
        G.pre[c] = pre;
        G.post[c] = post;
        G.at[c] = all;
    }
}

// Exact diagonal 16x16 score block of sub-block w over this slab's channels, for a
// sub-block whose decay span is too large for scaled matrix-core operands: every pair
// s <= t gets sum_d q_td k_sd 2^(u_td - u_sd) i_s with u the log2 running decay.
template <class C>
__device__ void ch_diag_exact(f32x4 &acc, const Raw<C> &r, const float ig[16], int lane) {
    float u[16][C::CPL];
#pragma unroll
    for (int c = 0; c < C::CPL; ++c) {
        float run = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            run += r.la[rr][c] * kLog2e;
            u[rr][c] = run;
        }
    }
    const int c16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
#pragma unroll
        for (int t = s; t < 16; ++t) {
            float part = 0.f;
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) part += r.q[t].get(c) * r.k[s].get(c) * fexp2(u[t][c] - u[s][c]);
            const float tot = wave_sum(part * ig[s]);
            if (c16 == t && g == (s >> 2)) acc[s & 3] += tot;
        }
    }
}

// ------------------------------------------------------------------------------------
// The pairs of 16-token blocks (query block i, key block j <= i) of a diagonal tile that
// each wave computes; wave w always owns the diagonal pair (w, w).
__device__ __forceinline__ void pair_of(int w, int k, int &i, int &j) {
    // k = 0: (w, w); k = 1, 2: off-diagonal pairs; (-1) when absent.
    const int tab[4][2][2] = {{{1, 0}, {3, 2}}, {{2, 0}, {3, 1}}, {{2, 1}, {-1, -1}}, {{3, 0}, {-1, -1}}};
    if (k == 0) {
        i = w;
        j = w;
    } else {
        i = tab[w][k - 1][0];
        j = tab[w][k - 1][1];
    }
}

// ------------------------------------------------------------------------------------
// chunk_output_kernel: grid = BH * nseg * ndv workgroups of 256 threads.
template <class C>
__global__ __launch_bounds__(256, 1) void chunk_output_kernel(KArgs a) {
    using OpT = typename C::OpT;
    using Frag = typename C::Frag;
    using InT = typename C::InT;
    extern __shared__ __align__(256) unsigned char smem[];
    const LdsPlan lp = lds_plan(C::OPB, C::DK, C::CH, a.nt);
    OpT *sQ = reinterpret_cast<OpT *>(smem + lp.q);
    OpT *sK = reinterpret_cast<OpT *>(smem + lp.k);
    OpT *sQI = reinterpret_cast<OpT *>(smem + lp.qi);
    OpT *sKT = reinterpret_cast<OpT *>(smem + lp.kst);
    OpT *sP = reinterpret_cast<OpT *>(smem + lp.pbuf);
    OpT *sV = reinterpret_cast<OpT *>(smem + lp.vb);
    OpT *sVo = reinterpret_cast<OpT *>(smem + lp.voff);
    OpT *sPK = reinterpret_cast<OpT *>(smem + lp.prevke);
    float *sAb = reinterpret_cast<float *>(smem + lp.ablk);
    float *sAi = reinterpret_cast<float *>(smem + lp.ainv);
    float *sQTF = reinterpret_cast<float *>(smem + lp.qtf);
    float *sAt = reinterpret_cast<float *>(smem + lp.atile);
    float *sBr = reinterpret_cast<float *>(smem + lp.brow);
    float *sLr = reinterpret_cast<float *>(smem + lp.lrow);

    int id = xcd_remap((int)blockIdx.x, a.nwg);
    const int dvt = id % a.ndv;
    id /= a.ndv;
    const int seg = id % a.nseg;
    const int bh = id / a.nseg;
    const int h = bh % a.H;
    const int tid = (int)threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = a.L, Dv = a.Dv;
    const int dv0 = dvt * kDvTile;
    const int col = dv0 + 16 * w + c16;  // value column of this lane's accumulators
    const int t_begin = seg * a.seg_len;
    const int t_end = min(L, t_begin + a.seg_len);
    const size_t bhL = (size_t)bh * L;

    Base<C> b;
    b.q = reinterpret_cast<const InT *>(a.q) + bhL * C::DK;
    b.k = reinterpret_cast<const InT *>(a.k) + bhL * C::DK;
    b.v = reinterpret_cast<const InT *>(a.v) + bhL * Dv;
    b.la = a.gate == GLA_GATE_CHANNEL ? a.la + bhL * C::DK
           : a.gate == GLA_GATE_HEAD  ? a.la + bhL
           : a.gate == GLA_GATE_HEAD_CONST ? a.la + h
                                           : nullptr;
    b.li = a.li ? a.li + bhL : nullptr;
    b.L = L;
    b.Dv = Dv;
    b.gate = a.gate;

    // State S[d][col], d = 16n + 4g + e, held across chunks in registers.
    f32x4 S[C::NBD];
#pragma unroll
    for (int n = 0; n < C::NBD; ++n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int d = 16 * n + 4 * g + e;
            float x = 0.f;
            if (seg > 0)
                x = a.ws_state[(((size_t)bh * (a.nseg - 1) + (seg - 1)) * C::DK + d) * Dv + col];
            else if (a.s0)
                x = a.s0[((size_t)bh * C::DK + d) * Dv + col];
            S[n][e] = x;
        }
    }
    f32x4 dS[C::MT ? C::NBD : 1];

    Raw<C> raw;
    if (t_begin < t_end) load_unit<C, true>(raw, b, t_begin, 0, true, w, lane, tid, dv0);

    for (int c0 = t_begin; c0 < t_end; c0 += a.chunk) {
        float Wc[C::NSLAB][C::CPL];  // per-channel decay from the chunk start to the tile start
#pragma unroll
        for (int s = 0; s < C::NSLAB; ++s)
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) Wc[s][c] = 1.f;
        float Bc = 0.f;  // scalar gates: log2 decay from the chunk start to the tile start
        if constexpr (C::MT) {
#pragma unroll
            for (int n = 0; n < C::NBD; ++n) dS[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const int ntile = min(a.nt, (t_end - c0 + kTile - 1) / kTile);

        for (int tau = 0; tau < ntile; ++tau) {
            const int T0 = c0 + kTile * tau;
            f32x4 O[4];
            f32x4 Pd[3];
#pragma unroll
            for (int i = 0; i < 4; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 3; ++i) Pd[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            float Tt = 0.f;  // scalar gates: log2 decay across this tile

#pragma unroll 1
            for (int sl = 0; sl < C::NSLAB; ++sl) {
                OpT *sQs = sQ + (C::MT ? sl : 0) * 64 * C::RP;
                bool harsh = false;
                float ekr[16];  // scalar gates: key factor (tile end reference, input gate)
                // ---------------- preparation of this unit -> LDS
                if (sl == 0) v_to_lds<C>(raw, sV, tid);
                if constexpr (C::CH) {
                    ChGate<C> G;
                    ch_gate<C>(G, raw, sAb, sAi, w, lane);
                    harsh = G.harsh;
                    float ig[16];
                    {
                        const float y = raw.lis * kLog2e;
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) ig[rr] = fexp2(__shfl(y, 16 * w + rr));
                    }
                    if (harsh) ch_diag_exact<C>(Pd[0], raw, ig, lane);
                    float fqi[C::CPL];
#pragma unroll
                    for (int c = 0; c < C::CPL; ++c) {
                        fqi[c] = Wc[sl][c] * G.pre[c];
                        const int d = sl * C::SLAB + C::CPL * lane + c;
                        if (w == 0) sAt[tau * C::DK + d] = G.at[c];
                        if constexpr (C::MT) sQTF[w * C::DK + d] = G.pre[c];
                        Wc[sl][c] *= G.at[c];
                    }
                    const int chl = C::CPL * lane;
                    OpT *pk = nullptr;
                    if constexpr (C::MT) {
                        if (tau < a.nt - 1) pk = sPK + (size_t)((tau * C::NSLAB + sl) * 64) * C::RP;
                    }
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        typename C::Half kt4[C::CPL];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int rr = 4 * g4 + e;
                            const int row = 16 * w + rr;
                            OpT qd[C::CPL], ko[C::CPL], qi[C::CPL], ke[C::CPL];
#pragma unroll
                            for (int c = 0; c < C::CPL; ++c) {
                                const float qf = raw.q[rr].get(c) * G.eq[rr][c];
                                const float kf = raw.k[rr].get(c) * G.ek[rr][c] * ig[rr];
                                qd[c] = (OpT)qf;
                                ko[c] = (OpT)kf;
                                qi[c] = (OpT)(qf * fqi[c]);
                                ke[c] = (OpT)(kf * G.post[c]);
                                kt4[c][e] = ke[c];
                            }
#pragma unroll
                            for (int c = 0; c < C::CPL; ++c) {
                                sQs[row * C::RP + chl + c] = qd[c];
                                sK[row * C::RP + chl + c] = ko[c];
                                sQI[row * C::RP + chl + c] = qi[c];
                                if constexpr (C::MT) {
                                    if (pk) pk[row * C::RP + chl + c] = ke[c];
                                }
                            }
                        }
#pragma unroll
                        for (int c = 0; c < C::CPL; ++c)
                            *reinterpret_cast<typename C::Half *>(sKT + (chl + c) * C::KTP + kslot(16 * w + 4 * g4)) =
                                kt4[c];
                    }
                } else {
                    // scalar gates: running log2 decay over the tile's rows (lane = row)
                    const float x = raw.las * kLog2e;
                    const float y = raw.lis * kLog2e;
                    const float bl = scan_incl(x, lane);
                    Tt = __shfl(bl, 63);
                    if (w == 0 && sl == 0) {
                        sBr[kTile * tau + lane] = Bc + bl;
                        sLr[kTile * tau + lane] = y;
                    }
                    float eb[16];
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) {
                        const float blr = __shfl(bl, 16 * w + rr);
                        const float yr = __shfl(y, 16 * w + rr);
                        eb[rr] = fexp2(Bc + blr);
                        ekr[rr] = fexp2(Tt - blr + yr);
                    }
                    const int chl = C::CPL * lane;
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        typename C::Half kt4[C::CPL];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int rr = 4 * g4 + e;
                            const int row = 16 * w + rr;
#pragma unroll
                            for (int c = 0; c < C::CPL; ++c) {
                                const float qf = raw.q[rr].get(c);
                                const float kf = raw.k[rr].get(c);
                                sQs[row * C::RP + chl + c] = (OpT)qf;
                                sK[row * C::RP + chl + c] = (OpT)kf;
                                sQI[row * C::RP + chl + c] = (OpT)(qf * eb[rr]);
                                kt4[c][e] = (OpT)(kf * ekr[rr]);
                            }
                        }
#pragma unroll
                        for (int c = 0; c < C::CPL; ++c)
                            *reinterpret_cast<typename C::Half *>(sKT + (chl + c) * C::KTP + kslot(16 * w + 4 * g4)) =
                                kt4[c];
                    }
                }
                lds_barrier();

                // ---------------- prefetch the next unit while this one computes
                {
                    int Tn = -1, sn = 0;
                    if (sl + 1 < C::NSLAB) {
                        Tn = T0;
                        sn = sl + 1;
                    } else if (tau + 1 < ntile) {
                        Tn = T0 + kTile;
                    } else if (c0 + a.chunk < t_end) {
                        Tn = c0 + a.chunk;
                    }
                    if (Tn >= 0) load_unit<C, true>(raw, b, Tn, sn, sn == 0, w, lane, tid, dv0);
                }

                // ---------------- inter-chunk term: O += QI . S (rows of this slab)
                {
                    Frag sb[C::KSTEP];
#pragma unroll
                    for (int m = 0; m < C::KSTEP; ++m) {
                        const int n0 = sl * C::NBS + 2 * m;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            sb[m][e] = (OpT)S[n0][e];
                            sb[m][e + 4] = (OpT)S[n0 + 1][e];
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const OpT *row = sQI + (16 * i + c16) * C::RP;
#pragma unroll
                        for (int m = 0; m < C::KSTEP; ++m) {
                            const Frag af = ld4x2<C>(row + 32 * m + 4 * g, row + 32 * m + 16 + 4 * g);
                            O[i] = mma(af, sb[m], O[i]);
                        }
                    }
                }

                // ---------------- diagonal-tile score blocks (transposed): P^T(j,i) over this slab
#pragma unroll
                for (int kp = 0; kp < 3; ++kp) {
                    int i, j;
                    pair_of(w, kp, i, j);
                    if (i < 0) continue;
                    if (kp == 0 && harsh) continue;  // computed exactly during preparation
                    f32x4 acc = Pd[kp];
                    const OpT *krow = sK + (16 * j + c16) * C::RP;
                    const OpT *qrow = sQs + (16 * i + c16) * C::RP;
#pragma unroll
                    for (int m = 0; m < C::KSTEP; ++m) {
                        const int ch = 32 * m + 8 * g;
                        Frag af = ld8<C>(krow + ch);
                        Frag bf = ld8<C>(qrow + ch);
                        if constexpr (C::CH) {
                            if (i == j) {
                                af = scale8<C>(af, lds_ld<f32x4>(sAi + w * C::SLAB + ch),
                                               lds_ld<f32x4>(sAi + w * C::SLAB + ch + 4));
                            } else if (j + 1 < i) {
                                f32x4 r0 = lds_ld<f32x4>(sAb + (j + 1) * C::SLAB + ch);
                                f32x4 r1 = lds_ld<f32x4>(sAb + (j + 1) * C::SLAB + ch + 4);
                                if (j + 2 < i) {
                                    r0 *= lds_ld<f32x4>(sAb + (j + 2) * C::SLAB + ch);
                                    r1 *= lds_ld<f32x4>(sAb + (j + 2) * C::SLAB + ch + 4);
                                }
                                bf = scale8<C>(bf, r0, r1);
                            }
                        }
                        acc = mma(af, bf, acc);
                    }
                    Pd[kp] = acc;
                }

                // ---------------- chunk-state contribution of this tile (rows of this slab)
#pragma unroll
                for (int n = 0; n < C::NBS; ++n) {
                    const int nn = sl * C::NBS + n;
                    f32x4 at;
                    if constexpr (C::CH) {
                        at = lds_ld<f32x4>(sAt + tau * C::DK + sl * C::SLAB + 16 * n + 4 * g);
                    } else {
                        const float x = fexp2(Tt);
                        at = f32x4{x, x, x, x};
                    }
                    f32x4 acc = C::MT ? dS[nn] : S[nn];
                    acc *= at;
                    const OpT *kt = sKT + (16 * n + c16) * C::KTP;
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        const Frag af = ld8<C>(kt + (p * 4 + g) * 8);
                        const Frag bf = ld8<C>(sV + ((p * 4 + g) * 64 + 16 * w + c16) * 8);
                        acc = mma(af, bf, acc);
                    }
                    if constexpr (C::MT)
                        dS[nn] = acc;
                    else
                        S[nn] = acc;
                }
                lds_barrier();
            }  // slabs

            // ---------------- diagonal tile: mask, store scores, multiply by values
#pragma unroll
            for (int kp = 0; kp < 3; ++kp) {
                int i, j;
                pair_of(w, kp, i, j);
                if (i < 0) continue;
                typename C::Half pv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 4 * g + e;  // key row in block j
                    float x = Pd[kp][e];
                    if (i == j && s > c16) x = 0.f;
                    if constexpr (!C::CH) {
                        if (!(i == j && s > c16)) {
                            const int ts = kTile * tau + 16 * i + c16, ss = kTile * tau + 16 * j + s;
                            x *= fexp2(sBr[ts] - sBr[ss] + sLr[ss]);
                        }
                    }
                    pv[e] = (OpT)x;
                }
                *reinterpret_cast<typename C::Half *>(sP + ((i * 2 + (j >> 1)) * 64 + lane) * 8 + 4 * (j & 1)) = pv;
            }
            if (w == 0 || w == 2) {  // key blocks after the query block stay zero
                const typename C::Half z{(OpT)0.f, (OpT)0.f, (OpT)0.f, (OpT)0.f};
                *reinterpret_cast<typename C::Half *>(sP + ((w * 2 + (w >> 1)) * 64 + lane) * 8 + 4) = z;
            }
            lds_barrier();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int np = (i >> 1) + 1;
                for (int p = 0; p < np; ++p) {
                    const Frag af = ld8<C>(sP + ((i * 2 + p) * 64 + lane) * 8);
                    const Frag bf = ld8<C>(sV + ((p * 4 + g) * 64 + 16 * w + c16) * 8);
                    O[i] = mma(af, bf, O[i]);
                }
            }

            // ---------------- earlier tiles of the same chunk (large chunks)
            if constexpr (C::MT) {
#pragma unroll 1
                for (int kj = 0; kj < tau; ++kj) {
                    lds_barrier();  // previous readers of sP / sVo are done
                    {
                        Raw<C> vr;
                        const int Tk = c0 + kTile * kj;
                        const int cq = dv0 + 4 * (tid & 15);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int t = Tk + 4 * (tid >> 4) + e;  // always < L (an earlier, full tile)
                            const InT *p = b.v + (size_t)t * Dv + cq;
                            if constexpr (C::F32)
                                vr.v[e].x = *reinterpret_cast<const float4 *>(p);
                            else
                                vr.v[e].x = *reinterpret_cast<const uint2 *>(p);
                        }
                        v_to_lds<C>(vr, sVo, tid);
                    }
                    f32x4 Po[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) Po[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
                    for (int sl = 0; sl < C::NSLAB; ++sl) {
                        const OpT *qrow = sQ + (size_t)(sl * 64 + 16 * w + c16) * C::RP;
#pragma unroll
                        for (int m = 0; m < C::KSTEP; ++m) {
                            const int ch = 32 * m + 8 * g;
                            Frag bf = ld8<C>(qrow + ch);
                            if constexpr (C::CH) {
                                const int d = sl * C::SLAB + ch;
                                f32x4 f0 = lds_ld<f32x4>(sQTF + w * C::DK + d);
                                f32x4 f1 = lds_ld<f32x4>(sQTF + w * C::DK + d + 4);
                                for (int tp = kj + 1; tp < tau; ++tp) {
                                    f0 *= lds_ld<f32x4>(sAt + tp * C::DK + d);
                                    f1 *= lds_ld<f32x4>(sAt + tp * C::DK + d + 4);
                                }
                                bf = scale8<C>(bf, f0, f1);
                            }
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                Frag af;
                                if constexpr (C::CH) {
                                    af = ld8<C>(sPK + (size_t)((kj * C::NSLAB + sl) * 64 + 16 * j + c16) * C::RP + ch);
                                } else {
                                    const int t = c0 + kTile * kj + 16 * j + c16;
                                    const InT *kp = b.k + (size_t)t * C::DK + sl * C::SLAB + ch;
                                    if constexpr (C::F32) {
                                        const float4 x0 = *reinterpret_cast<const float4 *>(kp);
                                        const float4 x1 = *reinterpret_cast<const float4 *>(kp + 4);
                                        af = f32x8{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                                    } else {
                                        const uint4 x = *reinterpret_cast<const uint4 *>(kp);
                                        const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                                        for (int e = 0; e < 4; ++e) {
                                            af[2 * e] = (OpT)__uint_as_float(wv[e] << 16);
                                            af[2 * e + 1] = (OpT)__uint_as_float(wv[e] & 0xffff0000u);
                                        }
                                    }
                                }
                                Po[j] = mma(af, bf, Po[j]);
                            }
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        typename C::Half pv;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float x = Po[j][e];
                            if constexpr (!C::CH) {
                                const int ts = kTile * tau + 16 * w + c16, ss = kTile * kj + 16 * j + 4 * g + e;
                                x *= fexp2(sBr[ts] - sBr[ss] + sLr[ss]);
                            }
                            pv[e] = (OpT)x;
                        }
                        *reinterpret_cast<typename C::Half *>(sP + ((w * 2 + (j >> 1)) * 64 + lane) * 8 + 4 * (j & 1)) =
                            pv;
                    }
                    lds_barrier();
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
#pragma unroll
                        for (int p = 0; p < 2; ++p) {
                            const Frag af = ld8<C>(sP + ((i * 2 + p) * 64 + lane) * 8);
                            const Frag bf = ld8<C>(sVo + ((p * 4 + g) * 64 + 16 * w + c16) * 8);
                            O[i] = mma(af, bf, O[i]);
                        }
                    }
                }
            }

            // ---------------- store the tile's outputs
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = T0 + 16 * i + 4 * g + e;
                    if (t < L) a.out[(bhL + t) * Dv + col] = O[i][e];
                }
            }
            if constexpr (!C::CH) Bc += Tt;
            lds_barrier();  // LDS tile arrays are rewritten by the next unit
        }  // tiles

        if constexpr (C::MT) {
            // end of a multi-tile chunk: S <- diag(decay across the chunk) S + dS
#pragma unroll
            for (int n = 0; n < C::NBD; ++n) {
                f32x4 ach;
                if constexpr (C::CH) {
                    ach = f32x4{1.f, 1.f, 1.f, 1.f};
                    for (int tp = 0; tp < ntile; ++tp) ach *= lds_ld<f32x4>(sAt + tp * C::DK + 16 * n + 4 * g);
                } else {
                    const float x = fexp2(Bc);
                    ach = f32x4{x, x, x, x};
                }
                S[n] = S[n] * ach + dS[n];
            }
            lds_barrier();  // sAt is rewritten by the next chunk
        }
    }  // chunks

    if (seg == a.nseg - 1 && a.fin) {
#pragma unroll
        for (int n = 0; n < C::NBD; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.fin[((size_t)bh * C::DK + 16 * n + 4 * g + e) * Dv + col] = S[n][e];
    }
}

// ------------------------------------------------------------------------------------
// segment_state_kernel: grid = BH * (nseg - 1) * ndv.  The state segment `seg` produces
// from zero, sum_s diag(decay from s to the segment end) i_s k_s^T v_s, accumulated tile by
// tile (dS <- diag(tile decay) dS + K~^T V), and the decay across the segment.
template <class C>
__global__ __launch_bounds__(256, 1) void segment_state_kernel(KArgs a) {
    using OpT = typename C::OpT;
    using Frag = typename C::Frag;
    using InT = typename C::InT;
    extern __shared__ __align__(256) unsigned char smem[];
    const LdsPlan lp = lds_plan(C::OPB, C::DK, C::CH, 1);
    OpT *sKT = reinterpret_cast<OpT *>(smem + lp.kst);
    OpT *sV = reinterpret_cast<OpT *>(smem + lp.vb);
    float *sAb = reinterpret_cast<float *>(smem + lp.ablk);
    float *sAi = reinterpret_cast<float *>(smem + lp.ainv);
    float *sAt = reinterpret_cast<float *>(smem + lp.atile);
    float *sAs = reinterpret_cast<float *>(smem + lp.aseg);

    const int nsm = a.nseg - 1;
    int id = xcd_remap((int)blockIdx.x, a.nwg);
    const int dvt = id % a.ndv;
    id /= a.ndv;
    const int seg = id % nsm;
    const int bh = id / nsm;
    const int h = bh % a.H;
    const int tid = (int)threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = a.L, Dv = a.Dv;
    const int dv0 = dvt * kDvTile;
    const int col = dv0 + 16 * w + c16;
    const int t_begin = seg * a.seg_len;
    const int t_end = min(L, t_begin + a.seg_len);
    const size_t bhL = (size_t)bh * L;

    Base<C> b;
    b.q = nullptr;
    b.k = reinterpret_cast<const InT *>(a.k) + bhL * C::DK;
    b.v = reinterpret_cast<const InT *>(a.v) + bhL * Dv;
    b.la = a.gate == GLA_GATE_CHANNEL ? a.la + bhL * C::DK
           : a.gate == GLA_GATE_HEAD  ? a.la + bhL
           : a.gate == GLA_GATE_HEAD_CONST ? a.la + h
                                           : nullptr;
    b.li = a.li ? a.li + bhL : nullptr;
    b.L = L;
    b.Dv = Dv;
    b.gate = a.gate;

    if constexpr (C::CH) {
        for (int d = tid; d < C::DK; d += kThreads) sAs[d] = 1.f;
    }
    float Bs = 0.f;  // scalar gates: log2 decay across the segment so far
    f32x4 dS[C::NBD];
#pragma unroll
    for (int n = 0; n < C::NBD; ++n) dS[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    Raw<C> raw;
    load_unit<C, false>(raw, b, t_begin, 0, true, w, lane, tid, dv0);
    for (int T0 = t_begin; T0 < t_end; T0 += kTile) {
        float Tt = 0.f;
#pragma unroll 1
        for (int sl = 0; sl < C::NSLAB; ++sl) {
            if (sl == 0) v_to_lds<C>(raw, sV, tid);
            const int chl = C::CPL * lane;
            if constexpr (C::CH) {
                ChGate<C> G;
                ch_gate<C>(G, raw, sAb, sAi, w, lane);
                float ig[16];
                {
                    const float y = raw.lis * kLog2e;
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) ig[rr] = fexp2(__shfl(y, 16 * w + rr));
                }
#pragma unroll
                for (int c = 0; c < C::CPL; ++c) {
                    const int d = sl * C::SLAB + chl + c;
                    if (w == 0) {
                        sAt[d] = G.at[c];
                        sAs[d] *= G.at[c];
                    }
                }
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    typename C::Half kt4[C::CPL];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int rr = 4 * g4 + e;
#pragma unroll
                        for (int c = 0; c < C::CPL; ++c)
                            kt4[c][e] = (OpT)(raw.k[rr].get(c) * G.ek[rr][c] * ig[rr] * G.post[c]);
                    }
#pragma unroll
                    for (int c = 0; c < C::CPL; ++c)
                        *reinterpret_cast<typename C::Half *>(sKT + (chl + c) * C::KTP + kslot(16 * w + 4 * g4)) = kt4[c];
                }
            } else {
                const float x = raw.las * kLog2e;
                const float y = raw.lis * kLog2e;
                const float bl = scan_incl(x, lane);
                Tt = __shfl(bl, 63);
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    typename C::Half kt4[C::CPL];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int rr = 4 * g4 + e;
                        const float f = fexp2(Tt - __shfl(bl, 16 * w + rr) + __shfl(y, 16 * w + rr));
#pragma unroll
                        for (int c = 0; c < C::CPL; ++c) kt4[c][e] = (OpT)(raw.k[rr].get(c) * f);
                    }
#pragma unroll
                    for (int c = 0; c < C::CPL; ++c)
                        *reinterpret_cast<typename C::Half *>(sKT + (chl + c) * C::KTP + kslot(16 * w + 4 * g4)) = kt4[c];
                }
            }
            lds_barrier();
            {
                int Tn = -1, sn = 0;
                if (sl + 1 < C::NSLAB) {
                    Tn = T0;
                    sn = sl + 1;
                } else if (T0 + kTile < t_end) {
                    Tn = T0 + kTile;
                }
                if (Tn >= 0) load_unit<C, false>(raw, b, Tn, sn, sn == 0, w, lane, tid, dv0);
            }
#pragma unroll
            for (int n = 0; n < C::NBS; ++n) {
                const int nn = sl * C::NBS + n;
                f32x4 at;
                if constexpr (C::CH) {
                    at = lds_ld<f32x4>(sAt + sl * C::SLAB + 16 * n + 4 * g);
                } else {
                    const float x = fexp2(Tt);
                    at = f32x4{x, x, x, x};
                }
                f32x4 acc = dS[nn] * at;
                const OpT *kt = sKT + (16 * n + c16) * C::KTP;
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const Frag af = ld8<C>(kt + (p * 4 + g) * 8);
                    const Frag bf = ld8<C>(sV + ((p * 4 + g) * 64 + 16 * w + c16) * 8);
                    acc = mma(af, bf, acc);
                }
                dS[nn] = acc;
            }
            lds_barrier();
        }
        if constexpr (!C::CH) Bs += Tt;
    }

    float *st = a.ws_state + ((size_t)bh * nsm + seg) * C::DK * Dv;
#pragma unroll
    for (int n = 0; n < C::NBD; ++n)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[(size_t)(16 * n + 4 * g + e) * Dv + col] = dS[n][e];
    if (dvt == 0) {
        float *dc = a.ws_decay + ((size_t)bh * nsm + seg) * C::DK;
        for (int d = tid; d < C::DK; d += kThreads) dc[d] = C::CH ? sAs[d] : fexp2(Bs);
    }
}

// ------------------------------------------------------------------------------------
// segment_scan_kernel: grid (ceil(Dk*Dv/1024), BH).  S_in[0] = initial state (or 0);
// S_in[j+1] = diag(decay_j) S_in[j] + local_j, written over local_j.
__global__ __launch_bounds__(256) void segment_scan_kernel(KArgs a, int dk) {
    const int bh = (int)blockIdx.y;
    const size_t n = (size_t)dk * a.Dv;
    const size_t idx = ((size_t)blockIdx.x * kThreads + threadIdx.x) * 4;
    if (idx >= n) return;
    const int d = (int)(idx / a.Dv);
    const int nsm = a.nseg - 1;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.s0) s = *reinterpret_cast<const float4 *>(a.s0 + (size_t)bh * n + idx);
    for (int j = 0; j < nsm; ++j) {
        float4 *p = reinterpret_cast<float4 *>(a.ws_state + ((size_t)bh * nsm + j) * n + idx);
        const float dec = a.ws_decay[((size_t)bh * nsm + j) * dk + d];
        const float4 x = *p;
        s.x = s.x * dec + x.x;
        s.y = s.y * dec + x.y;
        s.z = s.z * dec + x.z;
        s.w = s.w * dec + x.w;
        *p = s;
    }
}

// ------------------------------------------------------------------------------------
// Launchers.
template <class C>
static hipError_t launch_cfg(const KArgs &a, hipStream_t st) {
    hipError_t err;
    if (a.nseg > 1) {
        const LdsPlan l1 = lds_plan(C::OPB, C::DK, C::CH, 1);
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(&segment_state_kernel<C>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)l1.total);
        if (err != hipSuccess) return err;
        KArgs a1 = a;
        a1.nwg = (a.B * a.H) * (a.nseg - 1) * a.ndv;
        hipLaunchKernelGGL(segment_state_kernel<C>, dim3(a1.nwg), dim3(kThreads), l1.total, st, a1);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        const int nx = (C::DK * a.Dv + 1023) / 1024;
        hipLaunchKernelGGL(segment_scan_kernel, dim3(nx, a.B * a.H), dim3(kThreads), 0, st, a, C::DK);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const LdsPlan l3 = lds_plan(C::OPB, C::DK, C::CH, a.nt);
    err = hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_output_kernel<C>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)l3.total);
    if (err != hipSuccess) return err;
    KArgs a3 = a;
    a3.nwg = (a.B * a.H) * a.nseg * a.ndv;
    hipLaunchKernelGGL(chunk_output_kernel<C>, dim3(a3.nwg), dim3(kThreads), l3.total, st, a3);
    return hipGetLastError();
}

template <bool F32, int DK>
static hipError_t launch_dk(const KArgs &a, bool ch, bool mt, hipStream_t st) {
    if (ch) {
        if (mt) return launch_cfg<Cfg<F32, DK, true, true>>(a, st);
        return launch_cfg<Cfg<F32, DK, true, false>>(a, st);
    }
    if (mt) return launch_cfg<Cfg<F32, DK, false, true>>(a, st);
    return launch_cfg<Cfg<F32, DK, false, false>>(a, st);
}

hipError_t launch_forward(const KArgs &a, bool f32, int dk, hipStream_t st) {
    const bool ch = a.gate == GLA_GATE_CHANNEL;
    const bool mt = a.nt > 1;
    if (f32) {
        if (dk == 64) return launch_dk<true, 64>(a, ch, mt, st);
        if (dk == 128) return launch_dk<true, 128>(a, ch, mt, st);
        return launch_dk<true, 256>(a, ch, mt, st);
    }
    if (dk == 64) return launch_dk<false, 64>(a, ch, mt, st);
    if (dk == 128) return launch_dk<false, 128>(a, ch, mt, st);
    return launch_dk<false, 256>(a, ch, mt, st);
}

}  // namespace gla
