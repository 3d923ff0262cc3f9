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
// Work split of a workgroup (4 waves): wave w owns 16 value columns for all matrix
// products, and prepares the gate-scaled operands of the tile's 16-token block w.
//
// Numerics.  Gates are applied in the product domain: per-step decays alpha = 2^(log2e *
// log_alpha) are multiplied into running products, so every factor that multiplies an
// operand is <= 1, except the key factor of a diagonal 16x16 block, which is bounded by
// the block's own decay span (checked; a block whose span is too large is computed exactly
// on the vector ALU instead).  Scalar gates (none / per head) keep q and k raw in the
// score product and multiply each score by its exact decay afterwards.  Operands computed
// from bf16 inputs are fp16; fp32 inputs keep fp32 operands.  Accumulation, states and
// outputs are fp32.
//
// Global memory is read and written through buffer resources whose size is the valid
// extent of the (batch, head) slice: rows past the sequence end read as zero and their
// stores are dropped by the hardware range check.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "gla.h"
#include "gla_layout.h"

namespace gla {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr float kLog2e = 1.4426950408889634f;

// log2 of a per-token decay for running sums in log space, floored at -150: below it the
// fp32 factor 2^x is zero either way, and the floor keeps the running sums small enough
// that differences of two of them keep fp32 precision (a gate of log -1e4 would otherwise
// make them about 1.4e4 and cost two to three significant digits).  NaN passes through.
__device__ __forceinline__ float log2_decay(float la) {
    const float x = la * kLog2e;
    return x < -150.f ? -150.f : x;
}
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// ------------------------------------------------------------------------------------
// Instance configuration.
template <bool F32_, int DK_, bool CH_, bool MT_, int H16_ = 0>
struct Cfg {
    static constexpr bool F32 = F32_;  // fp32 inputs and operands (else bf16 inputs, fp16 operands)
    // Inputs given as fp16 instead of bf16, one bit per operand (kOpQ, kOpK, kOpV): the
    // backward pass feeds its scaled output gradient this way.
    static constexpr int H16 = H16_;
    static constexpr int DK = DK_;
    static constexpr bool CH = CH_;    // per-channel gate
    static constexpr bool MT = MT_;    // chunk of several 64-token tiles
    using OpT = typename std::conditional<F32, float, f16>::type;
    using Frag = typename std::conditional<F32, f32x8, f16x8>::type;
    using Half = typename std::conditional<F32, f32x4, f16x4>::type;
    using InT = typename std::conditional<F32, float, uint16_t>::type;
    static constexpr int OPB = F32 ? 4 : 2;
    static constexpr int IB = F32 ? 4 : 2;      // input element bytes
    static constexpr int CPL = (!F32 && DK >= 128) ? 2 : 1;
    static constexpr int SLAB = 64 * CPL;
    static constexpr int NSLAB = DK / SLAB;
    static constexpr int RP = SLAB + 16 / OPB;  // +16 B per row against LDS bank conflicts
    static constexpr int KTP = 64 + 16 / OPB;
    static constexpr int NBD = DK / 16;         // 16-row blocks of the state
    static constexpr int KSTEP = SLAB / 32;     // 32-deep MFMA steps per slab
    static constexpr int NBS = SLAB / 16;       // 16-row state blocks per slab
    // Smallest decay of a 16-token block whose diagonal block still uses the matrix cores:
    // the key operand there is scaled by up to 1/decay (2^8 for fp16 operands).
    static constexpr float kMinDiagDecay = F32 ? 1e-30f : 0.00390625f;
};

// ------------------------------------------------------------------------------------
// Small device helpers.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Barrier that also makes this workgroup's earlier global stores visible to its other waves.
__device__ __forceinline__ void full_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ float h_lo(uint32_t x) { return (float)__builtin_bit_cast(f16x2, x)[0]; }
__device__ __forceinline__ float h_hi(uint32_t x) { return (float)__builtin_bit_cast(f16x2, x)[1]; }
enum { kOpQ = 0, kOpK = 1, kOpV = 2 };
// Low / high 16-bit input of a packed pair of operand OP as fp32.
template <class C, int OP>
__device__ __forceinline__ float in_lo(uint32_t x) { return ((C::H16 >> OP) & 1) ? h_lo(x) : bf_lo(x); }
template <class C, int OP>
__device__ __forceinline__ float in_hi(uint32_t x) { return ((C::H16 >> OP) & 1) ? h_hi(x) : bf_hi(x); }

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint64_t bytes) {
    const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n, kRsrcFlags);
}
__device__ __forceinline__ uint32_t bld32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2 bld64(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
template <int AUX = 0>
__device__ __forceinline__ u32x4 bld128(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
}

// Cross-lane steps on the vector ALU (DPP) and the scalar unit (readlane) rather than through
// the LDS crossbar (ds_bpermute), whose round trips sit on the producers' critical path.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp(float x) {
    // lanes without a source in range, and rows outside ROWS, read 0
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, false));
}
// x of lane n (wave-uniform n), through a scalar register.
__device__ __forceinline__ float lane_bcast(float x, int n) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), n));
}
// Sum over the calling lane's 16-lane row, in every lane of it (row rotations by 8, 4, 2, 1).
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0x128>(x);
    x += dpp<0x124>(x);
    x += dpp<0x122>(x);
    x += dpp<0x121>(x);
    return x;
}
// Sum over the wave (the four row sums added in row order), the same in every lane.
__device__ __forceinline__ float wave_sum(float x) {
    x = row_sum16(x);
    return (lane_bcast(x, 0) + lane_bcast(x, 16)) + (lane_bcast(x, 32) + lane_bcast(x, 48));
}
// Inclusive prefix sum over the wave's lanes: row shifts by 1, 2, 4, 8 within each 16-lane
// row, then the end of row 0 (row broadcast 15) into rows 1 and 3 and the end of row 1 (row
// broadcast 31) into rows 2 and 3.
__device__ __forceinline__ float scan_incl(float x, [[maybe_unused]] int lane) {
    x += dpp<0x111>(x);
    x += dpp<0x112>(x);
    x += dpp<0x114>(x);
    x += dpp<0x118>(x);
    x += dpp<0x142, 0xa>(x);
    x += dpp<0x143, 0xc>(x);
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

// Transposing LDS read of 16-bit operands (gfx950): within each group of 16 lanes, lane
// 4e + q supplies the address of 4 consecutive elements and lane j receives element j & 3 of
// the vectors of lanes (j >> 2), 4 + (j >> 2), 8 + (j >> 2), 12 + (j >> 2), in that order.
__device__ __forceinline__ f16x4 lds_tr16(const f16 *p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const auto lp = (__attribute__((address_space(3))) s16x4 *)(p);
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
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
// Lane n of the calling lane's 16-lane row (DPP row broadcast); n must fold to a constant.
__device__ __forceinline__ uint32_t row_bcast(uint32_t v, int n) {
#define GLA_RB(N) \
    case N: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + N, 0xf, 0xf, false);
    switch (n) {
        GLA_RB(0) GLA_RB(1) GLA_RB(2) GLA_RB(3) GLA_RB(4) GLA_RB(5) GLA_RB(6) GLA_RB(7)
        GLA_RB(8) GLA_RB(9) GLA_RB(10) GLA_RB(11) GLA_RB(12) GLA_RB(13) GLA_RB(14)
        default: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + 15, 0xf, 0xf, false);
    }
#undef GLA_RB
}
// Eight fp16 per-channel factors of MFMA k-step m for a lane of row g, from one dword per lane
// that holds factor dword 16 (lane>>2 & 3) + 4 g + (lane & 3) of the row (see fac_dword).
__device__ __forceinline__ f16x8 fac_frag(uint32_t f, int m) {
    const u32x4 d{row_bcast(f, 4 * m), row_bcast(f, 4 * m + 1), row_bcast(f, 4 * m + 2), row_bcast(f, 4 * m + 3)};
    return __builtin_bit_cast(f16x8, d);
}
// The factor dword a lane (g, c16) loads once per tile: k-step c16 >> 2, dword c16 & 3 of the
// eight channels 32 m + 8 g ..; rows of ndw dwords (ndw = 16 x k-steps).
__device__ __forceinline__ int fac_dword(int g, int c16, int ndw) { return (16 * (c16 >> 2) + 4 * g + (c16 & 3)) & (ndw - 1); }

// 8 fp32 values times per-element factors, rounded once to operands.
template <class C>
__device__ __forceinline__ typename C::Frag scale8f(const float *x, const f32x4 &s0, const f32x4 &s1) {
    using OpT = typename C::OpT;
    typename C::Frag r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (OpT)(x[e] * s0[e]);
        r[e + 4] = (OpT)(x[e + 4] * s1[e]);
    }
    return r;
}
// 8 consecutive operands from global memory through a buffer resource.
template <class C, int AUX>
__device__ __forceinline__ typename C::Frag gld8(rsrc_t r, uint32_t off) {
    if constexpr (C::F32) {
        const u32x4 a = bld128<AUX>(r, off), b = bld128<AUX>(r, off + 16);
        return f32x8{__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]), __uint_as_float(a[3]),
                     __uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]), __uint_as_float(b[3])};
    } else {
        const u32x4 a = bld128<AUX>(r, off);
        return __builtin_bit_cast(f16x8, a);
    }
}
// 8 consecutive raw inputs (bf16 or fp32) from global memory as operands.
template <class C, int OP>
__device__ __forceinline__ typename C::Frag gld8_in(rsrc_t r, uint32_t off) {
    if constexpr (C::F32) {
        return gld8<C, 0>(r, off);
    } else {
        const u32x4 x = bld128(r, off);
        if constexpr ((C::H16 >> OP) & 1) return __builtin_bit_cast(f16x8, x);
        typename C::Frag f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[2 * e] = (f16)bf_lo(x[e]);
            f[2 * e + 1] = (f16)bf_hi(x[e]);
        }
        return f;
    }
}

// Output tile through LDS: each consumer wave writes its 16 columns of the 64-row tile
// (accumulator layout: rows 16i + 4g + e, column 16 cw + c16), and after a barrier stores
// 16 whole rows of 64 columns with 16-byte stores (rows past the sequence end are dropped
// by the buffer range check).
__device__ __forceinline__ void stage_out(float *sO, const f32x4 (&O)[4], int cw, int g, int c16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) sO[(16 * i + 4 * g + e) * 68 + 16 * cw + c16] = O[i][e];
}
// Whole-row stores of the output tile with the non-temporal cache policy (gfx950 `nt`): the
// output is written once and not read back, and streaming it past the caches keeps the
// inputs the column-slice workgroups of a head share (and the segment states) resident:
// 1.5-4% on the scalar-gate and segmented workloads.
constexpr int kStoreNT = 2;
__device__ __forceinline__ void store_staged(const float *sO, rsrc_t out, int T0, int Dv, int dv0, int cw,
                                             int lane) {
    const int c4 = lane & 15;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int row = 16 * cw + 4 * rr + (lane >> 4);
        const f32x4 x = lds_ld<f32x4>(sO + row * 68 + 4 * c4);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), out,
                                               (int)(((uint32_t)(T0 + row) * Dv + dv0 + 4 * c4) * 4u), 0, kStoreNT);
    }
}

// Rows of a backward pass's dot-product source (KArgs::dot_src) for the lane's four output
// rows, at the destination rows the stores use (four bf16 each), loaded ahead of the stores.
struct DotPre {
    u32x2 s[4];
};
__device__ __forceinline__ void load_dot_pre(DotPre &p, rsrc_t src, int T0, int L, int Dv, int dv0, int cw, int lane,
                                             bool rev) {
    const int c4 = lane & 15;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int t = T0 + 16 * cw + 4 * rr + (lane >> 4);
        // rows past the sequence end read row 0 (in range) and store nothing
        const uint32_t dst = t < L ? (uint32_t)(rev ? L - 1 - t : t) : 0u;
        p.s[rr] = bld64(src, (dst * (uint32_t)Dv + (uint32_t)(dv0 + 4 * c4)) * 2u);
    }
}
// The dot product of a stored row segment x with its source row segment, summed over the 16
// lanes that hold the row's 64 columns; the first of them writes it to drow[dst].
__device__ __forceinline__ void store_dot(const u32x2 &s, const f32x4 &x, float *drow, int dst, bool valid, int c4) {
    const float part = row_sum16(bf_lo(s[0]) * x[0] + bf_hi(s[0]) * x[1] + bf_lo(s[1]) * x[2] + bf_hi(s[1]) * x[3]);
    if (c4 == 0 && valid) drow[dst] = part;
}

// The same for the backward pass's instances: row t goes to row L-1-t when rev, times
// oinv and (has_li) times exp of the destination row's log input gate, added to what the
// output holds when acc; rows past the sequence end are not stored.  With DOT, each stored
// row's dot product with its preloaded source row goes to drow (when non-null).
template <bool DOT>
__device__ __forceinline__ void store_staged_map(const float *sO, rsrc_t out, rsrc_t oli, int T0, int L, int Dv,
                                                 int dv0, int cw, int lane, bool rev, bool has_li, float oinv,
                                                 bool acc, const DotPre &dp, float *drow) {
    const int c4 = lane & 15;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int row = 16 * cw + 4 * rr + (lane >> 4);
        const int t = T0 + row;
        const int dst = rev ? L - 1 - t : t;
        float f = oinv;
        if (has_li) f *= fexp2(__uint_as_float(bld32(oli, (uint32_t)dst * 4u)) * kLog2e);
        f32x4 x = lds_ld<f32x4>(sO + row * 68 + 4 * c4);
        x *= f;
        const uint32_t off = ((uint32_t)dst * Dv + dv0 + 4 * c4) * 4u;
        if (acc && t < L) x += __builtin_bit_cast(f32x4, bld128(out, off));
        if (t < L) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), out, (int)off, 0, 0);
        if constexpr (DOT) store_dot(dp.s[rr], x, drow, dst, t < L && drow != nullptr, c4);
    }
}
// The same with the global loads (the log input gates, the output rows to add to) issued a
// phase earlier by load_map_pre, so that the stores do not wait a memory round trip (used by
// the scalar-gate kernel, whose consumers issue no other global loads; in the per-channel
// kernel the consumers' value prefetch is in flight, and the wait for loads that a run-time
// flag may have skipped then waits for the prefetch).
struct MapPre {
    f32x4 x[4];   // output rows to add to (acc)
    float li[4];  // log input gates of the destination rows (has_li)
};
__device__ __forceinline__ void load_map_pre(MapPre &p, rsrc_t out, rsrc_t oli, int T0, int L, int Dv, int dv0,
                                             int cw, int lane, bool rev, bool has_li, bool acc) {
    const int c4 = lane & 15;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int t = T0 + 16 * cw + 4 * rr + (lane >> 4);
        // rows past the sequence end read row 0 (in range) and are not stored
        const uint32_t dst = t < L ? (uint32_t)(rev ? L - 1 - t : t) : 0u;
        p.li[rr] = has_li ? __uint_as_float(bld32(oli, dst * 4u)) : 0.f;
        p.x[rr] = acc ? __builtin_bit_cast(f32x4, bld128(out, (dst * Dv + dv0 + 4 * c4) * 4u)) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
}
template <bool DOT>
__device__ __forceinline__ void store_staged_map(const float *sO, rsrc_t out, const MapPre &p, int T0, int L, int Dv,
                                                 int dv0, int cw, int lane, bool rev, bool has_li, float oinv,
                                                 bool acc, const DotPre &dp, float *drow) {
    const int c4 = lane & 15;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int row = 16 * cw + 4 * rr + (lane >> 4);
        const int t = T0 + row;
        const int dst = rev ? L - 1 - t : t;
        float f = oinv;
        if (has_li) f *= fexp2(p.li[rr] * kLog2e);
        f32x4 x = lds_ld<f32x4>(sO + row * 68 + 4 * c4);
        x *= f;
        if (acc) x += p.x[rr];
        const uint32_t off = ((uint32_t)dst * Dv + dv0 + 4 * c4) * 4u;
        if (t < L) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), out, (int)off, 0, 0);
        if constexpr (DOT) store_dot(dp.s[rr], x, drow, dst, t < L && drow != nullptr, c4);
    }
}

// Output mapping of a backward-pass instance, set up once per workgroup; dsrc and drow are
// the dot-product source of the workgroup's (batch, head) (a zero-size range when there is
// none: its loads return zero) and its row of dot_out for value tile dvt (or null).
struct OutMap {
    rsrc_t li, dsrc;
    float *drow;
    float inv;
    bool rev, has_li, acc;
};
// dq and dk passes of the backward (a scalar gate and an fp16 q or k operand) form the dot
// products of their stored rows with q or k
template <class C>
constexpr bool kDotPass = !C::CH && (C::H16 == (1 << kOpQ) || C::H16 == (1 << kOpK));
__device__ __forceinline__ OutMap make_out_map(const KArgs &a, int bh, int dvt) {
    OutMap m;
    const bool dot = a.dot_out != nullptr && a.dot_src != nullptr;
    m.dsrc = dot ? make_rsrc(reinterpret_cast<const char *>(a.dot_src) + (size_t)bh * a.L * a.Dv * 2,
                             (uint64_t)a.L * a.Dv * 2)
                 : make_rsrc(a.out, 0);
    m.drow = dot ? a.dot_out + ((size_t)dvt * a.B * a.H + bh) * a.L : nullptr;
    m.rev = a.out_rev != 0;
    m.has_li = a.out_li != nullptr;
    m.li = m.has_li ? make_rsrc(a.out_li + (size_t)bh * a.L, (uint64_t)a.L * 4) : make_rsrc(a.out, 0);
    m.inv = a.out_mx ? 1.f / grad_scale_of(a.out_mx[bh]) : 1.f;
    m.acc = a.out_acc != 0;
    return m;
}

// ------------------------------------------------------------------------------------
// Raw input of one unit (64-token tile x one slab of key channels), prefetched into
// registers.  Thread (wave w, lane) holds rows 16w..16w+15 of the tile for its CPL key
// channels; value pieces are rows 4*(tid>>4)+e, columns 4*(tid&15)..+3 of the 64x64 tile.
template <class C>
struct Raw {
    uint32_t q[16], k[16];              // CPL channels (bf16 pair, bf16 in the low half, or fp32 bits)
    float la[C::CH ? 16 : 1][C::CPL];   // per-channel log gates
    float las, lis;                     // log gate / log input gate of row (tile start + lane)
    uint32_t v[4][C::F32 ? 4 : 2];      // 4 values of one row
    __device__ float qf(int r, int c) const {
        return C::F32 ? __uint_as_float(q[r]) : (c ? in_hi<C, kOpQ>(q[r]) : in_lo<C, kOpQ>(q[r]));
    }
    __device__ float kf(int r, int c) const {
        return C::F32 ? __uint_as_float(k[r]) : (c ? in_hi<C, kOpK>(k[r]) : in_lo<C, kOpK>(k[r]));
    }
    __device__ float vf(int e, int j) const {
        if constexpr (C::F32) return __uint_as_float(v[e][j]);
        else return (j & 1) ? in_hi<C, kOpV>(v[e][j >> 1]) : in_lo<C, kOpV>(v[e][j >> 1]);
    }
};

// Buffer resources of one (batch, head) slice.
struct Rs {
    rsrc_t q, k, v, la, li, out;
    int gate, L;
    uint32_t gstride;  // bytes between the scalar gates of consecutive rows (0: one value or none)
    bool has_li;
    bool rev;          // backward-pass instances: token t reads q, k, v row L-1-t
    uint32_t qks;      // backward-pass instances: elements between rows of q and k
};

// Row of q, k, v that token t reads.  Past the sequence end (t >= L) a reversed row is
// negative, and its 32-bit byte offset lies past the slice, so it reads zero like t >= L does.
template <class C>
__device__ __forceinline__ uint32_t in_row(const Rs &rs, int t) {
    if constexpr (C::H16 != 0) return (uint32_t)(rs.rev ? rs.L - 1 - t : t);
    else return (uint32_t)t;
}
// Row of a per-channel gate that token t reads: reversed passes take the gate of the token
// after (row L - t); token 0 and the rows past the sequence end read row L, past the slice:
// zero, no decay (a padding row must not decay the final state).
template <class C>
__device__ __forceinline__ uint32_t gate_row(const Rs &rs, int t) {
    if constexpr (C::H16 != 0) return (uint32_t)(rs.rev ? (t < rs.L ? rs.L - t : rs.L) : t);
    else return (uint32_t)t;
}

template <class C>
__device__ __forceinline__ Rs make_rs(const KArgs &a, int bh, int h) {
    Rs r;
    const size_t bhL = (size_t)bh * a.L;
    const uint64_t L = (uint64_t)a.L;
    size_t qs = C::DK;
    if constexpr (C::H16 != 0) {
        if (a.qk_stride) qs = (size_t)a.qk_stride;
        r.qks = (uint32_t)qs;
    }
    r.q = make_rsrc(reinterpret_cast<const char *>(a.q) + bhL * qs * C::IB, L * qs * C::IB);
    r.k = make_rsrc(reinterpret_cast<const char *>(a.k) + bhL * qs * C::IB, L * qs * C::IB);
    r.v = make_rsrc(reinterpret_cast<const char *>(a.v) + bhL * a.Dv * C::IB, L * a.Dv * C::IB);
    r.out = make_rsrc(a.out + bhL * a.Dv, L * a.Dv * 4);
    if (a.gate == GLA_GATE_CHANNEL)
        r.la = make_rsrc(a.la + bhL * C::DK, L * C::DK * 4);
    else if (a.gate == GLA_GATE_HEAD)
        r.la = make_rsrc(a.la + bhL, L * 4);
    else if (a.gate == GLA_GATE_HEAD_CONST)
        r.la = make_rsrc(a.la + h, 4);
    else
        r.la = make_rsrc(a.out, 0);  // reads return zero
    r.li = a.li ? make_rsrc(a.li + bhL, L * 4) : make_rsrc(a.out, 0);
    r.gate = a.gate;
    r.L = a.L;
    r.gstride = a.gate == GLA_GATE_HEAD ? 4u : 0u;
    r.has_li = a.li != nullptr;
    r.rev = a.in_rev != 0;
    return r;
}

template <class C, bool WQ>
__device__ __forceinline__ void load_unit(Raw<C> &r, const Rs &rs, int T0, int sl, int w, int lane, int tid, int dv0,
                                          int Dv) {
    const int ch0 = sl * C::SLAB + C::CPL * lane;
    uint32_t qks = C::DK;
    if constexpr (C::H16 != 0) qks = rs.qks;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const uint32_t off = (in_row<C>(rs, T0 + 16 * w + rr) * qks + ch0) * C::IB;
        if constexpr (C::CPL == 2 || C::F32) {
            if constexpr (WQ) r.q[rr] = bld32(rs.q, off);
            r.k[rr] = bld32(rs.k, off);
        } else {
            if constexpr (WQ) r.q[rr] = __builtin_amdgcn_raw_buffer_load_b16(rs.q, (int)off, 0, 0);
            r.k[rr] = __builtin_amdgcn_raw_buffer_load_b16(rs.k, (int)off, 0, 0);
        }
        if constexpr (C::CH) {
            const uint32_t goff = (gate_row<C>(rs, T0 + 16 * w + rr) * C::DK + ch0) * 4u;
            if constexpr (C::CPL == 2) {
                const u32x2 g2 = bld64(rs.la, goff);
                r.la[rr][0] = __uint_as_float(g2[0]);
                r.la[rr][1] = __uint_as_float(g2[1]);
            } else {
                r.la[rr][0] = __uint_as_float(bld32(rs.la, goff));
            }
        }
    }
    const uint32_t t = (uint32_t)(T0 + lane);
    if constexpr (!C::CH) {
        // per head: [L]; fixed per head: one value, valid while the row exists
        if (rs.gate == GLA_GATE_HEAD)
            r.las = __uint_as_float(bld32(rs.la, t * 4u));
        else if (rs.gate == GLA_GATE_HEAD_CONST)
            r.las = (int)t < rs.L ? __uint_as_float(bld32(rs.la, 0)) : 0.f;
        else
            r.las = 0.f;
    }
    r.lis = __uint_as_float(bld32(rs.li, t * 4u));
    {
        const uint32_t c0 = dv0 + 4 * (tid & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t off = (in_row<C>(rs, T0 + 4 * (tid >> 4) + e) * Dv + c0) * C::IB;
            if constexpr (C::F32) {
                const u32x4 x = bld128(rs.v, off);
#pragma unroll
                for (int j = 0; j < 4; ++j) r.v[e][j] = x[j];
            } else {
                const u32x2 x = bld64(rs.v, off);
                r.v[e][0] = x[0];
                r.v[e][1] = x[1];
            }
        }
    }
}

// Slot of token s (0..63 in the tile) in the k-slot order of the value and key^T operands.
__device__ __forceinline__ int kslot(int s) { return (((s >> 5) * 4 + ((s >> 2) & 3)) * 8) + ((s >> 4) & 1) * 4 + (s & 3); }

// LDS bank spreading.  Rows of key^T keep their 8-slot groups XOR-swizzled by (row >> 4) & 7
// (the producers write four tokens of 16 channels whose rows are 2 or 4 apart); columns of
// the value tile are XOR-swizzled by (column >> 3) & 3 (the producers write columns 4 apart).
// Readers apply the same maps and still read 16 contiguous bytes per lane.
template <class C>
__device__ __forceinline__ int kt_off(int r, int s) {
    return r * C::KTP + ((((s >> 3) ^ (r >> 4)) & 7) << 3) + (s & 7);
}
__device__ __forceinline__ int vsw(int c) { return c ^ ((c >> 3) & 3); }
// Position of channel c inside its 32-channel group in q, k and qi rows of the
// warp-specialised kernels: the 8 channels one lane feeds to the q . S product (which follow
// the state accumulators' rows 4g + e of two 16-row blocks) become 16 contiguous bytes.
// Scores see q and k under the same permutation, which leaves their dot products unchanged.
__device__ __forceinline__ int chperm(int c) {
    return (c & ~31) + 8 * ((c & 15) >> 2) + 4 * ((c >> 4) & 1) + (c & 3);
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
        for (int e = 0; e < 4; ++e) h4[e] = (OpT)r.vf(e, j);
        *reinterpret_cast<H *>(sV + ((p * 4 + g) * 64 + vsw(c0 + j)) * 8 + hh * 4) = h4;
    }
}



// CPL operands of one row into LDS.
template <class C>
__device__ __forceinline__ void st_row(typename C::OpT *row, const float *x) {
    if constexpr (C::CPL == 2) {
        *reinterpret_cast<f16x2 *>(row) = f16x2{(f16)x[0], (f16)x[1]};
    } else {
        *row = (typename C::OpT)x[0];
    }
}

// ------------------------------------------------------------------------------------
// Per-channel gate of one unit.  Thread rows r of 16-token block w:
//   eq[r] = decay from the block start through row r (inclusive), ek[r] = decay after row r
//   to the block end; ab[u] = decay across block u (exchanged through LDS); at = decay
//   across the tile.
template <class C>
struct ChGate {
    float eq[16][C::CPL], ek[16][C::CPL];
    float ab[4][C::CPL];
    float pre[C::CPL], post[C::CPL], at[C::CPL];
    bool harsh;
};

template <class C>
__device__ __forceinline__ void ch_gate(ChGate<C> &G, const Raw<C> &r, float *sAb, int w, int lane) {
#pragma unroll
    for (int c = 0; c < C::CPL; ++c) {
        float run = 1.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const float al = fexp2(r.la[rr][c] * kLog2e);
            G.ek[rr][c] = al;  // alpha, turned into the suffix product below
            run *= al;
            G.eq[rr][c] = run;
        }
        run = 1.f;
#pragma unroll
        for (int rr = 15; rr >= 0; --rr) {
            const float al = G.ek[rr][c];
            G.ek[rr][c] = run;
            run *= al;
        }
    }
    bool small = false;
    const int chl = C::CPL * lane;
    if constexpr (C::CPL == 2) {
        *reinterpret_cast<float2 *>(sAb + w * C::SLAB + chl) = make_float2(G.eq[15][0], G.eq[15][1]);
    } else {
        sAb[w * C::SLAB + chl] = G.eq[15][0];
    }
#pragma unroll
    for (int c = 0; c < C::CPL; ++c) small |= !(G.eq[15][c] >= C::kMinDiagDecay);
    G.harsh = __ballot(small) != 0ull;
    lds_barrier();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if constexpr (C::CPL == 2) {
            const float2 x = lds_ld<float2>(sAb + u * C::SLAB + chl);
            G.ab[u][0] = x.x;
            G.ab[u][1] = x.y;
        } else {
            G.ab[u][0] = sAb[u * C::SLAB + chl];
        }
    }
#pragma unroll
    for (int c = 0; c < C::CPL; ++c) {
        float pre = 1.f, post = 1.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u < w) pre *= G.ab[u][c];
            if (u > w) post *= G.ab[u][c];
        }
        G.pre[c] = pre;
        G.post[c] = post;
        G.at[c] = pre * G.eq[15][c] * post;
    }
}

// Exact diagonal 16x16 score block of block w over this slab's channels, for a block whose
// decay span is too large for scaled matrix-core operands: every pair s <= t gets
// sum_d q_td k_sd 2^(u_td - u_sd) i_s with u the log2 running decay.
template <class C>
__device__ __attribute__((noinline)) f32x4 ch_diag_exact(f32x4 acc, Raw<C> r, int lane, bool has_li) {
    float u[16][C::CPL];
#pragma unroll
    for (int c = 0; c < C::CPL; ++c) {
        float run = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            run += log2_decay(r.la[rr][c]);
            u[rr][c] = run;
        }
    }
    const int c16 = lane & 15, g = lane >> 4;
    const int w = lane;  // unused
    (void)w;
    const float y = r.lis * kLog2e;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    float ig[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) ig[rr] = has_li ? fexp2(lane_bcast(y, 16 * wv + rr)) : 1.f;
    for (int s = 0; s < 16; ++s) {
        for (int t = s; t < 16; ++t) {
            float part = 0.f;
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) part += r.qf(t, c) * r.kf(s, c) * fexp2(u[t][c] - u[s][c]);
            const float tot = wave_sum(part * ig[s]);
            if (c16 == t && g == (s >> 2)) {
                if ((s & 3) == 0) acc[0] += tot;
                else if ((s & 3) == 1) acc[1] += tot;
                else if ((s & 3) == 2) acc[2] += tot;
                else acc[3] += tot;
            }
        }
    }
    return acc;
}

// ------------------------------------------------------------------------------------
// Score blocks of a diagonal tile: pairs (query block i, key block j <= i).  Wave w computes
// three pairs (waves 2 and 3 repeat one pair to keep the instruction stream uniform; its
// result is not stored).  Operand rows (per-channel gate):
//   diagonal (w, w):         KD block w  x  QD block w
//   adjacent (i, i-1):       KO block i-1 x  QD block i
//   (2,0), (3,1), (3,0):     referenced to the end of block 1 through X
struct Pairs {
    int i[3], j[3];
    int arow[3], brow[3];  // row offsets in the selected arrays
    bool ax[3], bx[3];     // operand from X instead of (KO | KD | raw k) / (QD | raw q)
};
__device__ __forceinline__ void set_pair(Pairs &P, int kp, int i, int j, bool ch) {
    P.i[kp] = i;
    P.j[kp] = j;
    if (ch && j + 1 < i) {
        // keys of block j and queries of block i referenced to the end of block 1
        P.ax[kp] = j == 0;
        P.arow[kp] = j == 0 ? 0 : 16 * j;
        P.bx[kp] = i == 3;
        P.brow[kp] = i == 3 ? 16 : 16 * i;
    } else {
        P.ax[kp] = false;
        P.arow[kp] = 16 * j;
        P.bx[kp] = false;
        P.brow[kp] = 16 * i;
    }
}
__device__ __forceinline__ Pairs make_pairs(int w, bool ch) {
    Pairs P;
    set_pair(P, 0, w, w, ch);
    switch (w) {
        case 0: set_pair(P, 1, 1, 0, ch); set_pair(P, 2, 3, 2, ch); break;
        case 1: set_pair(P, 1, 2, 0, ch); set_pair(P, 2, 3, 1, ch); break;
        case 2: set_pair(P, 1, 2, 1, ch); set_pair(P, 2, 2, 1, ch); break;
        default: set_pair(P, 1, 3, 0, ch); set_pair(P, 2, 3, 0, ch); break;
    }
    return P;
}

// ------------------------------------------------------------------------------------
// chunk_output_kernel: grid = BH * nseg * ndv (* qsplit) workgroups of 256 threads.
// With a.qsplit > 1 (large chunks, every chunk its own segment) the workgroups of one chunk
// each output one query tile qi against the chunk-start state from the scan: the second level
// of sequence parallelism of the tiled large-chunk form.  Workgroup qi prepares tiles
// 0 .. qi (their decays, and for a per-channel gate their scaled keys, which every workgroup
// of the chunk writes to the same scratch slot with the same bytes) and runs the products of
// tile qi only; the workgroup of the last tile of the last chunk also advances the state to
// the final state.
template <class C>
__global__ __launch_bounds__(256, 1) void chunk_output_kernel(KArgs a) {
    static_assert(C::H16 == 0, "the backward pass's instances run the ws and sg kernels");
    using OpT = typename C::OpT;
    using Frag = typename C::Frag;
    using Half = typename C::Half;
    extern __shared__ __align__(256) unsigned char smem[];
    const LdsPlan lp = lds_plan(C::OPB, C::DK, C::CH, a.nt);
    OpT *sQ = reinterpret_cast<OpT *>(smem + lp.q);
    OpT *sK = reinterpret_cast<OpT *>(smem + lp.k);
    OpT *sKD = reinterpret_cast<OpT *>(smem + lp.kd);
    OpT *sX = reinterpret_cast<OpT *>(smem + lp.x);
    OpT *sQI = reinterpret_cast<OpT *>(smem + lp.qi);
    OpT *sKT = reinterpret_cast<OpT *>(smem + lp.kst);
    OpT *sP = reinterpret_cast<OpT *>(smem + lp.pbuf);
    OpT *sV = reinterpret_cast<OpT *>(smem + lp.vb);
    OpT *sVo = reinterpret_cast<OpT *>(smem + lp.voff);
    float *sAb = reinterpret_cast<float *>(smem + lp.ablk);
    float *sQTF = reinterpret_cast<float *>(smem + lp.qtf);
    float *sAt = reinterpret_cast<float *>(smem + lp.atile);
    float *sBr = reinterpret_cast<float *>(smem + lp.brow);
    float *sLr = reinterpret_cast<float *>(smem + lp.lrow);

    const int wg = (int)blockIdx.x;
    int id = xcd_remap(wg, a.nwg);
    const int dvt = id % a.ndv;
    id /= a.ndv;
    const bool qs = C::MT && a.qsplit > 1;
    int qi = 0;  // with qs: the query tile this workgroup outputs
    if (qs) {
        qi = id % a.qsplit;
        id /= a.qsplit;
    }
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
    // with qs the segment is one chunk; a tile past the sequence end has nothing to output
    if (qs && t_begin + kTile * qi >= t_end) return;
    const bool last_seg = seg == a.nseg - 1;
    // with qs, the workgroup of the last tile of the last chunk also advances the state
    const bool fin_wg = !qs || (last_seg && t_begin + kTile * (qi + 1) >= t_end);
    const int chl = C::CPL * lane;
    const Rs rs = make_rs<C>(a, bh, h);
    rsrc_t rke = make_rsrc(a.out, 0);
    if constexpr (C::CH && C::MT) {
        const uint64_t kb = ke_scratch_bytes(C::OPB, C::DK, true, a.nt);
        const uint64_t slot = qs ? (uint64_t)bh * a.nseg + seg : (uint64_t)wg;
        rke = make_rsrc(reinterpret_cast<char *>(a.ws_ke) + slot * kb, kb);
    }

    // State S[d][col], d = 16n + 4g + e, held across chunks in registers.
    f32x4 S[C::NBD];
#pragma unroll
    for (int n = 0; n < C::NBD; ++n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int d = 16 * n + 4 * g + e;
            float x = 0.f;
            if (seg > 0)
                x = a.ws_state[(((size_t)bh * (a.nseg - 1) * a.nsub + seg * a.nsub - 1) * C::DK + d) * Dv + col];
            else if (a.s0)
                x = a.s0[((size_t)bh * C::DK + d) * Dv + col];
            S[n][e] = x;
        }
    }
    f32x4 dS[C::MT ? C::NBD : 1];

    Raw<C> raw;
    load_unit<C, true>(raw, rs, t_begin, 0, w, lane, tid, dv0, Dv);

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
        const int tau_end = qs ? qi + 1 : ntile;

        for (int tau = 0; tau < tau_end; ++tau) {
            const int T0 = c0 + kTile * tau;
            // with qs only tile qi is output; the tiles before it are prepared for its pairs
            const bool out_tile = !qs || tau == qi;
            f32x4 O[4];
            f32x4 Pd[3];
#pragma unroll
            for (int i = 0; i < 4; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 3; ++i) Pd[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            float Tt = 0.f;  // scalar gates: log2 decay across this tile
            Frag vfr[2];
            bool harsh = false;

#pragma unroll 1
            for (int sl = 0; sl < C::NSLAB; ++sl) {
                OpT *sQs = sQ + (C::MT ? sl : 0) * 64 * C::RP;
                // ---------------- preparation of this unit -> LDS
                if (sl == 0) v_to_lds<C>(raw, sV, tid);
                if constexpr (C::CH) {
                    ChGate<C> G;
                    ch_gate<C>(G, raw, sAb, w, lane);
                    harsh = G.harsh;
                    float ig[16];
                    if (rs.has_li) {
                        const float y = raw.lis * kLog2e;
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) ig[rr] = fexp2(lane_bcast(y, 16 * w + rr));
                    } else {
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) ig[rr] = 1.f;
                    }
                    if (harsh) Pd[0] = ch_diag_exact<C>(Pd[0], raw, lane, rs.has_li);
                    float fqi[C::CPL], ainv[C::CPL], xs[C::CPL];
#pragma unroll
                    for (int c = 0; c < C::CPL; ++c) {
                        fqi[c] = Wc[sl][c] * G.pre[c];
                        ainv[c] = frcp(G.eq[15][c]);
                        xs[c] = w == 0 ? G.ab[1][c] : G.ab[2][c];  // X scale for waves 0 and 3
                        const int d = sl * C::SLAB + chl + c;
                        if (w == 0) sAt[tau * C::DK + d] = G.at[c];
                        if constexpr (C::MT) sQTF[w * C::DK + d] = G.pre[c];
                        Wc[sl][c] *= G.at[c];
                    }
                    const bool mt_store = C::MT && tau < a.nt - 1;
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        Half kt4[C::CPL];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int rr = 4 * g4 + e;
                            const int row = 16 * w + rr;
                            float qd[C::CPL], ko[C::CPL], kd[C::CPL], qi[C::CPL], ke[C::CPL], xv[C::CPL];
#pragma unroll
                            for (int c = 0; c < C::CPL; ++c) {
                                qd[c] = raw.qf(rr, c) * G.eq[rr][c];
                                ko[c] = raw.kf(rr, c) * ig[rr] * G.ek[rr][c];
                                kd[c] = ko[c] * ainv[c];
                                qi[c] = qd[c] * fqi[c];
                                ke[c] = ko[c] * G.post[c];
                                xv[c] = (w == 0 ? ko[c] : qd[c]) * xs[c];
                                kt4[c][e] = (OpT)ke[c];
                            }
                            st_row<C>(sQs + row * C::RP + chl, qd);
                            st_row<C>(sK + row * C::RP + chl, ko);
                            st_row<C>(sKD + row * C::RP + chl, kd);
                            st_row<C>(sQI + row * C::RP + chl, qi);
                            if (w == 0) st_row<C>(sX + rr * C::RP + chl, xv);
                            if (w == 3) st_row<C>(sX + (16 + rr) * C::RP + chl, xv);
                            if constexpr (C::MT) {
                                if (mt_store) {
                                    const uint32_t off = (uint32_t)(((tau * 64 + row) * C::DK + sl * C::SLAB + chl) * C::OPB);
                                    uint32_t bits;
                                    if constexpr (C::CPL == 2) {
                                        bits = __builtin_bit_cast(uint32_t, f16x2{(f16)ke[0], (f16)ke[1]});
                                    } else if constexpr (C::F32) {
                                        bits = __float_as_uint(ke[0]);
                                    } else {
                                        bits = (uint32_t)__builtin_bit_cast(uint16_t, (f16)ke[0]);
                                    }
                                    if constexpr (C::OPB == 2 && C::CPL == 1)
                                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)bits, rke, (int)off, 0, 0);
                                    else
                                        __builtin_amdgcn_raw_buffer_store_b32(bits, rke, (int)off, 0, 0);
                                }
                            }
                        }
#pragma unroll
                        for (int c = 0; c < C::CPL; ++c)
                            *reinterpret_cast<Half *>(sKT + kt_off<C>(chl + c, kslot(16 * w + 4 * g4))) = kt4[c];
                    }
                } else {
                    // scalar gates: running log2 decay over the tile's rows (lane = row)
                    const float x = log2_decay(raw.las);
                    const float y = raw.lis * kLog2e;
                    const float bl = scan_incl(x, lane);
                    Tt = lane_bcast(bl, 63);
                    if (w == 0 && sl == 0) {
                        sBr[kTile * tau + lane] = Bc + bl;
                        sLr[kTile * tau + lane] = y;
                    }
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        Half kt4[C::CPL];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int rr = 4 * g4 + e;
                            const int row = 16 * w + rr;
                            const float blr = lane_bcast(bl, 16 * w + rr);
                            const float eb = fexp2(Bc + blr);
                            const float ekr = fexp2(Tt - blr + lane_bcast(y, 16 * w + rr));
                            float qv[C::CPL], kv[C::CPL], qi[C::CPL];
#pragma unroll
                            for (int c = 0; c < C::CPL; ++c) {
                                qv[c] = raw.qf(rr, c);
                                kv[c] = raw.kf(rr, c);
                                qi[c] = qv[c] * eb;
                                kt4[c][e] = (OpT)(kv[c] * ekr);
                            }
                            st_row<C>(sQs + row * C::RP + chl, qv);
                            st_row<C>(sK + row * C::RP + chl, kv);
                            st_row<C>(sQI + row * C::RP + chl, qi);
                        }
#pragma unroll
                        for (int c = 0; c < C::CPL; ++c)
                            *reinterpret_cast<Half *>(sKT + kt_off<C>(chl + c, kslot(16 * w + 4 * g4))) = kt4[c];
                    }
                }
                if constexpr (C::CH && C::MT)
                    full_barrier();  // also publishes this tile's key scratch to the other waves
                else
                    lds_barrier();

                // ---------------- prefetch the next unit while this one computes.  Issued
                // unconditionally (after the last unit it reads rows past the segment, which
                // are never used; past the (batch, head) extent the range check returns zero),
                // so the compiler does not merge register copies that wait for the loads.
                {
                    int Tn = c0 + a.chunk, sn = 0;
                    if (sl + 1 < C::NSLAB) {
                        Tn = T0;
                        sn = sl + 1;
                    } else if (tau + 1 < ntile) {
                        Tn = T0 + kTile;
                    }
                    load_unit<C, true>(raw, rs, Tn, sn, w, lane, tid, dv0, Dv);
                }

                if (sl == 0) {
#pragma unroll
                    for (int p = 0; p < 2; ++p) vfr[p] = ld8<C>(sV + ((p * 4 + g) * 64 + vsw(16 * w + c16)) * 8);
                }

                // ---------------- diagonal-tile score blocks (transposed): P^T(j,i) over this slab
                if (out_tile) {
                    const Pairs pr = make_pairs(w, C::CH);
                    const OpT *pa[3], *pb[3];
#pragma unroll
                    for (int kp = 0; kp < 3; ++kp) {
                        const OpT *ka = (C::CH && kp == 0) ? sKD : (pr.ax[kp] ? sX : sK);
                        pa[kp] = ka + (pr.arow[kp] + c16) * C::RP;
                        pb[kp] = (pr.bx[kp] ? sX : sQs) + (pr.brow[kp] + c16) * C::RP;
                    }
#pragma unroll
                    for (int m = 0; m < C::KSTEP; ++m) {
                        const int ch = 32 * m + 8 * g;
                        Frag af[3], bf[3];
#pragma unroll
                        for (int kp = 0; kp < 3; ++kp) {
                            af[kp] = ld8<C>(pa[kp] + ch);
                            bf[kp] = ld8<C>(pb[kp] + ch);
                        }
                        if (!harsh) Pd[0] = mma(af[0], bf[0], Pd[0]);
                        Pd[1] = mma(af[1], bf[1], Pd[1]);
                        Pd[2] = mma(af[2], bf[2], Pd[2]);
                    }
                }

                // ---------------- inter-chunk term: O += QI . S (rows of this slab)
                if (out_tile) {
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
                    for (int m = 0; m < C::KSTEP; ++m) {
                        Frag qa[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const OpT *row = sQI + (16 * i + c16) * C::RP + 32 * m + 4 * g;
                            qa[i] = ld4x2<C>(row, row + 16);
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i) O[i] = mma(qa[i], sb[m], O[i]);
                    }
                }

                // ---------------- chunk-state contribution of this tile (rows of this slab)
                if (fin_wg) {
                    f32x4 acc[C::NBS];
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
                        acc[n] = (C::MT ? dS[nn] : S[nn]) * at;
                    }
#pragma unroll
                    for (int p = 0; p < 2; ++p) {
                        Frag ka[C::NBS];
#pragma unroll
                        for (int n = 0; n < C::NBS; ++n) ka[n] = ld8<C>(sKT + kt_off<C>(16 * n + c16, (p * 4 + g) * 8));
#pragma unroll
                        for (int n = 0; n < C::NBS; ++n) acc[n] = mma(ka[n], vfr[p], acc[n]);
                    }
#pragma unroll
                    for (int n = 0; n < C::NBS; ++n) {
                        const int nn = sl * C::NBS + n;
                        if constexpr (C::MT)
                            dS[nn] = acc[n];
                        else
                            S[nn] = acc[n];
                    }
                }
                if (sl + 1 < C::NSLAB) lds_barrier();  // the next slab rewrites the slab arrays
            }  // slabs

            // ---------------- diagonal tile: mask, store scores, multiply by values
            if (out_tile) {
                const Pairs pr = make_pairs(w, C::CH);
#pragma unroll
                for (int kp = 0; kp < 3; ++kp) {
                    if (kp == 2 && w >= 2) continue;  // repeated pair
                    const int i = pr.i[kp], j = pr.j[kp];
                    Half pv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 4 * g + e;  // key row in block j
                        const bool masked = i == j && s > c16;
                        float x = masked ? 0.f : Pd[kp][e];
                        if constexpr (!C::CH) {
                            if (!masked) {
                                const int ts = kTile * tau + 16 * i + c16, ss = kTile * tau + 16 * j + s;
                                x *= fexp2(sBr[ts] - sBr[ss] + sLr[ss]);
                            }
                        }
                        pv[e] = (OpT)x;
                    }
                    *reinterpret_cast<Half *>(sP + ((i * 2 + (j >> 1)) * 64 + lane) * 8 + 4 * (j & 1)) = pv;
                }
                if (w == 0 || w == 2) {  // key blocks after the query block stay zero
                    const Half z{(OpT)0.f, (OpT)0.f, (OpT)0.f, (OpT)0.f};
                    *reinterpret_cast<Half *>(sP + ((w * 2 + (w >> 1)) * 64 + lane) * 8 + 4) = z;
                }
            }
            lds_barrier();
            if (out_tile) {
                Frag pa[6];
                pa[0] = ld8<C>(sP + ((0 * 2 + 0) * 64 + lane) * 8);
                pa[1] = ld8<C>(sP + ((1 * 2 + 0) * 64 + lane) * 8);
                pa[2] = ld8<C>(sP + ((2 * 2 + 0) * 64 + lane) * 8);
                pa[3] = ld8<C>(sP + ((3 * 2 + 0) * 64 + lane) * 8);
                pa[4] = ld8<C>(sP + ((2 * 2 + 1) * 64 + lane) * 8);
                pa[5] = ld8<C>(sP + ((3 * 2 + 1) * 64 + lane) * 8);
#pragma unroll
                for (int i = 0; i < 4; ++i) O[i] = mma(pa[i], vfr[0], O[i]);
                O[2] = mma(pa[4], vfr[1], O[2]);
                O[3] = mma(pa[5], vfr[1], O[3]);
            }

            // ---------------- earlier tiles of the same chunk (large chunks)
            if (C::MT && out_tile) {
#pragma unroll 1
                for (int kj = 0; kj < tau; ++kj) {
                    lds_barrier();  // previous readers of sP / sVo are done
                    {
                        Raw<C> vr;
                        const int Tk = c0 + kTile * kj;
                        const uint32_t cq = dv0 + 4 * (tid & 15);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t off = ((uint32_t)(Tk + 4 * (tid >> 4) + e) * Dv + cq) * C::IB;
                            if constexpr (C::F32) {
                                const u32x4 x = bld128(rs.v, off);
#pragma unroll
                                for (int jj = 0; jj < 4; ++jj) vr.v[e][jj] = x[jj];
                            } else {
                                const u32x2 x = bld64(rs.v, off);
                                vr.v[e][0] = x[0];
                                vr.v[e][1] = x[1];
                            }
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
                            Frag af[4];
                            if constexpr (C::CH) {
                                const int d = sl * C::SLAB + ch;
                                f32x4 f0 = lds_ld<f32x4>(sQTF + w * C::DK + d);
                                f32x4 f1 = lds_ld<f32x4>(sQTF + w * C::DK + d + 4);
                                for (int tp = kj + 1; tp < tau; ++tp) {
                                    f0 *= lds_ld<f32x4>(sAt + tp * C::DK + d);
                                    f1 *= lds_ld<f32x4>(sAt + tp * C::DK + d + 4);
                                }
                                bf = scale8<C>(bf, f0, f1);
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    af[j] = gld8<C, 1>(rke, (uint32_t)(((kj * 64 + 16 * j + c16) * C::DK + d) * C::OPB));
                            } else {
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    af[j] = gld8_in<C, kOpK>(rs.k, (uint32_t)(((c0 + kTile * kj + 16 * j + c16) * C::DK +
                                                                         sl * C::SLAB + ch) * C::IB));
                            }
#pragma unroll
                            for (int j = 0; j < 4; ++j) Po[j] = mma(af[j], bf, Po[j]);
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        Half pv;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float x = Po[j][e];
                            if constexpr (!C::CH) {
                                const int ts = kTile * tau + 16 * w + c16, ss = kTile * kj + 16 * j + 4 * g + e;
                                x *= fexp2(sBr[ts] - sBr[ss] + sLr[ss]);
                            }
                            pv[e] = (OpT)x;
                        }
                        *reinterpret_cast<Half *>(sP + ((w * 2 + (j >> 1)) * 64 + lane) * 8 + 4 * (j & 1)) = pv;
                    }
                    lds_barrier();
                    {
                        Frag vo[2], pa[8];
#pragma unroll
                        for (int p = 0; p < 2; ++p) vo[p] = ld8<C>(sVo + ((p * 4 + g) * 64 + vsw(16 * w + c16)) * 8);
#pragma unroll
                        for (int q = 0; q < 8; ++q) pa[q] = ld8<C>(sP + (q * 64 + lane) * 8);
#pragma unroll
                        for (int p = 0; p < 2; ++p)
#pragma unroll
                            for (int i = 0; i < 4; ++i) O[i] = mma(pa[i * 2 + p], vo[p], O[i]);
                    }
                }
            }

            // ---------------- store the tile's outputs (rows past the sequence end are dropped)
            if (out_tile) {
                const uint32_t ob = ((uint32_t)(T0 + 4 * g) * Dv + col) * 4u;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O[i][e]), rs.out,
                                                              (int)(ob + (uint32_t)((16 * i + e) * Dv * 4)), 0, 0);
            }
            if constexpr (!C::CH) Bc += Tt;
            lds_barrier();  // LDS tile arrays are rewritten by the next unit
        }  // tiles

        if (C::MT && fin_wg) {
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

    if (last_seg && fin_wg && a.fin) {
#pragma unroll
        for (int n = 0; n < C::NBD; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.fin[((size_t)bh * C::DK + 16 * n + 4 * g + e) * Dv + col] = S[n][e];
    }
}

// ------------------------------------------------------------------------------------
// Warp-specialised chunk output for 64-token chunks whose key channels fit one slab.
// grid = BH * nseg * ndv workgroups of 512 threads.  Waves 4..7 (producers) load chunk k+1
// and prepare its gate-scaled operands while waves 0..3 (consumers) run the matrix
// products of chunk k; every SIMD holds one producer and one consumer wave, so the
// vector-ALU gate work and the matrix-core work of neighbouring chunks overlap.  Two
// barriers per chunk:
//   phase A  consumers: score blocks and inter-chunk term of chunk k; values of chunk k+1
//            from registers into buffer (k+1)&1, loads of the values of chunk k+2
//            producers: gates of chunk k+1 (block decays, factors, exact partial scores
//            and, for scalar gates, keys^T into buffer (k+1)&1); fp16 operands: q, k of
//            chunk k+1 into buffer (k+1)&1; loads of chunk k+2
//   B1
//   phase B  consumers: scores x values, state update (buffer k&1), output staging
//            producers: fp32 operands: q, k of chunk k+1 into the single buffers;
//            per-channel gate: keys^T scaled to the chunk end, the chunk decay and the
//            products of block decays into buffer (k+1)&1 (they need the decays of all
//            four blocks, published before B1)
//   B2       consumers: staged output tile to memory
// Producer lane mapping: producer wave pw owns the 16-row block pw; lane l owns channels
// CPL*l .. +CPL-1, so every load instruction covers whole rows of q, k and the gates, and a
// lane walks its block's 16 rows for the running decay products.

// The loads of one unit in three groups: the producers reissue the q/k and gate groups for
// the chunk after next as soon as they have consumed those registers; the consumers load the
// values (wave index in place of pw).
template <class C>
__device__ __forceinline__ void load_p_v(Raw<C> &r, const Rs &rs, int T0, int pw, int lane, int dv0, int Dv) {
    const int tp = 64 * pw + lane;
    const uint32_t c0 = dv0 + 4 * (tp & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t off = (in_row<C>(rs, T0 + 4 * (tp >> 4) + e) * Dv + c0) * C::IB;
        if constexpr (C::F32) {
            const u32x4 x = bld128(rs.v, off);
#pragma unroll
            for (int j = 0; j < 4; ++j) r.v[e][j] = x[j];
        } else {
            const u32x2 x = bld64(rs.v, off);
            r.v[e][0] = x[0];
            r.v[e][1] = x[1];
        }
    }
}
template <class C>
__device__ __forceinline__ void load_p_gates(Raw<C> &r, const Rs &rs, int T0, int pw, int lane) {
    if constexpr (C::CH) {
        const int ch0 = C::CPL * lane;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const uint32_t goff = (gate_row<C>(rs, T0 + 16 * pw + rr) * C::DK + ch0) * 4u;
            if constexpr (C::CPL == 2) {
                const u32x2 g2 = bld64(rs.la, goff);
                r.la[rr][0] = __uint_as_float(g2[0]);
                r.la[rr][1] = __uint_as_float(g2[1]);
            } else {
                r.la[rr][0] = __uint_as_float(bld32(rs.la, goff));
            }
        }
    }
    // scalar gates: one branch-free load for every kind (per token: stride 4; fixed per head:
    // stride 0, masked past the sequence end where it is used; none: empty resource)
    const uint32_t t = (uint32_t)(T0 + lane);
    if constexpr (!C::CH) r.las = __uint_as_float(bld32(rs.la, t * rs.gstride));
    r.lis = __uint_as_float(bld32(rs.li, t * 4u));
}
template <class C>
__device__ __forceinline__ void load_p_qk(Raw<C> &r, const Rs &rs, int T0, int pw, int lane) {
    const int ch0 = C::CPL * lane;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const uint32_t off = (in_row<C>(rs, T0 + 16 * pw + rr) * C::DK + ch0) * C::IB;
        if constexpr (C::CPL == 2 || C::F32) {
            r.q[rr] = bld32(rs.q, off);
            r.k[rr] = bld32(rs.k, off);
        } else {
            r.q[rr] = __builtin_amdgcn_raw_buffer_load_b16(rs.q, (int)off, 0, 0);
            r.k[rr] = __builtin_amdgcn_raw_buffer_load_b16(rs.k, (int)off, 0, 0);
        }
    }
}

// CPL operands of one row packed into 32 bits (fp16 pair / one fp16 / one fp32).
template <class C>
__device__ __forceinline__ uint32_t pack_ops(const float *x) {
    if constexpr (C::F32) {
        return __float_as_uint(x[0]);
    } else if constexpr (C::CPL == 2) {
        return __builtin_bit_cast(uint32_t, f16x2{(f16)x[0], (f16)x[1]});
    } else {
        return (uint32_t)__builtin_bit_cast(uint16_t, (f16)x[0]);
    }
}
template <class C>
__device__ __forceinline__ void st_packed(typename C::OpT *row, uint32_t v) {
    if constexpr (C::F32 || C::CPL == 2)
        *reinterpret_cast<uint32_t *>(row) = v;
    else
        *reinterpret_cast<uint16_t *>(row) = (uint16_t)v;
}

template <class C>
struct ProdVals {
    uint32_t qd[16];                     // packed q operands of rows 16pw+rr for phase B
    uint32_t ko[16];                     // packed k operands (block-end reference)
    float kf[C::CH ? 16 : 1][C::CPL];    // per-channel gate: k at the block end, fp32, for keys^T
    float ag[C::CPL];                    // per-channel gate: decay across this block
};

// q and k rows of block pw into the buffers at sQ, sK.
template <class C>
__device__ __forceinline__ void ws_store_qk(const ProdVals<C> &pv, typename C::OpT *sQ, typename C::OpT *sK,
                                            int pw, int lane) {
    const int pc = chperm(C::CPL * lane);  // rows hold channels in chperm order
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const int row = 16 * pw + rr;
        st_packed<C>(sQ + row * C::RP + pc, pv.qd[rr]);
        st_packed<C>(sK + row * C::RP + pc, pv.ko[rr]);
    }
}

// Exact diagonal-block partial scores of block pw when some of its channels decay too
// strongly across the block for scaled fp16 operands (rare; kept out of line so the common
// path keeps its registers).  For every pair s <= t of the block: the sum over the
// strongly decayed channels of q_td k_sd 2^(u_td - u_sd) i_s, u the log2 running decay,
// reduced over the wave's lanes (all channels) into dst[t (t + 1) / 2 + s].
template <class C>
__device__ __attribute__((noinline)) void ws_exact_block(Raw<C> raw, float *dst, int pw, int lane, bool has_li) {
    float u[16][C::CPL], hcm[C::CPL];
#pragma unroll
    for (int c = 0; c < C::CPL; ++c) {
        float run = 0.f, prod = 1.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            run += log2_decay(raw.la[rr][c]);
            u[rr][c] = run;
            prod *= fexp2(raw.la[rr][c] * kLog2e);
        }
        hcm[c] = !(prod >= C::kMinDiagDecay) ? 1.f : 0.f;
    }
    const float y = raw.lis * kLog2e;
    float ig[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) ig[rr] = has_li ? fexp2(lane_bcast(y, 16 * pw + rr)) : 1.f;
    for (int t = 0; t < 16; ++t) {
        for (int s2 = 0; s2 <= t; ++s2) {
            float part = 0.f;
#pragma unroll
            for (int c = 0; c < C::CPL; ++c)
                part += hcm[c] * raw.qf(t, c) * raw.kf(s2, c) * fexp2(u[t][c] - u[s2][c]);
            part *= ig[s2];
            part = wave_sum(part);
            if (lane == 0) dst[t * (t + 1) / 2 + s2] = part;
        }
    }
}

// Producer phase A: gates of one chunk (block pw), values, block decays and exact partial
// scores into buffer nb; scalar gates also write keys^T.  q/k operands stay in registers.
template <class C>
__device__ __forceinline__ void ws_produce_a(ProdVals<C> &pv, Raw<C> &raw, const LdsPlanWs &lp,
                                             unsigned char *smem, int nb, int pw, int lane, bool has_li,
                                             bool row_valid, const Rs &rs, int Tn, int dv0, int Dv) {
    using OpT = typename C::OpT;
    using Half = typename C::Half;
    const int ch0 = C::CPL * lane;
    unsigned char *buf = smem + lp.dbl + (uint32_t)nb * lp.dstride;
    OpT *sKT = reinterpret_cast<OpT *>(buf + lp.kst);
    float *sAb = reinterpret_cast<float *>(buf + lp.ab);
    float *sAi = reinterpret_cast<float *>(buf + lp.ainv);
    float ig[16];
    {
        const float y = raw.lis * kLog2e;
        if constexpr (C::CH) {
            if (has_li) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) ig[rr] = fexp2(lane_bcast(y, 16 * pw + rr));
            } else {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) ig[rr] = 1.f;
            }
        }
    }

    if constexpr (C::CH) {
        float eq[16][C::CPL], ek[16][C::CPL];
#pragma unroll
        for (int c = 0; c < C::CPL; ++c) {
            float run = 1.f;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const float al = fexp2(raw.la[rr][c] * kLog2e);
                ek[rr][c] = al;
                run *= al;
                eq[rr][c] = run;
            }
            run = 1.f;
#pragma unroll
            for (int rr = 15; rr >= 0; --rr) {
                const float al = ek[rr][c];
                ek[rr][c] = run;
                run *= al;
            }
        }
        bool any_h = false;
        float fa[C::CPL], fi[C::CPL];
#pragma unroll
        for (int c = 0; c < C::CPL; ++c) {
            const float ag = eq[15][c];
            pv.ag[c] = ag;
            const bool hc = !(ag >= C::kMinDiagDecay);
            any_h |= hc;
            fa[c] = ag;
            fi[c] = hc ? 0.f : frcp(ag);
            // block decays scale q and k fragments: stored in the rows' chperm channel order
            sAb[pw * C::SLAB + chperm(ch0 + c)] = ag;
            if constexpr (C::F32) sAi[pw * C::SLAB + chperm(ch0 + c)] = fi[c];
        }
        {
            OpT *sF = reinterpret_cast<OpT *>(buf + lp.fh);
            const int pc = chperm(ch0);
            if (pw < 3) st_packed<C>(sF + (kFhA0 + pw) * C::SLAB + pc, pack_ops<C>(fa));
            st_packed<C>(sF + (kFhInv + pw) * C::SLAB + pc, pack_ops<C>(fi));
        }
        // channels of this block whose decay is too strong: exact partial scores (rare)
        const bool harsh = __ballot(any_h) != 0ull;
        if (harsh)
            ws_exact_block<C>(raw, reinterpret_cast<float *>(buf + lp.xact) + pw * 136, pw, lane, has_li);
        if (lane == 0) reinterpret_cast<int *>(buf + lp.xflag)[pw] = harsh ? 1 : 0;
        load_p_gates<C>(raw, rs, Tn, pw, lane);
        __builtin_amdgcn_sched_barrier(0);  // keep the reload ahead of the work below
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float qd[C::CPL], ko[C::CPL];
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) {
                qd[c] = raw.qf(rr, c) * eq[rr][c];
                ko[c] = raw.kf(rr, c) * ig[rr] * ek[rr][c];
                pv.kf[rr][c] = ko[c];
            }
            pv.qd[rr] = pack_ops<C>(qd);
            pv.ko[rr] = pack_ops<C>(ko);
        }
        load_p_qk<C>(raw, rs, Tn, pw, lane);
        if (lp.qkd) ws_store_qk<C>(pv, reinterpret_cast<OpT *>(buf + lp.q), reinterpret_cast<OpT *>(buf + lp.k), pw, lane);
    } else {
        // scalar gates: running log2 decay over the tile's rows (lane = row); rows past the
        // sequence end carry no decay (a fixed per-head gate is loaded for them too)
        float *sBr = sAb;  // [64] log2 running decay, row 63 = decay across the tile
        float *sLr = sAi;  // [64] log2 input gate
        const float x = row_valid ? log2_decay(raw.las) : 0.f;
        const float y = raw.lis * kLog2e;
        const float bl = scan_incl(x, lane);
        const float Tt = lane_bcast(bl, 63);
        if (pw == 0) {
            sBr[lane] = bl;
            sLr[lane] = y;
        }
        const float wk = fexp2(Tt - bl + y);  // weight of key row `lane` in the state update
        load_p_gates<C>(raw, rs, Tn, pw, lane);
        __builtin_amdgcn_sched_barrier(0);  // keep the reload ahead of the work below
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            Half kt4[C::CPL];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 4 * g4 + e;
                const float ekr = lane_bcast(wk, 16 * pw + rr);
                float qv[C::CPL], kv[C::CPL];
#pragma unroll
                for (int c = 0; c < C::CPL; ++c) {
                    qv[c] = raw.qf(rr, c);
                    kv[c] = raw.kf(rr, c);
                    kt4[c][e] = (OpT)(kv[c] * ekr);
                }
                pv.qd[rr] = pack_ops<C>(qv);
                pv.ko[rr] = pack_ops<C>(kv);
            }
#pragma unroll
            for (int c = 0; c < C::CPL; ++c)
                *reinterpret_cast<Half *>(sKT + kt_off<C>(ch0 + c, kslot(16 * pw + 4 * g4))) = kt4[c];
        }
        load_p_qk<C>(raw, rs, Tn, pw, lane);
        if (lp.qkd) ws_store_qk<C>(pv, reinterpret_cast<OpT *>(buf + lp.q), reinterpret_cast<OpT *>(buf + lp.k), pw, lane);
    }
}

// Producer phase B: q and k of the prepared chunk into the single buffers; per-channel gate:
// keys^T scaled to the chunk end (decay of the blocks after this one, from the block decays
// all producer waves published before B1) and the chunk decay into buffer nb.
template <class C>
__device__ __forceinline__ void ws_produce_b(const ProdVals<C> &pv, const LdsPlanWs &lp, unsigned char *smem,
                                             int nb, int pw, int lane) {
    using OpT = typename C::OpT;
    using Half = typename C::Half;
    const int ch0 = C::CPL * lane;
    const int pc = chperm(ch0);  // rows hold channels in chperm order
    if (!lp.qkd) ws_store_qk<C>(pv, reinterpret_cast<OpT *>(smem + lp.q), reinterpret_cast<OpT *>(smem + lp.k), pw, lane);
    if constexpr (C::CH) {
        unsigned char *buf = smem + lp.dbl + (uint32_t)nb * lp.dstride;
        const float *sAb = reinterpret_cast<const float *>(buf + lp.ab);
        OpT *sKT = reinterpret_cast<OpT *>(buf + lp.kst);
        float post[C::CPL], all[C::CPL];
#pragma unroll
        for (int c = 0; c < C::CPL; ++c) {
            float p1 = 1.f, a = 1.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float au = u == pw ? pv.ag[c] : sAb[u * C::SLAB + chperm(ch0 + c)];
                a *= au;
                if (u > pw) p1 *= au;
            }
            post[c] = p1;
            all[c] = a;
        }
        if (pw == 0) {
            float *sAt = reinterpret_cast<float *>(buf + lp.at);
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) sAt[ch0 + c] = all[c];
        } else {
            // products of block decays for the inter-chunk term and the rescaled queries:
            // wave 1 a_0 a_1, wave 2 a_0 a_1 a_2, wave 3 a_1 a_2
            float f[C::CPL];
#pragma unroll
            for (int c = 0; c < C::CPL; ++c) {
                const int cp = chperm(ch0 + c);
                const float a1 = sAb[C::SLAB + cp];
                const float a2 = pw == 1 ? 1.f : sAb[2 * C::SLAB + cp];
                const float a0 = pw == 3 ? 1.f : sAb[cp];
                f[c] = a0 * a1 * a2;
            }
            const int row = pw == 1 ? kFhP2 : pw == 2 ? kFhP3 : kFhA12;
            st_packed<C>(reinterpret_cast<OpT *>(buf + lp.fh) + row * C::SLAB + pc, pack_ops<C>(f));
        }
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            Half kt4[C::CPL];
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int c = 0; c < C::CPL; ++c) kt4[c][e] = (OpT)(pv.kf[4 * g4 + e][c] * post[c]);
#pragma unroll
            for (int c = 0; c < C::CPL; ++c)
                *reinterpret_cast<Half *>(sKT + kt_off<C>(ch0 + c, kslot(16 * pw + 4 * g4))) = kt4[c];
        }
    }
}

template <class C, bool LI>
__global__ __launch_bounds__(512, 1) void chunk_output_ws_kernel(KArgs a) {
    static_assert(!C::MT && C::NSLAB == 1, "single-tile, single-slab configuration");
    using OpT = typename C::OpT;
    using Frag = typename C::Frag;
    using Half = typename C::Half;
    extern __shared__ __align__(256) unsigned char smem[];
    const LdsPlanWs lp = lds_plan_ws(C::OPB, C::DK);

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
    const int t_begin = seg * a.seg_len;
    const int t_end = min(L, t_begin + a.seg_len);
    const int nch = (t_end - t_begin + kTile - 1) / kTile;
    const Rs rs = make_rs<C>(a, bh, h);
    [[maybe_unused]] const OutMap om = C::H16 != 0 ? make_out_map(a, bh, dvt) : OutMap{};

    if (w >= 4) {
        // ============================ producers
        const int pw = w - 4;
        Raw<C> raw;
        ProdVals<C> pv;
        // The loop body is unconditional: in the last iteration the producers prepare a chunk
        // past the segment end into buffers no consumer reads again, and the prefetch two
        // chunks ahead reads rows past the (batch, head) extent as zero through the buffer
        // range check.  Conditional loads would make the compiler merge register copies
        // that wait for the whole prefetch as soon as it is issued.
        load_p_qk<C>(raw, rs, t_begin, pw, lane);
        load_p_gates<C>(raw, rs, t_begin, pw, lane);
        ws_produce_a<C>(pv, raw, lp, smem, 0, pw, lane, LI, t_begin + lane < L, rs, t_begin + kTile, dv0, Dv);
        lds_barrier();  // block decays of chunk 0 published
        ws_produce_b<C>(pv, lp, smem, 0, pw, lane);
        lds_barrier();
        for (int kc = 0; kc < nch; ++kc) {
            // prepares chunk kc + 1 and reloads the registers with chunk kc + 2 group by group
            ws_produce_a<C>(pv, raw, lp, smem, (kc + 1) & 1, pw, lane, LI, t_begin + kTile * (kc + 1) + lane < L,
                            rs, t_begin + kTile * (kc + 2), dv0, Dv);
            lds_barrier();  // B1
            ws_produce_b<C>(pv, lp, smem, (kc + 1) & 1, pw, lane);
            lds_barrier();  // B2
        }
        return;
    }

    // ================================ consumers
    const int cw = w;
    const int col = dv0 + 16 * cw + c16;
    OpT *sP = reinterpret_cast<OpT *>(smem + lp.pbuf);

    f32x4 S[C::NBD];
#pragma unroll
    for (int n = 0; n < C::NBD; ++n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int d = 16 * n + 4 * g + e;
            float x = 0.f;
            if (seg > 0)
                x = a.ws_state[(((size_t)bh * (a.nseg - 1) * a.nsub + seg * a.nsub - 1) * C::DK + d) * Dv + col];
            else if (a.s0)
                x = a.s0[((size_t)bh * C::DK + d) * Dv + col];
            S[n][e] = x;
        }
    }
    // values: the consumers stage them (chunk k + 1 into buffer (k + 1) & 1 while working on
    // chunk k), one prefetched chunk in registers
    Raw<C> vraw;
    load_p_v<C>(vraw, rs, t_begin, cw, lane, dv0, Dv);
    v_to_lds<C>(vraw, reinterpret_cast<OpT *>(smem + lp.dbl + lp.vb), 64 * cw + lane);
    load_p_v<C>(vraw, rs, t_begin + kTile, cw, lane, dv0, Dv);
    lds_barrier();  // producers: block decays of chunk 0 published
    lds_barrier();  // chunk 0 prepared

    // this wave's score blocks: (query block i, key block j); pair 0 is the diagonal (cw, cw)
    int pi[3], pj[3];
    pi[0] = cw;
    pj[0] = cw;
    switch (cw) {
        case 0: pi[1] = 1; pj[1] = 0; pi[2] = 3; pj[2] = 2; break;
        case 1: pi[1] = 2; pj[1] = 0; pi[2] = 3; pj[2] = 1; break;
        case 2: pi[1] = 2; pj[1] = 1; pi[2] = 2; pj[2] = 1; break;
        default: pi[1] = 3; pj[1] = 0; pi[2] = 3; pj[2] = 0; break;
    }

    for (int kc = 0; kc < nch; ++kc) {
        const int b = kc & 1;
        const int T0 = t_begin + kTile * kc;
        const unsigned char *qkbase = lp.qkd ? smem + lp.dbl + b * lp.dstride : smem;
        const OpT *sQ = reinterpret_cast<const OpT *>(qkbase + lp.q);
        const OpT *sK = reinterpret_cast<const OpT *>(qkbase + lp.k);
        const OpT *sKT = reinterpret_cast<const OpT *>(smem + (lp.dbl + (b) * lp.dstride + lp.kst));
        const OpT *sV = reinterpret_cast<const OpT *>(smem + (lp.dbl + (b) * lp.dstride + lp.vb));
        const float *sAb = reinterpret_cast<const float *>(smem + (lp.dbl + (b) * lp.dstride + lp.ab));
        const float *sAi = reinterpret_cast<const float *>(smem + (lp.dbl + (b) * lp.dstride + lp.ainv));
        const float *sAt = reinterpret_cast<const float *>(smem + (lp.dbl + (b) * lp.dstride + lp.at));
        const OpT *sF = reinterpret_cast<const OpT *>(smem + (lp.dbl + (b) * lp.dstride + lp.fh));

        v_to_lds<C>(vraw, reinterpret_cast<OpT *>(smem + lp.dbl + (b ^ 1) * lp.dstride + lp.vb), 64 * cw + lane);
        // the dot-product source rows of this tile's stores, issued before the value prefetch so
        // that the stores' wait for them does not wait for it
        [[maybe_unused]] DotPre dp{};
        if constexpr (kDotPass<C>) {
            load_dot_pre(dp, om.dsrc, T0, L, Dv, dv0, cw, lane, om.rev);
            __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the prefetch
        }
        load_p_v<C>(vraw, rs, T0 + 2 * kTile, cw, lane, dv0, Dv);

        // ---------------- phase A: score blocks P^T(j, i) over the key channels and the
        // inter-chunk term, sharing the q fragments.  Per-channel gate: the queries of block i
        // are referenced to the block start, so block i multiplies diag(decay across blocks
        // 0..i-1) S, formed on the state fragment (the permuted q row holds, at 32m + 8g,
        // channels 32m + 4g + e and 32m + 16 + 4g + e: the state rows of this lane, and the
        // block decays are stored in the same order); key block j of a pair (i, j) with
        // j + 1 < i meets queries rescaled across the blocks between them, and the diagonal
        // pair uses keys referenced to the block start (block-end keys times 1/decay).
        // Scalar gate: raw q times S, each output row scaled by 2^(b_t) afterwards.  Each
        // wave's score pairs are spelled out per wave (wave-uniform switch).
        f32x4 Pd[3], O[4];
#pragma unroll
        for (int kp = 0; kp < 3; ++kp) Pd[kp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        // fp16 per-channel factors: one dword of each needed row per lane for the whole tile
        uint32_t fw[6] = {0u, 0u, 0u, 0u, 0u, 0u};
        if constexpr (C::CH && !C::F32) {
            const uint32_t *sFd = reinterpret_cast<const uint32_t *>(sF);
            const int fd = fac_dword(g, c16, C::SLAB / 2);
            constexpr int RW = C::SLAB / 2;  // dwords per factor row
            fw[0] = sFd[kFhA0 * RW + fd];
            fw[1] = sFd[kFhP2 * RW + fd];
            fw[2] = sFd[kFhP3 * RW + fd];
            fw[3] = sFd[(kFhInv + cw) * RW + fd];
            if (cw == 1) {
                fw[4] = sFd[kFhA1 * RW + fd];
                fw[5] = sFd[kFhA2 * RW + fd];
            } else if (cw == 3) {
                fw[4] = sFd[kFhA12 * RW + fd];
            }
        }
#pragma unroll
        for (int m = 0; m < C::KSTEP; ++m) {
            const int ch = 32 * m + 8 * g;
            Frag qf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) qf[i] = ld8<C>(sQ + (16 * i + c16) * C::RP + ch);
            float sv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sv[e] = S[2 * m][e];
                sv[e + 4] = S[2 * m + 1][e];
            }
            Frag sb;
#pragma unroll
            for (int e = 0; e < 8; ++e) sb[e] = (OpT)sv[e];
            O[0] = mma(qf[0], sb, O[0]);
            const auto kf = [&](int j) { return ld8<C>(sK + (16 * j + c16) * C::RP + ch); };
            if constexpr (C::CH && !C::F32) {
                // fp16 operands: the factors are fp16 too, applied with packed multiplies
                O[1] = mma(qf[1], sb * fac_frag(fw[0], m), O[1]);
                O[2] = mma(qf[2], sb * fac_frag(fw[1], m), O[2]);
                O[3] = mma(qf[3], sb * fac_frag(fw[2], m), O[3]);
                const Frag fi = fac_frag(fw[3], m);
                switch (cw) {
                    case 0: {
                        const Frag k0 = kf(0), k2 = kf(2);
                        Pd[0] = mma(k0 * fi, qf[0], Pd[0]);
                        Pd[1] = mma(k0, qf[1], Pd[1]);
                        Pd[2] = mma(k2, qf[3], Pd[2]);
                        break;
                    }
                    case 1: {
                        const Frag k1 = kf(1), k0 = kf(0);
                        Pd[0] = mma(k1 * fi, qf[1], Pd[0]);
                        Pd[1] = mma(k0, qf[2] * fac_frag(fw[4], m), Pd[1]);
                        Pd[2] = mma(k1, qf[3] * fac_frag(fw[5], m), Pd[2]);
                        break;
                    }
                    case 2: {
                        const Frag k2 = kf(2), k1 = kf(1);
                        Pd[0] = mma(k2 * fi, qf[2], Pd[0]);
                        Pd[1] = mma(k1, qf[2], Pd[1]);
                        break;
                    }
                    default: {
                        const Frag k3 = kf(3), k0 = kf(0);
                        Pd[0] = mma(k3 * fi, qf[3], Pd[0]);
                        Pd[1] = mma(k0, qf[3] * fac_frag(fw[4], m), Pd[1]);
                        break;
                    }
                }
            } else if constexpr (C::CH) {
                const f32x4 a0l = lds_ld<f32x4>(sAb + ch), a0h = lds_ld<f32x4>(sAb + ch + 4);
                const f32x4 a1l = lds_ld<f32x4>(sAb + C::SLAB + ch), a1h = lds_ld<f32x4>(sAb + C::SLAB + ch + 4);
                const f32x4 a2l = lds_ld<f32x4>(sAb + 2 * C::SLAB + ch), a2h = lds_ld<f32x4>(sAb + 2 * C::SLAB + ch + 4);
                {
                    f32x4 pl = a0l, ph = a0h;
                    O[1] = mma(qf[1], scale8f<C>(sv, pl, ph), O[1]);
                    pl *= a1l;
                    ph *= a1h;
                    O[2] = mma(qf[2], scale8f<C>(sv, pl, ph), O[2]);
                    pl *= a2l;
                    ph *= a2h;
                    O[3] = mma(qf[3], scale8f<C>(sv, pl, ph), O[3]);
                }
                const f32x4 il = lds_ld<f32x4>(sAi + cw * C::SLAB + ch), ih = lds_ld<f32x4>(sAi + cw * C::SLAB + ch + 4);
                switch (cw) {
                    case 0: {
                        const Frag k0 = kf(0), k2 = kf(2);
                        Pd[0] = mma(scale8<C>(k0, il, ih), qf[0], Pd[0]);
                        Pd[1] = mma(k0, qf[1], Pd[1]);
                        Pd[2] = mma(k2, qf[3], Pd[2]);
                        break;
                    }
                    case 1: {
                        const Frag k1 = kf(1), k0 = kf(0);
                        Pd[0] = mma(scale8<C>(k1, il, ih), qf[1], Pd[0]);
                        Pd[1] = mma(k0, scale8<C>(qf[2], a1l, a1h), Pd[1]);
                        Pd[2] = mma(k1, scale8<C>(qf[3], a2l, a2h), Pd[2]);
                        break;
                    }
                    case 2: {
                        const Frag k2 = kf(2), k1 = kf(1);
                        Pd[0] = mma(scale8<C>(k2, il, ih), qf[2], Pd[0]);
                        Pd[1] = mma(k1, qf[2], Pd[1]);
                        break;
                    }
                    default: {
                        const Frag k3 = kf(3), k0 = kf(0);
                        Pd[0] = mma(scale8<C>(k3, il, ih), qf[3], Pd[0]);
                        Pd[1] = mma(k0, scale8<C>(qf[3], a1l * a2l, a1h * a2h), Pd[1]);
                        break;
                    }
                }
            } else {
#pragma unroll
                for (int i = 1; i < 4; ++i) O[i] = mma(qf[i], sb, O[i]);
                switch (cw) {
                    case 0: {
                        const Frag k0 = kf(0), k2 = kf(2);
                        Pd[0] = mma(k0, qf[0], Pd[0]);
                        Pd[1] = mma(k0, qf[1], Pd[1]);
                        Pd[2] = mma(k2, qf[3], Pd[2]);
                        break;
                    }
                    case 1: {
                        const Frag k1 = kf(1), k0 = kf(0);
                        Pd[0] = mma(k1, qf[1], Pd[0]);
                        Pd[1] = mma(k0, qf[2], Pd[1]);
                        Pd[2] = mma(k1, qf[3], Pd[2]);
                        break;
                    }
                    case 2: {
                        const Frag k2 = kf(2), k1 = kf(1);
                        Pd[0] = mma(k2, qf[2], Pd[0]);
                        Pd[1] = mma(k1, qf[2], Pd[1]);
                        break;
                    }
                    default: {
                        const Frag k3 = kf(3), k0 = kf(0);
                        Pd[0] = mma(k3, qf[3], Pd[0]);
                        Pd[1] = mma(k0, qf[3], Pd[1]);
                        break;
                    }
                }
            }
        }
        if constexpr (C::CH) {
            // channels of strongly decayed blocks: exact partial scores from the producers
            const float *sXa = reinterpret_cast<const float *>(smem + (lp.dbl + (b) * lp.dstride + lp.xact));
            const int *sXf = reinterpret_cast<const int *>(smem + (lp.dbl + (b) * lp.dstride + lp.xflag));
            if (sXf[cw]) {
                const float *src = sXa + cw * 136;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s2 = 4 * g + e;
                    if (s2 <= c16) Pd[0][e] += src[c16 * (c16 + 1) / 2 + s2];
                }
            }
        }
        // mask, decay (scalar gates), store scores in MFMA A-operand order
#pragma unroll
        for (int kp = 0; kp < 3; ++kp) {
            if (kp == 2 && cw >= 2) continue;  // repeated pair
            const int i = pi[kp], j = pj[kp];
            Half pvv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s2 = 4 * g + e;
                const bool masked = i == j && s2 > c16;
                float x = masked ? 0.f : Pd[kp][e];
                if constexpr (!C::CH) {
                    if (!masked) x *= fexp2(sAb[16 * i + c16] - sAb[16 * j + s2] + sAi[16 * j + s2]);
                }
                pvv[e] = (OpT)x;
            }
            *reinterpret_cast<Half *>(sP + ((i * 2 + (j >> 1)) * 64 + lane) * 8 + 4 * (j & 1)) = pvv;
        }
        if (cw == 0 || cw == 2) {
            const Half z{(OpT)0.f, (OpT)0.f, (OpT)0.f, (OpT)0.f};
            *reinterpret_cast<Half *>(sP + ((cw * 2 + (cw >> 1)) * 64 + lane) * 8 + 4) = z;
        }
        if constexpr (!C::CH) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 bq = lds_ld<f32x4>(sAb + 16 * i + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) O[i][e] *= fexp2(bq[e]);
            }
        }
        lds_barrier();  // B1: scores stored; producers may rewrite q, k

        // ---------------- phase B: scores x values, state update, output
        Frag vfr[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) vfr[p] = ld8<C>(sV + ((p * 4 + g) * 64 + vsw(16 * cw + c16)) * 8);
        {
            Frag pa[6];
            pa[0] = ld8<C>(sP + ((0 * 2 + 0) * 64 + lane) * 8);
            pa[1] = ld8<C>(sP + ((1 * 2 + 0) * 64 + lane) * 8);
            pa[2] = ld8<C>(sP + ((2 * 2 + 0) * 64 + lane) * 8);
            pa[3] = ld8<C>(sP + ((3 * 2 + 0) * 64 + lane) * 8);
            pa[4] = ld8<C>(sP + ((2 * 2 + 1) * 64 + lane) * 8);
            pa[5] = ld8<C>(sP + ((3 * 2 + 1) * 64 + lane) * 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) O[i] = mma(pa[i], vfr[0], O[i]);
            O[2] = mma(pa[4], vfr[1], O[2]);
            O[3] = mma(pa[5], vfr[1], O[3]);
        }
        {
            f32x4 acc[C::NBD];
            // fp16 per-channel path: lane (g, c16) loads the tile decays of rows 16 n + 4 g + e,
            // n = c16 >> 1, e = 2 (c16 & 1) + {0, 1}; row broadcasts hand them to the row's lanes
            f32x2 atw{0.f, 0.f};
            if constexpr (C::CH && !C::F32)
                atw = lds_ld<f32x2>(sAt + 16 * ((c16 >> 1) & (C::NBD - 1)) + 4 * g + 2 * (c16 & 1));
#pragma unroll
            for (int n = 0; n < C::NBD; ++n) {
                f32x4 at;
                if constexpr (C::CH && !C::F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        at[e] = __uint_as_float(row_bcast(__float_as_uint(atw[e & 1]), 2 * n + (e >> 1)));
                } else if constexpr (C::CH) {
                    at = lds_ld<f32x4>(sAt + 16 * n + 4 * g);
                } else {
                    const float x = fexp2(sAb[63]);
                    at = f32x4{x, x, x, x};
                }
                acc[n] = S[n] * at;
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                Frag ka[C::NBD];
#pragma unroll
                for (int n = 0; n < C::NBD; ++n) ka[n] = ld8<C>(sKT + kt_off<C>(16 * n + c16, (p * 4 + g) * 8));
#pragma unroll
                for (int n = 0; n < C::NBD; ++n) acc[n] = mma(ka[n], vfr[p], acc[n]);
            }
#pragma unroll
            for (int n = 0; n < C::NBD; ++n) S[n] = acc[n];
        }
        stage_out(reinterpret_cast<float *>(smem + lp.ostage), O, cw, g, c16);
        lds_barrier();  // B2
        if constexpr (C::H16 != 0)
            store_staged_map<kDotPass<C>>(reinterpret_cast<const float *>(smem + lp.ostage), rs.out, om.li, T0, L, Dv,
                                          dv0, cw, lane, om.rev, om.has_li, om.inv, om.acc, dp, om.drow);
        else
            store_staged(reinterpret_cast<const float *>(smem + lp.ostage), rs.out, T0, Dv, dv0, cw, lane);
    }

    if (seg == a.nseg - 1 && a.fin) {
#pragma unroll
        for (int n = 0; n < C::NBD; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.fin[((size_t)bh * C::DK + 16 * n + 4 * g + e) * Dv + col] = S[n][e];
    }
}

// ------------------------------------------------------------------------------------
// Warp-specialised chunk output for scalar gates (none, per head and token, fixed per
// head) with bf16 inputs, 64-token chunks and Dk = 256.  grid = BH * nseg * ndv
// workgroups of 512 threads.
//
// Producers (waves 4..7): wave pw owns the 16 rows of block pw and lane l the channels
// 4l .. 4l+3, so every load covers a whole row and a lane owns consecutive tokens of its
// channels for the transposed keys.  Consumers (waves 0..3): 16 value columns each, the
// Dk x 16 state in registers.  Per tile k:
//   phase A  consumers: score blocks (q, and the keys read transposed from k^T), O =
//            diag(2^b) (q . S), state update S <- 2^T S + k^T (diag(w) v) with the key
//            weights w = 2^(T - b + l) on the value operand (q, values and rows: buffer
//            k&1; k^T: single buffer)
//            producers: decay scan, values, rows and fp16 q of tile k+1 into buffer
//            (k+1)&1, fp16 keys of tile k+1 into registers; loads of tile k+2
//   B1
//   phase B  consumers: masked scores x values, output stores
//            producers: k^T of tile k+1 into the single buffer
//   B2
// With a scalar gate the queries need no scaling to the tile start: the inter-chunk
// product takes raw q and its output rows are scaled by 2^(b_t) in fp32.
// q rows hold their channels in the chperm order; k^T rows (one per channel) hold their
// tokens in k-slot order, with the 16-byte units of a row XOR-swizzled by bits 2-4 of the
// row and a row pitch of 96 halves: the state update's 16-byte reads (16 consecutive rows,
// one unit each) and the transposed 8-byte reads of the score products (4 consecutive rows
// times 4 consecutive units) then both fall on distinct LDS banks.  The value tile uses the
// vsw swizzle.

__device__ __forceinline__ int kt_off_sg(int r, int s) { return r * 96 + ((((s >> 3) ^ (r >> 2)) & 7) << 3) + (s & 7); }

template <class C>
struct RawSg {
    u32x2 q[16], k[16];  // 4 bf16 channels (4 * lane ..) of rows 16 pw + rr
    uint32_t v[4][2];    // 4 values of one row
    float las, lis;      // log gate and log input gate of row (tile start + lane)
};

template <class C>
__device__ __forceinline__ void load_unit_sg(RawSg<C> &r, const Rs &rs, int T0, int pw, int lane, int dv0, int Dv) {
    const int ch0 = 4 * lane;  // a wave's load covers one whole row
    uint32_t qks = C::DK;
    if constexpr (C::H16 != 0) qks = rs.qks;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        const uint32_t off = (in_row<C>(rs, T0 + 16 * pw + rr) * qks + ch0) * 2u;
        r.q[rr] = bld64(rs.q, off);
        r.k[rr] = bld64(rs.k, off);
    }
    // One branch-free load for every scalar gate kind: per token (stride 4), fixed per head
    // (stride 0, masked past the sequence end where it is used), none (empty resource).
    const uint32_t t = (uint32_t)(T0 + lane);
    r.las = __uint_as_float(bld32(rs.la, t * rs.gstride));
    r.lis = __uint_as_float(bld32(rs.li, t * 4u));
    const int tp = 64 * pw + lane;
    const uint32_t c0 = dv0 + 4 * (tp & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t off = (in_row<C>(rs, T0 + 4 * (tp >> 4) + e) * Dv + c0) * 2u;
        const u32x2 x = bld64(rs.v, off);
        r.v[e][0] = x[0];
        r.v[e][1] = x[1];
    }
}

template <class C>
struct ProdSg {
    f16x4 kt[4][4];  // [channel][token group]: fp16 keys of 4 consecutive tokens
};

// Phase A: values, row data and q rows into buffer nb, the keys of the tile into registers.
template <class C>
__device__ __forceinline__ void sg_produce_a(ProdSg<C> &pv, const RawSg<C> &raw, const LdsPlanSg &lp,
                                             unsigned char *smem, int nb, int pw, int lane, bool row_valid) {
    // values in MFMA B-operand order (as v_to_lds)
    {
        f16 *sV = reinterpret_cast<f16 *>(smem + lp.vb) + nb * 4096;
        const int tid = 64 * pw + lane;
        const int quad = tid >> 4;
        const int p = quad >> 3, hh = (quad >> 2) & 1, gq = quad & 3;
        const int c0 = 4 * (tid & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f16x4 h4;
#pragma unroll
            for (int e = 0; e < 4; ++e) h4[e] = (f16)((j & 1) ? in_hi<C, kOpV>(raw.v[e][j >> 1]) : in_lo<C, kOpV>(raw.v[e][j >> 1]));
            *reinterpret_cast<f16x4 *>(sV + ((p * 4 + gq) * 64 + vsw(c0 + j)) * 8 + hh * 4) = h4;
        }
    }
    // running log2 decay over the tile's rows (lane = row) and the key weights
    const float x = row_valid ? log2_decay(raw.las) : 0.f;
    const float y = raw.lis * kLog2e;
    const float bl = scan_incl(x, lane);
    if (pw == 0) {
        const float T = lane_bcast(bl, 63);
        float *sR = reinterpret_cast<float *>(smem + lp.rows) + nb * 192;
        sR[lane] = bl;
        sR[64 + lane] = y;
        sR[128 + lane] = fexp2(T - bl + y);  // weight of key row `lane` in the state update
    }
    f16 *sQ = reinterpret_cast<f16 *>(smem + lp.q) + nb * 64 * (C::DK + 8);
    const int pc = chperm(4 * lane);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
        float qf[4], kf[4];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            qf[2 * c] = in_lo<C, kOpQ>(raw.q[rr][c]);
            qf[2 * c + 1] = in_hi<C, kOpQ>(raw.q[rr][c]);
            kf[2 * c] = in_lo<C, kOpK>(raw.k[rr][c]);
            kf[2 * c + 1] = in_hi<C, kOpK>(raw.k[rr][c]);
        }
        *reinterpret_cast<u32x2 *>(sQ + (16 * pw + rr) * (C::DK + 8) + pc) =
            u32x2{__builtin_bit_cast(uint32_t, f16x2{(f16)qf[0], (f16)qf[1]}),
                  __builtin_bit_cast(uint32_t, f16x2{(f16)qf[2], (f16)qf[3]})};
#pragma unroll
        for (int c = 0; c < 4; ++c) pv.kt[c][rr >> 2][rr & 3] = (f16)kf[c];
    }
}

// Phase B: the keys^T of the prepared tile into the single buffer.
template <class C>
__device__ __forceinline__ void sg_produce_b(const ProdSg<C> &pv, const LdsPlanSg &lp, unsigned char *smem, int pw,
                                             int lane) {
    const int ch0 = 4 * lane;
    f16 *sKT = reinterpret_cast<f16 *>(smem + lp.kst);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<f16x4 *>(sKT + kt_off_sg(ch0 + c, kslot(16 * pw + 4 * g4))) = pv.kt[c][g4];
}

template <class C>
__global__ __launch_bounds__(512, 1) void chunk_output_sg_kernel(KArgs a) {
    static_assert(!C::F32 && !C::CH && !C::MT && C::DK == 256, "bf16, scalar gate, 64-token tiles, Dk = 256");
    constexpr int DK = C::DK;
    constexpr int RP = DK + 8;
    constexpr int KSTEP = DK / 32;
    constexpr int NBD = DK / 16;
    extern __shared__ __align__(256) unsigned char smem[];
    const LdsPlanSg lp = lds_plan_sg(DK);

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
    const int t_begin = seg * a.seg_len;
    const int t_end = min(L, t_begin + a.seg_len);
    const int nch = (t_end - t_begin + kTile - 1) / kTile;
    const Rs rs = make_rs<C>(a, bh, h);
    [[maybe_unused]] const OutMap om = C::H16 != 0 ? make_out_map(a, bh, dvt) : OutMap{};

    if (w >= 4) {
        // ============================ producers
        // Unconditional loop body, as in the per-channel kernel: the last iteration prepares
        // a tile past the segment into buffers no consumer reads again, and the prefetch two
        // tiles ahead reads rows past the (batch, head) extent as zero.
        // Two register sets for the raw tiles, alternating over an unrolled pair of
        // iterations, so the prefetch never has to be copied into the other set (a copy
        // waits for the load).  Each iteration has two barriers, as the consumers'; the
        // uniform breaks end the loop after exactly nch iterations.
        const int pw = w - 4;
        RawSg<C> ra, rb;
        ProdSg<C> pv;
        load_unit_sg<C>(ra, rs, t_begin, pw, lane, dv0, Dv);
        sg_produce_a<C>(pv, ra, lp, smem, 0, pw, lane, t_begin + lane < L);
        load_unit_sg<C>(rb, rs, t_begin + kTile, pw, lane, dv0, Dv);
        sg_produce_b<C>(pv, lp, smem, pw, lane);
        lds_barrier();
        for (int kc = 0;; kc += 2) {
            sg_produce_a<C>(pv, rb, lp, smem, (kc + 1) & 1, pw, lane, t_begin + kTile * (kc + 1) + lane < L);
            load_unit_sg<C>(ra, rs, t_begin + kTile * (kc + 2), pw, lane, dv0, Dv);
            lds_barrier();  // B1
            sg_produce_b<C>(pv, lp, smem, pw, lane);
            lds_barrier();  // B2
            if (kc + 1 >= nch) break;
            sg_produce_a<C>(pv, ra, lp, smem, (kc + 2) & 1, pw, lane, t_begin + kTile * (kc + 2) + lane < L);
            load_unit_sg<C>(rb, rs, t_begin + kTile * (kc + 3), pw, lane, dv0, Dv);
            lds_barrier();  // B1
            sg_produce_b<C>(pv, lp, smem, pw, lane);
            lds_barrier();  // B2
            if (kc + 2 >= nch) break;
        }
        return;
    }

    // ================================ consumers
    const int cw = w;
    const int col = dv0 + 16 * cw + c16;
    const f16 *sKT = reinterpret_cast<const f16 *>(smem + lp.kst);
    f16 *sP = reinterpret_cast<f16 *>(smem + lp.pbuf);

    f32x4 S[NBD];
#pragma unroll
    for (int n = 0; n < NBD; ++n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int d = 16 * n + 4 * g + e;
            float x = 0.f;
            if (seg > 0)
                x = a.ws_state[(((size_t)bh * (a.nseg - 1) * a.nsub + seg * a.nsub - 1) * DK + d) * Dv + col];
            else if (a.s0)
                x = a.s0[((size_t)bh * DK + d) * Dv + col];
            S[n][e] = x;
        }
    }
    lds_barrier();  // tile 0 prepared

    // this wave's score blocks (query block i, key block j); pair 0 is the diagonal
    int pi[3], pj[3];
    pi[0] = cw;
    pj[0] = cw;
    switch (cw) {
        case 0: pi[1] = 1; pj[1] = 0; pi[2] = 3; pj[2] = 2; break;
        case 1: pi[1] = 2; pj[1] = 0; pi[2] = 3; pj[2] = 1; break;
        case 2: pi[1] = 2; pj[1] = 1; pi[2] = 2; pj[2] = 1; break;
        default: pi[1] = 3; pj[1] = 0; pi[2] = 3; pj[2] = 0; break;
    }

    for (int kc = 0; kc < nch; ++kc) {
        const int b = kc & 1;
        const int T0 = t_begin + kTile * kc;
        const f16 *sQ = reinterpret_cast<const f16 *>(smem + lp.q) + b * 64 * RP;
        const f16 *sV = reinterpret_cast<const f16 *>(smem + lp.vb) + b * 4096;
        const float *sB = reinterpret_cast<const float *>(smem + lp.rows) + b * 192;
        const float *sL = sB + 64;
        const float *sW = sB + 128;

        // ---------------- phase A: score blocks P^T(j, i) and the inter-chunk term
        // O = diag(2^b) (q . S), sharing the q fragments: the permuted q row holds, at
        // 32m + 8g, channels 32m + 4g + e and 32m + 16 + 4g + e, the rows of state blocks 2m
        // and 2m+1.  Each wave's score pairs are spelled out per wave (wave-uniform switch).
        f32x4 Pd[3], O[4];
#pragma unroll
        for (int kp = 0; kp < 3; ++kp) Pd[kp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < KSTEP; ++m) {
            const int ch = 32 * m + 8 * g;
            f16x8 qf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) qf[i] = lds_ld<f16x8>(sQ + (16 * i + c16) * RP + ch);
            f16x8 sb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sb[e] = (f16)S[2 * m][e];
                sb[e + 4] = (f16)S[2 * m + 1][e];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) O[i] = mma(qf[i], sb, O[i]);
            // key rows 16j + c16 over the channels of this step, read transposed from k^T:
            // source lane 4e + qq of a 16-lane group supplies tokens 16j + 4qq .. +3 of channel
            // 32m + 4g + e (and 32m + 16 + 4g + e), the slot order of the permuted q rows
            const int s_tr = kslot(4 * (c16 & 3)), r_tr = 32 * m + 4 * g + (c16 >> 2);
            const auto kf = [&](int j) {
                const f16x4 lo = lds_tr16(sKT + kt_off_sg(r_tr, s_tr + kslot(16 * j)));
                const f16x4 hi = lds_tr16(sKT + kt_off_sg(r_tr + 16, s_tr + kslot(16 * j)));
                return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            };
            switch (cw) {
                case 0: {
                    const f16x8 k0 = kf(0), k2 = kf(2);
                    Pd[0] = mma(k0, qf[0], Pd[0]);
                    Pd[1] = mma(k0, qf[1], Pd[1]);
                    Pd[2] = mma(k2, qf[3], Pd[2]);
                    break;
                }
                case 1: {
                    const f16x8 k1 = kf(1), k0 = kf(0);
                    Pd[0] = mma(k1, qf[1], Pd[0]);
                    Pd[1] = mma(k0, qf[2], Pd[1]);
                    Pd[2] = mma(k1, qf[3], Pd[2]);
                    break;
                }
                case 2: {
                    const f16x8 k2 = kf(2), k1 = kf(1);
                    Pd[0] = mma(k2, qf[2], Pd[0]);
                    Pd[1] = mma(k1, qf[2], Pd[1]);
                    break;
                }
                default: {
                    const f16x8 k3 = kf(3), k0 = kf(0);
                    Pd[0] = mma(k3, qf[3], Pd[0]);
                    Pd[1] = mma(k0, qf[3], Pd[1]);
                    break;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 bq = lds_ld<f32x4>(sB + 16 * i + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) O[i][e] *= fexp2(bq[e]);
        }
        // mask and exact decay of the scores, stored in MFMA A-operand order
#pragma unroll
        for (int kp = 0; kp < 3; ++kp) {
            if (kp == 2 && cw >= 2) continue;  // repeated pair
            const int i = pi[kp], j = pj[kp];
            const float bt = sB[16 * i + c16];
            f16x4 pvv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s2 = 4 * g + e;
                const bool masked = i == j && s2 > c16;
                const float x = Pd[kp][e] * fexp2(bt - sB[16 * j + s2] + sL[16 * j + s2]);
                pvv[e] = (f16)(masked ? 0.f : x);
            }
            *reinterpret_cast<f16x4 *>(sP + ((i * 2 + (j >> 1)) * 64 + lane) * 8 + 4 * (j & 1)) = pvv;
        }
        if (cw == 0 || cw == 2) {
            const f16x4 z{(f16)0.f, (f16)0.f, (f16)0.f, (f16)0.f};
            *reinterpret_cast<f16x4 *>(sP + ((cw * 2 + (cw >> 1)) * 64 + lane) * 8 + 4) = z;
        }
        // state update S <- 2^T S + K^T diag(w) V, the key weights on the value operand: slot
        // 8g + e of step p is token 32p + 4g + e, slot 8g + 4 + e token 32p + 16 + 4g + e
        f16x8 vfr[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) vfr[p] = lds_ld<f16x8>(sV + ((p * 4 + g) * 64 + vsw(16 * cw + c16)) * 8);
        {
            const float at = fexp2(sB[63]);
#pragma unroll
            for (int n = 0; n < NBD; ++n) S[n] *= at;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const f32x4 w0 = lds_ld<f32x4>(sW + 32 * p + 4 * g), w1 = lds_ld<f32x4>(sW + 32 * p + 16 + 4 * g);
                f16x8 vw;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vw[e] = (f16)((float)vfr[p][e] * w0[e]);
                    vw[e + 4] = (f16)((float)vfr[p][e + 4] * w1[e]);
                }
#pragma unroll
                for (int n = 0; n < NBD; ++n) {
                    const int r = 16 * n + c16;
                    S[n] = mma(lds_ld<f16x8>(sKT + kt_off_sg(r, (p * 4 + g) * 8)), vw, S[n]);
                }
            }
        }
        lds_barrier();  // B1: scores stored; k^T free for the next tile
        // the mapped output stage's loads for this tile, a phase ahead of the stores (the
        // consumers issue no other global loads, so waiting for them waits for nothing else)
        [[maybe_unused]] MapPre mp;
        if constexpr (C::H16 != 0) load_map_pre(mp, rs.out, om.li, T0, L, Dv, dv0, cw, lane, om.rev, om.has_li, om.acc);
        [[maybe_unused]] DotPre dp{};
        if constexpr (kDotPass<C>) load_dot_pre(dp, om.dsrc, T0, L, Dv, dv0, cw, lane, om.rev);

        // ---------------- phase B: scores x values, output
        {
            f16x8 pa[6];
            pa[0] = lds_ld<f16x8>(sP + ((0 * 2 + 0) * 64 + lane) * 8);
            pa[1] = lds_ld<f16x8>(sP + ((1 * 2 + 0) * 64 + lane) * 8);
            pa[2] = lds_ld<f16x8>(sP + ((2 * 2 + 0) * 64 + lane) * 8);
            pa[3] = lds_ld<f16x8>(sP + ((3 * 2 + 0) * 64 + lane) * 8);
            pa[4] = lds_ld<f16x8>(sP + ((2 * 2 + 1) * 64 + lane) * 8);
            pa[5] = lds_ld<f16x8>(sP + ((3 * 2 + 1) * 64 + lane) * 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) O[i] = mma(pa[i], vfr[0], O[i]);
            O[2] = mma(pa[4], vfr[1], O[2]);
            O[3] = mma(pa[5], vfr[1], O[3]);
        }
        stage_out(reinterpret_cast<float *>(smem + lp.ostage), O, cw, g, c16);
        lds_barrier();  // B2
        if constexpr (C::H16 != 0)
            store_staged_map<kDotPass<C>>(reinterpret_cast<const float *>(smem + lp.ostage), rs.out, mp, T0, L, Dv,
                                          dv0, cw, lane, om.rev, om.has_li, om.inv, om.acc, dp, om.drow);
        else
            store_staged(reinterpret_cast<const float *>(smem + lp.ostage), rs.out, T0, Dv, dv0, cw, lane);
    }

    if (seg == a.nseg - 1 && a.fin) {
#pragma unroll
        for (int n = 0; n < NBD; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.fin[((size_t)bh * DK + 16 * n + 4 * g + e) * Dv + col] = S[n][e];
    }
}

// ------------------------------------------------------------------------------------
// segment_state_kernel: grid = BH * (nseg - 1) * nsub * ndv.  The state sub-segment j (a
// run of whole tiles; the nsub runs of a segment differ by at most one tile) produces from zero, sum_s diag(decay from s to the sub-segment end)
// i_s k_s^T v_s, accumulated tile by tile (dS <- diag(tile decay) dS + K~^T V), and the decay
// across the sub-segment.
template <class C>
__global__ __launch_bounds__(256, 3) void segment_state_kernel(KArgs a) {
    using OpT = typename C::OpT;
    using Frag = typename C::Frag;
    using Half = typename C::Half;
    extern __shared__ __align__(256) unsigned char smem[];
    const LdsPlanState lp = lds_plan_state(C::OPB, C::DK);
    OpT *sKT = reinterpret_cast<OpT *>(smem + lp.kst);
    OpT *sV = reinterpret_cast<OpT *>(smem + lp.vb);
    float *sAb = reinterpret_cast<float *>(smem + lp.ablk);
    float *sAt = reinterpret_cast<float *>(smem + lp.atile);
    float *sAs = reinterpret_cast<float *>(smem + lp.aseg);

    const int nsm = (a.nseg - 1) * a.nsub;
    int id = xcd_remap((int)blockIdx.x, a.nwg);
    const int dvt = id % a.ndv;
    id /= a.ndv;
    const int seg = id % nsm;  // sub-segment
    const int bh = id / nsm;
    const int h = bh % a.H;
    const int tid = (int)threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = a.L, Dv = a.Dv;
    const int dv0 = dvt * kDvTile;
    const int col = dv0 + 16 * w + c16;
    // sub-segment jj of segment sg: tiles [tiles * jj / nsub, tiles * (jj + 1) / nsub) of it
    const int tiles = a.seg_len / kTile;
    const int sg = seg / a.nsub, jj = seg % a.nsub;
    const int t_begin = sg * a.seg_len + kTile * ((tiles * jj) / a.nsub);
    const int t_end = min(L, sg * a.seg_len + kTile * ((tiles * (jj + 1)) / a.nsub));
    const int chl = C::CPL * lane;
    const Rs rs = make_rs<C>(a, bh, h);

    if constexpr (C::CH) {
        for (int d = tid; d < C::DK; d += kThreads) sAs[d] = 1.f;
    }
    float Bs = 0.f;  // scalar gates: log2 decay across the segment so far
    f32x4 dS[C::NBD];
#pragma unroll
    for (int n = 0; n < C::NBD; ++n) dS[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    Raw<C> raw;
    load_unit<C, false>(raw, rs, t_begin, 0, w, lane, tid, dv0, Dv);
    for (int T0 = t_begin; T0 < t_end; T0 += kTile) {
        float Tt = 0.f;
        Frag vfr[2];
#pragma unroll 1
        for (int sl = 0; sl < C::NSLAB; ++sl) {
            if (sl == 0) v_to_lds<C>(raw, sV, tid);
            if constexpr (C::CH) {
                ChGate<C> G;
                ch_gate<C>(G, raw, sAb, w, lane);
                float ig[16];
                if (rs.has_li) {
                    const float y = raw.lis * kLog2e;
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) ig[rr] = fexp2(lane_bcast(y, 16 * w + rr));
                } else {
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) ig[rr] = 1.f;
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
                    Half kt4[C::CPL];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int rr = 4 * g4 + e;
#pragma unroll
                        for (int c = 0; c < C::CPL; ++c)
                            kt4[c][e] = (OpT)(raw.kf(rr, c) * ig[rr] * G.ek[rr][c] * G.post[c]);
                    }
#pragma unroll
                    for (int c = 0; c < C::CPL; ++c)
                        *reinterpret_cast<Half *>(sKT + kt_off<C>(chl + c, kslot(16 * w + 4 * g4))) = kt4[c];
                }
            } else {
                const float x = log2_decay(raw.las);
                const float y = raw.lis * kLog2e;
                const float bl = scan_incl(x, lane);
                Tt = lane_bcast(bl, 63);
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    Half kt4[C::CPL];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int rr = 4 * g4 + e;
                        const float f = fexp2(Tt - lane_bcast(bl, 16 * w + rr) + lane_bcast(y, 16 * w + rr));
#pragma unroll
                        for (int c = 0; c < C::CPL; ++c) kt4[c][e] = (OpT)(raw.kf(rr, c) * f);
                    }
#pragma unroll
                    for (int c = 0; c < C::CPL; ++c)
                        *reinterpret_cast<Half *>(sKT + kt_off<C>(chl + c, kslot(16 * w + 4 * g4))) = kt4[c];
                }
            }
            lds_barrier();
            {
                // unconditional prefetch, as in the chunk-output kernel
                int Tn = T0 + kTile, sn = 0;
                if (sl + 1 < C::NSLAB) {
                    Tn = T0;
                    sn = sl + 1;
                }
                load_unit<C, false>(raw, rs, Tn, sn, w, lane, tid, dv0, Dv);
            }
            if (sl == 0) {
#pragma unroll
                for (int p = 0; p < 2; ++p) vfr[p] = ld8<C>(sV + ((p * 4 + g) * 64 + vsw(16 * w + c16)) * 8);
            }
            f32x4 acc[C::NBS];
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
                acc[n] = dS[nn] * at;
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                Frag ka[C::NBS];
#pragma unroll
                for (int n = 0; n < C::NBS; ++n) ka[n] = ld8<C>(sKT + kt_off<C>(16 * n + c16, (p * 4 + g) * 8));
#pragma unroll
                for (int n = 0; n < C::NBS; ++n) acc[n] = mma(ka[n], vfr[p], acc[n]);
            }
#pragma unroll
            for (int n = 0; n < C::NBS; ++n) dS[sl * C::NBS + n] = acc[n];
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
// segment_scan_kernel: grid (ceil(Dk*Dv/1024), BH).  Carries the state over the
// sub-segments, S <- diag(decay_j) S + local_j from the initial state (or 0), and writes the
// state entering segment s (after sub-segment s*nsub - 1) over that sub-segment's entry.
__global__ __launch_bounds__(256) void segment_scan_kernel(KArgs a, int dk) {
    const int bh = (int)blockIdx.y;
    const size_t n = (size_t)dk * a.Dv;
    const size_t idx = ((size_t)blockIdx.x * kThreads + threadIdx.x) * 4;
    if (idx >= n) return;
    const int d = (int)(idx / a.Dv);
    const int nsm = (a.nseg - 1) * a.nsub;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.s0) s = *reinterpret_cast<const float4 *>(a.s0 + (size_t)bh * n + idx);
    float *ws = a.ws_state + (size_t)bh * nsm * n + idx;
    const float *wd = a.ws_decay + (size_t)bh * nsm * dk + d;
    // batches of 8 sub-segments: all loads of a batch are issued before its stores
    for (int j0 = 0; j0 < nsm; j0 += 8) {
        float4 x[8];
        float dec[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = min(j0 + u, nsm - 1);
            x[u] = *reinterpret_cast<const float4 *>(ws + (size_t)j * n);
            dec[u] = wd[(size_t)j * dk];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u;
            if (j < nsm) {
                s.x = s.x * dec[u] + x[u].x;
                s.y = s.y * dec[u] + x[u].y;
                s.z = s.z * dec[u] + x[u].z;
                s.w = s.w * dec[u] + x[u].w;
                if ((j + 1) % a.nsub == 0) *reinterpret_cast<float4 *>(ws + (size_t)j * n) = s;
            }
        }
    }
}

// ------------------------------------------------------------------------------------
// Launchers.

// Raise a kernel's dynamic-LDS limit to the whole 160 KB once per device (the attribute
// belongs to the function on the current device); `done` holds one bit per device ordinal.
static hipError_t ensure_lds_limit(const void *fn, std::atomic<uint64_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

template <class C>
static hipError_t launch_cfg(const KArgs &a, hipStream_t st) {
    hipError_t err;
    // a row stride for q and k is read by the backward instances of the scalar-gate Dk = 256
    // kernel only
    if (a.qk_stride != 0 && !(C::H16 != 0 && !C::F32 && !C::CH && !C::MT && C::DK == 256))
        return hipErrorInvalidValue;
    // entry states given (state_t): only the chunk-output kernel runs
    if (a.nseg > 1 && !a.state_t) {
        const LdsPlanState l1 = lds_plan_state(C::OPB, C::DK);
        static std::atomic<uint64_t> done_state{0};
        err = ensure_lds_limit(reinterpret_cast<const void *>(&segment_state_kernel<C>), done_state);
        if (err != hipSuccess) return err;
        KArgs a1 = a;
        a1.nwg = (a.B * a.H) * (a.nseg - 1) * a.nsub * a.ndv;
        hipLaunchKernelGGL(segment_state_kernel<C>, dim3(a1.nwg), dim3(kThreads), l1.total, st, a1);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        const int nx = (C::DK * a.Dv + 1023) / 1024;
        hipLaunchKernelGGL(segment_scan_kernel, dim3(nx, a.B * a.H), dim3(kThreads), 0, st, a, C::DK);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    KArgs a3 = a;
    a3.nwg = (a.B * a.H) * a.nseg * a.ndv * (a.qsplit > 1 ? a.qsplit : 1);
    if constexpr (!C::F32 && !C::CH && !C::MT && C::DK == 256) {
        const LdsPlanSg lg = lds_plan_sg(C::DK);
        static std::atomic<uint64_t> done_sg{0};
        err = ensure_lds_limit(reinterpret_cast<const void *>(&chunk_output_sg_kernel<C>), done_sg);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(chunk_output_sg_kernel<C>, dim3(a3.nwg), dim3(2 * kThreads), lg.total, st, a3);
        return hipGetLastError();
    } else if constexpr (!C::MT && C::NSLAB == 1) {
        const LdsPlanWs lw = lds_plan_ws(C::OPB, C::DK);
        // the input gate is a compile-time choice: without it the producers carry no gate factor
        static std::atomic<uint64_t> done_ws[2] = {{0}, {0}};
        const void *fn = a.li ? reinterpret_cast<const void *>(&chunk_output_ws_kernel<C, true>)
                              : reinterpret_cast<const void *>(&chunk_output_ws_kernel<C, false>);
        err = ensure_lds_limit(fn, done_ws[a.li ? 1 : 0]);
        if (err != hipSuccess) return err;
        if (a.li)
            hipLaunchKernelGGL((chunk_output_ws_kernel<C, true>), dim3(a3.nwg), dim3(2 * kThreads), lw.total, st, a3);
        else
            hipLaunchKernelGGL((chunk_output_ws_kernel<C, false>), dim3(a3.nwg), dim3(2 * kThreads), lw.total, st, a3);
        return hipGetLastError();
    } else {
        const LdsPlan l3 = lds_plan(C::OPB, C::DK, C::CH, a.nt);
        static std::atomic<uint64_t> done_out{0};
        err = ensure_lds_limit(reinterpret_cast<const void *>(&chunk_output_kernel<C>), done_out);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(chunk_output_kernel<C>, dim3(a3.nwg), dim3(kThreads), l3.total, st, a3);
        return hipGetLastError();
    }
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

// ------------------------------------------------------------------------------------
// step_kernel: one token of the recurrence.  grid = BH * (Dv / 64) workgroups of 256
// threads; a workgroup owns one (batch, head) and 64 value columns.  Thread t updates
// columns 4(t & 15) .. +3 of the state rows d = (t >> 4) + 16 j (float4 loads and stores,
// 256 contiguous bytes per row), accumulates its part of o = q S_new, and the 16 row groups
// are summed through LDS.
template <bool F32>
__global__ __launch_bounds__(256) void step_kernel(gla_step_desc d) {
    __shared__ float sq[4096], sk[4096], sa[4096];
    __shared__ float4 part[16][16];
    const int ndv = (d.Dv + 63) / 64;  // the last tile of a Dv that is not a multiple of 64 is partial
    const int bh = (int)blockIdx.x / ndv, dvt = (int)blockIdx.x % ndv;
    const int h = bh % d.H;
    const int tid = (int)threadIdx.x;
    const int Dk = d.Dk, Dv = d.Dv;
    const auto in = [&](const void *p, size_t i) -> float {
        if constexpr (F32) return reinterpret_cast<const float *>(p)[i];
        else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p)[i] << 16);
    };
    float ig = 1.f;
    if (d.log_ig) ig = fexp2(d.log_ig[bh] * kLog2e);
    float ascalar = 1.f;
    if (d.gate_kind == GLA_GATE_HEAD) ascalar = fexp2(d.log_alpha[bh] * kLog2e);
    else if (d.gate_kind == GLA_GATE_HEAD_CONST) ascalar = fexp2(d.log_alpha[h] * kLog2e);
    for (int r = tid; r < Dk; r += 256) {
        sq[r] = in(d.q, (size_t)bh * Dk + r);
        sk[r] = in(d.k, (size_t)bh * Dk + r) * ig;
        sa[r] = d.gate_kind == GLA_GATE_CHANNEL ? fexp2(d.log_alpha[(size_t)bh * Dk + r] * kLog2e) : ascalar;
    }
    __syncthreads();
    const int cq = tid & 15, rg = tid >> 4;
    const int c0 = dvt * 64 + 4 * cq;
    const bool cval = c0 < Dv;  // Dv is a multiple of 4: a column quad is in range or past it
    float vv[4] = {0.f, 0.f, 0.f, 0.f};
    if (cval) {
#pragma unroll
        for (int j = 0; j < 4; ++j) vv[j] = in(d.v, (size_t)bh * Dv + c0 + j);
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float *S = d.state + (size_t)bh * Dk * Dv + c0;
    for (int r = rg; cval && r < Dk; r += 16) {
        float4 *p = reinterpret_cast<float4 *>(S + (size_t)r * Dv);
        float4 x = *p;
        const float a = sa[r], kr = sk[r], qr = sq[r];
        x.x = a * x.x + kr * vv[0];
        x.y = a * x.y + kr * vv[1];
        x.z = a * x.z + kr * vv[2];
        x.w = a * x.w + kr * vv[3];
        *p = x;
        acc.x += qr * x.x;
        acc.y += qr * x.y;
        acc.z += qr * x.z;
        acc.w += qr * x.w;
    }
    part[rg][cq] = acc;
    __syncthreads();
    if (tid < 16 && dvt * 64 + 4 * tid < Dv) {
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int g = 0; g < 16; ++g) {
            const float4 y = part[g][tid];
            o.x += y.x;
            o.y += y.y;
            o.z += y.z;
            o.w += y.w;
        }
        *reinterpret_cast<float4 *>(d.out + (size_t)bh * Dv + dvt * 64 + 4 * tid) = o;
    }
}

hipError_t launch_step(const gla_step_desc &d, hipStream_t st) {
    const int grid = d.B * d.H * ((d.Dv + 63) / 64);
    if (d.in_dtype == GLA_DTYPE_F32)
        hipLaunchKernelGGL(step_kernel<true>, dim3(grid), dim3(256), 0, st, d);
    else
        hipLaunchKernelGGL(step_kernel<false>, dim3(grid), dim3(256), 0, st, d);
    return hipGetLastError();
}

template <int M>
static hipError_t launch_h16(const KArgs &a, int dk, hipStream_t st) {
    if (dk == 64) return launch_cfg<Cfg<false, 64, false, false, M>>(a, st);
    if (dk == 128) return launch_cfg<Cfg<false, 128, false, false, M>>(a, st);
    return launch_cfg<Cfg<false, 256, false, false, M>>(a, st);
}

// h16: which of q, k, v (bits kOpQ, kOpK, kOpV) are fp16 rather than bf16.  Only one fp16
// operand and 64-token chunks: the forms the backward pass runs (with a per-channel gate only
// the value operand, Dk <= 128).
hipError_t launch_forward(const KArgs &a, bool f32, int h16, int dk, hipStream_t st) {
    const bool ch = a.gate == GLA_GATE_CHANNEL;
    const bool mt = a.nt > 1;
    if (h16 && ch) {
        if (mt || f32 || h16 != 1 << kOpV) return hipErrorInvalidValue;
        if (dk == 64) return launch_cfg<Cfg<false, 64, true, false, 1 << kOpV>>(a, st);
        if (dk == 128) return launch_cfg<Cfg<false, 128, true, false, 1 << kOpV>>(a, st);
        return hipErrorInvalidValue;
    }
    if (h16) {
        if (mt || f32) return hipErrorInvalidValue;
        if (h16 == 1 << kOpQ) return launch_h16<1 << kOpQ>(a, dk, st);
        if (h16 == 1 << kOpK) return launch_h16<1 << kOpK>(a, dk, st);
        if (h16 == 1 << kOpV) return launch_h16<1 << kOpV>(a, dk, st);
        return hipErrorInvalidValue;
    }
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
