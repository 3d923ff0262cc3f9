// gla_rows.h -- building blocks of the chunk kernels that keep a (batch, head)'s state slice
// in registers and walk its sequence chunk by chunk (the delta rule and the mLSTM):
// operand types, buffer-resource access, the matrix-core products in the slot order shared
// by LDS rows and accumulators, and the staging of a chunk's q, k, k^T and v^T rows.
//
// Slot order.  The 16x16 accumulator of lane (g, c) holds rows 4g+e, column c.  When the
// contraction index of a 32-deep product is ordered so that k-slot 8g+j is row 4g+j (j < 4)
// or 16+4g+j-4 (j >= 4) of the step's 32 rows, an accumulator pair is directly a B operand.
// Channel rows (q, k) and token rows (k^T, v^T, scores) are stored in LDS in that order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gla_rows {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kC = 64;                   // tokens per chunk

// Configuration of a kernel instance: operand type (fp32 or fp16 from bf16), Dk and the
// threads of a workgroup (which share the staging of a chunk; the value tile has NT / 4
// columns).
template <bool F32_, int DK_, int NT_ = 256>
struct Cfg {
    static constexpr bool F32 = F32_;
    static constexpr int DK = DK_;
    static constexpr int NT = NT_;
    using OpT = typename std::conditional<F32, float, f16>::type;
    using Frag = typename std::conditional<F32, f32x8, f16x8>::type;  // one 32-deep operand
    using Quad = typename std::conditional<F32, f32x4, f16x4>::type;  // 4 consecutive operands
    static constexpr int OB = F32 ? 4 : 2;
    static constexpr int IB = F32 ? 4 : 2;
    static constexpr int RQ = DK + 16 / OB;  // row stride of channel rows (q, k)
    static constexpr int RT = kC + 16 / OB;  // row stride of token rows (scores, K^T, V^T)
    static constexpr int NB = DK / 16;       // 16-row blocks of the state
    static constexpr int NM = DK / 32;       // 32-deep steps over the channels
    static constexpr int NP = DK / 4;        // 4-element pieces of a channel row
    static constexpr int QSTEP = NT / NP;    // token quads apart of a thread's pieces
    static constexpr int QPT = 16 / QSTEP;   // token quads per thread (16 quads per chunk)
    static constexpr int NVQ = NT / 16;      // 4-column quads of the value tile
    using Piece = typename std::conditional<F32, u32x4, u32x2>::type;  // 4 raw inputs
    static_assert(QSTEP >= 1 && QPT >= 1 && QSTEP * QPT == 16, "threads must tile a chunk's rows");
};

// ------------------------------------------------------------------------------------
__device__ __forceinline__ void barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ rsrc_t make_rsrc(const void *p, uint64_t bytes) {
    const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n, kRsrcFlags);
}
__device__ __forceinline__ u32x4 bld128(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ float bld_f32(rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void bst_f32(float x, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, (int)off, 0, 0);
}
// log2 of a per-token decay, floored at -150 (the factor is zero either way; the floor
// keeps running sums small enough for their differences to keep fp32 precision).
__device__ __forceinline__ float log2_decay(float la) {
    const float x = la * kLog2e;
    return x < -150.f ? -150.f : x;
}
// One DPP step: x of the lane CTRL selects (rows outside ROWS, and lanes whose source lies
// outside their row, read `none`).
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_or(float x, float none) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(none), __float_as_int(x), CTRL, ROWS, 0xf, false));
}
// Inclusive prefix of op over the wave's lanes on the vector ALU (no LDS crossbar): row
// shifts by 1, 2, 4, 8 within each 16-lane row, then the end of row 0 (row broadcast 15) into
// rows 1 and 3 and the end of row 1 (row broadcast 31) into rows 2 and 3; id is op's identity.
template <class Op>
__device__ __forceinline__ float scan_dpp(float x, float id, Op op) {
    x = op(x, dpp_or<0x111>(x, id));
    x = op(x, dpp_or<0x112>(x, id));
    x = op(x, dpp_or<0x114>(x, id));
    x = op(x, dpp_or<0x118>(x, id));
    x = op(x, dpp_or<0x142, 0xa>(x, id));
    x = op(x, dpp_or<0x143, 0xc>(x, id));
    return x;
}
__device__ __forceinline__ float scan_incl(float x, [[maybe_unused]] int lane) {
    return scan_dpp(x, 0.f, [](float u, float v) { return u + v; });
}
// x of lane n (wave-uniform n), through a scalar register.
__device__ __forceinline__ float lane_bcast(float x, int n) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), n));
}
// gfx950 lane-swap moves (v_permlane16_swap / v_permlane32_swap) of x with itself: the first
// result holds rows (0, 0, 2, 2) / halves (0, 0) of x, the second rows (1, 1, 3, 3) / halves
// (1, 1), rows being 16 lanes and halves 32.
__device__ __forceinline__ float add_xor16(float x) {  // x + x of lane (l ^ 16)
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {  // x + x of lane (l ^ 32)
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Row R (0..3) of x in every row: x of lane 16 R + (l & 15).
template <int R>
__device__ __forceinline__ float row_to_all(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const uint32_t y = a[R & 1];  // rows (R&1, R&1, 2+(R&1), 2+(R&1))
    const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
    return __uint_as_float(b[R >> 1]);
}
// Workgroups i and i+8, ... go to the same XCD; consecutive logical workgroups (the value
// slices of one head, which read the same q and k) are placed on one XCD to share its L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
    if ((n & 7) != 0) return i;
    return (i & 7) * (n >> 3) + (i >> 3);
}

// Position of index x (0..31) inside its 32-group: slot 8g+j holds 4g+j (j < 4) and
// 16+4g+j-4 (j >= 4).
__device__ __forceinline__ int pos32(int x) { return x < 16 ? 8 * (x >> 2) + (x & 3) : 8 * ((x - 16) >> 2) + 4 + (x & 3); }
__device__ __forceinline__ int perm(int x) { return (x & ~31) + pos32(x & 31); }
// Column of token slot x in row `row` of k^T: the eight 8-slot groups of a row are permuted
// by an XOR with bits 4..6 of the row, so that the transposed stores of the staging step
// (four consecutive rows per thread, 4 rows apart across threads) spread over the banks.
__device__ __forceinline__ int kt_col(int row, int x) { return (((x >> 3) ^ (row >> 4)) & 7) * 8 + (x & 7); }

// 32-deep product with fp16 operands, or the same contraction as eight fp32 4-deep steps
// (element e of every lane's eight values forms step e).
__device__ __forceinline__ f32x4 mma(const f16x8 &a, const f16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8 &a, const f32x8 &b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}
// 16-deep product: lane (g, c) gives A[c][4g+e] and B[4g+e][c] (e < 4), so a 16x16
// accumulator is directly a B operand.
template <bool F32>
__device__ __forceinline__ f32x4 mma16(const f32x4 &a, const f32x4 &b, f32x4 c) {
    if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
        return c;
    } else {
        const f16x4 ah{(f16)a[0], (f16)a[1], (f16)a[2], (f16)a[3]};
        const f16x4 bh{(f16)b[0], (f16)b[1], (f16)b[2], (f16)b[3]};
        return __builtin_amdgcn_mfma_f32_16x16x16f16(ah, bh, c, 0, 0, 0);
    }
}

template <class C>
__device__ __forceinline__ typename C::Frag ld_frag(const typename C::OpT *p) {
    if constexpr (C::F32) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
        return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
        return *reinterpret_cast<const f16x8 *>(p);
    }
}
// Operand from two 16x16 accumulators (rows 4g+e of blocks 2m and 2m+1), times s.
template <class C>
__device__ __forceinline__ typename C::Frag acc_frag(const f32x4 &lo, const f32x4 &hi, float s = 1.f) {
    using OpT = typename C::OpT;
    typename C::Frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = (OpT)(lo[e] * s);
        f[e + 4] = (OpT)(hi[e] * s);
    }
    return f;
}
// The same with a per-row factor.
template <class C>
__device__ __forceinline__ typename C::Frag acc_frag_rows(const f32x4 &lo, const f32x4 &hi, const f32x4 &slo,
                                                          const f32x4 &shi) {
    using OpT = typename C::OpT;
    typename C::Frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = (OpT)(lo[e] * slo[e]);
        f[e + 4] = (OpT)(hi[e] * shi[e]);
    }
    return f;
}

// The rounding residual of an operand, as a second operand: x = hi + lo to about 2^-22 of x
// (fp16 operands); zero with fp32 operands, where no split is needed.
template <class C>
__device__ __forceinline__ typename C::Frag residual(const f32x4 &lo, const f32x4 &hi, const typename C::Frag &f,
                                                     const f32x4 &slo, const f32x4 &shi) {
    using OpT = typename C::OpT;
    typename C::Frag r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (OpT)(lo[e] * slo[e] - (float)f[e]);
        r[e + 4] = (OpT)(hi[e] * shi[e] - (float)f[e + 4]);
    }
    return r;
}

// Raw 4-element pieces of the next chunk, held in registers while the current one runs:
// thread tid holds piece tid % NP of the channel rows of token quads tid / NP + j QSTEP (q
// and k) and columns 4 (tid % NVQ).. of token quad tid / NVQ (v).
template <class C>
struct Pieces {
    typename C::Piece q[C::QPT][4], k[C::QPT][4], v[4];
};

template <class C>
__device__ __forceinline__ typename C::Piece ld_piece(rsrc_t r, uint32_t off) {
    if constexpr (C::F32) return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}

// The next chunk's loads can be issued in groups (q rows, k rows, v) at different points
// of the current chunk, so that their issue overlaps the work in between.
template <class C>
__device__ __forceinline__ void prefetch_rows(typename C::Piece (&dst)[C::QPT][4], rsrc_t r, int T0, int tid) {
    const int c = tid % C::NP;
#pragma unroll
    for (int j = 0; j < C::QPT; ++j) {
        const int a = tid / C::NP + j * C::QSTEP;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
            dst[j][tt] = ld_piece<C>(r, ((uint32_t)(T0 + 4 * a + tt) * C::DK + 4 * c) * C::IB);
    }
}
template <class C>
__device__ __forceinline__ void prefetch_v(typename C::Piece (&dst)[4], rsrc_t rv, int T0, int tid, int dv0, int Dv) {
    const int a = tid / C::NVQ, cv = tid % C::NVQ;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
        dst[tt] = ld_piece<C>(rv, ((uint32_t)(T0 + 4 * a + tt) * Dv + dv0 + 4 * cv) * C::IB);
}

// Element e (0..3) of a raw piece as fp32.
template <class C>
__device__ __forceinline__ float el(const typename C::Piece &x, int e) {
    if constexpr (C::F32) return __uint_as_float(x[e]);
    else return (e & 1) ? bf_hi(x[e >> 1]) : bf_lo(x[e >> 1]);
}

template <class C>
__device__ __forceinline__ void store_quad(typename C::OpT *p, float a, float b, float c, float d) {
    using Q = typename C::Quad;
    using OpT = typename C::OpT;
    *reinterpret_cast<Q *>(p) = Q{(OpT)a, (OpT)b, (OpT)c, (OpT)d};
}

// The prefetched q, k and v pieces into LDS: q and k rows (channels in slot order), k^T
// (tokens in slot order, 8-slot groups permuted by kt_col) and v^T (tokens in slot order).
// Four consecutive channels or tokens starting at a multiple of 4 occupy four consecutive
// slots.
template <class C>
__device__ __forceinline__ void stage_rows(const Pieces<C> &pf, typename C::OpT *sQ, typename C::OpT *sK,
                                           typename C::OpT *sKt, typename C::OpT *sVt, int tid) {
    const int c = tid % C::NP;
    const int pc = perm(4 * c);
#pragma unroll
    for (int j = 0; j < C::QPT; ++j) {
        const int a = tid / C::NP + j * C::QSTEP;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int t = 4 * a + tt;
            store_quad<C>(sQ + t * C::RQ + pc, el<C>(pf.q[j][tt], 0), el<C>(pf.q[j][tt], 1), el<C>(pf.q[j][tt], 2),
                          el<C>(pf.q[j][tt], 3));
            store_quad<C>(sK + t * C::RQ + pc, el<C>(pf.k[j][tt], 0), el<C>(pf.k[j][tt], 1), el<C>(pf.k[j][tt], 2),
                          el<C>(pf.k[j][tt], 3));
        }
        const int tp = perm(4 * a);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            store_quad<C>(sKt + (4 * c + e) * C::RT + kt_col(4 * c + e, tp), el<C>(pf.k[j][0], e), el<C>(pf.k[j][1], e),
                          el<C>(pf.k[j][2], e), el<C>(pf.k[j][3], e));
    }
    {
        const int a = tid / C::NVQ, cv = tid % C::NVQ;
        const int tp = perm(4 * a);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            store_quad<C>(sVt + (4 * cv + e) * C::RT + tp, el<C>(pf.v[0], e), el<C>(pf.v[1], e), el<C>(pf.v[2], e),
                          el<C>(pf.v[3], e));
    }
}

}  // namespace gla_rows
