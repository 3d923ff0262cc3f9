// gla_bwd.hip -- the element-wise and reduction kernels of the backward pass (gla_bwd).
//
// The backward pass of the recurrence S_t = diag(a_t) S_{t-1} + i_t k_t^T v_t, o_t = q_t S_t
// runs three chunkwise forward passes (gla_kernels.hip) on re-ordered operands; this file
// prepares those operands and turns their outputs into the gradients.  With G_t the
// gradient with respect to S_t and R the reversal of the token order (R(x)_u = x_{L-1-u}):
//
//   dv = i . R(forward(q = R(k), k = R(q), v = R(dout), gate a', S0 = dfinal))
//   dk = i . R(forward(q = R(v), k = R(dout), v = R(q), gate a', S0 = dfinal^T))
//   dq =       forward(q = dout, k = v, v = k, gate a, input gate i, S0 = initial^T)
//
// where the reversed passes take the log gate a'_u = log a_{L-u} (u >= 1), a'_0 = 0, so that
// the decay between reversed positions is the decay between the original ones; the first
// pass's final state is G_0 and the third's is the forward final state, transposed.  The
// log-gate gradient is the reverse running sum of q_t . dq_t - k_t . dk_t (plus the
// final-state term at the last token), and dlog_ig_t = k_t . dk_t.  All scalars fp32.
//
// With bf16 inputs the passes run on the fp16 matrix-core path: q, k and v stay bf16 and the
// output gradient (fp32) enters as fp16, multiplied per (batch, head) by a power of two s
// that brings its largest magnitude into [4, 8) (the final-state gradient's largest
// magnitude counts at 1/64, as it enters the passes' fp32 states).  Every pass output is
// linear in that operand, so the gradients are the outputs times 1/s, exactly.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla.h"
#include "gla_layout.h"

namespace gla {

namespace {

constexpr float kLog2eB = 1.4426950408889634f;

__device__ __forceinline__ float in_at(const void *p, int dt, size_t i) {
    if (dt == GLA_DTYPE_F32) return reinterpret_cast<const float *>(p)[i];
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p)[i] << 16);
}

__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float scale_of(uint32_t mbits) { return grad_scale_of(mbits); }

// Largest magnitude per (batch, head) of the output gradient (n4 float4 per slice, blocks
// j < nb of the slice's nb + nbf) and of the final-state gradient over 64 (nf4 float4 per
// slice, blocks nb .. nb + nbf - 1), kPerBlock float4 a block, one partial maximum per block
// into part[bh * (nb + nbf) + j].
constexpr int kPerThread = 8;
constexpr int kPerBlock = 256 * kPerThread;
__global__ __launch_bounds__(256) void bwd_absmax_kernel(const float *dout, const float *dfin, float *part,
                                                        size_t n4, size_t nf4, int nb, int nbf) {
    __shared__ float red[4];
    const size_t bh = blockIdx.x / (unsigned)(nb + nbf);
    const int j = (int)(blockIdx.x % (unsigned)(nb + nbf));
    const int tid = (int)threadIdx.x;
    const bool fin = j >= nb;
    const float4 *src = fin ? reinterpret_cast<const float4 *>(dfin) + bh * nf4
                            : reinterpret_cast<const float4 *>(dout) + bh * n4;
    const size_t n = fin ? nf4 : n4;
    const size_t i0 = (size_t)(fin ? j - nb : j) * kPerBlock;
    const size_t i1 = i0 + kPerBlock < n ? i0 + kPerBlock : n;
    float4 x[kPerThread];
    if (i1 - i0 == (size_t)kPerBlock) {
        // a whole block: all loads issued before any is used
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) x[u] = src[i0 + (size_t)u * 256 + tid];
    } else {
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            const size_t i = i0 + (size_t)u * 256 + tid;
            x[u] = i < i1 ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    float m = 0.f;
#pragma unroll
    for (int u = 0; u < kPerThread; ++u)
        m = fmaxf(m, fmaxf(fmaxf(fabsf(x[u].x), fabsf(x[u].y)), fmaxf(fabsf(x[u].z), fabsf(x[u].w))));
    if (fin) m *= 0.015625f;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// mx[bh] = bit pattern of the largest of the slice's np partial maxima (one wave per slice).
__global__ __launch_bounds__(256) void bwd_absmax_final_kernel(const float *part, uint32_t *mx, int np, int BH) {
    const int bh = (int)(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int lane = (int)threadIdx.x & 63;
    if (bh >= BH) return;
    float m = 0.f;
    for (int i = lane; i < np; i += 64) m = fmaxf(m, part[(size_t)bh * np + i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) mx[bh] = __float_as_uint(m);
}

// The scaled output gradient as fp16, in token order (fwd) and, when rev is given, reversed.
__global__ __launch_bounds__(256) void bwd_dout16_kernel(const float *dout, const uint32_t *mx, h16x8 *fwd,
                                                        h16x8 *rev, int L, int d8, size_t total) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const size_t row = i / (size_t)d8;
    const int c = (int)(i % (size_t)d8);
    const size_t bh = row / (size_t)L;
    const int t = (int)(row % (size_t)L);
    const float s = scale_of(mx[bh]);
    const float4 a = reinterpret_cast<const float4 *>(dout)[2 * i];
    const float4 b = reinterpret_cast<const float4 *>(dout)[2 * i + 1];
    const h16x8 h = {(_Float16)(a.x * s), (_Float16)(a.y * s), (_Float16)(a.z * s), (_Float16)(a.w * s),
                     (_Float16)(b.x * s), (_Float16)(b.y * s), (_Float16)(b.z * s), (_Float16)(b.w * s)};
    fwd[i] = h;
    if (rev) rev[(bh * L + (L - 1 - t)) * (size_t)d8 + c] = h;
}

// dst = s * src per (batch, head) slice of m elements.
__global__ __launch_bounds__(256) void bwd_scale_kernel(const float *src, const uint32_t *mx, float *dst, size_t m,
                                                       size_t total) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    dst[i] = src[i] * scale_of(mx[i / m]);
}

// Reversed, fp32 copies of one [L, D] row set per (b, h): dst[bh][u][:] = src[bh][L-1-u][:].
__global__ __launch_bounds__(256) void bwd_reverse_kernel(const void *src, int dt, float *dst, int L, int D,
                                                         size_t total) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const size_t row = i / (size_t)D;
    const int c = (int)(i % (size_t)D);
    const size_t bh = row / (size_t)L;
    const int u = (int)(row % (size_t)L);
    dst[i] = in_at(src, dt, (bh * L + (L - 1 - u)) * (size_t)D + c);
}

// Log gate of the reversed passes in the per-head-and-token layout [BH, L].
__global__ __launch_bounds__(256) void bwd_gate_kernel(const float *la, int kind, float *dst, int H, int L,
                                                      size_t total) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const size_t bh = i / (size_t)L;
    const int u = (int)(i % (size_t)L);
    float x = 0.f;
    if (u > 0) x = kind == GLA_GATE_HEAD ? la[bh * L + (L - u)] : la[bh % H];
    dst[i] = x;
}

// [BH][R][C] -> [BH][C][R], times the slice's scale when mx is given.
// One 64 x 64 tile per workgroup through LDS (rows read and written whole); R and C are
// multiples of 64.
__global__ __launch_bounds__(256) void bwd_transpose_kernel(const float *src, const uint32_t *mx, float *dst, int R,
                                                           int C) {
    __shared__ float tile[64][65];
    const int tr = R / 64, tc = C / 64;
    size_t id = blockIdx.x;
    const int bc = (int)(id % (unsigned)tc);
    id /= (unsigned)tc;
    const int br = (int)(id % (unsigned)tr);
    const size_t bh = id / (unsigned)tr;
    const float sc = mx ? scale_of(mx[bh]) : 1.f;
    const size_t m = (size_t)R * C;
    const float *s = src + bh * m;
    float *o = dst + bh * m;
    const int x = (int)threadIdx.x & 63, y0 = (int)threadIdx.x >> 6;
    for (int y = y0; y < 64; y += 4) tile[y][x] = s[(size_t)(br * 64 + y) * C + bc * 64 + x] * sc;
    __syncthreads();
    for (int y = y0; y < 64; y += 4) o[(size_t)(bc * 64 + y) * R + br * 64 + x] = tile[x][y];
}

// In place, the transpose of the square N x N segment-entry states of a pass's workspace:
// entry j*nsub-1 (j = 1 .. nseg-1) of each slice's (nseg-1)*nsub state entries.  The dk pass
// state is the dv pass's transposed, so these turn the dv pass's entry states into the dk
// pass's.  One workgroup per pair of 64 x 64 tiles (bi <= bj) of a matrix; both tiles are read
// into LDS (whole rows) before either is written back, each in the other's place.
__global__ __launch_bounds__(256) void bwd_transpose_entries_kernel(float *ws, int N, int nseg, int nsub) {
    __shared__ float ta[64][65], tb[64][65];
    const int T = N / 64, npair = T * (T + 1) / 2;
    size_t id = blockIdx.x;
    int pr = (int)(id % (unsigned)npair);
    id /= (unsigned)npair;
    const int j = (int)(id % (unsigned)(nseg - 1)) + 1;
    const size_t bh = id / (unsigned)(nseg - 1);
    int bi = 0;
    while (pr >= T - bi) {
        pr -= T - bi;
        ++bi;
    }
    const int bj = bi + pr;
    float *m = ws + (bh * (size_t)(nseg - 1) * nsub + (size_t)j * nsub - 1) * N * N;
    const int x = (int)threadIdx.x & 63, y0 = (int)threadIdx.x >> 6;
    for (int y = y0; y < 64; y += 4) {
        ta[y][x] = m[(size_t)(bi * 64 + y) * N + bj * 64 + x];
        tb[y][x] = m[(size_t)(bj * 64 + y) * N + bi * 64 + x];
    }
    __syncthreads();
    for (int y = y0; y < 64; y += 4) {
        m[(size_t)(bi * 64 + y) * N + bj * 64 + x] = tb[x][y];
        m[(size_t)(bj * 64 + y) * N + bi * 64 + x] = ta[x][y];
    }
}

// One wave per token: dk_t = i_t oB[L-1-t], dv_t = i_t oA[L-1-t]; g_t = q_t . dq_t - k_t . dk_t;
// dlog_ig_t = k_t . dk_t.  Without oA / oB the passes stored dk, dv and dq in place (scaled
// and un-reversed) and only the dot products are formed.  Dk and Dv are at most 256.
__global__ __launch_bounds__(256) void bwd_post_kernel(gla_bwd_desc d, const float *oA, const float *oB, float *g,
                                                      size_t ntok) {
    const size_t tok = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tok >= ntok) return;
    const int lane = threadIdx.x & 63;
    const int L = d.L, Dk = d.Dk, Dv = d.Dv;
    const size_t bh = tok / (size_t)L;
    const int t = (int)(tok % (size_t)L);
    const size_t rtok = bh * L + (L - 1 - t);
    float qdq = 0.f, kdk = 0.f;
    if (!oB) {
        for (int c = lane; c < Dk; c += 64) {
            kdk += in_at(d.k, d.in_dtype, tok * Dk + c) * d.dk[tok * Dk + c];
            qdq += in_at(d.q, d.in_dtype, tok * Dk + c) * d.dq[tok * Dk + c];
        }
    } else {
        const float ig = d.log_ig ? exp2f(d.log_ig[tok] * kLog2eB) : 1.f;
        for (int c = lane; c < Dk; c += 64) {
            const float dkv = ig * oB[rtok * Dk + c];
            d.dk[tok * Dk + c] = dkv;
            kdk += in_at(d.k, d.in_dtype, tok * Dk + c) * dkv;
            qdq += in_at(d.q, d.in_dtype, tok * Dk + c) * d.dq[tok * Dk + c];
        }
        for (int c = lane; c < Dv; c += 64) d.dv[tok * Dv + c] = ig * oA[rtok * Dv + c];
    }
    qdq = wave_sum64(qdq);
    kdk = wave_sum64(kdk);
    if (lane == 0) {
        if (g) g[tok] = qdq - kdk;
        if (d.dlog_ig) d.dlog_ig[tok] = kdk;
    }
}

// g_t = q_t . dq_t - k_t . dk_t and dlog_ig_t = k_t . dk_t from the stored gradients: 2^lg =
// Dk / 4 lanes per token (four channels each, 16-byte gradient loads), 64 / 2^lg tokens per
// wave.
__global__ __launch_bounds__(256) void bwd_dot_kernel(gla_bwd_desc d, float *g, size_t ntok, int lg) {
    const int lane = (int)threadIdx.x & 63;
    const int G = 1 << lg;
    const size_t tok = ((size_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (size_t)(64 >> lg) + (size_t)(lane >> lg);
    const int c = (lane & (G - 1)) * 4;
    const size_t Dk = (size_t)d.Dk;
    float qdq = 0.f, kdk = 0.f;
    if (tok < ntok) {
        const size_t o = tok * Dk + c;
        const float4 dq = *reinterpret_cast<const float4 *>(d.dq + o);
        const float4 dk = *reinterpret_cast<const float4 *>(d.dk + o);
        float q[4], k[4];
        if (d.in_dtype == GLA_DTYPE_F32) {
            const float4 a = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(d.q) + o);
            const float4 b = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(d.k) + o);
            q[0] = a.x, q[1] = a.y, q[2] = a.z, q[3] = a.w;
            k[0] = b.x, k[1] = b.y, k[2] = b.z, k[3] = b.w;
        } else {
            const uint2 a = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(d.q) + o);
            const uint2 b = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(d.k) + o);
            q[0] = __uint_as_float(a.x << 16), q[1] = __uint_as_float(a.x & 0xffff0000u);
            q[2] = __uint_as_float(a.y << 16), q[3] = __uint_as_float(a.y & 0xffff0000u);
            k[0] = __uint_as_float(b.x << 16), k[1] = __uint_as_float(b.x & 0xffff0000u);
            k[2] = __uint_as_float(b.y << 16), k[3] = __uint_as_float(b.y & 0xffff0000u);
        }
        qdq = q[0] * dq.x + q[1] * dq.y + q[2] * dq.z + q[3] * dq.w;
        kdk = k[0] * dk.x + k[1] * dk.y + k[2] * dk.z + k[3] * dk.w;
    }
    for (int o = G >> 1; o > 0; o >>= 1) {
        qdq += __shfl_xor(qdq, o);
        kdk += __shfl_xor(kdk, o);
    }
    if ((lane & (G - 1)) == 0 && tok < ntok) {
        if (g) g[tok] = qdq - kdk;
        if (d.dlog_ig) d.dlog_ig[tok] = kdk;
    }
}

// The same from the dot products the bf16 dq and dk passes formed as they stored their rows:
// qp and kp hold, per 64-column tile j < nj, q_t . dq_t and k_t . dk_t over the tile's
// channels ([nj][ntok]; qp null when g is not wanted), summed here in tile order.
__global__ __launch_bounds__(256) void bwd_dot_sum_kernel(const float *qp, const float *kp, int nj, size_t ntok,
                                                          float *g, float *dli) {
    const size_t tok = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (tok >= ntok) return;
    float qdq = 0.f, kdk = 0.f;
    for (int j = 0; j < nj; ++j) {
        if (qp) qdq += qp[(size_t)j * ntok + tok];
        kdk += kp[(size_t)j * ntok + tok];
    }
    if (g) g[tok] = qdq - kdk;
    if (dli) dli[tok] = kdk;
}

// The final-state term of the last token's g: the sum over (j, d) of dfinal^T[j][d] S_fin^T[j][d]
// (dfT and finC both transposed; times 1/s when dfT carries the scale).  One workgroup per
// (b, h) in a fixed order, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void bwd_fin_term_kernel(const float *dfT, const float *finC, const uint32_t *mx,
                                                          float *g, int L, size_t n4) {
    __shared__ float red[4];
    const size_t bh = blockIdx.x;
    const float4 *a = reinterpret_cast<const float4 *>(dfT) + bh * n4;
    const float4 *b = reinterpret_cast<const float4 *>(finC) + bh * n4;
    const int tid = (int)threadIdx.x;
    float sum = 0.f;
#pragma unroll 4
    for (size_t i = tid; i < n4; i += 256) {
        const float4 x = a[i], y = b[i];
        sum += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
    }
    sum = wave_sum64(sum);
    if ((tid & 63) == 0) red[tid >> 6] = sum;
    __syncthreads();
    if (tid == 0) {
        const float inv = mx ? 1.f / scale_of(mx[bh]) : 1.f;
        g[bh * L + L - 1] += ((red[0] + red[1]) + (red[2] + red[3])) * inv;
    }
}

// One workgroup per (b, h): the reverse running sum of g into dlog_alpha (per head and token
// gate), or the weighted total sum_u (u+1) g_u into part[bh] (fixed per-head gate).
__global__ __launch_bounds__(256) void bwd_gate_reduce_kernel(gla_bwd_desc d, const float *g, float *part) {
    __shared__ float red[256];
    __shared__ float carry;
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int L = d.L;
    const float *gb = g + (size_t)bh * L;
    if (d.gate_kind == GLA_GATE_HEAD) {
        if (tid == 0) carry = 0.f;
        __syncthreads();
        // blocks of 256 tokens from the end; inclusive suffix scan inside a block
        for (int end = L; end > 0; end -= 256) {
            const int t = end - 1 - tid;
            red[tid] = t >= 0 ? gb[t] : 0.f;
            __syncthreads();
            for (int o = 1; o < 256; o <<= 1) {
                const float y = tid >= o ? red[tid - o] : 0.f;
                __syncthreads();
                red[tid] += y;
                __syncthreads();
            }
            const float c0 = carry;
            if (t >= 0) d.dlog_alpha[(size_t)bh * L + t] = red[tid] + c0;
            __syncthreads();
            if (tid == 255) carry = c0 + red[255];
            __syncthreads();
        }
    } else {
        float s = 0.f;
        for (int t = tid; t < L; t += 256) s += (float)(t + 1) * gb[t];
        red[tid] = s;
        __syncthreads();
        for (int o = 128; o > 0; o >>= 1) {
            if (tid < o) red[tid] += red[tid + o];
            __syncthreads();
        }
        if (tid == 0) part[bh] = red[0];
    }
}

// dinitial_state = diag(alpha_0) G_0: the first pass's final state times the first token's
// decay (and 1/s when finA carries the scale).
// Workgroup = 1,024 consecutive elements (four per thread) of one (batch, head) slice of
// m = Dk * Dv elements, a multiple of 4,096.
__global__ __launch_bounds__(256) void bwd_dinit_kernel(gla_bwd_desc d, const float *finA, const uint32_t *mx,
                                                       int m) {
    const unsigned nb = (unsigned)m / 1024u;
    const size_t bh = blockIdx.x / nb;
    const int e = (int)(blockIdx.x % nb) * 1024 + 4 * (int)threadIdx.x;  // element within the slice
    float a0 = mx ? 1.f / scale_of(mx[bh]) : 1.f;
    if (d.gate_kind == GLA_GATE_HEAD) a0 *= exp2f(d.log_alpha[bh * d.L] * kLog2eB);
    else if (d.gate_kind == GLA_GATE_HEAD_CONST) a0 *= exp2f(d.log_alpha[bh % d.H] * kLog2eB);
    else if (d.gate_kind == GLA_GATE_CHANNEL)  // row r of G_0 decays with channel r of token 0
        a0 *= exp2f(d.log_alpha[bh * d.L * d.Dk + e / d.Dv] * kLog2eB);
    const size_t i = bh * (size_t)m + e;
    float4 x = *reinterpret_cast<const float4 *>(finA + i);
    x.x *= a0, x.y *= a0, x.z *= a0, x.w *= a0;
    *reinterpret_cast<float4 *>(d.dinitial_state + i) = x;
}

// Fixed per-head gate: dlog_alpha[h] = sum over the batch of the per-(b, h) totals.
__global__ __launch_bounds__(256) void bwd_head_sum_kernel(const float *part, float *dla, int B, int H) {
    const int h = blockIdx.x * 256 + threadIdx.x;
    if (h >= H) return;
    float s = 0.f;
    for (int b = 0; b < B; ++b) s += part[(size_t)b * H + h];
    dla[h] = s;
}

// Strided 2-D copy of 16-byte units: row r of n16 units from src + r * ss to dst + r * ds
// (strides in 16-byte units).  Splits a pass over value columns into halves and places the
// halves' states.
__global__ __launch_bounds__(256) void bwd_copy2d_kernel(const uint4 *src, size_t ss, uint4 *dst, size_t ds, size_t n16,
                                                        size_t total) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const size_t r = i / n16, c = i % n16;
    dst[r * ds + c] = src[r * ss + c];
}

inline unsigned nblk(size_t n, unsigned per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t bwd_copy2d(const void *src, size_t src_stride, void *dst, size_t dst_stride, size_t rows, size_t row_bytes,
                      hipStream_t st) {
    if ((src_stride | dst_stride | row_bytes) % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(dst) & 15) != 0)
        return hipErrorInvalidValue;
    const size_t n16 = row_bytes / 16, total = rows * n16;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_copy2d_kernel, dim3(nblk(total, 256)), dim3(256), 0, st, reinterpret_cast<const uint4 *>(src),
                       src_stride / 16, reinterpret_cast<uint4 *>(dst), dst_stride / 16, n16, total);
    return hipGetLastError();
}

hipError_t bwd_reverse(const void *src, int dt, float *dst, int BH, int L, int D, hipStream_t st) {
    const size_t total = (size_t)BH * L * D;
    hipLaunchKernelGGL(bwd_reverse_kernel, dim3(nblk(total, 256)), dim3(256), 0, st, src, dt, dst, L, D, total);
    return hipGetLastError();
}

hipError_t bwd_gate(const float *la, int kind, float *dst, int BH, int H, int L, hipStream_t st) {
    const size_t total = (size_t)BH * L;
    hipLaunchKernelGGL(bwd_gate_kernel, dim3(nblk(total, 256)), dim3(256), 0, st, la, kind, dst, H, L, total);
    return hipGetLastError();
}

hipError_t bwd_transpose(const float *src, const uint32_t *mx, float *dst, int BH, int R, int C, hipStream_t st) {
    const size_t tiles = (size_t)BH * (R / 64) * (C / 64);
    hipLaunchKernelGGL(bwd_transpose_kernel, dim3((unsigned)tiles), dim3(256), 0, st, src, mx, dst, R, C);
    return hipGetLastError();
}

hipError_t bwd_transpose_entries(float *ws, int BH, int N, int nseg, int nsub, hipStream_t st) {
    if (nseg < 2) return hipSuccess;
    const int T = N / 64;
    const size_t blocks = (size_t)BH * (size_t)(nseg - 1) * (size_t)(T * (T + 1) / 2);
    hipLaunchKernelGGL(bwd_transpose_entries_kernel, dim3((unsigned)blocks), dim3(256), 0, st, ws, N, nseg, nsub);
    return hipGetLastError();
}

size_t bwd_absmax_parts(int L, int Dv, int Dk, bool dfin) {
    return nblk((size_t)L * Dv / 4, kPerBlock) + (dfin ? nblk((size_t)Dk * Dv / 4, kPerBlock) : 0);
}

// Per-(batch, head) scale of the output gradient into mx (bit patterns of the largest
// magnitudes, through bwd_absmax_parts(...) partials per slice in part), then its fp16
// copies (token order and reversed).
hipError_t bwd_dout16(const float *dout, const float *dfin, float *part, uint32_t *mx, _Float16 *fwd, _Float16 *rev,
                      int BH, int L, int Dv, int Dk, hipStream_t st) {
    const size_t n4 = (size_t)L * Dv / 4, nf4 = dfin ? (size_t)Dk * Dv / 4 : 0;
    const int nb = (int)nblk(n4, kPerBlock), nbf = (int)nblk(nf4, kPerBlock);
    hipLaunchKernelGGL(bwd_absmax_kernel, dim3((unsigned)((size_t)(nb + nbf) * BH)), dim3(256), 0, st, dout, dfin,
                       part, n4, nf4, nb, nbf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_absmax_final_kernel, dim3(nblk((size_t)BH, 4)), dim3(256), 0, st, part, mx, nb + nbf, BH);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t total = (size_t)BH * L * (Dv / 8);
    hipLaunchKernelGGL(bwd_dout16_kernel, dim3(nblk(total, 256)), dim3(256), 0, st, dout, mx,
                       reinterpret_cast<h16x8 *>(fwd), reinterpret_cast<h16x8 *>(rev), L, Dv / 8, total);
    return hipGetLastError();
}

hipError_t bwd_scale(const float *src, const uint32_t *mx, float *dst, int BH, size_t m, hipStream_t st) {
    const size_t total = (size_t)BH * m;
    hipLaunchKernelGGL(bwd_scale_kernel, dim3(nblk(total, 256)), dim3(256), 0, st, src, mx, dst, m, total);
    return hipGetLastError();
}

hipError_t bwd_finish(const gla_bwd_desc &d, const float *oA, const float *oB, float *g, const float *finA,
                      const float *finC, const float *dfT, float *part, const uint32_t *mx, const float *dqp,
                      const float *dkp, hipStream_t st) {
    const int BH = d.B * d.H;
    const size_t ntok = (size_t)BH * d.L;
    hipError_t e = hipSuccess;
    if (oB) {
        hipLaunchKernelGGL(bwd_post_kernel, dim3(nblk(ntok, 4)), dim3(256), 0, st, d, oA, oB, g, ntok);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (dkp && (g || d.dlog_ig)) {
        hipLaunchKernelGGL(bwd_dot_sum_kernel, dim3(nblk(ntok, 256)), dim3(256), 0, st, dqp, dkp, d.Dk / 64, ntok, g,
                           d.dlog_ig);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (g || d.dlog_ig) {
        const int lg = d.Dk == 64 ? 4 : (d.Dk == 128 ? 5 : 6);  // Dk / 4 lanes per token
        const size_t per_block = (size_t)4 * (64 >> lg);
        hipLaunchKernelGGL(bwd_dot_kernel, dim3(nblk(ntok, (unsigned)per_block)), dim3(256), 0, st, d, g, ntok, lg);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const size_t m = (size_t)d.Dk * d.Dv;
    if (g && dfT) {
        hipLaunchKernelGGL(bwd_fin_term_kernel, dim3((unsigned)BH), dim3(256), 0, st, dfT, finC, mx, g, d.L, m / 4);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (g) {
        hipLaunchKernelGGL(bwd_gate_reduce_kernel, dim3(BH), dim3(256), 0, st, d, g, part);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (d.dinitial_state) {
        hipLaunchKernelGGL(bwd_dinit_kernel, dim3((unsigned)((size_t)BH * (m / 1024))), dim3(256), 0, st, d, finA, mx,
                           (int)m);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (g && d.gate_kind == GLA_GATE_HEAD_CONST) {
        hipLaunchKernelGGL(bwd_head_sum_kernel, dim3(nblk((size_t)d.H, 256)), dim3(256), 0, st, part, d.dlog_alpha,
                           d.B, d.H);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace gla
