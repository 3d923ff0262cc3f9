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

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla.h"

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

// fp32 copy in the same order.
__global__ __launch_bounds__(256) void bwd_convert_kernel(const void *src, int dt, float *dst, size_t total) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    dst[i] = in_at(src, dt, i);
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

// [BH][R][C] -> [BH][C][R]
__global__ __launch_bounds__(256) void bwd_transpose_kernel(const float *src, float *dst, int R, int C,
                                                           size_t total) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const size_t m = (size_t)R * C;
    const size_t bh = i / m;
    const size_t rc = i % m;
    const int r = (int)(rc / C), c = (int)(rc % C);
    dst[bh * m + (size_t)c * R + r] = src[i];
}

// One wave per token: dk_t = i_t oB[L-1-t], dv_t = i_t oA[L-1-t]; g_t = q_t . dq_t - k_t . dk_t;
// dlog_ig_t = k_t . dk_t.  Dk and Dv are at most 256 (four values per lane).
__global__ __launch_bounds__(256) void bwd_post_kernel(gla_bwd_desc d, const float *oA, const float *oB, float *g,
                                                      size_t ntok) {
    const size_t tok = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tok >= ntok) return;
    const int lane = threadIdx.x & 63;
    const int L = d.L, Dk = d.Dk, Dv = d.Dv;
    const size_t bh = tok / (size_t)L;
    const int t = (int)(tok % (size_t)L);
    const size_t rtok = bh * L + (L - 1 - t);
    const float ig = d.log_ig ? exp2f(d.log_ig[tok] * kLog2eB) : 1.f;
    float qdq = 0.f, kdk = 0.f;
    for (int c = lane; c < Dk; c += 64) {
        const float dkv = ig * oB[rtok * Dk + c];
        d.dk[tok * Dk + c] = dkv;
        kdk += in_at(d.k, d.in_dtype, tok * Dk + c) * dkv;
        qdq += in_at(d.q, d.in_dtype, tok * Dk + c) * d.dq[tok * Dk + c];
    }
    for (int c = lane; c < Dv; c += 64) d.dv[tok * Dv + c] = ig * oA[rtok * Dv + c];
    qdq = wave_sum64(qdq);
    kdk = wave_sum64(kdk);
    if (lane == 0) {
        if (g) g[tok] = qdq - kdk;
        if (d.dlog_ig) d.dlog_ig[tok] = kdk;
    }
}

// One workgroup per (b, h): adds the final-state term to the last token's g, then the
// reverse running sum (per head and token gate) or the weighted total sum_u (u+1) g_u (fixed
// per-head gate, into part[bh]); and dinitial_state = a_0 G_0.
__global__ __launch_bounds__(256) void bwd_gate_reduce_kernel(gla_bwd_desc d, float *g, const float *finA,
                                                             const float *finC, float *part) {
    __shared__ float red[256];
    __shared__ float carry;
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int L = d.L, Dk = d.Dk, Dv = d.Dv;
    const size_t m = (size_t)Dk * Dv;
    if (g) {
        if (d.dfinal_state) {
            // sum over (d, j) of dfinal[d][j] * S_fin[d][j]; finC holds S_fin transposed [j][d]
            float s = 0.f;
            for (size_t i = tid; i < m; i += 256) {
                const int r = (int)(i / Dv), c = (int)(i % Dv);
                s += d.dfinal_state[bh * m + i] * finC[bh * m + (size_t)c * Dk + r];
            }
            red[tid] = s;
            __syncthreads();
            for (int o = 128; o > 0; o >>= 1) {
                if (tid < o) red[tid] += red[tid + o];
                __syncthreads();
            }
            if (tid == 0) g[(size_t)bh * L + L - 1] += red[0];
            __syncthreads();
        }
        float *gb = g + (size_t)bh * L;
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
    if (d.dinitial_state) {
        float a0 = 1.f;
        if (d.gate_kind == GLA_GATE_HEAD) a0 = exp2f(d.log_alpha[(size_t)bh * L] * kLog2eB);
        else if (d.gate_kind == GLA_GATE_HEAD_CONST) a0 = exp2f(d.log_alpha[bh % d.H] * kLog2eB);
        for (size_t i = tid; i < m; i += 256) d.dinitial_state[bh * m + i] = a0 * finA[bh * m + i];
    }
}

// Fixed per-head gate: dlog_alpha[h] = sum over the batch of the per-(b, h) totals.
__global__ __launch_bounds__(256) void bwd_head_sum_kernel(const float *part, float *dla, int B, int H) {
    const int h = blockIdx.x * 256 + threadIdx.x;
    if (h >= H) return;
    float s = 0.f;
    for (int b = 0; b < B; ++b) s += part[(size_t)b * H + h];
    dla[h] = s;
}

inline unsigned nblk(size_t n, unsigned per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t bwd_reverse(const void *src, int dt, float *dst, int BH, int L, int D, hipStream_t st) {
    const size_t total = (size_t)BH * L * D;
    hipLaunchKernelGGL(bwd_reverse_kernel, dim3(nblk(total, 256)), dim3(256), 0, st, src, dt, dst, L, D, total);
    return hipGetLastError();
}

hipError_t bwd_convert(const void *src, int dt, float *dst, size_t total, hipStream_t st) {
    hipLaunchKernelGGL(bwd_convert_kernel, dim3(nblk(total, 256)), dim3(256), 0, st, src, dt, dst, total);
    return hipGetLastError();
}

hipError_t bwd_gate(const float *la, int kind, float *dst, int BH, int H, int L, hipStream_t st) {
    const size_t total = (size_t)BH * L;
    hipLaunchKernelGGL(bwd_gate_kernel, dim3(nblk(total, 256)), dim3(256), 0, st, la, kind, dst, H, L, total);
    return hipGetLastError();
}

hipError_t bwd_transpose(const float *src, float *dst, int BH, int R, int C, hipStream_t st) {
    const size_t total = (size_t)BH * R * C;
    hipLaunchKernelGGL(bwd_transpose_kernel, dim3(nblk(total, 256)), dim3(256), 0, st, src, dst, R, C, total);
    return hipGetLastError();
}

hipError_t bwd_finish(const gla_bwd_desc &d, const float *oA, const float *oB, float *g, const float *finA,
                      const float *finC, float *part, hipStream_t st) {
    const int BH = d.B * d.H;
    const size_t ntok = (size_t)BH * d.L;
    hipLaunchKernelGGL(bwd_post_kernel, dim3(nblk(ntok, 4)), dim3(256), 0, st, d, oA, oB, g, ntok);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (g || d.dinitial_state) {
        hipLaunchKernelGGL(bwd_gate_reduce_kernel, dim3(BH), dim3(256), 0, st, d, g, finA, finC, part);
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
