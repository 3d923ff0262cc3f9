// gla_mlstm.h -- arguments of the mLSTM kernel (exponential input gate and normaliser),
// shared by the host entry point and the gfx950 kernel.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace gla_mlstm {

struct MlstmArgs {
    const void *q, *k, *v;              // [B,H,L,Dk], [B,H,L,Dk], [B,H,L,Dv] in the input dtype
    const float *lf, *li;               // [B,H,L] log forget gate, log input gate
    const float *c0, *n0, *m0;          // stabilised initial state [B,H,Dk,Dv], [B,H,Dk], [B,H]; all or none
    float *out;                         // [B,H,L,Dv]
    float *fin_c, *fin_n, *fin_m;       // stabilised final state, each optional
    int B, H, L, Dv;
    int ndv;                            // value slices of wg_cols columns
    int nwg;                            // workgroups = B * H * ndv
};

// Value columns per workgroup: 128 (eight waves, two per SIMD) for fp16 operands with Dk = 256
// when Dv is a multiple of 128, else 64 (four waves).
int wg_cols(bool f32, int dk, int dv);
// LDS bytes of one workgroup (fp32 or fp16 operands, Dk, value columns).
uint32_t lds_bytes(bool f32, int dk, int cols);
hipError_t launch(const MlstmArgs &a, bool f32, int dk, hipStream_t st);

}  // namespace gla_mlstm
