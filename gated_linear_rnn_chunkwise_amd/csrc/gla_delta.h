// gla_delta.h -- arguments of the delta-rule kernel, shared by the host entry point and the
// gfx950 kernel.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace gla_delta {

struct DeltaArgs {
    const void *q, *k, *v;   // [B,H,L,Dk], [B,H,L,Dk], [B,H,L,Dv] in the input dtype
    const float *beta;       // [B,H,L]
    const float *la;         // per gate kind: [B,H,L], [H], or null
    const float *s0;         // [B,H,Dk,Dv] or null
    float *out;              // [B,H,L,Dv]
    float *fin;              // [B,H,Dk,Dv] or null
    int B, H, L, Dv;
    int gate;                // enum gla_gate: NONE, HEAD or HEAD_CONST
    int ndv;                 // 64-column value slices
    int nwg;                 // workgroups = B * H * ndv
};

// LDS bytes of one workgroup (fp32 or fp16 operands, Dk).
uint32_t lds_bytes(bool f32, int dk);
hipError_t launch(const DeltaArgs &a, bool f32, int dk, hipStream_t st);

}  // namespace gla_delta
