// gla_layout.h -- sizes shared by the host planner and the gfx950 kernels.
//
// One workgroup = 4 waves of 64 lanes.  A workgroup owns one (batch, head), one sequence
// segment and one 64-column slice of the value dimension; wave w owns 16 of those columns.
// Tokens are processed in 64-token tiles (a chunk of C > 64 tokens is C/64 tiles, the
// tiled large-chunk scheme of Tiled Flash Linear Attention, abstract); key channels are
// processed in slabs of 64 lanes x CPL channels.
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define GLA_HD __host__ __device__
#else
#define GLA_HD
#endif

namespace gla {

constexpr int kTile = 64;       // tokens per tile
constexpr int kThreads = 256;   // 4 waves
constexpr int kDvTile = 64;     // value columns per workgroup
constexpr int kMaxChunk = 512;  // largest chunk size
constexpr uint32_t kMaxLds = 160u * 1024u;  // LDS per CU on gfx950

// Channels handled by one lane in a slab: 2 for 16-bit operands and Dk >= 128, else 1.
GLA_HD inline int chan_per_lane(int opb, int dk) { return (opb == 2 && dk >= 128) ? 2 : 1; }

// Byte offsets of the workgroup's LDS arrays (dynamic shared memory).
struct LdsPlan {
    uint32_t q;      // [nq][64][rp] q scaled to its 16-token block start (per-channel gate) or raw q (scalar);
                     //              nq = slabs when a chunk has several tiles, else 1
    uint32_t k;      // [64][rp]     k scaled to its block end (per-channel) or raw k (scalar)
    uint32_t kd;     // [64][rp]     k scaled to its block start: key operand of diagonal blocks (per-channel)
    uint32_t x;      // [32][rp]     block-0 keys and block-3 queries referenced to the end of block 1 (per-channel)
    uint32_t qi;     // [64][rp]     q scaled to the chunk start
    uint32_t kst;    // [slab][ktp]  k scaled to the tile end, transposed, in MFMA k-slot order
    uint32_t pbuf;   // [4][2][64][8] masked score tile, MFMA A-operand order
    uint32_t vb;     // [2][4][64][8] value tile, MFMA B-operand order
    uint32_t voff;   // same, value tile of an earlier key tile (several tiles per chunk)
    uint32_t ablk;   // [4][slab] fp32 decay across each 16-token block (per-channel)
    uint32_t qtf;    // [4][dk]   fp32 decay from the tile start to each block start (per-channel, several tiles)
    uint32_t atile;  // [nt][dk]  fp32 decay across each tile of the chunk (per-channel)
    uint32_t aseg;   // [dk]      fp32 decay across the segment (segment-state kernel)
    uint32_t brow;   // [nt*64]   fp32 log2 running decay from the chunk start (scalar gates)
    uint32_t lrow;   // [nt*64]   fp32 log2 input gate (scalar gates)
    uint32_t total;
};

GLA_HD inline LdsPlan lds_plan(int opb, int dk, bool per_channel, int nt) {
    const int cpl = chan_per_lane(opb, dk);
    const int slab = 64 * cpl;
    const int nslab = dk / slab;
    const int rp = slab + 16 / opb;
    const int ktp = 64 + 16 / opb;
    const uint32_t a64 = 64u * (uint32_t)rp * (uint32_t)opb;
    const bool mt = nt > 1;
    uint32_t off = 0;
    LdsPlan p{};
#define GLA_TAKE(field, bytes)                      \
    do {                                            \
        p.field = off;                              \
        off += ((uint32_t)(bytes) + 255u) & ~255u;  \
    } while (0)
    GLA_TAKE(q, a64 * (uint32_t)(mt ? nslab : 1));
    GLA_TAKE(k, a64);
    if (per_channel) {
        GLA_TAKE(kd, a64);
        GLA_TAKE(x, a64 / 2);
    }
    GLA_TAKE(qi, a64);
    GLA_TAKE(kst, (uint32_t)slab * (uint32_t)ktp * (uint32_t)opb);
    GLA_TAKE(pbuf, 4096u * (uint32_t)opb);
    GLA_TAKE(vb, 4096u * (uint32_t)opb);
    if (mt) GLA_TAKE(voff, 4096u * (uint32_t)opb);
    if (per_channel) {
        GLA_TAKE(ablk, 4u * slab * 4u);
        if (mt) GLA_TAKE(qtf, 4u * dk * 4u);
    }
    GLA_TAKE(atile, (uint32_t)nt * (uint32_t)(per_channel ? dk : 1) * 4u);
    GLA_TAKE(aseg, (uint32_t)dk * 4u);
    GLA_TAKE(brow, (uint32_t)nt * 64u * 4u);
    GLA_TAKE(lrow, (uint32_t)nt * 64u * 4u);
#undef GLA_TAKE
    p.total = off;
    return p;
}

// LDS of the segment-state kernel: keys^T scaled to the tile end and the value tile of one
// slab, the per-channel block and tile decays, and the running decay across the segment.
struct LdsPlanState {
    uint32_t kst, vb, ablk, atile, aseg, total;
};

GLA_HD inline LdsPlanState lds_plan_state(int opb, int dk) {
    const int slab = 64 * chan_per_lane(opb, dk);
    const int ktp = 64 + 16 / opb;
    auto al = [](uint32_t x) { return (x + 255u) & ~255u; };
    LdsPlanState p{};
    uint32_t off = 0;
    p.kst = off;
    off += al((uint32_t)slab * (uint32_t)ktp * (uint32_t)opb);
    p.vb = off;
    off += al(4096u * (uint32_t)opb);
    p.ablk = off;
    off += al(4u * (uint32_t)slab * 4u);
    p.atile = off;
    off += al((uint32_t)dk * 4u);
    p.aseg = off;
    off += al((uint32_t)dk * 4u);
    p.total = off;
    return p;
}

// LDS of the warp-specialised chunk-output kernel (64-token chunks, one slab): four
// producer waves prepare chunk k+1 while four consumer waves run the matrix products of
// chunk k.  Arrays read by the consumers only before the mid-iteration barrier are single
// (q, k); arrays read after it are double-buffered by chunk parity.
// Rows of the operand-precision gate factors of the warp-specialised kernel (a_u = decay
// across 16-token block u of the tile, per channel).
enum : int {
    kFhA0 = 0,    // a_0
    kFhA1 = 1,    // a_1
    kFhA2 = 2,    // a_2
    kFhA12 = 3,   // a_1 a_2
    kFhInv = 4,   // rows 4 + u: 1 / a_u, 0 for channels whose block u is handled exactly
    kFhP2 = 8,    // a_0 a_1
    kFhP3 = 9,    // a_0 a_1 a_2
    kFhRows = 10
};

struct LdsPlanWs {
    uint32_t q, k;  // [64][rp], channels in the chperm order: inside each double buffer (fp16
                    // operands, qkd = 1) or single buffers at the front (fp32 operands)
    uint32_t qkd;
    // double-buffered block: buffer b starts at dbl + b * dstride; offsets inside a buffer:
    uint32_t dbl, dstride;
    uint32_t kst;   // [slab][ktp]
    uint32_t vb;    // [4096] value tile
    uint32_t ab;    // [4][slab] fp32 decay across each 16-token block, channels in chperm order (per-channel); [64] log2 running
                    //           decay of each row (scalar gates)
    uint32_t ainv;  // fp32 operands: [4][slab] 1/decay of each block, 0 for channels handled exactly, chperm order
                    //           (per-channel); [64] log2 input gate of each row (scalar gates)
    uint32_t at;    // [slab] fp32 decay across the tile (per-channel)
    uint32_t xact;  // [4 blocks][136] fp32 exact diagonal-block partial scores
    uint32_t xflag; // [4] int32: partial present (right after xact)
    uint32_t fh;    // [10][slab] per-channel gate factors in operand precision, chperm order:
                    //           rows kFh* below
    uint32_t pbuf;  // [4096] masked score tile
    uint32_t ostage;  // [64][68] fp32 output tile, staged for whole-row stores
    uint32_t total;
};

GLA_HD inline LdsPlanWs lds_plan_ws(int opb, int dk) {
    const int cpl = chan_per_lane(opb, dk);
    const int slab = 64 * cpl;
    const int rp = slab + 16 / opb;
    const int ktp = 64 + 16 / opb;
    const uint32_t a64 = 64u * (uint32_t)rp * (uint32_t)opb;
    auto al = [](uint32_t x) { return (x + 255u) & ~255u; };
    LdsPlanWs p{};
    // fp16 operands: q and k double-buffered (the producers write a chunk's rows while the
    // consumers read the previous chunk's), which fills the 160 KB exactly for Dk = 128
    p.qkd = opb == 2 ? 1u : 0u;
    uint32_t off = 0, in = 0;
    uint32_t &qk = p.qkd ? in : off;
    p.q = qk;
    qk += al(a64);
    p.k = qk;
    qk += al(a64);
    p.kst = in;
    in += al((uint32_t)slab * (uint32_t)ktp * (uint32_t)opb);
    p.vb = in;
    in += al(4096u * (uint32_t)opb);
    p.ab = in;
    in += al(4u * (uint32_t)slab * 4u);
    p.ainv = in;
    in += al(p.qkd ? 64u * 4u : 4u * (uint32_t)slab * 4u);
    p.at = in;
    in += al((uint32_t)slab * 4u);
    p.xact = in;
    p.xflag = in + 4u * 136u * 4u;
    in += al(4u * 136u * 4u + 4u * 4u);
    p.fh = in;
    in += al((uint32_t)kFhRows * (uint32_t)slab * (uint32_t)opb);
    p.dbl = off;
    p.dstride = in;
    off += 2u * in;
    p.pbuf = off;
    off += al(4096u * (uint32_t)opb);
    p.ostage = off;
    off += al(64u * 68u * 4u);
    p.total = off;
    return p;
}

// The warp-specialised kernel runs every 64-token-chunk case whose key channels fit one
// slab (bf16 with Dk <= 128, fp32 with Dk = 64); the launcher makes the same choice.
GLA_HD inline bool use_ws_kernel(int opb, int dk, int nt) { return nt == 1 && dk == 64 * chan_per_lane(opb, dk); }

// LDS of the scalar-gate warp-specialised kernel (bf16 inputs, 64-token chunks, Dk = 256).
// q, k and the scaled keys^T are single buffers (consumers read them before the mid-tile
// barrier); values and row decays are double-buffered by tile parity.
struct LdsPlanSg {
    uint32_t q;     // [2][64][dk + 8] fp16 q, channels permuted inside 32-channel groups
    uint32_t kst;   // [dk][96] fp16 keys, transposed, k-slot order, 16-byte units swizzled by row
    uint32_t vb;    // [2][4096] fp16 value tiles
    uint32_t rows;  // [2][192] fp32: log2 running decay of each row, log2 input gate, key weight
    uint32_t pbuf;  // [4096] fp16 masked scores
    uint32_t ostage;  // [64][68] fp32 output tile, staged for whole-row stores
    uint32_t total;
};

GLA_HD inline LdsPlanSg lds_plan_sg(int dk) {
    auto al = [](uint32_t x) { return (x + 255u) & ~255u; };
    LdsPlanSg p{};
    uint32_t off = 0;
    p.q = off;
    off += al(2u * 64u * (uint32_t)(dk + 8) * 2u);
    p.kst = off;
    off += al((uint32_t)dk * 96u * 2u);
    p.vb = off;
    off += al(2u * 4096u * 2u);
    p.rows = off;
    off += al(2u * 192u * 4u);
    p.pbuf = off;
    off += al(4096u * 2u);
    p.ostage = off;
    off += al(64u * 68u * 4u);
    p.total = off;
    return p;
}

// The scalar-gate kernel runs bf16 inputs with Dk = 256, 64-token tiles and no per-channel
// gate; the launcher makes the same choice.
GLA_HD inline bool use_sg_kernel(int opb, int dk, int nt, bool per_channel) {
    return opb == 2 && nt == 1 && dk == 256 && !per_channel;
}

// Global scratch per chunk-output workgroup: keys of the earlier tiles of the current chunk
// scaled to their tile end (per-channel gate with several tiles per chunk), [nt-1][64][dk].
GLA_HD inline uint64_t ke_scratch_bytes(int opb, int dk, bool per_channel, int nt) {
    return (per_channel && nt > 1) ? (uint64_t)(nt - 1) * 64u * (uint64_t)dk * (uint64_t)opb : 0u;
}

// Arguments of the three kernels.
struct KArgs {
    const void *q, *k, *v;
    const float *la, *li, *s0;
    float *out, *fin;
    float *ws_state;  // [BH][(nseg-1)*nsub][Dk][Dv]: local sub-segment states; the scan writes the
                      // state entering segment s over entry s*nsub-1
    float *ws_decay;  // [BH][(nseg-1)*nsub][Dk]: decay across each sub-segment
    void *ws_ke;      // [slots][nt-1][64][Dk] operand scratch (per-channel gate, several tiles per
                      // chunk): one slot per workgroup, or per (batch, head, chunk) with qsplit
    int B, H, L, Dv;
    int chunk, nt;    // chunk size as the kernels run it and its 64-token tiles
    int qsplit;       // > 1: one workgroup per query tile of a chunk (each chunk its own segment)
    int gate;         // enum gla_gate
    int seg_len;      // tokens per segment (a multiple of the chunk size)
    int nseg, ndv;    // segments; 64-column value tiles
    int nsub;         // sub-segments per segment in the segment-state kernel
    int nwg;          // workgroups of the launch (for the XCD-aware remap)
    // Output mapping of the backward pass's instances (fp16 operands; ignored elsewhere):
    // row t is stored at row L-1-t when out_rev, times 1/s with s the scale of out_mx[bh]
    // (when non-null) and times exp(out_li[bh][destination row]) (when non-null).
    int out_rev;
    const float *out_li;
    const uint32_t *out_mx;
    int in_rev;       // token t reads q, k, v row L-1-t and a per-channel gate's row L-t (zero
                      // for t = 0); scalar gates are given in the pass's token order
    int out_acc;      // backward-pass instances: add the mapped rows to the output instead of
                      // storing them (a pass split over value columns sums its halves)
    // Backward dq and dk passes (instances with a scalar gate and an fp16 q or k operand):
    // for each stored row, its dot product with the same row of dot_src (bf16 [BH][L][Dv] in
    // sequence order: q for the dq pass, k for the dk pass) over the workgroup's 64 columns,
    // into dot_out[dvt][bh][row] (dot_out null: none).
    const void *dot_src;
    float *dot_out;
    // Segment-entry states given: entry s*nsub-1 of ws_state already holds the state entering
    // segment s (prepared by the caller); the segment-state kernel and the scan do not run.
    int state_t;
    // Backward instances of the Dk = 256 scalar-gate kernel: elements between consecutive rows
    // of q and k (0: Dk), so a pass reads a column half of wider rows in place.
    int qk_stride;
};

#if defined(__HIPCC__)
// Power-of-two scale of the backward pass's output gradient from the bit pattern of its
// largest magnitude m: s = 2^(2 - e) for m in [2^e, 2^(e+1)), so that m s lies in [4, 8);
// the exponent of s is kept in [-126, 126] (m zero or subnormal: 2^126; m infinite or NaN:
// 2^-126).
__device__ inline float grad_scale_of(uint32_t mbits) {
    const int e = (int)((mbits >> 23) & 0xffu) - 127;
    int x = 2 - e;
    x = x < -126 ? -126 : (x > 126 ? 126 : x);
    return __uint_as_float((uint32_t)(127 + x) << 23);
}
#endif

}  // namespace gla
