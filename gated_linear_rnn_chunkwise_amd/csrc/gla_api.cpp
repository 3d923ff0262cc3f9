// gla_api.cpp -- the C ABI declared in gla.h: argument validation, launch planning,
// workspace handling and dispatch to the gfx950 kernels.
//
// Validation runs entirely on the host before any HIP call, so every error path can be
// exercised without a GPU.  Planning picks how many sequence segments to process in
// parallel: when (batch x heads x value tiles) already fills the GPU the sequence is one
// segment and no state is written to memory; otherwise the sequence is cut into segments
// whose boundary states are formed by a state kernel and joined by a scan.  This is the
// trade of memory movement against parallelism named in the GLA abstract (Gated Linear
// Attention Transformers with Hardware-Efficient Training), and sequence-level
// parallelism for small batches (talk summary, 59:59).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "gla.h"
#include "gla_delta.h"
#include "gla_mlstm.h"
#include "gla_layout.h"

namespace gla {
hipError_t launch_forward(const KArgs &a, bool f32, int h16, int dk, hipStream_t st);
hipError_t launch_step(const gla_step_desc &d, hipStream_t st);
hipError_t bwd_reverse(const void *src, int dt, float *dst, int BH, int L, int D, hipStream_t st);
hipError_t bwd_gate(const float *la, int kind, float *dst, int BH, int H, int L, hipStream_t st);
hipError_t bwd_transpose(const float *src, const uint32_t *mx, float *dst, int BH, int R, int C, hipStream_t st);
hipError_t bwd_transpose_entries(float *ws, int BH, int N, int nseg, int nsub, hipStream_t st);
size_t bwd_absmax_parts(int L, int Dv, int Dk, bool dfin);
hipError_t bwd_dout16(const float *dout, const float *dfin, float *part, uint32_t *mx, _Float16 *fwd, _Float16 *rev,
                      int BH, int L, int Dv, int Dk, hipStream_t st);
hipError_t bwd_scale(const float *src, const uint32_t *mx, float *dst, int BH, size_t m, hipStream_t st);
hipError_t bwd_copy2d(const void *src, size_t src_stride, void *dst, size_t dst_stride, size_t rows, size_t row_bytes,
                      hipStream_t st);
hipError_t bwd_finish(const gla_bwd_desc &d, const float *oA, const float *oB, float *g, const float *finA,
                      const float *finC, const float *dfT, float *part, const uint32_t *mx, const float *dqp,
                      const float *dkp, hipStream_t st);
constexpr int kH16Q = 1, kH16K = 2, kH16V = 4;  // fp16 operand bits of launch_forward
size_t chan_scratch_floats(int BH, int L, int Dk, int Dv, bool g_rows);
hipError_t chan_backward(const gla_bwd_desc &d, const float *s0T, const float *dfT, float *finA, float *finC,
                         float *scratch, bool skip_dv, const _Float16 *fdo, const uint32_t *mx, hipStream_t st);
}

namespace {

constexpr int kTargetWorkgroups = 256;     // one per compute unit on MI355X
// The segment-state kernel fits three workgroups per compute unit.  Its state grid is aimed at
// about three per CU for scalar gates and two per CU for per-channel gates, whose gate work
// per tile is heavier (measured on the RetNet and long-sequence GLA workloads: 3-4% apart).
constexpr int kTargetStateWorkgroups = 768;
constexpr int kTargetStateWorkgroupsChannel = 512;
// A walk of at most this many 64-token tiles runs as one segment: the segment-state kernel and
// the scan cost about as much as they save there (measured at L = 1024, B*H = 1..32).  Longer
// walks with fewer than kTargetWorkgroups workgroups are always split: one workgroup walking
// 1,024 tiles took 2.46 ms where 128 segments took 0.095 ms.
constexpr int kShortWalkTiles = 16;

struct Plan {
    int nt, nc, ndv, seg_chunks, nseg, seg_len, nsub;
    int knt;  // 64-token tiles per chunk as the kernels run it: nt with tile pairs, else 1
    int qsplit;  // workgroups per chunk and value tile: knt with query tiles, else 1
    int grid_state, grid_scan, grid_out;
    size_t ws_state_bytes, ws_decay_bytes, ws_ke_bytes, ws_bytes;
    uint32_t lds_out, lds_state;
};

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t align256(size_t x) { return (x + 255u) & ~size_t(255u); }

// An empty call (B, H or L zero) has no output rows, and the state after no tokens is the
// state before them.  Its per-token arrays may be NULL.
inline bool empty_call(int64_t B, int64_t H, int64_t L) { return B == 0 || H == 0 || L == 0; }

// dst[i] = src[i], or 0 without src, for i < n: the final state of an empty sequence.
__global__ __launch_bounds__(256) void state_copy_kernel(float *dst, const float *src, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        dst[i] = src ? src[i] : 0.f;
}
int state_copy(float *dst, const float *src, size_t n, void *stream) {
    if (!dst || n == 0) return GLA_OK;
    const size_t blocks = std::min<size_t>((n + 255) / 256, 65536);
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       dst, src, n);
    return hipGetLastError() == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

// Argument checks (no HIP call).  Returns GLA_OK or an error status.
int validate(const gla_desc *d) {
    if (!d) return GLA_ERR_INVALID_ARG;
    if (d->B < 0 || d->H < 0 || d->L < 0 || d->Dk <= 0 || d->Dv <= 0 || d->chunk <= 0) return GLA_ERR_INVALID_ARG;
    const bool empty = empty_call(d->B, d->H, d->L);
    if (!empty && (!d->q || !d->k || !d->v || !d->out)) return GLA_ERR_INVALID_ARG;
    if (d->seg_chunks < 0 || (d->flags & ~int32_t(GLA_FLAG_TILE_PAIRS | GLA_FLAG_QUERY_TILES)) != 0)
        return GLA_ERR_INVALID_ARG;
    // query tiles make every chunk its own segment
    if ((d->flags & GLA_FLAG_QUERY_TILES) && d->seg_chunks > 1) return GLA_ERR_INVALID_ARG;
    if (d->in_dtype != GLA_DTYPE_BF16 && d->in_dtype != GLA_DTYPE_F32) return GLA_ERR_INVALID_ARG;
    if (d->gate_kind < GLA_GATE_NONE || d->gate_kind > GLA_GATE_HEAD_CONST) return GLA_ERR_INVALID_ARG;
    if (!empty && (d->gate_kind == GLA_GATE_NONE) != (d->log_alpha == nullptr)) return GLA_ERR_INVALID_ARG;
    const void *ptrs[] = {d->q, d->k, d->v, d->out, d->log_alpha, d->log_ig, d->initial_state, d->final_state,
                          d->workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GLA_ERR_INVALID_ARG;
    if (d->workspace && d->workspace_bytes == 0) return GLA_ERR_INVALID_ARG;
    // size products in int64 with headroom: element counts must stay below 2^40
    const int64_t lim = int64_t(1) << 40;
    const int64_t bh = int64_t(d->B) * d->H;
    if (bh > (int64_t(1) << 24)) return GLA_ERR_INVALID_ARG;
    if (bh * d->L > lim / std::max(d->Dk, d->Dv)) return GLA_ERR_INVALID_ARG;
    if (bh * int64_t(d->Dk) * d->Dv > lim) return GLA_ERR_INVALID_ARG;
    return GLA_OK;
}

// Support matrix and launch plan.  Returns GLA_OK, GLA_ERR_UNSUPPORTED.
int make_plan(const gla_desc *d, Plan *p) {
    if (empty_call(d->B, d->H, d->L)) return GLA_ERR_INVALID_ARG;  // entry points handle empty calls first
    if (d->Dk != 64 && d->Dk != 128 && d->Dk != 256) return GLA_ERR_UNSUPPORTED;
    if (d->Dv % gla::kDvTile != 0 || d->Dv > 4096) return GLA_ERR_UNSUPPORTED;
    // Chunks of 16 and 32 tokens run as 64-token tiles: the state is carried per tile, which
    // is the same map (the chunkwise form is exact for every chunk size).
    if (d->chunk != 16 && d->chunk != 32 && (d->chunk % gla::kTile != 0 || d->chunk > gla::kMaxChunk))
        return GLA_ERR_UNSUPPORTED;
    const int chunk = d->chunk < gla::kTile ? gla::kTile : d->chunk;
    // Kernels address one (batch, head) slice through a buffer resource with 32-bit byte
    // offsets, and prefetch up to two chunks past the segment end.
    if ((int64_t(d->L) + 2 * gla::kMaxChunk) * std::max(d->Dk, d->Dv) * 4 >= (int64_t(1) << 32))
        return GLA_ERR_UNSUPPORTED;
    const bool f32 = d->in_dtype == GLA_DTYPE_F32;
    const bool ch = d->gate_kind == GLA_GATE_CHANNEL;
    p->nt = chunk / gla::kTile;
    // Without tile pairs the state is advanced tile by tile: the kernels walk 64-token chunks.
    const bool qtiles = (d->flags & GLA_FLAG_QUERY_TILES) != 0;
    p->knt = (d->flags & (GLA_FLAG_TILE_PAIRS | GLA_FLAG_QUERY_TILES)) ? p->nt : 1;
    p->qsplit = qtiles ? p->knt : 1;
    p->nc = (d->L + chunk - 1) / chunk;
    p->ndv = d->Dv / gla::kDvTile;
    const int64_t bh = int64_t(d->B) * d->H;
    const int64_t wg1 = bh * p->ndv;
    int sc;
    if (qtiles) {
        sc = 1;  // the chunk-start states are materialised by the segment-state kernel and scan
    } else if (d->seg_chunks > 0) {
        sc = std::min(d->seg_chunks, p->nc);
    } else if (wg1 >= kTargetWorkgroups || (int64_t(d->L) + gla::kTile - 1) / gla::kTile <= kShortWalkTiles) {
        sc = p->nc;
    } else {
        const int64_t want = (kTargetWorkgroups + wg1 - 1) / wg1;
        const int64_t nseg = std::min<int64_t>(want, p->nc);
        sc = (int)((p->nc + nseg - 1) / nseg);
    }
    p->seg_chunks = sc;
    p->nseg = (p->nc + sc - 1) / sc;
    p->seg_len = sc * chunk;
    // Segment boundary states are sums of sub-segment states, computed by more workgroups
    // than there are boundaries: nsub (sub-segments of a segment, whose tile counts differ
    // by at most one) brings the state grid nearest to its target.
    p->nsub = 1;
    if (p->nseg > 1) {
        const int64_t base = bh * (p->nseg - 1) * p->ndv;
        const int tiles = p->seg_len / gla::kTile;
        const int64_t target = ch ? kTargetStateWorkgroupsChannel : kTargetStateWorkgroups;
        const int64_t want = (target + base / 2) / base;
        p->nsub = (int)std::max<int64_t>(1, std::min<int64_t>(want, tiles));
    }
    const int64_t nss = int64_t(p->nseg - 1) * p->nsub;
    const int64_t g3 = bh * p->nseg * p->ndv * p->qsplit;
    const int64_t g1 = p->nseg > 1 ? bh * nss * p->ndv : 0;
    if (g3 > INT32_MAX || g1 > INT32_MAX) return GLA_ERR_UNSUPPORTED;
    p->grid_out = (int)g3;
    p->grid_state = (int)g1;
    p->grid_scan = p->nseg > 1 ? (int)(bh * ((int64_t(d->Dk) * d->Dv + 1023) / 1024)) : 0;
    const int opb = f32 ? 4 : 2;
    if (gla::use_sg_kernel(opb, d->Dk, p->knt, ch))
        p->lds_out = gla::lds_plan_sg(d->Dk).total;
    else if (gla::use_ws_kernel(opb, d->Dk, p->knt))
        p->lds_out = gla::lds_plan_ws(opb, d->Dk).total;
    else
        p->lds_out = gla::lds_plan(opb, d->Dk, ch, p->knt).total;
    p->lds_state = gla::lds_plan_state(opb, d->Dk).total;
    if (p->lds_out > gla::kMaxLds || p->lds_state > gla::kMaxLds) return GLA_ERR_UNSUPPORTED;
    p->ws_state_bytes = align256(size_t(bh) * size_t(nss) * size_t(d->Dk) * size_t(d->Dv) * 4u);
    p->ws_decay_bytes = align256(size_t(bh) * size_t(nss) * size_t(d->Dk) * 4u);
    if (p->nseg <= 1) p->ws_state_bytes = p->ws_decay_bytes = 0;
    // key scratch: one slot per output workgroup, or per (batch, head, chunk) with query tiles
    const int64_t ke_slots = p->qsplit > 1 ? bh * p->nseg : g3;
    p->ws_ke_bytes = align256(size_t(ke_slots) * (size_t)gla::ke_scratch_bytes(opb, d->Dk, ch, p->knt));
    p->ws_bytes = p->ws_state_bytes + p->ws_decay_bytes + p->ws_ke_bytes;
    return GLA_OK;
}

int checked_plan(const gla_desc *d, Plan *p) {
    const int st = validate(d);
    if (st != GLA_OK) return st;
    return make_plan(d, p);
}

// The kernels take Dk in {64, 128, 256} and Dv a multiple of 64.  The forward entry points
// also take any other Dk that is a multiple of 16 up to 256 and any other Dv that is a
// multiple of 16 up to 4096, through zero-padded copies in the workspace: the padded key and
// query channels are zero (their state rows stay zero and add nothing to the outputs, and a
// per-channel gate is padded with log decay 0), and the padded value columns are dropped.
bool native_shape(const gla_desc *d) {
    return (d->Dk == 64 || d->Dk == 128 || d->Dk == 256) && d->Dv % gla::kDvTile == 0;
}
constexpr size_t kNotPadded = ~size_t(0);
struct PadPlan {
    gla_desc inner;  // the padded call (pointers are set when it runs)
    Plan plan;       // its launch plan
    size_t q, k, v, la, s0, out, fin, ws;  // workspace offsets, or kNotPadded
    size_t total;    // workspace bytes: padded copies plus the padded call's own workspace
};
int pad_plan(const gla_desc *d, PadPlan *pp) {
    if (d->Dk % 16 != 0 || d->Dk > 256 || d->Dv % 16 != 0 || d->Dv > 4096) return GLA_ERR_UNSUPPORTED;
    const size_t eb = d->in_dtype == GLA_DTYPE_F32 ? 4 : 2;
    const int dkp = d->Dk <= 64 ? 64 : (d->Dk <= 128 ? 128 : 256);
    const int dvp = (d->Dv + gla::kDvTile - 1) / gla::kDvTile * gla::kDvTile;
    gla_desc in = *d;
    in.Dk = dkp;
    in.Dv = dvp;
    in.workspace = nullptr;
    in.workspace_bytes = 0;
    const int st = checked_plan(&in, &pp->plan);
    if (st != GLA_OK) return st;
    pp->inner = in;
    const size_t bh = size_t(d->B) * d->H, bhl = bh * size_t(d->L);
    const bool pk = dkp != d->Dk, pv = dvp != d->Dv;
    size_t off = 0;
    const auto take = [&](bool need, size_t bytes) {
        if (!need) return kNotPadded;
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    pp->q = take(pk, bhl * dkp * eb);
    pp->k = take(pk, bhl * dkp * eb);
    pp->v = take(pv, bhl * dvp * eb);
    pp->la = take(pk && d->gate_kind == GLA_GATE_CHANNEL, bhl * dkp * 4);
    pp->s0 = take(d->initial_state != nullptr, bh * dkp * dvp * 4);
    pp->out = take(pv, bhl * dvp * 4);
    pp->fin = take(d->final_state != nullptr, bh * dkp * dvp * 4);
    pp->ws = take(pp->plan.ws_bytes > 0, pp->plan.ws_bytes);
    pp->total = off;
    return GLA_OK;
}

}  // namespace

// The support check of an empty call: the same shape with one token of one (batch, head).
int empty_support(const gla_desc *d) {
    gla_desc one = *d;
    one.B = one.H = one.L = 1;
    const void *x = reinterpret_cast<const void *>(uintptr_t(256));
    float *y = reinterpret_cast<float *>(uintptr_t(256));
    one.q = one.k = one.v = x;
    one.out = y;
    one.log_alpha = d->gate_kind == GLA_GATE_NONE ? nullptr : y;
    one.log_ig = d->log_ig ? y : nullptr;
    one.workspace = nullptr;
    one.workspace_bytes = 0;
    if (native_shape(&one)) {
        Plan p;
        return make_plan(&one, &p);
    }
    PadPlan pp;
    return pad_plan(&one, &pp);
}

// An empty forward call: the final state (when asked for) is the initial state, or zero.
int fwd_empty(const gla_desc *d, void *stream) {
    const int st = empty_support(d);
    if (st != GLA_OK) return st;
    if (d->L != 0) return GLA_OK;  // no (batch, head) slices
    return state_copy(d->final_state, d->initial_state, size_t(d->B) * d->H * d->Dk * d->Dv, stream);
}

extern "C" {

int gla_version(void) { return GLA_VERSION; }

const char *gla_status_string(int status) {
    switch (status) {
        case GLA_OK: return "ok";
        case GLA_ERR_INVALID_ARG: return "invalid argument";
        case GLA_ERR_UNSUPPORTED: return "unsupported configuration";
        case GLA_ERR_WORKSPACE: return "workspace too small or allocation failed";
        case GLA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int gla_workspace_size(const gla_desc *d, size_t *bytes) {
    if (!bytes) return GLA_ERR_INVALID_ARG;
    int st = validate(d);
    if (st != GLA_OK) return st;
    if (empty_call(d->B, d->H, d->L)) {
        if ((st = empty_support(d)) != GLA_OK) return st;
        *bytes = 0;
        return GLA_OK;
    }
    if (!native_shape(d)) {
        PadPlan pp;
        if ((st = pad_plan(d, &pp)) != GLA_OK) return st;
        *bytes = pp.total;
        return GLA_OK;
    }
    Plan p;
    if ((st = make_plan(d, &p)) != GLA_OK) return st;
    *bytes = p.ws_bytes;
    return GLA_OK;
}

int gla_query_plan(const gla_desc *d, gla_plan *out) {
    if (!out) return GLA_ERR_INVALID_ARG;
    int st = validate(d);
    if (st != GLA_OK) return st;
    if (empty_call(d->B, d->H, d->L)) {
        if ((st = empty_support(d)) != GLA_OK) return st;
        *out = gla_plan{};  // nothing runs
        return GLA_OK;
    }
    Plan p;
    size_t ws_total = 0;
    if (!native_shape(d)) {
        PadPlan pp;
        if ((st = pad_plan(d, &pp)) != GLA_OK) return st;
        p = pp.plan;
        ws_total = pp.total;
    } else {
        if ((st = make_plan(d, &p)) != GLA_OK) return st;
        ws_total = p.ws_bytes;
    }
    out->seg_chunks = p.seg_chunks;
    out->n_seg = p.nseg;
    out->dv_tiles = p.ndv;
    out->tiles_per_chunk = p.nt;
    out->grid_state = p.grid_state;
    out->grid_scan = p.grid_scan;
    out->grid_out = p.grid_out;
    out->tile_pairs = p.knt > 1 ? 1 : 0;
    out->query_tiles = p.qsplit > 1 ? 1 : 0;
    out->workspace_bytes = ws_total;
    return GLA_OK;
}

}  // extern "C"

namespace {

// Output mapping of a backward pass (KArgs::out_rev, out_li, out_mx).
struct OutMapArgs {
    int rev = 0;
    const float *li = nullptr;
    const uint32_t *mx = nullptr;
    int in_rev = 0;  // the pass reads q, k, v in reversed token order
    int acc = 0;     // add to the output instead of storing
    const void *dot_src = nullptr;  // dq and dk passes: rows to dot with the stored rows
    float *dot_out = nullptr;       // [Dv/64][BH][L] dot products per 64-column tile
    int state_t = 0;  // the workspace already holds the segment-entry states, transposed
    int qk_stride = 0;  // elements between rows of the pass's q and k (0: its Dk)
};

// The forward pass; h16 marks operands given as fp16 instead of bf16 and om maps the output
// rows (backward passes only).
int fwd_run(const gla_desc *d, int h16, void *stream, const OutMapArgs &om = OutMapArgs()) {
    Plan p;
    const int st = checked_plan(d, &p);
    if (st != GLA_OK) return st;
    if (d->workspace && d->workspace_bytes < p.ws_bytes) return GLA_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    void *ws = nullptr;
    bool owned = false;
    if (p.ws_bytes > 0) {
        if (d->workspace) {
            ws = d->workspace;
        } else {
            if (hipMallocAsync(&ws, p.ws_bytes, s) != hipSuccess || !ws) {
                (void)hipGetLastError();
                return GLA_ERR_WORKSPACE;
            }
            owned = true;
        }
    }

    gla::KArgs a{};
    a.q = d->q;
    a.k = d->k;
    a.v = d->v;
    a.la = d->log_alpha;
    a.li = d->log_ig;
    a.s0 = d->initial_state;
    a.out = d->out;
    a.fin = d->final_state;
    a.ws_state = ws ? reinterpret_cast<float *>(ws) : nullptr;
    a.ws_decay = ws ? reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + p.ws_state_bytes) : nullptr;
    a.ws_ke = ws ? reinterpret_cast<char *>(ws) + p.ws_state_bytes + p.ws_decay_bytes : nullptr;
    a.B = d->B;
    a.H = d->H;
    a.L = d->L;
    a.Dv = d->Dv;
    a.chunk = gla::kTile * p.knt;
    a.nt = p.knt;
    a.qsplit = p.qsplit;
    a.gate = d->gate_kind;
    a.seg_len = p.seg_len;
    a.nseg = p.nseg;
    a.nsub = p.nsub;
    a.ndv = p.ndv;
    a.nwg = p.grid_out;
    a.out_rev = om.rev;
    a.out_li = om.li;
    a.out_mx = om.mx;
    a.in_rev = om.in_rev;
    a.out_acc = om.acc;
    a.dot_src = om.dot_src;
    a.dot_out = om.dot_out;
    a.state_t = om.state_t;
    a.qk_stride = om.qk_stride;
    if (om.state_t && (!d->workspace || p.nseg < 2)) return GLA_ERR_INVALID_ARG;

    const hipError_t err = gla::launch_forward(a, d->in_dtype == GLA_DTYPE_F32, h16, d->Dk, s);
    if (owned) (void)hipFreeAsync(ws, s);
    return err == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

// Zero-filling copy in 16-byte units: dst[g][r][u] = src[g][r][u] for r < s_rows and
// u < s_units, else 0, for groups g of d_rows rows of d_units units (the destination may be
// wider or narrower than the source in either dimension).
__global__ __launch_bounds__(256) void pad_copy_kernel(const uint4 *src, uint32_t s_units, uint32_t s_rows, uint4 *dst,
                                                       uint32_t d_units, uint32_t d_rows, uint64_t n) {
    for (uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x; i < n; i += (uint64_t)gridDim.x * 256u) {
        const uint32_t u = (uint32_t)(i % d_units);
        const uint64_t rg = i / d_units;
        const uint32_t r = (uint32_t)(rg % d_rows);
        const uint64_t g = rg / d_rows;
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (u < s_units && r < s_rows) x = src[(g * s_rows + r) * s_units + u];
        dst[i] = x;
    }
}
bool pad_copy(const void *src, size_t s_row_bytes, size_t s_rows, void *dst, size_t d_row_bytes, size_t d_rows,
              size_t groups, hipStream_t st) {
    const uint64_t n = (uint64_t)groups * d_rows * (d_row_bytes / 16);
    if (n == 0) return true;
    const uint64_t blocks = std::min<uint64_t>((n + 255) / 256, 1u << 16);
    hipLaunchKernelGGL(pad_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const uint4 *>(src),
                       (uint32_t)(s_row_bytes / 16), (uint32_t)s_rows, static_cast<uint4 *>(dst),
                       (uint32_t)(d_row_bytes / 16), (uint32_t)d_rows, n);
    return hipGetLastError() == hipSuccess;
}

// The forward pass of a shape the kernels do not take directly, on zero-padded copies (see
// pad_plan).  ws: workspace of at least pp.total bytes.
int fwd_padded(const gla_desc *d, const PadPlan &pp, char *ws, void *stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const size_t eb = d->in_dtype == GLA_DTYPE_F32 ? 4 : 2;
    const size_t bh = size_t(d->B) * d->H, bhl = bh * size_t(d->L);
    const int dkp = pp.inner.Dk, dvp = pp.inner.Dv;
    gla_desc in = pp.inner;
    const auto at = [&](size_t o) { return ws + o; };
    bool ok = true;
    if (pp.q != kNotPadded) {
        ok = ok && pad_copy(d->q, d->Dk * eb, 1, at(pp.q), dkp * eb, 1, bhl, s);
        ok = ok && pad_copy(d->k, d->Dk * eb, 1, at(pp.k), dkp * eb, 1, bhl, s);
        in.q = at(pp.q);
        in.k = at(pp.k);
    }
    if (pp.v != kNotPadded) {
        ok = ok && pad_copy(d->v, d->Dv * eb, 1, at(pp.v), dvp * eb, 1, bhl, s);
        in.v = at(pp.v);
    }
    if (pp.la != kNotPadded) {
        ok = ok && pad_copy(d->log_alpha, d->Dk * 4, 1, at(pp.la), dkp * 4, 1, bhl, s);
        in.log_alpha = reinterpret_cast<const float *>(at(pp.la));
    }
    if (pp.s0 != kNotPadded) {
        ok = ok && pad_copy(d->initial_state, d->Dv * 4, d->Dk, at(pp.s0), dvp * 4, dkp, bh, s);
        in.initial_state = reinterpret_cast<const float *>(at(pp.s0));
    }
    if (pp.out != kNotPadded) in.out = reinterpret_cast<float *>(at(pp.out));
    if (pp.fin != kNotPadded) in.final_state = reinterpret_cast<float *>(at(pp.fin));
    if (pp.ws != kNotPadded) {
        in.workspace = at(pp.ws);
        in.workspace_bytes = pp.plan.ws_bytes;
    }
    if (!ok) return GLA_ERR_HIP;
    int st = fwd_run(&in, 0, stream);
    if (st != GLA_OK) return st;
    if (pp.out != kNotPadded) ok = ok && pad_copy(at(pp.out), dvp * 4, 1, d->out, d->Dv * 4, 1, bhl, s);
    if (pp.fin != kNotPadded) ok = ok && pad_copy(at(pp.fin), dvp * 4, dkp, d->final_state, d->Dv * 4, d->Dk, bh, s);
    return ok ? GLA_OK : GLA_ERR_HIP;
}

// gla_fwd_ex for every shape: native shapes run directly, others on padded copies in a
// workspace that is the caller's or allocated stream-ordered here.
int fwd_entry(const gla_desc *d, void *stream) {
    int st = validate(d);
    if (st != GLA_OK) return st;
    if (empty_call(d->B, d->H, d->L)) return fwd_empty(d, stream);
    if (native_shape(d)) return fwd_run(d, 0, stream);
    PadPlan pp;
    if ((st = pad_plan(d, &pp)) != GLA_OK) return st;
    if (d->workspace && d->workspace_bytes < pp.total) return GLA_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    void *ws = d->workspace;
    bool owned = false;
    if (!ws && pp.total > 0) {
        if (hipMallocAsync(&ws, pp.total, s) != hipSuccess || !ws) {
            (void)hipGetLastError();
            return GLA_ERR_WORKSPACE;
        }
        owned = true;
    }
    st = fwd_padded(d, pp, static_cast<char *>(ws), stream);
    if (owned) (void)hipFreeAsync(ws, s);
    return st;
}

}  // namespace

// ------------------------------------------------------------------------------------
// Scratch of gla_fwd_noalloc: a device array built into the library.  Each GPU holds its own
// copy at its own address, resolved once per device with that device current.  In host code
// `scratch` names a host-side stand-in, never the device memory: only the resolved address
// is ever passed to a kernel.
namespace {

static __device__ __align__(256) unsigned char scratch[GLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];  // per device; nullptr until resolved (guarded by g_scratch_mu)

// Address of the current device's copy of `scratch`.
int scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return GLA_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return GLA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return GLA_ERR_HIP;
        }
        g_scratch_addr[dev] = ptr;
    }
    *out = g_scratch_addr[dev];
    return GLA_OK;
}

}  // namespace

extern "C" {

int gla_fwd_ex(const gla_desc *d, void *stream) { return fwd_entry(d, stream); }

int gla_fwd_noalloc(const gla_desc *d, void *stream) {
    int st = validate(d);
    if (st != GLA_OK) return st;
    if (d->workspace != nullptr || d->workspace_bytes != 0) return GLA_ERR_INVALID_ARG;
    if (empty_call(d->B, d->H, d->L)) return fwd_empty(d, stream);
    if (!native_shape(d)) {
        PadPlan pp;
        if ((st = pad_plan(d, &pp)) != GLA_OK) return st;
        if (pp.total > size_t(GLA_NOALLOC_SCRATCH_BYTES)) return GLA_ERR_WORKSPACE;
        void *ptr = nullptr;
        if ((st = scratch_address(&ptr)) != GLA_OK) return st;
        return fwd_padded(d, pp, static_cast<char *>(ptr), stream);
    }
    Plan p;
    if ((st = make_plan(d, &p)) != GLA_OK) return st;
    if (p.ws_bytes > size_t(GLA_NOALLOC_SCRATCH_BYTES)) return GLA_ERR_WORKSPACE;
    gla_desc f = *d;
    if (p.ws_bytes > 0) {
        void *ptr = nullptr;
        if ((st = scratch_address(&ptr)) != GLA_OK) return st;
        f.workspace = ptr;
        f.workspace_bytes = GLA_NOALLOC_SCRATCH_BYTES;
    }
    // with the workspace given, the forward pass allocates nothing
    return fwd_run(&f, 0, stream);
}

int gla_step(const gla_step_desc *d, void *stream) {
    if (!d) return GLA_ERR_INVALID_ARG;
    if (d->B < 0 || d->H < 0 || d->Dk <= 0 || d->Dv <= 0) return GLA_ERR_INVALID_ARG;
    if (d->in_dtype != GLA_DTYPE_BF16 && d->in_dtype != GLA_DTYPE_F32) return GLA_ERR_INVALID_ARG;
    if (d->gate_kind < GLA_GATE_NONE || d->gate_kind > GLA_GATE_HEAD_CONST) return GLA_ERR_INVALID_ARG;
    if (int64_t(d->B) * d->H == 0) return GLA_OK;  // no sequences to advance
    if (!d->q || !d->k || !d->v || !d->state || !d->out) return GLA_ERR_INVALID_ARG;
    if ((d->gate_kind == GLA_GATE_NONE) != (d->log_alpha == nullptr)) return GLA_ERR_INVALID_ARG;
    const void *ptrs[] = {d->q, d->k, d->v, d->log_alpha, d->log_ig, d->state, d->out};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GLA_ERR_INVALID_ARG;
    const int64_t bh = int64_t(d->B) * d->H;
    if (bh > (int64_t(1) << 24) || bh * int64_t(d->Dk) * d->Dv > (int64_t(1) << 40)) return GLA_ERR_INVALID_ARG;
    if (d->Dk > 4096 || d->Dv % 16 != 0 || d->Dv > 4096) return GLA_ERR_UNSUPPORTED;
    if (bh * ((d->Dv + 63) / 64) > INT32_MAX) return GLA_ERR_UNSUPPORTED;
    return gla::launch_step(*d, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

int gla_fwd(const void *q, const void *k, const void *v, const float *log_alpha, void *out, float *final_state,
            int B, int H, int L, int Dk, int Dv, int chunk, void *stream) {
    gla_desc d{};
    d.B = B;
    d.H = H;
    d.L = L;
    d.Dk = Dk;
    d.Dv = Dv;
    d.chunk = chunk;
    d.in_dtype = GLA_DTYPE_BF16;
    d.gate_kind = log_alpha ? GLA_GATE_CHANNEL : GLA_GATE_NONE;
    d.q = q;
    d.k = k;
    d.v = v;
    d.log_alpha = log_alpha;
    d.out = reinterpret_cast<float *>(out);
    d.final_state = final_state;
    return gla_fwd_ex(&d, stream);
}

}  // extern "C"

// ------------------------------------------------------------------------------------
// Backward pass: operand preparation, three chunkwise forward passes, and the reductions
// (gla_bwd.hip has the method).

namespace {

bool bwd_dim_ok(int x) { return x == 64 || x == 128 || x == 256; }

// Dv = 512 with bf16 inputs and a scalar gate (or none): the dk and dq passes, whose key
// dimension is Dv, run over the two 256-column halves of the values (the gradient of the
// state splits by value columns) and their outputs add.
constexpr int kDvHalf = 256;
bool bwd_split_dv(const gla_bwd_desc *d) {
    return d->Dv == 2 * kDvHalf && d->in_dtype == GLA_DTYPE_BF16 && d->gate_kind != GLA_GATE_CHANNEL;
}

int validate_bwd(const gla_bwd_desc *d) {
    if (!d) return GLA_ERR_INVALID_ARG;
    if (d->B < 0 || d->H < 0 || d->L < 0 || d->Dk <= 0 || d->Dv <= 0) return GLA_ERR_INVALID_ARG;
    const bool empty = empty_call(d->B, d->H, d->L);
    if (!empty && (!d->q || !d->k || !d->v || !d->dout || !d->dq || !d->dk || !d->dv)) return GLA_ERR_INVALID_ARG;
    if (d->in_dtype != GLA_DTYPE_BF16 && d->in_dtype != GLA_DTYPE_F32) return GLA_ERR_INVALID_ARG;
    if (d->gate_kind < GLA_GATE_NONE || d->gate_kind > GLA_GATE_HEAD_CONST) return GLA_ERR_INVALID_ARG;
    if (!empty && (d->gate_kind == GLA_GATE_NONE) != (d->log_alpha == nullptr)) return GLA_ERR_INVALID_ARG;
    if (d->gate_kind == GLA_GATE_NONE && d->dlog_alpha) return GLA_ERR_INVALID_ARG;
    if (!empty && d->dlog_ig && !d->log_ig) return GLA_ERR_INVALID_ARG;
    const void *ptrs[] = {d->q, d->k, d->v, d->log_alpha, d->log_ig, d->initial_state, d->dout, d->dfinal_state,
                          d->dq, d->dk, d->dv, d->dlog_alpha, d->dlog_ig, d->dinitial_state, d->workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GLA_ERR_INVALID_ARG;
    if (d->workspace && d->workspace_bytes == 0) return GLA_ERR_INVALID_ARG;
    const int64_t lim = int64_t(1) << 40;
    const int64_t bh = int64_t(d->B) * d->H;
    if (bh > (int64_t(1) << 24)) return GLA_ERR_INVALID_ARG;
    if (bh * d->L > lim / std::max(d->Dk, d->Dv)) return GLA_ERR_INVALID_ARG;
    if (!bwd_dim_ok(d->Dk) || !(bwd_dim_ok(d->Dv) || bwd_split_dv(d))) return GLA_ERR_UNSUPPORTED;
    // one (batch, head) slice is addressed with 32-bit byte offsets, as in the forward pass
    if ((int64_t(d->L) + 2 * gla::kMaxChunk) * std::max(d->Dk, d->Dv) * 4 >= (int64_t(1) << 32))
        return GLA_ERR_UNSUPPORTED;
    return GLA_OK;
}

// The forward pass of one of the three backward passes (64-token chunks; fp32 operands for
// fp32 inputs, else bf16 with the output gradient as fp16).
gla_desc bwd_pass_desc(const gla_bwd_desc *d, int dk, int dv, const void *q, const void *k, const void *v,
                       int gate_kind, const float *la, const float *li, const float *s0, float *out, float *fin) {
    gla_desc f{};
    f.B = d->B;
    f.H = d->H;
    f.L = d->L;
    f.Dk = dk;
    f.Dv = dv;
    f.chunk = gla::kTile;
    f.in_dtype = d->in_dtype;
    f.gate_kind = gate_kind;
    f.q = q;
    f.k = k;
    f.v = v;
    f.log_alpha = la;
    f.log_ig = li;
    f.initial_state = s0;
    f.out = out;
    f.final_state = fin;
    return f;
}

// The per-channel backward's dv pass (key-gated) runs on the forward kernel's fp16 path for
// bf16 inputs with Dk <= 128, otherwise on chan_pass_kernel; the other two passes run on
// chan_vg16_kernel (fp16 operands) for bf16 inputs and on chan_pass_kernel for fp32.
bool chan_dv_fast(const gla_bwd_desc *d) { return d->in_dtype == GLA_DTYPE_BF16 && d->Dk <= 128; }

struct BwdPlan {
    size_t chs, rq, rk, rv, rdo, fdo, mx, mxp, s0A, lar, oA, oB, finA, finC, s0T, dfT, g, part, fws, total;
    size_t dqp, dkp;  // bf16: the dq and dk passes' dot products q . dq, k . dk per 64-column tile
    size_t s0h, finH;  // Dv split: a state half, a final-state half
    size_t fws_bytes;
};

// Scratch layout; offsets are 256-byte aligned.  Returns GLA_OK or the status of a forward
// pass's own plan.
int bwd_plan(const gla_bwd_desc *d, BwdPlan *p) {
    const size_t bh = size_t(d->B) * d->H, L = size_t(d->L), Dk = size_t(d->Dk), Dv = size_t(d->Dv);
    const bool bf = d->in_dtype == GLA_DTYPE_BF16;
    const bool gate = d->gate_kind != GLA_GATE_NONE;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    if (d->gate_kind == GLA_GATE_CHANNEL) {
        // per-channel gate: the passes read the caller's tensors; scratch for the transposed
        // states, the final states and the log-gate scan; for bf16 inputs also the fp16 output
        // gradient and its scales; with the dv pass on the forward kernel (bf16, Dk <= 128)
        // also the scaled final-state gradient and that pass's own workspace
        *p = BwdPlan{};
        p->finA = take(bh * Dk * Dv * 4);
        p->finC = take(bh * Dk * Dv * 4);
        p->s0T = d->initial_state ? take(bh * Dk * Dv * 4) : 0;
        p->dfT = d->dfinal_state ? take(bh * Dk * Dv * 4) : 0;
        p->chs = take(gla::chan_scratch_floats(d->B * d->H, d->L, d->Dk, d->Dv, !bf) * 4);
        p->fws_bytes = 0;
        if (bf) {
            p->fdo = take(bh * L * Dv * 2);
            p->mx = take(bh * 4);
            p->mxp = take(bh * gla::bwd_absmax_parts(d->L, d->Dv, d->Dk, d->dfinal_state != nullptr) * 4);
        }
        if (chan_dv_fast(d)) {
            p->s0A = d->dfinal_state ? take(bh * Dk * Dv * 4) : 0;
            const void *x = reinterpret_cast<const void *>(uintptr_t(256));
            float *y = reinterpret_cast<float *>(uintptr_t(256));
            const gla_desc f = bwd_pass_desc(d, d->Dk, d->Dv, x, x, x, GLA_GATE_CHANNEL, y, nullptr, nullptr, y, y);
            size_t n = 0;
            const int st = gla_workspace_size(&f, &n);
            if (st != GLA_OK) return st;
            p->fws_bytes = n;
            p->fws = take(n);
        }
        p->total = off;
        return GLA_OK;
    }
    // operand copies: fp32 reversed q, k, v and output gradient for fp32 inputs; for bf16
    // inputs the passes read q, k, v reversed in place and the output gradient as fp16
    p->rq = bf ? 0 : take(bh * L * Dk * 4);
    p->rk = bf ? 0 : take(bh * L * Dk * 4);
    p->rv = bf ? 0 : take(bh * L * Dv * 4);
    p->rdo = bf ? 0 : take(bh * L * Dv * 4);
    p->fdo = bf ? take(bh * L * Dv * 2) : 0;
    p->mx = bf ? take(bh * 4) : 0;
    p->mxp = bf ? take(bh * gla::bwd_absmax_parts(d->L, d->Dv, d->Dk, d->dfinal_state != nullptr) * 4) : 0;
    p->s0A = (bf && d->dfinal_state) ? take(bh * Dk * Dv * 4) : 0;
    p->lar = gate ? take(bh * L * 4) : 0;
    p->oA = bf ? 0 : take(bh * L * Dv * 4);
    p->oB = bf ? 0 : take(bh * L * Dk * 4);
    p->finA = take(bh * Dk * Dv * 4);
    p->finC = take(bh * Dk * Dv * 4);
    p->s0T = d->initial_state ? take(bh * Dk * Dv * 4) : 0;
    p->dfT = d->dfinal_state ? take(bh * Dk * Dv * 4) : 0;
    p->g = gate ? take(bh * L * 4) : 0;
    p->part = take(bh * 4);
    const bool split = bwd_split_dv(d);
    // bf16: the dq and dk passes form q . dq and k . dk as they store (with the value split,
    // the second half's passes, whose stored rows are the sums of both halves) (offset 0
    // means none: fdo is taken first for bf16)
    const bool need_g = gate && d->dlog_alpha;
    const bool dots = bf && (need_g || d->dlog_ig);
    p->dqp = (dots && need_g) ? take((Dk / 64) * bh * L * 4) : 0;
    p->dkp = dots ? take((Dk / 64) * bh * L * 4) : 0;
    const int kd = split ? kDvHalf : d->Dv;  // key dimension of the dk and dq passes
    p->s0h = split ? take(bh * kDvHalf * Dk * 4) : 0;
    p->finH = split ? take(bh * kDvHalf * Dk * 4) : 0;
    // the forward passes run one after the other on the stream and share one workspace
    const void *x = reinterpret_cast<const void *>(uintptr_t(256));
    float *y = reinterpret_cast<float *>(uintptr_t(256));
    const int rgate = gate ? GLA_GATE_HEAD : GLA_GATE_NONE;
    const float *rla = gate ? y : nullptr;
    gla_desc f[3] = {bwd_pass_desc(d, d->Dk, d->Dv, x, x, x, rgate, rla, nullptr, nullptr, y, y),
                     bwd_pass_desc(d, kd, d->Dk, x, x, x, rgate, rla, nullptr, nullptr, y, nullptr),
                     bwd_pass_desc(d, kd, d->Dk, x, x, x, d->gate_kind, d->log_alpha, d->log_ig, nullptr, y, y)};
    size_t fw = 0;
    for (const gla_desc &fd : f) {
        size_t n = 0;
        const int st = gla_workspace_size(&fd, &n);
        if (st != GLA_OK) return st;
        fw = std::max(fw, n);
    }
    p->fws_bytes = fw;
    p->fws = take(fw);
    p->total = off;
    return GLA_OK;
}

}  // namespace

int gla_bwd_workspace_size(const gla_bwd_desc *d, size_t *bytes) {
    if (!bytes) return GLA_ERR_INVALID_ARG;
    int st = validate_bwd(d);
    if (st != GLA_OK) return st;
    if (empty_call(d->B, d->H, d->L)) {
        *bytes = 0;
        return GLA_OK;
    }
    BwdPlan p;
    if ((st = bwd_plan(d, &p)) != GLA_OK) return st;
    *bytes = p.total;
    return GLA_OK;
}

int gla_bwd(const gla_bwd_desc *d, void *stream) {
    int st = validate_bwd(d);
    if (st != GLA_OK) return st;
    if (empty_call(d->B, d->H, d->L)) {
        // no tokens: the final state is the initial state, so its gradient passes through
        // unchanged, and a fixed per-head gate acted on nothing (its gradient is zero); the
        // per-token gradients have no rows
        if (d->L != 0) return GLA_OK;
        st = state_copy(d->dinitial_state, d->dfinal_state, size_t(d->B) * d->H * d->Dk * d->Dv, stream);
        if (st == GLA_OK && d->gate_kind == GLA_GATE_HEAD_CONST)
            st = state_copy(d->dlog_alpha, nullptr, size_t(d->H), stream);
        return st;
    }
    BwdPlan p;
    if ((st = bwd_plan(d, &p)) != GLA_OK) return st;
    if (d->workspace && d->workspace_bytes < p.total) return GLA_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *ws = reinterpret_cast<char *>(d->workspace);
    bool owned = false;
    if (!ws) {
        void *m = nullptr;
        if (hipMallocAsync(&m, p.total, s) != hipSuccess || !m) {
            (void)hipGetLastError();
            return GLA_ERR_WORKSPACE;
        }
        ws = reinterpret_cast<char *>(m);
        owned = true;
    }
    auto F = [&](size_t off) { return reinterpret_cast<float *>(ws + off); };
    const int BH = d->B * d->H, L = d->L, Dk = d->Dk, Dv = d->Dv, dt = d->in_dtype;
    const bool gate = d->gate_kind != GLA_GATE_NONE;
    const bool bf = dt == GLA_DTYPE_BF16;
    int rc = GLA_OK;
    auto ok = [&](hipError_t e) {
        if (e != hipSuccess && rc == GLA_OK) rc = GLA_ERR_HIP;
        return rc == GLA_OK;
    };
    auto fwd = [&](const gla_desc &f0, int h16, const OutMapArgs &om) {
        if (rc != GLA_OK) return false;
        gla_desc f = f0;
        f.workspace = p.fws_bytes ? ws + p.fws : nullptr;
        f.workspace_bytes = p.fws_bytes;
        const int r = fwd_run(&f, bf ? h16 : 0, stream, bf ? om : OutMapArgs());
        if (r != GLA_OK) rc = r;
        return rc == GLA_OK;
    };
    auto V = [&](size_t off) { return static_cast<void *>(ws + off); };
    if (d->gate_kind == GLA_GATE_CHANNEL) {
        if (d->initial_state) ok(gla::bwd_transpose(d->initial_state, nullptr, F(p.s0T), BH, Dk, Dv, s));
        if (d->dfinal_state) ok(gla::bwd_transpose(d->dfinal_state, nullptr, F(p.dfT), BH, Dk, Dv, s));
        const float *s0T = d->initial_state ? F(p.s0T) : nullptr;
        const float *dfT = d->dfinal_state ? F(p.dfT) : nullptr;
        const bool fast = chan_dv_fast(d);
        uint32_t *cmx = bf ? reinterpret_cast<uint32_t *>(ws + p.mx) : nullptr;
        const _Float16 *cfdo = bf ? reinterpret_cast<const _Float16 *>(ws + p.fdo) : nullptr;
        // the output gradient times a power-of-two scale s per (batch, head), as fp16
        if (bf)
            ok(gla::bwd_dout16(d->dout, d->dfinal_state, F(p.mxp), cmx, reinterpret_cast<_Float16 *>(ws + p.fdo),
                               nullptr, BH, L, Dv, Dk, s));
        if (fast) {
            // dv: key-gated forward pass over the reversed sequence on the fp16 path, as for
            // scalar gates; the kernel reads the per-channel gate reversed and shifted in place
            if (d->dfinal_state) ok(gla::bwd_scale(d->dfinal_state, cmx, F(p.s0A), BH, size_t(Dk) * Dv, s));
            OutMapArgs om;
            om.rev = 1;
            om.li = d->log_ig;
            om.mx = cmx;
            om.in_rev = 1;
            fwd(bwd_pass_desc(d, Dk, Dv, d->k, d->q, V(p.fdo), GLA_GATE_CHANNEL, d->log_alpha, nullptr,
                              d->dfinal_state ? F(p.s0A) : nullptr, d->dv, F(p.finA)),
                gla::kH16V, om);
        }
        if (rc == GLA_OK)
            ok(gla::chan_backward(*d, s0T, dfT, F(p.finA), F(p.finC), F(p.chs), fast, cfdo, cmx, s));
        // the dv pass's final state is scaled by s only on the forward kernel's path
        if (rc == GLA_OK)
            ok(gla::bwd_finish(*d, nullptr, nullptr, nullptr, F(p.finA), F(p.finC), dfT, nullptr, fast ? cmx : nullptr,
                               nullptr, nullptr, s));
        if (owned) (void)hipFreeAsync(ws, s);
        return rc;
    }
    uint32_t *mx = bf ? reinterpret_cast<uint32_t *>(ws + p.mx) : nullptr;
    // operands of the three passes
    if (bf) {
        // the scaled output gradient as fp16 (the reversed passes read it, and q, k, v, from
        // the end)
        ok(gla::bwd_dout16(d->dout, d->dfinal_state, F(p.mxp), mx, reinterpret_cast<_Float16 *>(ws + p.fdo), nullptr,
                           BH, L, Dv, Dk, s));
        if (d->dfinal_state) ok(gla::bwd_scale(d->dfinal_state, mx, F(p.s0A), BH, size_t(Dk) * Dv, s));
    } else {
        ok(gla::bwd_reverse(d->q, dt, F(p.rq), BH, L, Dk, s)) &&
            ok(gla::bwd_reverse(d->k, dt, F(p.rk), BH, L, Dk, s)) &&
            ok(gla::bwd_reverse(d->v, dt, F(p.rv), BH, L, Dv, s)) &&
            ok(gla::bwd_reverse(d->dout, GLA_DTYPE_F32, F(p.rdo), BH, L, Dv, s));
    }
    if (gate) ok(gla::bwd_gate(d->log_alpha, d->gate_kind, F(p.lar), BH, d->H, L, s));
    if (d->initial_state) ok(gla::bwd_transpose(d->initial_state, nullptr, F(p.s0T), BH, Dk, Dv, s));
    if (d->dfinal_state) ok(gla::bwd_transpose(d->dfinal_state, mx, F(p.dfT), BH, Dk, Dv, s));
    const int rgate = gate ? GLA_GATE_HEAD : GLA_GATE_NONE;
    const float *rla = gate ? F(p.lar) : nullptr;
    const float *s0A = d->dfinal_state ? (bf ? F(p.s0A) : d->dfinal_state) : nullptr;
    const void *fdo = bf ? V(p.fdo) : d->dout;
    // bf16: the reversed passes store their rows un-reversed, times i_t / s, straight into dv
    // and dk, and the dq pass its rows times 1/s; fp32: the post kernel does this.
    OutMapArgs om_rev, om_q;
    om_rev.rev = 1;
    om_rev.li = d->log_ig;
    om_rev.mx = mx;
    om_rev.in_rev = 1;
    om_q.mx = mx;
    // operands of the reversed passes: the caller's q, k, v and the fp16 output gradient read
    // from the end (bf16), or the reversed fp32 copies
    const void *rq = bf ? d->q : V(p.rq), *rk = bf ? d->k : V(p.rk), *rv = bf ? d->v : V(p.rv);
    const void *rdo = bf ? fdo : V(p.rdo);
    // dv (reversed; its final state is the gradient of the state after token 0)
    const gla_desc fA = bwd_pass_desc(d, Dk, Dv, rk, rq, rdo, rgate, rla, nullptr, s0A, bf ? d->dv : F(p.oA), F(p.finA));
    fwd(fA, gla::kH16V, om_rev);
    if (!bwd_split_dv(d)) {
        // dk (reversed, keys and values exchanged), with k . dk per stored row (bf16)
        OutMapArgs om_k = om_rev, om_dq = om_q;
        if (p.dkp) {
            om_k.dot_src = d->k;
            om_k.dot_out = F(p.dkp);
        }
        const gla_desc fB = bwd_pass_desc(d, Dv, Dk, rv, rdo, rq, rgate, rla, nullptr,
                                          d->dfinal_state ? F(p.dfT) : nullptr, bf ? d->dk : F(p.oB), nullptr);
        // Its state is the dv pass's transposed: the same gate, keys and values exchanged, and
        // the initial state transposed.  With Dk = Dv both passes plan the same segments, and
        // (bf16: the passes share the workspace) the dk pass starts its segments from the dv
        // pass's segment-entry states, still in the workspace and transposed there in place,
        // instead of forming its own.
        Plan pA, pB;
        if (bf && Dk == Dv && checked_plan(&fA, &pA) == GLA_OK && checked_plan(&fB, &pB) == GLA_OK &&
            pA.nseg > 1 && pA.nseg == pB.nseg && pA.nsub == pB.nsub && pA.seg_len == pB.seg_len &&
            pA.knt == 1 && pB.knt == 1 && rc == GLA_OK) {
            om_k.state_t = ok(gla::bwd_transpose_entries(F(p.fws), BH, Dk, pA.nseg, pA.nsub, s)) ? 1 : 0;
        }
        fwd(fB, gla::kH16K, om_k);
        // dq (keys and values exchanged; its final state is the forward final state, transposed),
        // with q . dq per stored row (bf16, when the log-gate gradient is wanted)
        if (p.dqp) {
            om_dq.dot_src = d->q;
            om_dq.dot_out = F(p.dqp);
        }
        fwd(bwd_pass_desc(d, Dv, Dk, fdo, d->v, d->k, d->gate_kind, d->log_alpha, d->log_ig,
                          d->initial_state ? F(p.s0T) : nullptr, d->dq, F(p.finC)),
            gla::kH16Q, om_dq);
    } else {
        // the same two passes over each 256-column half of the values (and of the output
        // gradient): G splits by value columns, so dk and dq are the sums of the halves'
        // outputs, and the dq pass's final state is the half's rows of the transposed final state.
        // The passes read the halves in place: q and k rows of Dv elements, from column 256 hh.
        const size_t half_bytes = size_t(kDvHalf) * 2, st_half = size_t(kDvHalf) * Dk * 4;
        for (int hh = 0; hh < 2 && rc == GLA_OK; ++hh) {
            const void *vh = static_cast<const char *>(d->v) + hh * half_bytes;
            const void *dh = static_cast<const char *>(fdo) + hh * half_bytes;
            if (d->dfinal_state)
                ok(gla::bwd_copy2d(reinterpret_cast<const char *>(F(p.dfT)) + hh * st_half, size_t(Dv) * Dk * 4,
                                   V(p.s0h), st_half, size_t(BH), st_half, s));
            OutMapArgs om_k = om_rev, om_d = om_q;
            om_k.acc = om_d.acc = hh;
            om_k.qk_stride = om_d.qk_stride = Dv;
            if (hh == 1 && p.dkp) {
                om_k.dot_src = d->k;
                om_k.dot_out = F(p.dkp);
            }
            if (hh == 1 && p.dqp) {
                om_d.dot_src = d->q;
                om_d.dot_out = F(p.dqp);
            }
            fwd(bwd_pass_desc(d, kDvHalf, Dk, vh, dh, rq, rgate, rla, nullptr,
                              d->dfinal_state ? F(p.s0h) : nullptr, d->dk, nullptr),
                gla::kH16K, om_k);
            if (d->initial_state)
                ok(gla::bwd_copy2d(reinterpret_cast<const char *>(F(p.s0T)) + hh * st_half, size_t(Dv) * Dk * 4,
                                   V(p.s0h), st_half, size_t(BH), st_half, s));
            fwd(bwd_pass_desc(d, kDvHalf, Dk, dh, vh, d->k, d->gate_kind, d->log_alpha, d->log_ig,
                              d->initial_state ? F(p.s0h) : nullptr, d->dq, F(p.finH)),
                gla::kH16Q, om_d);
            ok(gla::bwd_copy2d(V(p.finH), st_half, reinterpret_cast<char *>(F(p.finC)) + hh * st_half,
                               size_t(Dv) * Dk * 4, size_t(BH), st_half, s));
        }
    }
    if (rc == GLA_OK)
        ok(gla::bwd_finish(*d, bf ? nullptr : F(p.oA), bf ? nullptr : F(p.oB),
                           (gate && d->dlog_alpha) ? F(p.g) : nullptr, F(p.finA), F(p.finC),
                           d->dfinal_state ? F(p.dfT) : nullptr, F(p.part), mx, p.dqp ? F(p.dqp) : nullptr,
                           p.dkp ? F(p.dkp) : nullptr, s));
    if (owned) (void)hipFreeAsync(ws, s);
    return rc;
}

// ------------------------------------------------------------------------------------
// Delta rule (delta_kernels.hip).

extern "C" int gla_delta_fwd(const gla_delta_desc *d, void *stream) {
    if (!d) return GLA_ERR_INVALID_ARG;
    if (d->B < 0 || d->H < 0 || d->L < 0 || d->Dk <= 0 || d->Dv <= 0 || d->chunk <= 0) return GLA_ERR_INVALID_ARG;
    const bool empty = empty_call(d->B, d->H, d->L);
    if (!empty && (!d->q || !d->k || !d->v || !d->beta || !d->out)) return GLA_ERR_INVALID_ARG;
    if (d->in_dtype != GLA_DTYPE_BF16 && d->in_dtype != GLA_DTYPE_F32) return GLA_ERR_INVALID_ARG;
    if (d->gate_kind != GLA_GATE_NONE && d->gate_kind != GLA_GATE_HEAD && d->gate_kind != GLA_GATE_HEAD_CONST)
        return d->gate_kind == GLA_GATE_CHANNEL ? GLA_ERR_UNSUPPORTED : GLA_ERR_INVALID_ARG;
    if (!empty && (d->gate_kind == GLA_GATE_NONE) != (d->log_alpha == nullptr)) return GLA_ERR_INVALID_ARG;
    const void *ptrs[] = {d->q, d->k, d->v, d->beta, d->log_alpha, d->initial_state, d->out, d->final_state};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GLA_ERR_INVALID_ARG;
    const int64_t lim = int64_t(1) << 40;
    const int64_t bh = int64_t(d->B) * d->H;
    if (bh > (int64_t(1) << 24)) return GLA_ERR_INVALID_ARG;
    if (bh * d->L > lim / std::max(d->Dk, d->Dv)) return GLA_ERR_INVALID_ARG;
    if (bh * int64_t(d->Dk) * d->Dv > lim) return GLA_ERR_INVALID_ARG;
    const bool f32 = d->in_dtype == GLA_DTYPE_F32;
    if (d->chunk != 64) return GLA_ERR_UNSUPPORTED;
    if (f32 ? d->Dk != 64 : (d->Dk != 64 && d->Dk != 128 && d->Dk != 256)) return GLA_ERR_UNSUPPORTED;
    if (d->Dv % 64 != 0 || d->Dv > 4096) return GLA_ERR_UNSUPPORTED;
    // one (batch, head) slice is addressed with 32-bit byte offsets, one chunk past the end
    // read by the prefetch
    if ((int64_t(d->L) + 128) * std::max(d->Dk, d->Dv) * 4 >= (int64_t(1) << 32)) return GLA_ERR_UNSUPPORTED;
    if (gla_delta::lds_bytes(f32, d->Dk) > gla::kMaxLds) return GLA_ERR_UNSUPPORTED;
    const int64_t nwg = bh * (d->Dv / 64);
    if (nwg > INT32_MAX) return GLA_ERR_UNSUPPORTED;
    if (empty)  // the final state of no tokens is the initial state
        return d->L == 0 ? state_copy(d->final_state, d->initial_state, size_t(bh) * d->Dk * d->Dv, stream) : GLA_OK;
    gla_delta::DeltaArgs a{};
    a.q = d->q;
    a.k = d->k;
    a.v = d->v;
    a.beta = d->beta;
    a.la = d->log_alpha;
    a.s0 = d->initial_state;
    a.out = d->out;
    a.fin = d->final_state;
    a.B = d->B;
    a.H = d->H;
    a.L = d->L;
    a.Dv = d->Dv;
    a.gate = d->gate_kind;
    a.ndv = d->Dv / 64;
    a.nwg = (int)nwg;
    return gla_delta::launch(a, f32, d->Dk, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? GLA_OK
                                                                                               : GLA_ERR_HIP;
}

// ------------------------------------------------------------------------------------
// mLSTM with exponential input gate and normaliser (mlstm_kernels.hip).

namespace {

// Sequence segments of the mLSTM for small B*H with long sequences.  The segments run as extra
// heads of a sequence Ls = L / nseg tokens long ([B, H, L] viewed as [B, H*nseg, Ls]): a first
// pass from the zero state gives every segment's own stabilised state (its outputs are
// overwritten later), a join carries the state across the segments, and a second pass runs every
// segment from the state entering it.  The state is C = e^m C', n = e^m n'; across segment s,
// whose log forget gates sum to F_s, the entering state (C'_e, n'_e, m_e) and the segment's own
// (C'_l, n'_l, m_l) join as m = max(F_s + m_e, m_l), C' = e^(F_s + m_e - m) C'_e + e^(m_l - m) C'_l
// (and n' alike).
constexpr float kNoState = -1.0e30f;  // m of the zero state: every weight against it is 0

// Segments for a launch of nwg workgroups over L tokens: 1 (one walk) when the grid is
// already half full, the length is not whole 64-token tiles, or a walk is short; else the
// largest divisor of the tile count that brings the grid nearest to one workgroup per CU.
int mlstm_segments(int64_t nwg, int L) {
    if (nwg >= 128 || L % 64 != 0 || L / 64 < 32) return 1;
    const int tiles = L / 64;
    const int64_t target = std::max<int64_t>(2, 256 / nwg);
    int best = 1;
    for (int n = 2; n <= tiles && n <= target; ++n)
        if (tiles % n == 0) best = n;
    return best;
}

__global__ __launch_bounds__(256) void mlstm_fsum_kernel(const float *lf, float *F, int Ls) {
    __shared__ float red[256];
    const float *p = lf + (size_t)blockIdx.x * Ls;
    float x = 0.f;
    for (int i = (int)threadIdx.x; i < Ls; i += 256) x += p[i];
    red[threadIdx.x] = x;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) F[blockIdx.x] = red[0];
}

// One thread per element of a slice's state (C', then n', then m): the states entering the
// segments, in order, from the initial state (or the zero state).
__global__ __launch_bounds__(256) void mlstm_join_kernel(const float *F, const float *lC, const float *ln,
                                                         const float *lm, const float *c0, const float *n0,
                                                         const float *m0, float *eC, float *en, float *em, int S,
                                                         size_t nC, size_t nN, size_t total) {
    const size_t per = nC + nN + 1;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
        const size_t bh = i / per, e = i % per;
        float me = m0 ? m0[bh] : kNoState;
        float x = 0.f;
        if (e < nC) x = c0 ? c0[bh * nC + e] : 0.f;
        else if (e < nC + nN) x = n0 ? n0[bh * nN + (e - nC)] : 0.f;
        for (int s = 0; s < S; ++s) {
            const size_t r = bh * S + s;
            float xl = 0.f;
            if (e < nC) {
                eC[r * nC + e] = x;
                xl = lC[r * nC + e];
            } else if (e < nC + nN) {
                en[r * nN + (e - nC)] = x;
                xl = ln[r * nN + (e - nC)];
            } else {
                em[r] = me;
            }
            const float md = F[r] + me, ml = lm[r];
            const float mn = fmaxf(md, ml);
            x = expf(md - mn) * x + expf(ml - mn) * xl;
            me = mn;
        }
    }
}

// The final state: the state after the last segment of each slice.
__global__ __launch_bounds__(256) void mlstm_last_kernel(const float *lC, const float *ln, const float *lm, float *fC,
                                                         float *fn, float *fm, int S, size_t nC, size_t nN,
                                                         size_t total) {
    const size_t per = nC + nN + 1;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
        const size_t bh = i / per, e = i % per, r = bh * S + S - 1;
        if (e < nC) {
            if (fC) fC[bh * nC + e] = lC[r * nC + e];
        } else if (e < nC + nN) {
            if (fn) fn[bh * nN + (e - nC)] = ln[r * nN + (e - nC)];
        } else if (fm) {
            fm[bh] = lm[r];
        }
    }
}

int mlstm_segmented(const gla_mlstm_desc *d, bool f32, int cols, int nseg, void *stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const size_t bh = size_t(d->B) * d->H, S = size_t(nseg), nC = size_t(d->Dk) * d->Dv, nN = size_t(d->Dk);
    const size_t rows = bh * S;
    const size_t fl = rows + 2 * (rows * (nC + nN + 1));  // F, the segments' own states, the entering states
    float *w = nullptr;
    if (hipMallocAsync(reinterpret_cast<void **>(&w), fl * 4, st) != hipSuccess || !w) {
        (void)hipGetLastError();
        return GLA_ERR_WORKSPACE;
    }
    float *F = w, *lC = F + rows, *ln = lC + rows * nC, *lm = ln + rows * nN;
    float *eC = lm + rows, *en = eC + rows * nC, *em = en + rows * nN;
    gla_mlstm::MlstmArgs a{};
    a.q = d->q;
    a.k = d->k;
    a.v = d->v;
    a.lf = d->log_f;
    a.li = d->log_i;
    a.out = d->out;
    a.fin_c = lC;
    a.fin_n = ln;
    a.fin_m = lm;
    a.B = d->B;
    a.H = d->H * nseg;
    a.L = d->L / nseg;
    a.Dv = d->Dv;
    a.ndv = d->Dv / cols;
    a.nwg = (int)(rows * a.ndv);
    int rc = GLA_OK;
    if (gla_mlstm::launch(a, f32, d->Dk, st) != hipSuccess) rc = GLA_ERR_HIP;
    const size_t total = bh * (nC + nN + 1);
    const unsigned blocks = (unsigned)std::min<size_t>((total + 255) / 256, 65536);
    if (rc == GLA_OK) {
        hipLaunchKernelGGL(mlstm_fsum_kernel, dim3((unsigned)rows), dim3(256), 0, st, d->log_f, F, a.L);
        hipLaunchKernelGGL(mlstm_join_kernel, dim3(blocks), dim3(256), 0, st, F, lC, ln, lm, d->initial_C, d->initial_n,
                           d->initial_m, eC, en, em, nseg, nC, nN, total);
        if (hipGetLastError() != hipSuccess) rc = GLA_ERR_HIP;
    }
    if (rc == GLA_OK) {
        a.c0 = eC;
        a.n0 = en;
        a.m0 = em;
        if (gla_mlstm::launch(a, f32, d->Dk, st) != hipSuccess) rc = GLA_ERR_HIP;
    }
    if (rc == GLA_OK && (d->final_C || d->final_n || d->final_m)) {
        hipLaunchKernelGGL(mlstm_last_kernel, dim3(blocks), dim3(256), 0, st, lC, ln, lm, d->final_C, d->final_n,
                           d->final_m, nseg, nC, nN, total);
        if (hipGetLastError() != hipSuccess) rc = GLA_ERR_HIP;
    }
    (void)hipFreeAsync(w, st);
    return rc;
}

}  // namespace

extern "C" int gla_mlstm_fwd(const gla_mlstm_desc *d, void *stream) {
    if (!d) return GLA_ERR_INVALID_ARG;
    if (d->B < 0 || d->H < 0 || d->L < 0 || d->Dk <= 0 || d->Dv <= 0 || d->chunk <= 0) return GLA_ERR_INVALID_ARG;
    const bool empty = empty_call(d->B, d->H, d->L);
    if (!empty && (!d->q || !d->k || !d->v || !d->log_f || !d->log_i || !d->out)) return GLA_ERR_INVALID_ARG;
    if (d->reserved != 0) return GLA_ERR_INVALID_ARG;
    if (d->in_dtype != GLA_DTYPE_BF16 && d->in_dtype != GLA_DTYPE_F32) return GLA_ERR_INVALID_ARG;
    const int given = (d->initial_C != nullptr) + (d->initial_n != nullptr) + (d->initial_m != nullptr);
    if (given != 0 && given != 3) return GLA_ERR_INVALID_ARG;
    const void *ptrs[] = {d->q,         d->k,         d->v,         d->log_f,   d->log_i,   d->initial_C, d->initial_n,
                          d->initial_m, d->out,       d->final_C,   d->final_n, d->final_m};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GLA_ERR_INVALID_ARG;
    const int64_t lim = int64_t(1) << 40;
    const int64_t bh = int64_t(d->B) * d->H;
    if (bh > (int64_t(1) << 24)) return GLA_ERR_INVALID_ARG;
    if (bh * d->L > lim / std::max(d->Dk, d->Dv)) return GLA_ERR_INVALID_ARG;
    if (bh * int64_t(d->Dk) * d->Dv > lim) return GLA_ERR_INVALID_ARG;
    const bool f32 = d->in_dtype == GLA_DTYPE_F32;
    if (d->chunk != 64) return GLA_ERR_UNSUPPORTED;
    if (f32 ? d->Dk != 64 : (d->Dk != 64 && d->Dk != 128 && d->Dk != 256)) return GLA_ERR_UNSUPPORTED;
    if (d->Dv % 64 != 0 || d->Dv > 4096) return GLA_ERR_UNSUPPORTED;
    // one (batch, head) slice is addressed with 32-bit byte offsets, one chunk past the end
    // read by the prefetch
    if ((int64_t(d->L) + 128) * std::max(d->Dk, d->Dv) * 4 >= (int64_t(1) << 32)) return GLA_ERR_UNSUPPORTED;
    const int cols = gla_mlstm::wg_cols(f32, d->Dk, d->Dv);
    if (gla_mlstm::lds_bytes(f32, d->Dk, cols) > gla::kMaxLds) return GLA_ERR_UNSUPPORTED;
    const int64_t nwg = bh * (d->Dv / cols);
    if (nwg > INT32_MAX) return GLA_ERR_UNSUPPORTED;
    if (empty) {
        // the final state of no tokens is the initial state, or the zero state (C', n', m) = 0
        if (d->L != 0) return GLA_OK;
        int st = state_copy(d->final_C, d->initial_C, size_t(bh) * d->Dk * d->Dv, stream);
        if (st == GLA_OK) st = state_copy(d->final_n, d->initial_n, size_t(bh) * d->Dk, stream);
        if (st == GLA_OK) st = state_copy(d->final_m, d->initial_m, size_t(bh), stream);
        return st;
    }
    const int nseg = mlstm_segments(nwg, d->L);
    if (nseg > 1) return mlstm_segmented(d, f32, cols, nseg, stream);
    gla_mlstm::MlstmArgs a{};
    a.q = d->q;
    a.k = d->k;
    a.v = d->v;
    a.lf = d->log_f;
    a.li = d->log_i;
    a.c0 = d->initial_C;
    a.n0 = d->initial_n;
    a.m0 = d->initial_m;
    a.out = d->out;
    a.fin_c = d->final_C;
    a.fin_n = d->final_n;
    a.fin_m = d->final_m;
    a.B = d->B;
    a.H = d->H;
    a.L = d->L;
    a.Dv = d->Dv;
    a.ndv = d->Dv / cols;
    a.nwg = (int)nwg;
    return gla_mlstm::launch(a, f32, d->Dk, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? GLA_OK
                                                                                               : GLA_ERR_HIP;
}
