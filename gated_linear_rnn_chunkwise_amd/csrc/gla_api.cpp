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

#include "gla.h"
#include "gla_layout.h"

namespace gla {
hipError_t launch_forward(const KArgs &a, bool f32, int h16, int dk, hipStream_t st);
hipError_t launch_step(const gla_step_desc &d, hipStream_t st);
hipError_t bwd_reverse(const void *src, int dt, float *dst, int BH, int L, int D, hipStream_t st);
hipError_t bwd_gate(const float *la, int kind, float *dst, int BH, int H, int L, hipStream_t st);
hipError_t bwd_transpose(const float *src, const uint32_t *mx, float *dst, int BH, int R, int C, hipStream_t st);
size_t bwd_absmax_parts(int L, int Dv, int Dk, bool dfin);
hipError_t bwd_dout16(const float *dout, const float *dfin, float *part, uint32_t *mx, _Float16 *fwd, _Float16 *rev,
                      int BH, int L, int Dv, int Dk, hipStream_t st);
hipError_t bwd_scale(const float *src, const uint32_t *mx, float *dst, int BH, size_t m, hipStream_t st);
hipError_t bwd_finish(const gla_bwd_desc &d, const float *oA, const float *oB, float *g, const float *finA,
                      const float *finC, const float *dfT, float *part, const uint32_t *mx, hipStream_t st);
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
constexpr int64_t kSmallProblem = 65536;   // head-tokens below which segmenting does not pay

struct Plan {
    int nt, nc, ndv, seg_chunks, nseg, seg_len, nsub;
    int knt;  // 64-token tiles per chunk as the kernels run it: nt with tile pairs, else 1
    int grid_state, grid_scan, grid_out;
    size_t ws_state_bytes, ws_decay_bytes, ws_ke_bytes, ws_bytes;
    uint32_t lds_out, lds_state;
};

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t align256(size_t x) { return (x + 255u) & ~size_t(255u); }

// Argument checks (no HIP call).  Returns GLA_OK or an error status.
int validate(const gla_desc *d) {
    if (!d) return GLA_ERR_INVALID_ARG;
    if (!d->q || !d->k || !d->v || !d->out) return GLA_ERR_INVALID_ARG;
    if (d->B <= 0 || d->H <= 0 || d->L <= 0 || d->Dk <= 0 || d->Dv <= 0 || d->chunk <= 0) return GLA_ERR_INVALID_ARG;
    if (d->seg_chunks < 0 || (d->flags & ~int32_t(GLA_FLAG_TILE_PAIRS)) != 0) return GLA_ERR_INVALID_ARG;
    if (d->in_dtype != GLA_DTYPE_BF16 && d->in_dtype != GLA_DTYPE_F32) return GLA_ERR_INVALID_ARG;
    if (d->gate_kind < GLA_GATE_NONE || d->gate_kind > GLA_GATE_HEAD_CONST) return GLA_ERR_INVALID_ARG;
    if ((d->gate_kind == GLA_GATE_NONE) != (d->log_alpha == nullptr)) return GLA_ERR_INVALID_ARG;
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
    if (d->Dk != 64 && d->Dk != 128 && d->Dk != 256) return GLA_ERR_UNSUPPORTED;
    if (d->Dv % gla::kDvTile != 0 || d->Dv > 4096) return GLA_ERR_UNSUPPORTED;
    if (d->chunk % gla::kTile != 0 || d->chunk > gla::kMaxChunk) return GLA_ERR_UNSUPPORTED;
    // Kernels address one (batch, head) slice through a buffer resource with 32-bit byte
    // offsets, and prefetch up to two chunks past the segment end.
    if ((int64_t(d->L) + 2 * gla::kMaxChunk) * std::max(d->Dk, d->Dv) * 4 >= (int64_t(1) << 32))
        return GLA_ERR_UNSUPPORTED;
    const bool f32 = d->in_dtype == GLA_DTYPE_F32;
    const bool ch = d->gate_kind == GLA_GATE_CHANNEL;
    p->nt = d->chunk / gla::kTile;
    // Without tile pairs the state is advanced tile by tile: the kernels walk 64-token chunks.
    p->knt = (d->flags & GLA_FLAG_TILE_PAIRS) ? p->nt : 1;
    p->nc = (d->L + d->chunk - 1) / d->chunk;
    p->ndv = d->Dv / gla::kDvTile;
    const int64_t bh = int64_t(d->B) * d->H;
    const int64_t wg1 = bh * p->ndv;
    int sc;
    if (d->seg_chunks > 0) {
        sc = std::min(d->seg_chunks, p->nc);
    } else if (wg1 >= kTargetWorkgroups || bh * d->L <= kSmallProblem) {
        sc = p->nc;
    } else {
        const int64_t want = (kTargetWorkgroups + wg1 - 1) / wg1;
        const int64_t nseg = std::min<int64_t>(want, p->nc);
        sc = (int)((p->nc + nseg - 1) / nseg);
    }
    p->seg_chunks = sc;
    p->nseg = (p->nc + sc - 1) / sc;
    p->seg_len = sc * d->chunk;
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
    const int64_t g3 = bh * p->nseg * p->ndv;
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
    p->ws_ke_bytes = align256(size_t(g3) * (size_t)gla::ke_scratch_bytes(opb, d->Dk, ch, p->knt));
    p->ws_bytes = p->ws_state_bytes + p->ws_decay_bytes + p->ws_ke_bytes;
    return GLA_OK;
}

int checked_plan(const gla_desc *d, Plan *p) {
    const int st = validate(d);
    if (st != GLA_OK) return st;
    return make_plan(d, p);
}

}  // namespace

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
    Plan p;
    const int st = checked_plan(d, &p);
    if (st != GLA_OK) return st;
    *bytes = p.ws_bytes;
    return GLA_OK;
}

int gla_query_plan(const gla_desc *d, gla_plan *out) {
    if (!out) return GLA_ERR_INVALID_ARG;
    Plan p;
    const int st = checked_plan(d, &p);
    if (st != GLA_OK) return st;
    out->seg_chunks = p.seg_chunks;
    out->n_seg = p.nseg;
    out->dv_tiles = p.ndv;
    out->tiles_per_chunk = p.nt;
    out->grid_state = p.grid_state;
    out->grid_scan = p.grid_scan;
    out->grid_out = p.grid_out;
    out->tile_pairs = p.knt > 1 ? 1 : 0;
    out->workspace_bytes = p.ws_bytes;
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

    const hipError_t err = gla::launch_forward(a, d->in_dtype == GLA_DTYPE_F32, h16, d->Dk, s);
    if (owned) (void)hipFreeAsync(ws, s);
    return err == hipSuccess ? GLA_OK : GLA_ERR_HIP;
}

}  // namespace

extern "C" {

int gla_fwd_ex(const gla_desc *d, void *stream) { return fwd_run(d, 0, stream); }

int gla_step(const gla_step_desc *d, void *stream) {
    if (!d || !d->q || !d->k || !d->v || !d->state || !d->out) return GLA_ERR_INVALID_ARG;
    if (d->B <= 0 || d->H <= 0 || d->Dk <= 0 || d->Dv <= 0) return GLA_ERR_INVALID_ARG;
    if (d->in_dtype != GLA_DTYPE_BF16 && d->in_dtype != GLA_DTYPE_F32) return GLA_ERR_INVALID_ARG;
    if (d->gate_kind < GLA_GATE_NONE || d->gate_kind > GLA_GATE_HEAD_CONST) return GLA_ERR_INVALID_ARG;
    if ((d->gate_kind == GLA_GATE_NONE) != (d->log_alpha == nullptr)) return GLA_ERR_INVALID_ARG;
    const void *ptrs[] = {d->q, d->k, d->v, d->log_alpha, d->log_ig, d->state, d->out};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GLA_ERR_INVALID_ARG;
    const int64_t bh = int64_t(d->B) * d->H;
    if (bh > (int64_t(1) << 24) || bh * int64_t(d->Dk) * d->Dv > (int64_t(1) << 40)) return GLA_ERR_INVALID_ARG;
    if (d->Dk > 4096 || d->Dv % 64 != 0 || d->Dv > 4096) return GLA_ERR_UNSUPPORTED;
    if (bh * (d->Dv / 64) > INT32_MAX) return GLA_ERR_UNSUPPORTED;
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

int validate_bwd(const gla_bwd_desc *d) {
    if (!d || !d->q || !d->k || !d->v || !d->dout || !d->dq || !d->dk || !d->dv) return GLA_ERR_INVALID_ARG;
    if (d->B <= 0 || d->H <= 0 || d->L <= 0 || d->Dk <= 0 || d->Dv <= 0) return GLA_ERR_INVALID_ARG;
    if (d->in_dtype != GLA_DTYPE_BF16 && d->in_dtype != GLA_DTYPE_F32) return GLA_ERR_INVALID_ARG;
    if (d->gate_kind < GLA_GATE_NONE || d->gate_kind > GLA_GATE_HEAD_CONST) return GLA_ERR_INVALID_ARG;
    if ((d->gate_kind == GLA_GATE_NONE) != (d->log_alpha == nullptr)) return GLA_ERR_INVALID_ARG;
    if (d->gate_kind == GLA_GATE_NONE && d->dlog_alpha) return GLA_ERR_INVALID_ARG;
    if (d->dlog_ig && !d->log_ig) return GLA_ERR_INVALID_ARG;
    const void *ptrs[] = {d->q, d->k, d->v, d->log_alpha, d->log_ig, d->initial_state, d->dout, d->dfinal_state,
                          d->dq, d->dk, d->dv, d->dlog_alpha, d->dlog_ig, d->dinitial_state, d->workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GLA_ERR_INVALID_ARG;
    if (d->workspace && d->workspace_bytes == 0) return GLA_ERR_INVALID_ARG;
    const int64_t lim = int64_t(1) << 40;
    const int64_t bh = int64_t(d->B) * d->H;
    if (bh > (int64_t(1) << 24)) return GLA_ERR_INVALID_ARG;
    if (bh * d->L > lim / std::max(d->Dk, d->Dv)) return GLA_ERR_INVALID_ARG;
    if (!bwd_dim_ok(d->Dk) || !bwd_dim_ok(d->Dv)) return GLA_ERR_UNSUPPORTED;
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
    // the forward passes run one after the other on the stream and share one workspace
    const void *x = reinterpret_cast<const void *>(uintptr_t(256));
    float *y = reinterpret_cast<float *>(uintptr_t(256));
    const int rgate = gate ? GLA_GATE_HEAD : GLA_GATE_NONE;
    const float *rla = gate ? y : nullptr;
    gla_desc f[3] = {bwd_pass_desc(d, d->Dk, d->Dv, x, x, x, rgate, rla, nullptr, nullptr, y, y),
                     bwd_pass_desc(d, d->Dv, d->Dk, x, x, x, rgate, rla, nullptr, nullptr, y, nullptr),
                     bwd_pass_desc(d, d->Dv, d->Dk, x, x, x, d->gate_kind, d->log_alpha, d->log_ig, nullptr, y, y)};
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
    BwdPlan p;
    if ((st = bwd_plan(d, &p)) != GLA_OK) return st;
    *bytes = p.total;
    return GLA_OK;
}

int gla_bwd(const gla_bwd_desc *d, void *stream) {
    int st = validate_bwd(d);
    if (st != GLA_OK) return st;
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
                               s));
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
    fwd(bwd_pass_desc(d, Dk, Dv, rk, rq, rdo, rgate, rla, nullptr, s0A, bf ? d->dv : F(p.oA), F(p.finA)), gla::kH16V,
        om_rev);
    // dk (reversed, keys and values exchanged)
    fwd(bwd_pass_desc(d, Dv, Dk, rv, rdo, rq, rgate, rla, nullptr, d->dfinal_state ? F(p.dfT) : nullptr,
                      bf ? d->dk : F(p.oB), nullptr),
        gla::kH16K, om_rev);
    // dq (keys and values exchanged; its final state is the forward final state, transposed)
    fwd(bwd_pass_desc(d, Dv, Dk, fdo, d->v, d->k, d->gate_kind, d->log_alpha, d->log_ig,
                      d->initial_state ? F(p.s0T) : nullptr, d->dq, F(p.finC)),
        gla::kH16Q, om_q);
    if (rc == GLA_OK)
        ok(gla::bwd_finish(*d, bf ? nullptr : F(p.oA), bf ? nullptr : F(p.oB),
                           (gate && d->dlog_alpha) ? F(p.g) : nullptr, F(p.finA), F(p.finC),
                           d->dfinal_state ? F(p.dfT) : nullptr, F(p.part), mx, s));
    if (owned) (void)hipFreeAsync(ws, s);
    return rc;
}
