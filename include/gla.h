/*
 * gla.h -- C ABI of the MI355X (gfx950) chunkwise gated linear attention forward pass.
 *
 * The operation.  For every batch b and head h, with a Dk x Dv fp32 state S (zero, or
 * the given initial state, before the first token):
 *
 *     S_t = diag(alpha_t) S_{t-1} + i_t k_t^T v_t ,     o_t = q_t S_t .
 *
 * Softmax-free attention is a linear recurrence over a matrix-valued state [Hardware-
 * Efficient Training of Linear Attention Models, talk summary, 4:04]; gated linear
 * attention lets a data-dependent gate alpha_t in (0,1]^Dk decay the state [Gated Linear
 * Attention Transformers with Hardware-Efficient Training, abstract]; the optional scalar
 * input gate i_t is the sigmoid input gate of the mLSTM variant [Tiled Flash Linear
 * Attention, abstract].  The gate decays the rows (key channels) of the state before the
 * current token is written; there is no scale factor and no normaliser.
 *
 * How it is computed.  Chunkwise: the sequence is cut into chunks of `chunk` tokens;
 * inside a chunk the causal pairwise term is a masked matrix product and the state enters
 * through one product with the chunk's queries; between chunks the state is carried by a
 * recurrence [talk summary, 11:58].  Chunks larger than 64 tokens are split again into
 * 64-token query and key tiles [Tiled Flash Linear Attention, abstract].  The result is
 * the same map as the recurrence; only floating-point rounding differs.
 *
 * Numbers.  q, k, v are bf16 or fp32; gates are fp32 natural logs; the output, the
 * states and all accumulation are fp32.  With bf16 inputs the products that involve a
 * computed operand (gate-rescaled q and k, the masked score matrix, the carried state)
 * take fp16 operands on the matrix cores, and per-channel decay factors are applied to
 * those operands in fp16; with fp32 inputs every operand stays fp32.  fp16 holds
 * magnitudes up to 65504 with 11 significant bits, so with bf16 inputs q, k, v and the
 * entries of the carried state must stay below that (larger data needs fp32 inputs).
 *
 * Layout and ownership.  Every tensor is dense, row-major and contiguous on the device,
 * with the shapes given below, and 16-byte aligned.  The caller owns all memory; the
 * library never frees or keeps a pointer it is given.  Inputs are not modified.
 *
 * Gate values.  log_alpha and log_ig must be finite; -infinity is not accepted (the
 * kernels form differences of running sums of log gates, and -inf - -inf is NaN).  For a
 * gate of zero pass a large negative finite value such as -1e4, whose exponential is an
 * exact zero in fp32.  Gates are expected to be <= 0 (alpha, i in (0, 1]); positive log
 * gates are computed as given but may overflow.  NaN inputs propagate to the outputs.
 * Values are not checked on the host.
 *
 * Empty calls.  B, H or L may be zero (none negative).  Such a call has no output rows, and
 * the pointers of its per-token arrays may then be NULL; the state after no tokens is the
 * state before them, so with L = 0 and B*H > 0 a final state asked for is the initial state
 * (zero without one) and the backward's initial-state gradient is the final-state gradient,
 * written by one small copy kernel.  Sizes, dtypes and the support matrix are still checked.
 *
 * Asynchrony and errors.  Every call validates its arguments on the host before any HIP
 * call; on a validation error it returns a negative status, launches nothing and writes
 * nothing.  Otherwise it enqueues its kernels on `stream` (a hipStream_t; NULL is the
 * default stream) and returns without synchronising; outputs are valid once the stream
 * has completed the work.  GLA_ERR_HIP reports launch-time errors only.  The only mutable
 * global state is a per-device record (atomic bit masks) of which kernels have had their
 * shared-memory limit raised, and the per-device scratch of gla_fwd_noalloc with its
 * address cache (mutex-guarded); calls other than gla_fwd_noalloc are re-entrant.  Two
 * calls that share an output, a final state or a caller workspace must not run
 * concurrently.
 */
#ifndef GLA_H
#define GLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GLA_VERSION 10700 /* major * 10000 + minor * 100 + patch */

/* Status codes.  0 is success; errors are negative. */
enum gla_status {
    GLA_OK = 0,
    GLA_ERR_INVALID_ARG = -1, /* NULL required pointer, a negative size (a zero Dk, Dv or
                                 chunk), misaligned pointer,
                                 size product overflow, gate layout inconsistent with kind */
    GLA_ERR_UNSUPPORTED = -2, /* valid but outside the support matrix below */
    GLA_ERR_WORKSPACE = -3,   /* caller workspace too small, or workspace allocation failed */
    GLA_ERR_HIP = -4          /* a HIP launch or runtime call failed */
};

/* Element type of q, k and v. */
enum gla_dtype { GLA_DTYPE_BF16 = 0, GLA_DTYPE_F32 = 1 };

/* How log_alpha is laid out and broadcast to the per-channel decay of the state rows. */
enum gla_gate {
    GLA_GATE_NONE = 0,       /* log_alpha == NULL: alpha = 1 (plain linear attention) */
    GLA_GATE_CHANNEL = 1,    /* [B, H, L, Dk]: one decay per key channel (GLA) */
    GLA_GATE_HEAD = 2,       /* [B, H, L]: one decay per head and token (mLSTM forget gate) */
    GLA_GATE_HEAD_CONST = 3  /* [H]: one fixed decay per head (RetNet-style) */
};

/* Bits of gla_desc.flags. */
enum gla_flag {
    /* Chunks of more than 64 tokens compute the terms between the 64-token tiles of a chunk
     * as tile pairs against the state at the chunk start (the tiled large-chunk form of
     * Tiled Flash Linear Attention).  Without the flag the state is advanced after every
     * 64-token tile and those terms come through it; both forms give the same result up to
     * rounding, and without the flag fewer operations are needed because the state never
     * leaves the registers. */
    GLA_FLAG_TILE_PAIRS = 1,
    /* The tile-pair form with its second level of sequence parallelism [Tiled Flash Linear
     * Attention, abstract: parallelism inside each chunk]: every chunk is its own segment
     * (its start state is materialised by the segment-state pass and scan; seg_chunks must
     * be 0 or 1, else GLA_ERR_INVALID_ARG), and each 64-token query tile of a chunk is
     * computed by a workgroup of its own against that state, with tile pairs for the earlier
     * tiles of the chunk.  Implies GLA_FLAG_TILE_PAIRS.  Same result up to rounding; it moves
     * more bytes than either form above (the chunk states are written, scanned and read once
     * per query tile, and each query tile re-reads the earlier tiles of its chunk). */
    GLA_FLAG_QUERY_TILES = 2
};

/* Full description of one forward call. */
typedef struct gla_desc {
    int32_t B, H, L, Dk, Dv; /* batch, heads, sequence length, key and value head dims */
    int32_t chunk;           /* chunk size C of the chunkwise algorithm (16, 32 or k * 64) */
    int32_t in_dtype;        /* enum gla_dtype of q, k, v */
    int32_t gate_kind;       /* enum gla_gate */
    const void *q;           /* [B, H, L, Dk] in_dtype */
    const void *k;           /* [B, H, L, Dk] in_dtype */
    const void *v;           /* [B, H, L, Dv] in_dtype */
    const float *log_alpha;  /* layout per gate_kind; must be NULL iff gate_kind == NONE */
    const float *log_ig;     /* [B, H, L] log input gate, or NULL (i_t = 1) */
    const float *initial_state; /* [B, H, Dk, Dv] state before token 0, or NULL (zero) */
    float *out;              /* [B, H, L, Dv] output */
    float *final_state;      /* [B, H, Dk, Dv] state after token L-1, or NULL */
    int32_t seg_chunks;      /* chunks per sequence segment; 0 = chosen by the library.
                                Segments are processed in parallel and joined by a scan of
                                their boundary states (see gla_fwd_ex). */
    int32_t flags;           /* gla_flag bits; other bits set -> GLA_ERR_INVALID_ARG */
    void *workspace;         /* device scratch or NULL (the library allocates it on the stream) */
    size_t workspace_bytes;  /* size of `workspace` */
} gla_desc;

/* What a call would launch (for tests, profiling and the benchmark). */
typedef struct gla_plan {
    int32_t seg_chunks;      /* chunks per segment actually used */
    int32_t n_seg;           /* number of sequence segments */
    int32_t dv_tiles;        /* value-dimension tiles of 64 columns */
    int32_t tiles_per_chunk; /* 64-token tiles per chunk (chunk / 64) */
    int32_t grid_state;      /* workgroups of the segment-state kernel (0 if not launched) */
    int32_t grid_scan;       /* workgroups of the segment-scan kernel (0 if not launched) */
    int32_t grid_out;        /* workgroups of the chunk-output kernel */
    int32_t tile_pairs;      /* 1 if the tile-pair form runs (GLA_FLAG_TILE_PAIRS and chunk > 64) */
    int32_t query_tiles;     /* 1 if each query tile has a workgroup (GLA_FLAG_QUERY_TILES, chunk > 64) */
    size_t workspace_bytes;  /* device scratch the call needs (0 = none) */
} gla_plan;

/* Forward pass with the headline argument list.  q, k, v: bf16 [B,H,L,Dk|Dv];
 * log_alpha: fp32 [B,H,L,Dk] per-channel log gate, or NULL for no gate; out: fp32
 * [B,H,L,Dv]; final_state: fp32 [B,H,Dk,Dv] or NULL; chunk: chunk size; stream: hipStream_t.
 * Any scratch it needs is allocated and freed stream-ordered on `stream`.
 * Returns a gla_status. */
int gla_fwd(const void *q, const void *k, const void *v, const float *log_alpha, void *out,
            float *final_state, int B, int H, int L, int Dk, int Dv, int chunk, void *stream);

/* General forward pass: input dtype, every gate kind, input gate, initial state, segment
 * length and caller workspace.  When d->workspace is NULL and scratch is needed it is
 * allocated and freed stream-ordered on `stream`; otherwise d->workspace_bytes must be at
 * least what gla_workspace_size reports, else GLA_ERR_WORKSPACE.
 * Support matrix (else GLA_ERR_UNSUPPORTED): chunk 16, 32, or a multiple of 64 in
 * [64, 512] (chunks of 16 and 32 tokens run as 64-token tiles, the same map, and seg_chunks
 * then counts 64-token tiles); Dk a multiple of 16 up to 256 and Dv a multiple of 16 up to
 * 4096.  Dk in {64, 128, 256} with Dv a multiple of 64 runs directly; other shapes run on
 * zero-padded copies in the workspace (q, k and a per-channel gate padded to the next Dk of
 * 64, 128, 256 with zero channels, v and the output to the next multiple of 64 columns, the
 * states to both; the same result, plus the copies' bytes and workspace); L >= 0 with
 * (L + 1024) * max(Dk, Dv) * 4 < 2^32 (one (batch, head) slice is addressed with 32-bit
 * byte offsets, which allows L up to about 1M for Dv = 1024); and the operand tiles of
 * one workgroup must fit the 160 KB of LDS of a compute unit.  That last rule only bites
 * with GLA_FLAG_TILE_PAIRS or GLA_FLAG_QUERY_TILES and fp32 inputs: chunk > 64 is then unsupported for Dk = 256,
 * and for Dk = 128 under a per-channel gate.  Returns a gla_status. */
int gla_fwd_ex(const gla_desc *d, void *stream);

/* Device scratch available to gla_fwd_noalloc on each GPU: 32 MiB. */
#define GLA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Forward pass that allocates no memory, for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same operation,
 * arguments, support matrix and kernels as gla_fwd_ex, except the scratch: d->workspace must
 * be NULL and d->workspace_bytes 0 (else GLA_ERR_INVALID_ARG); the scratch the call needs
 * (gla_workspace_size; only sequence-segmented calls, the tile-pair and query-tile forms and
 * shapes run on padded copies need any) comes
 * from a device array of GLA_NOALLOC_SCRATCH_BYTES built into the library, one per GPU,
 * held from the first call on that GPU until the process ends.  A call that needs more
 * returns GLA_ERR_WORKSPACE and launches nothing.  The first call on a GPU resolves the
 * array's address with that GPU current (a HIP runtime query, no allocation).
 * Every call on one GPU shares that GPU's array and leaves its contents behind (nothing in
 * it is read before this call writes it): calls that overlap in time on one GPU, on
 * different streams or from different host threads, race on it and must be serialised by
 * the caller.  Returns a gla_status. */
int gla_fwd_noalloc(const gla_desc *d, void *stream);

/* Scratch bytes gla_fwd_ex needs for `d` (no HIP call).  Returns a gla_status. */
int gla_workspace_size(const gla_desc *d, size_t *bytes);

/* Launch plan gla_fwd_ex would use for `d` (no HIP call).  Returns a gla_status. */
int gla_query_plan(const gla_desc *d, gla_plan *plan);

/* One token of the recurrence for every (batch, head): the recurrent (decoding) form, one
 * rank-1 write of the state followed by one vector-matrix read [Hardware-Efficient Training
 * of Linear Attention Models, talk summary, 4:04 and 7:36]:
 *
 *     S <- diag(alpha) S + i k^T v ,     o = q S .
 *
 * A chunkwise forward pass over L tokens followed by steps for tokens L, L+1, ... gives the
 * same outputs as one forward pass over all of them (the state is the final state of the
 * forward pass).  Everything is dense and row-major on the device, 16-byte aligned.  */
typedef struct gla_step_desc {
    int32_t B, H, Dk, Dv;    /* batch, heads, key and value head dims */
    int32_t in_dtype;        /* enum gla_dtype of q, k, v */
    int32_t gate_kind;       /* enum gla_gate; CHANNEL: [B, H, Dk], HEAD: [B, H], HEAD_CONST: [H] */
    const void *q;           /* [B, H, Dk] */
    const void *k;           /* [B, H, Dk] */
    const void *v;           /* [B, H, Dv] */
    const float *log_alpha;  /* layout per gate_kind; must be NULL iff gate_kind == NONE */
    const float *log_ig;     /* [B, H] log input gate, or NULL (i = 1) */
    float *state;            /* [B, H, Dk, Dv] fp32 state, read and updated in place */
    float *out;              /* [B, H, Dv] fp32 output */
} gla_step_desc;

/* Recurrent step.  Support matrix (else GLA_ERR_UNSUPPORTED): Dk in [1, 4096], Dv a
 * multiple of 16 up to 4096.  Validation as for gla_fwd_ex (GLA_ERR_INVALID_ARG for NULL
 * required pointers, negative B or H, Dk or Dv <= 0, misalignment, a gate pointer
 * inconsistent with its kind; B*H = 0 advances no sequence and returns GLA_OK).
 * The state must not alias q, k, v, the gates or the output.  Asynchronous on `stream`;
 * allocates nothing.  Returns a gla_status. */
int gla_step(const gla_step_desc *d, void *stream);

/* Gradients of the forward pass (the backward pass used in training [Hardware-Efficient
 * Training of Linear Attention Models, talk summary, 7:36]): for a scalar loss with
 * gradient dout = d loss / d out and dfinal_state = d loss / d final_state, the gradients
 * with respect to q, k, v, the log gates and the initial state.  They follow from the
 * definition by differentiating each step; computed chunkwise on the GPU.
 *
 * Method: with G_t = d loss / d S_t, which obeys the same recurrence
 * run backwards in time (G_t = q_t^T dout_t + diag(alpha_{t+1}) G_{t+1}, G_{L-1} starting
 * from dfinal_state), dv_t = i_t k_t G_t, dk_t = i_t (G_t v_t^T)^T and dq_t = dout_t S_t^T;
 * each is a chunkwise forward pass over re-ordered operands (time reversed for dv and dk,
 * keys and values exchanged for dk and dq).  With a per-channel gate the dk and dq passes
 * decay their states on the value side, S_t = S_{t-1} diag(alpha_t) + ..., which their own
 * kernel computes.  The log-gate gradients follow from d loss / d B_t = q_t * dq_t -
 * k_t * dk_t (B_t the running sum of log decays, per channel; a dot product over channels
 * for scalar gates; plus the final-state term at the last token) summed from t to the end,
 * and dlog_ig_t = k_t . dk_t.
 * Precision: fp32 inputs run the passes in fp32.  bf16 inputs run every pass on fp16
 * matrix-core operands (the forward kernels' fp16 path for the passes they compute, a
 * value-gated kernel of the same numerics for the per-channel dk and dq passes), with q, k,
 * v as given and dout entering as fp16 after a per-(batch, head) power-of-two scale that
 * puts its largest magnitude in [4, 8) (dfinal_state counts at 1/64 of its magnitude); the
 * scale is divided out exactly.  Only the per-channel dv pass with Dk = 256 runs in fp32.
 * The fp16 range of the forward pass applies to q, k, v and to the passes' states.
 *
 * Shapes: q, k [B,H,L,Dk] and v [B,H,L,Dv] in in_dtype; gates as in gla_desc; dout
 * [B,H,L,Dv] fp32; dfinal_state [B,H,Dk,Dv] fp32 or NULL (zero); outputs fp32: dq, dk
 * [B,H,L,Dk], dv [B,H,L,Dv], dlog_alpha in the layout of log_alpha (must be NULL when
 * gate_kind is NONE; NULL otherwise skips it), dlog_ig [B,H,L] (may be non-NULL only with
 * log_ig), dinitial_state [B,H,Dk,Dv] or NULL.  Outputs must not alias inputs or each
 * other. */
typedef struct gla_bwd_desc {
    int32_t B, H, L, Dk, Dv;
    int32_t in_dtype;             /* enum gla_dtype of q, k, v */
    int32_t gate_kind;            /* enum gla_gate */
    const void *q, *k, *v;
    const float *log_alpha;       /* must be NULL iff gate_kind == NONE */
    const float *log_ig;          /* [B, H, L] or NULL */
    const float *initial_state;   /* [B, H, Dk, Dv] or NULL */
    const float *dout;            /* [B, H, L, Dv] */
    const float *dfinal_state;    /* [B, H, Dk, Dv] or NULL */
    float *dq, *dk, *dv;
    float *dlog_alpha;
    float *dlog_ig;
    float *dinitial_state;
    void *workspace;              /* device scratch or NULL (allocated on the stream) */
    size_t workspace_bytes;
} gla_bwd_desc;

/* Backward pass.  Support matrix (else GLA_ERR_UNSUPPORTED): every gate kind; Dk and Dv in
 * {64, 128, 256}; also Dv = 512 with bf16 inputs and a gate other than per-channel (the dk
 * and dq passes, whose key dimension is Dv, then run over the two 256-column halves of v and
 * dout and add: the state gradient splits by value columns); L as for gla_fwd_ex.
 * Validation and asynchrony as for gla_fwd_ex.  Returns a gla_status. */
int gla_bwd(const gla_bwd_desc *d, void *stream);

/* Scratch bytes gla_bwd needs for `d` (no HIP call).  Returns a gla_status. */
int gla_bwd_workspace_size(const gla_bwd_desc *d, size_t *bytes);

/* The delta rule: DeltaNet and Gated DeltaNet, computed chunkwise.  For every (batch, head),
 * with a Dk x Dv fp32 state S (zero, or the given initial state, before the first token):
 *
 *     S_t = alpha_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t ,     o_t = q_t S_t .
 *
 * beta_t is the writing strength of token t [Hardware-Efficient Training of Linear Attention
 * Models, talk summary, 22:36]; the update is one gradient step of size beta_t on
 * 1/2 |k_t S - v_t|^2, the state acting as a fast weight, and Gated DeltaNet adds a scalar
 * decay alpha_t in the manner of Mamba-2 [same talk, 31:16], here applied to the previous
 * state before the token is written (alpha_t = 1 for DeltaNet).  The transition is identity
 * plus rank one; the chunkwise form carries its product over a chunk with the WY
 * representation (a unit lower-triangular solve per chunk) [same talk, 31:16], and gives the
 * same map as the recurrence up to rounding.  beta and keys are used as given: the step is a
 * contraction of the state along k_t only while 0 <= beta_t |k_t|^2 <= 2 (unit-norm keys and
 * beta in [0, 1] keep every state bounded; other values are computed as given).
 *
 * Numbers: bf16 inputs run the matrix products on fp16 operands (q, k, v converted, computed
 * operands rounded once) with fp32 accumulation, and the triangular solve's diagonal blocks
 * in fp32; fp32 inputs keep fp32 operands throughout.  States and outputs are fp32. */
typedef struct gla_delta_desc {
    int32_t B, H, L, Dk, Dv;     /* batch, heads, sequence length, key and value head dims */
    int32_t chunk;               /* chunk size; 64 (the kernel's chunk) */
    int32_t in_dtype;            /* enum gla_dtype of q, k, v */
    int32_t gate_kind;           /* GLA_GATE_NONE (DeltaNet), GLA_GATE_HEAD (Gated DeltaNet,
                                    [B, H, L]) or GLA_GATE_HEAD_CONST ([H]) */
    const void *q;               /* [B, H, L, Dk] in_dtype */
    const void *k;               /* [B, H, L, Dk] in_dtype */
    const void *v;               /* [B, H, L, Dv] in_dtype */
    const float *beta;           /* [B, H, L] fp32 writing strength */
    const float *log_alpha;      /* natural log of alpha_t per gate_kind; NULL iff NONE */
    const float *initial_state;  /* [B, H, Dk, Dv] or NULL (zero) */
    float *out;                  /* [B, H, L, Dv] */
    float *final_state;          /* [B, H, Dk, Dv] or NULL */
} gla_delta_desc;

/* Delta-rule forward pass.  Support matrix (else GLA_ERR_UNSUPPORTED): chunk 64; bf16 inputs
 * with Dk in {64, 128, 256}, fp32 inputs with Dk = 64; Dv a multiple of 64 up to 4096; L as
 * for gla_fwd_ex.  One workgroup per (batch, head, 64 value columns) walks the whole
 * sequence (no sequence segments: the state transition of a segment is a full Dk x Dk
 * matrix, not a decay).  log_alpha must be finite (as for gla_fwd_ex).  Validation,
 * ownership and asynchrony as for gla_fwd_ex; allocates nothing.  Returns a gla_status. */
int gla_delta_fwd(const gla_delta_desc *d, void *stream);

/* The mLSTM with exponential input gate and normaliser (the xLSTM's matrix memory, the
 * mLSTM of Beck et al. (2024) to which the Tiled Flash Linear Attention abstract applies its
 * kernels; the abstract's sigmoid-input-gate variant, gla_fwd_ex with GLA_GATE_HEAD and
 * log_ig, drops the normaliser).  For every (batch, head), with f_t = exp(log_f_t) and
 * i_t = exp(log_i_t):
 *
 *     C_t = f_t C_{t-1} + i_t k_t^T v_t ,   n_t = f_t n_{t-1} + i_t k_t ,
 *     out_t = q_t C_t / max(|q_t . n_t|, 1) ,
 *
 * C Dk x Dv and n of Dk entries, zero before the first token unless an initial state is
 * given.  The pages print neither the exponential gate nor the normaliser; this is the cell
 * as its source defines it.  The input gate is unbounded, so states cross the ABI stabilised:
 * (C', n', m) with C = exp(m) C' and n = exp(m) n' (m a natural log).  The kernel walks
 * 64-token chunks carrying (C', n', m) with m the running maximum of the log weights, so
 * every factor it applies is at most 1; the output equals the recurrence's up to rounding.
 *
 * Numbers: bf16 inputs run the matrix products on fp16 operands (q, k, v converted, scores
 * and weighted values rounded once) with fp32 accumulation; the normaliser and all gate
 * arithmetic are fp32.  fp32 inputs keep fp32 operands.  Outputs and states are fp32. */
typedef struct gla_mlstm_desc {
    int32_t B, H, L, Dk, Dv;     /* batch, heads, sequence length, key and value head dims */
    int32_t chunk;               /* chunk size; 64 (the kernel's chunk) */
    int32_t in_dtype;            /* enum gla_dtype of q, k, v */
    int32_t reserved;            /* 0 */
    const void *q;               /* [B, H, L, Dk] in_dtype */
    const void *k;               /* [B, H, L, Dk] in_dtype (any key scaling is the caller's) */
    const void *v;               /* [B, H, L, Dv] in_dtype */
    const float *log_f;          /* [B, H, L] fp32 natural log of the forget gate, finite */
    const float *log_i;          /* [B, H, L] fp32 natural log of the input gate, finite */
    const float *initial_C;      /* [B, H, Dk, Dv] stabilised C', or NULL: the three initial  */
    const float *initial_n;      /* [B, H, Dk] stabilised n'          fields are all given or */
    const float *initial_m;      /* [B, H] m                          all NULL (zero state)  */
    float *out;                  /* [B, H, L, Dv] */
    float *final_C;              /* [B, H, Dk, Dv] stabilised C' after the last token, or NULL */
    float *final_n;              /* [B, H, Dk] or NULL */
    float *final_m;              /* [B, H] or NULL */
} gla_mlstm_desc;

/* mLSTM forward pass.  Support matrix (else GLA_ERR_UNSUPPORTED): chunk 64; bf16 inputs with
 * Dk in {64, 128, 256}, fp32 inputs with Dk = 64; Dv a multiple of 64 up to 4096; L as for
 * gla_fwd_ex.  One workgroup per (batch, head, value slice) walks the whole sequence; when
 * those are fewer than 128 and L is a multiple of 64 with at least 32 tiles, the sequence
 * runs as segments instead (every segment's own state from zero, the states joined across the
 * segments through their summed log forget gates, every segment again from the state entering
 * it: about twice the work, on up to 256 workgroups).  GLA_ERR_INVALID_ARG: a NULL required
 * pointer, negative sizes, a misaligned pointer (16 bytes), reserved != 0, or an initial state
 * given in part.  Ownership and asynchrony as for gla_fwd_ex; allocates nothing, except the
 * segmented form's scratch (the segment states, stream-ordered on `stream`; GLA_ERR_WORKSPACE
 * if that fails).  Returns a gla_status. */
int gla_mlstm_fwd(const gla_mlstm_desc *d, void *stream);

/* Static English text for a status code (never NULL). */
const char *gla_status_string(int status);

/* GLA_VERSION of the built library. */
int gla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H */
