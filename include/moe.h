/*
 * moe.h -- C ABI of the block-scaled routed-expert MoE layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer is the Inkling 2 Small routed-expert MoE: a sigmoid router with
 * an additive per-expert selection bias picks the top 8 of 384 experts (no
 * shared experts); each expert is a capped SwiGLU FFN (hidden 4608, expert
 * FFN 2304) stored block-scaled, NVFP4 in layers 0-39 and MXFP8 in layers
 * 40-47, with W4A4 / W8A8 activation quantization.  Sources: TokenSpeed blog
 * "TML Inkling 2 Small at Day 0", table "What's new in Inkling 2 Small" (MoE
 * and Checkpoint rows); Miles docs "inkling-2-small" section 1 (sigmoid
 * routing, soft-capped SwiGLU), section 2 (hidden 4608, FFN 2304) and
 * section 5.3 (W4A4 / W8A8); SGLang cookbook "Inkling-2-Small" section 2
 * ("Checkpoints", "Parallelism", "MegaMoE"); SGLang blog "SGLang and Miles
 * Add Day-0 Support for Inkling 2 Small", section "Performance" (router
 * sigmoid + bias + top-k fused, quantization folded into the expert GEMMs).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns and
 *    frees every buffer, including the workspace.  The library never
 *    allocates, frees or synchronizes; all work is enqueued on `stream` (a
 *    hipStream_t, NULL = the default stream) in order.
 *  - Return value: MOE_OK (0) or a negative status (moe_status_string).
 *    Argument errors are detected on the host before anything is enqueued.
 *    Faults inside kernels surface at the caller's next synchronization.
 *  - Only gfx950 devices are accepted (MOE_ERR_UNSUPPORTED_DEVICE otherwise),
 *    as the pages' ROCm recipes accept gfx950 only (SGLang cookbook section
 *    2, "AMD").
 *  - Inputs are assumed finite.
 *  - Alignment: bf16 activation and output arrays (x, out) and the expert
 *    code arrays (w13, w2) must be 16-byte aligned, as must the quantized
 *    codes of moe_quantize_act; fp32, int32 and scale arrays 4-byte aligned;
 *    the workspace 256-byte aligned.  A misaligned pointer is
 *    MOE_ERR_INVALID_ARG.
 *  - The library is stateless apart from a per-device architecture check
 *    cached on first use; calls on different streams do not share state
 *    except through the caller's buffers.
 *
 * Element formats (little-endian bytes, rows contiguous):
 *  - bf16 activations: [rows][cols] uint16 bit patterns.
 *  - E2M1 (FP4) codes: two per byte, element 2i in the low nibble.
 *  - E4M3 (FP8, finite variant, max 448) and E8M0 (power of two 2^(c-127))
 *    scale bytes.
 *  - NVFP4 = E2M1 elements, one E4M3 scale per 16 consecutive elements of a
 *    row, and one fp32 scale per scale domain (a row of activations; one per
 *    (expert, matrix) for weights).
 *  - MXFP8 = E4M3 elements, one E8M0 scale per 32 consecutive elements.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,        /* null pointer, bad shape or config value */
  MOE_ERR_UNSUPPORTED_DEVICE = -2, /* the current device is not gfx950 */
  MOE_ERR_WORKSPACE_TOO_SMALL = -3,
  MOE_ERR_TOO_MANY_TOKENS = -4,    /* T > cfg->max_tokens */
  MOE_ERR_UNSUPPORTED_FORMAT = -5,
  MOE_ERR_LAUNCH = -6,             /* a kernel launch failed (hipGetLastError) */
  MOE_ERR_HIP = -7,                /* another HIP runtime call failed */
  MOE_ERR_SCRATCH_TOO_SMALL = -8   /* moe_forward_noalloc: the batch needs more
                                      than its fixed scratch buffer */
};

enum moe_fmt { MOE_FMT_NVFP4 = 1, MOE_FMT_MXFP8 = 2 };

/* Cap applied around the SwiGLU; c = cfg->cap.
 * SOFT_GATE_UP: g' = c tanh(g/c), u' = c tanh(u/c), h = silu(g') u'
 * HARD_GATE_UP: g' = min(g, c), u' = clamp(u, -c, c), h = silu(g') u'
 * SOFT_OUT:     h = c tanh(silu(g) u / c)
 * NONE:         h = silu(g) u
 * The pages call the SwiGLU "capped" (SGLang cookbook section 2, TokenSpeed
 * table) and "soft-capped" (Miles docs section 1) without a formula; the
 * default is SOFT_GATE_UP. */
enum moe_cap_form {
  MOE_CAP_SOFT_GATE_UP = 0,
  MOE_CAP_HARD_GATE_UP = 1,
  MOE_CAP_SOFT_OUT = 2,
  MOE_CAP_NONE = 3
};

/* Enqueue values for moe_dtype arguments. */
enum moe_dtype { MOE_DTYPE_BF16 = 0, MOE_DTYPE_F32 = 1 };

/* Where NVFP4 activation rows (x for the gate/up GEMM, h for the down GEMM)
 * take their fp32 scale.  The pages require only that it span each expert's
 * full input width (SGLang cookbook "Inkling-2-Small", section 2,
 * "Parallelism"); which of these the checkpoint uses is not stated.
 *  PER_ROW:    each row its own, max|row| / 2688 (the default).
 *  PER_TENSOR: one for the whole tensor of the call, max / 2688 over all T
 *              x rows, and over all local (token, expert) h rows.
 *  STATIC:     the fixed values act_gs_static[0] (x) and [1] (h).
 * MXFP8 carries no fp32 scale and ignores this field. */
enum moe_act_gs { MOE_ACT_GS_PER_ROW = 0, MOE_ACT_GS_PER_TENSOR = 1, MOE_ACT_GS_STATIC = 2 };

/* Layer configuration (host struct, read during the call only). */
typedef struct moe_config {
  int32_t hidden;             /* H: 4608 for Inkling 2 Small; multiple of 128 */
  int32_t ffn;                /* F: expert FFN width, 2304; multiple of 128 */
  int32_t num_experts;        /* E: 384; 1..1024 */
  int32_t top_k;              /* k: 8; 1..min(E, 32) */
  int32_t expert_begin;       /* first expert held by this GPU */
  int32_t num_local_experts;  /* experts [expert_begin, expert_begin + n) are
                                 computed here; pairs routed elsewhere are
                                 skipped (an expert-parallel share) */
  int32_t fmt;                /* enum moe_fmt of the expert weights and of the
                                 activation quantization (W4A4 / W8A8) */
  int32_t cap_form;           /* enum moe_cap_form */
  float cap;                  /* c, e.g. 7.0 */
  int32_t norm_topk;          /* 1: gate weights divided by their sum over k */
  float routed_scale;         /* gate weights multiplied by this (1.0) */
  int32_t max_tokens;         /* largest T the workspace is sized for */
  int32_t act_gs;             /* enum moe_act_gs (NVFP4 activations) */
  float act_gs_static[2];     /* MOE_ACT_GS_STATIC: positive finite fp32
                                 scales of x and of h (at most 2^120) */
} moe_config;

/* Byte order of the expert weight arrays. */
enum moe_layout {
  MOE_LAYOUT_CANONICAL = 0, /* row-major, as a checkpoint stores it (below) */
  MOE_LAYOUT_PACKED = 1     /* the same bytes permuted by moe_prepare_weights */
};

/* Expert weights of the LOCAL experts, expert-major.  Canonical layout:
 * For local expert i (global id expert_begin + i), with H = hidden, F = ffn:
 *  NVFP4: w13    [i][2F][H/2]   E2M1 codes; rows 0..F-1 gate, F..2F-1 up
 *         w13_sc [i][2F][H/16]  E4M3 block scales
 *         w2     [i][H][F/2]    E2M1 codes of the down projection
 *         w2_sc  [i][H][F/16]   E4M3 block scales
 *         gs     [i][3]         fp32 scales of gate, up, down
 *  MXFP8: w13    [i][2F][H]     E4M3 codes; w13_sc [i][2F][H/32] E8M0
 *         w2     [i][H][F]      E4M3 codes; w2_sc  [i][H][F/32]  E8M0
 *         gs     unused (may be NULL).
 * The packed layout holds exactly the same arrays (same sizes, same gs) with
 * the bytes of every 16-row x 128-column tile reordered so that each
 * wavefront load of the expert GEMMs reads one contiguous kilobyte. */
typedef struct moe_expert_weights {
  const uint8_t* w13;
  const uint8_t* w13_sc;
  const uint8_t* w2;
  const uint8_t* w2_sc;
  const float* gs;
  int32_t layout;           /* enum moe_layout */
} moe_expert_weights;

/* Optional per-stage timing: events[2*s] is recorded before stage s and
 * events[2*s+1] after it, on `stream`.  Entries are hipEvent_t handles
 * created by the caller; NULL entries are skipped. */
enum moe_stage {
  MOE_STAGE_QUANT_X = 0, MOE_STAGE_DISPATCH = 1, MOE_STAGE_GATE_UP = 2,
  MOE_STAGE_QUANT_H = 3, MOE_STAGE_DOWN = 4, MOE_STAGE_COMBINE = 5,
  MOE_STAGE_COUNT = 6
};

/* ---------------------------------------------------------------------- */

/* Status text (static storage).  Host only. */
const char* moe_status_string(int status);

/* MOE_OK if the device architecture name (hipDeviceProp_t.gcnArchName, e.g.
 * "gfx950:sramecc+:xnack-") names gfx950, else MOE_ERR_UNSUPPORTED_DEVICE.
 * Pure host function; `arch` is a host string. */
int moe_check_arch(const char* arch);

/* Validate a configuration (host).  MOE_OK or MOE_ERR_INVALID_ARG /
 * MOE_ERR_UNSUPPORTED_FORMAT. */
int moe_validate_config(const moe_config* cfg);

/* Bytes of workspace moe_route, moe_dispatch, moe_forward and
 * moe_forward_fused need for up to cfg->max_tokens tokens: the library's
 * counterpart of the per-rank token buffer that bounds one MoE forward
 * (SGLang cookbook "Inkling-2-Small", section 2, "MegaMoE": a buffer sized
 * for 4096 tokens per rank).  It holds the router's partial logits, the
 * quantized tokens, the dispatch, and the intermediate h and y rows of every
 * (token, expert) pair.  Host only; *bytes is a host pointer.  The
 * workspace needs no initial contents: every call writes what it later
 * reads (moe_forward_fused's control words are cleared by its own first
 * launch). */
int moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Activation quantization in cfg->fmt (the W4A4 / W8A8 step; Miles docs
 * section 5.3).  x: [rows][cols] bf16 (dtype MOE_DTYPE_BF16) or fp32; cols
 * a multiple of 32.  site: 0 for the gate/up input x, 1 for the down input
 * h (selects act_gs_static[site]).
 *  NVFP4: codes [rows][cols/2], scales [rows][cols/16] E4M3, row_gs [rows]
 *         fp32.  Row scale gs per cfg->act_gs: PER_ROW A = max|row|, gs =
 *         A/2688 (1 and an all-zero row if A == 0); PER_TENSOR the same
 *         over all rows (every row_gs entry then holds it); STATIC
 *         act_gs_static[site].  Per block of 16: s = E4M3(a_b / (6 gs)),
 *         codes E2M1(v * (1 / (s gs))), all in IEEE fp32, round to nearest
 *         even, saturating; a zero scale zeroes its block.  The fp32 scale
 *         spans the row's full width (SGLang cookbook section 2,
 *         "Parallelism").
 *  MXFP8: codes [rows][cols], scales [rows][cols/32] E8M0, row_gs unused.
 *         Per block of 32: X = 2^(floor(log2 amax) - 8) (2^-127 for a zero
 *         block), codes E4M3(v / X) saturating.
 * ws: device scratch of at least 1028 bytes, 4-byte aligned, for NVFP4 with
 * PER_TENSOR (two passes: partial maxima, then the shared scale); unused
 * (may be NULL) otherwise.  The result is bit-identical to the definition
 * above. */
int moe_quantize_act(const moe_config* cfg, int32_t site, int32_t dtype, const void* x, int32_t rows,
                     int32_t cols, uint8_t* codes, uint8_t* scales, float* row_gs, void* ws, size_t ws_bytes,
                     void* stream);

/* The capped SwiGLU of the expert epilogue on n fp32 (gate, up) pairs:
 * h[i] = cap form cfg->cap_form with c = cfg->cap applied to (g[i], u[i])
 * (enum moe_cap_form), evaluated with the same device arithmetic as the
 * gate/up GEMMs' epilogues (hardware exponential and reciprocal; tanh from
 * an odd series below |x| = 1/8).  Arrays 4-byte aligned, n >= 0.  Lets a
 * caller measure the epilogue's error against an exact evaluation. */
int moe_cap_swiglu(const moe_config* cfg, const float* g, const float* u, int64_t n, float* h, void* stream);

/* moe_encode_weights: expert weight matrices to the checkpoint formats on
 * the GPU, with every scale recomputed from the data -- what a weight sync
 * does when it re-encodes updated experts (Miles docs "inkling-2-small",
 * section 5; formats: SGLang cookbook "Inkling-2-Small", section 2
 * "Checkpoints").
 *  w: nmat matrices [nmat][rows][cols], bf16 (dtype MOE_DTYPE_BF16) or fp32,
 *     16-byte aligned; cols a multiple of 32.  Values are assumed finite.
 *  NVFP4: codes [nmat][rows][cols/2] (16-byte aligned), E4M3 block scales
 *     [nmat][rows][cols/16]; one fp32 scale per matrix: A = max|w| over the
 *     matrix, gs = A/2688 (1 if A == 0), then the blocks exactly as in
 *     moe_quantize_act with that gs.  Matrix m's gs is written to
 *     gs[(m / gs_group) * gs_stride + m % gs_group]: for the canonical
 *     moe_expert_weights of n experts, encode the gate/up matrices as
 *     [n][2][F][H] with gs_group 2, gs_stride 3 into gs, and the down
 *     matrices [n][H][F] with gs_group 1, gs_stride 3 into gs + 2.
 *     ws: device scratch of at least 4 * nmat bytes (caller-owned).
 *  MXFP8: codes [nmat][rows][cols], E8M0 scales [nmat][rows][cols/32]
 *     exactly as moe_quantize_act; gs, gs_group, gs_stride and ws unused.
 * Asynchronous on `stream`; bit-identical to the definition.  Errors:
 * MOE_ERR_UNSUPPORTED_FORMAT, MOE_ERR_INVALID_ARG (shape, alignment, null
 * pointers), MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_UNSUPPORTED_DEVICE,
 * MOE_ERR_LAUNCH. */
int moe_encode_weights(int32_t fmt, int32_t dtype, const void* w, int32_t nmat, int32_t rows, int32_t cols,
                       uint8_t* codes, uint8_t* scales, float* gs, int32_t gs_group, int32_t gs_stride,
                       void* ws, size_t ws_bytes, void* stream);

/* moe_decode_weights: the inverse view, to fp32 [nmat][rows][cols]: NVFP4
 * element = (E2M1 value * E4M3 block scale) * gs (the first product exact,
 * one fp32 rounding), MXFP8 element = E4M3 value * 2^(scale - 127) (one
 * fp32 rounding; may overflow to inf above the fp32 range).  Layouts and gs
 * addressing as in moe_encode_weights; codes 8-byte aligned. */
int moe_decode_weights(int32_t fmt, const uint8_t* codes, const uint8_t* scales, const float* gs,
                       int32_t gs_group, int32_t gs_stride, int32_t nmat, int32_t rows, int32_t cols, float* out,
                       void* stream);

/* Router (SGLang blog "Performance": sigmoid, bias and top-k in one step;
 * Miles docs section 1: sigmoid routing, top-8 of 384).
 *  x [T][H] bf16; w_router [E][H] bf16; bias [E] fp32.
 *  z = x w_router^T (fp32 accumulation); s = sigmoid(z); the k experts with
 *  the largest s + bias are chosen, listed in descending order, ties to the
 *  lower expert index; topk_w[t][j] = s[id] / sum_j s[id_j] (if norm_topk)
 *  times routed_scale.
 *  Outputs: topk_ids [T][k] int32, topk_w [T][k] fp32, near_tie [T] uint8
 *  (1 when the k-th and (k+1)-th selection scores differ by less than 1e-6;
 *  may be NULL).  ws: workspace of ws_bytes (moe_workspace_size). */
int moe_route(const moe_config* cfg, const void* x, int32_t T, const void* w_router,
              const float* bias, int32_t* topk_ids, float* topk_w, uint8_t* near_tie,
              void* ws, size_t ws_bytes, void* stream);

/* Dispatch of (token, slot) pairs to the local experts: a stable counting
 * sort of the pair ids p = t*k + j by expert id (the "dispatch" stage of the
 * SGLang cookbook's MegaMoE description, section 2).
 *  topk_ids [T][k] int32 (ids outside [0, E) are an error only in the sense
 *  that they are treated as non-local).
 *  expert_offsets [num_local+1]: pairs of local expert i occupy
 *  sorted_pairs[expert_offsets[i] .. expert_offsets[i+1]), in increasing p.
 *  pair_pos [T*k]: position of pair p in sorted_pairs, or -1 if its expert
 *  is not local.  Any output may be NULL except expert_offsets. */
int moe_dispatch(const moe_config* cfg, const int32_t* topk_ids, int32_t T,
                 int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                 void* ws, size_t ws_bytes, void* stream);

/* One-time repack of the local experts' weights from the canonical layout
 * into the packed layout the expert GEMMs stream fastest (load-time work,
 * like a serving engine's weight loading; no value changes: every code and
 * scale byte moves, none is re-encoded).  src: canonical arrays; dst: arrays
 * of the same sizes (host struct with device pointers, owned by the caller;
 * must not overlap src).  dst->gs is not written (the fp32 scales keep their
 * layout; point dst->gs at src->gs).  Sets dst->layout = MOE_LAYOUT_PACKED.
 * Tile (g, s) of a matrix with K columns covers rows 16g..16g+15 and
 * columns 128s..128s+127; tiles are stored in (g, s) order, each in the
 * lane order of the MFMA operand (lane l = row 16g + l%16, column group
 * l/16):
 *  NVFP4 codes: 1024 B per tile, lane l's 16 bytes at 16 l (its 32 codes
 *         at columns 128s + 32(l/16)); scales: 128 B per tile, lane l's two
 *         E4M3 bytes at 2 l.
 *  MXFP8 codes: 2048 B per tile, lane l's bytes for columns
 *         128s + 16(l/16) + [0,16) at 16 l and for columns
 *         128s + 64 + 16(l/16) + [0,16) at 1024 + 16 l; scales: 64 B per
 *         tile, lane l's E8M0 byte (block 4s + l/16) at l. */
int moe_prepare_weights(const moe_config* cfg, const moe_expert_weights* src, moe_expert_weights* dst,
                        void* stream);

/* The expert half of the layer for T tokens already routed (topk_ids /
 * topk_w from moe_route, or replayed from elsewhere: Miles docs section 5.3,
 * rollout routing replay):
 *   x quantized per row in cfg->fmt; for each pair (t, j) whose expert e is
 *   local: [g | u] = x_q[t] W13[e]^T, h = capped SwiGLU(g, u) (fp32),
 *   h quantized per (t, e) row in cfg->fmt, y = h_q W2[e]^T (fp32);
 *   out[t] = bf16_rne(sum_j topk_w[t][j] y[t, j]) summed in j order over
 *   the local pairs (a partial sum when only some experts are local).
 *  x [T][H] bf16; out [T][H] bf16.  weights: local experts (host struct
 *  pointing at device arrays).  events: optional stage timing (host array of
 *  2*MOE_STAGE_COUNT hipEvent_t, or NULL; events[2s] is recorded before stage
 *  s and events[2s+1] after it).  Stages that share a launch: with at most
 *  4096 (token, slot) pairs, x quantization and dispatch run as one kernel,
 *  timed by the QUANT_X pair (the DISPATCH pair is recorded back to back);
 *  in MXFP8, h is encoded by the gate/up kernel (the QUANT_H pair is empty). */
int moe_forward(const moe_config* cfg, const void* x, int32_t T, const int32_t* topk_ids,
                const float* topk_w, const moe_expert_weights* weights, void* out,
                void* ws, size_t ws_bytes, void* stream, void* const* events);

/* moe_forward with the expert half in one launch: the single-launch fused
 * MoE of the pages (SGLang blog "SGLang and Miles Add Day-0 Support for
 * Inkling 2 Small", "Performance"; SGLang cookbook "Inkling-2-Small"
 * section 2, "MegaMoE").  After the one-launch x quantization + dispatch,
 * one kernel runs gate/up + capped SwiGLU, h quantization, down and the
 * combine as work items, one workgroup each, in the order a device-side
 * counter hands them out; an item waits only on items before it, so the
 * launch drains whatever the number of resident workgroups.  Each wait is
 * also bounded (about a second of polling; reaching the bound needs a device
 * fault elsewhere): a wait that runs out sets an error word in the
 * workspace, every later wait returns at once, the launch completes and the
 * combine writes bf16 NaN instead of sums (moe_forward_fused_status reads
 * the word).  Same arguments, workspace,
 * result (bit-identical to moe_forward) and errors as moe_forward.  It
 * applies when T * top_k <= 4096 and the expected rows per local expert
 * (T * top_k / num_experts) are at most 48; other batches run moe_forward's
 * launch sequence.  events: the GATE_UP pair times the single launch;
 * the QUANT_H, DOWN and COMBINE pairs are recorded back to back after it.
 * cfg->act_gs PER_TENSOR and STATIC run the launch sequence as well. */
int moe_forward_fused(const moe_config* cfg, const void* x, int32_t T, const int32_t* topk_ids,
                      const float* topk_w, const moe_expert_weights* weights, void* out,
                      void* ws, size_t ws_bytes, void* stream, void* const* events);

/* moe_route followed by moe_forward, with routing, x quantization and
 * dispatch in ONE launch for small batches (T <= 256 tokens and T * top_k
 * <= 4096 pairs; NVFP4 with a per-tensor activation scale excepted), where
 * the layer is bound by launches and the waits between them (TokenSpeed blog
 * "TML Inkling 2 Small at Day 0", the paragraph after the "What's new"
 * table; SGLang blog "SGLang and Miles Add Day-0 Support for Inkling 2
 * Small", "Performance").  The expert half follows as in moe_forward.
 * Arguments: those of moe_route and moe_forward together.  Results
 * (topk_ids, topk_w, near_tie, out) are bit-identical to moe_route +
 * moe_forward.  Inside the one launch, work items wait for earlier ones
 * through completion flags tagged with a per-call value, so the workspace
 * still needs no initial contents; each wait is bounded (reaching the bound
 * needs a device fault elsewhere), and a token whose routing wait ran out
 * gets NaN gate weights and a NaN output row.  Larger batches run moe_route's
 * and moe_forward's launches.  events: the QUANT_X pair times the one
 * launch, the DISPATCH pair is empty; the other stages as in moe_forward. */
int moe_route_forward(const moe_config* cfg, const void* x, int32_t T, const void* w_router, const float* bias,
                      int32_t* topk_ids, float* topk_w, uint8_t* near_tie, const moe_expert_weights* weights,
                      void* out, void* ws, size_t ws_bytes, void* stream, void* const* events);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and result (bit-identical to moe_forward),
 * with the workspace taken from a buffer the library holds on each device
 * instead of from the caller.  The caller still passes inputs and outputs.
 *  - The buffer: a fixed device array of moe_noalloc_scratch_bytes() =
 *    64 MiB, one per GPU the library runs on, kept until the process ends;
 *    its address on a device is looked up once, on the first call there.
 *  - A call needs the workspace moe_workspace_size reports for a config with
 *    max_tokens = T; above 64 MiB it returns MOE_ERR_SCRATCH_TOO_SMALL
 *    before enqueueing anything (at Inkling size, hidden 4608, FFN 2304,
 *    384 experts, top-8: up to 269 tokens in NVFP4, 363 in MXFP8).
 *    T > cfg->max_tokens is
 *    MOE_ERR_TOO_MANY_TOKENS.
 *  - No hipMalloc / hipFree or allocating call, no synchronization; every
 *    call writes all of the buffer it later reads, so no contents need to
 *    carry over between calls.
 *  - All calls on one GPU share its buffer: calls that can overlap on one
 *    GPU (different streams, different host threads without ordering)
 *    race and corrupt each other's results.  Serialize them, e.g. on one
 *    stream.
 * No stage events.  Errors as moe_forward, plus MOE_ERR_SCRATCH_TOO_SMALL. */
int moe_forward_noalloc(const moe_config* cfg, const void* x, int32_t T, const int32_t* topk_ids,
                        const float* topk_w, const moe_expert_weights* weights, void* out, void* stream);

/* Bytes of moe_forward_noalloc's per-device buffer (host only). */
size_t moe_noalloc_scratch_bytes(void);

/* Status of the last moe_forward_fused call on workspace ws (same cfg and
 * T): enqueues on `stream` a store of its error word to *err (device int32):
 * 0 when every dependency wait of the single launch was met; 1 when one ran
 * out of polls, in which case every combine item wrote bf16 NaN (0x7FC0) to
 * its part of `out` instead of a sum.  For a (cfg, T) that ran moe_forward's
 * launch sequence instead, *err is 0.  Setting the environment variable
 * MOE_FUSED_TEST_FAIL to 1 makes moe_forward_fused start with the error word
 * set (a test hook for this path: every wait then returns at once). */
int moe_forward_fused_status(const moe_config* cfg, int32_t T, const void* ws, size_t ws_bytes, int32_t* err,
                             void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
