/*
 * moe.h -- C ABI of the fused routed + shared-expert MoE layer forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (one forward, one GPU):
 *
 *   y_t = sum_j w_tj * E_{e_tj}(x_t) + gamma_t * S(x_t)
 *
 * - top-k (or grouped top-k) routing whose weights already carry the routed
 *   scaling factor (vLLM PR 65207, "Purpose", commit 1: the scaling factor is
 *   folded into the top-k weights rather than applied to the MoE output);
 * - a token-by-expert sort with per-expert padding (same PR, commit 2, and the
 *   review's "moe_sorting without zeroing" experiment);
 * - a two-stage routed grouped GEMM: stage 1 = gate/up with SiLU-mul, stage 2
 *   = down whose epilogue does the weighted scatter-reduce and accumulates
 *   the shared-expert output given as an addend (vLLM PR 65207, commit 2);
 * - a shared expert gated by sigmoid(x . g), the gate computed as a K-length
 *   dot product with the sigmoid folded in (vLLM PR 56789, "Summary" and
 *   "Commits");
 * - per-token activation scales and per-expert weight scales applied to the
 *   fp32 accumulator before the activation and the fused quantisation, and
 *   MX 32-element block scales (AITER PR 6106, "Technical Details");
 * - the shared expert either as always-selected pseudo-experts of the routed
 *   op (vLLM PR 61503, "Overview": fused heterogeneous MoE) or on a second
 *   stream that signals an event right before stage 2 (vLLM PR 65207,
 *   commit 2).  Pseudo-expert fusion requires the shared weights to use the
 *   routed experts' format (SGLang PR 27057, "Modifications", item 1).
 *
 * Conventions for every entry point:
 * - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *   aligned, row-major and dense.  The library never allocates and never
 *   frees.  Its mutable state is one thread-local slot holding the HIP
 *   error behind the calling thread's last MOE_ERR_HIP (read with
 *   moe_last_hip_error) and, for moe_forward_noalloc only, its per-device
 *   scratch array; calls are otherwise stateless and reentrant.
 * - Every argument is validated on the host before anything is launched; an
 *   invalid call returns an error and launches nothing.  Launch failures
 *   return MOE_ERR_HIP; faults inside kernels surface at the caller's next
 *   synchronisation.
 * - Work is enqueued asynchronously on the given stream(s).  No entry point
 *   synchronises with the host or reads device data on the host, so every
 *   call can be captured into a HIP graph.
 * - Inputs are finite; behaviour for NaN/Inf inputs is undefined.
 *
 * Supported formats (x / weights / stage-1 output h):
 *   F32  : x F32, weights F32, h F32
 *   BF16 : x BF16, weights BF16, h BF16
 *   MXFP8: x BF16 quantised in-layer to MX-32 e4m3, weights FP8_E4M3 + MX32
 *          e8m0 scales, h MX-32 e4m3 (from bf16-rounded h)
 *   A8W8 : x FP8_E4M3 + fp32 per-row (token) scale, weights FP8_E4M3 + fp32
 *          per-expert scale (one for W13, one for W2), h per-row e4m3 with an
 *          fp32 row scale (from bf16-rounded h)
 *   MXFP4: as MXFP8 with FP4_E2M1 weights + MX32 e8m0 scales (the MXFP4
 *          checkpoints of vLLM PR 65207, "Purpose", commit 3); H, I and I_s
 *          multiples of 256; sorted blocks of at most 128 rows
 * FP8_E4M3 is the OCP e4m3fn format (max 448, no infinities).  FP4_E2M1 is
 * the OCP MX FP4 element (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives),
 * two per byte, the element of even index in the low nibble: a weight row of
 * K elements is K / 2 bytes.
 *
 * Weight layout: W13 is [n][2*I][H] with the I gate rows first and the I up
 * rows second; W2 is [n][H][I].  Products are x . W^T.  MX32 scales are e8m0
 * bytes [n][2*I][H/32] and [n][H][I/32] (one per 32 consecutive K elements).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* bad shape, pointer, alignment or parameter */
  MOE_ERR_UNSUPPORTED = -2, /* valid request the library does not provide */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  MOE_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_FP4_E2M1 = 3 } moe_dtype;

typedef enum {
  MOE_SCALE_NONE = 0,
  MOE_SCALE_PER_ROW = 1,    /* activations: one fp32 scale per row (token) */
  MOE_SCALE_PER_EXPERT = 2, /* weights: one fp32 scale per expert matrix */
  MOE_SCALE_MX32 = 3        /* e8m0 byte per 32 consecutive K elements */
} moe_scale;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

typedef enum {
  MOE_SHARED_NONE = 0,   /* no shared expert */
  MOE_SHARED_PSEUDO = 1, /* ceil(I_s/I) always-selected pseudo-experts */
  MOE_SHARED_AUX = 2,    /* dense shared expert on the aux stream */
  MOE_SHARED_AUTO = 3    /* PSEUDO when eligible, else AUX */
} moe_shared_mode;

typedef enum { MOE_STAGE2_STORE = 0, MOE_STAGE2_ACCUMULATE = 1 } moe_stage2_mode;

/* Gated activation of stage 1, h = act(a_gate) * a_up (AITER PR 6106,
 * "Technical Details": the activation follows the scales and the bias on the
 * fp32 accumulator).  SILU: g * sigmoid(g).  GELU_TANH: the tanh form of
 * GELU, g/2 * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3))). */
typedef enum { MOE_ACT_SILU = 0, MOE_ACT_GELU_TANH = 1 } moe_activation;

typedef enum {
  MOE_FEATURE_ACCUMULATE_OUTPUT = 1, /* stage 2 accumulates onto an addend */
  MOE_FEATURE_PSEUDO_SHARED = 2,     /* heterogeneous shared pseudo-experts */
  MOE_FEATURE_AUX_STREAM = 3,        /* shared expert on a second stream */
  MOE_FEATURE_MXFP8 = 4,
  MOE_FEATURE_A8W8 = 5,
  MOE_FEATURE_F32 = 6,
  MOE_FEATURE_BF16 = 7,
  MOE_FEATURE_MXFP4 = 8,
  MOE_FEATURE_EXPERT_BIAS = 9, /* per-expert bias on the stage-1 and stage-2 accumulators */
  MOE_FEATURE_GELU_TANH = 10,  /* MOE_ACT_GELU_TANH */
  MOE_FEATURE_ROUTER_GEMM = 11 /* moe_forward_args.router_w: logits computed in the prologue */
} moe_feature;

/* Weight layout.  Logically every weight matrix is row-major: rows = output
 * features, row_bytes = K * element size (rows % 16 == 0, row_bytes % 128 ==
 * 0).  The GEMM kernels read it in a tiled order instead, so that each 64-lane
 * MFMA operand load is 1024 contiguous bytes: 16-row x 128-byte tiles of 2048
 * contiguous bytes, row block major, K tile minor.  Inside a tile, byte b
 * (0..15) of 16-byte chunk c (0..7) of tile row r (0..15) sits at
 *     (c / 4) * 1024 + ((c % 4) * 16 + r) * 16 + b.
 * MX32 scale matrices (rows x row_bytes / 32 bytes, one e8m0 byte per 32
 * elements) are tiled alike: 16 rows x 4 scale bytes per 64-byte tile, scale
 * q (0..3) of tile row r at q * 16 + r.  Matrices of consecutive experts stay
 * consecutive (a tiled [n][rows][row_bytes] array is n tiled matrices back to
 * back), and a 16-row-aligned row range stays a contiguous byte range.
 * FP4_E2M1 rows go through the same byte tiling: each 1 KiB half of a tile is
 * then one 128-element K step in operand order.
 * moe_pack_weights / moe_pack_mx_scales convert once, at load time. */
typedef enum {
  MOE_LAYOUT_ROW_MAJOR = 0, /* accepted only by the pack functions */
  MOE_LAYOUT_TILED = 1      /* required by moe_forward, moe_stage1, moe_stage2_accum */
} moe_layout;

/* One family of expert weights (routed: n = E, width I; shared: n = 1, width I_s). */
typedef struct {
  const void* w13;       /* [n][2*width][H] gate rows then up rows */
  const void* w2;        /* [n][H][width] */
  const void* w13_scale; /* PER_EXPERT: float[n]; MX32: uint8 [n][2*width][H/32]; else NULL */
  const void* w2_scale;  /* PER_EXPERT: float[n]; MX32: uint8 [n][H][width/32]; else NULL */
  int32_t dtype;         /* moe_dtype */
  int32_t scale;         /* moe_scale: NONE, PER_EXPERT or MX32 */
  int32_t layout;        /* moe_layout of w13, w2 and MX32 scales: must be MOE_LAYOUT_TILED */
  /* optional per-expert biases, fp32, each NULL for none (AITER PR 6106,
   * "Technical Details": added to the fp32 accumulator after the scales and
   * before the activation): b13 [n][2*width] (gate entries, then up entries)
   * on stage 1's a = x . W13^T; b2 [n][H] on stage 2's o = h . W2^T, before
   * the routing weight or the shared gate multiplies o */
  const float* b13;
  const float* b2;
} moe_weights;

/* Everything one layer forward needs. */
typedef struct {
  int32_t T, H, E, I, I_s, topk; /* I_s = 0: no shared expert; T = 0: empty batch (a no-op) */
  /* routing */
  int32_t score;            /* moe_score */
  int32_t n_group;          /* 1 = no groups; E % n_group == 0 */
  int32_t topk_group;       /* groups kept, 1 <= topk_group <= n_group */
  int32_t group_score_topk; /* group score = sum of its top-1 or top-2 scores */
  int32_t renormalize;      /* 1: weights renormalised over the k selected */
  float routed_scaling_factor;
  const float* logits; /* [T][E] fp32 router logits */
  const float* bias;   /* [E] fp32 selection bias (sigmoid scoring) or NULL */
  /* input activations */
  const void* x;             /* [T][H] */
  int32_t x_dtype;           /* moe_dtype */
  const float* x_row_scale;  /* A8W8: [T] fp32 per-token scale; else NULL */
  /* experts */
  moe_weights routed;
  moe_weights shared;
  const void* gate_w;  /* [H] in x's dtype (F32/BF16), NULL = ungated (gamma = 1) */
  int32_t shared_mode; /* moe_shared_mode */
  int32_t block_m;     /* rows per sorted block: 0 = automatic, else 16, 32, 64, 128 or 256 (not F32) */
  /* output */
  void* out;         /* [T][H] */
  int32_t out_dtype; /* F32 or BF16 */
  /* optional instrumentation: NULL, or 7 caller-created timing events: [0]
   * before the prologue, [1] after the prologue, [2] after the sort (recorded
   * on the main stream), [3]/[4] the start/end of the routed stage-1 GEMM
   * kernel and [5]/[6] those of the routed stage-2 GEMM kernel (stamped by
   * the kernels' own dispatch) */
  hipEvent_t* timing_events;
  int32_t activation; /* moe_activation of routed and shared experts (0 = SILU) */
  /* optional router projection [E][H], row-major (F32 when x is F32, else
   * BF16; F32 accumulation): when not NULL the layer computes the router
   * logits x . router_w^T itself in the prologue -- a GEMM launch before the
   * routing launch, or for F32 x one launch that also routes (A8W8: from the
   * dequantised codes, code * x_row_scale) -- and logits is not read (may be
   * NULL) */
  const void* router_w;
} moe_forward_args;

/* Pure host check of a forward request; makes no HIP call.  Returns MOE_OK,
 * MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED.  Preconditions (after vLLM PR
 * 65207, "Purpose", commit 2 conditions): out is exactly [T][H]; H, I, I_s are
 * multiples of 16 (of 32 for MX, AITER PR 6106 "Technical Details"), and of
 * the GEMM K tile (H % 128 and I % 128 for FP8, % 64 for BF16, % 32 for F32);
 * E % n_group == 0; topk <= topk_group * E / n_group; E / n_group >= 2 when
 * group_score_topk == 2; pointers 16-byte aligned; PSEUDO mode needs the
 * shared weights in the routed format (SGLang PR 27057, "Modifications") and,
 * for A8W8, I_s <= I (one row scale per shared row). */
moe_status moe_validate(const moe_forward_args* a);

/* Bytes of device workspace moe_forward needs for this request (0 on an
 * invalid request).  Depends on shapes, formats, mode and block_m only. */
size_t moe_workspace_bytes(const moe_forward_args* a);

/* The whole layer: the routed experts' output plus the gated shared expert's,
 * the shared part either fused into the routed grouped GEMM as always-selected
 * pseudo-experts (vLLM PR 61503, "Overview": one fused heterogeneous MoE op)
 * or run on a second stream whose result stage 2 accumulates as its addend
 * after waiting on a ready event right before stage 2 (vLLM PR 65207,
 * "Purpose", commit 2).  Launch sequence:
 *   PSEUDO/NONE: prologue (route + gate dot + MX quant of x) -> sort (also
 *                clears the arrival counters) -> stage 1 -> stage 2 (per-pair
 *                rows; the last arrival per (token, column tile) sums them in
 *                slot order and rounds once into out).  At T <= 64 with
 *                16-row blocks there is no sort launch (each block finds its
 *                pairs itself), and with softmax scores over E <= 64 experts
 *                (E a multiple of 4, no groups, bf16/fp32) the routing runs
 *                inside the stage-1 launch: stage 1 -> stage 2.
 *   AUX:         main runs the prologue and records ev_fork; aux waits on it
 *                and runs dense shared stage 1 and shared stage 2 (STORE of
 *                gamma*S(x) into the addend buffer), then records ev_ready.
 *                Main runs the sort and routed stage 1 concurrently, waits on
 *                ev_ready on the device, then routed stage 2 sums the addend
 *                and the routed pair rows.
 * workspace: device buffer of at least moe_workspace_bytes(a) bytes, 256-byte
 * aligned; its contents on entry are irrelevant.  main/aux: distinct streams
 * in AUX mode (aux ignored otherwise).  ev_fork/ev_ready: caller-created
 * events (ignored unless AUX).  The workspace and the events must not be used
 * by an overlapping call.  T = 0 returns MOE_OK after validation and touches
 * nothing (workspace, streams and events may be NULL). */
moe_status moe_forward(const moe_forward_args* a, void* workspace, size_t workspace_bytes,
                       hipStream_t main, hipStream_t aux, hipEvent_t ev_fork,
                       hipEvent_t ev_ready);

/* Largest workspace moe_forward_noalloc provides (bytes). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_forward without a caller workspace, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The workspace is a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES in the library, one copy per GPU, held until the
 * process ends; its address on the current device is looked up on the first
 * call on that device (the library's only other state: a mutex-guarded table
 * of those addresses).  Arguments and launch sequence as moe_forward; the
 * streams and events must belong to the current device.  Returns
 * MOE_ERR_WORKSPACE when moe_workspace_bytes(a) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (decode-sized batches fit: the workspace grows
 * with T * (topk + shared chunks) * H), MOE_ERR_HIP if the look-up fails.
 * Nothing is allocated.  Every call on a GPU shares that GPU's array, whose
 * contents a call never relies on: two calls that overlap in time on one
 * GPU (different streams, or the aux stream of one with the main stream of
 * the other) race and give undefined results. */
moe_status moe_forward_noalloc(const moe_forward_args* a, hipStream_t main, hipStream_t aux,
                               hipEvent_t ev_fork, hipEvent_t ev_ready);

/* ---- the individual steps (what moe_forward composes) ---------------- */

/* Top-k routing (vLLM PR 65207, "Purpose", commit 1).  One row per token:
 * topk_ids[t][j] (int32, rank order) and topk_w[t][j] (fp32) for j < topk,
 * weights = softmax probabilities (softmax scoring) or sigmoid scores (sigmoid
 * scoring), renormalised over the selection when renormalize != 0, times
 * routed_scaling_factor.  Sigmoid selection ranks sigmoid(logit) + bias;
 * softmax selection ranks logits; ties go to the lower expert (and group)
 * index.  Groups: n_group blocks of E/n_group consecutive experts, scored by
 * the sum of their top group_score_topk (1 or 2) selection scores; the best
 * topk_group groups are eligible.  Slots j = topk .. topk+n_pseudo-1 receive
 * id E + (j - topk) and weight gamma[t] (1 when gamma is NULL).
 * Arrays: logits [T][E], bias [E] or NULL, gamma [T] or NULL, topk_ids and
 * topk_w [T][topk + n_pseudo].  Limits: E <= 512, topk + n_pseudo <= 64. */
moe_status moe_route(const float* logits, const float* bias, int32_t T, int32_t E,
                     int32_t topk, int32_t n_group, int32_t topk_group,
                     int32_t group_score_topk, int32_t score, int32_t renormalize,
                     float routed_scaling_factor, int32_t n_pseudo, const float* gamma,
                     int32_t* topk_ids, float* topk_w, hipStream_t stream);

/* Shared-expert gate as a K-length dot product with the sigmoid folded in
 * (vLLM PR 56789, "Commits"): gate_out[t] = sigmoid(sum_h x[t][h] * g[h])
 * (apply_sigmoid != 0) or the plain dot, fp32 accumulation, fp32 output.
 * x [T][H] and g [H] in x_dtype (F32 or BF16). */
moe_status shared_gate_dot(const void* x, int32_t x_dtype, const void* g, int32_t T,
                           int32_t H, int32_t apply_sigmoid, float* gate_out,
                           hipStream_t stream);

/* Router logits l = x . router_w^T (the projection in front of the routing
 * of vLLM PR 65207, "Purpose", commit 1; the same matrix-core kernel
 * moe_forward runs for the same shapes, without the routing: for BF16 and
 * FP8_E4M3 x a tiled GEMM of 128 tokens x 64 experts per workgroup, whose
 * logits the forward then routes in a second launch; for F32 x the kernel of
 * the forward's fused prologue).  A forward fed these logits therefore routes
 * exactly as one given the router weights.
 * x [T][H] in x_dtype: F32 (router_w F32), BF16 (router_w BF16) or FP8_E4M3
 * codes with x_row_scale [T] fp32 (router_w BF16; l = scale_t * codes . w);
 * router_w [E][H] row-major; logits [T][E] fp32 out.  H % 64 == 0 (% 32 for
 * F32), E <= 512, pointers 16-byte aligned (x_row_scale 4).  Errors:
 * MOE_ERR_INVALID_ARG for bad shapes or pointers, MOE_ERR_UNSUPPORTED for
 * another x_dtype, MOE_ERR_HIP for a failed launch. */
moe_status moe_router_logits(const void* x, int32_t x_dtype, const float* x_row_scale, const void* router_w,
                             int32_t T, int32_t H, int32_t E, float* logits, hipStream_t stream);

/* In-layer MX-32 quantisation of bf16 activations (OCP MX v1.0; AITER PR
 * 6106, "Technical Details": 32-element K blocks, K % 32 == 0): per block of
 * 32 along H, scale byte = clamp(floor(log2 amax) - 8, -127, 127) + 127 (0 for
 * an all-zero block) and codes = e4m3 RNE of v * 2^-(byte-127), saturated to
 * +-448.  x [T][H] bf16 -> codes [T][H] uint8, scales [T][H/32] uint8. */
moe_status moe_quant_mx(const void* x, int32_t T, int32_t H, uint8_t* codes,
                        uint8_t* scales, hipStream_t stream);

/* Sorted-buffer capacity in rows: T*k_total + min(n_experts, T*k_total)*(block_m-1),
 * rounded up to a multiple of block_m.  Host-only. */
int32_t moe_sort_capacity(int32_t T, int32_t k_total, int32_t n_experts, int32_t block_m);

/* Device scratch bytes moe_sort_tokens can use to sort large pair counts
 * with two launches instead of one workgroup (0 when it would not use it).
 * Host-only. */
size_t moe_sort_scratch_bytes(int32_t T, int32_t k_total, int32_t n_experts);

/* Converts a row-major weight matrix (or several stacked ones) to the tiled
 * layout described at moe_layout.  src, dst: device, 16-byte aligned, not
 * overlapping, rows * row_bytes bytes each; rows % 16 == 0, row_bytes % 128 ==
 * 0.  The caller owns both buffers.  Asynchronous on stream. */
moe_status moe_pack_weights(const void* src, void* dst, int64_t rows, int32_t row_bytes,
                            hipStream_t stream);

/* Converts a row-major MX32 scale matrix ([rows][scale_bytes] e8m0 bytes,
 * scale_bytes = row_bytes / 32 of the matching weight matrix) to the tiled
 * layout.  rows % 16 == 0, scale_bytes % 4 == 0; src, dst: device, 4-byte
 * aligned, not overlapping.  Asynchronous on stream. */
moe_status moe_pack_mx_scales(const void* src, void* dst, int64_t rows, int32_t scale_bytes,
                              hipStream_t stream);

/* Token-by-expert sort (vLLM PR 65207, commit 2 and the review's sorting
 * experiment).  For pair p = t*k_total + j with expert topk_ids[p]:
 * counts[e] = number of pairs of expert e; offsets[e] = exclusive scan of the
 * counts padded to multiples of block_m (offsets has n_experts+1 entries);
 * sorted_pair_ids[offsets[e] + i] = i-th smallest pair index of expert e, the
 * padding slots and the tail up to capacity hold T*k_total; block_expert[b] =
 * expert of block b for b < *num_blocks (-1 after it, up to capacity/block_m);
 * *num_blocks = offsets[n_experts] / block_m.  Empty experts get no block.
 * scratch/scratch_bytes: optional device scratch of moe_sort_scratch_bytes()
 * bytes (NULL: one workgroup sorts everything; same result, slower for large
 * pair counts).  zero_ptr/zero_bytes (optional, zero_bytes % 16 == 0): a region
 * cleared by the same launch.  Arrays: sorted_pair_ids [capacity],
 * block_expert [capacity/block_m], counts [n_experts], offsets [n_experts+1].
 * Limits: n_experts <= 576, T*k_total < 2^31. */
moe_status moe_sort_tokens(const int32_t* topk_ids, int32_t T, int32_t k_total,
                           int32_t n_experts, int32_t block_m, int32_t capacity,
                           int32_t* sorted_pair_ids, int32_t* block_expert, int32_t* counts,
                           int32_t* offsets, int32_t* num_blocks, void* scratch,
                           size_t scratch_bytes, void* zero_ptr, size_t zero_bytes,
                           hipStream_t stream);

/* Arguments of the two GEMM stages.  Expert index e < E is routed expert e;
 * E <= e < E + n_pseudo is shared pseudo-expert p = e - E: rows
 * [p*I, min((p+1)*I, I_s)) of the shared gate and up halves and the same
 * columns of the shared W2 (exact by linearity of the down projection and the
 * elementwise activation-mul), with the same entries of the shared b13; the
 * shared b2 belongs to pseudo-expert 0 alone.  dense = 1 instead runs the whole shared expert
 * (width I_s) over tokens 0..T-1 with no sorted problem. */
typedef struct {
  int32_t T, H, E, I, I_s, n_pseudo, k_total;
  moe_weights routed, shared;
  /* stage-1 input: F32/BF16 x [T][H]; MXFP8: codes [T][H] + e8m0 x_scale
   * [T][H/32]; A8W8: codes [T][H] + fp32 x_scale [T] */
  const void* x;
  const void* x_scale;
  /* sorted problem (from moe_sort_tokens) */
  int32_t dense;
  int32_t block_m;    /* 16, 32, 64, 128 or 256 (not F32); dense mode: any of these */
  int32_t max_blocks; /* capacity / block_m (sorted) or ceil(T / block_m) (dense) */
  const int32_t* sorted_pair_ids;
  const int32_t* block_expert;
  const int32_t* num_blocks;
  /* stage-1 output h, one row per sorted slot (dense: per token), row stride
   * ld_h = I (sorted) or I_s (dense): F32/BF16 values; MXFP8: codes + e8m0
   * h_scale [rows][ld_h/32]; A8W8: BF16 values + h_scale = fp32 row amax
   * [rows] (must be zero before stage 1; stage 2 derives the row scale).
   * A8W8 stage 2 first quantises every row of h in place (the e4m3 codes
   * v * 448 / amax go to the first ld_h bytes of the row's 2*ld_h-byte
   * storage), so h holds codes, not BF16 values, after moe_stage2_accum. */
  void* h;
  void* h_scale;
  /* stage 2 */
  const float* pair_w; /* sorted: [T][k_total] pair weights (topk_w) */
  const float* gamma;  /* dense: [T] gate values or NULL (= 1) */
  float* acc;          /* STORE: [T][H] fp32 destination of gamma_t * S(x_t);
                          ACCUMULATE: [T][H] fp32 addend, or NULL for none */
  float* pair_out;     /* ACCUMULATE: scratch of T*k_total*H*4 bytes for the
                          per-pair rows pair_w[t][j] * E_{e_tj}(x_t), pair
                          t*k_total+j (contents on entry and exit unspecified) */
  void* out;           /* [T][H] in out_dtype, written by the last arrival */
  int32_t out_dtype;
  int32_t mode;        /* STORE (dense only) or ACCUMULATE (sorted only) */
  int32_t* counters;   /* ACCUMULATE: moe_stage2_counters(T, H) int32, zero on
                          entry: [T][H/64] arrival counts (per token and
                          64-column tile, or per token and group of tiles),
                          then the work-queue state of the stage-2 kernels */
  int32_t expected_arrivals; /* contributions per token: must equal k_total */
  hipEvent_t addend_ready;   /* waited on (device-side) before stage 2, or NULL */
  int32_t activation;        /* moe_activation (stage 1) */
} moe_stage_args;

/* Number of int32 counters moe_stage2_accum (ACCUMULATE) needs, all zero on
 * entry: T * (H/64) arrival counts, then 16 words of work-queue state. */
static inline size_t moe_stage2_counters(int32_t T, int32_t H) { return (size_t)T * (size_t)(H / 64) + 16; }

/* Stage 1 (vLLM PR 65207, "Purpose", commit 2 names the two AITER stages):
 * for every sorted block of rows of expert e, a = x_gathered . W13[e]^T in
 * fp32, times the per-token and per-expert scales (AITER PR 6106, "Technical
 * Details": applied to the fp32 accumulator before activation and fused
 * quantisation; MX scales per 32-element K block inside the K loop), then
 * h = SiLU(a_gate) * a_up, rounded/quantised to the stage-1 output format. */
moe_status moe_stage1(const moe_stage_args* a, hipStream_t stream);

/* Stage 2 with the shared-expert addend accumulated in its epilogue (vLLM PR
 * 65207, "Purpose", commit 2): o = h . W2[e]^T in fp32 times the scales.
 * ACCUMULATE stores pair_w * o as the pair's row in pair_out; the last of the
 * k_total contributions to a (token, 64-column tile) computes
 * addend + sum_j row[t*k_total + j] in fp32, j in slot order, and rounds it
 * once into out (deterministic: the result does not depend on the order in
 * which workgroups finish).  The one-wave kernels (16-row blocks) keep the
 * rows in fp32; the 32-128-row kernels store each (pair, 64-column tile) as
 * one 128-byte line of 16-bit words carrying 15-bit values and the tile's
 * power-of-two scale, which holds every value to within 2^-13 of the tile's
 * largest magnitude (a non-finite tile yields NaN).  STORE writes gamma_t * o into acc (the addend of
 * a later ACCUMULATE).  Waits on addend_ready first when it is not NULL. */
moe_status moe_stage2_accum(const moe_stage_args* a, hipStream_t stream);

/* Capability query (vLLM PR 65207, "Dependencies": the accumulate path is
 * feature-detected).  Returns 1 when supported, 0 otherwise. */
int32_t moe_query_feature(int32_t feature);

/* Static string for a status code. */
const char* moe_status_str(int32_t status);

/* Description of the HIP error behind the last MOE_ERR_HIP returned to the
 * calling thread ("" if none).  Every entry point that launches work first
 * drops an error left pending by the caller's earlier runtime calls, so a
 * MOE_ERR_HIP names a failure of this library's own calls. */
const char* moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
