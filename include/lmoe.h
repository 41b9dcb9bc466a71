/*
 * lmoe.h -- C ABI of the LatentMoE feed-forward layer (forward pass) on
 * AMD MI355X (gfx950).
 *
 * The layer (page "Nemotron 3 Ultra 架构深度拆解报告", CH5 §5.6 "7 步数据流",
 * Steps 1-7, router moved onto the latent as the page's summary (CH0) and the
 * page "NVIDIA Nemotron 3 Super 技术解读" §2.2 describe it):
 *
 *   z    = x W1^T                          fc1_latent            [T, R]
 *   l    = z Wg^T, s = sigmoid(l)          fp32 router           [T, E]
 *   I    = top-K of (s + bias), single group, ties to the lower expert id
 *   w    = rho * s[I] / (sum s[I] + 1e-20)  rho = routed_scaling_factor
 *   r    = sum_k w_k relu(z Wup[I_k]^T)^2 Wdn[I_k]^T            [T, R]
 *   y    = r W2^T + relu(x Wsu^T)^2 Wsd^T  fc2_latent + shared   [T, D]
 *
 * Optionally (lmoe_config.fuse) the layer also takes over the two steps of
 * its block on either side (page "Nemotron 3 Ultra 架构深度拆解报告", CH9 §9.3:
 * pre-norm RMSNorm, mixer, residual add); x is then the block's residual
 * stream h:
 *
 *   PRENORM   the layer runs on RMSNorm(h) = r * bf16(gamma * h) with
 *             r = 1 / sqrt(mean(h^2) + norm_eps) per token: the GEMM operand
 *             is the bf16 rounding of gamma * h and r scales the fp32 results
 *             of the latent and shared-up projections (RMSNorm in exact
 *             arithmetic, one bf16 rounding, placed where it can be
 *             reproduced exactly);
 *   RESIDUAL  y = h + (layer output), added in fp32 before the bf16 rounding.
 *
 * Sizes follow the model's config keys (page "Nemotron-3-Labs-Ultra-Math-SFT"
 * article, 核心配置速查表): D = hidden_size, R = moe_latent_size,
 * E = n_routed_experts, K = num_experts_per_tok, F = moe_intermediate_size,
 * S = moe_shared_expert_intermediate_size.
 *
 * Conventions for every entry point:
 *  - bf16 tensors are passed as uint16_t bit patterns; every matrix is
 *    row-major and dense, weights stored out x in (a linear layer's layout),
 *    expert weights as 3-D (expert, out, in) tensors (§5.1 of the page above);
 *  - all tensor pointers are DEVICE pointers, 16-byte aligned, owned by the
 *    caller; the library never allocates or frees device memory;
 *  - `stream` is a hipStream_t (NULL = the null stream); work is enqueued
 *    asynchronously and nothing synchronises the host;
 *  - arguments are checked on the host before any HIP call; on error nothing
 *    is enqueued and the status says why.  Device faults surface at the
 *    caller's next synchronisation.  Inputs must be finite.
 *  - one handle owns one workspace: lmoe_forward and lmoe_route on one
 *    handle use the same workspace (lmoe_route its router-logits part), so
 *    calls on one handle must not overlap: issue them on one stream, or
 *    order them with events.
 *  - lmoe_create creates one auxiliary HIP stream (non-blocking, default
 *    priority) and two events per handle, used to run the shared expert's up
 *    projection concurrently with the latent projection and the router
 *    (forked from `stream` at the start of the forward for small batches,
 *    after the latent projection otherwise, and joined back before the
 *    output projection); lmoe_destroy releases them.  A forward makes no
 *    other HIP object, so any forward (the first included) can be captured
 *    into a HIP graph.
 */
#ifndef LMOE_H
#define LMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMOE_OK = 0,
  LMOE_ERR_INVALID_ARG = -1,     /* NULL / misaligned / aliased pointer, bad value */
  LMOE_ERR_UNSUPPORTED = -2,     /* a configuration this library does not implement */
  LMOE_ERR_TOO_MANY_TOKENS = -3, /* T > max_tokens of the handle */
  LMOE_ERR_WORKSPACE = -4,       /* workspace missing or smaller than lmoe_workspace_size */
  LMOE_ERR_HIP = -5,             /* a HIP launch or copy returned an error */
  LMOE_ERR_SCRATCH = -6          /* lmoe_forward_noalloc: the forward needs more than
                                    LMOE_NOALLOC_SCRATCH_BYTES of scratch */
} lmoe_status;

/* Path selection for the expert and projection GEMMs.  AUTO picks by token
 * count: weight streaming for small batches, LDS-tiled MFMA otherwise (the
 * projections split over k into fp32 partial sums while T <= 256, to fill
 * the GPU); the other values force one tiling for every GEMM (used by tests;
 * TILED still splits the projections over k when T <= 256).  Results agree
 * across paths to rounding. */
typedef enum { LMOE_PATH_AUTO = 0, LMOE_PATH_STREAM = 1, LMOE_PATH_TILED = 2 } lmoe_path;

/* Storage of the routed experts' weights.  BF16: expert_up / expert_down.
 * MXFP4 (block-scaled FP4 with the E2M1 elements of CH8 §8.1 of the page
 * "Nemotron 3 Ultra 架构深度拆解报告"; block layout: lmoe_quantize_mxfp4):
 * the *_mxfp4 / *_scale fields; the expert GEMMs decode the weights exactly
 * to bf16, streaming them for small batches and, for large ones, copying
 * the FP4 codes into the LDS-tiled GEMM's tiles and decoding them right
 * before the MFMAs (the same lmoe_path choice as bf16 weights; R and F must
 * be multiples of 128).  Everything else stays bf16 / fp32. */
typedef enum { LMOE_EXPERTS_BF16 = 0, LMOE_EXPERTS_MXFP4 = 1 } lmoe_expert_format;

/* Block steps fused into the layer (bits of lmoe_config.fuse; CH9 §9.3 of
 * the page "Nemotron 3 Ultra 架构深度拆解报告"): the block's pre-norm RMSNorm
 * (needs lmoe_weights.norm_weight) and its residual add.  See the top of
 * this file for the exact arithmetic. */
typedef enum { LMOE_FUSE_PRENORM = 1, LMOE_FUSE_RESIDUAL = 2 } lmoe_fuse;

typedef struct {
  int32_t hidden_size;                         /* D; multiple of 64 */
  int32_t moe_latent_size;                     /* R; multiple of 64 */
  int32_t n_routed_experts;                    /* E; 1..1024 */
  int32_t num_experts_per_tok;                 /* K; 1..min(E, 64) */
  int32_t moe_intermediate_size;               /* F; multiple of 64 */
  int32_t moe_shared_expert_intermediate_size; /* S; multiple of 64 */
  int32_t n_group;    /* routing groups (§5.5): divides E into groups of >= 2
                         experts (any size when 1); at most 64 */
  int32_t topk_group; /* groups kept per token: 1..n_group, and
                         K <= topk_group * E / n_group */
  float routed_scaling_factor;                 /* rho, finite (5.0 in the model) */
  int32_t max_tokens;                          /* largest T a forward may use; sizes the workspace */
  int32_t path;                                /* lmoe_path */
  int32_t expert_format;                       /* lmoe_expert_format */
  int32_t fuse;                                /* lmoe_fuse bits; 0 = the layer alone */
  float norm_eps;                              /* RMSNorm epsilon, finite, >= 0 (PRENORM) */
} lmoe_config;

/* Device pointers; the handle borrows them and they must outlive it. */
typedef struct {
  const uint16_t *fc1_latent;  /* bf16 [R, D] */
  const float *router;         /* fp32 [E, R]  gate weight */
  const float *router_bias;    /* fp32 [E]     e_score_correction_bias */
  const uint16_t *expert_up;   /* bf16 [E, F, R] */
  const uint16_t *expert_down; /* bf16 [E, R, F] */
  const uint16_t *fc2_latent;  /* bf16 [D, R] */
  const uint16_t *shared_up;   /* bf16 [S, D] */
  const uint16_t *shared_down; /* bf16 [D, S] */
  /* MXFP4 experts (expert_format = LMOE_EXPERTS_MXFP4; else unused): */
  const uint8_t *expert_up_mxfp4;   /* [E, F, R/2] codes, 16-byte aligned */
  const uint8_t *expert_up_scale;   /* [E, F, R/32] block scales */
  const uint8_t *expert_down_mxfp4; /* [E, R, F/2] codes, 16-byte aligned */
  const uint8_t *expert_down_scale; /* [E, R, F/32] block scales */
  /* LMOE_FUSE_PRENORM only (may be NULL otherwise): */
  const uint16_t *norm_weight;      /* bf16 [D] RMSNorm weight gamma */
} lmoe_weights;

/* Optional device outputs of intermediate values (tests, monitoring).  Any
 * field may be NULL.  Shapes for a forward of T tokens: */
typedef struct {
  float *z_f32;           /* [T, R] fp32 latent (the router's input) */
  int32_t *topk_idx;      /* [T, K] selected experts, ascending id per token */
  float *topk_w;          /* [T, K] routing weights, same order as topk_idx */
  int32_t *expert_counts; /* [E] tokens routed to each expert */
  float *r_latent;        /* [T, R] fp32 weighted sum of expert outputs */
} lmoe_taps;

typedef struct lmoe_handle lmoe_handle;

/* Bytes of device workspace a handle with this configuration needs for
 * forwards of up to cfg->max_tokens tokens: the intermediate tensors of page
 * "Nemotron 3 Ultra 架构深度拆解报告", CH5 §5.6 Steps 1-7 (latent, router
 * logits, top-K, the expert-sorted rows of Step 6's grouping, the experts'
 * hidden and output rows, the weighted sum) plus the shared expert's hidden
 * rows; layout and sizes in the library source.  0 if the configuration is
 * invalid or unsupported.  Pure host function. */
size_t lmoe_workspace_size(const lmoe_config *cfg);

/* Set up one layer (the module of CH5 §5.6 of the page above, bound to its
 * weights): validate `cfg` and `w` (host checks first: on any error nothing
 * is created and *out is NULL), carve `workspace` (device memory of at
 * least lmoe_workspace_size(cfg) bytes, 256-byte aligned, caller-owned; the
 * library never frees it) and return a host-side handle in *out, which
 * borrows `w` and `workspace`.  Its only HIP calls create the handle's
 * auxiliary stream and two events on the current device (LMOE_ERR_HIP if
 * they fail, e.g. with no GPU; nothing is left behind).
 * Debug aid: if the environment variable LMOE_DEBUG is set (and not "0")
 * when the handle is created, lmoe_forward and lmoe_route synchronise the
 * stream (and the handle's auxiliary stream) after every stage and return
 * LMOE_ERR_HIP at the first stage whose launch or execution failed, naming
 * it on stderr.  Same kernels and results; such calls block the host and
 * cannot be captured into a HIP graph. */
lmoe_status lmoe_create(const lmoe_config *cfg, const lmoe_weights *w, void *workspace,
                        size_t workspace_bytes, lmoe_handle **out);

/* y = LatentMoE(x) for T tokens.  x: bf16 [T, D], y: bf16 [T, D] (must not
 * overlap x).  T = 0 is a no-op.  `taps` may be NULL.  Page steps 1-7.
 * With fuse bits set: x is the residual stream h and y = h + LatentMoE(
 * RMSNorm(h)) (or either part alone); taps->z_f32 is then the latent of the
 * normalised input. */
lmoe_status lmoe_forward(lmoe_handle *h, const uint16_t *x, int32_t T, uint16_t *y,
                         void *stream, const lmoe_taps *taps);

/* Router only (page steps 1-4 on a given latent): from z_f32 [T, R] fp32
 * write topk_idx [T, K] (ascending expert id) and topk_w [T, K]. */
lmoe_status lmoe_route(lmoe_handle *h, const float *z_f32, int32_t T, int32_t *topk_idx,
                       float *topk_w, void *stream);

/* MXFP4 quantiser for expert weights: w is bf16 [rows, cols] (row-major,
 * cols a multiple of 32, 16-byte aligned); writes codes [rows, cols/2]
 * (16-byte aligned; element 2i of a row in the low nibble of byte i, code
 * = sign bit 3 | E2M1 magnitude code 0..7 for 0, 0.5, 1, 1.5, 2, 3, 4, 6)
 * and scales [rows, cols/32] (block b of a row holds elements 32b..32b+31
 * and its value is 2^(scale - 127)).  Per block: e = floor(log2 max|w|) - 2
 * clipped to [-127, 127] (-127 for an all-zero block); each element is
 * |w| / 2^e rounded to the nearest E2M1 magnitude, ties to the even code,
 * clamped at 6, signed unless it rounds to 0.  Inputs must be finite.
 * Device pointers; asynchronous on `stream`. */
lmoe_status lmoe_quantize_mxfp4(const uint16_t *w, int64_t rows, int32_t cols, uint8_t *codes,
                                uint8_t *scales, void *stream);

/* Release a handle from lmoe_create: its auxiliary stream, events and any
 * profiling events, and the host-side handle (no device memory is freed:
 * the caller owns all of it).  Work already enqueued on the handle's
 * streams must have finished.  NULL is a no-op. */
void lmoe_destroy(lmoe_handle *h);

/* Static, NUL-terminated text for a status code of this header (not owned
 * by the caller); "unknown status" for any other value.  Pure host function. */
const char *lmoe_status_string(lmoe_status s);

/* ---- allocation-free forward --------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as lmoe_forward (same kernels, same results bit for bit) without a
 * handle or a workspace.  Its scratch (the workspace a handle for exactly T
 * tokens would need) lives in one static device array of
 * LMOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; at the full layer shape (hidden 8192, latent
 * 2048, 512 experts top-22) that covers up to about 90 tokens, e.g. the
 * 32-token decode batch.  Larger forwards return LMOE_ERR_SCRATCH before any
 * launch.  Nothing is allocated and no stream or event is created: the
 * shared expert runs on `stream` after the others.  The first call on a
 * device looks up the array's address there (make it outside graph
 * capture).  `cfg` and `w` are checked as by lmoe_create, x and y as by
 * lmoe_forward; T <= cfg->max_tokens; `stream` must belong to the current
 * device.  Every call on one GPU uses that GPU's one array (it keeps the
 * last call's contents; nothing in it needs clearing): calls that overlap
 * on one GPU, on any streams, race and give wrong results. */
#define LMOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
lmoe_status lmoe_forward_noalloc(const lmoe_config *cfg, const lmoe_weights *w,
                                 const uint16_t *x, int32_t T, uint16_t *y, void *stream);

/* ---- per-kernel timing (HIP events on the forward's stream) ------------ */

/* Number of timed stages of lmoe_forward and the name of stage i.  Stages
 * 0..7 run back to back on the forward's stream (the last one, proj_out,
 * includes the wait for the auxiliary stream; the first, proj_latent,
 * includes the pre-norm kernel when it is fused); stage 8 ("shared_up") is
 * timed on the auxiliary stream and overlaps the stages before proj_out.
 * For T <= 64 (weight-streaming projections) stage 8 also runs the shared
 * expert's down projection and proj_out covers fc2_latent only, adding the
 * shared output before its single rounding. */
int32_t lmoe_num_stages(void);
const char *lmoe_stage_name(int32_t i);

/* Start timing: the next up to `max_forwards` calls of lmoe_forward record
 * a HIP event before and after each stage (events are created here; a
 * hipEventCreate failure returns LMOE_ERR_HIP).  max_forwards <= 4096. */
lmoe_status lmoe_profile_begin(lmoe_handle *h, int32_t max_forwards);

/* Stop timing: wait for the recorded events, write the summed milliseconds
 * of each stage over the recorded forwards into ms[0..n_stages) and the
 * number of recorded forwards into *n_forwards; destroy the events. */
lmoe_status lmoe_profile_end(lmoe_handle *h, float *ms, int32_t n_stages, int32_t *n_forwards);

#ifdef __cplusplus
}
#endif

#endif /* LMOE_H */
