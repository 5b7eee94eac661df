/*
 * lmoe — latent mixture-of-experts block forward on AMD MI355X (gfx950).
 *
 * C ABI of the library liblmoe.so. The block computed by lmoe_forward is the one
 * described for Muse Spark Open's MoE layers (LMSYS blog "SGLang and Miles Add
 * Day-0 Support for Muse Spark Open", section "MoE with pooler, unpooler and
 * per-expert normalization"; vLLM day-0 summary, section "Latent MoE"):
 *
 *   logits = x . W_router^T (+ b_router)                  [T, E]   fp32
 *   ids, w = top-k(logits), softmax over the k selected    [T, k]
 *   P      = x . W_pool^T                                  [T, Dp]
 *   xp     = P / sqrt(mean(P^2) + eps_pool) * g_pool
 *   for each selected expert e of token t (slot j):
 *     h    = silu(xp . W_gate[e]^T) * (xp . W_up[e]^T)     [F]
 *     y    = h . W_down[e]^T                               [Dp]
 *     z    = y / sqrt(mean(y^2) + eps_expert) * g_expert[e]
 *   u      = sum_j w_j * z_j    (accumulated in fp32)      [T, Dp]
 *   out    = u . W_unpool^T                                [T, D]
 *
 * Precision (BF16 activations): fp32 accumulation everywhere; router logits,
 * routing weights and the weighted sum are fp32; the pooled expert input xp, the
 * SwiGLU output h, each expert output y (whose RMS is taken from its BF16 values,
 * as the blog's "Fused per-expert post-norm" section describes) and the sum u
 * (the unpooler's GEMM input) are held as bfloat16.
 *
 * Conventions for every function below:
 *  - Pointers inside lmoe_weights / lmoe_aux and the x / out arguments are DEVICE
 *    pointers on the device that was current at lmoe_create; every other pointer
 *    is a host pointer. Device pointers must be 16-byte aligned.
 *  - All matrices are row-major; weights use the [out][in] convention, so every
 *    GEMM reads both operands along the contiguous inner dimension.
 *  - Functions return an lmoe_status. On an error nothing is enqueued and
 *    lmoe_last_error() describes it (thread-local). No C++ exception crosses
 *    this interface.
 */
#ifndef LMOE_H
#define LMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LMOE_ABI_VERSION 1

typedef struct lmoe_ctx* lmoe_handle;

typedef enum {
  LMOE_OK = 0,
  LMOE_E_INVAL = -1,        /* bad argument: null/misaligned pointer, bad size, T > max_tokens */
  LMOE_E_UNSUPPORTED = -2,  /* valid but not implemented: shape or dtype combination */
  LMOE_E_NOMEM = -3,        /* workspace allocation failed */
  LMOE_E_HIP = -4           /* a HIP runtime call or kernel launch failed */
} lmoe_status;

typedef enum {
  LMOE_F32 = 0,
  LMOE_BF16 = 1,
  LMOE_MXFP4 = 2,           /* expert weights: E2M1 codes + one E8M0 scale per 32 along K */
  LMOE_MXFP8_E4M3 = 3       /* not a configuration value: the format the MXFP4 path gives its
                               expert inputs (see lmoe_mx_quantize_e4m3) */
} lmoe_dtype;

#define LMOE_FLAG_ROUTER_BIAS 1u   /* lmoe_weights.b_router is present */
#define LMOE_FLAG_PACKED_EXPERTS 2u /* w_gate_up and w_down are in the packed expert
                                       layout (lmoe_pack_experts); needs bf16
                                       activations and experts, d_pooled a multiple
                                       of 256, d_ff a multiple of 128, and
                                       max_tokens * top_k * max(d_ff, d_pooled) * 2
                                       and 4 * d_ff * d_pooled below 2^31 */

/* Block configuration (host struct, copied at create).
 * Shapes: d_model (D), d_pooled (Dp), d_ff (F) must be multiples of 64;
 * 1 <= n_experts (E) <= 1024; 1 <= top_k (k) <= min(E, 16); max_tokens >= 1.
 * act_dtype: LMOE_F32 or LMOE_BF16 — dtype of x, W_router, W_pool, W_unpool.
 * expert_wdtype: act_dtype, or LMOE_MXFP4 (with act_dtype LMOE_BF16, d_pooled
 * and d_ff multiples of 1024): MXFP4 expert weights as the LMSYS blog's "NVFP4
 * as a third MMA type" section describes the format (E2M1 values, one UE8M0
 * scale per 32 along K; encodings of OCP Microscaling v1.0). The experts'
 * inputs — the normalized pooled row xp and the SwiGLU output h — are then
 * quantized on the fly to MXFP8 E4M3 blocks of 32 (lmoe_mx_quantize_e4m3's
 * rule), multiplied on the block-scaled MFMA with fp32 accumulation, and each
 * expert output is held as bfloat16 as in the BF16 configuration.
 * out_dtype: LMOE_F32 (the unpooler's fp32 accumulators as they are) or
 * act_dtype (those accumulators rounded to nearest even).
 * Gammas and the router bias are always fp32. */
typedef struct {
  int32_t abi_version;      /* LMOE_ABI_VERSION */
  int32_t d_model;
  int32_t d_pooled;
  int32_t d_ff;
  int32_t n_experts;
  int32_t top_k;
  float eps_pool;           /* RMSNorm eps of the pooled input */
  float eps_expert;         /* RMSNorm eps of each expert output */
  int32_t act_dtype;        /* lmoe_dtype */
  int32_t expert_wdtype;    /* lmoe_dtype */
  int32_t out_dtype;        /* lmoe_dtype: LMOE_F32 or act_dtype */
  int32_t max_tokens;       /* the workspace is sized for this many tokens */
  uint32_t flags;           /* LMOE_FLAG_* */
} lmoe_config;

/* Weights: device pointers, BORROWED. The caller keeps them alive and unchanged
 * until lmoe_destroy; the library never copies or repacks them. */
typedef struct {
  const void* w_router;     /* [E][D]   act_dtype */
  const float* b_router;    /* [E] fp32, required iff flags has LMOE_FLAG_ROUTER_BIAS */
  const void* w_pool;       /* [Dp][D]  act_dtype */
  const float* g_pool;      /* [Dp] fp32 */
  const void* w_gate_up;    /* [E][2F][Dp]: rows [0, F) gate, rows [F, 2F) up.
                               MXFP4: [E][2F][Dp/2] bytes, element 2i in the low nibble */
  const uint8_t* s_gate_up; /* MXFP4: [E][2F][Dp/32] E8M0 scales; otherwise NULL */
  const void* w_down;       /* [E][Dp][F]. MXFP4: [E][Dp][F/2] bytes */
  const uint8_t* s_down;    /* MXFP4: [E][Dp][F/32] E8M0 scales; otherwise NULL */
  const float* g_expert;    /* [E][Dp] fp32 */
  const void* w_unpool;     /* [D][Dp]  act_dtype */
} lmoe_weights;

/* Optional outputs of the routing steps (device pointers; any may be NULL).
 * Filled by the same lmoe_forward call, asynchronously on its stream. */
typedef struct {
  float* logits;            /* [T][E] fp32, bias included */
  int32_t* topk_ids;        /* [T][k], logit descending (NaN as -inf), ties to the lower expert id */
  float* topk_w;            /* [T][k] softmax of the selected logits (non-finite: see below) */
  int32_t* expert_offsets;  /* [E+1] exclusive prefix sum of the per-expert counts */
  int32_t* sorted_assign;   /* [T*k] assignment t*k+j at each sorted position;
                               order (expert asc, token asc) */
} lmoe_aux;

/* Create a handle: validates cfg and the weight pointers, allocates the
 * workspace for cfg->max_tokens on the current device. *out receives the handle
 * (NULL on error). */
lmoe_status lmoe_create(const lmoe_config* cfg, const lmoe_weights* w, lmoe_handle* out);

/* Non-finite values. Router logits that are NaN (a NaN or an infinity in the
 * token's x row makes them so) rank as -inf, and ties, -inf ones included, go
 * to the lower expert id, so every token selects k distinct valid experts and
 * the permutation stays exact. The weights are the softmax of the selected
 * logits (NaN read as -inf); when the largest selected one is infinite (all
 * -inf, e.g. a -inf router bias on every expert, or some +inf) they are equal
 * shares among the slots holding it and 0 elsewhere. A token whose x row holds
 * a NaN gets NaN outputs; rows never mix, so other tokens are unaffected. */

/* Run the block on T tokens: x [T][D] -> out [T][D] (out_dtype), enqueued on
 * hip_stream (a hipStream_t; NULL is the null stream). Asynchronous: kernel
 * faults surface at the caller's next synchronization. T == 0 enqueues nothing
 * and returns LMOE_OK; T > max_tokens is LMOE_E_INVAL. out must not overlap x.
 * The handle's workspace is shared: calls on one handle must not overlap in time
 * (use one stream per handle). aux may be NULL.
 * A call may be captured into a HIP graph (stream capture) and the graph
 * replayed: it enqueues kernels only (no allocation, memset or host
 * synchronization); a replay computes what the captured call computed, for the
 * same x, out, T and aux pointers. Stage timing (lmoe_set_timing) records
 * nothing while the stream captures. */
lmoe_status lmoe_forward(lmoe_handle h, const void* x, void* out, int32_t T, void* hip_stream,
                         const lmoe_aux* aux);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as lmoe_forward, with the same results bit for bit, but with no
 * handle and no lmoe_create, and allocating nothing. cfg and w are checked as
 * lmoe_create checks them (cfg->max_tokens bounds T) and are not kept; x, out,
 * T, hip_stream and aux are as for lmoe_forward. The workspace is the
 * library's static scratch of LMOE_NOALLOC_SCRATCH_BYTES per device (held by
 * each GPU the library runs on until the process ends), laid out for T tokens;
 * a T whose workspace (lmoe_workspace_bytes with max_tokens = T) exceeds it is
 * LMOE_E_INVAL, with nothing enqueued. At the full Muse Spark Open shapes that
 * admits T <= 301 with BF16 experts (36.4 MiB at T = 128) and T <= 382 with
 * MXFP4 experts.
 * Every call on a GPU shares that GPU's scratch: calls on one device must not
 * overlap in time (one stream, or ordered streams), or they race. The first
 * call on a device looks up the scratch's address there. */
#define LMOE_NOALLOC_SCRATCH_BYTES (64u << 20)

lmoe_status lmoe_forward_noalloc(const lmoe_config* cfg, const lmoe_weights* w, const void* x, void* out,
                                 int32_t T, void* hip_stream, const lmoe_aux* aux);

/* Free the workspace and the handle. NULL is allowed (LMOE_OK). The caller must
 * make sure no enqueued forward on this handle is still running. */
lmoe_status lmoe_destroy(lmoe_handle h);

/* Quantize n fp32 values (device pointer x, n a multiple of 32) to MXFP8 E4M3
 * (OCP Microscaling v1.0): each block of 32 consecutive values shares one E8M0
 * scale 2^X with X = floor(log2(max |v|)) - 8, clamped to [-127, 127] (an
 * all-zero block takes -127); each value becomes the E4M3 code of v / 2^X,
 * rounded to nearest with ties to even and saturated at 448. codes: n bytes,
 * scales: n/32 bytes (device). x and codes 16-byte aligned; values finite.
 * This is the rule the MXFP4-expert path applies to its expert inputs.
 * Asynchronous on hip_stream; LMOE_E_INVAL on bad arguments (nothing enqueued). */
lmoe_status lmoe_mx_quantize_e4m3(const float* x, int64_t n, uint8_t* codes, uint8_t* scales,
                                  void* hip_stream);

/* Re-encode NVFP4 expert weights as MXFP4 (the form lmoe_create takes with
 * expert_wdtype LMOE_MXFP4), for checkpoints stored in NVFP4.
 * NVFP4 as the LMSYS blog's "NVFP4 as a third MMA type" section describes it:
 * E2M1 values with one UE4M3 block scale per 16 elements, plus one FP32 scale
 * per weight matrix; its "AMD support" section runs such a checkpoint on
 * MI355X through the MXFP4 path. Each element's value e2m1 * ue4m3 * g is
 * formed in FP32 (the minifloat product is exact; the product with g rounds to
 * nearest-even), then every 32-element block is MX-quantized as OCP
 * Microscaling v1.0 gives it for MXFP4: shared exponent X = floor(log2(amax))
 * - 2, clamped to [-127, 127] (an all-zero block takes -127); each element is
 * the E2M1 code of v / 2^X, nearest with ties to even, saturated at 6; -0 is
 * stored as +0. The UE4M3 byte's top bit is ignored. A block with a NaN scale
 * (0x7F), a non-finite g or a value that overflows FP32 gets the E8M0 NaN
 * scale 0xFF and zero codes.
 * Layouts (device, row-major; element 2i of a row in the low nibble of byte i):
 *   codes        [n_mats][rows][cols/2]   E2M1, 16-byte aligned
 *   scales16     [n_mats][rows][cols/16]  UE4M3, 2-byte aligned
 *   global_scale [n_mats]                 FP32 (one per matrix), 4-byte aligned
 *   out_codes    [n_mats][rows][cols/2]   E2M1, 16-byte aligned; may be codes
 *                                         itself (in place), else disjoint
 *   out_scales   [n_mats][rows][cols/32]  E8M0, disjoint from everything else
 * cols must be a multiple of 32; a zero size enqueues nothing. For a layer's
 * experts, n_mats = E with rows = 2F, cols = Dp (gate/up) or rows = Dp,
 * cols = F (down). Asynchronous on hip_stream; LMOE_E_INVAL on bad arguments
 * (nothing enqueued); the caller owns every buffer. */
lmoe_status lmoe_nvfp4_to_mxfp4(const uint8_t* codes, const uint8_t* scales16, const float* global_scale,
                                int64_t n_mats, int64_t rows, int64_t cols, uint8_t* out_codes,
                                uint8_t* out_scales, void* hip_stream);

/* Copy bf16 expert weights into the packed expert layout that lmoe_create
 * reads with LMOE_FLAG_PACKED_EXPERTS (a load-time step, like the re-encoding
 * above; the forward then streams each 64-row x 64-column piece of a weight
 * matrix as one contiguous 8 KiB block instead of 64 row segments 2 cols bytes
 * apart). Not a step of the block's computation: the same values, reordered.
 * Each of the n_mats matrices is [rows][cols] bf16 row-major in src; in dst it
 * is a sequence of blocks of 64 rows x 64 columns, block (g, s) (rows
 * [64 g, 64 g + 64), columns [64 s, 64 s + 64)) at element offset
 * (g * cols / 64 + s) * 4096 of the matrix, its row r at r * 64 and column c at
 * c; matrices follow each other every rows * cols elements, as in src. rows and
 * cols must be multiples of 64; src and dst are device pointers, 16-byte
 * aligned, and must not overlap; a zero size enqueues nothing. For a layer's
 * experts: n_mats = E with rows = 2F, cols = Dp (w_gate_up) and rows = Dp,
 * cols = F (w_down). Asynchronous on hip_stream; LMOE_E_INVAL on bad arguments
 * (nothing enqueued); the caller owns both buffers. */
lmoe_status lmoe_pack_experts(const void* src, void* dst, int64_t n_mats, int64_t rows, int64_t cols,
                              void* hip_stream);

/* Device workspace bytes a handle with this configuration allocates. */
lmoe_status lmoe_workspace_bytes(const lmoe_config* cfg, size_t* out);

/* Per-stage device timing. When enabled, lmoe_forward records a HIP event pair
 * around every stage on its stream; lmoe_get_timing waits for the recorded
 * events and returns the accumulated milliseconds per stage and the number of
 * forward calls timed, then resets the accumulators. */
typedef enum {
  LMOE_STAGE_PROJ_IN = 0,   /* router + pooler GEMM (one launch) */
  LMOE_STAGE_TOPK = 1,      /* top-k + softmax + per-chunk expert masks */
  LMOE_STAGE_SORT = 2,      /* counting-sort scan + scatter + tile list */
  LMOE_STAGE_POOL_NORM = 3, /* pooled RMSNorm */
  LMOE_STAGE_GATE_UP = 4,   /* grouped gate/up GEMM + SwiGLU */
  LMOE_STAGE_DOWN = 5,      /* grouped down GEMM + sum-of-squares partials */
  LMOE_STAGE_COMBINE = 6,   /* per-expert RMSNorm + weighted sum */
  LMOE_STAGE_UNPOOL = 7,    /* unpooler GEMM */
  LMOE_NUM_STAGES = 8
} lmoe_stage;

lmoe_status lmoe_set_timing(lmoe_handle h, int enable);
lmoe_status lmoe_get_timing(lmoe_handle h, float* ms_per_stage /* [LMOE_NUM_STAGES] */,
                            int32_t* n_forward);

/* Static description of a status code. */
const char* lmoe_status_str(lmoe_status s);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* lmoe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LMOE_H */
