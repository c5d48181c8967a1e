/*
 * moe_fp4.h -- C ABI of the MI355X (gfx950) FP4 mixture-of-experts feed-forward layer.
 *
 * The layer is the MoE FFN component described on the MoE module page of the Rust
 * inference engine (spark_model/layers/moe/mod.rs): a router GEMM, top-K expert
 * selection (softmax; sigmoid with a per-expert correction bias; or a static
 * token-to-expert hash table), per selected expert a gate+up projection with
 * SiLU(gate)*up and a down projection, and a routing-weighted sum blended into
 * the residual. Expert weights are 4-bit E2M1 in NVFP4 or MXFP4 storage (doc of
 * MoeLayer.experts_scale_kind on that page).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless marked "host". The caller owns all memory;
 *   the library never allocates device memory. Scratch space is the caller's
 *   workspace (size from moe_workspace_size).
 * - Every call is asynchronous on `stream`: it validates on the host, enqueues
 *   kernels and returns. No call waits for the device, except
 *   moe_get_device_error, which synchronises `stream` to read the error word.
 * - With a shared expert whose launches would leave most of the chip idle (on the decode
 *   GEMV: below 8 tokens, or sizes the MFMA tiles do not take; on the MFMA kernels from 256
 *   tokens, whose K is then kept whole),
 *   moe_experts_forward and moe_layer_forward fork a side stream of `stream` (one per
 *   caller stream, created on the first such call made while `stream` is not being
 *   captured, non-blocking, default priority, kept until the process ends): the shared
 *   expert runs there beside the dispatch and the routed experts and is joined back by an
 *   event before the blend, so the call is still one ordered unit on `stream` (and captures
 *   into a graph as a fork and a join). Between the two (MFMA launches with K split over
 *   blocks, which fill the chip) it runs on `stream` after the routed experts.
 *   moe_layer_forward_noalloc never forks.
 *   Indices and weights stay on the device (module doc: no device-to-host sync).
 * - bf16 tensors are passed as uint16_t bit patterns; every activation is
 *   row-major [tokens, hidden]. Activations (x, x_experts, out, residual), norm_gamma,
 *   weight arrays and the workspace must be 16-byte aligned (the kernels use 128-bit
 *   loads); a misaligned pointer is rejected (MOE_ERR_INVALID_ARG, or MOE_ERR_WORKSPACE
 *   for the workspace).
 * - Host validation is O(1) and happens before any launch; a failing call
 *   enqueues nothing and returns a negative moe_status.
 * - Data errors that only the device can see (an expert id outside [0, E + Z), a
 *   token id outside [0, vocab), a hash-table entry outside [0, E + Z)) do not stop
 *   the call: the offending slot is dropped (id -1, weight 0) and bits are set
 *   in the workspace's device error word (moe_get_device_error).
 * - Results are deterministic: identical inputs give bitwise identical outputs
 *   (no floating-point atomics; fixed reduction orders).
 * - Calls that share one workspace must be ordered on one stream.
 */
#ifndef MOE_FP4_H
#define MOE_FP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point (0 = success). */
typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad dimension, misaligned pointer, bad mode */
  MOE_ERR_UNSUPPORTED = -2, /* valid request outside the library's limits (sizes, path) */
  MOE_ERR_WORKSPACE = -3,   /* workspace null or smaller than moe_workspace_size */
  MOE_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  MOE_ERR_FORMAT = -5       /* weight format tag unknown or inconsistent with its scales;
                               never silently decoded as the other format (cf. the
                               MoE module page, MoeLayer::e8m0_or: a format mismatch
                               must be loud) */
} moe_status;

/* Device error word bits (moe_get_device_error). */
enum {
  MOE_DEVERR_EXPERT_ID = 1, /* an expert id outside [0, num_experts) reached dispatch */
  MOE_DEVERR_TOKEN_ID = 2,  /* hash routing: a token id outside [0, vocab) */
  MOE_DEVERR_TABLE = 4,     /* hash routing: a tid2eid entry outside [0, num_experts) */
  MOE_DEVERR_Y_RANGE = 8    /* prefill: a routed expert output whose fp16 intermediate store
                               (round to nearest even) left the fp16 range (|y| >= 65520) or
                               was not finite; it was stored saturated to +-65504 */
};

/* Expert weight storage formats (MoE module page, doc of MoeLayer.experts_scale_kind;
 * MoE constructor page: the FP8 expert kernels and pointer tables, and the BF16 grouped
 * GEMM for FP8-source weights dequantised to BF16 at load). */
enum {
  MOE_FMT_NVFP4 = 0, /* E2M1 codes + one FP8-E4M3 (OCP "FN") scale per 16 values along K
                        + one f32 global scale per expert tensor: w = e2m1 * e4m3 * global */
  MOE_FMT_MXFP4 = 1, /* E2M1 codes + one E8M0 scale per 32 values along K: w = e2m1 * 2^(s-127) */
  MOE_FMT_FP8 = 2,   /* E4M3 (OCP "FN") codes + one f32 scale per 128 x 128 block (rows x K):
                        w = e4m3 * scale[n / 128][k / 128]; k <= 16384 */
  MOE_FMT_BF16 = 3   /* bf16 values, no scales */
};

/* Routing score (MoE module page: doc of correction_bias_dev; constructor page: top-K kernels). */
enum {
  MOE_SCORE_SOFTMAX = 0,       /* key = logit; weight = softmax probability */
  MOE_SCORE_SIGMOID = 1,       /* key = fp32(sigmoid(logit)) + correction_bias (selection only);
                                  weight = sigmoid(logit) */
  MOE_SCORE_SQRT_SOFTPLUS = 2, /* key = fp32(sqrt(softplus(logit))) + correction_bias
                                  (selection only); weight = sqrt(softplus(logit)) (the
                                  DeepSeek-V4 sqrtsoftplus top-K kernels of the constructor
                                  page); the score is evaluated in fp64, rounded once */
  MOE_SCORE_SOFTMAX_BIAS = 3   /* key = fp32(softmax probability) + correction_bias (selection
                                  only); weight = the probability (the LongCat softmax+bias
                                  top-K kernels of the constructor page); the probabilities
                                  are evaluated in fp64, rounded once */
};

/* Expert selection (MoE module page: doc of tid2eid_dev). */
enum {
  MOE_SELECT_TOPK = 0, /* the top_k largest keys; ties go to the lower expert index */
  MOE_SELECT_HASH = 1  /* ids = tid2eid[token_id][0..top_k); weights = score at those ids */
};

/* Expert-path choice (both paths compute the same function). */
enum {
  MOE_PATH_AUTO = 0,    /* decode when tokens*top_k/min(E, tokens*top_k) < 4 rows per expert
                           (and the decode limit below holds), else prefill */
  MOE_PATH_DECODE = 1,  /* HBM-streaming GEMV kernels (needs 4 * max(hidden, inter,
                           shared_inter) * 2 bytes <= MOE_DECODE_MAX_LDS) */
  MOE_PATH_PREFILL = 2  /* expert-grouped MFMA GEMM kernels (needs hidden, inter % 64 == 0) */
};

/* Build limits (checked on the host). */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOP_K 32
#define MOE_DECODE_MAX_LDS (160 * 1024) /* decode stages 4 activation rows per tile in LDS */

/* One projection of a group of experts, in storage form (host struct, device pointers).
 * K is contiguous per output row n in every format.
 *   NVFP4 / MXFP4:
 *     packed       uint8 [experts, n, k/2]: byte j of a row holds code 2j in its low nibble
 *                  and code 2j+1 in its high nibble
 *     scales       uint8 [experts, n, k/16] E4M3 codes (NVFP4) or [experts, n, k/32] E8M0
 *     global_scale f32 [experts] for NVFP4; must be NULL for MXFP4
 *   FP8:  packed uint8 [experts, n, k] E4M3 codes; scales f32 [experts, ceil(n/128),
 *         ceil(k/128)]; global_scale NULL
 *   BF16: packed bf16 [experts, n, k]; scales and global_scale NULL
 *   gate/up: n = inter, k = hidden.  down: n = hidden, k = inter.
 * packed and scales must be 16-byte aligned; k % 32 == 0. A weight whose pointers do not
 * match its format tag is MOE_ERR_FORMAT. */
typedef struct {
  int32_t format;
  const uint8_t* packed;
  const uint8_t* scales;
  const float* global_scale;
  int32_t experts;
  int32_t n;
  int32_t k;
} moe_fp4_weight;

/* The three projections of an expert group (routed: experts = num_experts; shared: 1). */
typedef struct {
  moe_fp4_weight gate;
  moe_fp4_weight up;
  moe_fp4_weight down;
} moe_expert_weights;

/* Layer configuration (host struct). */
typedef struct {
  int32_t tokens;       /* T >= 0 (T == 0: the call returns MOE_OK and touches no pointer) */
  int32_t hidden;       /* H, multiple of 32 */
  int32_t num_experts;  /* E in [1, MOE_MAX_EXPERTS] */
  int32_t top_k;        /* k in [1, min(E, MOE_MAX_TOP_K)] */
  int32_t inter;        /* I, routed-expert intermediate size, multiple of 32 */
  int32_t score_mode;   /* MOE_SCORE_* */
  int32_t select_mode;  /* MOE_SELECT_* */
  int32_t renormalize;  /* 1: divide the k weights by their sum */
  float routed_scaling; /* multiplies the (renormalised) routed weights; 1.0 = none */
  int32_t has_shared;   /* 1: one always-on shared expert with weight 1 */
  int32_t shared_inter; /* intermediate size of the shared expert (multiple of 32) */
  int32_t pre_norm;     /* 1: RMSNorm(x)*gamma feeds the experts; the router sees raw x
                           (MoE module page, doc of MoeLayer.pre_expert_norm) */
  float norm_eps;       /* RMSNorm epsilon */
  int64_t vocab;        /* hash routing: rows of tid2eid */
  int32_t path;         /* MOE_PATH_* */
  int32_t zero_experts; /* Z >= 0 zero-computation experts (constructor page: the LongCat
                           router logit width num_experts + zero_expert_num and its
                           zero-expert add kernel). The router then has E + Z outputs
                           (router_w [E + Z, H]; logit_bias, correction_bias, logits
                           [.., E + Z]) and a slot whose id is in [E, E + Z) adds
                           weight * expert input (identity) instead of running an expert.
                           E + Z <= MOE_MAX_EXPERTS, top_k <= E + Z. */
} moe_config;

/* Human-readable name of a moe_status value (host; static string). */
const char* moe_status_string(int status);

/* Bytes of workspace that moe_route / moe_experts_forward / moe_layer_forward need for
 * `cfg` (host; pure function of the config). One workspace serves all three calls.
 * The MoE module page keeps the layer's scratch in fixed-size device buffers sized once
 * at construction so that a captured graph can replay the layer (field docs of
 * zero_accum_dev and of the routing/dispatch buffers); here the caller owns that memory
 * and sizes it with this query. Returns MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED for a
 * config the other calls would reject, else writes *bytes_out (host pointer). */
int moe_workspace_size(const moe_config* cfg, size_t* bytes_out);

/* Router + top-K selection (constructor page: router GEMM with fp32 output and the
 * softmax / sigmoid-with-bias / hash top-K kernels).
 *   x            bf16 [T, H] router input; may be NULL when logits_in is given
 *   (E + Z router outputs: Z = cfg->zero_experts, usually 0)
 *   router_w     bf16 [E + Z, H]; may be NULL when logits_in is given
 *   logit_bias   f32 [E + Z] added to every logit before scoring, or NULL
 *   correction_bias f32 [E + Z] (sigmoid, sqrt-softplus, softmax+bias; selection key
 *                only), or NULL
 *   token_ids    int32 [T] (hash only), tid2eid int64 [vocab, top_k] (hash only)
 *   logits_in    f32 [T, E + Z]: route from these logits instead of computing them, or NULL
 *   logits_out   f32 [T, E + Z] receives the logits, or NULL
 *   topk_ids     int32 [T, top_k] out: best first (key descending, then index ascending);
 *                -1 marks a slot dropped by a data error (hash routing)
 *   topk_w       f32 [T, top_k] out: routing weights (0 for dropped slots)
 * Logits are fp32(x . W_r^T + logit_bias), the dot product accumulated in fp64 and
 * rounded once. */
int moe_route(const moe_config* cfg, const uint16_t* x, const uint16_t* router_w,
              const float* logit_bias, const float* correction_bias,
              const int32_t* token_ids, const int64_t* tid2eid, const float* logits_in,
              float* logits_out, int32_t* topk_ids, float* topk_w, void* workspace,
              size_t workspace_bytes, hipStream_t stream);

/* Experts + weighted-sum blend for given routing (module doc: gate+up, SiLU*up, down;
 * weighted-sum blend into the residual).
 *   x_experts  bf16 [T, H] expert input (already normalised if a pre-norm applies)
 *   topk_ids   int32 [T, top_k], topk_w f32 [T, top_k]: ids in [E, E + Z) are zero-
 *              computation experts (y = x_experts row); ids outside [0, E + Z) are dropped
 *              and flagged MOE_DEVERR_EXPERT_ID
 *   routed     host struct of the routed experts (experts == E, gate/up n == inter)
 *   shared     host struct of the shared expert (experts == 1), or NULL if !has_shared
 *   residual   bf16 [T, H], or NULL for zero
 *   out        bf16 [T, H]: bf16_rne(residual + sum_j w_j y_j + y_shared), fp32 sum in
 *              slot order; may alias residual, must not alias x_experts */
int moe_experts_forward(const moe_config* cfg, const uint16_t* x_experts,
                        const int32_t* topk_ids, const float* topk_w,
                        const moe_expert_weights* routed, const moe_expert_weights* shared,
                        const uint16_t* residual, uint16_t* out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* The whole layer: [RMSNorm] -> router -> top-K -> experts -> blend (MoE module page,
 * module doc: router GEMM, top-K selection, gate+up with SiLU*up, down, then the
 * routing-weighted sum blended into the residual; doc of pre_expert_norm for the
 * optional RMSNorm of the expert input). Routing decisions stay on the device; the call
 * never synchronises with the host (module doc). Errors as for moe_route and
 * moe_experts_forward; nothing is enqueued when the host checks fail.
 *   norm_gamma bf16 [H] (pre_norm only; 16-byte aligned)
 *   dbg_logits f32 [T, E + Z], dbg_ids int32 [T, top_k], dbg_w f32 [T, top_k]: optional
 *              copies of the routing decisions (NULL to skip)
 * Other arguments as in moe_route and moe_experts_forward. */
int moe_layer_forward(const moe_config* cfg, const uint16_t* x, const uint16_t* norm_gamma,
                      const uint16_t* router_w, const float* logit_bias,
                      const float* correction_bias, const int32_t* token_ids,
                      const int64_t* tid2eid, const moe_expert_weights* routed,
                      const moe_expert_weights* shared, const uint16_t* residual,
                      uint16_t* out, float* dbg_logits, int32_t* dbg_ids, float* dbg_w,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Largest workspace moe_layer_forward_noalloc can use (its fixed device array per GPU). */
#define MOE_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)

/* moe_layer_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments and results
 * as moe_layer_forward, without the workspace: the layer's scratch is a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, which that GPU holds from the
 * first such call on it until the process ends (that call also looks its address up, on the
 * device of `stream`). The call itself allocates nothing. A config whose workspace
 * (moe_workspace_size) exceeds MOE_NOALLOC_SCRATCH_BYTES is rejected with MOE_ERR_WORKSPACE
 * before anything is enqueued. Every call on one GPU shares that GPU's array and leaves the
 * last call's contents in it, so calls that may overlap on one GPU (different streams, or
 * different host threads without ordering) race; order them on one stream. Nothing in the
 * array needs to start at zero: every call writes what it reads. */
int moe_layer_forward_noalloc(const moe_config* cfg, const uint16_t* x,
                              const uint16_t* norm_gamma, const uint16_t* router_w,
                              const float* logit_bias, const float* correction_bias,
                              const int32_t* token_ids, const int64_t* tid2eid,
                              const moe_expert_weights* routed, const moe_expert_weights* shared,
                              const uint16_t* residual, uint16_t* out, float* dbg_logits,
                              int32_t* dbg_ids, float* dbg_w, hipStream_t stream);

/* Test entry: decode expert `expert` of `w` to f32 [n, k] with the device routine of
 * the chosen path (MOE_PATH_DECODE: E2M1 to bf16 then the block scale as an fp32
 * factor; MOE_PATH_PREFILL: the bf16 MFMA operand), times the NVFP4 global scale.
 * Every value is exact, so the result is bit-comparable with the format definition. */
int moe_debug_dequant_fp4(const moe_fp4_weight* w, int32_t expert, int32_t path, float* out,
                          hipStream_t stream);

/* Measurement probes (not part of the layer): the achievable rates that the kernels'
 * rooflines are read against, reproducible with bench.py --microbench. Each enqueues one
 * kernel on `stream` and returns at once; the caller times it (events) and owns every
 * buffer. None reads or writes anything but the buffers named here.
 *
 * moe_probe_stream_read: reads `bytes` (a multiple of 16) from `src` (16-byte aligned)
 *   with 16-byte loads, one contiguous chunk per block of 256 threads over
 *   MOE_PROBE_READ_BLOCKS blocks, eight loads in flight per thread. `sink`:
 *   MOE_PROBE_READ_BLOCKS floats, written only on a data pattern that never occurs (it
 *   keeps the loads). MOE_ERR_INVALID_ARG on a null or misaligned pointer or a bad size.
 * moe_probe_mfma_blocks: blocks that moe_probe_mfma launches for `blocks_per_cu` (1 or 2):
 *   compute units x blocks_per_cu, or a negative moe_status.
 * moe_probe_mfma: each 4-wave block (one wave per SIMD) runs `iters` rounds of 8
 *   independent MFMAs on register operands. kind 0: v_mfma_f32_32x32x16_bf16 (32768
 *   flops each); kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 x E4M3 operands
 *   (131072 flops each; the pages' block-scaled FP4 MMA, MoE constructor page); kind 2:
 *   the prefill GEMM's step, two MXFP4 operands decoded to bf16 per 8 bf16 MFMAs.
 *   `sink`, `cycles`: moe_probe_mfma_blocks(blocks_per_cu) entries each; cycles[b] =
 *   shader-clock cycles (s_memtime) between block b's first and last instruction. */
#define MOE_PROBE_READ_BLOCKS 2048
int moe_probe_stream_read(const void* src, size_t bytes, float* sink, hipStream_t stream);
int moe_probe_mfma_blocks(int32_t blocks_per_cu);
int moe_probe_mfma(int32_t kind, int32_t iters, int32_t blocks_per_cu, float* sink,
                   uint64_t* cycles, hipStream_t stream);

/* Profiling aid: stage boundaries of moe_layer_forward, in launch order. */
enum {
  MOE_STAGE_BEGIN = 0,        /* before the first kernel of the call */
  MOE_STAGE_ROUTED = 1,       /* after RMSNorm (if any), the router GEMM and the top-K; with
                                 few tokens the top-K runs fused with the dispatch build
                                 and is counted in the next stage */
  MOE_STAGE_DISPATCHED = 2,   /* after the dispatch build */
  MOE_STAGE_GATE_UP = 3,      /* after the routed experts' gate+up (+SiLU*up) kernel */
  MOE_STAGE_DOWN = 4,         /* after the routed experts' down kernel */
  MOE_STAGE_SHARED = 5,       /* after the shared expert's two kernels (none: same as DOWN) */
  MOE_STAGE_COMBINED = 6,     /* after the weighted-sum blend */
  MOE_STAGE_COUNT = 7
};

/* Profiling aid (host): the NEXT moe_layer_forward call made on this host thread
 * records events[i] (caller-created HIP events) on its stream at boundary i, for
 * i < count (NULL entries are skipped), then forgets the array. Elapsed times between
 * consecutive events are the stage durations on that stream. events == NULL cancels a
 * pending request. */
int moe_set_stage_events(hipEvent_t* events, int32_t count);

/* Synchronise `stream`, then copy the device error word of `workspace` (MOE_DEVERR_*
 * bits of the last moe_experts_forward / moe_layer_forward on it) to *host_err. */
int moe_get_device_error(const void* workspace, size_t workspace_bytes, int32_t* host_err,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP4_H */
