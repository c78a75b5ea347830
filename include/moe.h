/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts block.
 *
 * One MoE block maps each token's hidden vector x_t (length d) to an output
 * vector of the same length. The block is the one the Qwen3.6 / Qwen3.8-Max
 * pages describe:
 *   - a linear router gives one score (logit) per expert from the token's
 *     embedding (Qwen3.6 neural-network explorer page, section on the MoE
 *     router);
 *   - a softmax over the experts and a per-token top-k keep the k most probable
 *     experts (same section), optionally renormalising their k probabilities to
 *     sum to one;
 *   - each kept expert is a SwiGLU feed-forward network
 *     y = (silu(x Wg) * (x Wu)) Wd without biases (hidden_act "silu",
 *     moe_intermediate_size: Qwen3.8-Max architecture page, config.json
 *     listing; the overview page's parameter table counts three d x I matrices
 *     per expert), and the k outputs are summed with their routing weights;
 *   - one shared expert of size shared_expert_intermediate_size runs on every
 *     token and is added with no weight (explorer page, router section;
 *     Qwen3-Next article on hyper.ai).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, owned by the caller, row-major
 *     and densely packed. The library never allocates, frees or synchronises;
 *     all work is enqueued in order on `stream` and its results are valid once
 *     the stream reaches them. Device faults surface at the caller's next sync.
 *   - Floating tensors of x, the expert weights, y and out have element type
 *     dims->dtype (MOE_F32 = float, MOE_BF16 = bfloat16 bits); the router weight,
 *     router bias, routing weights and gaps are always float; indices int32.
 *   - Arguments are validated on the host before any launch. On failure the
 *     call returns a non-zero moe_status, enqueues nothing, and
 *     moe_last_error() describes the problem (thread-local text).
 *   - Limits: T >= 0 (T = 0 is a no-op); 1 <= E <= 1024; 1 <= k <= min(E, 16);
 *     T*k + T < 2^31; d, I multiples of 8 (>= 8); I_shared = 0 (no shared
 *     expert) or a multiple of 8; renormalize 0 or 1. Float/bf16 tensors must be
 *     16-byte aligned, int32/float vectors 4-byte aligned, the workspace 256-byte
 *     aligned.
 *   - `ws` is a caller-owned device scratch buffer of at least
 *     moe_workspace_size() bytes. Any step may be given the same buffer; its
 *     contents need no initialisation and are not meaningful to the caller.
 *     Calls that share a workspace must not overlap in time (use one stream).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* bad pointer, size, alignment or dtype */
  MOE_ERR_UNSUPPORTED = 2, /* valid in principle but beyond this library's limits */
  MOE_ERR_WORKSPACE = 3,   /* ws missing or smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4          /* a HIP launch failed; moe_last_error() has the HIP error text */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Shapes of one call. Names follow the model configuration: d = hidden_size,
 * E = num_experts, k = num_experts_per_tok, I = moe_intermediate_size,
 * I_shared = shared_expert_intermediate_size. */
typedef struct {
  int64_t T;           /* tokens in the batch */
  int32_t d;           /* hidden size */
  int32_t E;           /* routed experts */
  int32_t k;           /* experts kept per token */
  int32_t I;           /* routed expert intermediate size */
  int32_t I_shared;    /* shared expert intermediate size, 0 = none */
  int32_t dtype;       /* moe_dtype of x, expert weights, y and out */
  int32_t renormalize; /* 1: the k routing weights are renormalised to sum to 1 */
} moe_dims;

/* Bytes of device workspace every entry point below needs for these dims. */
moe_status moe_workspace_size(const moe_dims* dims, size_t* bytes);

/* Router and softmax top-k (Qwen3.6 neural-network explorer page, router section: a small
 * linear network maps the token's embedding to one score per expert, a softmax turns the scores
 * into one probability per expert, and the K most probable experts are kept; the configuration
 * listing on the Qwen3.8-Max architecture page gives num_experts and num_experts_per_tok).
 *   x          [T, d]   dtype
 *   w_router   [d, E]   float; logits l = x w_router (+ router_bias) in fp32
 *   router_bias[E]      float or NULL
 * Outputs:
 *   topk_idx   [T, k]   int32, the k experts with the largest logits, by
 *                       descending logit, ties to the lower index
 *   topk_w     [T, k]   float, softmax probabilities over all E experts of the
 *                       kept ones; divided by their sum when renormalize = 1
 *   topk_gap   [T]      float or NULL: l_(k) - l_(k+1) (+inf when k = E), the
 *                       margin that decides the selection
 *   ws, ws_bytes        the caller's workspace (moe_workspace_size): the logits are summed over
 *                       K splits, whose fp32 partials [splits][T][E] live there, as do the three
 *                       bf16 parts of w_router the MFMA path multiplies by (an exact split of each
 *                       fp32 weight). The function allocates nothing, so the scratch comes in here.
 * Errors: MOE_ERR_INVALID_ARG for bad dims or pointers, MOE_ERR_WORKSPACE for a missing or short
 * ws, MOE_ERR_HIP if a launch fails; nothing is enqueued on any error. */
moe_status moe_router_topk(const moe_dims* dims, const void* x, const float* w_router, const float* router_bias,
                           int32_t* topk_idx, float* topk_w, float* topk_gap, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* moe_router_topk plus router statistics for load balancing (the configuration listing on
 * the Qwen3.8-Max architecture page sets router_aux_loss_coef; the loss formula is not on the
 * pages, so the statistics such a loss is built from are returned):
 *   expert_counts [E] int32  tokens that select expert e
 *   prob_mean     [E] float  mean over the T tokens of e's probability under the softmax over
 *                            all E logits (0 when T = 0)
 * Sums run in fp64 in a fixed order: the results do not depend on scheduling. */
moe_status moe_router_topk_stats(const moe_dims* dims, const void* x, const float* w_router, const float* router_bias,
                                 int32_t* topk_idx, float* topk_w, float* topk_gap, int32_t* expert_counts,
                                 float* prob_mean, void* ws, size_t ws_bytes, hipStream_t stream);

/* Dispatch: group the T*k (token, expert) pairs by expert (explorer page, router section: the
 * token is sent to each of the experts it keeps, so every expert receives the tokens that chose
 * it and can process them together).
 *   topk_idx        [T, k]  int32 (from moe_router_topk); a token's indices in
 *                           [0, E) must be distinct, as top-k selection makes them
 * Outputs:
 *   expert_offsets  [E + 1] int32, expert e owns sorted slots
 *                           [expert_offsets[e], expert_offsets[e+1]); offsets[E] = T*k
 *   sorted_token    [T*k]   int32, token of each sorted slot; within an expert,
 *                           tokens ascend (stable)
 *   slot_of         [T*k]   int32, slot_of[t*k + j] = sorted slot of (t, topk_idx[t, j])
 * Pairs whose index lies outside [0, E) are skipped: their slot_of is -1 and
 * offsets[E] counts only the others (moe_combine then leaves them out).
 * ws: the caller's workspace (per-chunk expert counts). Errors as moe_router_topk. */
moe_status moe_permute(const moe_dims* dims, const int32_t* topk_idx, int32_t* expert_offsets,
                       int32_t* sorted_token, int32_t* slot_of, void* ws, size_t ws_bytes, hipStream_t stream);

/* Routed and shared SwiGLU experts, each row once, unweighted. Each expert is
 * y = (silu(x Wg) * (x Wu)) Wd with no biases (Qwen3.8-Max architecture page, config.json listing:
 * hidden_act "silu", moe_intermediate_size I, shared_expert_intermediate_size I_shared; the overview
 * page's parameter table counts 3 d I parameters per expert); the shared expert runs on every token
 * (explorer page, router section: one expert that is always active).
 *   x               [T, d]      dtype
 *   expert_offsets, sorted_token: from moe_permute
 *   wg, wu          [E, d, I]   dtype; wd [E, I, d] dtype
 *   wg_s, wu_s      [d, I_shared], wd_s [I_shared, d] (ignored when I_shared = 0)
 * Output:
 *   y  [T*k + T, d] dtype (T*k rows when I_shared = 0): row s < T*k is expert
 *      e's output for token sorted_token[s], where s lies in e's slot range;
 *      row T*k + t is the shared expert's output for token t. */
moe_status moe_grouped_ffn(const moe_dims* dims, const void* x, const int32_t* expert_offsets,
                           const int32_t* sorted_token, const void* wg, const void* wu, const void* wd,
                           const void* wg_s, const void* wu_s, const void* wd_s, void* y, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* Weighted combine plus shared expert (explorer page, router section: the kept experts' outputs
 * are summed with their routing weights; the always-active shared expert's output is added, with
 * no weight since the pages name no gate for it):
 *   out[t] = sum_j topk_w[t, j] * y[slot_of[t*k + j]]  +  y[T*k + t] (if I_shared > 0)
 * summed in fp32 in the order j = 0..k-1 then the shared row; out [T, d] dtype.
 * Pairs with slot_of = -1 contribute nothing. */
moe_status moe_combine(const moe_dims* dims, const void* y, const int32_t* slot_of, const float* topk_w, void* out,
                       hipStream_t stream);

/* The whole block in one call: router/top-k, dispatch, experts, combine -- the MoE block of the
 * explorer page's router section (scores, softmax, the K most probable experts weighted, plus the
 * shared expert) with the expert shapes of the Qwen3.8-Max config.json listing.
 * x [T, d] in, out [T, d] out (out may not alias x); the other arguments as in the step entry
 * points above. topk_idx, topk_w, topk_gap may be NULL (then kept in the workspace). Errors as
 * moe_router_topk. */
moe_status moe_forward(const moe_dims* dims, const void* x, const float* w_router, const float* router_bias,
                       const void* wg, const void* wu, const void* wd, const void* wg_s, const void* wu_s,
                       const void* wd_s, void* out, int32_t* topk_idx, float* topk_w, float* topk_gap, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* FP8 expert weights (the Fondations page of the Qwen3.8-Max report names FP8 among the formats
 * and gives no scheme; this is the one used): weight-only OCP e4m3 (bias 7, 3 mantissa bits,
 * largest finite 448), one power-of-two fp32 scale per output column, codes by round to nearest
 * with ties to even:
 *   W[k, n] = e4m3(Q[n, k]) * s[n]
 *
 * moe_quantize_fp8: w [batch, K, N] (dtype, N-contiguous as the bf16 expert weights are stored)
 *   -> q: batch x K*N uint8 codes in code tiles, scale [batch, N] float; s[n] is the smallest
 *   power of two with max_k |w[k, n]| / s[n] <= 448 (1 for an all-zero column). A column that
 *   holds a non-finite weight gets a NaN scale (its non-finite weights get the NaN code).
 *   Code tiles: 128 columns x 32 K values, 4096 bytes, ordered by (column tile, K tile), i.e.
 *   tile (n / 128) * (K / 32) + k / 32 of each matrix. In a tile, with r = n % 128,
 *   j = k % 32, h = j / 16: Q[n, k] is byte 32 r + 16 (h ^ ((r / 8) % 2)) + j % 16.
 *   K % 32 == 0 and N % 128 == 0, else MOE_ERR_UNSUPPORTED; q 16-byte aligned; batch <= 65535. */
moe_status moe_quantize_fp8(const void* w, int32_t dtype, int64_t batch, int32_t K, int32_t N, uint8_t* q,
                            float* scale, hipStream_t stream);

/* moe_forward with FP8 expert weights (moe_quantize_fp8 layout): wg, wu codes of [E] matrices
 * with K = d, N = I and scales sg, su [E, I]; wd codes of [E] matrices with K = I, N = d and sd
 * [E, d]; the shared expert likewise (wg_s, wu_s: K = d, N = I_shared; wd_s: K = I_shared,
 * N = d) with sg_s, su_s [I_shared], sd_s [d]. x, out bf16 (dims.dtype = MOE_BF16);
 * d % 256 == 0 and I, I_shared % 128 == 0, else MOE_ERR_UNSUPPORTED. The products run on the bf16
 * MFMA with the codes widened exactly; the column scales are applied to the fp32 sums. */
moe_status moe_forward_fp8(const moe_dims* dims, const void* x, const float* w_router, const float* router_bias,
                           const uint8_t* wg, const uint8_t* wu, const uint8_t* wd, const float* sg, const float* su,
                           const float* sd, const uint8_t* wg_s, const uint8_t* wu_s, const uint8_t* wd_s,
                           const float* sg_s, const float* su_s, const float* sd_s, void* out, int32_t* topk_idx,
                           float* topk_w, float* topk_gap, void* ws, size_t ws_bytes, hipStream_t stream);

/* Steps either side of the block: zero-centred RMSNorm in front of it (the Qwen3-Next
 * article: Zero-Centered RMSNorm, parameters starting at zero, so the scale is 1 + gamma;
 * the Qwen3.8-Max architecture page's configuration listing: rms_norm_eps = 1e-6) and the
 * residual add after it (the overview page's parameter table counts two norms per layer
 * plus a final one, a norm in front of each MoE block).
 *
 * moe_rmsnorm:  h[t] = x[t] / sqrt(mean_i x[t,i]^2 + eps) * (1 + gamma)
 *   x, h [T, d] dtype; gamma [d] dtype; eps finite and >= 0. Computed in fp64 and rounded
 *   once to dtype (to nearest, ties to even). h may not alias x. */
moe_status moe_rmsnorm(const moe_dims* dims, const void* x, const void* gamma, double eps, void* h,
                       hipStream_t stream);

/* moe_combine with the residual row added last:
 *   out[t] = sum_j topk_w[t, j] y[slot_of[t*k + j]] + y[T*k + t] + residual[t]
 * residual [T, d] dtype (the block's input). */
moe_status moe_combine_residual(const moe_dims* dims, const void* y, const int32_t* slot_of, const float* topk_w,
                                const void* residual, void* out, hipStream_t stream);

/* The block between its neighbours: out = x + MoE(moe_rmsnorm(x)); the router and the experts
 * see the normalised rows (kept in the workspace). Arguments as moe_forward, plus gamma [d] and
 * eps as for moe_rmsnorm. out may not alias x. */
moe_status moe_forward_block(const moe_dims* dims, const void* x, const void* gamma, double eps,
                             const float* w_router, const float* router_bias, const void* wg, const void* wu,
                             const void* wd, const void* wg_s, const void* wu_s, const void* wd_s, void* out,
                             int32_t* topk_idx, float* topk_w, float* topk_gap, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same block, with the scratch space
 * taken from a buffer the library holds in device memory instead of a caller's workspace.
 *   - Arguments and results as moe_forward, without ws / ws_bytes.
 *   - The buffer is MOE_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, a static device array of the
 *     library's code object: every GPU the library runs on holds it until the process ends. Its
 *     address is looked up once per device, on the first call made with that device current.
 *   - Dims whose moe_workspace_size exceeds the buffer are rejected (MOE_ERR_UNSUPPORTED) before
 *     anything is enqueued: e.g. the d = 8192, E = 512, k = 10, I = I_shared = 2048 layer up to
 *     T = 64 tokens, the d = 2048, E = 256, k = 8, I = I_shared = 512 layer up to T = 1024.
 *   - No call allocates or frees memory (no hipMalloc, hipFree or allocating library routine).
 *   - All calls on one GPU share its buffer, and each call leaves its contents behind: calls that
 *     overlap in time on one GPU (several streams, several threads) race and must be serialised
 *     by the caller. The stream must belong to the current device. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_noalloc(const moe_dims* dims, const void* x, const float* w_router, const float* router_bias,
                               const void* wg, const void* wu, const void* wd, const void* wg_s, const void* wu_s,
                               const void* wd_s, void* out, int32_t* topk_idx, float* topk_w, float* topk_gap,
                               hipStream_t stream);

/* Instrumentation for timing one kernel of the path while the whole path runs.
 * The next moe_forward call made by the calling thread records `start` on its
 * stream immediately before launching the selected kernel and `stop` right
 * after it (hipEventRecord), then the request is cleared. Both events are
 * caller-owned (hipEventCreate); pass kernel = MOE_KERNEL_NONE to cancel.
 * Returns MOE_ERR_INVALID_ARG for an unknown kernel id or a NULL event. */
typedef enum {
  MOE_KERNEL_NONE = 0,
  MOE_KERNEL_ROUTER = 1,       /* router logits GEMM (+ top-k kernel, except as below) */
  MOE_KERNEL_PERMUTE = 2,      /* the dispatch kernels; for 1 <= T <= 4 with E > 64 and the
                                  vector router, one kernel doing top-k and dispatch */
  MOE_KERNEL_FFN_GATE_UP = 3,  /* grouped gate/up GEMM with fused silu*mul */
  MOE_KERNEL_FFN_DOWN = 4,     /* grouped down GEMM */
  MOE_KERNEL_COMBINE = 5       /* weighted combine + shared add */
} moe_kernel_id;

moe_status moe_profile_next_forward(int32_t kernel, hipEvent_t start, hipEvent_t stop);

/* Name of the main kernel that moe_forward (fp8 = 0) or moe_forward_fp8 (fp8 = 1) launches with
 * these dims for one step of the path (kernel: a moe_kernel_id other than MOE_KERNEL_NONE), as
 * it appears in a kernel trace, for labelling measurements. Host only: launches nothing, sets no
 * error text. Returns a static string, or NULL for invalid dims, an unknown id, or dims the FP8
 * path does not take. */
const char* moe_kernel_name(const moe_dims* dims, int32_t kernel, int32_t fp8);

/* Static name of a status code. */
const char* moe_status_string(moe_status status);

/* Detail text of the calling thread's last non-OK return ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
