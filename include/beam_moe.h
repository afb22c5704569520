/*
 * beam_moe.h - C ABI of the MI355X (gfx950) sparse-MoE block of Beam.
 *
 * The block (Beam launch post "Introducing Beam", section "Mixture of
 * Experts"; transformers model doc "Beam", section "Overview"):
 *   1. score all experts with a sigmoid of the router logits, computed in
 *      fp32 (launch post, "Residual Stream": the router is an fp32 island;
 *      model doc, "Overview": router weights and expert bias are kept fp32);
 *   2. add the learned per-expert bias to form the selection key (the bias
 *      balances load in place of an auxiliary loss, model doc "Overview");
 *   3. split the experts into n_group contiguous groups, score each group by
 *      the sum of its two largest keys and keep the topk_group best groups
 *      (Beam: 8 groups of 32, keep 4);
 *   4. choose the top_k experts with the largest keys inside the kept groups
 *      (Beam: 8), ordered by key descending, equal keys by lower index;
 *   5. normalise the chosen experts' unbiased sigmoid scores to sum to 1;
 *   6. run each chosen SwiGLU expert, y = W_down (silu(W_gate x) * (W_up x)),
 *      with the SwiGLU product in fp32 (launch post, "Residual Stream"), and
 *      sum the expert outputs weighted by routed_scaling_factor * weight
 *      (Beam: 2.5). There is no shared expert.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are device memory owned by the caller, contiguous,
 *     row-major, 16-byte aligned. The library allocates nothing, frees
 *     nothing, and keeps no state between calls other than cached device
 *     properties.
 *   - Calls are asynchronous: they validate their arguments on the host,
 *     enqueue kernels on `stream` (a hipStream_t; NULL = the default stream)
 *     and return. Outputs are valid once the stream has reached that point.
 *   - Every argument check runs before any HIP call; a failed check returns
 *     its status and enqueues nothing. A failed launch returns
 *     BEAM_ERR_HIP. Faults inside a kernel surface at the caller's next
 *     synchronisation, as for any HIP work. T == 0 returns BEAM_OK and
 *     enqueues nothing.
 *   - Results are deterministic: the same inputs on the same stream give
 *     bit-identical outputs (no floating-point atomics).
 *   - Calls that share one workspace must not overlap in time.
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum beam_status {
  BEAM_OK = 0,
  BEAM_ERR_NULL = 1,      /* a required pointer is NULL */
  BEAM_ERR_CONFIG = 2,    /* routing parameters outside the supported set */
  BEAM_ERR_SHAPE = 3,     /* T, hidden or intermediate outside the supported set */
  BEAM_ERR_DTYPE = 4,     /* unsupported dtype combination, or fp8 scales missing */
  BEAM_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned */
  BEAM_ERR_WORKSPACE = 6, /* workspace NULL or smaller than beam_moe_workspace_bytes() */
  BEAM_ERR_HIP = 7        /* the HIP runtime reported an error at launch */
} beam_status;

typedef enum beam_dtype {
  BEAM_F32 = 0,      /* IEEE binary32 */
  BEAM_BF16 = 1,     /* bfloat16 (upper 16 bits of binary32) */
  BEAM_FP8_E4M3 = 2  /* OCP FP8 E4M3 ("e4m3fn"): bias 7, no infinity, max 448 */
} beam_dtype;

/*
 * Layer shape and routing parameters. The names follow the model doc's
 * config fields (n_group, topk_group, routed_scaling_factor; model doc
 * "Beam", "Overview"). Beam's values: hidden 5120, intermediate 2560,
 * n_experts 256, n_group 8, topk_group 4, top_k 8, routed_scaling_factor 2.5.
 *
 * Supported set (anything else returns BEAM_ERR_CONFIG / BEAM_ERR_SHAPE /
 * BEAM_ERR_DTYPE):
 *   n_experts == 256;
 *   n_group a power of two in [1, 64] (groups of 256 / n_group >= 4 experts);
 *   1 <= topk_group <= n_group;
 *   1 <= top_k <= min(32, topk_group * 256 / n_group);
 *   hidden and intermediate positive multiples of 128, each <= 65536;
 *   routed_scaling_factor finite;
 *   x_dtype in {BEAM_F32, BEAM_BF16} (the output has the same dtype);
 *   w_dtype in {BEAM_BF16, BEAM_FP8_E4M3}.
 */
typedef struct beam_moe_config {
  int32_t hidden;
  int32_t intermediate;
  int32_t n_experts;
  int32_t n_group;
  int32_t topk_group;
  int32_t top_k;
  float routed_scaling_factor;
  int32_t x_dtype; /* beam_dtype */
  int32_t w_dtype; /* beam_dtype */
} beam_moe_config;

/*
 * Bytes of device workspace that beam_moe_route and beam_moe_forward need for
 * T tokens under `cfg` (the same figure serves both). Returns 0 if `cfg` is
 * NULL or invalid or T < 0. Pure host arithmetic; makes no HIP call.
 */
size_t beam_moe_workspace_bytes(const beam_moe_config* cfg, int32_t T);

/*
 * Routing only: steps 1-5 above.
 *   x             [T, hidden], x_dtype (bf16 or fp32). Upcast exactly to fp32.
 *   router_w      [n_experts, hidden] fp32; row e is expert e's router vector.
 *   expert_bias   [n_experts] fp32; enters the selection key only.
 *   topk_idx      out [T, top_k] int32: chosen experts, key descending.
 *   topk_w        out [T, top_k] fp32: normalised weights (sum 1, before the
 *                 routed_scaling_factor).
 *   router_logits out [T, n_experts] fp32 pre-sigmoid logits, or NULL
 *                 (returned on request, model doc "Beam", "Notes").
 *   expert_counts out [n_experts] int32 tokens per expert, or NULL.
 *   workspace     device scratch of at least beam_moe_workspace_bytes(cfg, T).
 * Errors: BEAM_ERR_NULL if cfg, x, router_w, expert_bias, topk_idx or topk_w
 * is NULL (or workspace when T > 0); see the conventions above.
 */
beam_status beam_moe_route(const beam_moe_config* cfg, int32_t T, const void* x,
                           const float* router_w, const float* expert_bias,
                           int32_t* topk_idx, float* topk_w, float* router_logits,
                           int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * The whole block: steps 1-6 above.
 *   x, router_w, expert_bias  as for beam_moe_route.
 *   w_gate, w_up  [n_experts, intermediate, hidden] (each expert's matrix is
 *                 [out, in] row-major), w_dtype.
 *   w_down        [n_experts, hidden, intermediate], w_dtype.
 *   w_gate_scale, w_up_scale  [n_experts, intermediate] fp32 and
 *   w_down_scale  [n_experts, hidden] fp32: per-output-row dequantisation
 *                 scales (the weight is code * scale). Required when w_dtype is
 *                 BEAM_FP8_E4M3, ignored (may be NULL) otherwise.
 *                 With fp8 weights the expert inputs are quantised to E4M3 per
 *                 row as well: x per token, the SwiGLU output per (token,
 *                 expert) row, each with scale amax / 448.
 *   out           out [T, hidden], x_dtype.
 *   topk_idx_out  out [T, top_k] int32 or NULL; topk_w_out out [T, top_k] fp32
 *                 or NULL; expert_counts_out out [n_experts] int32 or NULL;
 *   router_logits_out out [T, n_experts] fp32 or NULL.
 *   workspace     device scratch of at least beam_moe_workspace_bytes(cfg, T).
 * Errors: BEAM_ERR_NULL if cfg, x, router_w, expert_bias, w_gate, w_up, w_down
 * or out is NULL (or workspace when T > 0); BEAM_ERR_DTYPE if fp8 scales are
 * missing; see the conventions above.
 */
beam_status beam_moe_forward(const beam_moe_config* cfg, int32_t T, const void* x,
                             const float* router_w, const float* expert_bias,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const float* w_gate_scale, const float* w_up_scale,
                             const float* w_down_scale, void* out, int32_t* topk_idx_out,
                             float* topk_w_out, int32_t* expert_counts_out,
                             float* router_logits_out, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Static, NUL-terminated description of a status code; never NULL. */
const char* beam_moe_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* BEAM_MOE_H */
