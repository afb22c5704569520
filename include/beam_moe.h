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
 *     row-major, 16-byte aligned. The library allocates no device memory and
 *     keeps no state between calls (the optional stage timing below keeps
 *     its HIP events until beam_moe_profile_end).
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
  BEAM_FP8_E4M3 = 2, /* OCP FP8 E4M3 ("e4m3fn"): bias 7, no infinity, max 448 */
  BEAM_MXFP4 = 3,    /* OCP MXFP4: E2M1 codes (magnitudes 0, 0.5, 1, 1.5, 2, 3,
                        4, 6; sign in bit 3), two per byte with element 2j in
                        the low nibble, plus one E8M0 scale byte (value
                        2^(code - 127)) per 32 consecutive elements of a row */
  BEAM_E8M0 = 4      /* the MXFP4 scale bytes (beam_moe_pack_weights only) */
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
 *   hidden and intermediate positive multiples of 128, each <= 65536
 *   (multiples of 512 with BEAM_MXFP4 weights);
 *   routed_scaling_factor finite;
 *   x_dtype in {BEAM_F32, BEAM_BF16} (the output has the same dtype);
 *   w_dtype in {BEAM_BF16, BEAM_FP8_E4M3, BEAM_MXFP4};
 *   w_layout in {BEAM_LAYOUT_ROW_MAJOR, BEAM_LAYOUT_PACKED} (BEAM_MXFP4:
 *   BEAM_LAYOUT_PACKED only).
 */
typedef struct beam_moe_config {
  int32_t hidden;
  int32_t intermediate;
  int32_t n_experts;
  int32_t n_group;
  int32_t topk_group;
  int32_t top_k;
  float routed_scaling_factor;
  int32_t x_dtype;  /* beam_dtype */
  int32_t w_dtype;  /* beam_dtype */
  int32_t w_layout; /* beam_layout of w_gate, w_up, w_down */
} beam_moe_config;

/*
 * Storage layout of the expert weight matrices. Each expert's matrix has R
 * rows (output channels) and C columns (the reduction): w_gate and w_up
 * R = intermediate, C = hidden; w_down R = hidden, C = intermediate.
 *   BEAM_LAYOUT_ROW_MAJOR: element (r, c) at r * C + c ([out, in] row-major).
 *   BEAM_LAYOUT_PACKED: the MI355X matrix-core fragment layout, made from the
 *     row-major one by beam_moe_pack_weights. With S = 32 (bf16) or 128
 *     (fp8) and L = S / 4, element (r, c) is at
 *       ((r / 16) * (C / S) + c / S) * 16 * S
 *         + ((r % 16) + 16 * ((c % S) / L)) * L + c % L,
 *     so that each 16-row by S-column operand of one matrix-core step is one
 *     contiguous block (1 KB bf16, 2 KB fp8) in the order the 64 lanes of a
 *     wavefront consume it. Same size as row-major; the per-row fp8 scales
 *     keep their [n_experts, R] layout.
 *     MXFP4 codes use S = 128 and L = 32 with two codes per byte (each block
 *     is 1 KB: lane l's 16 bytes hold the 32 codes of row r % 16, columns
 *     32 (l / 16) .. + 31 of the step). Their scale bytes (row-major
 *     [n_experts, R, C / 32]) are packed as well: the scale of row r, column
 *     block b = c / 32 goes to byte
 *       ((r / 16) * (C / 512) + b / 16) * 256 + ((r % 16) + 16 * (b % 4)) * 4
 *         + (b % 16) / 4,
 *     so one 4-byte load gives a lane the scales of four consecutive steps.
 */
typedef enum beam_layout {
  BEAM_LAYOUT_ROW_MAJOR = 0,
  BEAM_LAYOUT_PACKED = 1
} beam_layout;

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
 * is NULL; BEAM_ERR_WORKSPACE if workspace is NULL or smaller than
 * beam_moe_workspace_bytes() (T > 0); see the conventions above.
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
 *   w_gate_scale, w_up_scale, w_down_scale  dequantisation scales, required
 *                 with quantised weights, ignored (may be NULL) with bf16:
 *                 BEAM_FP8_E4M3: fp32, [n_experts, intermediate] (gate, up)
 *                 and [n_experts, hidden] (down), one per output row (the
 *                 weight is code * scale);
 *                 BEAM_MXFP4: the packed E8M0 scale bytes (see beam_layout),
 *                 one per 32 weights of a row.
 *                 With fp8 or MXFP4 weights the expert inputs are quantised
 *                 to E4M3 per row: x per token, the SwiGLU output per (token,
 *                 expert) row, each with scale amax / 448.
 *   out           out [T, hidden], x_dtype.
 *   topk_idx_out  out [T, top_k] int32 or NULL; topk_w_out out [T, top_k] fp32
 *                 or NULL; expert_counts_out out [n_experts] int32 or NULL;
 *   router_logits_out out [T, n_experts] fp32 or NULL.
 *   workspace     device scratch of at least beam_moe_workspace_bytes(cfg, T).
 * Errors: BEAM_ERR_NULL if cfg, x, router_w, expert_bias, w_gate, w_up, w_down
 * or out is NULL; BEAM_ERR_WORKSPACE if workspace is NULL or smaller than
 * beam_moe_workspace_bytes() (T > 0); BEAM_ERR_DTYPE if fp8 scales are
 * missing; see the conventions above.
 */
beam_status beam_moe_forward(const beam_moe_config* cfg, int32_t T, const void* x,
                             const float* router_w, const float* expert_bias,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const void* w_gate_scale, const void* w_up_scale,
                             const void* w_down_scale, void* out, int32_t* topk_idx_out,
                             float* topk_w_out, int32_t* expert_counts_out,
                             float* router_logits_out, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * beam_moe_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments, results and kernels as
 * beam_moe_forward (minus workspace and workspace_bytes). Its scratch is a
 * static array of BEAM_MOE_NOALLOC_MAX_BYTES in device memory, one per GPU
 * the library runs on, held until the process ends; the call allocates and
 * frees nothing. 64 MiB holds the forward's workspace for up to 256 tokens at
 * Beam's shape (hidden 5120, intermediate 2560) with bf16, fp8 or MXFP4
 * experts; larger problems return BEAM_ERR_WORKSPACE before any HIP call
 * (beam_moe_workspace_bytes(cfg, T) tells the need). Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and give wrong results.
 * No part of the scratch needs to start at zero. The first call on a device
 * looks up the array's device address (hipGetSymbolAddress, the stream's
 * device current) and keeps it; a failure there returns BEAM_ERR_HIP.
 */
#define BEAM_MOE_NOALLOC_MAX_BYTES ((size_t)64 << 20)

beam_status beam_moe_forward_noalloc(const beam_moe_config* cfg, int32_t T, const void* x,
                                     const float* router_w, const float* expert_bias,
                                     const void* w_gate, const void* w_up, const void* w_down,
                                     const void* w_gate_scale, const void* w_up_scale,
                                     const void* w_down_scale, void* out, int32_t* topk_idx_out,
                                     float* topk_w_out, int32_t* expert_counts_out,
                                     float* router_logits_out, void* stream);

/*
 * One expert shard's share of the block, for expert parallelism (launch post
 * "Introducing Beam", section "Multi-GPU and multi-node": each expert lives
 * on one device; transformers model doc "Beam": ep_size). The routing is
 * computed over all experts exactly as in beam_moe_forward; the expert GEMMs
 * run only for experts [expert_begin, expert_end), whose weights are the only
 * ones given: w_gate, w_up [n, I, H], w_down [n, H, I] and their scales (same
 * dtypes and layouts as beam_moe_forward) for n = expert_end - expert_begin,
 * expert expert_begin first.
 *   out_partial[t] = rsf * sum over the slots j of token t whose expert lies
 *                    in the range of w[t, j] * FFN_e(x[t])   ([T, H], x dtype;
 *                    zeros for a token with no expert in the range).
 * The shards' partial outputs of a partition of the 256 experts sum to the
 * block output (up to the rounding of each partial sum to the output dtype).
 * Routing outputs (nullable) are those of all experts. Workspace as for
 * beam_moe_forward. Errors as for beam_moe_forward; BEAM_ERR_CONFIG unless
 * 0 <= expert_begin < expert_end <= 256.
 */
beam_status beam_moe_forward_shard(const beam_moe_config* cfg, int32_t T, const void* x,
                                  const float* router_w, const float* expert_bias,
                                  int32_t expert_begin, int32_t expert_end, const void* w_gate,
                                  const void* w_up, const void* w_down, const void* w_gate_scale,
                                  const void* w_up_scale, const void* w_down_scale,
                                  void* out_partial, int32_t* topk_idx_out, float* topk_w_out,
                                  int32_t* expert_counts_out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * The block followed by its place in Beam's residual stream, fused into the
 * final combine (launch post "Introducing Beam", section "Residual Stream";
 * model doc "Beam", "Overview": depth-scaled residual and sandwich norm):
 *   stream_out = sqrt((k-1)/k) * stream_in + RMSNorm(moe_out) / sqrt(k),
 *   RMSNorm(v) = v / sqrt(mean over hidden of v^2 + norm_eps) * norm_weight,
 * computed in fp32 per token from the fp32 sum of the expert outputs (the
 * MoE output itself is never stored). k is this sublayer's step: the input
 * embedding is step 1, then every attention and MLP sublayer adds one.
 *   stream_in   [T, hidden], x_dtype; may be the same memory as stream_out.
 *   norm_weight [hidden] fp32.
 *   norm_eps    finite, >= 0.
 *   step        k >= 2.
 * All other arguments as for beam_moe_forward (stream_out replaces out).
 * Errors: as beam_moe_forward; BEAM_ERR_NULL if residual, its stream_in or
 * norm_weight is NULL; BEAM_ERR_CONFIG if step < 2 or norm_eps is negative or
 * not finite; BEAM_ERR_SHAPE if hidden > 16384 (the row is staged in LDS).
 */
typedef struct beam_moe_residual {
  const void* stream_in;
  const float* norm_weight;
  float norm_eps;
  int32_t step;
} beam_moe_residual;

beam_status beam_moe_forward_residual(const beam_moe_config* cfg, int32_t T, const void* x,
                                      const float* router_w, const float* expert_bias,
                                      const void* w_gate, const void* w_up, const void* w_down,
                                      const void* w_gate_scale, const void* w_up_scale,
                                      const void* w_down_scale, const beam_moe_residual* residual,
                                      void* stream_out, int32_t* topk_idx_out, float* topk_w_out,
                                      int32_t* expert_counts_out, float* router_logits_out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Convert n_experts row-major [rows, cols] weight matrices at `src` into
 * BEAM_LAYOUT_PACKED at `dst` (same byte size), on `stream`. w_dtype:
 * BEAM_BF16 or BEAM_FP8_E4M3 (the matrices), BEAM_MXFP4 (the code matrices,
 * cols / 2 bytes per row) or BEAM_E8M0 (their scale bytes, cols / 32 per
 * row); cols is always the number of weights per row. A one-time transform
 * at weight-load time: the packed layout lets every matrix-core operand load
 * of the expert GEMMs read one contiguous block. src and dst are
 * caller-owned device memory, 16-byte aligned, and must not overlap.
 * Errors: BEAM_ERR_NULL (src or dst NULL), BEAM_ERR_SHAPE (n_experts < 1,
 * rows not a positive multiple of 16, cols not a positive multiple of 128
 * (512 for BEAM_MXFP4 and BEAM_E8M0), or more than 2^40 bytes in all),
 * BEAM_ERR_DTYPE, BEAM_ERR_ALIGN, BEAM_ERR_HIP (launch failed).
 */
beam_status beam_moe_pack_weights(const void* src, void* dst, int32_t n_experts, int32_t rows,
                                  int32_t cols, int32_t w_dtype, void* stream);

/*
 * The backward pass of the block, for training and adapter fine-tuning
 * (launch post "Introducing Beam", section "Post-training Beam": GRPO with
 * full recomputation and bf16 gradients; rank-16 adapters on the expert
 * layers). It recomputes the routing and the gate/up pass from x, then
 * applies the chain rule to L = sum(dout * out):
 *   slot j of token t, expert e, sorted row q, g = W_gate[e] x, u = W_up[e] x,
 *   h = silu(g) u, y = W_down[e] h, w the normalised weight, s the chosen
 *   sigmoid scores with sum S:
 *   dh = rsf w (W_down[e]^T dout[t]);  du = dh silu(g);  dg = dh u silu'(g)
 *   dx[t] = sum_j (W_gate[e]^T dg + W_up[e]^T du) + sum_j dz_j W_r[e_j]
 *   dw_j = rsf <dout[t], y>;  ds_j = (dw_j - sum_i w_i dw_i) / S;
 *   dz_j = ds_j s_j (1 - s_j);  d W_r[e] = sum over e's slots of dz x[t]
 *   d W_down[e] = sum (rsf w dout[t]) h^T;  d W_gate[e] = sum dg x[t]^T;
 *   d W_up[e] = sum du x[t]^T
 * The expert choice is piecewise constant: the selection bias gets no
 * gradient (it moves by beam_moe_update_bias instead).
 *
 * Scope: x_dtype BEAM_BF16; w_dtype BEAM_BF16 in BEAM_LAYOUT_PACKED; hidden
 * and intermediate multiples of 256 (else BEAM_ERR_DTYPE / BEAM_ERR_CONFIG /
 * BEAM_ERR_SHAPE).
 *   x [T, H] bf16, router_w [E, H] fp32, expert_bias [E] fp32: as for forward.
 *   w_gate, w_up: packed, as for forward (the gate/up recomputation).
 *   w_gate_t, w_up_t: beam_moe_pack_weights_transposed of w_gate / w_up
 *     (packed [E, H, I]); w_down_t: of w_down (packed [E, I, H]).
 *   dout [T, H] bf16: gradient of the block output.
 * Outputs (beam_moe_grads; all device memory, overwritten):
 *   dx [T, H] bf16 (required).
 *   d_router_w [E, H] fp32, or NULL to skip.
 *   d_w_gate, d_w_up [E, I, H] bf16 and d_w_down [E, H, I] bf16 (row-major,
 *     the forward's storage order): all three or none (NULL). Experts no
 *     token chose get zeros.
 * Workspace: beam_moe_backward_workspace_bytes(cfg, T, with_weight_grads).
 * Deterministic (no floating-point atomics). Errors as for the forward;
 * BEAM_ERR_NULL if grads or grads->dx is NULL or only some of the three
 * weight-gradient pointers are set.
 */
typedef struct beam_moe_grads {
  void* dx;
  float* d_router_w;
  void* d_w_gate;
  void* d_w_up;
  void* d_w_down;
} beam_moe_grads;

size_t beam_moe_backward_workspace_bytes(const beam_moe_config* cfg, int32_t T,
                                         int32_t with_weight_grads);

beam_status beam_moe_backward(const beam_moe_config* cfg, int32_t T, const void* x,
                              const float* router_w, const float* expert_bias, const void* w_gate,
                              const void* w_up, const void* w_gate_t, const void* w_up_t,
                              const void* w_down_t, const void* dout, const beam_moe_grads* grads,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The packed layout of each matrix's transpose: n_experts row-major
 * [rows, cols] bf16 matrices at `src` become the packed (BEAM_LAYOUT_PACKED)
 * form of [cols, rows] at `dst` (same size; the reduction runs along the
 * source rows). Used for the backward pass's products with W^T. rows and
 * cols multiples of 64; w_dtype BEAM_BF16 only. Errors: BEAM_ERR_NULL,
 * BEAM_ERR_SHAPE, BEAM_ERR_DTYPE, BEAM_ERR_ALIGN, BEAM_ERR_HIP.
 */
beam_status beam_moe_pack_weights_transposed(const void* src, void* dst, int32_t n_experts,
                                             int32_t rows, int32_t cols, int32_t w_dtype,
                                             void* stream);

/*
 * One load-balancing step of the selection bias (transformers model doc
 * "Beam", "Overview": a learned per-expert bias balances the load in place
 * of an auxiliary loss; the launch post names DeepSeek-V3's routing scheme,
 * whose balancing rule this is): for every expert,
 *   expert_bias[e] += gamma * sign(mean load - expert_counts[e]),
 * the sign taken exactly (integer comparison), the addition in fp32.
 * expert_bias [256] fp32 (in place), expert_counts [256] int32 (e.g. from
 * beam_moe_forward). Errors: BEAM_ERR_NULL, BEAM_ERR_CONFIG (n_experts not
 * 256 or gamma not finite), BEAM_ERR_ALIGN, BEAM_ERR_HIP.
 */
beam_status beam_moe_update_bias(float* expert_bias, const int32_t* expert_counts,
                                 int32_t n_experts, float gamma, void* stream);

/* Static, NUL-terminated description of a status code; never NULL. */
const char* beam_moe_status_string(int32_t status);

/*
 * Stage timing. The kernels of one call, in launch order (forward: all that
 * apply to its dtypes; route: the first two, plus the histogram and scan when
 * counts are requested; backward: the routing and permutation stages, then
 * the BEAM_STAGE_BWD_ ones).
 */
typedef enum beam_stage {
  BEAM_STAGE_ROUTER_LOGITS = 0, /* fp32 router logits */
  BEAM_STAGE_SELECT = 1,        /* sigmoid, bias, group top-2, kept groups, top-k, normalise */
  BEAM_STAGE_PERM_HIST = 2,     /* per-chunk expert histogram */
  BEAM_STAGE_PERM_SCAN = 3,     /* counts, offsets, GEMM tile list (up to 256 tokens:
                                   the whole permutation, one launch) */
  BEAM_STAGE_PERM_SCATTER = 4,  /* stable scatter into expert order */
  BEAM_STAGE_QUANT_X = 5,       /* fp8 weights only: per-token E4M3 quantisation of x */
  BEAM_STAGE_GATEUP = 6,        /* grouped gate/up GEMM + SwiGLU */
  BEAM_STAGE_QUANT_H = 7,       /* fp8 weights only: per-row E4M3 quantisation of h */
  BEAM_STAGE_DOWN = 8,          /* grouped down GEMM, scaled by rsf * weight */
  BEAM_STAGE_COMBINE = 9,       /* weighted combine into the output */
  /* backward pass */
  BEAM_STAGE_BWD_GATEUP = 10,   /* gate/up recomputation: g | u (and h transposed) */
  BEAM_STAGE_BWD_DOWN = 11,     /* W_down^T dout, SwiGLU backward: dg | du */
  BEAM_STAGE_BWD_DX = 12,       /* W_gate^T dg + W_up^T du per row */
  BEAM_STAGE_BWD_TOKEN = 13,    /* routing-weight gradient, dz, dx per token */
  BEAM_STAGE_BWD_ROUTER = 14,   /* router-weight gradient */
  BEAM_STAGE_BWD_TRANSPOSE = 15,/* transposed operand copies for the weight gradients */
  BEAM_STAGE_BWD_WGRAD = 16,    /* weight-gradient GEMMs */
  BEAM_STAGE_COUNT = 17
} beam_stage;

/*
 * beam_moe_profile_begin(mask): from now on, every route/forward/backward call in the
 * process records a pair of HIP timing events around the launch of each
 * stage s with bit (1 << s) set in `mask`, on the call's stream. Clears
 * earlier records. The library creates the events (no device memory).
 * beam_moe_profile_end(total_ms, launches): waits for the recorded events,
 * writes for every stage s < BEAM_STAGE_COUNT the summed elapsed
 * milliseconds total_ms[s] and the number of timed launches launches[s]
 * (either pointer may be NULL), releases the events and stops recording.
 * Both return BEAM_ERR_HIP if a HIP event call fails. Meant for measurement
 * runs; the events add a few microseconds per timed launch.
 */
beam_status beam_moe_profile_begin(uint32_t stage_mask);
beam_status beam_moe_profile_end(float* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* BEAM_MOE_H */
