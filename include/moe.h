/*
 * moe.h -- C ABI of libmoe.so: forward pass of a sparsely gated
 * Mixture-of-Experts FFN layer on AMD MI355X (gfx950).
 *
 * Sources (web pages on the method, cited by page and section):
 *   P1 "混合专家模型MoE入门实战：从零搭建可运行的小型MoE模型"
 *   P2 "MoE架构解析：混合专家模型原理与工程实践"
 *   P3 "MoE混合专家模型原理与实战：稀疏激活如何实现万亿参数高效推理"
 *   P4 "混合专家 MOE 是什么"
 *   P5 "MoE 混合专家模型串讲：从 Switch Transformer 到 DeepSeekMoE"
 *
 * The layer is five calls, run in this order on one stream:
 *   moe_router_topk -> moe_dispatch_permute -> moe_expert_ffn_grouped
 *   (routed experts, then shared experts) -> moe_combine -> moe_aux_loss.
 * Variants: moe_router_topk_noisy in place of moe_router_topk (noisy gating
 * in training mode), and moe_dispatch_permute without the row copy followed
 * by moe_expert_ffn_gathered in place of moe_expert_ffn_grouped for the
 * routed experts (the FFN reads x through the permutation).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE memory owned by the caller.  The library
 *     never allocates or frees device memory; scratch comes from a caller
 *     workspace sized by the matching *_workspace_size() call.
 *   - Every call is asynchronous on `stream` (0 = the null stream) and never
 *     synchronises the host.  Nothing is read back to the host.
 *   - Layouts are row-major and contiguous.  Matrices of experts are stored
 *     [out, in] (the router matrix W_g is [E, d], as P4 公式：三步走 shapes
 *     it: experts x input width).
 *   - Tensor pointers must be 16-byte aligned; bf16 rows need widths that
 *     are multiples of 8 elements and fp8 rows multiples of 16 elements.
 *   - Arguments are validated on the host before anything is launched; on
 *     error nothing is written and a negative moe_status is returned.
 *   - The library keeps no state between calls except the last HIP error
 *     code (per host thread).  Calls are reentrant; two calls that share
 *     output or workspace buffers must not overlap in time.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* bad shape, dtype, NULL or misaligned pointer, k outside [1, E] */
  MOE_ERR_UNSUPPORTED = -2,  /* valid combination that the library does not implement */
  MOE_ERR_HIP = -3,          /* a HIP launch failed; see moe_last_hip_error() */
  MOE_ERR_WORKSPACE = -4     /* workspace NULL or smaller than *_workspace_size() */
} moe_status;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8_E4M3 = 2           /* OCP E4M3FN: bias 7, max 448, no inf, S.1111.111 = NaN */
} moe_dtype;

typedef enum {
  MOE_GATE_PROB = 0,         /* g = p of the selected expert (P5 DeepSeekMoE 数学定义; P5 代码实战 top-1 gate) */
  MOE_GATE_RENORM = 1        /* g = p / sum of selected p  == softmax over the selected logits
                                (P1 §3.3; P2 §2.1 top_k_gating; P3 §3.1) */
} moe_gate_mode;

typedef enum {
  MOE_FFN_LINEAR = 0,        /* y = A x + b                         (P4 公式：三步走, step two) */
  MOE_FFN_RELU = 1,          /* y = W2 relu(W1 x + b1) + b2         (P1 §3.2, P3 §3.1 two-layer expert, with ReLU) */
  MOE_FFN_SWIGLU = 2,        /* y = W2 (silu(W1 x) * (W3 x))        (not on the pages; standard gated form) */
  MOE_FFN_GELU = 3           /* y = W2 gelu(W1 x + b1) + b2         (P1 §3.2 and P3 §3.1 experts: nn.GELU,
                                gelu(u) = u/2 (1 + erf(u/sqrt 2)), the exact form) */
} moe_ffn_kind;

typedef enum {
  MOE_CAP_CEIL = 0,
  MOE_CAP_FLOOR = 1
} moe_cap_round;

typedef enum {
  MOE_ROWS_PACKED = 0,       /* segment e reads rows [offsets[e], offsets[e+1]) of x_rows */
  MOE_ROWS_SHARED = 1        /* segment e reads rows [0, offsets[e+1]-offsets[e]) of x_rows
                                (shared experts: every segment is the same token batch) */
} moe_row_mode;

/* ABI version (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static text for a moe_status value. */
const char* moe_status_string(int status);

/* hipError_t of the last failed HIP call made by this host thread (0 = none). */
int moe_last_hip_error(void);

/*
 * Expert capacity C (host only, no device work).
 * P1 §4.2: capacity = factor * tokens / experts (1000, 8, 1.25 -> 156);
 * P5 专家容量: top-1 needs half the factor of top-2, so C scales with k.
 * Returns round(T * k * cf / E) (ceil or floor per `round_mode`), -1 (= no
 * limit) when cf <= 0, or MOE_ERR_INVALID_ARG (-1 is also "no limit", so
 * callers must check their arguments: T >= 0, k >= 1, E >= 1).
 */
int moe_capacity(int T, int k, int E, double cf, int round_mode);

/*
 * ---- (a) Router: logits, fp32 softmax, top-k, gates --------------------------
 * P4 公式：三步走: z = W_g x per token; P5 选择性精度: the router softmax runs
 * in float32.  P1 §3.3 / P2 §2.1 / P3 §3.1: keep the k largest, optionally
 * renormalise.
 *
 *   x           [T, d]  x_dt = MOE_F32 or MOE_BF16
 *   w_g         [E, d]  fp32
 *   b_g         [E]     fp32, or NULL for no router bias
 *   topk_idx    [T, k]  int32 out: expert ids, largest logit first; equal
 *                       logits give the lower expert id first
 *   topk_gate   [T, k]  fp32 out: gate weights per `gate_mode`
 *   prob_colsum [E]     fp32 out or NULL: sum over tokens of the softmax
 *                       probabilities (the P_e numerator of the aux loss)
 *   logits_dbg  [T, E]  fp32 out or NULL: the fp32 router logits
 * Constraints: 1 <= k <= E, T >= 0, d >= 1, d % 8 == 0 for bf16 x (else
 * MOE_ERR_INVALID_ARG);
 * E <= 256 and k <= 64 (else MOE_ERR_UNSUPPORTED).  T == 0 writes zeros to
 * prob_colsum and returns MOE_OK.  The workspace is needed whenever T > 0
 * or prob_colsum is requested.
 */
size_t moe_router_workspace_size(int T, int d, int E, int x_dt);
int moe_router_topk(const void* x, int x_dt, const float* w_g, const float* b_g,
                    int T, int d, int E, int k, int gate_mode,
                    int32_t* topk_idx, float* topk_gate, float* prob_colsum,
                    float* logits_dbg, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * ---- (a') Router with noisy gating (training mode) ---------------------------
 * P2 §2.1 (Noisy Top-k 门控): the router logits get a standard normal draw
 * times softplus(x W_noise) added before the top-k gating; P5 代码实战
 * (NoisyTop1Gate) gives the noise projection a bias and adds a floor of 1e-2
 * to the scale.  Per token t and expert e:
 *   z[t,e] = (x W_g^T)[t,e] + b_g[e]
 *            + noise[t,e] * (softplus((x W_n^T)[t,e] + b_n[e]) + noise_eps)
 * then everything as moe_router_topk does with its logits: fp32 softmax of
 * z, top-k of z, gates per `gate_mode` (MOE_GATE_RENORM is P2's softmax over
 * the selected noisy logits; MOE_GATE_PROB with k = 1 is P5's gate),
 * prob_colsum of the noisy softmax, logits_dbg = z.
 *
 *   w_n         [E, d]  fp32 noise projection
 *   b_n         [E]     fp32, or NULL for no bias
 *   noise       [T, E]  fp32 in: the normal draws, one per token and expert
 *                       (drawn by the caller, so that a run can be replayed)
 *   noise_eps   >= 0 and finite (0: P2's form, 1e-2: P5's), else
 *               MOE_ERR_INVALID_ARG
 * Every other argument, constraint and error as for moe_router_topk; the
 * workspace is sized by moe_router_noisy_workspace_size.  w_n and noise
 * must be 16-byte aligned; noise may be NULL only when T == 0.  Inference
 * (no noise) is moe_router_topk.
 */
size_t moe_router_noisy_workspace_size(int T, int d, int E, int x_dt);
int moe_router_topk_noisy(const void* x, int x_dt, const float* w_g, const float* b_g,
                          const float* w_n, const float* b_n, const float* noise, float noise_eps,
                          int T, int d, int E, int k, int gate_mode,
                          int32_t* topk_idx, float* topk_gate, float* prob_colsum,
                          float* logits_dbg, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * ---- (b) Dispatch: histogram, scan, stable token-order rank, capacity, permute
 * P1 §2.4: tokens of one expert are gathered together, run as a batch, and
 * scattered back.  P5 专家容量: beyond the capacity the remaining tokens skip
 * the expert (their expert output is 0).  Assignment (t, j) -> expert
 * e = topk_idx[t, j] has rank r = number of assignments to e from tokens
 * before t; it is kept iff capacity < 0 or r < capacity.
 *
 *   topk_idx      [T, k] int32 in (ids outside [0, E) are treated as dropped
 *                 and not counted)
 *   capacity      C >= 0, or -1 for no limit
 *   x             [T, d] in (x_dt MOE_F32 / MOE_BF16), may be NULL together
 *                 with x_perm to skip the row copy
 *   x_perm        [T*k, d] out: packed rows, Xp[dest_pos[t,j]] = x[t]; rows
 *                 at and beyond offsets[E] are left untouched
 *   counts_routed [E]   out: assignments per expert before capacity
 *   counts_kept   [E]   out: min(counts_routed, C)
 *   offsets       [E+1] out: exclusive scan of counts_kept
 *   dest_pos      [T,k] out: packed row of each assignment, -1 if dropped
 *   perm_token    [T*k] out: source token of each packed row; entries at and
 *                 beyond offsets[E] are left untouched
 * Every integer output is unique given topk_idx and is written
 * deterministically.
 */
size_t moe_dispatch_workspace_size(int T, int k, int E);
int moe_dispatch_permute(const int32_t* topk_idx, int T, int k, int E, int capacity,
                         const void* x, int x_dt, int d, void* x_perm,
                         int32_t* counts_routed, int32_t* counts_kept, int32_t* offsets,
                         int32_t* dest_pos, int32_t* perm_token,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ---- (c) Grouped expert FFN over variable-size segments ---------------------
 * Segment e = rows [offsets[e], offsets[e+1]) of the packed batch, run
 * through expert e (P1 §3.2 and P3 §3.1 two-layer FFN experts; P4 linear
 * expert).  The segment sizes are read on the device; `max_rows` is the
 * host-known bound (T*k for routed experts, T per shared expert).
 *
 *   kind      moe_ffn_kind
 *   x_rows    [max_rows, d] (row_mode PACKED) or [max segment, d] (SHARED),
 *             act_dt = MOE_F32 or MOE_BF16
 *   offsets   [E+1] int32 device, non-decreasing, offsets[0] = 0,
 *             offsets[E] <= max_rows
 *   w1        [E, d_ff, d]  (LINEAR: [E, d_out, d])
 *   w3        [E, d_ff, d]  SWIGLU only (up projection), else NULL
 *   w2        [E, d_out, d_ff]  RELU / SWIGLU / GELU, else NULL
 *   w_dt      MOE_F32 (needs act_dt MOE_F32), MOE_BF16 or MOE_FP8_E4M3
 *             (both need act_dt MOE_BF16)
 *   s1,s3,s2  fp32 per-output-row scales for fp8 weights ([E, rows]), else NULL;
 *             the weight is W[r, :] = s[r] * decode(q[r, :])
 *   b1        [E, rows of w1] fp32 or NULL;  b2 [E, d_out] fp32 or NULL
 *             (biases are not supported with SWIGLU)
 *   y_rows    [max_rows, d_out] out, act_dt; rows at and beyond offsets[E]
 *             are left untouched
 * Accumulation is fp32.  With bf16 activations the hidden layer is rounded
 * to bf16 between the two matrix products.
 * Constraints: E <= 1024; with bf16 activations d and d_ff multiples of 8
 * (16 for fp8 weights); no biases with SWIGLU (else MOE_ERR_UNSUPPORTED).
 * w3 must be given exactly for SWIGLU, w2 exactly for RELU / SWIGLU / GELU, the
 * scales exactly for fp8 weights, no b2 for LINEAR (else
 * MOE_ERR_INVALID_ARG).  max_rows == 0 returns MOE_OK without launching.
 * Products with K % 128 == 0 go through the LDS-DMA kernel, others through
 * the register-staged one; results differ only in the order of the fp32
 * accumulation.
 */
size_t moe_ffn_workspace_size(int kind, int act_dt, int max_rows, int E, int d, int d_ff, int d_out);
int moe_expert_ffn_grouped(int kind, const void* x_rows, int act_dt, int max_rows, int row_mode,
                           const int32_t* offsets, int E, int d, int d_ff, int d_out,
                           const void* w1, const void* w3, const void* w2, int w_dt,
                           const float* s1, const float* s3, const float* s2,
                           const float* b1, const float* b2,
                           void* y_rows, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * ---- (c') Grouped expert FFN reading its rows through the dispatch permutation
 * P1 §2.4 gathers the tokens of an expert into one batch before running it;
 * here the gather happens inside the first matrix product: packed row p of
 * segment e is row perm_token[p] of x, read in place, so the packed copy
 * Xp = x[perm_token] (moe_dispatch_permute with x and x_perm) need not exist.
 * The result is bit-identical to moe_dispatch_permute followed by
 * moe_expert_ffn_grouped in MOE_ROWS_PACKED mode.
 *
 *   x           [n_src, d]  the unpermuted activations (act_dt)
 *   n_src       rows of x (T), >= 0
 *   perm_token  [max_rows] int32 device: source row of each packed row, as
 *               moe_dispatch_permute writes it; entries below offsets[E] must
 *               lie in [0, n_src); NULL only when max_rows == 0
 * Every other argument, the workspace (moe_ffn_workspace_size), the
 * constraints and the errors are those of moe_expert_ffn_grouped in
 * MOE_ROWS_PACKED mode; perm_token must be 16-byte aligned.  Rows of x are
 * read through 32-bit offsets by the LDS-DMA kernel when n_src * d * 2 <
 * 2^31, otherwise by the register-staged kernel.
 */
int moe_expert_ffn_gathered(int kind, const void* x, int act_dt, int n_src, const int32_t* perm_token,
                            int max_rows, const int32_t* offsets, int E, int d, int d_ff, int d_out,
                            const void* w1, const void* w3, const void* w2, int w_dt,
                            const float* s1, const float* s3, const float* s2,
                            const float* b1, const float* b2,
                            void* y_rows, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * ---- (d) Combine: gate-weighted gather + shared experts + residual ----------
 * P1 §3.4 and P1 §4.3: weight * expert output accumulated into a
 * zero-initialised output; P3 §3.1: the same weighted sum over the k slots.
 * Dropped slots add nothing and the other gates are not renormalised.
 *
 *   y[t] = sum_{j : dest_pos[t,j] >= 0} topk_gate[t,j] * y_rows[dest_pos[t,j]]
 *        + sum_{s < n_shared} shared_y[s, t]  (+ residual[t])
 *
 *   y_rows    [*, d_out]  dt (MOE_F32 or MOE_BF16)
 *   shared_y  [n_shared, T, d_out] dt, or NULL when n_shared == 0
 *   residual  [T, d_out] dt, or NULL
 *   y         [T, d_out] out, dt.  Summation is fp32 in slot order, then the
 *             shared experts in order, then the residual.
 */
int moe_combine(const void* y_rows, int dt, const int32_t* dest_pos, const float* topk_gate,
                int T, int k, int d_out, const void* shared_y, int n_shared,
                const void* residual, void* y, hipStream_t stream);

/*
 * ---- Aux loss: Switch load balancing -------------------------------------------
 * P5 负载均衡损失函数: alpha * N * sum_i f_i * P_i, f_i the fraction of hard
 * assignments to expert i, P_i the mean router probability; P1 §3.4 divides
 * the selection counts by tokens * k.  f uses counts_routed (before capacity).
 *
 *   counts_routed [E] int32, prob_colsum [E] fp32 (from the router)
 *   loss          device fp32 scalar out
 * T == 0 writes 0.
 */
int moe_aux_loss(const int32_t* counts_routed, const float* prob_colsum, int T, int k, int E,
                 float alpha, float* loss, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
