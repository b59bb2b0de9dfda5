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
 * Variants: moe_router_topk_noisy or moe_router_topk_noisy_philox in place
 * of moe_router_topk (noisy gating in training mode, with the caller's
 * normal draws or with draws from a counter-based generator);
 * moe_dispatch_permute without the row copy followed by
 * moe_expert_ffn_gathered in place of moe_expert_ffn_grouped for the routed
 * experts (the FFN reads x through the permutation); and, for training,
 * moe_expert_ffn_grouped_train in place of moe_expert_ffn_grouped (the
 * first product's pre-activations kept for the backward calls below).
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
  MOE_ERR_WORKSPACE = -4,    /* workspace NULL or smaller than *_workspace_size() */
  MOE_ERR_SCRATCH_LIMIT = -5 /* the allocation-free call needs more than MOE_NOALLOC_SCRATCH_BYTES */
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
 * ---- (a'') Router without a workspace, for callers that cannot allocate --------
 * For callers that cannot call hipMalloc or pass a workspace (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same operation, arguments, outputs and errors as moe_router_topk, with its
 * scratch (what moe_router_workspace_size reports) in a fixed device array
 * of MOE_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  The call allocates nothing.  A call whose scratch
 * would exceed that size returns MOE_ERR_SCRATCH_LIMIT before any launch
 * (the Mixtral-shaped router needs 8 KB, the DeepSeekMoE-shaped one about
 * 4 MB; the 32768-token, 256-expert one does not fit).  Every call on one GPU
 * shares that GPU's array: two calls that overlap in time on the same GPU
 * (other streams or host threads) race; calls ordered on one stream do not.
 * The first call on a device looks up the array's address on it.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
int moe_router_topk_noalloc(const void* x, int x_dt, const float* w_g, const float* b_g,
                            int T, int d, int E, int k, int gate_mode,
                            int32_t* topk_idx, float* topk_gate, float* prob_colsum,
                            float* logits_dbg, hipStream_t stream);

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
 * ---- (a'') The noisy gate's draws from a counter-based generator ------------
 * The pages draw the normal sample inside the gate (P2 §2.1; P5 代码实战,
 * NoisyTop1Gate in training mode) and name no generator.  Here draw number
 * i of the stream (seed, offset) is fixed by those three integers alone:
 *   Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
 *   Easy as 1, 2, 3", SC 2011) with key (seed low 32 bits, seed high 32
 *   bits) on counter (j low, j high, offset low, offset high), j = i / 4,
 *   gives words w0..w3; with p = (i mod 4) / 2, u1 = (w[2p] + 1/2) 2^-32 and
 *   u2 = (w[2p+1] + 1/2) 2^-32, the draw is sqrt(-2 ln u1) cos(2 pi u2) for
 *   even i and sqrt(-2 ln u1) sin(2 pi u2) for odd i (Box-Muller), computed
 *   in fp64 and rounded once to fp32.
 * The noisy gate uses draw t * E + e for token t and expert e, so a
 * training step passes a fresh offset (or seed) and the same (seed, offset)
 * reproduces its draws.
 *
 * moe_router_topk_noisy_philox: moe_router_topk_noisy with noise[t, e] =
 * draw t * E + e, drawn inside the router's kernels (no [T, E] buffer).
 * Every other argument, constraint, workspace and error as for
 * moe_router_topk_noisy; moe_aux_loss_from_router reads its workspace with
 * noisy = 1.
 *
 * moe_gate_noise_philox: out[i] = draw i for i < n (fp32 [n] out, device
 * memory, 4-byte aligned), e.g. the [T, E] draws of one call of
 * moe_router_topk_noisy_philox for moe_router_topk_noisy or for a replay.
 * n = 0 launches nothing; n > 2^62 or out == NULL (n > 0) is
 * MOE_ERR_INVALID_ARG.
 */
int moe_router_topk_noisy_philox(const void* x, int x_dt, const float* w_g, const float* b_g,
                                 const float* w_n, const float* b_n, uint64_t seed, uint64_t offset,
                                 float noise_eps, int T, int d, int E, int k, int gate_mode,
                                 int32_t* topk_idx, float* topk_gate, float* prob_colsum,
                                 float* logits_dbg, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);
int moe_gate_noise_philox(uint64_t seed, uint64_t offset, size_t n, float* out, hipStream_t stream);

/*
 * ---- (b) Dispatch: histogram, scan, stable token-order rank, capacity, permute
 * P1 §2.4: tokens of one expert are gathered together, run as a batch, and
 * scattered back.  P5 专家容量: beyond the capacity the remaining tokens skip
 * the expert (their expert output is 0).  Assignment (t, j) -> expert
 * e = topk_idx[t, j] has rank r = number of assignments to e from tokens
 * before t; it is kept iff capacity < 0 or r < capacity.
 *
 *   topk_idx      [T, k] int32 in (ids outside [0, E) are treated as dropped
 *                 and not counted).  The ids of one token must be distinct,
 *                 as the router writes them (P1 §3.3: the k largest of E
 *                 scores are k different experts).  With a repeated id in a
 *                 token the integer outputs are unspecified, but every write
 *                 still stays inside the output buffers.
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
 * deterministically.  Any T, k and d the arguments allow: rows wider than
 * 64 KB, more than 256 slots per token or more than 64512 assignments take
 * the count/rank/permute kernels instead of the one-launch kernel, with the
 * same results.
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
 *               lie in [0, n_src) (an entry outside is clamped into that
 *               range, so no read leaves x); NULL only when max_rows == 0
 * Every other argument, the workspace (moe_ffn_workspace_size), the
 * constraints and the errors are those of moe_expert_ffn_grouped in
 * MOE_ROWS_PACKED mode; perm_token must be 16-byte aligned, and n_src == 0
 * with max_rows > 0 is MOE_ERR_INVALID_ARG.  Rows of x are
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
 * ---- (c'') Expert FFN on fp8 activations ---------------------------------------
 * P2's deployment paragraph quantises the expert weights (int8, -75% storage)
 * and P3 §4.2 runs INT4 experts next to an FP16 router: quantise the experts,
 * keep the router precise.  Here both matrix products of an expert run on
 * e4m3 values (OCP E4M3FN, v_mfma_scale_f32_32x32x64_f8f6f4, twice the bf16
 * MFMA rate): the inputs as per-row codes and scales from
 * moe_quantize_rows_e4m3, the weights as per-output-row codes and scales (as
 * moe_expert_ffn_grouped takes them).  The hidden layer is formed in fp32
 * from the scaled accumulators, rounded to bf16 and quantised per row the
 * same way before the second product.  Output bf16.  Accuracy: the matrix
 * cores cut each e4m3 product toward zero to 13 bits below the largest
 * product of its aligned group of 8 k (under 7 2^-13 max|x| max|w| per
 * group) and add the group sums with fp32 precision.
 *
 * moe_quantize_rows_e4m3: scale[r] = max_c |x[r, c]| / 448 (1 for an all-zero
 * row), q[r, c] = the e4m3 value nearest to x[r, c] / scale[r] (ties to
 * even); both divisions in IEEE fp32.  x [rows, cols] bf16 or fp32, 16-byte
 * aligned; q [rows, cols] uint8 (8-byte aligned), scale [rows] fp32;
 * cols % 8 == 0 (else MOE_ERR_UNSUPPORTED).
 *
 * moe_expert_ffn_fp8: segment e = rows [offsets[e], offsets[e+1]) run through
 * expert e (no biases).  Row p of segment e reads row gather[p] of xq (the
 * dispatch's perm_token: no packed copy) when gather is given (row_mode
 * PACKED only), else row p (PACKED) or row p - offsets[e] (SHARED); its
 * scale is x_scale at the same row.
 *   xq       [n_src or max_rows, d] e4m3 codes;  x_scale [same rows] fp32
 *   w1, w3   [E, d_ff, d] e4m3 (LINEAR: w1 [E, d_out, d]);  w2 [E, d_out, d_ff]
 *   s1, s3, s2  [E, rows] fp32 weight row scales
 *   y_rows   [max_rows, d_out] bf16 out; rows at and beyond offsets[E] untouched
 * d and d_ff multiples of 128, d_out of 8 (else MOE_ERR_UNSUPPORTED); E <= 1024.
 * The workspace (moe_ffn_fp8_workspace_size) holds, each part starting at a
 * multiple of 256 bytes: the tile map (E + 1 int32), then for the two-layer
 * kinds the hidden layer H [max_rows, d_ff] bf16, its codes [max_rows, d_ff]
 * uint8 and its row scales [max_rows] fp32 (rows below offsets[E] valid
 * after the call).
 */
int moe_quantize_rows_e4m3(const void* x, int x_dt, int rows, int cols, uint8_t* q, float* scale,
                           hipStream_t stream);
size_t moe_ffn_fp8_workspace_size(int kind, int max_rows, int E, int d_ff);
int moe_expert_ffn_fp8(int kind, const void* xq, const float* x_scale, int n_src, const int32_t* gather,
                       int row_mode, int max_rows, const int32_t* offsets, int E, int d, int d_ff, int d_out,
                       const void* w1, const void* w3, const void* w2, const float* s1, const float* s3,
                       const float* s2, void* y_rows, void* workspace, size_t workspace_bytes,
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
 * Any T >= 0 (beyond 65535 tokens each row of blocks takes several tokens).
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

/*
 * The same loss straight from a router call's workspace, for callers that
 * pass prob_colsum = NULL to moe_router_topk or moe_router_topk_noisy: the
 * router then leaves its per-block probability column sums in the workspace
 * and launches nothing more.  This call forms the column sums into
 * prob_colsum and the loss, in one launch for up to 32 experts (two beyond:
 * a single block would be slower than the extra launch).  Both equal, bit
 * for bit, what the router with prob_colsum followed by moe_aux_loss give
 * (the same fp64 partial sums and reduction trees).
 *   router_workspace  the workspace of that router call, not written to
 *                     since; T, d, E, x_dt as passed to it; noisy = 1 for
 *                     moe_router_topk_noisy, 0 for moe_router_topk
 *   counts_routed [E] int32; prob_colsum [E] fp32 out (required); loss out
 * Errors as moe_aux_loss, plus MOE_ERR_WORKSPACE when T > 0 and the
 * workspace is smaller than that router call needs.
 */
int moe_aux_loss_from_router(const int32_t* counts_routed, const void* router_workspace,
                             size_t workspace_bytes, int T, int d, int E, int x_dt, int noisy,
                             int k, float alpha, float* prob_colsum, float* loss,
                             hipStream_t stream);

/*
 * ==== Backward pass (training) ==================================================
 * Gradients of L = <dy, y> + daux * aux for the forward layer above, given
 * the layer-output gradient dy [T, d_out] and the aux-loss gradient daux.
 * P1 §4.3: the output is accumulated into zeros (index_add_), so each token's
 * gradient goes back to exactly the expert rows it came from, and the top-k
 * weight normalisation stays inside the graph; P1 §3.5: the training step
 * differentiates task loss + coef * aux loss; P3 §2.2: the router's gradient
 * comes back through the selected experts only; P5 负载均衡损失函数: f_i is
 * discrete and carries no gradient, P_i does.  The top-k selection and the
 * capacity drops are piecewise constant and pass no gradient.
 * Order of the calls: moe_combine_backward -> moe_expert_ffn_grouped_backward
 * (routed experts on the packed rows with the dYe rows; shared experts on x
 * with dy itself, MOE_ROWS_SHARED) -> moe_router_backward ->
 * moe_permute_backward.  Same conventions as the forward calls (device
 * pointers, caller workspaces, asynchronous, validated before any launch).
 * Reductions run in a fixed order: results are reproducible bit for bit.
 */

/*
 * Combine backward.  For each kept slot (dest_pos[t,j] >= 0):
 *   dy_rows[dest_pos[t,j]] = topk_gate[t,j] * dy[t]       (dt, rounded once)
 *   dgate[t,j]             = sum_c dy[t,c] * y_rows[dest_pos[t,j],c]  (fp32)
 * and dgate[t,j] = 0 for a dropped slot.  The gradient of each shared
 * expert's output and of the residual is dy itself.
 *   dy, y_rows  [T, d_out], [*, d_out] in dt (MOE_F32 or MOE_BF16)
 *   dy_rows     [*, d_out] out, dt: rows not referenced are left untouched
 *   dgate       [T, k] fp32 out
 * d_out must be a multiple of 8 (bf16) or 4 (fp32), else MOE_ERR_UNSUPPORTED.
 */
int moe_combine_backward(const void* dy, int dt, const void* y_rows, const int32_t* dest_pos,
                         const float* topk_gate, int T, int k, int d_out, void* dy_rows, float* dgate,
                         hipStream_t stream);

/*
 * Grouped expert FFN backward: for each segment (the rows routed to expert
 * e; MOE_ROWS_SHARED as in moe_expert_ffn_grouped), with X the segment's
 * input rows and dY their output gradients:
 *   LINEAR  y = W1 x + b1:             dX = dY W1, dW1 = dY^T X, db1 = sum dY
 *   RELU / GELU  h = W1 x + b1, a = act(h), y = W2 a + b2:
 *           dW2 = dY^T a, db2 = sum dY, dh = (dY W2) act'(h), dW1 = dh^T X,
 *           db1 = sum dh, dX = dh W1
 *   SWIGLU  h1 = W1 x, h3 = W3 x, a = silu(h1) h3, y = W2 a:
 *           da = dY W2, dh1 = da h3 silu'(h1), dh3 = da silu(h1),
 *           dW2 = dY^T a, dW1 = dh1^T X, dW3 = dh3^T X, dX = dh1 W1 + dh3 W3
 * h1, h3 (h) are recomputed from X and kept in fp32 (the derivatives of
 * SiLU and GELU have roots, where a bf16 pre-activation would only be
 * absolutely accurate); dh1, dh3 and a are rounded to bf16 between the
 * matrix products; the weight gradients accumulate in fp32 over the
 * segment's rows.
 *   x_rows   [max_rows, d] (PACKED) or [T, d] (SHARED), bf16
 *   dy_rows  [max_rows, d_out] (PACKED: the dy_rows of moe_combine_backward)
 *            or [T, d_out] (SHARED: dy), bf16
 *   dx_rows  [max_rows, d] out, bf16 (PACKED and SHARED alike: row r of the
 *            packed batch; shared expert s writes rows s T .. s T + T - 1)
 *   dw1      [E, rows of w1, d] fp32 out; dw3 [E, d_ff, d] (SWIGLU only);
 *   dw2      [E, d_out, d_ff] (two-layer kinds); db1, db2 [E, *] fp32, given
 *            exactly when b1, b2 are
 * bf16 activations and weights only (else MOE_ERR_UNSUPPORTED); d, d_ff and
 * d_out multiples of 8.  An expert with no rows gets zero gradients.
 */
size_t moe_ffn_backward_workspace_size(int kind, int max_rows, int E, int d, int d_ff, int d_out);
int moe_expert_ffn_grouped_backward(int kind, const void* x_rows, int act_dt, int max_rows, int row_mode,
                                    const int32_t* offsets, int E, int d, int d_ff, int d_out,
                                    const void* w1, const void* w3, const void* w2, int w_dt,
                                    const float* b1, const float* b2, const void* dy_rows, void* dx_rows,
                                    float* dw1, float* dw3, float* dw2, float* db1, float* db2,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Training forward and backward with the first product kept (no
 * recomputation in the backward).
 *
 * moe_expert_ffn_grouped_train: moe_expert_ffn_grouped for kind RELU, GELU
 * or SWIGLU with bf16 activations and weights (PACKED or SHARED rows), which
 * also writes the fp32 pre-activations of the first product, the values its
 * activation was applied to:
 *   h1  [max_rows, d_ff] fp32 out: W1 x + b1 (RELU, GELU), W1 x (SWIGLU)
 *   h3  [max_rows, d_ff] fp32 out: W3 x (SWIGLU only; NULL otherwise)
 * y_rows is the same, bit for bit, as moe_expert_ffn_grouped's.  Shapes the
 * LDS-DMA GEMM does not take (d not a multiple of 128, or a weight matrix of
 * 2 GiB and more) return MOE_ERR_UNSUPPORTED before writing y_rows, h1 or
 * h3: run moe_expert_ffn_grouped and moe_expert_ffn_grouped_backward then.
 * kind LINEAR, fp8 or fp32 data, or h1 == NULL with max_rows > 0, are
 * MOE_ERR_INVALID_ARG.  Workspace: moe_ffn_workspace_size.
 *
 * moe_expert_ffn_grouped_backward_kept: moe_expert_ffn_grouped_backward
 * with h1 (h3) the pre-activations kept by moe_expert_ffn_grouped_train for
 * the same rows and weights, read instead of recomputed; the gradients are
 * the same, bit for bit.  Its workspace (moe_ffn_backward_kept_workspace_size)
 * leaves out the two [max_rows, d_ff] fp32 buffers of the recomputation.
 */
int moe_expert_ffn_grouped_train(int kind, const void* x_rows, int act_dt, int max_rows, int row_mode,
                                 const int32_t* offsets, int E, int d, int d_ff, int d_out,
                                 const void* w1, const void* w3, const void* w2, int w_dt,
                                 const float* b1, const float* b2, void* y_rows, float* h1, float* h3,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);
size_t moe_ffn_backward_kept_workspace_size(int kind, int max_rows, int E, int d, int d_ff, int d_out);
int moe_expert_ffn_grouped_backward_kept(int kind, const void* x_rows, int act_dt, int max_rows, int row_mode,
                                         const int32_t* offsets, int E, int d, int d_ff, int d_out,
                                         const void* w1, const void* w3, const void* w2, int w_dt,
                                         const float* b1, const float* b2, const float* h1, const float* h3,
                                         const void* dy_rows, void* dx_rows, float* dw1, float* dw3, float* dw2,
                                         float* db1, float* db2, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * Router backward.  From the forward's fp32 logits z [T, E] (logits_dbg of
 * moe_router_topk), its top-k ids and gates and the gate gradients dgate of
 * moe_combine_backward, per token in fp32: p = softmax(z); the gate
 * gradient dp (MOE_GATE_PROB: dp[S_j] += dgate_j; MOE_GATE_RENORM: dp[S_j]
 * += (dgate_j - sum_i dgate_i gate_i) / sum_i p[S_i]); the balance loss
 * alpha E sum_e f_e P_e adds daux alpha E f_e / T to dp[e] of every token
 * (f_e = counts_routed[e] / (T k), constant); dz = p (dp - sum_e p dp).
 * Then dW_g = dz^T x and db_g = sum_t dz (token slices summed in fp32, the
 * slices in fp64, in order).  The input gradient dz W_g is added by
 * moe_permute_backward.
 *   dz    [T, E] fp32 out;  dw_g [E, d] fp32 out;  db_g [E] fp32 out or NULL
 * E <= 256 and T <= 65535 x 128 (else MOE_ERR_UNSUPPORTED).  T == 0 writes zero dw_g
 * and db_g.
 */
size_t moe_router_backward_workspace_size(int T, int d, int E);
int moe_router_backward(const void* x, int x_dt, const float* logits, const int32_t* topk_idx,
                        const float* topk_gate, const float* dgate, const int32_t* counts_routed,
                        int T, int d, int E, int k, int gate_mode, float alpha, float daux,
                        float* dz, float* dw_g, float* db_g, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * Permute backward (the transpose of Xp[dest_pos[t,j]] = x[t]) plus the other
 * paths into x, summed in fp32 in this order:
 *   dx[t] = sum_{j kept} dx_rows[dest_pos[t,j]] + sum_{s < n_shared} dx_shared[s, t]
 *           + dres[t] + sum_e dz[t,e] w_g[e, :]
 *   dx_rows    [*, d] dt (moe_expert_ffn_grouped_backward of the routed experts)
 *   dx_shared  [n_shared, T, d] dt or NULL (the shared experts' dx_rows)
 *   dres       [T, d] dt or NULL (dy when the layer adds the residual)
 *   dz, w_g    [T, E], [E, d] fp32, or dz NULL (no router term)
 *   dx         [T, d] out, dt
 */
int moe_permute_backward(const void* dx_rows, int dt, const int32_t* dest_pos, int T, int k, int d,
                         const void* dx_shared, int n_shared, const void* dres, const float* dz,
                         const float* w_g, int E, void* dx, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
