// (c) Grouped expert FFN over variable-size segments.
//
// Segment e holds the rows routed to expert e (P1 §2.4: one batch per
// expert).  Experts are Linear (P4 公式：三步走), Linear-ReLU-Linear (P1 §3.2,
// P3 §3.1) or SwiGLU.  The segment sizes live on the device (offsets), so
// the m-tile -> segment map is built on the device and no count is read back.
//
// bf16 / fp8 weights: two launches of the MFMA grouped GEMM
// (grouped_gemm.hip): gate/up (or the single Linear) with the activation
// fused into its epilogue, then the down projection.  fp32 weights: a plain
// fp32 kernel (one output per thread).
#include <math.h>

#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kMaxE = 1024;

// ------------------------------------------------------------ tile map

// ts[e] = sum over e' < e of ceil(len(e') / bm)   (ts has E + 1 entries)
__global__ __launch_bounds__(1024) void tile_map_kernel(const int32_t* __restrict__ offsets, int E, int bm,
                                                       int32_t* __restrict__ ts) {
  __shared__ int sc[1024];
  const int tid = threadIdx.x;
  int v = 0;
  if (tid < E) {
    int len = offsets[tid + 1] - offsets[tid];
    v = len > 0 ? (len + bm - 1) / bm : 0;
  }
  sc[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int u = tid >= o ? sc[tid - o] : 0;
    __syncthreads();
    sc[tid] += u;
    __syncthreads();
  }
  if (tid < E) ts[tid + 1] = sc[tid];
  if (tid == 0) ts[0] = 0;
}

// ------------------------------------------------------------ fp32 path

constexpr int kF32Cols = 64;
constexpr int kF32Rows = 4;

// out[a, n] = epi(sum_c in[row(a), c] * W[e, n, c]) with the segment of row a
// found by binary search on offsets.
template <int EPI>
__global__ __launch_bounds__(256) void ffn_f32_kernel(const float* __restrict__ in, int in_shared,
                                                     const int32_t* __restrict__ gather, int n_src,
                                                     const int32_t* __restrict__ offsets, int E, int K, int N,
                                                     const float* __restrict__ W, const float* __restrict__ W3,
                                                     const float* __restrict__ bias, float* __restrict__ out) {
  const int total = offsets[E];
  const int n = blockIdx.x * kF32Cols + (threadIdx.x & 63);
  if (n >= N) return;
  for (int a = blockIdx.y * kF32Rows + (threadIdx.x >> 6); a < total; a += gridDim.y * kF32Rows) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (offsets[mid] <= a) lo = mid; else hi = mid;
    }
    const int e = lo;
    // gathered rows are clamped into x, so no entry can address outside it
    const int src = gather ? min(max(gather[a], 0), n_src - 1) : (in_shared ? a - offsets[e] : a);
    const float* xr = in + static_cast<size_t>(src) * K;
    const float* wr = W + (static_cast<size_t>(e) * N + n) * K;
    float acc = 0.f, acc3 = 0.f;
    for (int c = 0; c < K; ++c) acc = fmaf(xr[c], wr[c], acc);
    if (EPI == EPI_SWIGLU) {
      const float* w3r = W3 + (static_cast<size_t>(e) * N + n) * K;
      for (int c = 0; c < K; ++c) acc3 = fmaf(xr[c], w3r[c], acc3);
    }
    if (bias) acc += bias[static_cast<size_t>(e) * N + n];
    float v = acc;
    v = act1<EPI>(acc);
    if (EPI == EPI_SWIGLU) v = silu_f32(acc) * acc3;
    out[static_cast<size_t>(a) * N + n] = v;
  }
}

template <int EPI>
int launch_f32(const float* in, int in_shared, const int32_t* gather, int n_src, const int32_t* offsets, int E, int K,
               int N, const float* W, const float* W3, const float* bias, float* out, int max_rows,
               hipStream_t stream) {
  int gy = (max_rows + kF32Rows - 1) / kF32Rows;
  if (gy > 65535) gy = 65535;
  if (gy < 1) gy = 1;
  dim3 grid((N + kF32Cols - 1) / kF32Cols, gy);
  hipLaunchKernelGGL((ffn_f32_kernel<EPI>), grid, dim3(256), 0, stream, in, in_shared, gather, n_src, offsets, E, K,
                     N, W, W3, bias, out);
  return check_launch();
}

inline int m_tiles_max(int max_rows, int E) { return (max_rows + kGemmBM - 1) / kGemmBM + E; }

int ffn_run(int kind, const void* x_rows, int act_dt, int max_rows, int row_mode, const int32_t* gather,
            int n_src, const int32_t* offsets, int E, int d, int d_ff, int d_out, const void* w1, const void* w3,
            const void* w2, int w_dt, const float* s1, const float* s3, const float* s2, const float* b1,
            const float* b2, void* y_rows, void* workspace, size_t workspace_bytes, hipStream_t stream,
            float* h1 = nullptr, float* h3 = nullptr);

}  // namespace

int current_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

int launch_tile_map(const int32_t* offsets, int E, int bm, int32_t* ts, hipStream_t stream) {
  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(1024), 0, stream, offsets, E, bm, ts);
  return check_launch();
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_ffn_workspace_size(int kind, int act_dt, int max_rows, int E, int d, int d_ff, int d_out) {
  (void)d;
  (void)d_out;
  if (max_rows < 0 || E < 1) return 0;
  size_t s = align_up(static_cast<size_t>(E + 1) * sizeof(int32_t), kWsAlign);
  if (act_dt == MOE_BF16) s += align_up(gemm_partial_bytes(current_cu_count()), kWsAlign);
  if (kind == MOE_FFN_RELU || kind == MOE_FFN_SWIGLU || kind == MOE_FFN_GELU) {
    const size_t esz = act_dt == MOE_F32 ? 4 : 2;
    s += align_up(static_cast<size_t>(max_rows) * static_cast<size_t>(d_ff > 0 ? d_ff : 0) * esz, kWsAlign);
  }
  return s;
}

int moe_expert_ffn_grouped(int kind, const void* x_rows, int act_dt, int max_rows, int row_mode,
                           const int32_t* offsets, int E, int d, int d_ff, int d_out, const void* w1,
                           const void* w3, const void* w2, int w_dt, const float* s1, const float* s3,
                           const float* s2, const float* b1, const float* b2, void* y_rows, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (row_mode != MOE_ROWS_PACKED && row_mode != MOE_ROWS_SHARED) return MOE_ERR_INVALID_ARG;
  return ffn_run(kind, x_rows, act_dt, max_rows, row_mode, nullptr, 0, offsets, E, d, d_ff, d_out, w1, w3, w2, w_dt,
                 s1, s3, s2, b1, b2, y_rows, workspace, workspace_bytes, stream);
}

int moe_expert_ffn_grouped_train(int kind, const void* x_rows, int act_dt, int max_rows, int row_mode,
                                 const int32_t* offsets, int E, int d, int d_ff, int d_out, const void* w1,
                                 const void* w3, const void* w2, int w_dt, const float* b1, const float* b2,
                                 void* y_rows, float* h1, float* h3, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (row_mode != MOE_ROWS_PACKED && row_mode != MOE_ROWS_SHARED) return MOE_ERR_INVALID_ARG;
  if (max_rows > 0 && !h1) return MOE_ERR_INVALID_ARG;
  if (kind == MOE_FFN_LINEAR) return MOE_ERR_INVALID_ARG;   // no activation: nothing to keep
  if (max_rows == 0) {
    // validate as the forward does, keep nothing
    return ffn_run(kind, x_rows, act_dt, 0, row_mode, nullptr, 0, offsets, E, d, d_ff, d_out, w1, w3, w2, w_dt,
                   nullptr, nullptr, nullptr, b1, b2, y_rows, workspace, workspace_bytes, stream);
  }
  return ffn_run(kind, x_rows, act_dt, max_rows, row_mode, nullptr, 0, offsets, E, d, d_ff, d_out, w1, w3, w2, w_dt,
                 nullptr, nullptr, nullptr, b1, b2, y_rows, workspace, workspace_bytes, stream, h1, h3);
}

int moe_expert_ffn_gathered(int kind, const void* x, int act_dt, int n_src, const int32_t* perm_token,
                            int max_rows, const int32_t* offsets, int E, int d, int d_ff, int d_out, const void* w1,
                            const void* w3, const void* w2, int w_dt, const float* s1, const float* s3,
                            const float* s2, const float* b1, const float* b2, void* y_rows, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (n_src < 0 || (max_rows > 0 && (!perm_token || n_src == 0)) || (perm_token && !aligned16(perm_token)))
    return MOE_ERR_INVALID_ARG;
  return ffn_run(kind, x, act_dt, max_rows, MOE_ROWS_PACKED, perm_token, n_src, offsets, E, d, d_ff, d_out, w1, w3,
                 w2, w_dt, s1, s3, s2, b1, b2, y_rows, workspace, workspace_bytes, stream);
}

size_t moe_ffn_fp8_workspace_size(int kind, int max_rows, int E, int d_ff) {
  if (max_rows < 0 || E < 1) return 0;
  size_t s = align_up(static_cast<size_t>(E + 1) * sizeof(int32_t), kWsAlign);
  if (kind == MOE_FFN_RELU || kind == MOE_FFN_SWIGLU || kind == MOE_FFN_GELU) {
    const size_t ff = static_cast<size_t>(max_rows) * static_cast<size_t>(d_ff > 0 ? d_ff : 0);
    s += align_up(ff * 2, kWsAlign) + align_up(ff, kWsAlign) + align_up(static_cast<size_t>(max_rows) * 4, kWsAlign);
  }
  return s;
}

int moe_expert_ffn_fp8(int kind, const void* xq, const float* x_scale, int n_src, const int32_t* gather, int row_mode,
                       int max_rows, const int32_t* offsets, int E, int d, int d_ff, int d_out, const void* w1,
                       const void* w3, const void* w2, const float* s1, const float* s3, const float* s2, void* y_rows,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (kind != MOE_FFN_LINEAR && kind != MOE_FFN_RELU && kind != MOE_FFN_SWIGLU && kind != MOE_FFN_GELU)
    return MOE_ERR_INVALID_ARG;
  if (row_mode != MOE_ROWS_PACKED && row_mode != MOE_ROWS_SHARED) return MOE_ERR_INVALID_ARG;
  if (gather && row_mode != MOE_ROWS_PACKED) return MOE_ERR_INVALID_ARG;
  if (max_rows < 0 || E < 1 || d < 1 || d_out < 1 || n_src < 0) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  const bool two = kind != MOE_FFN_LINEAR;
  if (two && d_ff < 1) return MOE_ERR_INVALID_ARG;
  if (d % 128 != 0 || (two && d_ff % 128 != 0) || d_out % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (!offsets || !w1 || !s1 || (max_rows > 0 && (!xq || !x_scale || !y_rows))) return MOE_ERR_INVALID_ARG;
  if (gather && max_rows > 0 && n_src == 0) return MOE_ERR_INVALID_ARG;
  if ((kind == MOE_FFN_SWIGLU) != (w3 != nullptr) || (kind == MOE_FFN_SWIGLU) != (s3 != nullptr))
    return MOE_ERR_INVALID_ARG;
  if (two != (w2 != nullptr) || two != (s2 != nullptr)) return MOE_ERR_INVALID_ARG;
  const void* p16[] = {xq, offsets, w1, w3, w2, y_rows, gather};
  for (const void* ptr : p16)
    if (ptr && !aligned16(ptr)) return MOE_ERR_INVALID_ARG;
  const void* p4[] = {x_scale, s1, s3, s2};
  for (const void* ptr : p4)
    if (ptr && (reinterpret_cast<uintptr_t>(ptr) & 3u)) return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < moe_ffn_fp8_workspace_size(kind, max_rows, E, d_ff) || !aligned16(workspace))
    return MOE_ERR_WORKSPACE;
  if (max_rows == 0) return MOE_OK;

  char* ws = static_cast<char*>(workspace);
  int32_t* ts = reinterpret_cast<int32_t*>(ws);
  ws += align_up(static_cast<size_t>(E + 1) * sizeof(int32_t), kWsAlign);
  const size_t ff = static_cast<size_t>(max_rows) * static_cast<size_t>(two ? d_ff : 0);
  uint16_t* H = two ? reinterpret_cast<uint16_t*>(ws) : nullptr;
  uint8_t* Hq = two ? reinterpret_cast<uint8_t*>(ws + align_up(ff * 2, kWsAlign)) : nullptr;
  float* sh = two ? reinterpret_cast<float*>(ws + align_up(ff * 2, kWsAlign) + align_up(ff, kWsAlign)) : nullptr;

  // the m-tile prefix: formed by the first GEMM launch itself for a few
  // segments, else by a launch of its own
  const bool ts_in_gemm = E <= kGemmTsBuildMaxE;
  int st = MOE_OK;
  if (!ts_in_gemm) {
    st = launch_tile_map(offsets, E, kGemmBM, ts, stream);
    if (st != MOE_OK) return st;
  }
  const int mtm = m_tiles_max(max_rows, E);
  GemmParams p1{};
  p1.A = static_cast<const uint16_t*>(xq);
  p1.a_shared = row_mode == MOE_ROWS_SHARED ? 1 : 0;
  p1.gather = gather;
  p1.a_rows = n_src;
  p1.offsets = offsets;
  p1.ts = ts;
  p1.ts_build = ts_in_gemm ? ts : nullptr;
  p1.E = E;
  p1.B1 = w1;
  p1.B3 = w3;
  p1.s1 = s1;
  p1.s3 = s3;
  p1.C = two ? H : static_cast<uint16_t*>(y_rows);
  p1.N = two ? d_ff : d_out;
  p1.K = d;
  p1.split_max = 1;
  p1.row_scale = x_scale;
  const int epi1 = kind == MOE_FFN_SWIGLU ? EPI_SWIGLU : kind == MOE_FFN_RELU ? EPI_RELU
                   : kind == MOE_FFN_GELU ? EPI_GELU : EPI_PLAIN;
  st = launch_grouped_gemm_f8(epi1, p1, mtm, stream);
  if (st != MOE_OK || !two) return st;
  // the hidden layer (bf16) quantised per row, rows below offsets[E] only
  st = launch_quant_rows(H, MOE_BF16, max_rows, d_ff, offsets + E, Hq, sh, stream);
  if (st != MOE_OK) return st;
  GemmParams p2{};
  p2.A = reinterpret_cast<const uint16_t*>(Hq);
  p2.offsets = offsets;
  p2.ts = ts;
  p2.E = E;
  p2.B1 = w2;
  p2.s1 = s2;
  p2.C = static_cast<uint16_t*>(y_rows);
  p2.N = d_out;
  p2.K = d_ff;
  p2.split_max = 1;
  p2.row_scale = sh;
  return launch_grouped_gemm_f8(EPI_PLAIN, p2, mtm, stream);
}

}  // extern "C"

namespace moe {
namespace {

int ffn_run(int kind, const void* x_rows, int act_dt, int max_rows, int row_mode, const int32_t* gather,
            int n_src, const int32_t* offsets, int E, int d, int d_ff, int d_out, const void* w1, const void* w3,
            const void* w2, int w_dt, const float* s1, const float* s3, const float* s2, const float* b1,
            const float* b2, void* y_rows, void* workspace, size_t workspace_bytes, hipStream_t stream,
            float* h1, float* h3) {
  if (kind != MOE_FFN_LINEAR && kind != MOE_FFN_RELU && kind != MOE_FFN_SWIGLU && kind != MOE_FFN_GELU)
    return MOE_ERR_INVALID_ARG;
  if (act_dt != MOE_F32 && act_dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (w_dt != MOE_F32 && w_dt != MOE_BF16 && w_dt != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  if (row_mode != MOE_ROWS_PACKED && row_mode != MOE_ROWS_SHARED) return MOE_ERR_INVALID_ARG;
  if (max_rows < 0 || E < 1 || d < 1 || d_out < 1) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  const bool two = kind != MOE_FFN_LINEAR;
  if (two && d_ff < 1) return MOE_ERR_INVALID_ARG;
  if ((w_dt == MOE_F32) != (act_dt == MOE_F32)) return MOE_ERR_UNSUPPORTED;
  if (!offsets || !w1 || (max_rows > 0 && (!x_rows || !y_rows))) return MOE_ERR_INVALID_ARG;
  if ((kind == MOE_FFN_SWIGLU) != (w3 != nullptr)) return MOE_ERR_INVALID_ARG;
  if (two != (w2 != nullptr)) return MOE_ERR_INVALID_ARG;
  if (kind == MOE_FFN_SWIGLU && (b1 || b2)) return MOE_ERR_UNSUPPORTED;
  if (!two && b2) return MOE_ERR_INVALID_ARG;
  const bool fp8 = w_dt == MOE_FP8_E4M3;
  if (fp8) {
    if (!s1 || (kind == MOE_FFN_SWIGLU && !s3) || (two && !s2)) return MOE_ERR_INVALID_ARG;
  } else if (s1 || s3 || s2) {
    return MOE_ERR_INVALID_ARG;
  }
  if (act_dt == MOE_BF16) {
    const int kmul = fp8 ? 16 : 8;
    if (d % kmul != 0 || (two && d_ff % kmul != 0)) return MOE_ERR_UNSUPPORTED;
  }
  // training forward: the first product's fp32 pre-activations kept too
  // (bf16 activations and weights, a two-layer kind, packed or shared rows)
  const bool stash = h1 != nullptr;
  if (stash && (act_dt != MOE_BF16 || w_dt != MOE_BF16 || !two || gather)) return MOE_ERR_INVALID_ARG;
  if (stash && (kind == MOE_FFN_SWIGLU) != (h3 != nullptr)) return MOE_ERR_INVALID_ARG;
  if (!stash && h3) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {x_rows, offsets, w1, w3, w2, s1, s3, s2, b1, b2, y_rows, h1, h3};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_ffn_workspace_size(kind, act_dt, max_rows, E, d, d_ff, d_out);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
  if (max_rows == 0) return MOE_OK;

  char* ws = static_cast<char*>(workspace);
  int32_t* ts = reinterpret_cast<int32_t*>(ws);
  ws += align_up(static_cast<size_t>(E + 1) * sizeof(int32_t), kWsAlign);
  const int n_cu = act_dt == MOE_BF16 ? current_cu_count() : 0;
  float* partial = nullptr;
  if (act_dt == MOE_BF16) {
    partial = reinterpret_cast<float*>(ws);
    ws += align_up(gemm_partial_bytes(n_cu), kWsAlign);
  }
  void* H = ws;
  const int shared_in = row_mode == MOE_ROWS_SHARED ? 1 : 0;
  const int n1 = two ? d_ff : d_out;

  if (act_dt == MOE_F32) {
    const float* X = static_cast<const float*>(x_rows);
    float* Y = static_cast<float*>(y_rows);
    if (kind == MOE_FFN_LINEAR)
      return launch_f32<EPI_PLAIN>(X, shared_in, gather, n_src, offsets, E, d, d_out, static_cast<const float*>(w1), nullptr,
                                   b1, Y, max_rows, stream);
    float* Hf = static_cast<float*>(H);
    const float* W1 = static_cast<const float*>(w1);
    int st = kind == MOE_FFN_RELU
                 ? launch_f32<EPI_RELU>(X, shared_in, gather, n_src, offsets, E, d, d_ff, W1, nullptr, b1, Hf, max_rows, stream)
             : kind == MOE_FFN_GELU
                 ? launch_f32<EPI_GELU>(X, shared_in, gather, n_src, offsets, E, d, d_ff, W1, nullptr, b1, Hf, max_rows, stream)
                 : launch_f32<EPI_SWIGLU>(X, shared_in, gather, n_src, offsets, E, d, d_ff, W1, static_cast<const float*>(w3),
                                          nullptr, Hf, max_rows, stream);
    if (st != MOE_OK) return st;
    return launch_f32<EPI_PLAIN>(Hf, 0, nullptr, 0, offsets, E, d_ff, d_out, static_cast<const float*>(w2), nullptr, b2,
                                 Y, max_rows, stream);
  }

  // the m-tile prefix: formed by the first GEMM launch itself for a few
  // segments, else by a launch of its own
  const bool ts_in_gemm = E <= kGemmTsBuildMaxE;
  int st = MOE_OK;
  if (!ts_in_gemm) {
    st = launch_tile_map(offsets, E, kGemmBM, ts, stream);
    if (st != MOE_OK) return st;
  }
  const int mtm = m_tiles_max(max_rows, E);

  GemmParams p1{};
  p1.A = static_cast<const uint16_t*>(x_rows);
  p1.a_shared = shared_in;
  p1.gather = gather;
  p1.a_rows = n_src;
  p1.offsets = offsets;
  p1.ts = ts;
  p1.ts_build = ts_in_gemm ? ts : nullptr;
  p1.E = E;
  p1.B1 = w1;
  p1.B3 = w3;
  p1.s1 = s1;
  p1.s3 = s3;
  p1.bias = b1;
  p1.C = two ? static_cast<uint16_t*>(H) : static_cast<uint16_t*>(y_rows);
  p1.N = n1;
  p1.K = d;
  p1.partial = partial;
  p1.n_cu = n_cu;
  p1.split_max = kGemmSplitMax;
  const int epi1 = kind == MOE_FFN_SWIGLU ? EPI_SWIGLU
                   : kind == MOE_FFN_RELU ? EPI_RELU
                   : kind == MOE_FFN_GELU ? EPI_GELU
                                          : EPI_PLAIN;
  if (stash) {
    p1.pre1 = h1;
    p1.pre3 = h3;
    st = launch_grouped_gemm_stash(epi1, p1, mtm, stream);
  } else {
    st = launch_grouped_gemm(epi1, fp8, p1, max_rows, mtm, stream);
  }
  if (st != MOE_OK || !two) return st;

  GemmParams p2{};
  p2.A = static_cast<const uint16_t*>(H);
  p2.a_shared = 0;
  p2.offsets = offsets;
  p2.ts = ts;
  p2.E = E;
  p2.B1 = w2;
  p2.s1 = s2;
  p2.bias = b2;
  p2.C = static_cast<uint16_t*>(y_rows);
  p2.N = d_out;
  p2.K = d_ff;
  p2.partial = partial;
  p2.n_cu = n_cu;
  p2.split_max = kGemmSplitMax;
  return launch_grouped_gemm(EPI_PLAIN, fp8, p2, max_rows, mtm, stream);
}

}  // namespace
}  // namespace moe
