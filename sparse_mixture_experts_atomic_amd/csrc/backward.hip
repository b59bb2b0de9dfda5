// Backward pass of the MoE layer: the gradients of <dy, y> + daux * aux.
//
// P1 §4.3: the layer output is accumulated into zeros with index_add_, so a
// token's output gradient goes back to exactly the expert rows it came from,
// and the top-k weight normalisation stays inside the graph.  P1 §3.5: the
// training step differentiates task loss + coef * aux.  P3 §2.2: the router's
// gradient comes back through the selected experts only.  P5 负载均衡损失函数:
// f_i (hard assignment share) carries no gradient, P_i (mean probability)
// does.  The top-k selection and the capacity drops are piecewise constant
// and pass no gradient.
//
// Calls, in reverse order of the forward ones:
//   moe_combine_backward            dYe = g dy per kept slot, dgate = dy . Ye
//   moe_expert_ffn_grouped_backward dXp, dW1, dW3, dW2, db1, db2 per segment
//   moe_router_backward             dz (gates, balance loss, softmax), dW_g, db_g
//   moe_permute_backward            dx = sum of the kept slots' dXp + shared
//                                   + residual + dz W_g
// Every reduction has a fixed order (no atomics), so results are
// reproducible bit for bit.
#include <math.h>

#include <algorithm>

#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kBwThreads = 256;

// sum over the 64 lanes of a wavefront (DPP butterflies, row shifts and row
// broadcasts; lanes outside a row read 0), returned to every lane
__device__ __forceinline__ float dpp_sum_f(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xf, 0xf, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

template <typename T> struct V8;
template <> struct V8<uint16_t> {      // 8 bf16 in 16 bytes
  static constexpr int W = 8;
  using type = uint4;
  __device__ __forceinline__ static void unpack(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static uint4 pack(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
};
template <> struct V8<float> {         // 4 fp32 in 16 bytes
  static constexpr int W = 4;
  using type = float4;
  __device__ __forceinline__ static void unpack(const float4& v, float* f) { f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; }
  __device__ __forceinline__ static float4 pack(const float* f) { return make_float4(f[0], f[1], f[2], f[3]); }
};

// ---------------------------------------------------------------- combine

// One block per token (grid x strided over tokens).  For each kept slot j:
// dYe[dest] = g[t, j] * dy[t] and dgate[t, j] = dy[t] . Ye[dest] (fp32, the
// threads' partial dot products summed by wavefront, then the four
// wavefronts in order); dropped slots get dgate 0 and write no row.
template <typename T>
__global__ __launch_bounds__(kBwThreads) void combine_bwd_kernel(const T* __restrict__ dy, const T* __restrict__ ye,
                                                                const int32_t* __restrict__ dest,
                                                                const float* __restrict__ gate, int T_, int k, int nvec,
                                                                T* __restrict__ dye, float* __restrict__ dgate) {
  using VT = typename V8<T>::type;
  constexpr int W = V8<T>::W;
  extern __shared__ float red[];       // [4 wavefronts][k]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const VT* dyv = reinterpret_cast<const VT*>(dy);
  const VT* yev = reinterpret_cast<const VT*>(ye);
  VT* dyev = reinterpret_cast<VT*>(dye);
  for (int t = blockIdx.x; t < T_; t += gridDim.x) {
    for (int j = 0; j < k; ++j) {
      const int d = dest[static_cast<size_t>(t) * k + j];
      const float g = gate[static_cast<size_t>(t) * k + j];
      float dot = 0.f;
      if (d >= 0) {
        for (int v = tid; v < nvec; v += kBwThreads) {
          float a[W], b[W], o[W];
          V8<T>::unpack(dyv[static_cast<size_t>(t) * nvec + v], a);
          V8<T>::unpack(yev[static_cast<size_t>(d) * nvec + v], b);
#pragma unroll
          for (int i = 0; i < W; ++i) {
            dot = fmaf(a[i], b[i], dot);
            o[i] = g * a[i];
          }
          dyev[static_cast<size_t>(d) * nvec + v] = V8<T>::pack(o);
        }
      }
      dot = dpp_sum_f(dot);
      if (lane == 0) red[wave * k + j] = dot;
    }
    __syncthreads();
    for (int j = tid; j < k; j += kBwThreads) {
      const int d = dest[static_cast<size_t>(t) * k + j];
      dgate[static_cast<size_t>(t) * k + j] = d >= 0 ? ((red[j] + red[k + j]) + red[2 * k + j]) + red[3 * k + j] : 0.f;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- router

// dz per token: p = softmax(z) in fp32 (as the forward), dp from the gates
// (prob: dp[S_j] += dg_j; renorm: dp[S_j] += (dg_j - sum_i dg_i g_i) / s)
// and the balance loss (dp[e] += coef * counts[e] for every token), then
// dz = p (dp - sum p dp).  One wavefront per token, expert e on lane e % 64,
// slot e / 64.  Per-block column sums of dz (for db_g) go to the workspace.
constexpr int kRbMaxE = 256;
template <int S>
__global__ __launch_bounds__(kBwThreads) void router_dz_kernel(const float* __restrict__ logits,
                                                              const int32_t* __restrict__ idx,
                                                              const float* __restrict__ gate,
                                                              const float* __restrict__ dgate,
                                                              const int32_t* __restrict__ counts, int T_, int E, int k,
                                                              int mode, float aux_coef, float* __restrict__ dz,
                                                              float* __restrict__ colpart) {
  __shared__ float wcol[4][kRbMaxE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  float csum[S];
  float aux[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    csum[i] = 0.f;
    const int e = lane + 64 * i;
    aux[i] = e < E ? aux_coef * static_cast<float>(counts[e]) : 0.f;
  }
  constexpr int kTokPerBlock = 16;
  const int t_end = min(T_, (blockIdx.x + 1) * kTokPerBlock);
  for (int t = blockIdx.x * kTokPerBlock + wave; t < t_end; t += 4) {
    float z[S], p[S], dp[S];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int e = lane + 64 * i;
      z[i] = e < E ? logits[static_cast<size_t>(t) * E + e] : -INFINITY;
      m = fmaxf(m, z[i]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int e = lane + 64 * i;
      p[i] = e < E ? expf(z[i] - m) : 0.f;
      s += p[i];
    }
    s = dpp_sum_f(s);
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      p[i] *= inv;
      dp[i] = aux[i];
    }
    // selected probabilities, their sum and sum dg g (renorm)
    float ssel = 0.f, c = 0.f;
    if (mode == MOE_GATE_RENORM) {
      for (int j = 0; j < k; ++j) {
        const int e = idx[static_cast<size_t>(t) * k + j];
        // p of expert e lives on lane e % 64, slot e / 64
        float pv = 0.f;
#pragma unroll
        for (int i = 0; i < S; ++i) {
          const float q = __shfl(p[i], e & 63);
          if ((e >> 6) == i) pv = q;
        }
        ssel += pv;
        c += dgate[static_cast<size_t>(t) * k + j] * gate[static_cast<size_t>(t) * k + j];
      }
    }
    for (int j = 0; j < k; ++j) {
      const int e = idx[static_cast<size_t>(t) * k + j];
      const float dg = dgate[static_cast<size_t>(t) * k + j];
      const float add = mode == MOE_GATE_RENORM ? (dg - c) / ssel : dg;
#pragma unroll
      for (int i = 0; i < S; ++i)
        if (lane + 64 * i == e) dp[i] += add;
    }
    float pd = 0.f;
#pragma unroll
    for (int i = 0; i < S; ++i) pd = fmaf(p[i], dp[i], pd);
    pd = dpp_sum_f(pd);
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        const float g = p[i] * (dp[i] - pd);
        dz[static_cast<size_t>(t) * E + e] = g;
        csum[i] += g;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < S; ++i)
    if (lane + 64 * i < E) wcol[wave][lane + 64 * i] = csum[i];
  __syncthreads();
  for (int e = tid; e < E; e += kBwThreads)
    colpart[static_cast<size_t>(blockIdx.x) * E + e] = ((wcol[0][e] + wcol[1][e]) + wcol[2][e]) + wcol[3][e];
}

// Partial dW_g[e, c] = sum over the block's token slice of dz[t, e] x[t, c]:
// block (column chunk of 256, slice of kRwSlice tokens, expert group of 8);
// fp32 sums over the slice, written to part[slice][e][c].
constexpr int kRwSlice = 128;
constexpr int kRwEg = 8;
template <typename XT>
__global__ __launch_bounds__(kBwThreads) void router_dw_kernel(const XT* __restrict__ x, const float* __restrict__ dz,
                                                              int T_, int d, int E, float* __restrict__ part) {
  __shared__ float dzs[kRwSlice][kRwEg];
  const int c = blockIdx.x * kBwThreads + threadIdx.x;
  const int t0 = blockIdx.y * kRwSlice;
  const int e0 = blockIdx.z * kRwEg;
  const int nt = min(kRwSlice, T_ - t0);
  for (int i = threadIdx.x; i < kRwSlice * kRwEg; i += kBwThreads) {
    const int tl = i / kRwEg, el = i % kRwEg;
    dzs[tl][el] = (tl < nt && e0 + el < E) ? dz[static_cast<size_t>(t0 + tl) * E + e0 + el] : 0.f;
  }
  __syncthreads();
  if (c >= d) return;
  float acc[kRwEg];
#pragma unroll
  for (int i = 0; i < kRwEg; ++i) acc[i] = 0.f;
  for (int tl = 0; tl < nt; ++tl) {
    const float xv = Elem<XT>::load(x, static_cast<size_t>(t0 + tl) * d + c);
#pragma unroll
    for (int i = 0; i < kRwEg; ++i) acc[i] = fmaf(dzs[tl][i], xv, acc[i]);
  }
#pragma unroll
  for (int i = 0; i < kRwEg; ++i)
    if (e0 + i < E) part[(static_cast<size_t>(blockIdx.y) * E + e0 + i) * d + c] = acc[i];
}

// out[i] = sum over s < ns of part[s * n + i], in slice order, in fp64
__global__ __launch_bounds__(kBwThreads) void slice_sum_kernel(const float* __restrict__ part, int ns, long n,
                                                              float* __restrict__ out) {
  const long i = static_cast<long>(blockIdx.x) * kBwThreads + threadIdx.x;
  if (i >= n) return;
  double s = 0.0;
  for (int q = 0; q < ns; ++q) s += static_cast<double>(part[static_cast<size_t>(q) * n + i]);
  out[i] = static_cast<float>(s);
}

// ---------------------------------------------------------------- permute

// dx[t] = sum over kept slots of dXp[dest[t, j]] + sum_s dXs[s, t] + dres[t]
// + sum_e dz[t, e] W_g[e, :], fp32 in that order; one thread per 16-byte
// output vector, tokens on grid y (strided past its limit).
template <typename T>
__global__ __launch_bounds__(kBwThreads) void permute_bwd_kernel(const T* __restrict__ dxp, const int32_t* __restrict__ dest,
                                                                int T_, int k, int nvec, const T* __restrict__ dxs,
                                                                int n_shared, const T* __restrict__ dres,
                                                                const float* __restrict__ dz, const float* __restrict__ w_g,
                                                                int E, T* __restrict__ dx) {
  using VT = typename V8<T>::type;
  constexpr int W = V8<T>::W;
  const int v = blockIdx.x * kBwThreads + threadIdx.x;
  if (v >= nvec) return;
  const VT* a = reinterpret_cast<const VT*>(dxp);
  for (int t = blockIdx.y; t < T_; t += gridDim.y) {
    float acc[W];
#pragma unroll
    for (int i = 0; i < W; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int d = dest[static_cast<size_t>(t) * k + j];
      if (d < 0) continue;
      float f[W];
      V8<T>::unpack(a[static_cast<size_t>(d) * nvec + v], f);
#pragma unroll
      for (int i = 0; i < W; ++i) acc[i] += f[i];
    }
    for (int s = 0; s < n_shared; ++s) {
      float f[W];
      V8<T>::unpack(reinterpret_cast<const VT*>(dxs)[(static_cast<size_t>(s) * T_ + t) * nvec + v], f);
#pragma unroll
      for (int i = 0; i < W; ++i) acc[i] += f[i];
    }
    if (dres) {
      float f[W];
      V8<T>::unpack(reinterpret_cast<const VT*>(dres)[static_cast<size_t>(t) * nvec + v], f);
#pragma unroll
      for (int i = 0; i < W; ++i) acc[i] += f[i];
    }
    if (dz) {
      const int d = nvec * W;
      for (int e = 0; e < E; ++e) {
        const float g = dz[static_cast<size_t>(t) * E + e];
        const float4* wr = reinterpret_cast<const float4*>(w_g + static_cast<size_t>(e) * d + v * W);
#pragma unroll
        for (int q = 0; q < W / 4; ++q) {
          const float4 w = wr[q];
          acc[4 * q] = fmaf(g, w.x, acc[4 * q]);
          acc[4 * q + 1] = fmaf(g, w.y, acc[4 * q + 1]);
          acc[4 * q + 2] = fmaf(g, w.z, acc[4 * q + 2]);
          acc[4 * q + 3] = fmaf(g, w.w, acc[4 * q + 3]);
        }
      }
    }
    reinterpret_cast<VT*>(dx)[static_cast<size_t>(t) * nvec + v] = V8<T>::pack(acc);
  }
}

// ---------------------------------------------------------------- bias sums

// out[e, c] = sum of rows r of segment e of M[*, c] (fp32, row order);
// shared: segment e's rows are 0 .. len - 1
__global__ __launch_bounds__(kBwThreads) void segment_colsum_kernel(const uint16_t* __restrict__ M, long ld, int N,
                                                                   const int32_t* __restrict__ offsets, int shared,
                                                                   float* __restrict__ out) {
  const int c = blockIdx.x * kBwThreads + threadIdx.x;
  const int e = blockIdx.y;
  if (c >= N) return;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  const int base = shared ? -r0 : 0;
  float s = 0.f;
  for (int r = r0; r < r1; ++r) s += bf16_to_f32(M[static_cast<size_t>(r + base) * ld + c]);
  out[static_cast<size_t>(e) * N + c] = s;
}

inline int gridy(int T) { return T < 65535 ? (T > 0 ? T : 1) : 65535; }

__global__ __launch_bounds__(kBwThreads) void zero_f32_kernel(float* __restrict__ p, long n) {
  for (long i = static_cast<long>(blockIdx.x) * kBwThreads + threadIdx.x; i < n; i += static_cast<long>(gridDim.x) * kBwThreads)
    p[i] = 0.f;
}

int zero_f32(float* p, size_t n, hipStream_t stream) {
  if (!p || n == 0) return MOE_OK;
  const size_t b = (n + kBwThreads - 1) / kBwThreads;
  hipLaunchKernelGGL(zero_f32_kernel, dim3(static_cast<unsigned>(b < 65536 ? b : 65536)), dim3(kBwThreads), 0, stream,
                     p, static_cast<long>(n));
  return check_launch();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_combine_backward(const void* dy, int dt, const void* y_rows, const int32_t* dest_pos, const float* topk_gate,
                         int T, int k, int d_out, void* dy_rows, float* dgate, hipStream_t stream) {
  if (T < 0 || k < 1 || d_out < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if ((dt == MOE_BF16 && d_out % 8) || (dt == MOE_F32 && d_out % 4)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!dy || !y_rows || !dest_pos || !topk_gate || !dy_rows || !dgate) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {dy, y_rows, dest_pos, topk_gate, dy_rows, dgate};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARG;
  const size_t lds = static_cast<size_t>(4) * k * sizeof(float);
  if (lds > 64 * 1024) return MOE_ERR_UNSUPPORTED;
  const int nb = T < 65536 ? T : 65536;
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(combine_bwd_kernel<uint16_t>, dim3(nb), dim3(kBwThreads), lds, stream,
                       static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(y_rows), dest_pos, topk_gate, T,
                       k, d_out / 8, static_cast<uint16_t*>(dy_rows), dgate);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<float>, dim3(nb), dim3(kBwThreads), lds, stream,
                       static_cast<const float*>(dy), static_cast<const float*>(y_rows), dest_pos, topk_gate, T, k,
                       d_out / 4, static_cast<float*>(dy_rows), dgate);
  return check_launch();
}

size_t moe_router_backward_workspace_size(int T, int d, int E) {
  if (T < 0 || d < 1 || E < 1) return 0;
  const size_t nb = (static_cast<size_t>(T) + 15) / 16;
  const size_t ns = (static_cast<size_t>(T) + kRwSlice - 1) / kRwSlice;
  return align_up((nb > 0 ? nb : 1) * E * sizeof(float), kWsAlign) +
         align_up((ns > 0 ? ns : 1) * E * static_cast<size_t>(d) * sizeof(float), kWsAlign);
}

int moe_router_backward(const void* x, int x_dt, const float* logits, const int32_t* topk_idx, const float* topk_gate,
                        const float* dgate, const int32_t* counts_routed, int T, int d, int E, int k, int gate_mode,
                        float alpha, float daux, float* dz, float* dw_g, float* db_g, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || d < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > kRbMaxE) return MOE_ERR_UNSUPPORTED;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (gate_mode != MOE_GATE_PROB && gate_mode != MOE_GATE_RENORM) return MOE_ERR_INVALID_ARG;
  if (!dw_g || (T > 0 && (!x || !logits || !topk_idx || !topk_gate || !dgate || !counts_routed || !dz)))
    return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {x, logits, topk_idx, topk_gate, dgate, counts_routed, dz, dw_g, db_g};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < moe_router_backward_workspace_size(T, d, E) || !aligned16(workspace))
    return MOE_ERR_WORKSPACE;
  const int nb = (T + 15) / 16;
  const int ns = (T + kRwSlice - 1) / kRwSlice;
  if (ns > 65535) return MOE_ERR_UNSUPPORTED;   // token slices of the weight gradient are grid rows
  float* colpart = static_cast<float*>(workspace);
  float* wpart = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          align_up(static_cast<size_t>(nb > 0 ? nb : 1) * E * sizeof(float), kWsAlign));
  if (T > 0) {
    const float coef = T > 0 ? daux * alpha * static_cast<float>(E) / (static_cast<float>(T) * k) / static_cast<float>(T) : 0.f;
    if (E <= 64)
      hipLaunchKernelGGL(router_dz_kernel<1>, dim3(nb), dim3(kBwThreads), 0, stream, logits, topk_idx, topk_gate,
                         dgate, counts_routed, T, E, k, gate_mode, coef, dz, colpart);
    else if (E <= 128)
      hipLaunchKernelGGL(router_dz_kernel<2>, dim3(nb), dim3(kBwThreads), 0, stream, logits, topk_idx, topk_gate,
                         dgate, counts_routed, T, E, k, gate_mode, coef, dz, colpart);
    else
      hipLaunchKernelGGL(router_dz_kernel<4>, dim3(nb), dim3(kBwThreads), 0, stream, logits, topk_idx, topk_gate,
                         dgate, counts_routed, T, E, k, gate_mode, coef, dz, colpart);
    int st = check_launch();
    if (st != MOE_OK) return st;
    const dim3 g((d + kBwThreads - 1) / kBwThreads, ns, (E + kRwEg - 1) / kRwEg);
    if (x_dt == MOE_BF16)
      hipLaunchKernelGGL(router_dw_kernel<uint16_t>, g, dim3(kBwThreads), 0, stream, static_cast<const uint16_t*>(x), dz,
                         T, d, E, wpart);
    else
      hipLaunchKernelGGL(router_dw_kernel<float>, g, dim3(kBwThreads), 0, stream, static_cast<const float*>(x), dz, T, d,
                         E, wpart);
    st = check_launch();
    if (st != MOE_OK) return st;
  }
  const long n = static_cast<long>(E) * d;
  hipLaunchKernelGGL(slice_sum_kernel, dim3(static_cast<unsigned>((n + kBwThreads - 1) / kBwThreads)), dim3(kBwThreads),
                     0, stream, wpart, T > 0 ? ns : 0, n, dw_g);
  int st = check_launch();
  if (st != MOE_OK || !db_g) return st;
  hipLaunchKernelGGL(slice_sum_kernel, dim3((E + kBwThreads - 1) / kBwThreads), dim3(kBwThreads), 0, stream, colpart,
                     T > 0 ? nb : 0, static_cast<long>(E), db_g);
  return check_launch();
}

int moe_permute_backward(const void* dx_rows, int dt, const int32_t* dest_pos, int T, int k, int d,
                         const void* dx_shared, int n_shared, const void* dres, const float* dz, const float* w_g, int E,
                         void* dx, hipStream_t stream) {
  if (T < 0 || k < 1 || d < 1 || n_shared < 0 || E < 0) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if ((dt == MOE_BF16 && d % 8) || (dt == MOE_F32 && d % 4)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!dx_rows || !dest_pos || !dx || (n_shared > 0 && !dx_shared) || (dz && (!w_g || E < 1)))
    return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {dx_rows, dest_pos, dx_shared, dres, dz, w_g, dx};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  const int W = dt == MOE_BF16 ? 8 : 4;
  const int nvec = d / W;
  const dim3 grid((nvec + kBwThreads - 1) / kBwThreads, gridy(T));
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(permute_bwd_kernel<uint16_t>, grid, dim3(kBwThreads), 0, stream,
                       static_cast<const uint16_t*>(dx_rows), dest_pos, T, k, nvec,
                       static_cast<const uint16_t*>(dx_shared), n_shared, static_cast<const uint16_t*>(dres), dz, w_g,
                       dz ? E : 0, static_cast<uint16_t*>(dx));
  else
    hipLaunchKernelGGL(permute_bwd_kernel<float>, grid, dim3(kBwThreads), 0, stream, static_cast<const float*>(dx_rows),
                       dest_pos, T, k, nvec, static_cast<const float*>(dx_shared), n_shared,
                       static_cast<const float*>(dres), dz, w_g, dz ? E : 0, static_cast<float*>(dx));
  return check_launch();
}

}  // extern "C"

// ------------------------------------------------------------------- FFN

namespace moe {
namespace {

// Transposed weights for dX = dh W (the first layer's weights, gate and up
// side by side for SwiGLU): out[e][n][k] = W1[e][k][n] for k < K1, else
// W3[e][k - K1][n]; n < N, k < Kt.  64 x 64 tiles through LDS, 16-byte
// loads and stores of whole 128-byte rows.  With them dX runs on the
// forward's LDS-DMA grouped GEMM (both operands K-contiguous), which reads
// what the register-transposing backward kernel asked of the L2 at a quarter
// of the bytes per MFMA.
__global__ __launch_bounds__(256) void transpose_w_kernel(const uint16_t* __restrict__ W1,
                                                          const uint16_t* __restrict__ W3, int K1, int Kt, int N,
                                                          uint16_t* __restrict__ out) {
  __shared__ uint4 tile[64 * 9];               // 64 rows (k) of 64 bf16, pitch 72 bf16
  const int e = blockIdx.z;
  const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  uint16_t* t16 = reinterpret_cast<uint16_t*>(tile);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i;
    const int r = q >> 3, c = q & 7;
    const int k = k0 + r, n = n0 + 8 * c;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (k < Kt && n < N) {
      const uint16_t* src = k < K1 ? W1 + (static_cast<size_t>(e) * K1 + k) * N
                                   : W3 + (static_cast<size_t>(e) * (Kt - K1) + (k - K1)) * N;
      v = *reinterpret_cast<const uint4*>(src + n);
    }
    tile[r * 9 + c] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i;
    const int r = q >> 3, c = q & 7;             // output row n0 + r, columns k0 + 8 c ..
    const int n = n0 + r, k = k0 + 8 * c;
    if (n < N && k < Kt) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = static_cast<uint32_t>(t16[(8 * c + 2 * j) * 72 + r]) |
               (static_cast<uint32_t>(t16[(8 * c + 2 * j + 1) * 72 + r]) << 16);
      *reinterpret_cast<uint4*>(out + (static_cast<size_t>(e) * N + n) * Kt + k) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Per-segment transposes for the weight gradients: out[f][128 ts[e] + r] =
// in[base_e + r][f] for the r < rows_e of segment e (base_e = offsets[e], or
// 0 when every segment reads the same rows), zero for the padding rows up to
// the next multiple of 128 (ts: the 128-row tile map).  64 x 64 tiles through
// LDS as in transpose_w_kernel; a tile never straddles two segments.
__global__ __launch_bounds__(256) void transpose_seg_kernel(const uint16_t* __restrict__ in, long ldin, int F,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ ts, int E, int shared,
                                                            uint16_t* __restrict__ out, long ldout) {
  __shared__ uint4 tile[64 * 9];
  const int k0 = blockIdx.y * 64, f0 = blockIdx.x * 64;
  if (k0 >= ts[E] * 128) return;
  int lo = 0, hi = E;                          // the segment: largest e with 128 ts[e] <= k0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ts[mid] * 128 <= k0) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int r0 = k0 - ts[e] * 128;
  const int rows = offsets[e + 1] - offsets[e];
  const long base = shared ? 0 : offsets[e];
  const int tid = threadIdx.x;
  uint16_t* t16 = reinterpret_cast<uint16_t*>(tile);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i;
    const int r = q >> 3, c = q & 7;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r0 + r < rows && f0 + 8 * c < F) v = *reinterpret_cast<const uint4*>(in + (base + r0 + r) * ldin + f0 + 8 * c);
    tile[r * 9 + c] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i;
    const int r = q >> 3, c = q & 7;             // output row f0 + r, columns k0 + 8 c ..
    if (f0 + r < F) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = static_cast<uint32_t>(t16[(8 * c + 2 * j) * 72 + r]) |
               (static_cast<uint32_t>(t16[(8 * c + 2 * j + 1) * 72 + r]) << 16);
      *reinterpret_cast<uint4*>(out + static_cast<size_t>(f0 + r) * ldout + k0 + 8 * c) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// out[e] = e M for e <= E (the row offsets of E segments of M rows)
__global__ void iota_kernel(int32_t* out, int E, int M) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) out[e] = e * M;
}

// workspace: the 128- and 256-row tile maps, the fp32 pre-activations h1
// (h3), the bf16 dh [max_rows, n1] ([max_rows, 2 n1] for SwiGLU: dh1 then dh3
// in each row) and activation a [max_rows, d_ff], the transposed first-layer
// weights [E, d, Kt] and the forward GEMM's split-tail partial sums
struct FfnBwdLayout {
  size_t ts128, ts256, h1, h3, dh, a, wt, wt_bytes, partial, kp, xt, dyt, at, dht, wofs_o, wofs_1, tsw_o, tsw_1, total;
};

FfnBwdLayout ffn_bwd_layout(int kind, int max_rows, int E, int d, int d_ff, int d_out, bool stashed = false) {
  FfnBwdLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes, kWsAlign);
    return at;
  };
  const bool two = kind != MOE_FFN_LINEAR;
  const size_t ff = static_cast<size_t>(max_rows) * static_cast<size_t>(d_ff > 0 ? d_ff : 0);
  const size_t kt = two ? static_cast<size_t>(d_ff) * (kind == MOE_FFN_SWIGLU ? 2 : 1) : static_cast<size_t>(d_out);
  L.ts128 = take(static_cast<size_t>(E + 1) * 4);
  L.ts256 = take(static_cast<size_t>(E + 1) * 4);
  // the recomputed pre-activations (none when the caller kept them)
  L.h1 = two && !stashed ? take(ff * 4) : 0;
  L.h3 = kind == MOE_FFN_SWIGLU && !stashed ? take(ff * 4) : 0;
  L.dh = two ? take(static_cast<size_t>(max_rows) * kt * 2) : 0;
  L.a = two ? take(ff * 2) : 0;
  // transposed weights (the first layer's [E, d, kt] for dX, before it the
  // second layer's [E, d_ff, d_out] for da), only for shapes whose products
  // cannot read the weights as stored
  const int n1 = two ? d_ff : d_out;
  const bool tb = grouped_gemm_tb_shape_ok(static_cast<int>(kt), d, n1) &&
                  (!two || grouped_gemm_tb_shape_ok(d_out, d_ff, d_out));
  L.wt = tb ? 0
            : take(static_cast<size_t>(E) * std::max(static_cast<size_t>(d) * kt,
                                                    two ? static_cast<size_t>(d_ff) * static_cast<size_t>(d_out) : 0) * 2);
  L.wt_bytes = tb ? 0 : 1;
  L.partial = take(static_cast<size_t>(current_cu_count()) * 256 * 256 * 4);
  // weight gradients: activations transposed per segment to [features, kp],
  // kp >= max_rows + 128 E bounds the sum of the segments padded to 128 rows
  L.kp = align_up(static_cast<size_t>(max_rows) + 128 * static_cast<size_t>(E), 64);   // 16-byte rows
  L.xt = take(static_cast<size_t>(d) * L.kp * 2);
  L.dyt = take(static_cast<size_t>(d_out) * L.kp * 2);
  L.at = two ? take(static_cast<size_t>(d_ff) * L.kp * 2) : 0;
  L.dht = two ? take(kt * L.kp * 2) : 0;
  L.wofs_o = take(static_cast<size_t>(E + 1) * 4);
  L.wofs_1 = take(static_cast<size_t>(E + 1) * 4);
  L.tsw_o = take(static_cast<size_t>(E + 1) * 4);
  L.tsw_1 = take(static_cast<size_t>(E + 1) * 4);
  L.total = o;
  return L;
}

// The backward of the grouped FFN; h1_in (h3_in): the first product's fp32
// pre-activations kept by the training forward, or nullptr to recompute them.
int ffn_backward_run(int kind, const void* x_rows, int act_dt, int max_rows, int row_mode, const int32_t* offsets,
                     int E, int d, int d_ff, int d_out, const void* w1, const void* w3, const void* w2, int w_dt,
                     const float* b1, const float* b2, const void* dy_rows, void* dx_rows, float* dw1, float* dw3,
                     float* dw2, float* db1, float* db2, const float* h1_in, const float* h3_in, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  if (kind != MOE_FFN_LINEAR && kind != MOE_FFN_RELU && kind != MOE_FFN_SWIGLU && kind != MOE_FFN_GELU)
    return MOE_ERR_INVALID_ARG;
  if (row_mode != MOE_ROWS_PACKED && row_mode != MOE_ROWS_SHARED) return MOE_ERR_INVALID_ARG;
  if (max_rows < 0 || E < 1 || d < 1 || d_out < 1) return MOE_ERR_INVALID_ARG;
  if (E > 1024) return MOE_ERR_UNSUPPORTED;
  const bool two = kind != MOE_FFN_LINEAR;
  if (two && d_ff < 1) return MOE_ERR_INVALID_ARG;
  if (act_dt != MOE_BF16 || w_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;   // bf16 activations and weights
  if (d % 8 || d_out % 8 || (two && d_ff % 8)) return MOE_ERR_UNSUPPORTED;
  if (!offsets || !w1 || !dw1 || (max_rows > 0 && (!x_rows || !dy_rows || !dx_rows))) return MOE_ERR_INVALID_ARG;
  if ((kind == MOE_FFN_SWIGLU) != (w3 != nullptr) || (kind == MOE_FFN_SWIGLU) != (dw3 != nullptr))
    return MOE_ERR_INVALID_ARG;
  if (two != (w2 != nullptr) || two != (dw2 != nullptr)) return MOE_ERR_INVALID_ARG;
  if (kind == MOE_FFN_SWIGLU && (b1 || b2)) return MOE_ERR_UNSUPPORTED;
  if (!two && b2) return MOE_ERR_INVALID_ARG;
  if ((b1 != nullptr) != (db1 != nullptr) || (b2 != nullptr) != (db2 != nullptr)) return MOE_ERR_INVALID_ARG;
  const bool stashed = h1_in != nullptr;
  if (stashed && (!two || (kind == MOE_FFN_SWIGLU) != (h3_in != nullptr))) return MOE_ERR_INVALID_ARG;
  if (!stashed && h3_in) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {x_rows, offsets, w1, w3, w2, b1, b2, dy_rows, dx_rows, dw1, dw3, dw2, db1, db2, h1_in, h3_in};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  const FfnBwdLayout lay = ffn_bwd_layout(kind, max_rows, E, d, d_ff, d_out, stashed);
  if (!workspace || workspace_bytes < lay.total || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
  if (max_rows == 0) {
    // no rows: every weight gradient is zero (a fill kernel, no memset node)
    const size_t n1 = static_cast<size_t>(two ? d_ff : d_out);
    int z = zero_f32(dw1, static_cast<size_t>(E) * n1 * d, stream);
    if (z == MOE_OK) z = zero_f32(dw3, static_cast<size_t>(E) * n1 * d, stream);
    if (z == MOE_OK && dw2) z = zero_f32(dw2, static_cast<size_t>(E) * d_out * d_ff, stream);
    if (z == MOE_OK) z = zero_f32(db1, static_cast<size_t>(E) * n1, stream);
    if (z == MOE_OK) z = zero_f32(db2, static_cast<size_t>(E) * d_out, stream);
    return z;
  }
  char* ws = static_cast<char*>(workspace);
  int32_t* ts128 = reinterpret_cast<int32_t*>(ws + lay.ts128);
  float* h1w = two && !stashed ? reinterpret_cast<float*>(ws + lay.h1) : nullptr;
  float* h3w = kind == MOE_FFN_SWIGLU && !stashed ? reinterpret_cast<float*>(ws + lay.h3) : nullptr;
  const float* h1 = stashed ? h1_in : h1w;
  const float* h3 = stashed ? h3_in : h3w;
  const int n1 = two ? d_ff : d_out;
  // dh: [max_rows, kt]; for SwiGLU dh1 in columns [0, d_ff), dh3 in [d_ff, 2 d_ff)
  const int kt = kind == MOE_FFN_SWIGLU ? 2 * n1 : n1;
  uint16_t* dh1 = two ? reinterpret_cast<uint16_t*>(ws + lay.dh) : nullptr;
  uint16_t* dh3 = kind == MOE_FFN_SWIGLU ? dh1 + n1 : nullptr;
  uint16_t* act = two ? reinterpret_cast<uint16_t*>(ws + lay.a) : nullptr;
  uint16_t* wt = lay.wt_bytes ? reinterpret_cast<uint16_t*>(ws + lay.wt) : nullptr;   // (the fallback's)
  const int shared = row_mode == MOE_ROWS_SHARED ? 1 : 0;
  const uint16_t* X = static_cast<const uint16_t*>(x_rows);
  const uint16_t* DY = static_cast<const uint16_t*>(dy_rows);

  int st = launch_tile_map(offsets, E, kBwdBM, ts128, stream);
  if (st != MOE_OK) return st;
  const int mt128 = (max_rows + kBwdBM - 1) / kBwdBM + E;

  // 1. recompute the first layer's pre-activations h1 (+ bias) and h3 in
  //    fp32 (forward layout, no activation): on the forward's LDS-DMA kernel
  //    with its fp32 pre-activation epilogue (one launch for gate and up),
  //    else on the backward kernel
  int32_t* ts256 = reinterpret_cast<int32_t*>(ws + lay.ts256);
  st = launch_tile_map(offsets, E, kGemmBM, ts256, stream);
  if (st != MOE_OK) return st;
  const int mt256 = (max_rows + kGemmBM - 1) / kGemmBM + E;
  bool pre_done = stashed;
  if (two && !stashed) {
    GemmParams f{};
    f.A = X;
    f.a_shared = shared;
    f.offsets = offsets;
    f.ts = ts256;
    f.E = E;
    f.B1 = w1;
    f.B3 = w3;
    f.bias = b1;
    f.N = d_ff;
    f.K = d;
    f.n_cu = current_cu_count();
    f.split_max = 1;
    f.pre1 = h1w;
    f.pre3 = h3w;
    st = launch_grouped_gemm_pre(kind == MOE_FFN_SWIGLU ? EPI_SWIGLU : EPI_PLAIN, f, mt256, stream);
    if (st == MOE_OK) pre_done = true;
    else if (st != MOE_ERR_UNSUPPORTED) return st;
  }
  if (two && !pre_done) {
    BwdGemmParams g{};
    g.A = X;
    g.lda = d;
    g.a_shared = shared;
    g.B = static_cast<const uint16_t*>(w1);
    g.ldb = d;
    g.b_estride = static_cast<long>(d_ff) * d;
    g.N = d_ff;
    g.K = d;
    g.K1 = d;
    g.offsets = offsets;
    g.ts = ts128;
    g.E = E;
    g.Cf = h1w;
    g.ldc = d_ff;
    g.bias = b1;
    st = launch_bwd_gemm(BWD_FWD, BWD_EPI_STORE, g, mt128, stream);
    if (st != MOE_OK) return st;
    if (h3) {
      g.B = static_cast<const uint16_t*>(w3);
      g.bias = nullptr;
      g.Cf = h3w;
      st = launch_bwd_gemm(BWD_FWD, BWD_EPI_STORE, g, mt128, stream);
      if (st != MOE_OK) return st;
    }
  }
  if (two) {
    // 2. da = dY W2 (K = d_out), with the activation's backward in the
    //    epilogue: dh1 (dh3) and the activation a.  On the forward's LDS-DMA
    //    kernel reading W2's rows as stored through transposing LDS reads;
    //    else over W2 transposed to [E, d_ff, d_out]; else on the backward
    //    kernel
    const int epi = kind == MOE_FFN_SWIGLU ? BWD_EPI_SWIGLU : kind == MOE_FFN_RELU ? BWD_EPI_RELU : BWD_EPI_GELU;
    GemmParams a{};
    a.A = DY;
    a.a_shared = shared;
    a.offsets = offsets;
    a.ts = ts256;
    a.E = E;
    a.B1 = wt;
    a.N = d_ff;
    a.K = d_out;
    a.n_cu = current_cu_count();
    a.split_max = 1;
    a.hin1 = h1;
    a.hin3 = h3;
    a.o1 = dh1;
    a.o2 = dh3;
    a.o3 = act;
    a.ldo = kt;
    a.B1 = w2;
    a.tb_k1 = d_out;
    st = launch_grouped_gemm_actbwd_tb(epi, a, mt256, stream);
    if (st == MOE_ERR_UNSUPPORTED && wt) {
      const dim3 tg((d_ff + 63) / 64, (d_out + 63) / 64, E);
      hipLaunchKernelGGL(transpose_w_kernel, tg, dim3(256), 0, stream, static_cast<const uint16_t*>(w2),
                         static_cast<const uint16_t*>(nullptr), d_out, d_out, d_ff, wt);
      st = check_launch();
      if (st != MOE_OK) return st;
      a.B1 = wt;
      st = launch_grouped_gemm_actbwd(epi, a, mt256, stream);
    }
    if (st != MOE_ERR_UNSUPPORTED && st != MOE_OK) return st;
  }
  if (two && st == MOE_ERR_UNSUPPORTED) {
    BwdGemmParams b{};
    b.A = DY;
    b.lda = d_out;
    b.a_shared = shared;
    b.B = static_cast<const uint16_t*>(w2);
    b.ldb = d_ff;
    b.b_estride = static_cast<long>(d_out) * d_ff;
    b.N = d_ff;
    b.K = d_out;
    b.K1 = d_out;
    b.offsets = offsets;
    b.ts = ts128;
    b.E = E;
    b.ldc = d_ff;
    b.ldo = kt;
    b.H1 = h1;
    b.H3 = h3;
    b.O1 = dh1;
    b.O2 = dh3;
    b.O3 = act;
    const int epi = kind == MOE_FFN_SWIGLU ? BWD_EPI_SWIGLU : kind == MOE_FFN_RELU ? BWD_EPI_RELU : BWD_EPI_GELU;
    st = launch_bwd_gemm(BWD_DGRAD, epi, b, mt128, stream);
    if (st != MOE_OK) return st;
  }
  // 3. dX = dh W13 over K = kt (dh1 W1 + dh3 W3 for SwiGLU; linear: dY W1):
  //    the forward's grouped GEMM reading the first layer's weights as stored
  //    (K rows: W1's, then W3's) through transposing LDS reads; else over the
  //    weights transposed to [E, d, kt] (both operands K-contiguous)
  {
    GemmParams g{};
    g.A = two ? dh1 : DY;
    g.a_shared = two ? 0 : shared;
    g.offsets = offsets;
    g.ts = ts256;
    g.E = E;
    g.C = static_cast<uint16_t*>(dx_rows);
    g.N = d;
    g.K = kt;
    g.partial = reinterpret_cast<float*>(ws + lay.partial);
    g.n_cu = current_cu_count();
    g.split_max = kGemmSplitMax;
    g.B1 = w1;
    g.B3 = w3;
    g.tb_k1 = n1;
    st = launch_grouped_gemm_tb(g, mt256, stream);
    if (st == MOE_ERR_UNSUPPORTED && wt) {
      const dim3 tg((d + 63) / 64, (kt + 63) / 64, E);
      hipLaunchKernelGGL(transpose_w_kernel, tg, dim3(256), 0, stream, static_cast<const uint16_t*>(w1),
                         static_cast<const uint16_t*>(w3), n1, kt, d, wt);
      st = check_launch();
      if (st != MOE_OK) return st;
      g.B1 = wt;
      g.B3 = nullptr;
      st = launch_grouped_gemm(EPI_PLAIN, false, g, max_rows, mt256, stream);
    }
    if (st != MOE_OK) return st;
  }
  // 4. weight gradients, K = the segment's rows: dW2 = dY^T a; dW1 = dh1^T X
  //    (linear: dY^T X); dW3 = dh3^T X.  On the forward's LDS-DMA GEMM over
  //    the activations transposed per segment (each segment padded to 128
  //    rows with zeros; segments of the transposed buffers start at 128 ts128[e]),
  //    else on the backward kernel (transposing in registers)
  const long kp = static_cast<long>(lay.kp);
  auto dma_fits = [&](int N) {
    return static_cast<size_t>(kGemmBM) * kp * 2 < (size_t(1) << 31) &&
           static_cast<size_t>(N) * kp * 2 < (size_t(1) << 31) && N % 8 == 0;
  };
  const bool wg_dma = dma_fits(d) && (!two || dma_fits(d_ff));
  if (wg_dma) {
    uint16_t* XT = reinterpret_cast<uint16_t*>(ws + lay.xt);
    uint16_t* DYT = reinterpret_cast<uint16_t*>(ws + lay.dyt);
    auto transpose = [&](const uint16_t* in, long ldin, int F, int sh, uint16_t* out) {
      const dim3 g((F + 63) / 64, static_cast<unsigned>((kp + 63) / 64));
      hipLaunchKernelGGL(transpose_seg_kernel, g, dim3(256), 0, stream, in, ldin, F, offsets, ts128, E, sh, out, kp);
      return check_launch();
    };
    auto wgrad_dma = [&](const uint16_t* A_, const uint16_t* B_, int M, int N, int32_t* wofs, int32_t* tsw,
                         float* out) {
      hipLaunchKernelGGL(iota_kernel, dim3(1), dim3(256), 0, stream, wofs, E, M);
      int r = check_launch();
      if (r != MOE_OK) return r;
      r = launch_tile_map(wofs, E, kGemmBM, tsw, stream);
      if (r != MOE_OK) return r;
      GemmParams g{};
      g.A = A_;
      g.a_shared = 1;
      g.offsets = wofs;
      g.ts = tsw;
      g.E = E;
      g.B1 = B_;
      g.N = N;
      g.pre1 = out;
      g.kseg = ts128;
      g.lda = kp;
      g.ldb = kp;
      g.n_cu = current_cu_count();
      return launch_grouped_gemm_wgrad(g, static_cast<int>((static_cast<long>(E) * M + kGemmBM - 1) / kGemmBM) + E,
                                       stream);
    };
    int32_t* wofs_o = reinterpret_cast<int32_t*>(ws + lay.wofs_o);
    int32_t* wofs_1 = reinterpret_cast<int32_t*>(ws + lay.wofs_1);
    int32_t* tsw_o = reinterpret_cast<int32_t*>(ws + lay.tsw_o);
    int32_t* tsw_1 = reinterpret_cast<int32_t*>(ws + lay.tsw_1);
    st = transpose(X, d, d, shared, XT);
    if (st == MOE_OK) st = transpose(DY, d_out, d_out, shared, DYT);
    if (st != MOE_OK) return st;
    if (two) {
      uint16_t* AT = reinterpret_cast<uint16_t*>(ws + lay.at);
      uint16_t* DHT = reinterpret_cast<uint16_t*>(ws + lay.dht);
      st = transpose(act, d_ff, d_ff, 0, AT);
      if (st == MOE_OK) st = transpose(dh1, kt, kt, 0, DHT);
      if (st == MOE_OK) st = wgrad_dma(DYT, AT, d_out, d_ff, wofs_o, tsw_o, dw2);
      if (st == MOE_OK) st = wgrad_dma(DHT, XT, n1, d, wofs_1, tsw_1, dw1);
      if (st == MOE_OK && dh3) st = wgrad_dma(DHT + static_cast<size_t>(n1) * kp, XT, n1, d, wofs_1, tsw_1, dw3);
    } else {
      st = wgrad_dma(DYT, XT, n1, d, wofs_1, tsw_1, dw1);
    }
    if (st != MOE_OK) return st;
  } else {
  auto wgrad = [&](const uint16_t* A, long lda, int a_sh, const uint16_t* B, long ldb, int b_sh, int M, int N,
                   float* out) {
    BwdGemmParams b{};
    b.A = A;
    b.lda = lda;
    b.a_shared = a_sh;
    b.B = B;
    b.ldb = ldb;
    b.b_estride = 0;
    b.b_shared = b_sh;
    b.M = M;
    b.N = N;
    b.offsets = offsets;
    b.E = E;
    b.Cf = out;
    b.ldc = N;
    b.c_estride = static_cast<long>(M) * N;
    return launch_bwd_gemm(BWD_WGRAD, BWD_EPI_STORE, b, 0, stream);
  };
  if (two) {
    st = wgrad(DY, d_out, shared, act, d_ff, 0, d_out, d_ff, dw2);
    if (st != MOE_OK) return st;
  }
  st = wgrad(two ? dh1 : DY, two ? kt : n1, two ? 0 : shared, X, d, shared, n1, d, dw1);
  if (st != MOE_OK) return st;
  if (dh3) {
    st = wgrad(dh3, kt, 0, X, d, shared, d_ff, d, dw3);
    if (st != MOE_OK) return st;
  }
  }
  // 5. bias gradients: sums over each segment's rows
  if (db1) {
    hipLaunchKernelGGL(segment_colsum_kernel, dim3((n1 + kBwThreads - 1) / kBwThreads, E), dim3(kBwThreads), 0, stream,
                       two ? dh1 : DY, static_cast<long>(n1), n1, offsets, two ? 0 : shared, db1);
    st = check_launch();
    if (st != MOE_OK) return st;
  }
  if (db2) {
    hipLaunchKernelGGL(segment_colsum_kernel, dim3((d_out + kBwThreads - 1) / kBwThreads, E), dim3(kBwThreads), 0,
                       stream, DY, static_cast<long>(d_out), d_out, offsets, shared, db2);
    st = check_launch();
  }
  return st;
}

}  // namespace
}  // namespace moe

extern "C" {

size_t moe_ffn_backward_workspace_size(int kind, int max_rows, int E, int d, int d_ff, int d_out) {
  if (max_rows < 0 || E < 1 || d < 1 || d_out < 1) return 0;
  return ffn_bwd_layout(kind, max_rows, E, d, d_ff, d_out).total;
}

size_t moe_ffn_backward_kept_workspace_size(int kind, int max_rows, int E, int d, int d_ff, int d_out) {
  if (max_rows < 0 || E < 1 || d < 1 || d_out < 1) return 0;
  return ffn_bwd_layout(kind, max_rows, E, d, d_ff, d_out, true).total;
}

int moe_expert_ffn_grouped_backward(int kind, const void* x_rows, int act_dt, int max_rows, int row_mode,
                                    const int32_t* offsets, int E, int d, int d_ff, int d_out, const void* w1,
                                    const void* w3, const void* w2, int w_dt, const float* b1, const float* b2,
                                    const void* dy_rows, void* dx_rows, float* dw1, float* dw3, float* dw2, float* db1,
                                    float* db2, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return ffn_backward_run(kind, x_rows, act_dt, max_rows, row_mode, offsets, E, d, d_ff, d_out, w1, w3, w2, w_dt, b1,
                          b2, dy_rows, dx_rows, dw1, dw3, dw2, db1, db2, nullptr, nullptr, workspace, workspace_bytes,
                          stream);
}

int moe_expert_ffn_grouped_backward_kept(int kind, const void* x_rows, int act_dt, int max_rows, int row_mode,
                                         const int32_t* offsets, int E, int d, int d_ff, int d_out, const void* w1,
                                         const void* w3, const void* w2, int w_dt, const float* b1, const float* b2,
                                         const float* h1, const float* h3, const void* dy_rows, void* dx_rows,
                                         float* dw1, float* dw3, float* dw2, float* db1, float* db2, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  if (max_rows > 0 && !h1) return MOE_ERR_INVALID_ARG;
  if (kind == MOE_FFN_LINEAR) return MOE_ERR_INVALID_ARG;
  if (max_rows == 0) {
    // nothing was kept; the gradients are zero as for the recomputing call
    return ffn_backward_run(kind, x_rows, act_dt, 0, row_mode, offsets, E, d, d_ff, d_out, w1, w3, w2, w_dt, b1, b2,
                            dy_rows, dx_rows, dw1, dw3, dw2, db1, db2, nullptr, nullptr, workspace, workspace_bytes,
                            stream);
  }
  return ffn_backward_run(kind, x_rows, act_dt, max_rows, row_mode, offsets, E, d, d_ff, d_out, w1, w3, w2, w_dt, b1,
                          b2, dy_rows, dx_rows, dw1, dw3, dw2, db1, db2, h1, h3, workspace, workspace_bytes, stream);
}

}  // extern "C"
