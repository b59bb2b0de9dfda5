// (d) Combine: y[t] = sum_j g[t,j] * Ye[dest[t,j]] (kept slots) + shared
// experts (+ residual), and the Switch load-balancing aux loss.
//
// P1 §3.4 / §4.3: weighted expert outputs accumulated into a zero output;
// P3 §3.1: the same weighted sum over the k slots; P5 专家容量: a dropped
// token's expert output is 0.  Aux: P5 负载均衡损失函数, P1 §3.4.
//
// Each output element is produced by one thread with fp32 accumulation in a
// fixed order (slots, then shared experts, then residual): no atomics, so
// the result does not depend on scheduling.
#include "moe_internal.hpp"

namespace moe {
namespace {

template <typename T, int VW> struct Vec;
template <> struct Vec<uint16_t, 8> {
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
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct Vec<float, 4> {
  using type = float4;
  __device__ __forceinline__ static void unpack(const float4& v, float* f) { f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; }
  __device__ __forceinline__ static float4 pack(const float* f) { return make_float4(f[0], f[1], f[2], f[3]); }
};
template <typename T> struct Vec<T, 1> {
  using type = T;
  __device__ __forceinline__ static void unpack(const T& v, float* f) { f[0] = Elem<T>::load(&v, 0); }
  __device__ __forceinline__ static T pack(const float* f) { T r; Elem<T>::store(&r, 0, f[0]); return r; }
};

// One thread = one 16-byte output vector of one token (grid y = token,
// strided past the grid-y limit).  The gate-weighted
// rows of the (up to 8 unrolled) slots are loaded together, so a wavefront has
// k row loads in flight; slot indices and gates are uniform across the
// wavefront's 64 vectors of the same token.
constexpr int kCbUnroll = 8;

template <typename T, int VW>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y_rows, const int32_t* __restrict__ dest_pos,
                                                     const float* __restrict__ gate, int T_, int k, int nvec,
                                                     const T* __restrict__ shared_y, int n_shared,
                                                     const T* __restrict__ residual, T* __restrict__ y) {
  using V = typename Vec<T, VW>::type;
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= nvec) return;
  const V* yr = reinterpret_cast<const V*>(y_rows);
  for (int t = blockIdx.y; t < T_; t += gridDim.y) {
    const int32_t* dp = dest_pos + static_cast<size_t>(t) * k;
    const float* gp = gate + static_cast<size_t>(t) * k;
    float acc[VW];
#pragma unroll
    for (int i = 0; i < VW; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += kCbUnroll) {
      V rv[kCbUnroll];
      int d[kCbUnroll];
#pragma unroll
      for (int u = 0; u < kCbUnroll; ++u) {
        d[u] = j0 + u < k ? dp[j0 + u] : -1;
        if (d[u] >= 0) rv[u] = yr[static_cast<size_t>(d[u]) * nvec + v];
      }
#pragma unroll
      for (int u = 0; u < kCbUnroll; ++u) {
        if (d[u] < 0) continue;
        const float g = gp[j0 + u];
        float f[VW];
        Vec<T, VW>::unpack(rv[u], f);
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[i] = fmaf(g, f[i], acc[i]);
      }
    }
    const V* sy = reinterpret_cast<const V*>(shared_y);
    for (int s = 0; s < n_shared; ++s) {
      float f[VW];
      Vec<T, VW>::unpack(sy[(static_cast<size_t>(s) * T_ + t) * nvec + v], f);
#pragma unroll
      for (int i = 0; i < VW; ++i) acc[i] += f[i];
    }
    if (residual) {
      float f[VW];
      Vec<T, VW>::unpack(reinterpret_cast<const V*>(residual)[static_cast<size_t>(t) * nvec + v], f);
#pragma unroll
      for (int i = 0; i < VW; ++i) acc[i] += f[i];
    }
    reinterpret_cast<V*>(y)[static_cast<size_t>(t) * nvec + v] = Vec<T, VW>::pack(acc);
  }
}

// k known at compile time (1 to 8): one thread per 16-byte output vector of
// one token (grid y = token, strided past the grid-y limit); the K slot rows are loaded together,
// then accumulated in slot order (dropped slots skipped), then the shared
// experts and the residual, as in combine_kernel.
template <typename T, int VW, int K>
__global__ __launch_bounds__(256) void combine_kk_kernel(const T* __restrict__ y_rows, const int32_t* __restrict__ dest_pos,
                                                        const float* __restrict__ gate, int T_, int nvec,
                                                        const T* __restrict__ shared_y, int n_shared,
                                                        const T* __restrict__ residual, T* __restrict__ y) {
  using V = typename Vec<T, VW>::type;
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= nvec) return;
  const V* yr = reinterpret_cast<const V*>(y_rows);
  for (int t = blockIdx.y; t < T_; t += gridDim.y) {
    int d[K];
    V rv[K];
#pragma unroll
    for (int u = 0; u < K; ++u) {
      d[u] = dest_pos[static_cast<size_t>(t) * K + u];
      if (d[u] >= 0) rv[u] = yr[static_cast<size_t>(d[u]) * nvec + v];
    }
    float acc[VW];
#pragma unroll
    for (int c = 0; c < VW; ++c) acc[c] = 0.f;
#pragma unroll
    for (int u = 0; u < K; ++u) {
      if (d[u] < 0) continue;
      const float g = gate[static_cast<size_t>(t) * K + u];
      float f[VW];
      Vec<T, VW>::unpack(rv[u], f);
#pragma unroll
      for (int c = 0; c < VW; ++c) acc[c] = fmaf(g, f[c], acc[c]);
    }
    const V* sy = reinterpret_cast<const V*>(shared_y);
    for (int sI = 0; sI < n_shared; ++sI) {
      float f[VW];
      Vec<T, VW>::unpack(sy[(static_cast<size_t>(sI) * T_ + t) * nvec + v], f);
#pragma unroll
      for (int c = 0; c < VW; ++c) acc[c] += f[c];
    }
    if (residual) {
      float f[VW];
      Vec<T, VW>::unpack(reinterpret_cast<const V*>(residual)[static_cast<size_t>(t) * nvec + v], f);
#pragma unroll
      for (int c = 0; c < VW; ++c) acc[c] += f[c];
    }
    reinterpret_cast<V*>(y)[static_cast<size_t>(t) * nvec + v] = Vec<T, VW>::pack(acc);
  }
}

// grid y: one token per row of blocks up to the device's grid-y limit;
// beyond it each row of blocks takes every gridDim.y-th token
constexpr int kCbMaxGridY = 65535;

template <typename T, int VW>
int launch_combine(const void* y_rows, const int32_t* dest_pos, const float* gate, int T_, int k, int d_out,
                   const void* shared_y, int n_shared, const void* residual, void* y, hipStream_t stream) {
  const int nvec = d_out / VW;
  const dim3 grid((nvec + 255) / 256, T_ < kCbMaxGridY ? T_ : kCbMaxGridY);   // (vector blocks of a row, tokens)
#define MOE_CB_K(KK)                                                                                          \
  hipLaunchKernelGGL((combine_kk_kernel<T, VW, KK>), grid, dim3(256), 0, stream, static_cast<const T*>(y_rows), \
                     dest_pos, gate, T_, nvec, static_cast<const T*>(shared_y), n_shared,                      \
                     static_cast<const T*>(residual), static_cast<T*>(y));                                    \
  return check_launch()
  switch (k) {
    case 1: MOE_CB_K(1);
    case 2: MOE_CB_K(2);
    case 3: MOE_CB_K(3);
    case 4: MOE_CB_K(4);
    case 5: MOE_CB_K(5);
    case 6: MOE_CB_K(6);
    case 7: MOE_CB_K(7);
    case 8: MOE_CB_K(8);
    default: break;
  }
#undef MOE_CB_K
  hipLaunchKernelGGL((combine_kernel<T, VW>), grid, dim3(256), 0, stream,
                     static_cast<const T*>(y_rows), dest_pos, gate, T_, k, nvec, static_cast<const T*>(shared_y),
                     n_shared, static_cast<const T*>(residual), static_cast<T*>(y));
  return check_launch();
}

// loss = alpha * E * sum_e (counts[e] / (T k)) * (colsum[e] / T); one block,
// fixed-order tree reduction.
__global__ __launch_bounds__(256) void aux_loss_kernel(const int32_t* __restrict__ counts,
                                                      const float* __restrict__ colsum, int T_, int k, int E,
                                                      float alpha, float* __restrict__ loss) {
  __shared__ float red[256];
  float s = 0.f;
  if (T_ > 0) {
    const float inv_tk = 1.0f / (static_cast<float>(T_) * static_cast<float>(k));
    const float inv_t = 1.0f / static_cast<float>(T_);
    for (int e = threadIdx.x; e < E; e += 256)
      s += (static_cast<float>(counts[e]) * inv_tk) * (colsum[e] * inv_t);
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = alpha * static_cast<float>(E) * red[0];
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_combine(const void* y_rows, int dt, const int32_t* dest_pos, const float* topk_gate, int T, int k,
                int d_out, const void* shared_y, int n_shared, const void* residual, void* y, hipStream_t stream) {
  if (T < 0 || k < 1 || d_out < 1 || n_shared < 0) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!y_rows || !dest_pos || !topk_gate || !y) return MOE_ERR_INVALID_ARG;
  if (n_shared > 0 && !shared_y) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {y_rows, dest_pos, topk_gate, y, shared_y, residual};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  if (dt == MOE_BF16) {
    if (d_out % 8 == 0)
      return launch_combine<uint16_t, 8>(y_rows, dest_pos, topk_gate, T, k, d_out, shared_y, n_shared, residual, y, stream);
    return launch_combine<uint16_t, 1>(y_rows, dest_pos, topk_gate, T, k, d_out, shared_y, n_shared, residual, y, stream);
  }
  if (d_out % 4 == 0)
    return launch_combine<float, 4>(y_rows, dest_pos, topk_gate, T, k, d_out, shared_y, n_shared, residual, y, stream);
  return launch_combine<float, 1>(y_rows, dest_pos, topk_gate, T, k, d_out, shared_y, n_shared, residual, y, stream);
}

int moe_aux_loss(const int32_t* counts_routed, const float* prob_colsum, int T, int k, int E, float alpha,
                 float* loss, hipStream_t stream) {
  if (T < 0 || k < 1 || E < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (!counts_routed || !prob_colsum || !loss) return MOE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(aux_loss_kernel, dim3(1), dim3(256), 0, stream, counts_routed, prob_colsum, T, k, E, alpha, loss);
  return check_launch();
}

}  // extern "C"
