// Per-row e4m3 quantisation of activations (expert inputs and hidden
// layers) for the fp8 expert path.
//
// P2's deployment paragraph and P3 §4.2 quantise the experts (int8, INT4)
// and keep the router precise; the format here is the stored weights' OCP
// E4M3FN and each row gets one fp32 scale, as each weight row does: s = the
// row's largest magnitude / 448 (1 for an all-zero row), codes = the value
// x / s rounded to the nearest e4m3 value (ties to even), both divisions in
// IEEE fp32.  The rounding is v_cvt_pk_fp8_f32 (round to nearest even); the
// quotient is clamped to +-448 first, which changes no code and keeps a
// quotient a rounding step above 448 off the NaN pattern.
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kQThreads = 256;

__device__ __forceinline__ float wave_max_abs(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xf, 0xf, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// 8 values of a row: raw (as loaded) and widened to fp32
template <typename XT> struct Row8;
template <> struct Row8<uint16_t> {
  typedef uint4 raw_t;
  __device__ __forceinline__ static raw_t fetch(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ static void widen(const raw_t& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void load(const uint16_t* p, float* f) { widen(fetch(p), f); }
};
template <> struct Row8<float> {
  struct raw_t { float4 a, b; };
  __device__ __forceinline__ static raw_t fetch(const float* p) {
    return raw_t{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  __device__ __forceinline__ static void widen(const raw_t& v, float* f) {
    f[0] = v.a.x; f[1] = v.a.y; f[2] = v.a.z; f[3] = v.a.w;
    f[4] = v.b.x; f[5] = v.b.y; f[6] = v.b.z; f[7] = v.b.w;
  }
  __device__ __forceinline__ static void load(const float* p, float* f) { widen(fetch(p), f); }
};

// the e4m3 codes of 8 values divided by s (IEEE), clamped to +-448 first
__device__ __forceinline__ uint2 codes8(const float* f, float s) {
  float g[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) g[i] = fminf(fmaxf(__fdiv_rn(f[i], s), -448.0f), 448.0f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(g[0], g[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(g[2], g[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(g[4], g[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(g[6], g[7], hi, true);
  return make_uint2(static_cast<uint32_t>(lo), static_cast<uint32_t>(hi));
}

// block max |x| of per-thread maxima (DPP within the wavefronts, then LDS)
__device__ __forceinline__ float block_amax(float m, float* red) {
  const int tid = threadIdx.x;
  m = wave_max_abs(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// rows of at most 8 R kQThreads values: the row is read once and held in
// registers (R pieces of 8 per thread) between the max and the codes
template <typename XT, int R>
__global__ __launch_bounds__(kQThreads) void quant_rows_reg_kernel(const XT* __restrict__ x, int rows, int cols,
                                                                  const int32_t* __restrict__ rows_dev,
                                                                  uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[kQThreads / 64];
  const int tid = threadIdx.x;
  const int nrows = rows_dev ? min(rows, *rows_dev) : rows;
  const int n8 = cols / 8;
  for (int r = blockIdx.x; r < nrows; r += gridDim.x) {
    const XT* xr = x + static_cast<size_t>(r) * cols;
    typename Row8<XT>::raw_t v[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int c = tid + kQThreads * i;
      v[i] = Row8<XT>::fetch(xr + 8 * min(c, n8 - 1));
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (tid + kQThreads * i < n8) {
        float f[8];
        Row8<XT>::widen(v[i], f);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
      }
    }
    const float amax = block_amax(m, red);
    const float s = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int c = tid + kQThreads * i;
      if (c < n8) {
        float f[8];
        Row8<XT>::widen(v[i], f);
        *reinterpret_cast<uint2*>(q + static_cast<size_t>(r) * cols + 8 * c) = codes8(f, s);
      }
    }
    if (tid == 0) scale[r] = s;
    __syncthreads();
  }
}

// longer rows: one block per row (grid-strided), read twice (max, then
// codes); 8 values per thread and step
template <typename XT>
__global__ __launch_bounds__(kQThreads) void quant_rows_kernel(const XT* __restrict__ x, int rows, int cols,
                                                              const int32_t* __restrict__ rows_dev,
                                                              uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[kQThreads / 64];
  const int tid = threadIdx.x;
  const int nrows = rows_dev ? min(rows, *rows_dev) : rows;
  const int n8 = cols / 8;
  for (int r = blockIdx.x; r < nrows; r += gridDim.x) {
    const XT* xr = x + static_cast<size_t>(r) * cols;
    float m = 0.f;
    for (int c = tid; c < n8; c += kQThreads) {
      float f[8];
      Row8<XT>::load(xr + 8 * c, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    }
    const float amax = block_amax(m, red);
    const float s = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    for (int c = tid; c < n8; c += kQThreads) {
      float f[8];
      Row8<XT>::load(xr + 8 * c, f);
      *reinterpret_cast<uint2*>(q + static_cast<size_t>(r) * cols + 8 * c) = codes8(f, s);
    }
    if (tid == 0) scale[r] = s;
    __syncthreads();
  }
}

}  // namespace

int launch_quant_rows(const void* x, int x_dt, int rows, int cols, const int32_t* rows_dev, uint8_t* q, float* scale,
                      hipStream_t stream) {
  if (rows <= 0) return MOE_OK;
  const int grid = rows < 65536 ? rows : 65536;
  const int n8 = cols / 8;
  const dim3 g(grid), b(kQThreads);
  if (x_dt == MOE_BF16) {
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    if (n8 <= 2 * kQThreads)
      hipLaunchKernelGGL((quant_rows_reg_kernel<uint16_t, 2>), g, b, 0, stream, xb, rows, cols, rows_dev, q, scale);
    else if (n8 <= 8 * kQThreads)
      hipLaunchKernelGGL((quant_rows_reg_kernel<uint16_t, 8>), g, b, 0, stream, xb, rows, cols, rows_dev, q, scale);
    else
      hipLaunchKernelGGL(quant_rows_kernel<uint16_t>, g, b, 0, stream, xb, rows, cols, rows_dev, q, scale);
  } else {
    const float* xf = static_cast<const float*>(x);
    if (n8 <= 2 * kQThreads)
      hipLaunchKernelGGL((quant_rows_reg_kernel<float, 2>), g, b, 0, stream, xf, rows, cols, rows_dev, q, scale);
    else if (n8 <= 4 * kQThreads)
      hipLaunchKernelGGL((quant_rows_reg_kernel<float, 4>), g, b, 0, stream, xf, rows, cols, rows_dev, q, scale);
    else
      hipLaunchKernelGGL(quant_rows_kernel<float>, g, b, 0, stream, xf, rows, cols, rows_dev, q, scale);
  }
  return check_launch();
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_quantize_rows_e4m3(const void* x, int x_dt, int rows, int cols, uint8_t* q, float* scale,
                           hipStream_t stream) {
  if (rows < 0 || cols < 1) return MOE_ERR_INVALID_ARG;
  if (x_dt != MOE_BF16 && x_dt != MOE_F32) return MOE_ERR_INVALID_ARG;
  if (cols % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scale) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7u) || (reinterpret_cast<uintptr_t>(scale) & 3u))
    return MOE_ERR_INVALID_ARG;
  return launch_quant_rows(x, x_dt, rows, cols, nullptr, q, scale, stream);
}

}  // extern "C"
