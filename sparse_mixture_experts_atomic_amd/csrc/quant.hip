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

template <typename XT> struct Row8;
template <> struct Row8<uint16_t> {
  __device__ __forceinline__ static void load(const uint16_t* p, float* f) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Row8<float> {
  __device__ __forceinline__ static void load(const float* p, float* f) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

// one block per row (grid-strided); 8 values per thread and step
template <typename XT>
__global__ __launch_bounds__(kQThreads) void quant_rows_kernel(const XT* __restrict__ x, int rows, int cols,
                                                              const int32_t* __restrict__ rows_dev,
                                                              uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[kQThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
    m = wave_max_abs(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    for (int c = tid; c < n8; c += kQThreads) {
      float f[8];
      Row8<XT>::load(xr + 8 * c, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = fminf(fmaxf(__fdiv_rn(f[i], s), -448.0f), 448.0f);
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
      *reinterpret_cast<uint2*>(q + static_cast<size_t>(r) * cols + 8 * c) =
          make_uint2(static_cast<uint32_t>(lo), static_cast<uint32_t>(hi));
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
  if (x_dt == MOE_BF16)
    hipLaunchKernelGGL(quant_rows_kernel<uint16_t>, dim3(grid), dim3(kQThreads), 0, stream,
                       static_cast<const uint16_t*>(x), rows, cols, rows_dev, q, scale);
  else
    hipLaunchKernelGGL(quant_rows_kernel<float>, dim3(grid), dim3(kQThreads), 0, stream, static_cast<const float*>(x),
                       rows, cols, rows_dev, q, scale);
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
