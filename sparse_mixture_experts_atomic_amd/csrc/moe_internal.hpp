// Internal helpers shared by the libmoe translation units: status handling
// on the host, bf16/fp8 conversions and small vector types on the device.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------- host side

void record_hip_error(hipError_t e);

// Checks the launch that was just enqueued; records the HIP error if any.
inline int check_launch() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    record_hip_error(e);
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr size_t kWsAlign = 256;

inline int dtype_bytes(int dt) {
  switch (dt) {
    case MOE_F32: return 4;
    case MOE_BF16: return 2;
    case MOE_FP8_E4M3: return 1;
    default: return 0;
  }
}

// -------------------------------------------------------------- device side

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats to bf16, round to nearest even, packed (lo in bits 0-15): one
// v_cvt_pk_bf16_f32 on gfx950.  Its results equal the bit-level rounding
// (u + 0x7fff + lsb) >> 16 for every finite value, denormals included, and
// a NaN stays a NaN (quiet, top payload bits kept).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

__device__ __forceinline__ float silu_f32(float u) { return u / (1.0f + expf(-u)); }

// ------------------------------------------------- grouped GEMM interface

enum { EPI_PLAIN = 0, EPI_RELU = 1, EPI_SWIGLU = 2, EPI_GELU = 3 };

// GELU in its exact form, u * Phi(u) = u / 2 * (1 + erf(u / sqrt 2)), with
// erfc(x), x >= 0, from Abramowitz and Stegun, Handbook of Mathematical
// Functions, formula 7.1.26: t = 1 / (1 + p x), erfc(x) = (a1 t + a2 t^2 +
// a3 t^3 + a4 t^4 + a5 t^5) e^(-x^2), absolute error below 1.5e-7 (well under
// the bf16 rounding of the result, and under fp32 tolerances).  Branch-free:
// one reciprocal, one exp2 and five FMAs, where the library erf branches per
// element and, unrolled over an epilogue's 128 values per lane, spills.
__device__ __forceinline__ float gelu_f32(float u) {
  const float x = fabsf(u) * 0.70710678118654752f;              // |u| / sqrt 2
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float q = fmaf(t, 1.061405429f, -1.453152027f);
  q = fmaf(t, q, 1.421413741f);
  q = fmaf(t, q, -0.284496736f);
  q = fmaf(t, q, 0.254829592f);
  const float y = q * t * __builtin_amdgcn_exp2f(-1.4426950408889634f * x * x);   // erfc(x)
  return 0.5f * u * (u >= 0.f ? 2.0f - y : y);
}

// activation of a non-gated first layer (identity for EPI_PLAIN)
template <int EPI>
__device__ __forceinline__ float act1(float v) {
  if constexpr (EPI == EPI_RELU) return fmaxf(v, 0.f);
  if constexpr (EPI == EPI_GELU) return gelu_f32(v);
  return v;
}

constexpr int kGemmBM = 256;   // rows per m-tile of the grouped GEMM

struct GemmParams {
  const uint16_t* A;         // bf16 rows [*, K]
  int a_shared;              // 1: segment e reads A rows from 0 (shared experts)
  const int32_t* gather;     // packed row -> row of A (null: row itself); not with a_shared
  int a_rows;                // rows of A when gathering (bounds the DMA offsets)
  const int32_t* offsets;    // [E+1] segment bounds
  const int32_t* ts;         // [E+1] m-tile prefix (tiles of kGemmBM rows)
  int E;
  const void* B1;            // [E, N, K] bf16 or e4m3 codes
  const void* B3;            // SwiGLU up projection [E, N, K]
  const float* s1;           // [E, N] e4m3 row scales (or null)
  const float* s3;
  const float* bias;         // [E, N] (or null)
  uint16_t* C;               // bf16 [*, N]
  int N;                     // output columns
  int K;
  float* partial;            // split-tail partial sums: n_cu x 256 x 256 fp32 (or null)
  int n_cu;                  // compute units (one block of the DMA kernel each)
  int split_max;             // most K parts of a split tile (1: no split)
};

// Bytes of the split-tail partial buffer for n_cu compute units.
inline size_t gemm_partial_bytes(int n_cu) { return static_cast<size_t>(n_cu > 0 ? n_cu : 0) * 256 * 256 * sizeof(float); }
constexpr int kGemmSplitMax = 4;

// Enqueues C = epi(A B^T) per segment.  m_tiles_max bounds ts[E] from above.
int launch_grouped_gemm(int epi, bool fp8, const GemmParams& p, int max_rows, int m_tiles_max, hipStream_t stream);

}  // namespace moe
