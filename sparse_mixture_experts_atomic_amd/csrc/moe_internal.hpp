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

// d/du of u * Phi(u) = Phi(u) + u phi(u); Phi from erfc by Abramowitz and
// Stegun 7.1.26 as in gelu_f32 (absolute error below 1.5e-7)
__device__ __forceinline__ float gelu_grad_f32(float u) {
  const float x = fabsf(u) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float q = fmaf(t, 1.061405429f, -1.453152027f);
  q = fmaf(t, q, 1.421413741f);
  q = fmaf(t, q, -0.284496736f);
  q = fmaf(t, q, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * x * x);   // e^(-u^2/2)
  const float erfc = q * t * e;
  const float Phi = 0.5f * (u >= 0.f ? 2.0f - erfc : erfc);
  return Phi + u * (0.3989422804014327f * e);
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
  // E <= 64 only: the first launch of a call forms the prefix from offsets
  // in each block, and block 0 leaves it here (= ts) for the launches after
  // it (null: ts is already built)
  int32_t* ts_build;
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
  const float* row_scale;    // fp8 activations: scale of each source row of A (or null)
  // launch_grouped_gemm_tb and launch_grouped_gemm_actbwd_tb: B[n][k] is
  // element (k, n) of the K x N matrix of expert e, rows k < tb_k1 in B1
  // ([E, tb_k1, N]) and the rest in B3 ([E, K - tb_k1, N])
  int tb_k1;
  float* pre1;               // pre-activation outputs (fp32 [*, N]; launch_grouped_gemm_pre and _stash):
  float* pre3;               //   gate (+ bias) and, for SwiGLU, up
  // launch_grouped_gemm_wgrad only: segment e takes K columns [128 kseg[e],
  // 128 kseg[e+1]) of A (rows from 0, pitch lda) and of B (shared by all
  // segments, pitch ldb); fp32 output to pre1
  const int32_t* kseg;
  long lda, ldb;
  // launch_grouped_gemm_actbwd only: the activation's backward in the
  // epilogue, from the fp32 pre-activations hin1 (hin3) [*, N]: o1 = dh1,
  // o2 = dh3 (row pitch ldo), o3 = the activation a (pitch N), bf16
  const float* hin1;
  const float* hin3;
  uint16_t* o1;
  uint16_t* o2;
  uint16_t* o3;
  long ldo;
};

// Most segments for which a grouped GEMM launch forms the m-tile prefix itself
// (one lane per segment) instead of a separate tile-map launch before it.
constexpr int kGemmTsBuildMaxE = 64;

// Bytes of the split-tail partial buffer for n_cu compute units.
inline size_t gemm_partial_bytes(int n_cu) { return static_cast<size_t>(n_cu > 0 ? n_cu : 0) * 256 * 256 * sizeof(float); }
constexpr int kGemmSplitMax = 4;

// Enqueues C = epi(A B^T) per segment.  m_tiles_max bounds ts[E] from above.
int launch_grouped_gemm(int epi, bool fp8, const GemmParams& p, int max_rows, int m_tiles_max, hipStream_t stream);

// Both operands e4m3 (A: codes, one byte per value, rows scaled by
// p.row_scale of their source row; B: codes with per-row scales p.s1/p.s3):
// C = epi(diag(row scales) A B^T diag(column scales)) per segment, bf16 out.
// K % 128 == 0, N % 8 == 0.
int launch_grouped_gemm_f8(int epi, const GemmParams& p, int m_tiles_max, hipStream_t stream);
// The first layer's pre-activations in fp32 (acc + bias to pre1; SwiGLU: gate
// to pre1, up to pre3) on the LDS-DMA kernel; bf16 weights, K % 128 == 0, no
// split tail.  MOE_ERR_UNSUPPORTED for shapes it does not take.
int launch_grouped_gemm_pre(int epi, const GemmParams& p, int m_tiles_max, hipStream_t stream);
// Weight gradients as grouped GEMMs on the LDS-DMA kernel: per segment e,
// pre1[e][M][N] (fp32; segments of M rows from p.offsets = e M) = A[:, K_e]
// B[:, K_e]^T over K_e = columns [128 kseg[e], 128 kseg[e+1]), both operands
// K-contiguous (activations transposed per segment, each zero-padded to a
// multiple of 128 columns).
// MOE_ERR_UNSUPPORTED for shapes it does not take.
int launch_grouped_gemm_wgrad(const GemmParams& p, int m_tiles_max, hipStream_t stream);
// da = dY W2 with the activation's backward in the epilogue (bwd_epi: one of
// BWD_EPI_SWIGLU, _RELU, _GELU) on the LDS-DMA kernel, B = W2 transposed to
// [E, d_ff, d_out]; MOE_ERR_UNSUPPORTED for shapes it does not take.
// The first product of a training forward: the activation to C as
// launch_grouped_gemm writes it, and the fp32 pre-activations (+ bias) to
// pre1 (SwiGLU: gate to pre1, up to pre3), [rows, N] each; MOE_ERR_UNSUPPORTED
// for shapes the LDS-DMA kernel does not take.
int launch_grouped_gemm_stash(int epi, const GemmParams& p, int m_tiles_max, hipStream_t stream);
int launch_grouped_gemm_actbwd(int bwd_epi, const GemmParams& p, int m_tiles_max, hipStream_t stream);
// The plain and the activation-backward products with B read from rows of
// K (the weights as stored, used transposed; see tb_k1); MOE_ERR_UNSUPPORTED
// for shapes the LDS-DMA kernel does not take.
int launch_grouped_gemm_tb(const GemmParams& p, int m_tiles_max, hipStream_t stream);
// Whether the transposed-B launches take a K x N product whose first k1 K
// rows come from B1 (the shape part of their checks)
inline bool grouped_gemm_tb_shape_ok(int K, int N, int k1) {
  return K > 0 && K % 128 == 0 && N >= 8 && N % 8 == 0 && k1 > 0 && k1 % 64 == 0 && k1 <= K &&
         static_cast<size_t>(256) * K * 2 < (size_t(1) << 31) && static_cast<size_t>(64) * N * 2 < (size_t(1) << 31);
}
int launch_grouped_gemm_actbwd_tb(int bwd_epi, const GemmParams& p, int m_tiles_max, hipStream_t stream);

// Per-row e4m3 quantisation (quant.hip): scale[r] = max |x[r, :]| / 448 (1
// for a zero row), q = e4m3(x / scale); rows_dev (device, or null) bounds the
// rows; cols % 8 == 0.
int launch_quant_rows(const void* x, int x_dt, int rows, int cols, const int32_t* rows_dev, uint8_t* q, float* scale,
                      hipStream_t stream);

// ts[e] = sum over e' < e of ceil(segment length / bm), ts[E] the total (one
// block, E <= 1024)
int launch_tile_map(const int32_t* offsets, int E, int bm, int32_t* ts, hipStream_t stream);

// compute units of the current device (0 if it cannot be queried)
int current_cu_count();

// ------------------------------------------- backward grouped GEMMs

enum { BWD_EPI_STORE = 0, BWD_EPI_SWIGLU = 1, BWD_EPI_RELU = 2, BWD_EPI_GELU = 3 };
enum { BWD_DGRAD = 0, BWD_WGRAD = 1, BWD_FWD = 2 };

// One grouped GEMM of the FFN backward (bwd_gemm.hip).  C(m, n) = sum_k
// A(m, k) B(n, k) with
//   dgrad (segments on M, rows of the packed batch; tile map ts of 128-row
//          tiles): A(m, k) = A[m * lda + k] (k < K1) or A2[m * lda + k - K1],
//          B(n, k) = B_e[k * ldb + n] (k < K1) or B2_e[(k - K1) * ldb + n],
//          B_e = B + e * b_estride; epilogue per BWD_EPI_* into O1/O2/O3
//          (bf16 [rows, N], row pitch ldc), reading H1/H3 at the same place;
//   wgrad (segments on K, one M x N output per expert): A(m, k) =
//          A[k * lda + m], B(n, k) = B[k * ldb + n], k over the segment's
//          rows; fp32 output Cf + e * c_estride, row pitch ldc;
//   fwd    (segments on M, forward layout): A(m, k) = A[m * lda + k],
//          B(n, k) = B_e[n * ldb + k]; fp32 output Cf (+ bias[e, n]).
// a_shared / b_shared: the operand's segment e starts at row 0 (shared
// experts: every segment is the same token batch).
struct BwdGemmParams {
  const uint16_t* A;
  const uint16_t* A2;
  long lda;
  int a_shared;
  const uint16_t* B;
  const uint16_t* B2;
  long ldb;
  long b_estride;
  int b_shared;
  int M, N, K, K1;
  const int32_t* offsets;
  const int32_t* ts;
  int E;
  float* Cf;
  long ldc;
  long c_estride;
  const float* bias;
  const float* H1;
  const float* H3;
  uint16_t* O1;
  uint16_t* O2;
  uint16_t* O3;
  long ldo;                  // row stride of O1 and O2 (0: ldc)
};
constexpr int kBwdBM = 128;   // rows per m-tile of the dgrad tile map

int launch_bwd_gemm(int mode, int epi, const BwdGemmParams& p, int m_tiles_max, hipStream_t stream);

}  // namespace moe
