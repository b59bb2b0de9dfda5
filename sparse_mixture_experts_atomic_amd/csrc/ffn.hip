// (c) Grouped expert FFN over variable-size segments.
//
// Segment e holds the rows routed to expert e (P1 §2.4: one batch per
// expert).  Experts are Linear (P4 公式：三步走), Linear-ReLU-Linear (P1 §3.2,
// P3 §3.1) or SwiGLU.  The segment sizes live on the device (offsets), so
// the m-tile -> segment map is built on the device and no count is read back.
//
// bf16 / fp8 weights: a grouped GEMM on gfx950 bf16 MFMA
// (v_mfma_f32_16x16x32_bf16) with double-buffered LDS tiles; fp8 e4m3 weight
// tiles are widened to bf16 on their way into LDS and their per-row scales
// are applied to the fp32 accumulators in the epilogue (the scale is per
// output row, so it factors out of the dot product).
// fp32 weights: a plain fp32 kernel (one output per thread).
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

// largest e in [0, E) with ts[e] <= m  (skips empty segments)
__device__ __forceinline__ int find_segment(const int32_t* ts, int E, int m) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (ts[mid] <= m) lo = mid; else hi = mid;
  }
  return lo;
}

// ------------------------------------------------------------ bf16 MFMA GEMM

constexpr int kBM = 128;        // rows per block tile
constexpr int kBN = 128;        // B rows (weight rows) per block tile
constexpr int kBK = 64;         // K per stage
constexpr int kGemmThreads = 256;

enum { EPI_PLAIN = 0, EPI_RELU = 1, EPI_SWIGLU = 2 };

struct GemmParams {
  const uint16_t* A;         // bf16 rows [*, K]
  int a_shared;              // 1: segment e reads A rows from 0 (shared experts)
  const int32_t* offsets;    // [E+1]
  const int32_t* ts;         // [E+1] m-tile prefix
  int E;
  const void* B1;            // [E, N, K] bf16 or e4m3
  const void* B3;            // SwiGLU up projection, [E, N, K]
  const float* s1;           // [E, N] fp8 row scales (or null)
  const float* s3;
  const float* bias;         // [E, N] (or null)
  uint16_t* C;               // bf16 [*, N]
  int N;                     // output columns
  int K;
};

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// 16 e4m3 codes -> 16 bf16 (exact: every e4m3 value is a bf16 value)
__device__ __forceinline__ void fp8x16_to_bf16(const uint4& q, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), false);
    auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), true);
    o[2 * i] = (__float_as_uint(f01[0]) >> 16) | (__float_as_uint(f01[1]) & 0xffff0000u);
    o[2 * i + 1] = (__float_as_uint(f23[0]) >> 16) | (__float_as_uint(f23[1]) & 0xffff0000u);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// Block tile: 128 rows x 128 weight rows, K stage 64, 4 wavefronts in a 2x2
// grid, each owning a 64x64 accumulator block = 4x4 MFMA 16x16 tiles.
// For SwiGLU each wavefront's 64 weight rows are 32 gate rows + the 32 up
// rows of the same hidden columns, so silu(gate) * up is formed in registers
// and a block produces 64 hidden columns.
// LDS rows are 64 bf16 = 8 chunks of 16 bytes; chunk c of row r is stored
// at position c ^ (r & 7) so that fragment reads spread over the banks.
template <int EPI, bool B_FP8>
__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_bf16_kernel(GemmParams p) {
  __shared__ uint4 As[2][kBM * 8];
  __shared__ uint4 Bs[2][kBN * 8];

  const int total = p.ts[p.E];
  const int mt_g = blockIdx.y;
  if (mt_g >= total) return;
  const int e = find_segment(p.ts, p.E, mt_g);
  const int seg0 = p.offsets[e];
  const int seg1 = p.offsets[e + 1];
  const int row0 = seg0 + (mt_g - p.ts[e]) * kBM;
  const int rows_valid = min(kBM, seg1 - row0);
  const int nt = blockIdx.x;
  const int K = p.K;
  const int N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // per-thread global sources for the A and B tile loads
  const uint16_t* a_src[4];
  int a_row[4], a_c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + kGemmThreads * i;
    const int r = q >> 3;
    a_row[i] = r;
    a_c[i] = q & 7;
    int rr = row0 + min(r, rows_valid - 1);
    if (p.a_shared) rr -= seg0;
    a_src[i] = p.A + static_cast<size_t>(rr) * K;
  }
  constexpr int kBLoads = B_FP8 ? 2 : 4;
  const uint8_t* b_src[kBLoads];
  int b_row[kBLoads], b_c[kBLoads];
#pragma unroll
  for (int i = 0; i < kBLoads; ++i) {
    const int q = tid + kGemmThreads * i;
    const int r = B_FP8 ? (q >> 2) : (q >> 3);
    b_row[i] = r;
    b_c[i] = B_FP8 ? (q & 3) : (q & 7);
    int n;
    const void* base = p.B1;
    if (EPI == EPI_SWIGLU) {
      const int w = r >> 6, q2 = r & 63;
      n = nt * 64 + w * 32 + (q2 & 31);
      if (q2 >= 32) base = p.B3;
    } else {
      n = nt * kBN + r;
    }
    n = min(n, N - 1);
    const size_t elem = B_FP8 ? 1 : 2;
    b_src[i] = static_cast<const uint8_t*>(base) + ((static_cast<size_t>(e) * N + n) * K) * elem;
  }

  uint4 ra[4];
  uint4 rb[kBLoads];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + a_c[i] * 8;
      ra[i] = k < K ? *reinterpret_cast<const uint4*>(a_src[i] + k) : zero4();
    }
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) {
      if (B_FP8) {
        const int k = k0 + b_c[i] * 16;
        rb[i] = k < K ? *reinterpret_cast<const uint4*>(b_src[i] + k) : zero4();
      } else {
        const int k = k0 + b_c[i] * 8;
        rb[i] = k < K ? *reinterpret_cast<const uint4*>(b_src[i] + static_cast<size_t>(k) * 2) : zero4();
      }
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) As[buf][a_row[i] * 8 + (a_c[i] ^ (a_row[i] & 7))] = ra[i];
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) {
      if (B_FP8) {
        uint4 lo, hi;
        fp8x16_to_bf16(rb[i], lo, hi);
        const int r = b_row[i];
        Bs[buf][r * 8 + ((2 * b_c[i]) ^ (r & 7))] = lo;
        Bs[buf][r * 8 + ((2 * b_c[i] + 1) ^ (r & 7))] = hi;
      } else {
        Bs[buf][b_row[i] * 8 + (b_c[i] ^ (b_row[i] & 7))] = rb[i];
      }
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int KT = (K + kBK - 1) / kBK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_tiles((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t af[4], bfr[4];
      const int c = kk * 4 + (lane >> 4);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int ar = wm * 64 + f * 16 + (lane & 15);
        const int br = wn * 64 + f * 16 + (lane & 15);
        uint4 va = As[buf][ar * 8 + (c ^ (ar & 7))];
        uint4 vb = Bs[buf][br * 8 + (c ^ (br & 7))];
        af[f] = *reinterpret_cast<bf16x8_t*>(&va);
        bfr[f] = *reinterpret_cast<bf16x8_t*>(&vb);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_tiles(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane/16)+r, column lane%16 of each tile
  const int col_in = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
      if (lr >= rows_valid) continue;
      uint16_t* crow = p.C + static_cast<size_t>(row0 + lr) * N;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = nt * 64 + wn * 32 + j * 16 + col_in;
          if (col >= N) continue;
          float g = acc[i][j][r];
          float u = acc[i][j + 2][r];
          if (p.s1) g *= p.s1[static_cast<size_t>(e) * N + col];
          if (p.s3) u *= p.s3[static_cast<size_t>(e) * N + col];
          crow[col] = f32_to_bf16(silu_f32(g) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = nt * kBN + wn * 64 + j * 16 + col_in;
          if (col >= N) continue;
          float v = acc[i][j][r];
          if (p.s1) v *= p.s1[static_cast<size_t>(e) * N + col];
          if (p.bias) v += p.bias[static_cast<size_t>(e) * N + col];
          if (EPI == EPI_RELU) v = fmaxf(v, 0.f);
          crow[col] = f32_to_bf16(v);
        }
      }
    }
  }
}

template <int EPI, bool B_FP8>
int launch_gemm(const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  const int n_cols_per_block = EPI == EPI_SWIGLU ? 64 : kBN;
  dim3 grid((p.N + n_cols_per_block - 1) / n_cols_per_block, m_tiles_max);
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<EPI, B_FP8>), grid, dim3(kGemmThreads), 0, stream, p);
  return check_launch();
}

int launch_gemm_any(int epi, bool fp8, const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  if (fp8) {
    if (epi == EPI_SWIGLU) return launch_gemm<EPI_SWIGLU, true>(p, m_tiles_max, stream);
    if (epi == EPI_RELU) return launch_gemm<EPI_RELU, true>(p, m_tiles_max, stream);
    return launch_gemm<EPI_PLAIN, true>(p, m_tiles_max, stream);
  }
  if (epi == EPI_SWIGLU) return launch_gemm<EPI_SWIGLU, false>(p, m_tiles_max, stream);
  if (epi == EPI_RELU) return launch_gemm<EPI_RELU, false>(p, m_tiles_max, stream);
  return launch_gemm<EPI_PLAIN, false>(p, m_tiles_max, stream);
}

// ------------------------------------------------------------ fp32 path

constexpr int kF32Cols = 64;
constexpr int kF32Rows = 4;

// out[a, n] = epi(sum_c in[row(a), c] * W[e, n, c]) with the segment of row a
// found by binary search on offsets.
template <int EPI>
__global__ __launch_bounds__(256) void ffn_f32_kernel(const float* __restrict__ in, int in_shared,
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
    const int src = in_shared ? a - offsets[e] : a;
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
    if (EPI == EPI_RELU) v = fmaxf(acc, 0.f);
    if (EPI == EPI_SWIGLU) v = silu_f32(acc) * acc3;
    out[static_cast<size_t>(a) * N + n] = v;
  }
}

template <int EPI>
int launch_f32(const float* in, int in_shared, const int32_t* offsets, int E, int K, int N, const float* W,
               const float* W3, const float* bias, float* out, int max_rows, hipStream_t stream) {
  int gy = (max_rows + kF32Rows - 1) / kF32Rows;
  if (gy > 65535) gy = 65535;
  if (gy < 1) gy = 1;
  dim3 grid((N + kF32Cols - 1) / kF32Cols, gy);
  hipLaunchKernelGGL((ffn_f32_kernel<EPI>), grid, dim3(256), 0, stream, in, in_shared, offsets, E, K, N, W, W3, bias, out);
  return check_launch();
}

inline int m_tiles_max(int max_rows, int E) { return (max_rows + kBM - 1) / kBM + E; }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_ffn_workspace_size(int kind, int act_dt, int max_rows, int E, int d, int d_ff, int d_out) {
  (void)d;
  (void)d_out;
  if (max_rows < 0 || E < 1) return 0;
  size_t s = align_up(static_cast<size_t>(E + 1) * sizeof(int32_t), kWsAlign);
  if (kind == MOE_FFN_RELU || kind == MOE_FFN_SWIGLU) {
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
  if (kind != MOE_FFN_LINEAR && kind != MOE_FFN_RELU && kind != MOE_FFN_SWIGLU) return MOE_ERR_INVALID_ARG;
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
  const void* ptrs[] = {x_rows, offsets, w1, w3, w2, s1, s3, s2, b1, b2, y_rows};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_ffn_workspace_size(kind, act_dt, max_rows, E, d, d_ff, d_out);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
  if (max_rows == 0) return MOE_OK;

  char* ws = static_cast<char*>(workspace);
  int32_t* ts = reinterpret_cast<int32_t*>(ws);
  void* H = ws + align_up(static_cast<size_t>(E + 1) * sizeof(int32_t), kWsAlign);
  const int shared_in = row_mode == MOE_ROWS_SHARED ? 1 : 0;
  const int n1 = two ? d_ff : d_out;

  if (act_dt == MOE_F32) {
    const float* X = static_cast<const float*>(x_rows);
    float* Y = static_cast<float*>(y_rows);
    if (kind == MOE_FFN_LINEAR)
      return launch_f32<EPI_PLAIN>(X, shared_in, offsets, E, d, d_out, static_cast<const float*>(w1), nullptr, b1, Y,
                                   max_rows, stream);
    float* Hf = static_cast<float*>(H);
    int st = kind == MOE_FFN_RELU
                 ? launch_f32<EPI_RELU>(X, shared_in, offsets, E, d, d_ff, static_cast<const float*>(w1), nullptr, b1,
                                        Hf, max_rows, stream)
                 : launch_f32<EPI_SWIGLU>(X, shared_in, offsets, E, d, d_ff, static_cast<const float*>(w1),
                                          static_cast<const float*>(w3), nullptr, Hf, max_rows, stream);
    if (st != MOE_OK) return st;
    return launch_f32<EPI_PLAIN>(Hf, 0, offsets, E, d_ff, d_out, static_cast<const float*>(w2), nullptr, b2, Y,
                                 max_rows, stream);
  }

  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(1024), 0, stream, offsets, E, kBM, ts);
  int st = check_launch();
  if (st != MOE_OK) return st;
  const int mtm = m_tiles_max(max_rows, E);
  if (mtm > 65535) return MOE_ERR_UNSUPPORTED;

  GemmParams p1{};
  p1.A = static_cast<const uint16_t*>(x_rows);
  p1.a_shared = shared_in;
  p1.offsets = offsets;
  p1.ts = ts;
  p1.E = E;
  p1.B1 = w1;
  p1.B3 = w3;
  p1.s1 = s1;
  p1.s3 = s3;
  p1.bias = b1;
  p1.C = two ? static_cast<uint16_t*>(H) : static_cast<uint16_t*>(y_rows);
  p1.N = n1;
  p1.K = d;
  const int epi1 = kind == MOE_FFN_SWIGLU ? EPI_SWIGLU : (kind == MOE_FFN_RELU ? EPI_RELU : EPI_PLAIN);
  st = launch_gemm_any(epi1, fp8, p1, mtm, stream);
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
  return launch_gemm_any(EPI_PLAIN, fp8, p2, mtm, stream);
}

}  // extern "C"
