// Grouped GEMM over variable-size expert segments on gfx950 bf16 MFMA.
//
// For each segment e (rows [offsets[e], offsets[e+1]) of A) and each weight
// matrix B_e [N, K] (stored [out, in], K contiguous):  C = epi(A_e B_e^T).
// This is the only dense contraction of the layer (the expert FFN matrices
// of P1 §3.2 / P3 §3.1 / P4 公式：三步走, one batch per expert as P1 §2.4
// describes).
//
// Two kernels share one device-built tile map (segment, m-tile, n-tile per
// block; no count goes back to the host) and the XCD-aware tile order (the
// blocks resident on one XCD, blockIdx % 8, take a contiguous range of
// tiles; per group of n-tiles: segment, n-tile, then the segment's m-tiles):
//  * grouped_gemm_dma_kernel (bf16 or e4m3 weights, K % 128 == 0): 256 x 256
//    tiles (128 x 256 for short segment tails), four wavefronts of 128 x 128
//    v_mfma_f32_32x32x16_bf16 fragments, operands moved global -> LDS by
//    global_load_lds_dwordx4 through a ring of five 32 KB half-slots, one DMA
//    every fourth MFMA; see the comments at the kernel.
//  * grouped_gemm_kernel (the rest): 256 x 128 tiles, 2x2 wavefronts,
//    register prefetch one stage ahead into a double-buffered LDS; e4m3
//    weights are widened to bf16 on the way into LDS (exact).
// In both, e4m3 row scales multiply the fp32 accumulators in the epilogue,
// and for SwiGLU each wavefront's weight rows are half gate and half up rows
// of the same hidden columns, so silu(gate) * up is formed in registers.
#include <type_traits>
#include <utility>

#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kNGroup = 8;      // n-tiles per ordering group

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

__device__ __forceinline__ int swz(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

// Workgroup barrier for LDS hand-off only: release/acquire fences scoped to
// LDS ("local") around s_barrier.  They order LDS accesses across the barrier
// and wait for this wave's LDS operations, but not for its global loads, so
// register prefetches stay in flight.  (__syncthreads also fences global
// memory, which would drain every outstanding load at each stage.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

// The m-tile prefix of the segments (tiles of kGemmBM rows) for this block:
// read from p.ts, or, when p.ts_build is set (E <= kGemmTsBuildMaxE), formed
// from the offsets by the first wavefront (a lane per segment, a wavefront
// scan) into lts (E + 1 ints of LDS) and also stored by block 0 to
// p.ts_build for the launches that follow.  Every thread of the block calls
// it (it ends with a block barrier when it builds).
__device__ __forceinline__ const int32_t* block_tile_prefix(const GemmParams& p, int32_t* lts) {
  if (!p.ts_build) return p.ts;
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    int v = 0;
    if (l < p.E) {
      const int len = p.offsets[l + 1] - p.offsets[l];
      v = len > 0 ? (len + kGemmBM - 1) / kGemmBM : 0;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o);
      if (l >= o) v += u;
    }
    if (l < p.E) lts[l + 1] = v;
    if (l == 0) lts[0] = 0;
    if (blockIdx.x == 0) {
      if (l < p.E) p.ts_build[l + 1] = v;
      if (l == 0) p.ts_build[0] = 0;
    }
  }
  __syncthreads();
  return lts;
}

// Register-staged kernel for shapes the DMA kernel does not take (K not a
// multiple of 128): block tile BM x BN (weight rows), 4 wavefronts in a 2x2
// grid, each owning a (BM/2) x (BN/2) accumulator tile; global -> registers
// one stage ahead, registers -> a double-buffered LDS, one barrier per stage.
// LDS rows of 32 bf16 = 4 chunks of 16 B, chunk c of row r stored at
// c ^ ((r >> 2) & 3) so 16 fragment rows hit 16 distinct bank groups; K tails
// load a clamped address and select zero.
template <int BM, int BN, int NH, int EPI, bool B_FP8>
__global__ __launch_bounds__(kThreads, BN == 128 ? 2 : 1) void grouped_gemm_kernel(GemmParams p) {
  constexpr int WM = BM / 2, WN = BN / 2;        // wave tile
  constexpr int FM = WM / 32, FN = WN / 32;      // 32x32 MFMA fragments per wave
  constexpr int BK = 32 * NH;                    // K per stage: NH halves of 32
  constexpr int A_LD = BM * 4 * NH / kThreads;   // 16-byte A loads per thread per stage
  constexpr int B_LD = B_FP8 ? BN * 2 * NH / kThreads : BN * 4 * NH / kThreads;
  constexpr int HC = EPI == EPI_SWIGLU ? BN / 2 : BN;   // output columns per block
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for the thread count");

  // [buffer][half][row * 4 + swizzled chunk]
  __shared__ uint4 As[2][NH][BM * 4];
  __shared__ uint4 Bs[2][NH][BN * 4];

  // ---- tile decode (XCD-aware, grouped over n) ----
  const int n_tiles = (p.N + HC - 1) / HC;
  const int m_total = p.ts[p.E];
  const int V = m_total * n_tiles;
  const int per = (V + kXcds - 1) / kXcds;
  const int b = blockIdx.x;
  const int slot = b / kXcds;
  if (slot >= per) return;
  const int L = (b % kXcds) * per + slot;
  if (L >= V) return;
  const int grp = L / (m_total * kNGroup);
  const int gs = min(kNGroup, n_tiles - grp * kNGroup);
  const int Lr = L - grp * m_total * kNGroup;
  const int e = find_segment(p.ts, p.E, Lr / gs);
  const int me = p.ts[e + 1] - p.ts[e];
  const int r = Lr - p.ts[e] * gs;
  const int mt_g = p.ts[e] + r % me;
  const int nt = grp * kNGroup + r / me;

  const int seg0 = p.offsets[e];
  const int seg1 = p.offsets[e + 1];
  const int row0 = seg0 + (mt_g - p.ts[e]) * BM;
  const int rows_valid = min(BM, seg1 - row0);
  const int K = p.K;
  const int N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // ---- per-thread global sources: a row's BK elements are 4*NH chunks of
  // 16 bytes (bf16) read by consecutive threads ----
  const uint16_t* a_src[A_LD];
  int a_slot[A_LD], a_k[A_LD], a_h[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int q = tid + kThreads * i;
    const int h = q / (BM * 4);
    const int r = (q % (BM * 4)) / 4;
    const int c = q % 4;
    a_h[i] = h;
    a_k[i] = h * 32 + c * 8;
    a_slot[i] = swz(r, c);
    int rr = row0 + min(r, rows_valid - 1);
    if (p.a_shared) rr -= seg0;
    if (p.gather) rr = min(max(p.gather[rr], 0), p.a_rows - 1);   // clamped: never outside A
    a_src[i] = p.A + static_cast<size_t>(rr) * K;
  }
  const uint8_t* b_src[B_LD];
  int b_r[B_LD], b_k[B_LD], b_h[B_LD], b_c[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int q = tid + kThreads * i;
    // bf16: a 16-byte chunk is 8 elements, 4 per half row; fp8: 16 elements,
    // 2 per half row (each widened to two bf16 chunks)
    const int per_half = B_FP8 ? 2 : 4;
    const int h = q / (BN * per_half);
    const int r = (q % (BN * per_half)) / per_half;
    const int c = q % per_half;
    b_r[i] = r;
    b_h[i] = h;
    b_k[i] = h * 32 + (B_FP8 ? c * 16 : c * 8);
    b_c[i] = B_FP8 ? c * 2 : c;               // first bf16 chunk within the half
    int n;
    const void* base = p.B1;
    if (EPI == EPI_SWIGLU) {
      const int w = r / WN, q2 = r % WN;
      n = nt * HC + w * (WN / 2) + q2 % (WN / 2);
      if (q2 >= WN / 2) base = p.B3;
    } else {
      n = nt * BN + r;
    }
    n = min(n, N - 1);
    const size_t elem = B_FP8 ? 1 : 2;
    b_src[i] = static_cast<const uint8_t*>(base) + ((static_cast<size_t>(e) * N + n) * K) * elem;
  }

  uint4 ra[A_LD];
  uint4 rb[B_LD];
  // K tails: the address is clamped into the row (always a valid load) and
  // the chunk is replaced by zeros, so there is no branch per load
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int k = k0 + a_k[i];
      const uint4 v = *reinterpret_cast<const uint4*>(a_src[i] + min(k, K - 8));
      ra[i] = k < K ? v : zero4();
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int k = k0 + b_k[i];
      const int kc = min(k, K - (B_FP8 ? 16 : 8));
      const size_t off = B_FP8 ? static_cast<size_t>(kc) : static_cast<size_t>(kc) * 2;
      const uint4 v = *reinterpret_cast<const uint4*>(b_src[i] + off);
      rb[i] = k < K ? v : zero4();
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) As[buf][a_h[i]][a_slot[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      if (B_FP8) {
        uint4 lo, hi;
        fp8x16_to_bf16(rb[i], lo, hi);
        Bs[buf][b_h[i]][swz(b_r[i], b_c[i])] = lo;
        Bs[buf][b_h[i]][swz(b_r[i], b_c[i] + 1)] = hi;
      } else {
        Bs[buf][b_h[i]][swz(b_r[i], b_c[i])] = rb[i];
      }
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // 32x32x16 operands: lane supplies row (lane % 32), k-chunk (lane / 32) of
  // the 16-wide k step.  A stage has 2*NH such sub-steps.
  const int fr = lane & 31;
  const int fc = lane >> 5;
  constexpr int NSUB = 2 * NH;
  auto read_frags = [&](int buf, int sub, bf16x8_t (&fa)[FM], bf16x8_t (&fb)[FN]) {
    const int h = sub >> 1, ks = sub & 1;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      uint4 v = Bs[buf][h][swz(wn * WN + j * 32 + fr, 2 * ks + fc)];
      fb[j] = *reinterpret_cast<bf16x8_t*>(&v);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      uint4 v = As[buf][h][swz(wm * WM + i * 32 + fr, 2 * ks + fc)];
      fa[i] = *reinterpret_cast<bf16x8_t*>(&v);
    }
  };
  // a wavefront whose rows all lie past the segment end (the partial last
  // tile of an expert) skips its MFMAs; it still loads and synchronises
  const bool wave_rows = wm * WM < rows_valid;
  auto mma = [&](const bf16x8_t (&fa)[FM], const bf16x8_t (&fb)[FN]) {
    if (!wave_rows) return;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  // Software pipeline, per stage kt (LDS buffer kt & 1):
  //   sub-step s: read the fragments of s+1 while the MFMAs of s run;
  //   after sub-step 0: write stage kt+1 (registers) into the other LDS
  //   buffer and issue the global loads of stage kt+2;
  //   before the last sub-step: barrier (stage kt+1 visible, every read of
  //   stage kt done), then the first fragments of stage kt+1 are read while
  //   the last MFMAs of stage kt run.
  const int KT = (K + BK - 1) / BK;
  load_stage(0);
  store_stage(0);
  if (KT > 1) load_stage(BK);
  lds_barrier();
  bf16x8_t fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  read_frags(0, 0, fa0, fb0);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < KT;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      bf16x8_t (&ca)[FM] = (sub & 1) ? fa1 : fa0;
      bf16x8_t (&cb)[FN] = (sub & 1) ? fb1 : fb0;
      bf16x8_t (&na)[FM] = (sub & 1) ? fa0 : fa1;
      bf16x8_t (&nb)[FN] = (sub & 1) ? fb0 : fb1;
      if (sub + 1 < NSUB) {
        read_frags(buf, sub + 1, na, nb);
      } else {
        lds_barrier();
        if (more) read_frags(buf ^ 1, 0, na, nb);
      }
      mma(ca, cb);
      if (sub == 0 && more) {
        store_stage(buf ^ 1);
        if (kt + 2 < KT) load_stage((kt + 2) * BK);
      }
    }
    // NSUB is even, so the next stage's first fragments sit in fa0/fb0
  }

  // ---- epilogue: element q of a 32x32 fragment is row 8*(q/4) + 4*(lane/32)
  // + q%4, column lane%32 ----
  uint16_t* C = p.C;
  if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int j = 0; j < FN / 2; ++j) {
      const int col = nt * HC + wn * (WN / 2) + j * 32 + fr;
      if (col >= N) continue;
      const float sg = p.s1 ? p.s1[static_cast<size_t>(e) * N + col] : 1.f;
      const float su = p.s3 ? p.s3[static_cast<size_t>(e) * N + col] : 1.f;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int lr = wm * WM + i * 32 + (q >> 2) * 8 + fc * 4 + (q & 3);
          if (lr < rows_valid) {
            const float g = acc[i][j][q] * sg;
            const float u = acc[i][j + FN / 2][q] * su;
            C[static_cast<size_t>(row0 + lr) * N + col] = f32_to_bf16(silu_f32(g) * u);
          }
        }
    }
  } else {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = nt * BN + wn * WN + j * 32 + fr;
      if (col >= N) continue;
      const float s = p.s1 ? p.s1[static_cast<size_t>(e) * N + col] : 1.f;
      const float bias = p.bias ? p.bias[static_cast<size_t>(e) * N + col] : 0.f;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int lr = wm * WM + i * 32 + (q >> 2) * 8 + fc * 4 + (q & 3);
          if (lr < rows_valid) {
            float v = acc[i][j][q] * s + bias;
            v = act1<EPI>(v);
            C[static_cast<size_t>(row0 + lr) * N + col] = f32_to_bf16(v);
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 weights, K % 128 == 0: operands go global -> LDS with
// global_load_lds_dwordx4 (no staging registers, no ds_write) in stages of 64
// columns of K, so that every DMA lane group reads whole 128-byte rows: the
// DMA path serves a fixed number of requests per clock, and 64-byte pieces
// halve its bytes per clock.  Block tile 256 x 256, four wavefronts of
// 128 x 128 (one wavefront per SIMD, accumulators in AGPRs).  The LDS image
// of an operand is a swizzled row-major layout (see dma_swz); a DMA lane
// writes slot base + lane, so each lane fetches the global chunk that belongs
// in its slot.
constexpr int kDmaKMult = 128;     // K granularity of the DMA kernel
constexpr int kDmaBK = 64;         // K columns per stage
// Pace of a 128- or 64-row bf16 tail tile: stage s + 1 may start no earlier
// than kTailStage shader cycles (s_memtime) per stage after the prologue.  A
// tail tile shares its weight tile with the 256-row tiles of the same n-tile,
// which start with it, but does a half or a quarter of their MFMAs: unpaced
// (~1400 or ~1100 cycles a stage against ~2400) it runs ahead, reads every
// weight stage from HBM before the others, and they miss in L2 too.  The
// workgroups of an XCD run in rounds, so finishing early gains nothing.  A
// target on the clock (not a fixed sleep) holds both tail sizes to the pace
// of the full tiles whatever the clock does.  Paced, the gate/up GEMM of the
// Mixtral-shaped layer reads 3.8 GB instead of 6.7 GB and the down GEMM
// 2.1 GB instead of 2.4 GB; 2200-2400 measured alike in time.
constexpr unsigned long long kTailStage = 2280;

// a pointer that is the same in every lane, moved to scalar registers
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uintptr_t v = reinterpret_cast<uintptr_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const T*>((static_cast<uintptr_t>(hi) << 32) | lo);
}

// One global_load_lds_dwordx4 in its scalar-base form: lane l copies the 16
// bytes at sbase + voff(l) to LDS byte address m0 + 16 l.  sbase and m0 must
// be wave-uniform.  Written as asm so that the compiler does not track it:
// its own tracking of these loads waits for every one in flight before any
// LDS read (vmcnt(0)), which would drain the ring at each k-step.  The
// instruction writes no register (its address operands are read at issue);
// completion is ordered by the explicit vmcnt waits and barriers below.  m0
// is restored, so code around the asm sees it unchanged.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t m0_value) {
  // readfirstlane gives the asm its own scalar copies (the compiler may keep
  // a uniform value in vector registers, which an "s" operand does not take)
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(m0_value);
  const void* sb = uniform_ptr(sbase);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sb), "s"(m0)
      : "memory");
}


__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>)
template <int N, typename F, int... I>
__device__ __forceinline__ void template_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void template_for(F&& f) {
  template_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// n DMAs spread evenly over a window of w MFMA positions: DMA j goes after
// position j * w / n; slot_at gives the DMA at a position (-1: none)
template <int W, int N>
constexpr int slot_pos(int j) { return j * W / N; }
template <int W, int N>
constexpr int slot_at(int i) {
  for (int j = 0; j < N; ++j)
    if (slot_pos<W, N>(j) == i) return j;
  return -1;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// row pitch (bf16 elements) of the split reduction's 128 x 128 staging block
constexpr int kEpPitch = 136;

// silu(u) = u / (1 + e^-u) with the hardware exp2 and reciprocal (relative
// error ~1e-7 each, far below the bf16 rounding of the result)
__device__ __forceinline__ float silu_fast(float u) {
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * u));
}

// chunk c (16 bytes) of row r of an LDS operand image with CH chunks per
// row.  Sixteen consecutive rows read at one chunk hit 16 distinct 16-byte
// bank groups: for CH = 4 the row sets the low two bits of the group and
// (r >> 2) & 3 is XORed into the chunk; for CH = 8, r & 1 picks the half and
// (r >> 1) & 7 is XORed in.
template <int CH>
__device__ __forceinline__ int dma_swz(int r, int c) {
  constexpr int SH = CH == 4 ? 2 : 1;
  return r * CH + (c ^ ((r >> SH) & (CH - 1)));
}

// Chunk swizzle of a transposed-B image (64 K rows of 32 16-byte chunks):
// the four K rows a half-wavefront's transposing read takes (k % 4 = 0..3)
// land 64 bytes apart, so they cover 256 distinct bytes
__device__ __forceinline__ int tb_swz(int k) { return 4 * (k & 3); }

// Split tail.  With V tiles and n_cu CUs (one block each), the last round
// holds rem = V % n_cu tiles and leaves the other CUs idle.  When that round
// is at most half full, its tiles are split along K into S parts (S <= n_cu /
// rem, <= split_max, whole stage pairs per part): tiles [0, full) run whole,
// then rem * S blocks each accumulate one K range of one of the last rem
// tiles into a partial buffer, and a reduction kernel sums the S parts in
// order and applies the epilogue.  Everything is derived on the device from
// the tile count, so no count goes back to the host.
struct SplitPlan {
  int full, rem, S, chunk;
};

__device__ __forceinline__ SplitPlan split_plan(int V, int KT, int R, int n_cu, int split_max) {
  SplitPlan sp{V, 0, 1, KT};
  if (split_max <= 1 || n_cu <= 0 || n_cu % kXcds != 0) return sp;
  const int rem = V % n_cu;
  if (rem == 0 || 2 * rem > n_cu) return sp;
  int S = min(split_max, n_cu / rem);
  S = min(S, KT / R);
  if (S <= 1) return sp;
  const int chunk = ((KT + S - 1) / S + R - 1) / R * R;
  S = (KT + chunk - 1) / chunk;
  if (S <= 1) return sp;
  sp.full = V - rem;
  sp.rem = rem;
  sp.S = S;
  sp.chunk = chunk;
  return sp;
}

// Epilogue of one wavefront's FM x 4 fragments of 32 x 32 (element q of a
// fragment is row 8 (q / 4) + 4 (lane / 32) + q % 4, column lane % 32),
// staged through an LDS block private to the wavefront, so that every lane
// then stores whole 16-byte pieces of output rows and no barrier is needed.
//   SwiGLU: fragments j and j + 2 hold the gate and up columns of the same
//   hidden units: 64 output columns, silu(gate) * up.
//   Plain/ReLU: 128 output columns (+ bias).
// e4m3 weights (p.s1 set): each column's accumulator is scaled by its weight
// row's scale first.
// row0: first output row of the wavefront, rows_valid: valid rows from there
// (may be <= 0), col0: first output column (pieces at col0 + c >= N are
// skipped; N % 8 == 0).  st must hold 32 FM x (OC + 8) bf16 of LDS that no
// other wavefront uses.
// RS: fp8 activations; rsl[r] (LDS) is the scale of the wavefront's row r,
// applied with the column scale before the activation.
template <int EPI, int FM, bool RS = false, bool PRE = false, int BWE = 0, bool NT = false>
__device__ __forceinline__ void wave_epilogue(const f32x16_t (&acc)[FM][4], uint16_t* st, const GemmParams& p, int e,
                                              int row0, int rows_valid, int col0, const float* rsl = nullptr) {
  constexpr int OC = EPI == EPI_SWIGLU ? 64 : 128;
  if constexpr (BWE != 0) {
    // the activation's backward (B rows plain, 128 columns), per 32-row
    // fragment: the fp32 accumulators staged through the wavefront's LDS
    // block (32 x 132 floats), then each lane takes pieces of 8 columns of a
    // row: 16-byte loads of the fp32 pre-activations, every output of the 8
    // elements formed at once, 16-byte stores.  BWE = 1 SwiGLU (dh1, dh3,
    // a), 2 ReLU, 3 GELU (dh, a).
    constexpr int FP = 128 + 4;
    float* sf = reinterpret_cast<float*>(st);
    const int N = p.N;
    const int lane = threadIdx.x & 63;
    const int fr = lane & 31, fc = lane >> 5;
    template_for<FM>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) sf[((q >> 2) * 8 + fc * 4 + (q & 3)) * FP + j * 32 + fr] = acc[i][j][q];
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = lane + 64 * u;
        const int r = c >> 4, cc = (c & 15) * 8;
        const int gr = i * 32 + r;
        const bool ok = gr < rows_valid && col0 + cc < N;
        const size_t o = ok ? static_cast<size_t>(row0 + gr) * N + col0 + cc : 0;
        float v[8], h1[8], h3[8];
        *reinterpret_cast<float4*>(v) = *reinterpret_cast<const float4*>(sf + r * FP + cc);
        *reinterpret_cast<float4*>(v + 4) = *reinterpret_cast<const float4*>(sf + r * FP + cc + 4);
        *reinterpret_cast<float4*>(h1) = *reinterpret_cast<const float4*>(p.hin1 + o);
        *reinterpret_cast<float4*>(h1 + 4) = *reinterpret_cast<const float4*>(p.hin1 + o + 4);
        if constexpr (BWE == 1) {
          *reinterpret_cast<float4*>(h3) = *reinterpret_cast<const float4*>(p.hin3 + o);
          *reinterpret_cast<float4*>(h3 + 4) = *reinterpret_cast<const float4*>(p.hin3 + o + 4);
        }
        uint32_t w0[4], w1[4], w2[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float x0[2], x1[2], x2[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int m = 2 * t + h;
            if constexpr (BWE == 1) {
              const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * h1[m]));
              const float si = h1[m] * sg;
              x0[h] = v[m] * h3[m] * sg * (1.0f + h1[m] * (1.0f - sg));
              x1[h] = v[m] * si;
              x2[h] = si * h3[m];
            } else if constexpr (BWE == 2) {
              x0[h] = h1[m] > 0.f ? v[m] : 0.f;
              x2[h] = fmaxf(h1[m], 0.f);
            } else {
              x0[h] = v[m] * gelu_grad_f32(h1[m]);
              x2[h] = gelu_f32(h1[m]);
            }
          }
          w0[t] = pack_bf16x2(x0[0], x0[1]);
          if constexpr (BWE == 1) w1[t] = pack_bf16x2(x1[0], x1[1]);
          w2[t] = pack_bf16x2(x2[0], x2[1]);
        }
        if (ok) {
          const size_t ro = static_cast<size_t>(row0 + gr);
          *reinterpret_cast<uint4*>(p.o1 + ro * p.ldo + col0 + cc) = make_uint4(w0[0], w0[1], w0[2], w0[3]);
          if constexpr (BWE == 1)
            *reinterpret_cast<uint4*>(p.o2 + ro * p.ldo + col0 + cc) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
          *reinterpret_cast<uint4*>(p.o3 + ro * N + col0 + cc) = make_uint4(w2[0], w2[1], w2[2], w2[3]);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
    });
    return;
  }
  if constexpr (PRE) {
    // fp32 outputs (gate (+ bias) to pre1, SwiGLU's up to pre3) staged
    // through the wavefront's LDS block in two passes (SwiGLU: gate, then
    // up, 128 rows x 64 columns; else rows 0-63, then 64-127, of 128
    // columns), then stored as whole 16-byte pieces of rows.  (Stored
    // straight from the accumulators, 4 bytes a lane, the epilogue of a
    // weight-gradient tile took longer than its 16 stages.)
    const int N = p.N;
    const int lane = threadIdx.x & 63;
    const int fr = lane & 31, fc = lane >> 5;
    constexpr int RP = EPI == EPI_SWIGLU ? 32 * FM : 16 * FM;   // rows per pass
    constexpr int PF = OC + 4;                                   // staging pitch (floats)
    static_assert(RP * PF * 4 <= 128 * (128 + 8) * 2, "staging block (the caller spaces the blocks so)");
    float* stf = reinterpret_cast<float*>(st);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      float* dst = (EPI == EPI_SWIGLU && pass == 1) ? p.pre3 : p.pre1;
      const int rb = EPI == EPI_SWIGLU ? 0 : pass * RP;          // first row of the pass
#pragma unroll
      for (int j = 0; j < OC / 32; ++j) {
        const int col = col0 + j * 32 + fr;
        const float bias =
            (EPI != EPI_SWIGLU && p.bias && col < N) ? p.bias[static_cast<size_t>(e) * N + col] : 0.f;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r = i * 32 + (q >> 2) * 8 + fc * 4 + (q & 3);
            if (r >= rb && r < rb + RP) {
              const float v = (EPI == EPI_SWIGLU && pass == 1) ? acc[i][j + 2][q] : acc[i][j][q] + bias;
              stf[(r - rb) * PF + j * 32 + fr] = v;
            }
          }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
#pragma unroll 4
      for (int u = 0; u < RP * (OC / 4) / 64; ++u) {
        const int c = lane + 64 * u;
        const int r = c / (OC / 4);
        const int pc = (c % (OC / 4)) * 4;
        if (rb + r < rows_valid && col0 + pc < N) {
          const float4 v = *reinterpret_cast<const float4*>(stf + r * PF + pc);
          float* o = dst + static_cast<size_t>(row0 + rb + r) * N + col0 + pc;
          if constexpr (NT) {
            // weight gradients: written once, read by no later kernel of the
            // pass; streamed past the L2 that holds the operands
            typedef float f4v_t __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(__builtin_bit_cast(f4v_t, v), reinterpret_cast<f4v_t*>(o));
          } else {
            *reinterpret_cast<float4*>(o) = v;
          }
        }
      }
      // the next pass overwrites the block: every lane's reads come first
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
    }
    return;
  }
  constexpr int PITCH = OC + 8;           // the two lane halves of a write land 16 banks apart
  constexpr int PR = OC / 8;              // 16-byte pieces per row
  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int fr = lane & 31;
  const int fc = lane >> 5;
#pragma unroll
  for (int j = 0; j < OC / 32; ++j) {
    const int col = col0 + j * 32 + fr;
    float bias = 0.f, sg = 1.f, su = 1.f;
    if (EPI != EPI_SWIGLU && p.bias) bias = col < N ? p.bias[static_cast<size_t>(e) * N + col] : 0.f;
    if (p.s1) {
      // e4m3 weights: the row scales of the output columns (gate and up rows
      // of the same hidden unit for SwiGLU)
      sg = col < N ? p.s1[static_cast<size_t>(e) * N + col] : 0.f;
      if (EPI == EPI_SWIGLU) su = col < N ? p.s3[static_cast<size_t>(e) * N + col] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 16; q += 2) {
        float v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float rs = 1.f;
          if constexpr (RS) rs = rsl[i * 32 + ((q + h) >> 2) * 8 + fc * 4 + ((q + h) & 3)];
          if (EPI == EPI_SWIGLU) {
            v[h] = silu_fast(acc[i][j][q + h] * (rs * sg)) * (acc[i][j + 2][q + h] * (rs * su));
          } else {
            v[h] = acc[i][j][q + h] * (rs * sg) + bias;
            v[h] = act1<EPI>(v[h]);
          }
        }
        const uint32_t pk = pack_bf16x2(v[0], v[1]);
        const int r = i * 32 + (q >> 2) * 8 + fc * 4 + (q & 3);   // rows r, r + 1
        st[r * PITCH + j * 32 + fr] = static_cast<uint16_t>(pk);
        st[(r + 1) * PITCH + j * 32 + fr] = static_cast<uint16_t>(pk >> 16);
      }
  }
  // the lanes of one wavefront read back what the others wrote: LDS
  // operations of a wavefront complete in order, the fence keeps the
  // compiler from moving the reads above the writes
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
#pragma unroll 4
  for (int u = 0; u < 32 * FM * PR / 64; ++u) {
    const int c = lane + 64 * u;
    const int r = c / PR;
    const int pc = (c % PR) * 8;
    if (r < rows_valid && col0 + pc < N) {
      const uint4 v = *reinterpret_cast<const uint4*>(st + r * PITCH + pc);
      *reinterpret_cast<uint4*>(p.C + static_cast<size_t>(row0 + r) * N + col0 + pc) = v;
    }
  }
}

// tile L of the grouped grid -> (segment e, n-tile nt, first row, valid rows).
// Within a group of gs n-tiles the order is segment, then n-tile, then the
// segment's m-tiles, so the m-tiles that share a weight tile are neighbours
// in L and run at the same time on one XCD whatever the segment lengths.
// MC > 0: a segment's m-tiles are taken in chunks of MC (segment, chunk,
// n-tile, m-tile of the chunk), so that a round of 32 tiles covers a few
// m-tiles by several n-tiles even when a segment has dozens of m-tiles (the
// weight gradients: 56 m-tiles of 256 output rows per expert at d_ff =
// 14336, where m fastest put 32 m-tiles of one n-tile in a round: 33
// operand streams for 32 tiles instead of 12).
struct TileCoord {
  int e, nt, row0, rows_valid, seg0;
};
template <int MC = 0>
__device__ __forceinline__ TileCoord tile_coord(const GemmParams& p, const int32_t* ts, int L, int m_total,
                                                int n_tiles, int BM) {
  const int grp = L / (m_total * kNGroup);
  const int gs = min(kNGroup, n_tiles - grp * kNGroup);
  const int Lr = L - grp * m_total * kNGroup;
  TileCoord t;
  t.e = find_segment(ts, p.E, Lr / gs);
  const int me = ts[t.e + 1] - ts[t.e];
  int r = Lr - ts[t.e] * gs;
  int m0 = 0, cs = me;
  if constexpr (MC > 0) {
    const int c = r / (MC * gs);
    m0 = c * MC;
    cs = min(MC, me - m0);
    r -= c * MC * gs;
  }
  const int mt_g = ts[t.e] + m0 + r % cs;
  t.nt = grp * kNGroup + r / cs;
  t.seg0 = p.offsets[t.e];
  t.row0 = t.seg0 + (mt_g - ts[t.e]) * BM;
  t.rows_valid = min(BM, p.offsets[t.e + 1] - t.row0);
  return t;
}

// The coordinates are the same in every lane (they depend on the block and
// the prefix only): moved to scalar registers, so that the addresses formed
// from them stay scalar whether the prefix was read from LDS or global memory.
__device__ __forceinline__ TileCoord uniform_tile(TileCoord t) {
  t.e = __builtin_amdgcn_readfirstlane(t.e);
  t.nt = __builtin_amdgcn_readfirstlane(t.nt);
  t.row0 = __builtin_amdgcn_readfirstlane(t.row0);
  t.rows_valid = __builtin_amdgcn_readfirstlane(t.rows_valid);
  t.seg0 = __builtin_amdgcn_readfirstlane(t.seg0);
  return t;
}

// Sum of the S K-parts of each split tile, in part order, then the epilogue.
// Four blocks per split tile, one per wavefront quadrant of the GEMM block
// (rows 128 (w / 2), columns 128 (w % 2)); thread (f, lane) of a block sums
// fragments (i = f, j = 0..3) of that quadrant and stages its bf16 results
// through LDS for 16-byte row stores.  Grid >= 4 * rem.
template <int EPI, int BK>
__global__ __launch_bounds__(kThreads) void split_reduce_kernel(GemmParams p) {
  constexpr int HC = EPI == EPI_SWIGLU ? 128 : 256;
  constexpr int R = 2;                   // split parts are whole stage pairs
  constexpr int OC = EPI == EPI_SWIGLU ? 64 : 128;   // output columns of a quadrant
  __shared__ uint16_t ep[128 * kEpPitch];
  const int n_tiles = (p.N + HC - 1) / HC;
  const int m_total = p.ts[p.E];
  const SplitPlan sp = split_plan(m_total * n_tiles, p.K / BK, R, p.n_cu, p.split_max);
  const int r = blockIdx.x >> 2;
  const int w = blockIdx.x & 3;
  if (r >= sp.rem) return;
  const TileCoord t = tile_coord(p, p.ts, sp.full + r, m_total, n_tiles, 256);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int fi = tid >> 6;
  const int fr = lane & 31;
  const int fc = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  f32x16_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.f;
  for (int s = 0; s < sp.S; ++s) {
    const float* base = p.partial + static_cast<size_t>(r * sp.S + s) * (256 * 256);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4* src = reinterpret_cast<const float4*>(base + ((static_cast<size_t>(w) * 16 + fi * 4 + j) * 64 + lane) * 16);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float4 x = src[v];
        acc[j][4 * v] += x.x;
        acc[j][4 * v + 1] += x.y;
        acc[j][4 * v + 2] += x.z;
        acc[j][4 * v + 3] += x.w;
      }
    }
  }
  // quadrant rows fi*32 + 8 (q/4) + 4 fc + q%4; LDS column = output column
  // of the quadrant
  const int N = p.N;
#pragma unroll
  for (int jj = 0; jj < (EPI == EPI_SWIGLU ? 2 : 4); ++jj) {
    const int lc = jj * 32 + fr;
    const int col = (EPI == EPI_SWIGLU ? t.nt * HC + wn * 64 : t.nt * 256 + wn * 128) + lc;
    float bias = 0.f, sg = 1.f, su = 1.f;
    if (EPI != EPI_SWIGLU && p.bias) bias = col < N ? p.bias[static_cast<size_t>(t.e) * N + col] : 0.f;
    if (p.s1) {
      sg = col < N ? p.s1[static_cast<size_t>(t.e) * N + col] : 0.f;
      if (EPI == EPI_SWIGLU) su = col < N ? p.s3[static_cast<size_t>(t.e) * N + col] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int lr = fi * 32 + (q >> 2) * 8 + fc * 4 + (q & 3);
      float v;
      if (EPI == EPI_SWIGLU) {
        v = silu_fast(acc[jj][q] * sg) * (acc[jj + 2][q] * su);
      } else {
        v = acc[jj][q] * sg + bias;
        v = act1<EPI>(v);
      }
      ep[lr * kEpPitch + lc] = f32_to_bf16(v);
    }
  }
  __syncthreads();
  constexpr int PR = OC / 8;                 // 16-byte pieces per row
  const int col0 = EPI == EPI_SWIGLU ? t.nt * HC + wn * 64 : t.nt * 256 + wn * 128;
  const int row_base = wm * 128;
#pragma unroll
  for (int u = 0; u < 128 * PR / kThreads; ++u) {
    const int c = tid + kThreads * u;
    const int lr = c / PR;
    const int pc = (c % PR) * 8;
    const int col = col0 + pc;
    if (row_base + lr < t.rows_valid && col < N) {
      const uint4 v = *reinterpret_cast<const uint4*>(ep + lr * kEpPitch + pc);
      *reinterpret_cast<uint4*>(p.C + static_cast<size_t>(t.row0 + row_base + lr) * N + col) = v;
    }
  }
}

// One block per tile.  FM = 4: the 256 x 256 tile (four wavefronts of
// 128 x 128); FM = 2: a 128 x 256 tile for the last m-tile of a segment with
// at most 128 rows (four wavefronts of 64 x 128: half the MFMA work, the same
// weight traffic).  Wavefront w owns rows 32 FM (w / 2) and B rows 128
// (w % 2).  Split units (unit >= 0) run stages [ks0, ks0 + nks) of a full
// tile and store raw accumulators.  (The tile body is a generic lambda
// rather than a function template: written as a function, the register
// allocator spilled some 200 accumulator registers around the stage loop.)
// XM: 0 the forward (bf16 or e4m3 C); 1 fp32 pre-activations (PRE epilogue);
// 2 weight gradients: per-segment K ranges (kseg), row pitches lda / ldb, B
// shared by the segments, fp32 output through the PRE epilogue
template <int EPI, int BK, bool FP8, int XM = 0>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_dma_kernel(GemmParams p) {
  // XM 7 and up: mode XM - 7 with B read from rows of K (TB): B[n][k] is
  // element (k, n) of a [K, N] matrix (a weight used transposed), each stage
  // a 64 x 256 image of K rows, read into MFMA operands by transposing LDS
  // reads.  Plain (7) and the activation backward (10-12) only.
  constexpr bool TB = XM >= 7;
  constexpr int XB = TB ? XM - 7 : XM;
  constexpr bool PRE = XB == 1 || XB == 2;
  constexpr bool WG = XB == 2;
  constexpr int BWE = XB >= 3 && XB <= 5 ? XB - 2 : 0;   // 3, 4, 5: the SwiGLU, ReLU, GELU backward epilogue
  constexpr bool STASH = XB == 6;             // the activation output and the fp32 pre-activations
  static_assert(!TB || (EPI == EPI_PLAIN && !FP8 && (XB == 0 || BWE != 0)), "transposed B: plain B rows only");
  constexpr int BM = 256;
  constexpr int R = 2;                  // split parts are whole stage pairs
  constexpr int HC = EPI == EPI_SWIGLU ? 128 : 256;
  static_assert(BK == kDmaBK, "stage depth");
  static_assert(4 * 128 * (128 + 8) * 2 <= 160 * 1024, "epilogue staging fits in the ring");
  __shared__ uint4 ring[5 * 256 * (kDmaBK / 8)];

  const int n_tiles = (p.N + HC - 1) / HC;
  // the m-tile prefix (formed here: in the last half-slot of the ring, which
  // no DMA fills before the barrier after the tile coordinates)
  const int32_t* ts = block_tile_prefix(p, reinterpret_cast<int32_t*>(ring + 4 * 256 * (kDmaBK / 8)));
  const int m_total = __builtin_amdgcn_readfirstlane(ts[p.E]);
  const int V = m_total * n_tiles;
  const int KT = p.K / BK;              // even
  const SplitPlan sp = split_plan(V, KT, R, p.n_cu, p.split_max);
  const int per = (sp.full + kXcds - 1) / kXcds;
  const int b = blockIdx.x;
  int L, unit = -1;
  if (b < kXcds * per) {
    L = (b % kXcds) * per + b / kXcds;   // blocks of one XCD take a contiguous range
    if (L >= sp.full) return;
  } else {
    unit = b - kXcds * per;              // split unit: tile full + unit / S, part unit % S
    if (unit >= sp.rem * sp.S) return;
    L = sp.full + unit / sp.S;
  }
  const int ks0 = unit < 0 ? 0 : (unit % sp.S) * sp.chunk;   // first stage of this block
  const TileCoord tc = uniform_tile(tile_coord<WG ? 4 : 0>(p, ts, L, m_total, n_tiles, BM));
  if (p.ts_build) __syncthreads();      // every lane has read the prefix before the ring fills
  // weight gradients: the segment's own K range (a multiple of 128, may be 0)
  // (kseg counts units of 128 columns)
  const int kb = WG ? p.kseg[tc.e] * kDmaKMult : 0;
  const int nks = WG ? (p.kseg[tc.e + 1] * kDmaKMult - kb) / BK
                     : (unit < 0 ? KT : min(sp.chunk, KT - ks0));   // stages (even, >= 2)
  auto tile = [&](auto fmc) __attribute__((always_inline)) {
    constexpr int FM = decltype(fmc)::value;
    constexpr int BN = 256;
    constexpr int BMA = 64 * FM;            // A rows of the tile
    constexpr int CH = BK / 8;              // 16-byte chunks per LDS row
    constexpr int NKS = BK / 16;            // MFMA k-steps per stage
    constexpr int WM = 32 * FM, WN = 128;
    constexpr int FN = WN / 32;
    constexpr int CHB = FP8 ? CH / 2 : CH;    // 16-byte chunks per B row (e4m3: one byte per value)
    constexpr int EB = FP8 ? 1 : 2;           // bytes per B value
    constexpr int LDA = BMA * CH / kThreads;  // DMA instructions per stage: A
    constexpr int LDB = BN * CHB / kThreads;  //   and B
    constexpr int RPI = kThreads / CH;        // rows covered by one DMA instruction: A
    constexpr int RPIB = kThreads / CHB;      //   and B
    constexpr int HALF = BN * CH;             // uint4 per half-slot (one operand of one stage)
    static_assert(BK == 64 && (FM == 4 || FM == 2 || (FM == 1 && !FP8)), "tile shapes");
    const int e = tc.e, nt = tc.nt, row0 = tc.row0, rows_valid = tc.rows_valid, seg0 = tc.seg0;
    const int K = p.K;
    const int N = p.N;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int fr = lane & 31;
    const int fc = lane >> 5;

    // DMA instruction i of this thread fills slot i * 256 + tid of an operand
    // image: row i * RPI + tid / CH, stored chunk tid % CH, which holds the
    // global chunk (tid % CH) ^ ((tid >> 4) % CH) (the swizzle term of that row,
    // the same for every i).  Addresses: a uniform base (advanced by 2 BK bytes
    // per stage) plus a 32-bit per-lane byte offset fixed for the whole loop.
    const int cq = (tid & (CH - 1)) ^ ((tid >> 4) & (CH - 1));
    // gathered rows (the dispatch permutation read in place): the base is A's
    // first row and each lane's offset that of its source row (the host
    // keeps a_rows * K * 2 below 2^31)
    const bool gat = p.gather != nullptr;
    const long lda = WG ? p.lda : K;
    const char* a_sb = uniform_ptr(reinterpret_cast<const char*>(
        gat ? p.A : p.A + static_cast<size_t>(p.a_shared ? row0 - seg0 : row0) * lda + kb));
    // (transposed B: no gather; the offsets are formed at each issue from the
    // lane's first row, which keeps seven registers free for the transposing
    // reads' addresses)
    uint32_t a_vo[TB ? 1 : LDA];
#pragma unroll
    for (int i = 0; i < (TB ? 1 : LDA); ++i) {
      const int r = min(i * RPI + tid / CH, rows_valid - 1);
      const int src = gat ? min(max(p.gather[row0 + r], 0), p.a_rows - 1) : r;   // clamped: never outside A
      a_vo[i] = static_cast<uint32_t>((src * lda + cq * 8) * 2);
    }
    const int cqb = (tid & (CHB - 1)) ^ ((tid >> 4) & (CHB - 1));
    const char* b_sb[LDB];
    uint32_t b_vo[LDB];
    if constexpr (TB) {
      // slot i * 256 + tid of a stage's image: K row i * 8 + tid / 32 (of 64),
      // stored chunk tid % 32 holding the row's global chunk (tid % 32) ^
      // tb_swz(row) of the n-tile's 256 columns (clamped into the matrix: the
      // columns past N feed discarded outputs)
      // (K row i * 8 + tid / 32 has the swizzle term of row tid / 32: one
      // lane offset serves every i, the row step goes into the uniform base)
      const int k = tid >> 5;
      const int n = min(nt * BN + 8 * ((tid & 31) ^ tb_swz(k)), N - 8);
      b_vo[0] = static_cast<uint32_t>((k * N + n) * 2);
      b_sb[0] = nullptr;
    }
#pragma unroll
    for (int i = 0; i < (TB ? 0 : LDB); ++i) {
      const int r = i * RPIB + tid / CHB;
      int n;
      const void* base = p.B1;
      if (EPI == EPI_SWIGLU) {
        // rows [128 w, 128 w + 64) are gate rows of hidden columns
        // nt * HC + 64 w + (0..63), the next 64 the up rows of the same columns;
        // one instruction's RPI rows lie in one such half
        n = nt * HC + (r >> 7) * 64 + (r & 63);
        if ((i * RPIB) & 64) base = p.B3;
      } else {
        n = nt * BN + r;
      }
      n = min(n, N - 1);
      if constexpr (WG) {
        b_sb[i] = uniform_ptr(static_cast<const char*>(base) + static_cast<size_t>(kb) * EB);
        b_vo[i] = static_cast<uint32_t>(n * p.ldb * EB + cqb * 16);
      } else {
        b_sb[i] = uniform_ptr(static_cast<const char*>(base) + static_cast<size_t>(e) * N * K * EB);
        b_vo[i] = static_cast<uint32_t>(n * K * EB + cqb * 16);
      }
    }
    const uint32_t wave_lds = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave)) * 1024u;
    // half-slot index (2 s + c) % 5 from (2 s) % 5 (both < 5)
    auto hs = [](int c) __attribute__((always_inline)) { return c >= 5 ? c - 5 : c; };
    // one DMA instruction: instruction q of operand A or B of stage st into
    // half-slot h
    auto issue_a = [&](int st, int h, int q) __attribute__((always_inline)) {
      if constexpr (TB) {
        const uint32_t vo = static_cast<uint32_t>((min(q * RPI + tid / CH, rows_valid - 1) * lda + cq * 8) * 2);
        dma16(a_sb + (ks0 + st) * BK * 2, vo, lds_addr(ring + h * HALF + q * 256) + wave_lds);
      } else {
        dma16(a_sb + (ks0 + st) * BK * 2, a_vo[q], lds_addr(ring + h * HALF + q * 256) + wave_lds);
      }
    };
    // transposed B: K row kg of expert e is at tb_lo + kg N 2 below tb_k1
    // (B1) and at tb_hi + kg N 2 from there on (B3; the origin shifted back
    // by tb_k1 rows), so a stage's base is one select and one multiply-add
    const uintptr_t tb_lo = TB ? reinterpret_cast<uintptr_t>(p.B1) + static_cast<uintptr_t>(e) * p.tb_k1 * N * 2 : 0;
    const uintptr_t tb_hi = TB ? reinterpret_cast<uintptr_t>(p.B3) +
                                     (static_cast<uintptr_t>(e) * (K - p.tb_k1) - p.tb_k1) * N * 2
                               : 0;
    auto issue_b = [&](int st, int h, int q) __attribute__((always_inline)) {
      if constexpr (TB) {
        const int kg = (ks0 + st) * BK;
        const uintptr_t base = (kg < p.tb_k1 ? tb_lo : tb_hi) + static_cast<uintptr_t>(kg + 8 * q) * N * 2;
        dma16(reinterpret_cast<const char*>(base), b_vo[0], lds_addr(ring + h * HALF + q * 256) + wave_lds);
      } else {
        dma16(b_sb[q] + (ks0 + st) * BK * EB, b_vo[q], lds_addr(ring + h * HALF + q * 256) + wave_lds);
      }
    };
    // transposed B: the 16-lane groups of a transposing read hand lane i
    // element i % 4 of the 8 bytes that lane 4 q + i / 4 of the group
    // addressed (q = 0..3).  Lane (fr, fc) needs K rows 16 ks + 8 fc + 0..7
    // of column wn WN + 32 r + fr, so lane j of a group addresses K row
    // 16 ks + 8 fc + 4 h + j / 4, columns 4 (j % 4) + 0..3 of the group's 16
    // (read h = 0, 1).  Byte offsets within a stage's image for k-step 0:
    // With the swizzle on chunk bits 2-3 (fragment r's bits), fragment r
    // sits at 64 (r ^ (k % 4)) bytes from the lane's fragment-0 chunk; read
    // h adds 4 K rows (2 KB), k-step ks 16 (8 KB).
    const int tb_q = (lane >> 2) & 3;                      // the lane's K row % 4
    const int tb_base = (8 * fc + tb_q) * 512 + (((wn * WN + (fr & 16)) >> 3) << 4) + (lane & 2) * 8 + (lane & 1) * 8;
    auto read_one = [&](const uint4* SA, const uint4* SB, int ks, int r, bf16x8_t (&fa)[FM], bf16x8_t (&fb)[FN])
        __attribute__((always_inline)) {
      if (r < FN && TB) {
        // two transposing reads (h = 0, 1) at the lane's fixed offsets; the
        // k-step adds 16 K rows (8 KB)
        const char* sb = reinterpret_cast<const char*>(SB) + tb_base + ((r ^ tb_q) << 6) + ks * (16 * 512);
        typedef short v4s_t __attribute__((ext_vector_type(4)));
        const v4s_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(sb));
        const v4s_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(sb + 4 * 512));
        fb[r] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      } else if (r < FN) {
        uint4 v = SB[dma_swz<CH>(wn * WN + r * 32 + fr, 2 * ks + fc)];
        fb[r] = *reinterpret_cast<bf16x8_t*>(&v);
      } else {
        uint4 v = SA[dma_swz<CH>(wm * WM + (r - FN) * 32 + fr, 2 * ks + fc)];
        fa[r - FN] = *reinterpret_cast<bf16x8_t*>(&v);
      }
    };
    // e4m3 weights: a lane reads 16 bytes of its B row per k-step pair p
    // (columns 32 p + 16 fc + 0..15); the first 8 feed k-step 2 p, the other 8
    // k-step 2 p + 1, so the A fragment of k-step ks takes bf16 chunk
    // 4 (ks / 2) + 2 fc + ks % 2 (the same columns; any order of the k values
    // inside one MFMA is fine as long as A and B agree).  The bytes are widened
    // with v_cvt_scalef32_pk_bf16_fp8 (scale 1: exact for every finite code).
    uint4 braw[FN];
    auto read_a8 = [&](const uint4* SA, int ks, int i, bf16x8_t (&fa)[FM]) __attribute__((always_inline)) {
      uint4 v = SA[dma_swz<CH>(wm * WM + i * 32 + fr, 4 * (ks >> 1) + 2 * fc + (ks & 1))];
      fa[i] = *reinterpret_cast<bf16x8_t*>(&v);
    };
    auto read_b8 = [&](const uint4* SB, int pair, int j) __attribute__((always_inline)) {
      braw[j] = SB[dma_swz<CHB>(wn * WN + j * 32 + fr, 2 * pair + fc)];
    };
    auto cvt_b8 = [&](int j, bool hi, bf16x8_t (&fb)[FN]) __attribute__((always_inline)) {
      const uint32_t w0 = hi ? braw[j].z : braw[j].x;
      const uint32_t w1 = hi ? braw[j].w : braw[j].y;
      uint4 o;
      o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
      o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
      o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
      o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
      fb[j] = __builtin_bit_cast(bf16x8_t, o);
    };

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    // MFMA q of a k-step: fragment row i = q / FN, columns in snake order
    // (ascending in even rows, descending in odd ones), so that each MFMA
    // shares an operand with the one before it (A along a row, B where two
    // rows meet).  Each accumulator still takes its k-steps in order, so the
    // results are bit for bit those of any other order; the operands that do
    // not change between MFMAs cost less power, and at the power limit that
    // is time (the Mixtral-shaped FFN 0.5% faster).
    auto mma_one = [&](int q, const bf16x8_t (&fa)[FM], const bf16x8_t (&fb)[FN]) __attribute__((always_inline)) {
      const int i = q / FN;
      const int j = (i & 1) ? FN - 1 - q % FN : q % FN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };

    bf16x8_t fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    // The 160 KB of LDS are five half-slots of 32 KB, each holding one operand
    // of one stage: stage s keeps A in half-slot (2 s) % 5 and B in (2 s + 1) % 5
    // (A of a 128-row tile fills half of it).
    // One stage, issued in a fixed order (sched_barrier keeps the compiler from
    // regrouping it); each MFMA is followed by about one LDS read and one DMA:
    //   k-steps 0-2: MFMAs with the next k-step's fragment reads;
    //   k-step 3: kPre MFMAs; wait for stage s + 1 (vmcnt), barrier s; the
    //   other MFMAs with the reads of stage s + 1's k-step 0.
    // Barrier s frees both half-slots of stage s.  The "window" from barrier s
    // to barrier s + 1 spans WIN MFMAs (the NM after barrier s, then k-steps
    // 0-2 and the kPre MFMAs of stage s + 1).  B(s + 2) goes out evenly over its
    // first half, into A(s)'s half-slot, then A(s + 3) over the second half,
    // into B(s)'s.  B(s + 2) must land by barrier s + 1, A(s + 3) only by
    // barrier s + 2.  The DMA path moves ~60 B/clk per CU at 128-byte rows, so
    // a stage's 64 KB take about half of its 2048 MFMA cycles; issued in bursts
    // they stall the MFMAs queued behind them, hence the spreading.
    // Compile-time flags: NEXT = stage s + 1 exists; PREB / PREA = this stage
    // issues the rest of B(s + 1) / A(s + 2) (window s - 1); POSTB = B(s + 2)'s
    // first part is issued after barrier s; WAITN = DMAs allowed in flight at
    // the wait (A(s + 2), issued last).
    constexpr int NQ = FM * FN;           // MFMAs per k-step
    constexpr int kPre = 2;
    constexpr int NM = NQ - kPre;         // MFMAs after the barrier
    constexpr int NRD = FM + FN;          // fragment reads per k-step
    constexpr int WIN = NQ * NKS;
    constexpr int SB_ = WIN / 2 / LDB;    // window positions between B DMAs
    constexpr int SA_ = WIN / 2 / LDA;    //   and between A DMAs
    static_assert(NKS == 4 && SB_ * LDB == WIN / 2 && SA_ * LDA == WIN / 2 && WIN - SA_ < WIN - kPre, "window layout");
    // window position i: B DMA i / SB_ if i < WIN/2 and i % SB_ == 0; A DMA (i - WIN/2) / SA_ likewise
    auto stage = [&](auto next, auto preb, auto prea, auto postb, auto waitn, int s, int cA)
        __attribute__((always_inline)) {
      const uint4* Ac = ring + cA * HALF;
      const uint4* Bc = ring + hs(cA + 1) * HALF;
      const uint4* An = ring + hs(cA + 2) * HALF;
      const uint4* Bn = ring + hs(cA + 3) * HALF;
      const int h_preb = hs(cA + 3);       // B(s + 1) = (2 s + 3) % 5
      const int h_prea = hs(cA + 4);       // A(s + 2) = (2 s + 4) % 5
      auto pre_dma = [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i < WIN / 2 && i % SB_ == 0 && decltype(preb)::value) issue_b(s + 1, h_preb, i / SB_);
        if constexpr (i >= WIN / 2 && (i - WIN / 2) % SA_ == 0 && decltype(prea)::value)
          issue_a(s + 2, h_prea, (i - WIN / 2) / SA_);
      };
      template_for<NKS - 1>([&](auto sc) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        auto& ca = (S & 1) ? fa1 : fa0;
        auto& cb = (S & 1) ? fb1 : fb0;
        auto& na = (S & 1) ? fa0 : fa1;
        auto& nb = (S & 1) ? fb0 : fb1;
        template_for<NQ>([&](auto qc) __attribute__((always_inline)) {
          constexpr int q = decltype(qc)::value;
          if constexpr (FP8) {
            // braw holds pair 0 (k-steps 0, 1) on entry, pair 1 from late in
            // k-step 0: k-step 0 widens its B fragments on demand and those of
            // k-step 1 next, k-step 1 those of k-step 2, k-step 2 those of 3
            if constexpr (S == 0 && q < FN) cvt_b8(q, false, fb0);
            mma_one(q, ca, cb);
            if constexpr (q % (NQ / FM) == 0) read_a8(Ac, S + 1, q / (NQ / FM), na);
            if constexpr (S == 0 && q >= FN && q < 2 * FN) cvt_b8(q - FN, true, fb1);
            if constexpr (S == 0 && q >= NQ - FN) read_b8(Bc, 1, q - (NQ - FN));
            if constexpr (S == 1 && q >= NQ - FN) cvt_b8(q - (NQ - FN), false, fb0);
            if constexpr (S == 2 && q < FN) cvt_b8(q, true, fb1);
          } else {
            mma_one(q, ca, cb);
#pragma unroll
            for (int c = q * NRD / NQ; c < (q + 1) * NRD / NQ; ++c) read_one(Ac, Bc, S + 1, c, na, nb);
          }
          pre_dma(std::integral_constant<int, NM + S * NQ + q>{});
          __builtin_amdgcn_sched_barrier(0);
        });
      });
      // k-step 3 (fa1/fb1)
      template_for<kPre>([&](auto qc) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        mma_one(q, fa1, fb1);
        pre_dma(std::integral_constant<int, WIN - kPre + q>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      wait_vmcnt<decltype(waitn)::value>();
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      template_for<NM>([&](auto qc) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        mma_one(kPre + q, fa1, fb1);
        if constexpr (decltype(next)::value) {
#pragma unroll
          for (int c = q * NRD / NM; c < (q + 1) * NRD / NM; ++c) {
            if constexpr (FP8) {
              if (c < FN) read_b8(Bn, 0, c);
              else read_a8(An, 0, c - FN, fa0);
            } else {
              read_one(An, Bn, 0, c, fa0, fb0);
            }
          }
        }
        if constexpr (q % SB_ == 0 && decltype(postb)::value) issue_b(s + 2, cA, q / SB_);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    using W0 = std::integral_constant<int, 0>;
    using WA = std::integral_constant<int, LDA>;
    // (weight gradients of an expert without rows: no stages, zero output)
    if (!WG || nks > 0) {
    if constexpr (FM <= 2 && !FP8) {
      // 128- and 64-row tiles, bf16: the mirrored ring.  A stage moves 48 KB (A is
      // half as tall) for half the MFMAs, so issued as above the B DMAs come
      // at one per two MFMAs and stall them.  Here B takes the even half-slot
      // of a stage and the long lead: stage s keeps B in (2 s) % 5 and A in
      // (2 s + 1) % 5; the window from barrier s to barrier s + 1 spreads all
      // twelve DMAs evenly, A(s + 2) first (into B(s)'s half-slot, landing by
      // barrier s + 1), then B(s + 3) (into A(s)'s, landing by barrier s + 2).
      // Each stage waits for its kTailStage target after its barrier (see there).
      // Window positions as in stage(); flags: POSTA = A(s + 2)'s first part
      // after barrier s; PREA / PREB = this stage issues the rest of A(s + 1)
      // / B(s + 2) (window s - 1); WAITN = DMAs allowed in flight at the
      // wait (B(s + 2), issued last).
      constexpr int NS = LDA + LDB;
      static_assert(slot_pos<WIN, NS>(LDA) >= NM && slot_pos<WIN, NS>(LDA - 1) < WIN - kPre, "mirrored window layout");
      unsigned long long t_pace = 0;   // shader clock when stage 0's MFMAs may start
      auto stage2 = [&](auto next, auto posta, auto prea, auto preb, auto waitn, int s, int cB)
          __attribute__((always_inline)) {
        const uint4* Bc = ring + cB * HALF;
        const uint4* Ac = ring + hs(cB + 1) * HALF;
        const uint4* Bn = ring + hs(cB + 2) * HALF;
        const uint4* An = ring + hs(cB + 3) * HALF;
        const int h_prea = hs(cB + 3);       // A(s + 1) = (2 s + 3) % 5
        const int h_preb = hs(cB + 4);       // B(s + 2) = (2 s + 4) % 5
        auto pre_dma = [&](auto ic) __attribute__((always_inline)) {
          constexpr int j = slot_at<WIN, NS>(decltype(ic)::value);
          if constexpr (j >= 0 && j < LDA && decltype(prea)::value) issue_a(s + 1, h_prea, j);
          if constexpr (j >= LDA && decltype(preb)::value) issue_b(s + 2, h_preb, j - LDA);
        };
        template_for<NKS - 1>([&](auto sc) __attribute__((always_inline)) {
          constexpr int S = decltype(sc)::value;
          auto& ca = (S & 1) ? fa1 : fa0;
          auto& cb = (S & 1) ? fb1 : fb0;
          auto& na = (S & 1) ? fa0 : fa1;
          auto& nb = (S & 1) ? fb0 : fb1;
          template_for<NQ>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            mma_one(q, ca, cb);
#pragma unroll
            for (int c = q * NRD / NQ; c < (q + 1) * NRD / NQ; ++c) read_one(Ac, Bc, S + 1, c, na, nb);
            pre_dma(std::integral_constant<int, NM + S * NQ + q>{});
            __builtin_amdgcn_sched_barrier(0);
          });
        });
        template_for<kPre>([&](auto qc) __attribute__((always_inline)) {
          constexpr int q = decltype(qc)::value;
          mma_one(q, fa1, fb1);
          pre_dma(std::integral_constant<int, WIN - kPre + q>{});
          __builtin_amdgcn_sched_barrier(0);
        });
        wait_vmcnt<decltype(waitn)::value>();
        lds_barrier();
        {
          const unsigned long long tgt = t_pace + static_cast<unsigned long long>(s + 1) * kTailStage;
          while (__builtin_amdgcn_s_memtime() < tgt) __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_sched_barrier(0);
        template_for<NM>([&](auto qc) __attribute__((always_inline)) {
          constexpr int q = decltype(qc)::value;
          mma_one(kPre + q, fa1, fb1);
          if constexpr (decltype(next)::value) {
#pragma unroll
            for (int c = q * NRD / NM; c < (q + 1) * NRD / NM; ++c) read_one(An, Bn, 0, c, fa0, fb0);
          }
          constexpr int j = slot_at<WIN, NS>(q);
          if constexpr (j >= 0 && j < LDA && decltype(posta)::value) issue_a(s + 2, cB, j);
          __builtin_amdgcn_sched_barrier(0);
        });
      };
      using WB = std::integral_constant<int, LDB>;
      // prologue: B(0), A(0), B(1), A(1), B(2) into half-slots 0 .. 4; wait for stage 0
#pragma unroll
      for (int q = 0; q < LDB; ++q) issue_b(0, 0, q);
#pragma unroll
      for (int q = 0; q < LDA; ++q) issue_a(0, 1, q);
#pragma unroll
      for (int q = 0; q < LDB; ++q) issue_b(1, 2, q);
#pragma unroll
      for (int q = 0; q < LDA; ++q) issue_a(1, 3, q);
      if (nks > 2) {
#pragma unroll
        for (int q = 0; q < LDB; ++q) issue_b(2, 4, q);
        wait_vmcnt<LDA + 2 * LDB>();
      } else {
        wait_vmcnt<LDA + LDB>();
      }
      lds_barrier();
#pragma unroll
      for (int r = 0; r < FM + FN; ++r) read_one(ring + HALF, ring, 0, r, fa0, fb0);
      t_pace = __builtin_amdgcn_s_memtime();
      if (nks == 2) {
        stage2(T_{}, F_{}, F_{}, F_{}, W0{}, 0, 0);
        stage2(F_{}, F_{}, F_{}, F_{}, W0{}, 1, 2);
      } else {
        stage2(T_{}, T_{}, F_{}, F_{}, WB{}, 0, 0);
        int cB = 2;
        for (int s = 1; s <= nks - 3; ++s) {
          stage2(T_{}, T_{}, T_{}, T_{}, WB{}, s, cB);
          cB = hs(cB + 2);
        }
        // s = nks - 2: only the rest of A(nks - 1) left to issue
        stage2(T_{}, F_{}, T_{}, F_{}, W0{}, nks - 2, cB);
        stage2(F_{}, F_{}, F_{}, F_{}, W0{}, nks - 1, hs(cB + 2));
      }
    } else {
      // prologue: A(0), B(0), A(1), B(1), A(2) into half-slots 0 .. 4; wait for stage 0
  #pragma unroll
      for (int q = 0; q < LDA; ++q) issue_a(0, 0, q);
  #pragma unroll
      for (int q = 0; q < LDB; ++q) issue_b(0, 1, q);
  #pragma unroll
      for (int q = 0; q < LDA; ++q) issue_a(1, 2, q);
  #pragma unroll
      for (int q = 0; q < LDB; ++q) issue_b(1, 3, q);
      if (nks > 2) {
  #pragma unroll
        for (int q = 0; q < LDA; ++q) issue_a(2, 4, q);
        wait_vmcnt<2 * LDA + LDB>();
      } else {
        wait_vmcnt<LDA + LDB>();
      }
      lds_barrier();
      if constexpr (FP8) {
  #pragma unroll
        for (int j = 0; j < FN; ++j) read_b8(ring + HALF, 0, j);
  #pragma unroll
        for (int i = 0; i < FM; ++i) read_a8(ring, 0, i, fa0);
      } else {
  #pragma unroll
        for (int r = 0; r < FM + FN; ++r) read_one(ring, ring + HALF, 0, r, fa0, fb0);
      }
      if (nks == 2) {
        stage(T_{}, F_{}, F_{}, F_{}, W0{}, 0, 0);
        stage(F_{}, F_{}, F_{}, F_{}, W0{}, 1, 2);
      } else {
        stage(T_{}, F_{}, F_{}, T_{}, WA{}, 0, 0);
        int cA = 2;
        for (int s = 1; s <= nks - 3; ++s) {
          stage(T_{}, T_{}, T_{}, T_{}, WA{}, s, cA);
          cA = hs(cA + 2);
        }
        // s = nks - 2: only the rest of B(nks - 1) left to issue
        stage(T_{}, T_{}, F_{}, F_{}, W0{}, nks - 2, cA);
        stage(F_{}, F_{}, F_{}, F_{}, W0{}, nks - 1, hs(cA + 2));
      }
    }

    }
    if constexpr (FM == 4) {
      if (unit >= 0) {
        // split unit: raw accumulators to the partial buffer, in the MFMA layout
        float* pt = p.partial + static_cast<size_t>(unit) * (256 * 256);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            float4* dst = reinterpret_cast<float4*>(pt + ((static_cast<size_t>(wave) * (FM * FN) + i * FN + j) * 64 + lane) * 16);
#pragma unroll
            for (int v = 0; v < 4; ++v)
              dst[v] = make_float4(acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2], acc[i][j][4 * v + 3]);
          }
        return;
      }
    }
    // the ring is free: the last LDS reads of every wavefront came before the
    // last barrier and no load is in flight
    constexpr int OC = EPI == EPI_SWIGLU ? 64 : 128;
    const int col0 = EPI == EPI_SWIGLU ? nt * HC + wn * 64 : nt * BN + wn * 128;
    // (the fp32 staging of PRE takes the 128 + 8 bf16 pitch whatever OC is)
    uint16_t* st = reinterpret_cast<uint16_t*>(ring) + wave * 128 * ((PRE || STASH ? 128 : OC) + 8);
    if constexpr (STASH) {
      // first the pre-activations (fp32), then the activation (bf16), each
      // staged through the wavefront's block (the first ends with a fence)
      wave_epilogue<EPI, FM, false, true>(acc, st, p, e, row0 + wm * WM, rows_valid - wm * WM, col0);
      wave_epilogue<EPI, FM, false, false>(acc, st, p, e, row0 + wm * WM, rows_valid - wm * WM, col0);
    } else {
      wave_epilogue<EPI, FM, false, PRE, BWE, WG>(acc, st, p, e, row0 + wm * WM, rows_valid - wm * WM, col0);
    }
  };
  if constexpr (!FP8) {
    if (unit < 0 && tc.rows_valid <= 64) {
      tile(std::integral_constant<int, 1>{});
      return;
    }
  }
  if (unit < 0 && tc.rows_valid <= 128)
    tile(std::integral_constant<int, 2>{});
  else
    tile(std::integral_constant<int, 4>{});
}

// ---------------------------------------------------------------------------
// e4m3 activations x e4m3 weights on v_mfma_scale_f32_32x32x64_f8f6f4 (unit
// scales; the per-row scales of both operands multiply the fp32
// accumulators in the epilogue).  One byte per value, so a stage of 128 K
// values has the byte geometry of a bf16 stage of 64: rows of 128 bytes,
// eight 16-byte chunks in the same LDS swizzle, DMA'd global -> LDS by
// global_load_lds_dwordx4 with per-lane offsets fixed for the whole loop
// (gathered rows: the offset of the source row).  Tile 256 x 256, four
// wavefronts of 128 x 128 (4 x 4 fragments, 256 accumulator registers).  A
// k-step is 64 values: a lane supplies 32 bytes of its row (row lane % 32,
// k-half lane / 32), read as two 16-byte chunks; A and B use the same lane
// to k mapping, which is all the product needs.
// The stages move through the bf16 kernel's ring of five 32 KB half-slots
// (stage s: A in half-slot (2 s) % 5, B in (2 s + 1) % 5) with its issue
// schedule: two k-steps of 16 MFMAs per stage; the window from barrier s to
// barrier s + 1 (the 14 MFMAs after barrier s, k-step 0 of stage s + 1 and
// the first 2 MFMAs of its k-step 1) issues B(s + 2) over its first half into
// A(s)'s half-slot and A(s + 3) over its second half into B(s)'s, one DMA per
// two MFMAs; the fragment reads of the next k-step go one per MFMA.  (A
// double buffer of two 64 KB stages waited for the next stage's DMAs in the
// middle of every stage: 40-53% MFMA busy.)
typedef int i32x8_t __attribute__((ext_vector_type(8)));
constexpr int kF8BK = 128;         // K values (bytes) per stage
constexpr int kF8Half = 256 * kF8BK / 16;    // uint4 per half-slot (one operand of one stage)
// the epilogue's staging (four wavefronts of 128 rows x 136 bf16 = 136 KB)
// and the row scales (2 KB) after it reuse the ring
constexpr int kF8Stg = 4 * 128 * (128 + 8) * 2;
static_assert(kF8Stg + 4 * 128 * 4 <= 5 * kF8Half * 16, "epilogue staging and row scales fit in the ring");

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_f8_kernel(GemmParams p) {
  constexpr int HC = EPI == EPI_SWIGLU ? 128 : 256;
  constexpr int CH = 8;                      // 16-byte chunks per LDS row
  constexpr int ND = 256 * CH / kThreads;    // DMA instructions per operand and stage (8)
  constexpr int HALF = kF8Half;
  constexpr int NQ = 16;                     // MFMAs per k-step
  constexpr int NKS = 2;                     // k-steps per stage
  constexpr int kPre = 2;                    // MFMAs of the last k-step before the barrier
  constexpr int NM = NQ - kPre;              // and after it
  constexpr int WIN = NQ * NKS;              // window positions
  constexpr int SP = WIN / 2 / ND;           // window positions between DMAs of one operand
  static_assert(SP * ND == WIN / 2 && WIN / 2 + (ND - 1) * SP <= WIN - kPre, "window layout");
  __shared__ uint4 ring[5 * HALF];           // 160 KB

  const int n_tiles = (p.N + HC - 1) / HC;
  // the m-tile prefix (formed here: in the last half-slot of the ring, which
  // no DMA fills before the barrier after the tile coordinates)
  const int32_t* ts = block_tile_prefix(p, reinterpret_cast<int32_t*>(ring + 4 * HALF));
  const int m_total = __builtin_amdgcn_readfirstlane(ts[p.E]);
  const int V = m_total * n_tiles;
  const int per = (V + kXcds - 1) / kXcds;
  const int b = blockIdx.x;
  if (b / kXcds >= per) return;
  const int L = (b % kXcds) * per + b / kXcds;   // blocks of one XCD take a contiguous range
  if (L >= V) return;
  const TileCoord tc = uniform_tile(tile_coord(p, ts, L, m_total, n_tiles, 256));
  if (p.ts_build) __syncthreads();      // every lane has read the prefix before the ring fills
  const int e = tc.e, nt = tc.nt, row0 = tc.row0, rows_valid = tc.rows_valid, seg0 = tc.seg0;
  const int K = p.K, N = p.N;
  const int KT = K / kF8BK;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31, fc = lane >> 5;

  // per-lane DMA offsets: instruction i fills rows 32 i + tid / 8, stored
  // chunk tid % 8, which holds the global chunk (tid % 8) ^ ((tid >> 4) % 8)
  const int cq = (tid & (CH - 1)) ^ ((tid >> 4) & (CH - 1));
  const bool gat = p.gather != nullptr;
  const uint8_t* A8 = reinterpret_cast<const uint8_t*>(p.A);
  const char* a_sb = uniform_ptr(reinterpret_cast<const char*>(
      gat ? A8 : A8 + static_cast<size_t>(p.a_shared ? row0 - seg0 : row0) * K));
  uint32_t a_vo[ND], b_vo[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    const int r = min(i * 32 + tid / CH, rows_valid - 1);
    const int src = gat ? min(max(p.gather[row0 + r], 0), p.a_rows - 1) : r;
    a_vo[i] = static_cast<uint32_t>(src * K + cq * 16);
    const int rb = i * 32 + tid / CH;
    int n;
    if (EPI == EPI_SWIGLU) n = nt * HC + (rb >> 7) * 64 + (rb & 63);
    else n = nt * 256 + rb;
    n = min(n, N - 1);
    b_vo[i] = static_cast<uint32_t>(n * K + cq * 16);
  }
  const char* b_sb1 = uniform_ptr(static_cast<const char*>(p.B1) + static_cast<size_t>(e) * N * K);
  const char* b_sb3 = EPI == EPI_SWIGLU ? uniform_ptr(static_cast<const char*>(p.B3) + static_cast<size_t>(e) * N * K)
                                        : b_sb1;
  const uint32_t wave_lds = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(wave)) * 1024u;
  auto hs = [](int c) __attribute__((always_inline)) { return c >= 5 ? c - 5 : c; };
  auto issue_a = [&](int st, int h, int q) __attribute__((always_inline)) {
    dma16(a_sb + st * kF8BK, a_vo[q], lds_addr(ring + h * HALF + q * 256) + wave_lds);
  };
  // SwiGLU: rows 64..127 of each 128-row half are up rows
  auto issue_b = [&](int st, int h, int q) __attribute__((always_inline)) {
    const char* bb = (EPI == EPI_SWIGLU && ((q * 32) & 64)) ? b_sb3 : b_sb1;
    dma16(bb + st * kF8BK, b_vo[q], lds_addr(ring + h * HALF + q * 256) + wave_lds);
  };
  // chunk c (0..15) of k-step ks's fragments: fragment c / 2 (A 0..3, B
  // 4..7), its 16-byte half c % 2 (chunk 4 ks + 2 fc + c % 2 of the row)
  auto read_chunk = [&](const uint4* SA, const uint4* SB, int ks, int c, i32x8_t (&f)[8])
      __attribute__((always_inline)) {
    const int r = c >> 1, h = c & 1;
    const uint4 v = r < 4 ? SA[dma_swz<CH>(wm * 128 + r * 32 + fr, 4 * ks + 2 * fc + h)]
                          : SB[dma_swz<CH>(wn * 128 + (r - 4) * 32 + fr, 4 * ks + 2 * fc + h)];
    f[r][4 * h] = static_cast<int>(v.x);
    f[r][4 * h + 1] = static_cast<int>(v.y);
    f[r][4 * h + 2] = static_cast<int>(v.z);
    f[r][4 * h + 3] = static_cast<int>(v.w);
  };
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  // a wavefront whose rows all lie past the segment's end skips its MFMAs
  const bool wave_rows = wm * 128 < rows_valid;
  // columns in snake order, as in the bf16 kernel
  auto mma = [&](const i32x8_t (&f)[8], int q) __attribute__((always_inline)) {
    const int i = q >> 2, j = (i & 1) ? 3 - (q & 3) : q & 3;
    if (wave_rows)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f[i], f[4 + j], acc[i][j], 0, 0, 0, 127, 0, 127);
  };
  i32x8_t f0[8], f1[8];                      // k-step 0 and k-step 1 fragments

  // One stage; flags as in the bf16 kernel: NEXT = stage s + 1 exists; PREB /
  // PREA = this stage issues the rest of B(s + 1) / A(s + 2) (window s - 1);
  // POSTB = B(s + 2)'s first part after barrier s; WAITN = DMAs allowed in
  // flight at the wait (A(s + 2), issued last).
  auto stage = [&](auto next, auto preb, auto prea, auto postb, auto waitn, int s, int cA)
      __attribute__((always_inline)) {
    const uint4* Ac = ring + cA * HALF;
    const uint4* Bc = ring + hs(cA + 1) * HALF;
    const uint4* An = ring + hs(cA + 2) * HALF;
    const uint4* Bn = ring + hs(cA + 3) * HALF;
    const int h_preb = hs(cA + 3);
    const int h_prea = hs(cA + 4);
    auto pre_dma = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < WIN / 2 && i % SP == 0 && decltype(preb)::value) issue_b(s + 1, h_preb, i / SP);
      if constexpr (i >= WIN / 2 && (i - WIN / 2) % SP == 0 && decltype(prea)::value)
        issue_a(s + 2, h_prea, (i - WIN / 2) / SP);
    };
    // k-step 0 (f0), reading k-step 1's fragments into f1
    template_for<NQ>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      mma(f0, q);
      read_chunk(Ac, Bc, 1, q, f1);
      pre_dma(std::integral_constant<int, NM + q>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    // k-step 1 (f1): kPre MFMAs, the wait and barrier s, then the rest with
    // stage s + 1's k-step 0 fragments into f0
    template_for<kPre>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      mma(f1, q);
      pre_dma(std::integral_constant<int, WIN - kPre + q>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    wait_vmcnt<decltype(waitn)::value>();
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    template_for<NM>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      mma(f1, kPre + q);
      if constexpr (decltype(next)::value) {
#pragma unroll
        for (int c = q * 16 / NM; c < (q + 1) * 16 / NM; ++c) read_chunk(An, Bn, 0, c, f0);
      }
      if constexpr (q % SP == 0 && decltype(postb)::value) issue_b(s + 2, cA, q / SP);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using W0 = std::integral_constant<int, 0>;
  using WA = std::integral_constant<int, ND>;
  // prologue: A(0), B(0), A(1), B(1), A(2) into half-slots 0 .. 4; wait for stage 0
#pragma unroll
  for (int q = 0; q < ND; ++q) issue_a(0, 0, q);
#pragma unroll
  for (int q = 0; q < ND; ++q) issue_b(0, 1, q);
  if (KT > 1) {
#pragma unroll
    for (int q = 0; q < ND; ++q) issue_a(1, 2, q);
#pragma unroll
    for (int q = 0; q < ND; ++q) issue_b(1, 3, q);
  }
  if (KT > 2) {
#pragma unroll
    for (int q = 0; q < ND; ++q) issue_a(2, 4, q);
    wait_vmcnt<3 * ND>();
  } else if (KT > 1) {
    wait_vmcnt<2 * ND>();
  } else {
    wait_vmcnt<0>();
  }
  lds_barrier();
#pragma unroll
  for (int c = 0; c < 16; ++c) read_chunk(ring, ring + HALF, 0, c, f0);
  if (KT == 1) {
    stage(F_{}, F_{}, F_{}, F_{}, W0{}, 0, 0);
  } else if (KT == 2) {
    stage(T_{}, F_{}, F_{}, F_{}, W0{}, 0, 0);
    stage(F_{}, F_{}, F_{}, F_{}, W0{}, 1, 2);
  } else {
    stage(T_{}, F_{}, F_{}, T_{}, WA{}, 0, 0);
    int cA = 2;
    for (int s = 1; s <= KT - 3; ++s) {
      stage(T_{}, T_{}, T_{}, T_{}, WA{}, s, cA);
      cA = hs(cA + 2);
    }
    // s = KT - 2: only the rest of B(KT - 1) left to issue
    stage(T_{}, T_{}, F_{}, F_{}, W0{}, KT - 2, cA);
    stage(F_{}, F_{}, F_{}, F_{}, W0{}, KT - 1, hs(cA + 2));
  }
  // the ring is free (the last LDS reads of every wavefront came before the
  // last barrier, no DMA is in flight): row scales of the wavefront's rows
  // after the staging area, then the epilogue
  float* rsl = reinterpret_cast<float*>(reinterpret_cast<char*>(ring) + kF8Stg) + wave * 128;
  for (int r = lane; r < 128; r += 64) {
    const int lr = min(wm * 128 + r, rows_valid - 1);
    const int grow = row0 + lr;
    const int src = gat ? min(max(p.gather[grow], 0), p.a_rows - 1) : (p.a_shared ? grow - seg0 : grow);
    rsl[r] = p.row_scale[src];
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  constexpr int OC = EPI == EPI_SWIGLU ? 64 : 128;
  const int col0 = EPI == EPI_SWIGLU ? nt * HC + wn * 64 : nt * 256 + wn * 128;
  wave_epilogue<EPI, 4, true>(acc, reinterpret_cast<uint16_t*>(ring) + wave * 128 * (OC + 8), p, e,
                              row0 + wm * 128, rows_valid - wm * 128, col0, rsl);
}

template <int EPI, int BK, bool FP8, int XM>
int launch_dma_pre(const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  constexpr bool PRE = XM >= 1 && XM != 7;   // (no split tail for the extra modes but the transposed-B plain one)
  constexpr int HC = EPI == EPI_SWIGLU ? 128 : 256;
  const long n_tiles = (p.N + HC - 1) / HC;
  long blocks = n_tiles * m_tiles_max;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;
  // the tail can matter only for a grid of a few rounds; otherwise no split
  // (and no reduction launch)
  const bool split = !PRE && p.split_max > 1 && p.partial && p.n_cu > 0 && n_tiles * m_tiles_max <= 4L * p.n_cu;
  if (split) blocks += p.n_cu;   // full + rem * S = V + rem * (S - 1) < V + n_cu
  if (blocks > 0x7fffffffL) return MOE_ERR_UNSUPPORTED;
  GemmParams q = p;
  if (!split) q.split_max = 1;
  hipLaunchKernelGGL((grouped_gemm_dma_kernel<EPI, BK, FP8, XM>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                     0, stream, q);
  int st = check_launch();
  if (st != MOE_OK || !split) return st;
  hipLaunchKernelGGL((split_reduce_kernel<EPI, BK>), dim3(static_cast<unsigned>(4 * p.n_cu)), dim3(kThreads), 0, stream,
                     p);
  return check_launch();
}

template <int EPI, int BK, bool FP8>
int launch_dma(const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  return launch_dma_pre<EPI, BK, FP8, 0>(p, m_tiles_max, stream);
}

template <int BM, int BN, int NH, int EPI, bool FP8>
int launch(const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  constexpr int HC = EPI == EPI_SWIGLU ? BN / 2 : BN;
  const long n_tiles = (p.N + HC - 1) / HC;
  long blocks = n_tiles * m_tiles_max;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;
  if (blocks > 0x7fffffffL) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, NH, EPI, FP8>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                     0, stream, p);
  return check_launch();
}

template <int BM, int BN, int NH>
int launch_epi(int epi, bool fp8, const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  if (fp8) {
    if (epi == EPI_SWIGLU) return launch<BM, BN, NH, EPI_SWIGLU, true>(p, m_tiles_max, stream);
    if (epi == EPI_RELU) return launch<BM, BN, NH, EPI_RELU, true>(p, m_tiles_max, stream);
    if (epi == EPI_GELU) return launch<BM, BN, NH, EPI_GELU, true>(p, m_tiles_max, stream);
    return launch<BM, BN, NH, EPI_PLAIN, true>(p, m_tiles_max, stream);
  }
  if (epi == EPI_SWIGLU) return launch<BM, BN, NH, EPI_SWIGLU, false>(p, m_tiles_max, stream);
  if (epi == EPI_RELU) return launch<BM, BN, NH, EPI_RELU, false>(p, m_tiles_max, stream);
  if (epi == EPI_GELU) return launch<BM, BN, NH, EPI_GELU, false>(p, m_tiles_max, stream);
  return launch<BM, BN, NH, EPI_PLAIN, false>(p, m_tiles_max, stream);
}

}  // namespace

int launch_grouped_gemm_f8(int epi, const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  if (p.K % kF8BK != 0 || p.N % 8 != 0 || !p.row_scale) return MOE_ERR_UNSUPPORTED;
  if (static_cast<size_t>(p.N) * p.K >= (size_t(1) << 31) || static_cast<size_t>(kGemmBM) * p.K >= (size_t(1) << 31) ||
      (p.gather && static_cast<size_t>(p.a_rows) * p.K >= (size_t(1) << 31)))
    return MOE_ERR_UNSUPPORTED;
  const long HC = epi == EPI_SWIGLU ? 128 : 256;
  const long n_tiles = (p.N + HC - 1) / HC;
  long blocks = n_tiles * m_tiles_max;
  blocks = (blocks + kXcds - 1) / kXcds * kXcds;
  if (blocks <= 0) return MOE_OK;
  if (blocks > 0x7fffffffL) return MOE_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  switch (epi) {
    case EPI_SWIGLU: hipLaunchKernelGGL(grouped_gemm_f8_kernel<EPI_SWIGLU>, grid, block, 0, stream, p); break;
    case EPI_RELU: hipLaunchKernelGGL(grouped_gemm_f8_kernel<EPI_RELU>, grid, block, 0, stream, p); break;
    case EPI_GELU: hipLaunchKernelGGL(grouped_gemm_f8_kernel<EPI_GELU>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(grouped_gemm_f8_kernel<EPI_PLAIN>, grid, block, 0, stream, p); break;
  }
  return check_launch();
}

// 256-row tiles throughout (one tile map serves both GEMMs of an FFN); the
// weight-row width is 256 unless that leaves too few tiles to fill 256 CUs
// a few times over, in which case 128.
int launch_grouped_gemm_pre(int epi, const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  const bool dma_ok = p.K % kDmaKMult == 0 && p.N % 8 == 0 && static_cast<size_t>(p.N) * p.K * 2 < (size_t(1) << 31) &&
                      static_cast<size_t>(kGemmBM) * p.K * 2 < (size_t(1) << 31) && !p.gather && !p.s1 &&
                      p.pre1 && (epi != EPI_SWIGLU || p.pre3);
  if (!dma_ok) return MOE_ERR_UNSUPPORTED;
  GemmParams q = p;
  q.split_max = 1;
  if (epi == EPI_SWIGLU) return launch_dma_pre<EPI_SWIGLU, kDmaBK, false, 1>(q, m_tiles_max, stream);
  if (epi == EPI_PLAIN) return launch_dma_pre<EPI_PLAIN, kDmaBK, false, 1>(q, m_tiles_max, stream);
  return MOE_ERR_UNSUPPORTED;
}

int launch_grouped_gemm_stash(int epi, const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  const bool dma_ok = p.K % kDmaKMult == 0 && p.N % 8 == 0 && static_cast<size_t>(p.N) * p.K * 2 < (size_t(1) << 31) &&
                      static_cast<size_t>(kGemmBM) * p.K * 2 < (size_t(1) << 31) && !p.gather && !p.s1 && p.C &&
                      p.pre1 && (epi != EPI_SWIGLU || p.pre3);
  if (!dma_ok) return MOE_ERR_UNSUPPORTED;
  GemmParams q = p;
  q.split_max = 1;
  if (epi == EPI_SWIGLU) return launch_dma_pre<EPI_SWIGLU, kDmaBK, false, 6>(q, m_tiles_max, stream);
  if (epi == EPI_RELU) return launch_dma_pre<EPI_RELU, kDmaBK, false, 6>(q, m_tiles_max, stream);
  if (epi == EPI_GELU) return launch_dma_pre<EPI_GELU, kDmaBK, false, 6>(q, m_tiles_max, stream);
  return MOE_ERR_UNSUPPORTED;
}

int launch_grouped_gemm_actbwd(int bwd_epi, const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  const bool ok = p.K % kDmaKMult == 0 && p.N % 8 == 0 && p.ldo % 8 == 0 &&
                  static_cast<size_t>(p.N) * p.K * 2 < (size_t(1) << 31) &&
                  static_cast<size_t>(kGemmBM) * p.K * 2 < (size_t(1) << 31) && !p.gather && !p.s1 && !p.bias &&
                  p.hin1 && p.o1 && p.o3 && (bwd_epi != BWD_EPI_SWIGLU || (p.hin3 && p.o2));
  if (!ok) return MOE_ERR_UNSUPPORTED;
  GemmParams q = p;
  q.split_max = 1;
  if (bwd_epi == BWD_EPI_SWIGLU) return launch_dma_pre<EPI_PLAIN, kDmaBK, false, 3>(q, m_tiles_max, stream);
  if (bwd_epi == BWD_EPI_RELU) return launch_dma_pre<EPI_PLAIN, kDmaBK, false, 4>(q, m_tiles_max, stream);
  if (bwd_epi == BWD_EPI_GELU) return launch_dma_pre<EPI_PLAIN, kDmaBK, false, 5>(q, m_tiles_max, stream);
  return MOE_ERR_UNSUPPORTED;
}

namespace {
bool tb_ok(const GemmParams& p) {
  static_assert(kDmaKMult == 128 && kDmaBK == 64 && kGemmBM == 256, "the shape check's constants");
  return grouped_gemm_tb_shape_ok(p.K, p.N, p.tb_k1) && (p.tb_k1 == p.K || p.B3) && !p.gather && !p.s1 && !p.bias;
}
}  // namespace

int launch_grouped_gemm_tb(const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  if (!tb_ok(p)) return MOE_ERR_UNSUPPORTED;
  if (p.split_max > 1 && !p.partial) return MOE_ERR_UNSUPPORTED;
  return launch_dma_pre<EPI_PLAIN, kDmaBK, false, 7>(p, m_tiles_max, stream);
}

int launch_grouped_gemm_actbwd_tb(int bwd_epi, const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  if (!tb_ok(p) || p.ldo % 8 != 0 || !p.hin1 || !p.o1 || !p.o3 || (bwd_epi == BWD_EPI_SWIGLU && (!p.hin3 || !p.o2)))
    return MOE_ERR_UNSUPPORTED;
  GemmParams q = p;
  q.split_max = 1;
  if (bwd_epi == BWD_EPI_SWIGLU) return launch_dma_pre<EPI_PLAIN, kDmaBK, false, 10>(q, m_tiles_max, stream);
  if (bwd_epi == BWD_EPI_RELU) return launch_dma_pre<EPI_PLAIN, kDmaBK, false, 11>(q, m_tiles_max, stream);
  if (bwd_epi == BWD_EPI_GELU) return launch_dma_pre<EPI_PLAIN, kDmaBK, false, 12>(q, m_tiles_max, stream);
  return MOE_ERR_UNSUPPORTED;
}

int launch_grouped_gemm_wgrad(const GemmParams& p, int m_tiles_max, hipStream_t stream) {
  // 31-bit per-lane byte offsets: 256 rows of A, N rows of B, at their pitches
  const bool ok = p.kseg && p.a_shared && p.pre1 && p.N % 8 == 0 && p.lda % 8 == 0 && p.ldb % 8 == 0 &&
                  static_cast<size_t>(kGemmBM) * p.lda * 2 < (size_t(1) << 31) &&
                  static_cast<size_t>(p.N) * p.ldb * 2 < (size_t(1) << 31) && !p.gather && !p.s1 && !p.bias;
  if (!ok) return MOE_ERR_UNSUPPORTED;
  GemmParams q = p;
  q.split_max = 1;
  q.K = kDmaKMult;              // (the per-segment K ranges come from kseg)
  return launch_dma_pre<EPI_PLAIN, kDmaBK, false, 2>(q, m_tiles_max, stream);
}

int launch_grouped_gemm(int epi, bool fp8, const GemmParams& p, int max_rows, int m_tiles_max, hipStream_t stream) {
  (void)max_rows;
  // LDS-DMA kernel: bf16 weights, K a multiple of the ring's K per round,
  // 16-byte output rows (N % 8 == 0), and 31-bit byte offsets inside one
  // expert's weight matrix and one m-tile
  const size_t wbytes = fp8 ? 1 : 2;
  const bool dma_ok = p.K % kDmaKMult == 0 && p.N % 8 == 0 && static_cast<size_t>(p.N) * p.K * wbytes < (size_t(1) << 31) &&
                      static_cast<size_t>(kGemmBM) * p.K * 2 < (size_t(1) << 31) &&
                      (!p.gather || static_cast<size_t>(p.a_rows) * p.K * 2 < (size_t(1) << 31));
  if (dma_ok && fp8) {
    if (epi == EPI_SWIGLU) return launch_dma<EPI_SWIGLU, kDmaBK, true>(p, m_tiles_max, stream);
    if (epi == EPI_RELU) return launch_dma<EPI_RELU, kDmaBK, true>(p, m_tiles_max, stream);
    if (epi == EPI_GELU) return launch_dma<EPI_GELU, kDmaBK, true>(p, m_tiles_max, stream);
    return launch_dma<EPI_PLAIN, kDmaBK, true>(p, m_tiles_max, stream);
  }
  if (dma_ok) {
    if (epi == EPI_SWIGLU) return launch_dma<EPI_SWIGLU, kDmaBK, false>(p, m_tiles_max, stream);
    if (epi == EPI_RELU) return launch_dma<EPI_RELU, kDmaBK, false>(p, m_tiles_max, stream);
    if (epi == EPI_GELU) return launch_dma<EPI_GELU, kDmaBK, false>(p, m_tiles_max, stream);
    return launch_dma<EPI_PLAIN, kDmaBK, false>(p, m_tiles_max, stream);
  }
  if (p.ts_build) {
    // the register-staged kernel reads a prefix built before it
    const int st = launch_tile_map(p.offsets, p.E, kGemmBM, p.ts_build, stream);
    if (st != MOE_OK) return st;
    GemmParams q = p;
    q.ts_build = nullptr;
    return launch_epi<kGemmBM, 128, 1>(epi, fp8, q, m_tiles_max, stream);
  }
  return launch_epi<kGemmBM, 128, 1>(epi, fp8, p, m_tiles_max, stream);
}

}  // namespace moe
