// Grouped GEMMs of the expert FFN's backward pass on gfx950 bf16 MFMA.
//
// The forward pass multiplies rows of a segment by a weight stored [out, in]
// with `in` contiguous (C = A B^T, both operands K-contiguous).  Its gradients
// need the two other layouts (P1 §4.3: every token's gradient must reach the
// expert rows it came from; P3 §2.2: only the selected experts get any):
//   dgrad   dA = dY W     A = dY [rows, K] (K-contiguous), B = W_e [K, N]
//                         (N-contiguous); segments on M (the packed rows).
//   wgrad   dW = dY^T X   A = dY [rows, M], B = X [rows, N], both with the
//                         reduction index (the segment's rows) outermost;
//                         one [M, N] output per expert, K = segment length.
// One kernel takes both: an operand whose reduction index is outermost is
// transposed in registers on its way into LDS (each thread loads two k-rows
// of 8 values and packs the 8 k-pairs with v_perm), so that the LDS image and
// the fragment reads are those of a K-contiguous operand.
//
// Tile 128 x 128 x 32, four wavefronts of 64 x 64 (2 x 2 fragments of
// v_mfma_f32_32x32x16_bf16), register prefetch of the next stage into a
// double-buffered LDS, one barrier per stage.  K tails and rows past a
// segment are zero-filled (clamped address, selected zero), so any segment
// length works.
//
// A third mode has the forward layout (both operands K-contiguous): it
// recomputes the first layer's pre-activations h = X W1^T (+ b1) into fp32.
// They stay fp32 because the derivatives of SiLU and GELU have roots (near
// u = -1.28 and u = -0.75) where a bf16-rounded h is only absolutely, not
// relatively, accurate, and a one-row segment's weight gradient is that one
// product.
//
// Epilogues (dgrad): bf16 store; SwiGLU backward (dh1 = da h3 silu'(h1),
// dh3 = da silu(h1), a = silu(h1) h3 from the fp32 pre-activations);
// ReLU / GELU backward (dh = da act'(h), a = act(h)).  wgrad: fp32 store.
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kBT = 256;          // threads
constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kBxcds = 8;
constexpr int kBGroup = 8;      // n-tiles per ordering group

__device__ __forceinline__ int bswz(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

// lo halves (k, k + 1) of word w of two rows / hi halves
__device__ __forceinline__ uint32_t pair_lo(uint32_t r0, uint32_t r1) { return __builtin_amdgcn_perm(r1, r0, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t r0, uint32_t r1) { return __builtin_amdgcn_perm(r1, r0, 0x07060302u); }

__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// largest e with ts[e] <= m
__device__ __forceinline__ int seg_of(const int32_t* ts, int E, int m) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ts[mid] <= m) lo = mid; else hi = mid;
  }
  return lo;
}


}  // namespace

// Tile (e, m-tile, n-tile) of a grouped backward GEMM; see the file header.
template <int MODE, int EPI>
__global__ __launch_bounds__(kBT, 2) void bwd_gemm_kernel(BwdGemmParams p) {
  constexpr bool SEGK = MODE == BWD_WGRAD;
  constexpr bool AT = SEGK;                 // A's reduction index outermost (wgrad), else K-contiguous
  constexpr bool BT = MODE != BWD_FWD;      // B's reduction index outermost, else K-contiguous (forward layout)
  __shared__ uint4 As[2][kBM * 4];
  __shared__ uint4 Bs[2][kBN * 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31, fc = lane >> 5;

  // ---- tile decode: blocks of one XCD (blockIdx % 8) take a contiguous
  // range of tiles.  The tiles come in groups of kBGroup n-tiles; inside a
  // group (dgrad) segment by segment, each segment's m-tiles for every
  // n-tile, or (wgrad) m-tile by m-tile, each for every n-tile of the group.
  // The 64 tiles an XCD runs at once (two per CU) then share 8 A and 8 B
  // tiles instead of one B tile and 64 A tiles. ----
  const int n_tiles = (p.N + kBN - 1) / kBN;
  int e, row0, rows_valid, nt, k_begin, k_end;
  long a_row0 = 0, b_row0 = 0;
  {
    int V, L;
    if constexpr (SEGK) {
      const int m_tiles = (p.M + kBM - 1) / kBM;
      V = p.E * m_tiles * n_tiles;
      const int per = (V + kBxcds - 1) / kBxcds;
      const int slot = blockIdx.x / kBxcds;
      if (slot >= per) return;
      L = (blockIdx.x % kBxcds) * per + slot;
      if (L >= V) return;
      e = L / (m_tiles * n_tiles);
      const int r = L - e * m_tiles * n_tiles;
      const int grp = r / (m_tiles * kBGroup);
      const int gs = min(kBGroup, n_tiles - grp * kBGroup);
      const int rr = r - grp * m_tiles * kBGroup;
      nt = grp * kBGroup + rr % gs;
      row0 = (rr / gs) * kBM;
      rows_valid = min(kBM, p.M - row0);
      k_begin = p.offsets[e];
      k_end = p.offsets[e + 1];
      // shared experts: every segment is the same token batch, rows from 0
      a_row0 = p.a_shared ? -static_cast<long>(k_begin) : 0;
      b_row0 = p.b_shared ? -static_cast<long>(k_begin) : 0;
    } else {
      const int m_total = p.ts[p.E];
      V = m_total * n_tiles;
      const int per = (V + kBxcds - 1) / kBxcds;
      const int slot = blockIdx.x / kBxcds;
      if (slot >= per) return;
      L = (blockIdx.x % kBxcds) * per + slot;
      if (L >= V) return;
      const int grp = L / (m_total * kBGroup);
      const int gs = min(kBGroup, n_tiles - grp * kBGroup);
      const int Lr = L - grp * m_total * kBGroup;
      e = seg_of(p.ts, p.E, Lr / gs);
      const int me = p.ts[e + 1] - p.ts[e];
      const int r = Lr - p.ts[e] * gs;
      nt = grp * kBGroup + r / me;
      const int seg0 = p.offsets[e];
      row0 = seg0 + (r % me) * kBM;
      rows_valid = min(kBM, p.offsets[e + 1] - row0);
      k_begin = 0;
      k_end = p.K;
      a_row0 = p.a_shared ? -static_cast<long>(seg0) : 0;
    }
  }
  const int n0 = nt * kBN;

  // ---- per-thread load plans ----
  // K-contiguous operand (dgrad A): rows r = q / 4, chunk c = q % 4, two per thread
  // reduction-outermost operand: thread (kp = tid / 16, c = tid % 16) loads
  // k-rows 2 kp, 2 kp + 1 of columns 8 c .. 8 c + 7 of the tile
  const int tkp = tid >> 4, tc = tid & 15;
  uint4 ra[2], rb[2];
  const uint16_t* __restrict__ Ab = p.A;
  const uint16_t* __restrict__ Bb = p.B + static_cast<size_t>(e) * p.b_estride;
  const uint16_t* __restrict__ Bb2 = p.B2 ? p.B2 + static_cast<size_t>(e) * p.b_estride : nullptr;

  auto load_stage = [&](int k0) __attribute__((always_inline)) {
    if constexpr (AT) {
      // A(m, k) = A[k * lda + m]: rows k0 + 2 tkp (+1), m = row0 + 8 tc ..
      const int m = min(row0 + 8 * tc, p.M - 8);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = k0 + 2 * tkp + h;
        const int kc = min(k, k_end - 1);
        const uint4 v = *reinterpret_cast<const uint4*>(Ab + static_cast<size_t>(kc + a_row0) * p.lda + m);
        ra[h] = k < k_end ? v : make_uint4(0u, 0u, 0u, 0u);
      }
    } else {
      // A(m, k) = A[(row0 + r) * lda + k]; K parts: k < K1 from A, else A2
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int q = tid + kBT * i;
        const int r = q >> 2, c = q & 3;
        const int row = row0 + min(r, rows_valid - 1);
        int k = k0 + 8 * c;
        const uint16_t* src = Ab;
        int kk = k;
        if (p.A2 && k >= p.K1) {
          src = p.A2;
          kk = k - p.K1;
        }
        const int kcl = min(kk, (p.A2 && k >= p.K1 ? p.K - p.K1 : p.K1) - 8);
        const uint4 v = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(row + a_row0) * p.lda + kcl);
        ra[i] = k < k_end ? v : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if constexpr (!BT) {
      // forward layout B(n, k) = B_e[n * ldb + k]: rows n = n0 + q / 4, chunk q % 4
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int q = tid + kBT * i;
        const int n = min(n0 + (q >> 2), p.N - 1);
        const int k = k0 + 8 * (q & 3);
        const uint4 v = *reinterpret_cast<const uint4*>(Bb + static_cast<size_t>(n) * p.ldb + min(k, p.K - 8));
        rb[i] = k < k_end ? v : make_uint4(0u, 0u, 0u, 0u);
      }
      return;
    }
    // B(n, k) = B[k * ldb + n]: rows k0 + 2 tkp (+1), n = n0 + 8 tc ..
    const int n = min(n0 + 8 * tc, p.N - 8);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + 2 * tkp + h;
      const uint16_t* src = Bb;
      int kk = k;
      if constexpr (!SEGK) {
        if (Bb2 && k >= p.K1) {
          src = Bb2;
          kk = k - p.K1;
        }
      }
      const int klim = SEGK ? k_end - 1 : ((Bb2 && k >= p.K1) ? p.K - p.K1 : p.K1) - 1;
      const int kc = min(kk, klim);
      const uint4 v = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(kc + b_row0) * p.ldb + n);
      rb[h] = k < k_end ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  // register image -> LDS: transposed operands write 8 words (k-pair 2 tkp,
  // 2 tkp + 1 of rows 8 tc .. 8 tc + 7); chunk tkp / 4, word tkp % 4
  auto store_t = [&](uint4* S, const uint4 (&r)[2]) __attribute__((always_inline)) {
    uint32_t* S32 = reinterpret_cast<uint32_t*>(S);
    const uint32_t w0[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
    const uint32_t w1[4] = {r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t v = (i & 1) ? pair_hi(w0[i >> 1], w1[i >> 1]) : pair_lo(w0[i >> 1], w1[i >> 1]);
      S32[bswz(8 * tc + i, tkp >> 2) * 4 + (tkp & 3)] = v;
    }
  };
  auto store_stage = [&](int buf) __attribute__((always_inline)) {
    if constexpr (AT) {
      store_t(As[buf], ra);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int q = tid + kBT * i;
        As[buf][bswz(q >> 2, q & 3)] = ra[i];
      }
    }
    if constexpr (BT) {
      store_t(Bs[buf], rb);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int q = tid + kBT * i;
        Bs[buf][bswz(q >> 2, q & 3)] = rb[i];
      }
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int nk = (k_end - k_begin + kBK - 1) / kBK;
  if (nk > 0) {
    load_stage(k_begin);
    store_stage(0);
    if (nk > 1) load_stage(k_begin + kBK);
    lds_sync();
    for (int s = 0; s < nk; ++s) {
      const int buf = s & 1;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          uint4 v = As[buf][bswz(wm * 64 + i * 32 + fr, 2 * ks + fc)];
          fa[i] = __builtin_bit_cast(bf16x8_t, v);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint4 v = Bs[buf][bswz(wn * 64 + j * 32 + fr, 2 * ks + fc)];
          fb[j] = __builtin_bit_cast(bf16x8_t, v);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      if (s + 1 < nk) {
        store_stage(buf ^ 1);
        if (s + 2 < nk) load_stage(k_begin + (s + 2) * kBK);
      }
      lds_sync();
    }
  }

  // ---- epilogue: element q of a fragment is row 8 (q / 4) + 4 fc + q % 4,
  // column fr ----
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + fr;
      if (col >= p.N) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int lr = wm * 64 + i * 32 + (q >> 2) * 8 + fc * 4 + (q & 3);
        if (lr >= rows_valid) continue;
        const float v = acc[i][j][q];
        if constexpr (SEGK) {
          p.Cf[static_cast<size_t>(e) * p.c_estride + static_cast<size_t>(row0 + lr) * p.ldc + col] = v;
        } else if constexpr (MODE == BWD_FWD) {
          // recomputed pre-activation, kept in fp32 (+ bias)
          p.Cf[static_cast<size_t>(row0 + lr) * p.ldc + col] = p.bias ? v + p.bias[static_cast<size_t>(e) * p.N + col] : v;
        } else {
          const size_t o = static_cast<size_t>(row0 + lr) * p.ldc + col;
          // O1, O2 (the dh outputs) may have their own row stride
          const size_t od = p.ldo ? static_cast<size_t>(row0 + lr) * p.ldo + col : o;
          if constexpr (EPI == BWD_EPI_STORE) {
            p.O1[od] = f32_to_bf16(v);
          } else if constexpr (EPI == BWD_EPI_SWIGLU) {
            const float h1 = p.H1[o], h3 = p.H3[o];
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * h1));
            const float si = h1 * sg;
            p.O1[od] = f32_to_bf16(v * h3 * sg * (1.0f + h1 * (1.0f - sg)));
            p.O2[od] = f32_to_bf16(v * si);
            p.O3[o] = f32_to_bf16(si * h3);
          } else if constexpr (EPI == BWD_EPI_RELU) {
            const float h = p.H1[o];
            p.O1[od] = f32_to_bf16(h > 0.f ? v : 0.f);
            p.O3[o] = f32_to_bf16(fmaxf(h, 0.f));
          } else {   // BWD_EPI_GELU
            const float h = p.H1[o];
            p.O1[od] = f32_to_bf16(v * gelu_grad_f32(h));
            p.O3[o] = f32_to_bf16(gelu_f32(h));
          }
        }
      }
    }
}

int launch_bwd_gemm(int mode, int epi, const BwdGemmParams& p, int m_tiles_max, hipStream_t stream) {
  const long n_tiles = (p.N + kBN - 1) / kBN;
  long tiles = mode == BWD_WGRAD ? static_cast<long>(p.E) * ((p.M + kBM - 1) / kBM) * n_tiles
                                 : static_cast<long>(m_tiles_max) * n_tiles;
  long blocks = (tiles + kBxcds - 1) / kBxcds * kBxcds;
  if (blocks <= 0) return MOE_OK;
  if (blocks > 0x7fffffffL) return MOE_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kBT);
  if (mode == BWD_WGRAD) {
    hipLaunchKernelGGL((bwd_gemm_kernel<BWD_WGRAD, BWD_EPI_STORE>), grid, block, 0, stream, p);
  } else if (mode == BWD_FWD) {
    hipLaunchKernelGGL((bwd_gemm_kernel<BWD_FWD, BWD_EPI_STORE>), grid, block, 0, stream, p);
  } else {
    switch (epi) {
      case BWD_EPI_SWIGLU: hipLaunchKernelGGL((bwd_gemm_kernel<BWD_DGRAD, BWD_EPI_SWIGLU>), grid, block, 0, stream, p); break;
      case BWD_EPI_RELU: hipLaunchKernelGGL((bwd_gemm_kernel<BWD_DGRAD, BWD_EPI_RELU>), grid, block, 0, stream, p); break;
      case BWD_EPI_GELU: hipLaunchKernelGGL((bwd_gemm_kernel<BWD_DGRAD, BWD_EPI_GELU>), grid, block, 0, stream, p); break;
      default: hipLaunchKernelGGL((bwd_gemm_kernel<BWD_DGRAD, BWD_EPI_STORE>), grid, block, 0, stream, p); break;
    }
  }
  return check_launch();
}

}  // namespace moe
