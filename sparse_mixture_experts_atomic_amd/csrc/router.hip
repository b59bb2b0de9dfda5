// (a) Router: logits z = x W_g^T (+ b_g) in fp32, softmax in fp32, top-k,
// gate weights, and per-block column sums of the probabilities.
//
// P4 公式：三步走 (router score W_g x, W_g shaped experts x width); P5
// 选择性精度 (the router softmax is computed in float32); P1 §3.3, P2 §2.1,
// P3 §3.1 (keep the k largest, optionally renormalised).
#include <math.h>

#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kRtTok = 32;       // tokens per block
constexpr int kRtExp = 64;       // experts per inner group
constexpr int kRtDc = 32;        // columns of d per LDS chunk
constexpr int kRtThreads = 256;
constexpr int kRtMaxE = 256;   // logits of a block stay in LDS
constexpr int kRtMaxK = 64;    // one selected slot per lane

struct RouterArgs {
  const void* x;
  const float* w_g;
  const float* b_g;
  int T, d, E, k, mode;
  int32_t* topk_idx;
  float* topk_gate;
  float* colsum_part;   // [gridDim.x, E]
  float* logits_dbg;
};

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// fp32 softmax and top-k of one token's logits z[0..E) by one wavefront:
// expert e lives on lane e % 64, slot e / 64; k rounds of a wavefront arg-max
// (largest logit, lower id on ties), the winning lane marks its slot taken.
// Adds the probabilities to wcol[0..E) and writes the outputs of token t.
__device__ __forceinline__ void token_softmax_topk(const float* z, int t, const RouterArgs& a, float* wcol,
                                                   int lane) {
  float m = -INFINITY;
  for (int e = lane; e < a.E; e += 64) m = fmaxf(m, z[e]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float s = 0.f;
  for (int e = lane; e < a.E; e += 64) s += expf(z[e] - m);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  const float inv = 1.0f / s;
  for (int e = lane; e < a.E; e += 64) {
    if (a.logits_dbg) a.logits_dbg[static_cast<size_t>(t) * a.E + e] = z[e];
    wcol[e] += expf(z[e] - m) * inv;
  }
  uint32_t taken = 0;
  float myp = 0.f;
  int myi = 0;
  float psum = 0.f;
  for (int j = 0; j < a.k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int e = lane, i = 0; e < a.E; e += 64, ++i) {
      if (!((taken >> i) & 1u) && better(z[e], e, bv, bi)) { bv = z[e]; bi = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    const float p = expf(bv - m) * inv;
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) { myp = p; myi = bi; }
    psum += p;
  }
  if (lane < a.k) {
    const size_t o = static_cast<size_t>(t) * a.k + lane;
    a.topk_idx[o] = myi;
    a.topk_gate[o] = a.mode == MOE_GATE_RENORM ? myp / psum : myp;
  }
}

// One block = 32 tokens x all E experts.  Logits are accumulated in
// registers (2 tokens x 4 experts per thread per 64-expert group) from LDS
// tiles of x and W_g, then kept in LDS for the softmax/top-k phase, which
// runs one wavefront per token.
template <typename XT>
__global__ __launch_bounds__(kRtThreads) void router_generic_kernel(RouterArgs a) {
  extern __shared__ float smem[];
  float* xs = smem;                          // [kRtDc][kRtTok]
  float* ws = xs + kRtDc * kRtTok;           // [kRtDc][kRtExp]
  float* lg = ws + kRtDc * kRtExp;           // [kRtTok][E]
  float* wcol = lg + kRtTok * a.E;           // [4 waves][E] probability partial sums

  const XT* x = static_cast<const XT*>(a.x);
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRtTok;
  const int tx = tid & 15;                   // expert quad
  const int ty = tid >> 4;                   // token pair

  for (int eg = 0; eg < a.E; eg += kRtExp) {
    // each 32-column chunk is summed in fp32, the running total in fp64, so
    // the rounding error does not grow with d the way one long fp32 chain does
    double tot[2][4] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
    for (int c0 = 0; c0 < a.d; c0 += kRtDc) {
      float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      // x chunk: 32 tokens x 32 columns, 4 per thread, stored column-major
      {
        int t = tid >> 3, c = (tid & 7) * 4;
        int tg = t0 + t;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int cg = c0 + c + i;
          float v = 0.f;
          if (tg < a.T && cg < a.d) v = Elem<XT>::load(x, static_cast<size_t>(tg) * a.d + cg);
          xs[(c + i) * kRtTok + t] = v;
        }
      }
      // W_g chunk: 64 experts x 32 columns, 8 per thread
      {
        int e = tid >> 2, c = (tid & 3) * 8;
        int eg2 = eg + e;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          int cg = c0 + c + i;
          float v = 0.f;
          if (eg2 < a.E && cg < a.d) v = a.w_g[static_cast<size_t>(eg2) * a.d + cg];
          ws[(c + i) * kRtExp + e] = v;
        }
      }
      __syncthreads();
#pragma unroll 8
      for (int c = 0; c < kRtDc; ++c) {
        float x0 = xs[c * kRtTok + ty * 2];
        float x1 = xs[c * kRtTok + ty * 2 + 1];
        float4 w = *reinterpret_cast<const float4*>(&ws[c * kRtExp + tx * 4]);
        acc[0][0] = fmaf(x0, w.x, acc[0][0]);
        acc[0][1] = fmaf(x0, w.y, acc[0][1]);
        acc[0][2] = fmaf(x0, w.z, acc[0][2]);
        acc[0][3] = fmaf(x0, w.w, acc[0][3]);
        acc[1][0] = fmaf(x1, w.x, acc[1][0]);
        acc[1][1] = fmaf(x1, w.y, acc[1][1]);
        acc[1][2] = fmaf(x1, w.z, acc[1][2]);
        acc[1][3] = fmaf(x1, w.w, acc[1][3]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) tot[i][j] += static_cast<double>(acc[i][j]);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int e = eg + tx * 4 + j;
        if (e < a.E) {
          float v = static_cast<float>(tot[i][j]);
          if (a.b_g) v += a.b_g[e];
          lg[(ty * 2 + i) * a.E + e] = v;
        }
      }
  }
  __syncthreads();

  // softmax + top-k: one wavefront per token
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int e = lane; e < a.E; e += 64) wcol[wave * a.E + e] = 0.f;
  for (int tl = wave; tl < kRtTok; tl += kRtThreads / 64) {
    const int t = t0 + tl;
    if (t >= a.T) break;
    token_softmax_topk(lg + tl * a.E, t, a, wcol + wave * a.E, lane);
  }
  __syncthreads();
  // per-block probability column sums, fixed order over the 4 waves
  for (int e = tid; e < a.E; e += kRtThreads) {
    float v = wcol[e] + wcol[a.E + e] + wcol[2 * a.E + e] + wcol[3 * a.E + e];
    a.colsum_part[static_cast<size_t>(blockIdx.x) * a.E + e] = v;
  }
}

// Streaming router for few experts (E <= 8), bf16 activations, d % 8 == 0,
// d <= 4096.  The work is bound by reading x once.  A block of 512 threads is
// split into token lanes of TPR threads; thread c of a lane keeps the fp32
// router weights of column chunk c (8 columns x 8 experts) in registers and
// streams the lane's tokens in halves of kSmTph: one 16-byte load and 64 FMAs
// per token, the next half's loads in flight while the current half is
// reduced.  The kSmTph x 8 per-thread partial logits of a half are
// reduce-scattered over the wavefront (each lane ends with one sum), the
// TPR / 64 wavefronts of a lane are added in LDS in a fixed order, and one
// thread per token does the fp32 softmax and top-k.  Per-block probability
// column sums go to the workspace for colsum_reduce_kernel.
constexpr int kSmE = 8;
constexpr int kSmThreads = 512;
constexpr int kSmTph = 8;                     // tokens per thread and half
constexpr int kSmHalves = 2;
constexpr int kSmTpt = kSmTph * kSmHalves;    // tokens per thread
constexpr int kSmNv = kSmTph * kSmE;          // partial logits per thread and half (64)

template <int TPR>
__global__ __launch_bounds__(kSmThreads) void router_stream_kernel(RouterArgs a) {
  constexpr int G = kSmThreads / TPR;         // token lanes per block
  constexpr int WPL = TPR / 64;               // wavefronts per token lane
  constexpr int TPB = G * kSmTpt;             // tokens per block
  static_assert(kSmNv == 64, "one reduced value per lane");
  __shared__ float wred[kSmHalves][kSmThreads / 64][kSmNv];
  __shared__ float lg[TPB][kSmE];
  __shared__ float pr[TPB][kSmE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = tid % TPR;                    // column chunk
  const int g = tid / TPR;                    // token lane
  const int nchunk = a.d / 8;
  const int t0 = blockIdx.x * TPB;
  const int tl0 = t0 + g * kSmTpt;            // first token of this lane
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const bool cv = c < nchunk;

  auto load_half = [&](int h, uint4 (&dst)[kSmTph]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kSmTph; ++i) {
      const int t = tl0 + h * kSmTph + i;
      dst[i] = (cv && t < a.T) ? *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * a.d + c * 8)
                               : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  uint4 xa[kSmTph], xb[kSmTph];
  load_half(0, xa);
  float w[kSmE][8];
#pragma unroll
  for (int e = 0; e < kSmE; ++e) {
    if (cv && e < a.E) {
      const float4 lo = *reinterpret_cast<const float4*>(a.w_g + static_cast<size_t>(e) * a.d + c * 8);
      const float4 hi = *reinterpret_cast<const float4*>(a.w_g + static_cast<size_t>(e) * a.d + c * 8 + 4);
      w[e][0] = lo.x; w[e][1] = lo.y; w[e][2] = lo.z; w[e][3] = lo.w;
      w[e][4] = hi.x; w[e][5] = hi.y; w[e][6] = hi.z; w[e][7] = hi.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) w[e][q] = 0.f;
    }
  }
  load_half(1, xb);
  auto half = [&](int h, const uint4 (&xv)[kSmTph]) __attribute__((always_inline)) {
    float v[kSmNv];                           // entry i * 8 + e
#pragma unroll
    for (int i = 0; i < kSmTph; ++i) {
      const uint32_t q[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
      float xf[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        xf[2 * m] = __uint_as_float(q[m] << 16);
        xf[2 * m + 1] = __uint_as_float(q[m] & 0xffff0000u);
      }
#pragma unroll
      for (int e = 0; e < kSmE; ++e) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) s = fmaf(xf[m], w[e][m], s);
        v[i * kSmE + e] = s;
      }
    }
    // reduce-scatter over the wavefront: in the round with partner lane ^ o
    // the lane keeps the upper half of its entries if (lane & o), so after
    // the six rounds lane l holds entry l summed over all 64 lanes
#pragma unroll
    for (int r = 0; r < 6; ++r) {
      const int o = 32 >> r;
      const int n = kSmNv >> (r + 1);
      const bool upper = (lane & o) != 0;
#pragma unroll
      for (int i = 0; i < n; ++i) {
        const float send = upper ? v[i] : v[i + n];
        const float keep = upper ? v[i + n] : v[i];
        v[i] = keep + __shfl_xor(send, o);
      }
    }
    wred[h][wave][lane] = v[0];
  };
  half(0, xa);
  half(1, xb);
  __syncthreads();
  // logits: token lane gg, half h, entry en = i * 8 + e, summed over the
  // lane's wavefronts
  for (int j = tid; j < kSmHalves * G * kSmNv; j += kSmThreads) {
    const int h = j / (G * kSmNv);
    const int gg = (j / kSmNv) % G, en = j % kSmNv;
    float sum = 0.f;
#pragma unroll
    for (int ww = 0; ww < WPL; ++ww) sum += wred[h][gg * WPL + ww][en];
    const int e = en % kSmE;
    lg[gg * kSmTpt + h * kSmTph + en / kSmE][e] = sum + ((a.b_g && e < a.E) ? a.b_g[e] : 0.f);
  }
  __syncthreads();
  if (tid < TPB) {
    const int t = t0 + tid;
    const float* z = lg[tid];
    float p[kSmE];
    for (int e = 0; e < kSmE; ++e) p[e] = 0.f;
    if (t < a.T) {
      float m = -INFINITY;
      for (int e = 0; e < a.E; ++e) m = fmaxf(m, z[e]);
      float s = 0.f;
      for (int e = 0; e < a.E; ++e) { p[e] = expf(z[e] - m); s += p[e]; }
      const float inv = 1.0f / s;
      for (int e = 0; e < a.E; ++e) {
        p[e] *= inv;
        if (a.logits_dbg) a.logits_dbg[static_cast<size_t>(t) * a.E + e] = z[e];
      }
      // top-k by repeated selection (largest logit, lower index on ties)
      uint32_t taken = 0;
      float psum = 0.f;
      float ps[kSmE];
      int is[kSmE];
      for (int j = 0; j < a.k; ++j) {
        int bi = -1;
        float bv = -INFINITY;
        for (int e = 0; e < a.E; ++e)
          if (!((taken >> e) & 1u) && (bi < 0 || z[e] > bv)) { bv = z[e]; bi = e; }
        taken |= 1u << bi;
        is[j] = bi;
        ps[j] = p[bi];
        psum += p[bi];
      }
      for (int j = 0; j < a.k; ++j) {
        a.topk_idx[static_cast<size_t>(t) * a.k + j] = is[j];
        a.topk_gate[static_cast<size_t>(t) * a.k + j] = a.mode == MOE_GATE_RENORM ? ps[j] / psum : ps[j];
      }
    }
    for (int e = 0; e < kSmE; ++e) pr[tid][e] = p[e];
  }
  __syncthreads();
  // block column sums in token order
  if (tid < a.E) {
    float cs = 0.f;
    for (int i = 0; i < TPB; ++i) cs += pr[i][tid];
    a.colsum_part[static_cast<size_t>(blockIdx.x) * a.E + tid] = cs;
  }
}

// MFMA router for bf16 activations.  W_g is split exactly into three bf16
// planes, w = hi + mid + lo, each the truncation of what the previous ones
// leave (a float's 24-bit significand in three 8-bit pieces), so every
// product with a bf16 x is exact and the logits are fp32 sums as in the VALU
// kernels.  A block takes 16 TG tokens and NE groups of 16 experts per pass;
// its 8 wavefronts split K by 32-column steps (wavefront w takes steps w,
// w + 8, ...) and keep kMfPd steps of loads in flight: per step a 16-byte x
// fragment per token group (v_mfma_f32_16x16x32_bf16 A operand: token lane %
// 16, columns 8 (lane / 16) ..) and 32 bytes of fp32 W_g per expert group (B
// operand: expert lane % 16, same columns), split in registers.  The
// wavefronts' partial logits are added in LDS in wavefront order, then one
// wavefront per token does the fp32 softmax and top-k, and per-block
// probability column sums go to the workspace.
constexpr int kMfWaves = 8;
constexpr int kMfThreads = 64 * kMfWaves;
constexpr int kMfPd = 4;                      // k-steps of loads in flight

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_mf;

// bf16 pair (lo in bits 0-15) from the high halves of two words
__device__ __forceinline__ uint32_t hi16_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// three exact bf16 planes of 8 fp32 values
__device__ __forceinline__ void split3(const float4& w0, const float4& w1, bf16x8_t& hi, bf16x8_t& mid,
                                       bf16x8_t& lo) {
  const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  uint32_t h[8], m[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = __float_as_uint(w[i]) & 0xffff0000u;
    const float r = w[i] - __uint_as_float(h[i]);          // exact
    m[i] = __float_as_uint(r) & 0xffff0000u;
    l[i] = __float_as_uint(r - __uint_as_float(m[i]));     // exact; fits in bf16
  }
  uint4 ph, pm, pl;
  ph.x = hi16_pair(h[0], h[1]); ph.y = hi16_pair(h[2], h[3]); ph.z = hi16_pair(h[4], h[5]); ph.w = hi16_pair(h[6], h[7]);
  pm.x = hi16_pair(m[0], m[1]); pm.y = hi16_pair(m[2], m[3]); pm.z = hi16_pair(m[4], m[5]); pm.w = hi16_pair(m[6], m[7]);
  pl.x = hi16_pair(l[0], l[1]); pl.y = hi16_pair(l[2], l[3]); pl.z = hi16_pair(l[4], l[5]); pl.w = hi16_pair(l[6], l[7]);
  hi = __builtin_bit_cast(bf16x8_t, ph);
  mid = __builtin_bit_cast(bf16x8_t, pm);
  lo = __builtin_bit_cast(bf16x8_t, pl);
}

template <int TG, int NE>
__global__ __launch_bounds__(kMfThreads) void router_mfma_kernel(RouterArgs a) {
  constexpr int TPB = 16 * TG;                // tokens per block
  constexpr int EC = 16 * NE;                 // experts per pass
  extern __shared__ float smem[];
  float* part = smem;                         // [kMfWaves][TPB][EC]
  float* lg = part + kMfWaves * TPB * EC;     // [TPB][E]
  float* wcol = lg + TPB * a.E;               // [kMfWaves][E]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 8;             // first column of the lane within a step
  const int t0 = blockIdx.x * TPB;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const int nks = (a.d + 31) / 32;
  const int my = nks > wave ? (nks - wave + kMfWaves - 1) / kMfWaves : 0;   // k-steps of this wavefront

  for (int e0 = 0; e0 < a.E; e0 += EC) {
    uint4 xb[kMfPd][TG];
    float4 wb[kMfPd][NE][2];
    auto load = [&](int i, uint4 (&xs)[TG], float4 (&ws)[NE][2]) __attribute__((always_inline)) {
      const int col = (wave + i * kMfWaves) * 32 + kq;
      const bool kv = i < my && col < a.d;    // d % 8 == 0: a lane's 8 columns are all in or all out
#pragma unroll
      for (int g = 0; g < TG; ++g) {
        const int t = t0 + g * 16 + r16;
        xs[g] = (kv && t < a.T) ? *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * a.d + col)
                                : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int n = 0; n < NE; ++n) {
        const int e = e0 + n * 16 + r16;
        if (kv && e < a.E) {
          const float4* src = reinterpret_cast<const float4*>(a.w_g + static_cast<size_t>(e) * a.d + col);
          ws[n][0] = src[0];
          ws[n][1] = src[1];
        } else {
          ws[n][0] = make_float4(0.f, 0.f, 0.f, 0.f);
          ws[n][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    };
    f32x4_mf acc[TG][NE];
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
      for (int n = 0; n < NE; ++n) acc[g][n] = f32x4_mf{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMfPd; ++j) load(j, xb[j], wb[j]);
    for (int i0 = 0; i0 < my; i0 += kMfPd) {
#pragma unroll
      for (int j = 0; j < kMfPd; ++j) {
        if (i0 + j < my) {
#pragma unroll
          for (int n = 0; n < NE; ++n) {
            bf16x8_t hi, mid, lo;
            split3(wb[j][n][0], wb[j][n][1], hi, mid, lo);
#pragma unroll
            for (int g = 0; g < TG; ++g) {
              const bf16x8_t xv = __builtin_bit_cast(bf16x8_t, xb[j][g]);
              acc[g][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, hi, acc[g][n], 0, 0, 0);
              acc[g][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, mid, acc[g][n], 0, 0, 0);
              acc[g][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, lo, acc[g][n], 0, 0, 0);
            }
          }
          load(i0 + j + kMfPd, xb[j], wb[j]);
        }
      }
    }
    // partial logits: lane holds expert n*16 + lane % 16 of tokens g*16 + 4 (lane / 16) + q
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
      for (int n = 0; n < NE; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          part[(wave * TPB + g * 16 + (lane >> 4) * 4 + q) * EC + n * 16 + r16] = acc[g][n][q];
    __syncthreads();
    for (int j = tid; j < TPB * EC; j += kMfThreads) {
      const int tl = j / EC, ec = j % EC, e = e0 + ec;
      if (e < a.E) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kMfWaves; ++w) s += part[(w * TPB + tl) * EC + ec];
        lg[tl * a.E + e] = s + (a.b_g ? a.b_g[e] : 0.f);
      }
    }
    __syncthreads();
  }

  // softmax + top-k: one wavefront per token
  for (int e = lane; e < a.E; e += 64) wcol[wave * a.E + e] = 0.f;
  for (int tl = wave; tl < TPB; tl += kMfWaves) {
    const int t = t0 + tl;
    if (t >= a.T) break;
    token_softmax_topk(lg + tl * a.E, t, a, wcol + wave * a.E, lane);
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += kMfThreads) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kMfWaves; ++w) v += wcol[w * a.E + e];
    a.colsum_part[static_cast<size_t>(blockIdx.x) * a.E + e] = v;
  }
}

// prob_colsum[e] = sum over blocks of the partial sums.  One block per
// expert: strided partial sums in double, then a fixed-order tree, so the
// result is deterministic and does not drift with the block count.
__global__ __launch_bounds__(256) void colsum_reduce_kernel(const float* part, int nb, int E, float* out) {
  __shared__ double red[256];
  const int e = blockIdx.x;
  double s = 0.0;
  for (int b = threadIdx.x; b < nb; b += 256) s += static_cast<double>(part[static_cast<size_t>(b) * E + e]);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[e] = static_cast<float>(red[0]);
}

inline int router_blocks(int T) { return (T + kRtTok - 1) / kRtTok; }

// block count of the streaming kernel for d columns (threads per token
// lane: a power of two >= 64 covering the d/8 chunks)
inline int stream_tpr(int d) {
  int tpr = 64;
  while (tpr < d / 8) tpr *= 2;
  return tpr;
}
inline int stream_blocks(int T, int d) {
  const int tpb = (kSmThreads / stream_tpr(d)) * kSmTpt;
  return (T + tpb - 1) / tpb;
}

// upper bound of the block count of either router kernel (per-block
// probability partial sums live in the workspace)
inline int router_max_blocks(int T) {
  const int small = (T + kSmTpt - 1) / kSmTpt;   // stream and MFMA kernels: at least 16 tokens per block
  const int generic = router_blocks(T);
  return small > generic ? small : generic;
}


// token groups of 16 per block of the MFMA router: enough blocks for the
// CUs, more tokens per block (fewer W_g reads) for long batches
inline int mfma_tg(int T) { return T >= 16384 ? 4 : (T >= 8192 ? 2 : 1); }
// expert groups of 16 per pass (TG * NE <= 8 keeps the partial sums in LDS)
inline int mfma_ne(int E, int tg) {
  int ne = (E + 15) / 16;
  ne = ne >= 4 ? 4 : (ne >= 2 ? 2 : 1);
  while (tg * ne > 8) ne /= 2;
  return ne;
}
inline size_t mfma_lds_bytes(int tg, int ne, int E) {
  return (static_cast<size_t>(kMfWaves) * 16 * tg * 16 * ne + static_cast<size_t>(16) * tg * E +
          static_cast<size_t>(kMfWaves) * E) * sizeof(float);
}
template <int TG, int NE>
int launch_mfma(const RouterArgs& a, int nb, size_t lds, hipStream_t stream) {
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&router_mfma_kernel<TG, NE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) {
      record_hip_error(e);
      return MOE_ERR_HIP;
    }
  }
  hipLaunchKernelGGL((router_mfma_kernel<TG, NE>), dim3(nb), dim3(kMfThreads), lds, stream, a);
  return check_launch();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_router_workspace_size(int T, int d, int E, int x_dt) {
  (void)d;
  (void)x_dt;
  if (T < 0 || E < 1) return 0;
  return align_up(static_cast<size_t>(router_max_blocks(T)) * E * sizeof(float), kWsAlign);
}

int moe_router_topk(const void* x, int x_dt, const float* w_g, const float* b_g, int T, int d, int E,
                    int k, int gate_mode, int32_t* topk_idx, float* topk_gate, float* prob_colsum,
                    float* logits_dbg, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || d < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > kRtMaxE || k > kRtMaxK) return MOE_ERR_UNSUPPORTED;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (gate_mode != MOE_GATE_PROB && gate_mode != MOE_GATE_RENORM) return MOE_ERR_INVALID_ARG;
  if (!w_g || !aligned16(w_g) || (b_g && !aligned16(b_g))) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x || !topk_idx || !topk_gate)) return MOE_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || (topk_idx && !aligned16(topk_idx)) || (topk_gate && !aligned16(topk_gate)) ||
      (prob_colsum && !aligned16(prob_colsum)) || (logits_dbg && !aligned16(logits_dbg)))
    return MOE_ERR_INVALID_ARG;
  const size_t need = moe_router_workspace_size(T, d, E, x_dt);
  if (prob_colsum && (!workspace || workspace_bytes < need || !aligned16(workspace))) return MOE_ERR_WORKSPACE;
  if (T > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return MOE_ERR_WORKSPACE;

  // bf16: the streaming VALU kernel for up to 8 experts (bound by reading x
  // once), the MFMA kernel beyond; fp32 activations: the generic kernel
  const bool small = x_dt == MOE_BF16 && E <= kSmE && d % 8 == 0 && d <= 8 * kSmThreads;
  const bool mf = x_dt == MOE_BF16 && !small;
  float* part = static_cast<float*>(workspace);
  const int tg = mfma_tg(T);
  const int ne = mfma_ne(E, tg);
  const int nb = small ? stream_blocks(T, d) : (mf ? (T + 16 * tg - 1) / (16 * tg) : router_blocks(T));
  if (T > 0 && small) {
    RouterArgs a{x, w_g, b_g, T, d, E, k, gate_mode, topk_idx, topk_gate, part, logits_dbg};
    const int tpr = stream_tpr(d);
    if (tpr == 64)
      hipLaunchKernelGGL(router_stream_kernel<64>, dim3(nb), dim3(kSmThreads), 0, stream, a);
    else if (tpr == 128)
      hipLaunchKernelGGL(router_stream_kernel<128>, dim3(nb), dim3(kSmThreads), 0, stream, a);
    else if (tpr == 256)
      hipLaunchKernelGGL(router_stream_kernel<256>, dim3(nb), dim3(kSmThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(router_stream_kernel<512>, dim3(nb), dim3(kSmThreads), 0, stream, a);
    int st = check_launch();
    if (st != MOE_OK) return st;
  }
  if (T > 0 && mf) {
    RouterArgs a{x, w_g, b_g, T, d, E, k, gate_mode, topk_idx, topk_gate, part, logits_dbg};
    const size_t lds = mfma_lds_bytes(tg, ne, E);
    int st = MOE_OK;
#define MOE_RT_MF(TG_, NE_) \
  if (tg == TG_ && ne == NE_) st = launch_mfma<TG_, NE_>(a, nb, lds, stream);
    MOE_RT_MF(1, 1) MOE_RT_MF(1, 2) MOE_RT_MF(1, 4) MOE_RT_MF(2, 1) MOE_RT_MF(2, 2) MOE_RT_MF(2, 4)
    MOE_RT_MF(4, 1) MOE_RT_MF(4, 2)
#undef MOE_RT_MF
    if (st != MOE_OK) return st;
  }
  if (T > 0 && !small && !mf) {
    RouterArgs a{x, w_g, b_g, T, d, E, k, gate_mode, topk_idx, topk_gate, part, logits_dbg};
    size_t lds = (static_cast<size_t>(kRtDc) * kRtTok + static_cast<size_t>(kRtDc) * kRtExp +
                  static_cast<size_t>(kRtTok) * E + 4 * static_cast<size_t>(E)) * sizeof(float);
    if (x_dt == MOE_F32)
      hipLaunchKernelGGL(router_generic_kernel<float>, dim3(nb), dim3(kRtThreads), lds, stream, a);
    else
      hipLaunchKernelGGL(router_generic_kernel<uint16_t>, dim3(nb), dim3(kRtThreads), lds, stream, a);
    int st = check_launch();
    if (st != MOE_OK) return st;
  }
  if (prob_colsum) {
    hipLaunchKernelGGL(colsum_reduce_kernel, dim3(E), dim3(256), 0, stream,
                       static_cast<const float*>(part), nb, E, prob_colsum);
    int st = check_launch();
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

}  // extern "C"
