// (a) Router: logits z = x W_g^T (+ b_g) in fp32, softmax in fp32, top-k,
// gate weights, and per-block column sums of the probabilities.
//
// P4 公式：三步走 (router score W_g x, W_g shaped experts x width); P5
// 选择性精度 (the router softmax is computed in float32); P1 §3.3, P2 §2.1,
// P3 §3.1 (keep the k largest, optionally renormalised).
#include <math.h>

#include <algorithm>
#include <mutex>

#include "moe_internal.hpp"

// Scratch of moe_router_topk_noalloc: the per-block probability column sums
// and (more than 8 experts) the partial logits, in a fixed device array
// instead of a caller workspace.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code this name is only a stand-in
// for the symbol: the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

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
  // noisy gating: z += noise[t, e] * (softplus((x W_n^T)[t, e] + b_n[e]) + eps)
  const float* w_n;
  const float* b_n;
  const float* noise;   // [T, E] standard normal draws, or nullptr: drawn here
  float eps;
  unsigned long long seed, offset;   // the counter-based stream of the draws
};

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
// As Easy as 1, 2, 3", SC 2011, section 5): ten rounds over a 128-bit
// counter under a 64-bit key; each round multiplies words 0 and 2 by fixed
// 32-bit multipliers, keeps the low halves, xors the high halves into the
// other two words with the key, and permutes; the key takes a Weyl step
// between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3, uint32_t k0,
                                              uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint32_t hi0 = __umulhi(kM0, c0), lo0 = kM0 * c0;
    const uint32_t hi1 = __umulhi(kM1, c2), lo1 = kM1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
}

// Box-Muller pair from two output words: u1, u2 = (word + 1/2) 2^-32 and
// sqrt(-2 ln u1) times cos (even draw) and sin (odd draw) of 2 pi u2, in
// fp64, each rounded once to fp32
__device__ __forceinline__ void box_muller_pair(uint32_t wa, uint32_t wb, float& even, float& odd) {
  const double u1 = (static_cast<double>(wa) + 0.5) * 0x1p-32;
  const double u2 = (static_cast<double>(wb) + 0.5) * 0x1p-32;
  const double r = sqrt(-2.0 * log(u1));
  double sn, cs;
  sincospi(2.0 * u2, &sn, &cs);
  even = static_cast<float>(r * cs);
  odd = static_cast<float>(r * sn);
}

// The four draws 4 j .. 4 j + 3 of the stream (seed, offset): counter block
// j (counter words: j low, j high, offset low, offset high; key: seed low,
// seed high); draws 4 j, 4 j + 1 from words 0, 1 and 4 j + 2, 4 j + 3 from
// words 2, 3.
__device__ __forceinline__ void philox_normal4(unsigned long long seed, unsigned long long offset,
                                               unsigned long long j, float (&v)[4]) {
  uint32_t c0 = static_cast<uint32_t>(j), c1 = static_cast<uint32_t>(j >> 32);
  uint32_t c2 = static_cast<uint32_t>(offset), c3 = static_cast<uint32_t>(offset >> 32);
  philox4x32_10(c0, c1, c2, c3, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
  box_muller_pair(c0, c1, v[0], v[1]);
  box_muller_pair(c2, c3, v[2], v[3]);
}

// Standard normal draw i of the stream: draw i mod 4 of block i / 4 (one
// Box-Muller pair is computed)
__device__ __forceinline__ float philox_normal(unsigned long long seed, unsigned long long offset,
                                               unsigned long long i) {
  const unsigned long long j = i >> 2;
  uint32_t c0 = static_cast<uint32_t>(j), c1 = static_cast<uint32_t>(j >> 32);
  uint32_t c2 = static_cast<uint32_t>(offset), c3 = static_cast<uint32_t>(offset >> 32);
  philox4x32_10(c0, c1, c2, c3, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
  const bool second = (i >> 1) & 1;
  float even, odd;
  box_muller_pair(second ? c2 : c0, second ? c3 : c1, even, odd);
  return (i & 1) ? odd : even;
}

// the noisy gate's draw for flat index t E + e
__device__ __forceinline__ float gate_draw(const RouterArgs& a, size_t i) {
  return a.noise ? a.noise[i] : philox_normal(a.seed, a.offset, i);
}

// ln(1 + e^u) without overflow for large u or loss of the small term
__device__ __forceinline__ float softplus_f(float u) { return fmaxf(u, 0.f) + log1pf(expf(-fabsf(u))); }

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Wavefront reductions in DPP steps (gfx9): butterflies inside quads, row
// shifts by 4 and 8, then the row-15 and row-31 broadcasts; the result is in
// lane 63 and is read back as a uniform value.  Lanes whose source lies
// outside the row keep the identity passed as the old value.  Six ALU steps
// instead of six dependent cross-lane LDS round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float identity, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int identity, int v) {
  return __builtin_amdgcn_update_dpp(identity, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xb1>(-INFINITY, v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4e>(-INFINITY, v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x114>(-INFINITY, v));   // row_shr:4
  v = fmaxf(v, dpp_f<0x118>(-INFINITY, v));   // row_shr:8
  v = fmaxf(v, dpp_f<0x142>(-INFINITY, v));   // row_bcast:15
  v = fmaxf(v, dpp_f<0x143>(-INFINITY, v));   // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xb1>(0.f, v);
  v += dpp_f<0x4e>(0.f, v);
  v += dpp_f<0x114>(0.f, v);
  v += dpp_f<0x118>(0.f, v);
  v += dpp_f<0x142>(0.f, v);
  v += dpp_f<0x143>(0.f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& bi) {
  const float ov = dpp_f<CTRL>(-INFINITY, bv);
  const int oi = dpp_i<CTRL>(0x7fffffff, bi);
  if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
}
// largest value over the wavefront, lower index on ties; uniform result
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  argmax_step<0xb1>(bv, bi);
  argmax_step<0x4e>(bv, bi);
  argmax_step<0x114>(bv, bi);
  argmax_step<0x118>(bv, bi);
  argmax_step<0x142>(bv, bi);
  argmax_step<0x143>(bv, bi);
  bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 63));
  bi = __builtin_amdgcn_readlane(bi, 63);
}

// fp32 softmax and top-k of one token's logits z[0..E) by one wavefront:
// expert e lives on lane e % 64, slot e / 64; k rounds of a wavefront arg-max
// (largest logit, lower id on ties), the winning lane marks its slot taken.
// Adds the probabilities to wcol[0..E) and writes the outputs of token t.
__device__ __forceinline__ void token_softmax_topk(const float* z, int t, const RouterArgs& a, float* wcol,
                                                   int lane) {
  constexpr int S = kRtMaxE / 64;             // slots per lane
  float zr[S], ex[S];
#pragma unroll
  for (int i = 0; i < S; ++i) zr[i] = lane + 64 * i < a.E ? z[lane + 64 * i] : -INFINITY;
  float m = zr[0];
#pragma unroll
  for (int i = 1; i < S; ++i) m = fmaxf(m, zr[i]);
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    ex[i] = lane + 64 * i < a.E ? expf(zr[i] - m) : 0.f;
    s += ex[i];
  }
  s = wave_sum(s);
  const float inv = 1.0f / s;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int e = lane + 64 * i;
    if (e < a.E) {
      if (a.logits_dbg) a.logits_dbg[static_cast<size_t>(t) * a.E + e] = zr[i];
      wcol[e] += ex[i] * inv;
    }
  }
  uint32_t taken = 0;
  float myp = 0.f;
  int myi = 0;
  float psum = 0.f;
  for (int j = 0; j < a.k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int e = lane + 64 * i;
      if (e < a.E && !((taken >> i) & 1u) && better(zr[i], e, bv, bi)) { bv = zr[i]; bi = e; }
    }
    wave_argmax(bv, bi);
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

// fp32 softmax and top-k of one token's logits, E <= 8, by a group of 8
// consecutive lanes: lane e of the group holds logit z of expert e (-inf past
// E).  k rounds of a group arg-max (largest logit, lower id on ties); lane j
// of the group keeps the winner of round j.  Writes the outputs of token t
// when t < T and returns the lane's probability (0 past E or T).
__device__ __forceinline__ float token8_softmax_topk(float z, int e, int t, const RouterArgs& a) {
  if (t >= a.T) return 0.f;                   // whole groups leave together
  float m = z;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 8));
  const float ex = e < a.E ? expf(z - m) : 0.f;
  float s = ex;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) s += __shfl_xor(s, o, 8);
  const float p = ex * (1.0f / s);
  if (a.logits_dbg && e < a.E) a.logits_dbg[static_cast<size_t>(t) * a.E + e] = z;
  bool taken = e >= a.E;
  float psum = 0.f, myp = 0.f;
  int myi = 0;
  for (int j = 0; j < a.k; ++j) {
    float bv = taken ? -INFINITY : z;
    int bi = taken ? 0x7fffffff : e;
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const float ov = __shfl_xor(bv, o, 8);
      const int oi = __shfl_xor(bi, o, 8);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    const float pw = __shfl(p, bi, 8);        // probability of the winner
    if (bi == e) taken = true;
    if (e == j) { myp = pw; myi = bi; }
    psum += pw;
  }
  if (e < a.k) {
    const size_t o = static_cast<size_t>(t) * a.k + e;
    a.topk_idx[o] = myi;
    a.topk_gate[o] = a.mode == MOE_GATE_RENORM ? myp / psum : myp;
  }
  return p;
}

// All-reductions over a row of 16 lanes (gfx9 DPP: quad butterflies, then
// rotations by 4 and 8 within the row; every lane ends with the result).
template <int CTRL>
__device__ __forceinline__ float dpp_r(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_ri(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_r<0xb1>(v));
  v = fmaxf(v, dpp_r<0x4e>(v));
  v = fmaxf(v, dpp_r<0x124>(v));              // row_ror:4
  return fmaxf(v, dpp_r<0x128>(v));           // row_ror:8
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_r<0xb1>(v);
  v += dpp_r<0x4e>(v);
  v += dpp_r<0x124>(v);
  return v + dpp_r<0x128>(v);
}
template <int CTRL>
__device__ __forceinline__ void row16_argmax_step(float& bv, int& bi) {
  const float ov = dpp_r<CTRL>(bv);
  const int oi = dpp_ri<CTRL>(bi);
  if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
}
__device__ __forceinline__ void row16_argmax(float& bv, int& bi) {
  row16_argmax_step<0xb1>(bv, bi);
  row16_argmax_step<0x4e>(bv, bi);
  row16_argmax_step<0x124>(bv, bi);
  row16_argmax_step<0x128>(bv, bi);
}

// fp32 softmax and top-k of one token's logits z[0..E) by a row of 16 lanes
// (E <= 16 NS, k <= 16): lane l of the row holds experts l + 16 i.  k rounds
// of a row arg-max (largest logit, lower id on ties); lane j of the row keeps
// the winner of round j.  Writes the token's outputs and its probabilities
// to pr[0..E).  Four tokens per wavefront at once, where one token per
// wavefront left 48 of 64 lanes idle in every reduction.
template <int NS>
__device__ __forceinline__ void token16_softmax_topk(const float* z, int t, const RouterArgs& a, float* pr, int l) {
  float zr[NS], ex[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) zr[i] = l + 16 * i < a.E ? z[l + 16 * i] : -INFINITY;
  float m = zr[0];
#pragma unroll
  for (int i = 1; i < NS; ++i) m = fmaxf(m, zr[i]);
  m = row16_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    ex[i] = l + 16 * i < a.E ? expf(zr[i] - m) : 0.f;
    s += ex[i];
  }
  s = row16_sum(s);
  const float inv = 1.0f / s;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = l + 16 * i;
    if (e < a.E) {
      if (a.logits_dbg) a.logits_dbg[static_cast<size_t>(t) * a.E + e] = zr[i];
      pr[e] = ex[i] * inv;
    }
  }
  uint32_t taken = 0;
  float myp = 0.f, psum = 0.f;
  int myi = 0;
  for (int j = 0; j < a.k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int e = l + 16 * i;
      if (e < a.E && !((taken >> i) & 1u) && better(zr[i], e, bv, bi)) { bv = zr[i]; bi = e; }
    }
    row16_argmax(bv, bi);
    const float p = expf(bv - m) * inv;
    if ((bi & 15) == l) taken |= 1u << (bi >> 4);
    if (l == j) { myp = p; myi = bi; }
    psum += p;
  }
  if (l < a.k) {
    const size_t o = static_cast<size_t>(t) * a.k + l;
    a.topk_idx[o] = myi;
    a.topk_gate[o] = a.mode == MOE_GATE_RENORM ? myp / psum : myp;
  }
}

// One block = 32 tokens x all E experts.  Logits are accumulated in
// registers (2 tokens x 4 experts per thread per 64-expert group) from LDS
// tiles of x and W_g, then kept in LDS for the softmax/top-k phase, which
// runs one wavefront per token.
template <typename XT, bool NOISY>
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

  // logits of 32 tokens x experts [eg, eg + 64) against the rows of W: each
  // 32-column chunk is summed in fp32, the running total in fp64, so the
  // rounding error does not grow with d the way one long fp32 chain does
  auto logits = [&](const float* W, int eg, double (&tot)[2][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) tot[i][j] = 0.0;
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
          if (eg2 < a.E && cg < a.d) v = W[static_cast<size_t>(eg2) * a.d + cg];
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
  };

  for (int eg = 0; eg < a.E; eg += kRtExp) {
    double tot[2][4];
    logits(a.w_g, eg, tot);
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
    if constexpr (NOISY) {
      // the same thread owns the same logits in both passes
      logits(a.w_n, eg, tot);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = eg + tx * 4 + j;
          const int t = t0 + ty * 2 + i;
          if (e < a.E && t < a.T) {
            float u = static_cast<float>(tot[i][j]);
            if (a.b_n) u += a.b_n[e];
            lg[(ty * 2 + i) * a.E + e] += gate_draw(a, static_cast<size_t>(t) * a.E + e) * (softplus_f(u) + a.eps);
          }
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

// The MFMA routers split W_g exactly into three bf16 planes, w = hi + mid +
// lo, each the truncation of what the previous ones leave (a float's 24-bit
// significand in three 8-bit pieces), so every product with a bf16 x is
// exact and the logits are fp32 sums of exact products.
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_mf;

// bf16 pair (lo in bits 0-15) from the high halves of two words
__device__ __forceinline__ uint32_t hi16_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// the value of lane (l + 8) mod 16 of the same 16-lane row (DPP row_ror:8)
__device__ __forceinline__ float dpp_swap8(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, false));
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

// MFMA router for bf16 activations and at most 8 experts.  A block takes tg
// groups of 16 tokens; the kw wavefronts of a group split the columns into
// 128-column chunks, two per wavefront and round (wavefront j takes chunks j
// and j + kw of each run of 2 kw).  A chunk is four 32-column k-steps of
// v_mfma_f32_16x16x32_bf16 with the tokens as rows: a lane loads 16 bytes of
// x per k-step (token lane % 16, columns 8 (lane / 16) ..).  W_g is split
// exactly into bf16 planes (see split3); the first MFMA's B
// operand holds hi of expert n in column n < 8 and mid of expert n - 8 in
// column n >= 8, the second adds lo in columns < 8, so logit e is column e
// plus column e + 8.  Lanes n and n + 8 need the same eight fp32 values of
// W_g row n % 8: each loads one half (so that a wavefront's load covers eight
// whole 128-byte rows) and takes the other half from its partner by DPP.
// The W_g loads go out before the x loads and are split while x is in
// flight: moving W_g from L2 costs more than the split.  The wavefronts'
// partial logits are added in LDS in wavefront order; 8 lanes per token do
// the fp32 softmax and top-k.  NOISY: the noise projection W_n goes through
// the same steps into a second accumulator (one chunk per wavefront and
// round, so that both fit in registers), and the noisy logit is formed
// before the softmax.
constexpr int kM8MaxE = 8;
constexpr int kM8Cpw = 2;                     // chunks per wavefront and round
constexpr int kM8Waves = 16;                  // at most, per block
constexpr int kM8Tok = 16 * kM8Waves;         // at most, per block
constexpr int kCUs = 256;                     // compute units of an MI355X

template <bool NOISY>
__global__ __launch_bounds__(64 * kM8Waves) void router_mf8_kernel(RouterArgs a, int kw, int tg) {
  constexpr int CPW = NOISY ? 1 : kM8Cpw;     // chunks per wavefront and round
  constexpr int NM = NOISY ? 2 : 1;           // matrices: W_g (and W_n)
  __shared__ float part[NM][kM8Waves][16][16];
  __shared__ float lg[kM8Tok][kM8MaxE];
  __shared__ float pr[kM8Tok][kM8MaxE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nthr = 64 * kw * tg;
  const int tpb = 16 * tg;
  const int g = wave / kw;                    // token group
  const int kv = wave % kw;                   // column slot
  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 8;
  const int t0 = blockIdx.x * tpb;
  const int t = t0 + g * 16 + r16;
  const bool tv = t < a.T;
  const int e = r16 & 7;
  const bool ev = e < a.E;
  const bool hl = r16 < 8;
  // loads are unconditional (clamped rows and columns) so that the compiler
  // can wait for them one by one; W_g columns past d and rows past E are
  // zeroed after the load, rows of x past T only feed discarded logits
  const uint16_t* xr = static_cast<const uint16_t*>(a.x) + static_cast<size_t>(tv ? t : a.T - 1) * a.d;
  const size_t wrow = static_cast<size_t>(ev ? e : a.E - 1) * a.d;
  const float* wr[NM];
  wr[0] = a.w_g + wrow;
  if constexpr (NOISY) wr[NM - 1] = a.w_n + wrow;
  f32x4_mf acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = f32x4_mf{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < a.d; c0 += CPW * kw * 128) {
    float4 wb[NM][CPW][4];                    // columns 0-3 (lanes < 8) or 4-7 of the lane's eight
    uint4 xb[CPW][4];
    bool ok[CPW][4];
#pragma unroll
    for (int i = 0; i < CPW; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int col = c0 + (kv + i * kw) * 128 + s * 32 + kq;
        ok[i][s] = ev && col < a.d;           // d % 8 == 0: a lane's 8 columns are all in or all out
        const int cc = col < a.d ? col : a.d - 8;
#pragma unroll
        for (int m = 0; m < NM; ++m) wb[m][i][s] = *reinterpret_cast<const float4*>(wr[m] + cc + (hl ? 0 : 4));
      }
#pragma unroll
    for (int i = 0; i < CPW; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int col = c0 + (kv + i * kw) * 128 + s * 32 + kq;
        xb[i][s] = *reinterpret_cast<const uint4*>(xr + (col < a.d ? col : a.d - 8));
      }
    // every load of the round is in flight before the first use
    __builtin_amdgcn_sched_barrier(0);
    uint4 b1[NM][CPW][4], b2[NM][CPW][4];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < CPW; ++i)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          // lanes n and n + 8 hold the two halves of the same eight W_g values
          const float4 mine = wb[m][i][s];
          const float4 other = make_float4(dpp_swap8(mine.x), dpp_swap8(mine.y), dpp_swap8(mine.z), dpp_swap8(mine.w));
          bf16x8_t hi, mid, lo;
          split3(hl ? mine : other, hl ? other : mine, hi, mid, lo);
          const uint4 h = __builtin_bit_cast(uint4, hi), mm = __builtin_bit_cast(uint4, mid),
                      l = __builtin_bit_cast(uint4, lo);
          // a mask rather than a select of the loaded values, which the
          // compiler would turn into a conditional load waited for at once
          const uint32_t m1 = ok[i][s] ? ~0u : 0u, m2 = (ok[i][s] && hl) ? ~0u : 0u;
          b1[m][i][s] = hl ? h : mm;
          b1[m][i][s].x &= m1; b1[m][i][s].y &= m1; b1[m][i][s].z &= m1; b1[m][i][s].w &= m1;
          b2[m][i][s] = make_uint4(l.x & m2, l.y & m2, l.z & m2, l.w & m2);
        }
    // the planes are ready before the first wait for x
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < CPW; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8_t xv = __builtin_bit_cast(bf16x8_t, xb[i][s]);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, __builtin_bit_cast(bf16x8_t, b1[m][i][s]), acc[m], 0, 0, 0);
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, __builtin_bit_cast(bf16x8_t, b2[m][i][s]), acc[m], 0, 0, 0);
        }
      }
  }
  // lane holds column r16 of tokens 4 (lane / 16) + q of its group
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q) part[m][wave][(lane >> 4) * 4 + q][r16] = acc[m][q];
  __syncthreads();
  for (int j = tid; j < tpb * kM8MaxE; j += nthr) {
    const int tl = j / kM8MaxE, ee = j % kM8MaxE;
    float z = 0.f;
    if (ee < a.E) {
      const int gg = tl / 16, tr = tl % 16;
      for (int w = 0; w < kw; ++w) {
        const float* pp = part[0][gg * kw + w][tr];
        z += pp[ee] + pp[ee + 8];
      }
      if (a.b_g) z += a.b_g[ee];
      if constexpr (NOISY) {
        float zn = 0.f;
        for (int w = 0; w < kw; ++w) {
          const float* pp = part[NM - 1][gg * kw + w][tr];
          zn += pp[ee] + pp[ee + 8];
        }
        if (a.b_n) zn += a.b_n[ee];
        const int t = t0 + tl;
        if (t < a.T) z += gate_draw(a, static_cast<size_t>(t) * a.E + ee) * (softplus_f(zn) + a.eps);
      }
    }
    lg[tl][ee] = z;
  }
  __syncthreads();
  // groups of 8 lanes per token (the stride keeps groups whole)
  for (int j = tid; j < tpb * kM8MaxE; j += nthr) {
    const int tl = j / kM8MaxE, ee = j % kM8MaxE;
    pr[tl][ee] = token8_softmax_topk(ee < a.E ? lg[tl][ee] : -INFINITY, ee, t0 + tl, a);
  }
  __syncthreads();
  // block column sums in token order
  if (tid < a.E) {
    float cs = 0.f;
    for (int i = 0; i < tpb; ++i) cs += pr[i][tid];
    a.colsum_part[static_cast<size_t>(blockIdx.x) * a.E + tid] = cs;
  }
}

// Router logits for bf16 activations and more than 8 experts as a tiled
// GEMM.  A block takes BM tokens x 64 experts x one slice of K; W_g is split
// exactly into its three bf16 planes (see split3) once per
// block and 64-column chunk, into LDS, where every token of the block uses
// it, and x is staged beside it.  Four wavefronts of (BM / 2) tokens x 32
// experts run v_mfma_f32_16x16x32_bf16 (one per plane).  The slice's partial
// logits go to part[slice][t][e]; router_finish_kernel adds the slices.
// The E rows are those of W_g stacked on those of the noise projection W_n:
// rows e < E1 come from W_g, the others from row e - E1 of W_n (E1 = E for
// the clean router, E = 2 E1 for noisy gating; the noisy router takes this
// kernel for any number of experts).
constexpr int kLgBN = 64;                     // experts per block
constexpr int kLgBK = 64;                     // columns per LDS chunk
constexpr int kLgPad = kLgBK + 8;             // LDS row pitch (bf16): 16 rows of a read hit distinct banks
constexpr int kLgThreads = 256;
constexpr int kLgFlush = 4;                   // chunks per fp32 run of the logits GEMM

template <int BM>
__global__ __launch_bounds__(kLgThreads) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                                  const float* __restrict__ w_g,
                                                                  const float* __restrict__ w_n, int E1, int T,
                                                                  int d, int E, int kslice, float* __restrict__ part) {
  constexpr int WT = BM / 2;                  // tokens per wavefront
  constexpr int FT = WT / 16;                 // 16-token fragments per wavefront
  constexpr int XL = BM * kLgBK / 8 / kLgThreads;     // 16-byte x loads per thread and chunk
  constexpr int WL = kLgBN * kLgBK / 4 / kLgThreads;  // 16-byte W_g loads per thread and chunk
  __shared__ uint16_t xs[BM * kLgPad];
  __shared__ uint16_t wp[3 * kLgBN * kLgPad]; // planes hi, mid, lo
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 8;
  const int t0 = blockIdx.x * BM;
  const int e0 = blockIdx.y * kLgBN;
  const int k0 = blockIdx.z * kslice;
  const int k1 = min(d, k0 + kslice);
  // each run of kLgFlush 64-column chunks is summed in fp32 (MFMA), the
  // running total in fp64, so that the rounding error does not grow with the
  // slice width the way one long fp32 chain's does (at d = 7168 that chain's
  // error reached 1e-5 of a logit)
  f32x4_mf acc[FT][2];
  double tot[FT][2][4];
#pragma unroll
  for (int i = 0; i < FT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) tot[i][j][q] = 0.0;
  // the next chunk's global loads are in flight while the current one is
  // multiplied out of LDS; d % 8 == 0 and slices are whole chunks, so a
  // piece is all in or all out
  uint4 xr[XL];
  float4 wr[WL];
  auto load = [&](int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int q = tid + kLgThreads * i;
      const int r = q / (kLgBK / 8), c = (q % (kLgBK / 8)) * 8;
      const int t = t0 + r, col = kc + c;
      xr[i] = (t < T && col < k1) ? *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * d + col)
                                  : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      const int q = tid + kLgThreads * i;
      const int r = q / (kLgBK / 4), c = (q % (kLgBK / 4)) * 4;
      const int e = e0 + r, col = kc + c;
      const float* wrow = e < E1 ? w_g + static_cast<size_t>(e) * d : w_n + static_cast<size_t>(e - E1) * d;
      wr[i] = (e < E && col < k1) ? *reinterpret_cast<const float4*>(wrow + col) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  if (k0 < k1) load(k0);
  for (int kc = k0; kc < k1; kc += kLgBK) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int q = tid + kLgThreads * i;
      const int r = q / (kLgBK / 8), c = (q % (kLgBK / 8)) * 8;
      *reinterpret_cast<uint4*>(xs + r * kLgPad + c) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      const int q = tid + kLgThreads * i;
      const int r = q / (kLgBK / 4), c = (q % (kLgBK / 4)) * 4;
      const float wv[4] = {wr[i].x, wr[i].y, wr[i].z, wr[i].w};
      uint32_t h[4], m[4], l[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        h[u] = __float_as_uint(wv[u]) & 0xffff0000u;
        const float rr = wv[u] - __uint_as_float(h[u]);           // exact
        m[u] = __float_as_uint(rr) & 0xffff0000u;
        l[u] = __float_as_uint(rr - __uint_as_float(m[u]));        // exact; fits in bf16
      }
      *reinterpret_cast<uint2*>(wp + (0 * kLgBN + r) * kLgPad + c) = make_uint2(hi16_pair(h[0], h[1]), hi16_pair(h[2], h[3]));
      *reinterpret_cast<uint2*>(wp + (1 * kLgBN + r) * kLgPad + c) = make_uint2(hi16_pair(m[0], m[1]), hi16_pair(m[2], m[3]));
      *reinterpret_cast<uint2*>(wp + (2 * kLgBN + r) * kLgPad + c) = make_uint2(hi16_pair(l[0], l[1]), hi16_pair(l[2], l[3]));
    }
    __syncthreads();
    if (kc + kLgBK < k1) load(kc + kLgBK);
    const int run = ((kc - k0) / kLgBK) % kLgFlush;          // chunk within the fp32 run
    if (run == 0) {
#pragma unroll
      for (int i = 0; i < FT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_mf{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < kLgBK / 32; ++ks) {
      bf16x8_t fa[FT], fb[2][3];
#pragma unroll
      for (int i = 0; i < FT; ++i)
        fa[i] = *reinterpret_cast<const bf16x8_t*>(xs + (wm * WT + i * 16 + r16) * kLgPad + ks * 32 + kq);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
          fb[j][pl] = *reinterpret_cast<const bf16x8_t*>(wp + (pl * kLgBN + wn * 32 + j * 16 + r16) * kLgPad + ks * 32 + kq);
#pragma unroll
      for (int i = 0; i < FT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int pl = 0; pl < 3; ++pl)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j][pl], acc[i][j], 0, 0, 0);
    }
    if (run == kLgFlush - 1 || kc + kLgBK >= k1) {
#pragma unroll
      for (int i = 0; i < FT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) tot[i][j][q] += static_cast<double>(acc[i][j][q]);
    }
    __syncthreads();
  }
  // lane holds expert column r16 of tokens 4 (lane / 16) + q of each fragment
  float* out = part + static_cast<size_t>(blockIdx.z) * T * E;
#pragma unroll
  for (int i = 0; i < FT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + wn * 32 + j * 16 + r16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + wm * WT + i * 16 + (lane >> 4) * 4 + q;
        if (t < T && e < E) out[static_cast<size_t>(t) * E + e] = static_cast<float>(tot[i][j][q]);
      }
    }
}

// Sum of the logit slices (in slice order) plus the router bias, then the
// fp32 softmax and top-k of each token by one wavefront, and per-block
// probability column sums (wavefronts added in order) to the workspace.
// NOISY: the partial rows hold 2 E logits per token, the clean ones then the
// noise projection's; the noisy logit is clean + b_g + draw * (softplus(
// projection + b_n) + eps).  PER: logits per thread, 16 E / 512 rounded up
// to a power of two.  Every load of a group of G slices (4, or 1 when there
// is a single slice), and the bias and draws, is in flight before the first
// wait: at one block per CU the kernel is a chain of memory round trips
// otherwise.
constexpr int kFnTok = 16;                    // tokens per block
constexpr int kFnWaves = 8;
constexpr int kFnThreads = 64 * kFnWaves;

template <bool NOISY, int PER, int G>
__global__ __launch_bounds__(kFnThreads) void router_finish_kernel(RouterArgs a, const float* __restrict__ part,
                                                                    int nslice) {
  constexpr int kFnGroup = G;                 // slices per round of loads
  // launch_finish picks PER with PER * kFnThreads >= kFnTok * E
  __shared__ float lg[kFnTok * kRtMaxE];
  __shared__ float wcol[kFnWaves * kRtMaxE];
  __shared__ float drs[NOISY ? kFnTok * kRtMaxE : 1];   // the block's draws when drawn here
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * kFnTok;
  for (int e = lane; e < a.E; e += 64) wcol[wave * a.E + e] = 0.f;
  const int n_ent = min(kFnTok, a.T - t0) * a.E;             // the block's tokens are contiguous
  const int PE = NOISY ? 2 * a.E : a.E;                      // partial logits per token
  const float* src = part + static_cast<size_t>(t0) * PE;
  // unconditional loads (clamped index); entries past the block's tokens
  // are not stored
  int jj[PER], off[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    jj[u] = min(tid + kFnThreads * u, n_ent - 1);
    off[u] = NOISY ? (jj[u] / a.E) * PE + jj[u] % a.E : jj[u];
  }
  float bg[PER], dr[PER], bn[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    bg[u] = 0.f;
    dr[u] = 0.f;
    bn[u] = 0.f;
  }
  if (a.b_g) {
#pragma unroll
    for (int u = 0; u < PER; ++u) bg[u] = a.b_g[jj[u] % a.E];
  }
  if constexpr (NOISY) {
    if (a.noise) {
#pragma unroll
      for (int u = 0; u < PER; ++u) dr[u] = a.noise[static_cast<size_t>(t0) * a.E + jj[u]];
    } else {
      // the block's draws [t0 E, t0 E + n_ent), a counter block (four
      // draws, two Box-Muller pairs) per thread, through LDS
      const unsigned long long base = static_cast<unsigned long long>(t0) * a.E;
      const unsigned long long jb = base >> 2, je = (base + n_ent + 3) >> 2;
      for (unsigned long long j = jb + tid; j < je; j += kFnThreads) {
        float v[4];
        philox_normal4(a.seed, a.offset, j, v);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const unsigned long long i = 4 * j + q;
          if (i >= base && i < base + n_ent) drs[i - base] = v[q];
        }
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < PER; ++u) dr[u] = drs[jj[u]];
    }
    if (a.b_n) {
#pragma unroll
      for (int u = 0; u < PER; ++u) bn[u] = a.b_n[jj[u] % a.E];
    }
  }
  float z[PER], zn[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    z[u] = 0.f;
    zn[u] = 0.f;
  }
  for (int s0 = 0; s0 < nslice; s0 += kFnGroup) {
    float v[kFnGroup][PER], vn[kFnGroup][PER];
#pragma unroll
    for (int q = 0; q < kFnGroup; ++q) {
      const float* ps = src + static_cast<size_t>(min(s0 + q, nslice - 1)) * a.T * PE;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        v[q][u] = ps[off[u]];
        if constexpr (NOISY) vn[q][u] = ps[off[u] + a.E];
      }
    }
    // slices past the last are added as 0 * v (the partials are finite)
#pragma unroll
    for (int q = 0; q < kFnGroup; ++q) {
      const float m = s0 + q < nslice ? 1.f : 0.f;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        z[u] += m * v[q][u];
        if constexpr (NOISY) zn[u] += m * vn[q][u];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    z[u] += bg[u];
    if constexpr (NOISY) z[u] += dr[u] * (softplus_f(zn[u] + bn[u]) + a.eps);
    const int j = tid + kFnThreads * u;
    if (j < n_ent) lg[j] = z[u];
  }
  __syncthreads();
  if (a.k <= 16) {
    // a row of 16 lanes per token (waves 0-3 take the block's 16 tokens), the
    // probabilities to LDS (pr aliases lg: each row reads its own token's
    // logits into registers before writing), column sums in token order
    float* pr = lg;
    if (tid < 16 * kFnTok) {
      const int tl = tid >> 4;
      const int t = t0 + tl;
      if (t < a.T) token16_softmax_topk<kRtMaxE / 16>(lg + tl * a.E, t, a, pr + tl * a.E, tid & 15);
      else
        for (int e = tid & 15; e < a.E; e += 16) pr[tl * a.E + e] = 0.f;
    }
    __syncthreads();
    for (int e = tid; e < a.E; e += kFnThreads) {
      float v = 0.f;
      for (int tl = 0; tl < kFnTok; ++tl) v += pr[tl * a.E + e];
      a.colsum_part[static_cast<size_t>(blockIdx.x) * a.E + e] = v;
    }
    return;
  }
  for (int tl = wave; tl < kFnTok; tl += kFnWaves) {
    const int t = t0 + tl;
    if (t >= a.T) break;
    token_softmax_topk(lg + tl * a.E, t, a, wcol + wave * a.E, lane);
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += kFnThreads) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kFnWaves; ++w) v += wcol[w * a.E + e];
    a.colsum_part[static_cast<size_t>(blockIdx.x) * a.E + e] = v;
  }
}

// finishing kernel for E experts: logits per thread and slices per round of
// loads as template arguments (a single slice: no clamped reloads of it)
template <bool NOISY, int G>
void launch_finish_g(const RouterArgs& a, const float* part, int nslice, int nb, hipStream_t stream) {
  const dim3 grid(nb), block(kFnThreads);
  if (a.E <= 32)
    hipLaunchKernelGGL((router_finish_kernel<NOISY, 1, G>), grid, block, 0, stream, a, part, nslice);
  else if (a.E <= 64)
    hipLaunchKernelGGL((router_finish_kernel<NOISY, 2, G>), grid, block, 0, stream, a, part, nslice);
  else if (a.E <= 128)
    hipLaunchKernelGGL((router_finish_kernel<NOISY, 4, G>), grid, block, 0, stream, a, part, nslice);
  else
    hipLaunchKernelGGL((router_finish_kernel<NOISY, 8, G>), grid, block, 0, stream, a, part, nslice);
}
template <bool NOISY>
void launch_finish(const RouterArgs& a, const float* part, int nslice, int nb, hipStream_t stream) {
  if (nslice == 1)
    launch_finish_g<NOISY, 1>(a, part, nslice, nb, stream);
  else
    launch_finish_g<NOISY, 4>(a, part, nslice, nb, stream);
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

// Column sums and balance loss in one launch, from the per-block partial
// column sums a router call left in its workspace, for up to ME experts.
// Every column sum is formed exactly as colsum_reduce_kernel forms it (256
// strided fp64 partial sums over the blocks, then the same tree: the two
// cross-wavefront steps in LDS, the other six by shuffles in wavefront 0,
// which pair the same lanes), and the loss exactly as aux_loss_kernel forms
// it (its tree steps of 32 and more only add zeros here), so both equal what
// moe_router_topk with prob_colsum followed by moe_aux_loss give, bit for
// bit.  Loads and LDS accesses are unconditional (clamped addresses):
// predicated ones compiled into a branch and a wait per element.
template <int ME>
__global__ __launch_bounds__(256) void aux_from_parts_kernel(const float* __restrict__ part, int nb, int E,
                                                             const int32_t* __restrict__ counts, int T_, int k,
                                                             float alpha, float* __restrict__ prob_colsum,
                                                             float* __restrict__ loss) {
  __shared__ double red[ME][256];
  __shared__ float csum[ME];
  const int i = threadIdx.x;
  const int lane = i & 63;
  double acc[ME];
#pragma unroll
  for (int c = 0; c < ME; ++c) acc[c] = 0.0;
  for (int b = i; b < nb; b += 256) {
    float v[ME];
#pragma unroll
    for (int c = 0; c < ME; ++c) v[c] = part[static_cast<size_t>(b) * E + min(c, E - 1)];
#pragma unroll
    for (int c = 0; c < ME; ++c) acc[c] += static_cast<double>(v[c]);
  }
#pragma unroll
  for (int c = 0; c < ME; ++c) red[c][i] = acc[c];
  __syncthreads();
  if (i < 128) {
    double x1[ME];
#pragma unroll
    for (int c = 0; c < ME; ++c) x1[c] = red[c][i + 128];
#pragma unroll
    for (int c = 0; c < ME; ++c) red[c][i] = acc[c] + x1[c];
  }
  __syncthreads();
  if (i >= 64) return;
  double v[ME];
#pragma unroll
  for (int c = 0; c < ME; ++c) v[c] = red[c][lane] + red[c][lane + 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
#pragma unroll
    for (int c = 0; c < ME; ++c) v[c] += __shfl_down(v[c], o);
  if (lane == 0) {
#pragma unroll
    for (int c = 0; c < ME; ++c) csum[c] = static_cast<float>(v[c]);
  }
  // the lanes of this wavefront read what lane 0 wrote: LDS operations of a
  // wavefront complete in order; the fence keeps the reads after the writes
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  const float cs = csum[min(lane, ME - 1)];
  if (lane < E) prob_colsum[lane] = cs;
  float sv = 0.f;
  if (T_ > 0 && lane < E) {
    const float inv_tk = 1.0f / (static_cast<float>(T_) * static_cast<float>(k));
    const float inv_t = 1.0f / static_cast<float>(T_);
    sv = (static_cast<float>(counts[lane]) * inv_tk) * (cs * inv_t);
  }
#pragma unroll
  for (int o = ME / 2; o > 0; o >>= 1) sv += __shfl_down(sv, o);
  if (lane == 0) *loss = alpha * static_cast<float>(E) * sv;
}
constexpr int kAxMaxE = 32;

inline int router_blocks(int T) { return (T + kRtTok - 1) / kRtTok; }

// upper bound of the block count of any router kernel (per-block
// probability partial sums live in the workspace)
inline int router_max_blocks(int T) {
  const int mfma = (T + 15) / 16;             // MFMA kernels: at least 16 tokens per block
  const int generic = router_blocks(T);
  return mfma > generic ? mfma : generic;
}


// wavefronts per token group (cpw 128-column chunks each per round) and token
// groups per block of router_mf8_kernel: whole rows in one round up to
// 16 cpw chunks; more tokens per block for narrow rows while the grid keeps
// at least one block per CU
inline void mf8_shape(int T, int d, int cpw, int& kw, int& tg) {
  const int nch = (d + 127) / 128;
  kw = (nch + cpw - 1) / cpw;
  if (kw > kM8Waves) kw = kM8Waves;
  tg = T / (16 * kCUs);
  if (tg > kM8Waves / kw) tg = kM8Waves / kw;
  if (tg < 1) tg = 1;
}
// tiled logits GEMM (more than 8 experts, bf16 x): token rows per block;
// K slices so that the grid has about one block per CU, each slice at least
// 256 columns; the slice width in whole 64-column chunks
inline int logit_bm(int T) { return T >= 8192 ? 128 : 64; }
inline int logit_slices(int T, int d, int E) {
  const long mn = static_cast<long>((T + logit_bm(T) - 1) / logit_bm(T)) * ((E + kLgBN - 1) / kLgBN);
  int ks = 1;
  while (mn * ks < kCUs && d / (2 * ks) >= 256) ks *= 2;
  return ks;
}
inline int logit_kslice(int d, int ks) { return ((d + ks - 1) / ks + kLgBK - 1) / kLgBK * kLgBK; }
// byte offset of the partial logits in the workspace (after the column sums)
inline size_t logit_ws_offset(int T, int E) {
  return align_up(static_cast<size_t>(router_max_blocks(T)) * E * sizeof(float), kWsAlign);
}

// blocks of the router kernel that writes the per-block column sums (the
// first nb x E floats of the workspace)
inline int router_nb(int T, int d, int E, int x_dt, bool noisy) {
  const bool m8 = x_dt == MOE_BF16 && E <= kM8MaxE;
  const bool mf = x_dt == MOE_BF16 && !m8;
  int kw8 = 1, tg8 = 1;
  mf8_shape(T, d, noisy ? 1 : kM8Cpw, kw8, tg8);
  return m8 ? (T + 16 * tg8 - 1) / (16 * tg8) : (mf ? (T + kFnTok - 1) / kFnTok : router_blocks(T));
}

// the launches of every router entry point; arguments already validated.
// noise == nullptr and !drawn: the clean router; drawn: the noisy router
// with its draws from the stream (seed, offset).  bf16: MFMA kernels (up to 8 experts: whole
// rows per block, one launch; otherwise the tiled logits GEMM, then the
// finishing kernel); fp32 activations: the generic kernel.
int router_run(const void* x, int x_dt, const float* w_g, const float* b_g, const float* w_n, const float* b_n,
               const float* noise, float eps, int T, int d, int E, int k, int gate_mode, int32_t* topk_idx,
               float* topk_gate, float* prob_colsum, float* logits_dbg, void* workspace, hipStream_t stream,
               bool drawn = false, unsigned long long seed = 0, unsigned long long offset = 0) {
  const bool noisy = noise != nullptr || drawn;
  const bool m8 = x_dt == MOE_BF16 && E <= kM8MaxE;
  const bool mf = x_dt == MOE_BF16 && !m8;
  float* part = static_cast<float*>(workspace);
  int kw8 = 1, tg8 = 1;
  mf8_shape(T, d, noisy ? 1 : kM8Cpw, kw8, tg8);
  const int nb = router_nb(T, d, E, x_dt, noisy);
  RouterArgs a{x,     w_g,     b_g,  T,   d,   E,   k,    gate_mode, topk_idx, topk_gate, part,
               logits_dbg, w_n, b_n, drawn ? nullptr : noise, eps, seed, offset};
  if (T > 0 && m8) {
    if (noisy)
      hipLaunchKernelGGL(router_mf8_kernel<true>, dim3(nb), dim3(64 * kw8 * tg8), 0, stream, a, kw8, tg8);
    else
      hipLaunchKernelGGL(router_mf8_kernel<false>, dim3(nb), dim3(64 * kw8 * tg8), 0, stream, a, kw8, tg8);
    int st = check_launch();
    if (st != MOE_OK) return st;
  }
  if (T > 0 && mf) {
    // noisy: the logits GEMM runs over W_g stacked on W_n (2 E rows)
    const int EL = noisy ? 2 * E : E;
    float* lgp = reinterpret_cast<float*>(static_cast<char*>(workspace) + logit_ws_offset(T, E));
    const int bm = logit_bm(T), ks = logit_slices(T, d, EL), kslice = logit_kslice(d, ks);
    const dim3 grid((T + bm - 1) / bm, (EL + kLgBN - 1) / kLgBN, ks);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const float* wn = noisy ? w_n : w_g;
    if (bm == 128)
      hipLaunchKernelGGL(router_logits_kernel<128>, grid, dim3(kLgThreads), 0, stream, xb, w_g, wn, E, T, d, EL,
                         kslice, lgp);
    else
      hipLaunchKernelGGL(router_logits_kernel<64>, grid, dim3(kLgThreads), 0, stream, xb, w_g, wn, E, T, d, EL,
                         kslice, lgp);
    int st = check_launch();
    if (st != MOE_OK) return st;
    if (noisy)
      launch_finish<true>(a, lgp, ks, nb, stream);
    else
      launch_finish<false>(a, lgp, ks, nb, stream);
    st = check_launch();
    if (st != MOE_OK) return st;
  }
  if (T > 0 && !mf && !m8) {
    size_t lds = (static_cast<size_t>(kRtDc) * kRtTok + static_cast<size_t>(kRtDc) * kRtExp +
                  static_cast<size_t>(kRtTok) * E + 4 * static_cast<size_t>(E)) * sizeof(float);
    if (noisy)
      hipLaunchKernelGGL((router_generic_kernel<float, true>), dim3(nb), dim3(kRtThreads), lds, stream, a);
    else
      hipLaunchKernelGGL((router_generic_kernel<float, false>), dim3(nb), dim3(kRtThreads), lds, stream, a);
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

// argument checks shared by both entry points (workspace excluded)
int router_check(const void* x, int x_dt, const float* w_g, const float* b_g, int T, int d, int E, int k,
                 int gate_mode, int32_t* topk_idx, float* topk_gate, float* prob_colsum, float* logits_dbg) {
  if (T < 0 || d < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > kRtMaxE || k > kRtMaxK) return MOE_ERR_UNSUPPORTED;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (x_dt == MOE_BF16 && d % 8 != 0) return MOE_ERR_INVALID_ARG;   // 16-byte row pieces
  if (gate_mode != MOE_GATE_PROB && gate_mode != MOE_GATE_RENORM) return MOE_ERR_INVALID_ARG;
  if (!w_g || !aligned16(w_g) || (b_g && !aligned16(b_g))) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!x || !topk_idx || !topk_gate)) return MOE_ERR_INVALID_ARG;
  if ((x && !aligned16(x)) || (topk_idx && !aligned16(topk_idx)) || (topk_gate && !aligned16(topk_gate)) ||
      (prob_colsum && !aligned16(prob_colsum)) || (logits_dbg && !aligned16(logits_dbg)))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

inline bool workspace_ok(int T, const float* prob_colsum, const void* workspace, size_t have, size_t need) {
  if ((T > 0 || prob_colsum) && (!workspace || have < need || !aligned16(workspace))) return false;
  return true;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept for later calls.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    record_hip_error(e);
    return MOE_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      record_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return MOE_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

namespace moe {
namespace {

// out[i] = standard normal draw i of the stream (seed, offset): a
// grid-stride loop over counter blocks, four draws each
__global__ __launch_bounds__(256) void gate_noise_kernel(unsigned long long seed, unsigned long long offset, size_t n,
                                                         float* __restrict__ out) {
  const size_t nb = (n + 3) / 4;
  for (size_t j = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; j < nb;
       j += static_cast<size_t>(gridDim.x) * blockDim.x) {
    float v[4];
    philox_normal4(seed, offset, j, v);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (4 * j + q < n) out[4 * j + q] = v[q];
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_gate_noise_philox(uint64_t seed, uint64_t offset, size_t n, float* out, hipStream_t stream) {
  if (n > (size_t(1) << 62)) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (!out) return MOE_ERR_INVALID_ARG;
  const size_t blocks = std::min<size_t>(((n + 3) / 4 + 255) / 256, 8 * 256);
  hipLaunchKernelGGL(gate_noise_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<unsigned long long>(seed), static_cast<unsigned long long>(offset), n, out);
  return check_launch();
}

size_t moe_router_workspace_size(int T, int d, int E, int x_dt) {
  if (T < 0 || E < 1) return 0;
  size_t s = logit_ws_offset(T, E);
  // partial logits of the tiled router GEMM
  if (x_dt == MOE_BF16 && E > kM8MaxE && d > 0)
    s += align_up(static_cast<size_t>(logit_slices(T, d, E)) * T * E * sizeof(float), kWsAlign);
  return s;
}

int moe_router_topk(const void* x, int x_dt, const float* w_g, const float* b_g, int T, int d, int E,
                    int k, int gate_mode, int32_t* topk_idx, float* topk_gate, float* prob_colsum,
                    float* logits_dbg, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = router_check(x, x_dt, w_g, b_g, T, d, E, k, gate_mode, topk_idx, topk_gate, prob_colsum, logits_dbg);
  if (st != MOE_OK) return st;
  if (!workspace_ok(T, prob_colsum, workspace, workspace_bytes, moe_router_workspace_size(T, d, E, x_dt)))
    return MOE_ERR_WORKSPACE;
  return router_run(x, x_dt, w_g, b_g, nullptr, nullptr, nullptr, 0.f, T, d, E, k, gate_mode, topk_idx, topk_gate,
                    prob_colsum, logits_dbg, workspace, stream);
}

int moe_router_topk_noalloc(const void* x, int x_dt, const float* w_g, const float* b_g, int T, int d, int E,
                            int k, int gate_mode, int32_t* topk_idx, float* topk_gate, float* prob_colsum,
                            float* logits_dbg, hipStream_t stream) {
  int st = router_check(x, x_dt, w_g, b_g, T, d, E, k, gate_mode, topk_idx, topk_gate, prob_colsum, logits_dbg);
  if (st != MOE_OK) return st;
  // the scratch this call needs is what moe_router_topk takes as workspace;
  // every byte the kernels read from it is written first in the same call
  if (moe_router_workspace_size(T, d, E, x_dt) > static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES))
    return MOE_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != MOE_OK) return st;
  return router_run(x, x_dt, w_g, b_g, nullptr, nullptr, nullptr, 0.f, T, d, E, k, gate_mode, topk_idx, topk_gate,
                    prob_colsum, logits_dbg, ws, stream);
}

size_t moe_router_noisy_workspace_size(int T, int d, int E, int x_dt) {
  if (T < 0 || E < 1) return 0;
  size_t s = logit_ws_offset(T, E);
  // partial logits of the tiled GEMM over W_g and W_n (2 E rows)
  if (x_dt == MOE_BF16 && d > 0)
    s += align_up(static_cast<size_t>(logit_slices(T, d, 2 * E)) * T * 2 * E * sizeof(float), kWsAlign);
  return s;
}

int moe_router_topk_noisy(const void* x, int x_dt, const float* w_g, const float* b_g, const float* w_n,
                          const float* b_n, const float* noise, float noise_eps, int T, int d, int E, int k,
                          int gate_mode, int32_t* topk_idx, float* topk_gate, float* prob_colsum,
                          float* logits_dbg, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = router_check(x, x_dt, w_g, b_g, T, d, E, k, gate_mode, topk_idx, topk_gate, prob_colsum, logits_dbg);
  if (st != MOE_OK) return st;
  if (!w_n || !aligned16(w_n) || (b_n && !aligned16(b_n))) return MOE_ERR_INVALID_ARG;
  if ((T > 0 && !noise) || (noise && !aligned16(noise))) return MOE_ERR_INVALID_ARG;
  if (!(noise_eps >= 0.f) || noise_eps > 3.0e38f) return MOE_ERR_INVALID_ARG;   // NaN, negative or infinite
  if (!workspace_ok(T, prob_colsum, workspace, workspace_bytes, moe_router_noisy_workspace_size(T, d, E, x_dt)))
    return MOE_ERR_WORKSPACE;
  // no tokens: only the (zero) column sums, as the clean router writes them
  return router_run(x, x_dt, w_g, b_g, w_n, b_n, T > 0 ? noise : nullptr, noise_eps, T, d, E, k, gate_mode,
                    topk_idx, topk_gate, prob_colsum, logits_dbg, workspace, stream);
}

int moe_router_topk_noisy_philox(const void* x, int x_dt, const float* w_g, const float* b_g, const float* w_n,
                                 const float* b_n, uint64_t seed, uint64_t offset, float noise_eps, int T, int d,
                                 int E, int k, int gate_mode, int32_t* topk_idx, float* topk_gate,
                                 float* prob_colsum, float* logits_dbg, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  int st = router_check(x, x_dt, w_g, b_g, T, d, E, k, gate_mode, topk_idx, topk_gate, prob_colsum, logits_dbg);
  if (st != MOE_OK) return st;
  if (!w_n || !aligned16(w_n) || (b_n && !aligned16(b_n))) return MOE_ERR_INVALID_ARG;
  if (!(noise_eps >= 0.f) || noise_eps > 3.0e38f) return MOE_ERR_INVALID_ARG;   // NaN, negative or infinite
  if (!workspace_ok(T, prob_colsum, workspace, workspace_bytes, moe_router_noisy_workspace_size(T, d, E, x_dt)))
    return MOE_ERR_WORKSPACE;
  return router_run(x, x_dt, w_g, b_g, w_n, b_n, nullptr, noise_eps, T, d, E, k, gate_mode, topk_idx, topk_gate,
                    prob_colsum, logits_dbg, workspace, stream, T > 0, seed, offset);
}

int moe_aux_loss_from_router(const int32_t* counts_routed, const void* router_workspace, size_t workspace_bytes,
                             int T, int d, int E, int x_dt, int noisy, int k, float alpha, float* prob_colsum,
                             float* loss, hipStream_t stream) {
  if (T < 0 || d < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > kRtMaxE) return MOE_ERR_UNSUPPORTED;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (!counts_routed || !loss || !prob_colsum || !aligned16(prob_colsum)) return MOE_ERR_INVALID_ARG;
  const size_t need = noisy ? moe_router_noisy_workspace_size(T, d, E, x_dt) : moe_router_workspace_size(T, d, E, x_dt);
  if (T > 0 && (!router_workspace || workspace_bytes < need || !aligned16(router_workspace))) return MOE_ERR_WORKSPACE;
  const int nb = T > 0 ? router_nb(T, d, E, x_dt, noisy != 0) : 0;
  if (E <= kAxMaxE) {
    const float* part = static_cast<const float*>(router_workspace);
    if (E <= 8)
      hipLaunchKernelGGL(aux_from_parts_kernel<8>, dim3(1), dim3(256), 0, stream, part, nb, E, counts_routed, T, k,
                         alpha, prob_colsum, loss);
    else
      hipLaunchKernelGGL(aux_from_parts_kernel<32>, dim3(1), dim3(256), 0, stream, part, nb, E, counts_routed, T, k,
                         alpha, prob_colsum, loss);
    return check_launch();
  }
  // more experts: one block per expert for the column sums (a single block
  // is slower there than the extra launch), then the loss
  hipLaunchKernelGGL(colsum_reduce_kernel, dim3(E), dim3(256), 0, stream, static_cast<const float*>(router_workspace),
                     nb, E, prob_colsum);
  const int st = check_launch();
  if (st != MOE_OK) return st;
  return moe_aux_loss(counts_routed, prob_colsum, T, k, E, alpha, loss, stream);
}

}  // extern "C"
