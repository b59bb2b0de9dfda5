// (b) Dispatch: per-expert histogram, exclusive scan, stable token-order
// rank with capacity truncation, and the row permutation Xp[dest] = x[t].
//
// P1 §2.4: the tokens of one expert are gathered into a batch and scattered
// back afterwards.  P5 专家容量: tokens beyond an expert's capacity skip it.
// The rank of assignment (t, j) to expert e is the number of assignments to
// e from tokens before t; it is kept iff rank < C.
//
// Determinism: atomics are used only where their order cannot matter (LDS
// counts, LDS bit-OR of lane masks).  Ranks come from prefix sums and
// popcounts of those masks, so every integer output is the unique answer.
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kDsTok = 256;          // tokens per block (4 wavefronts)
constexpr int kDsWaves = kDsTok / 64;
constexpr int kDsMaxE = 1024;

// block_counts[b][e] = assignments to e among the block's tokens
__global__ __launch_bounds__(kDsTok) void dispatch_count_kernel(const int32_t* __restrict__ idx, int T, int k,
                                                               int E, int32_t* __restrict__ block_counts) {
  __shared__ int cnt[kDsMaxE];
  for (int e = threadIdx.x; e < E; e += kDsTok) cnt[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kDsTok + threadIdx.x;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      int e = idx[static_cast<size_t>(t) * k + j];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kDsTok) block_counts[static_cast<size_t>(blockIdx.x) * E + e] = cnt[e];
}

// dest_pos / perm_token, plus (block 0) counts_routed, counts_kept and
// offsets.  Every block first derives from the per-block counts what it
// needs: the expert totals, their kept counts and the exclusive scan of those
// (offsets), and its own base = counts of the earlier blocks.  That is a few
// hundred integer loads per block and saves a separate scan launch.
// Within the block, lane order is token order: the lanes of a wavefront that
// chose expert e form the mask M_w[e] (LDS atomic OR), so a token's rank
// inside its wave is popcount(M_w[e] & lanes_below) and the earlier waves
// add popcount(M_w'[e]).
__global__ __launch_bounds__(kDsTok) void dispatch_rank_kernel(const int32_t* __restrict__ idx, int T, int k, int E,
                                                              int C, int nb, const int32_t* __restrict__ block_counts,
                                                              int32_t* __restrict__ counts_routed,
                                                              int32_t* __restrict__ counts_kept,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ dest_pos,
                                                              int32_t* __restrict__ perm_token) {
  extern __shared__ unsigned long long masks[];   // [kDsWaves][E], then int base[E], int off[E]
  int* base = reinterpret_cast<int*>(masks + kDsWaves * E);
  int* off = base + E;
  __shared__ int wsum[kDsTok / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < kDsWaves * E; i += kDsTok) masks[i] = 0ull;
  // totals, kept counts and this block's base, per expert
  for (int e = tid; e < E; e += kDsTok) {
    int total = 0, before = 0;
    for (int b = 0; b < nb; ++b) {
      const int c = block_counts[static_cast<size_t>(b) * E + e];
      total += c;
      if (b < static_cast<int>(blockIdx.x)) before += c;
    }
    const int kept = C < 0 ? total : min(total, C);
    base[e] = before;
    off[e] = kept;
    if (blockIdx.x == 0) {
      counts_routed[e] = total;
      counts_kept[e] = kept;
    }
  }
  __syncthreads();
  // exclusive scan of off[] (kept counts) over experts: each thread scans a
  // contiguous run, the run totals are scanned across the block
  const int per = (E + kDsTok - 1) / kDsTok;
  const int e0 = tid * per, e1 = min(E, e0 + per);
  int run = 0;
  for (int e = e0; e < e1; ++e) run += off[e];
  int incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int prefix = incl - run;
  for (int w = 0; w < wave; ++w) prefix += wsum[w];
  for (int e = e0; e < e1; ++e) {
    const int kept = off[e];
    off[e] = prefix;
    if (blockIdx.x == 0) offsets[e] = prefix;
    prefix += kept;
  }
  if (blockIdx.x == 0 && e1 == E && e0 < E) offsets[E] = prefix;
  if (blockIdx.x == 0 && E == 0 && tid == 0) offsets[0] = 0;
  const int t = blockIdx.x * kDsTok + tid;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[static_cast<size_t>(t) * k + j];
      if (e >= 0 && e < E) atomicOr(&masks[wave * E + e], 1ull << lane);
    }
  }
  __syncthreads();
  if (t >= T) return;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; ++j) {
    const size_t o = static_cast<size_t>(t) * k + j;
    const int e = idx[o];
    int dest = -1;
    if (e >= 0 && e < E) {
      int r = base[e];
      for (int w = 0; w < wave; ++w) r += __popcll(masks[w * E + e]);
      r += __popcll(masks[wave * E + e] & below);
      if (C < 0 || r < C) {
        dest = off[e] + r;
        perm_token[dest] = t;
      }
    }
    dest_pos[o] = dest;
  }
}

// T == 0: the counts are zero and the offsets all zero.
__global__ void dispatch_empty_kernel(int E, int32_t* counts_routed, int32_t* counts_kept, int32_t* offsets) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    offsets[e] = 0;
    if (e < E) {
      counts_routed[e] = 0;
      counts_kept[e] = 0;
    }
  }
}

// Xp[dest_pos[t, j]] = x[t] for kept slots.  Each block copies `rows`
// consecutive tokens; a row is read once and written k times.
template <typename V>
__global__ __launch_bounds__(256) void permute_rows_kernel(const V* __restrict__ x, const int32_t* __restrict__ dest_pos,
                                                          int T, int k, int nvec, int rows, V* __restrict__ xp) {
  const int t_begin = blockIdx.x * rows;
  const int t_end = min(T, t_begin + rows);
  for (int t = t_begin; t < t_end; ++t) {
    const int32_t* dp = dest_pos + static_cast<size_t>(t) * k;
    const V* src = x + static_cast<size_t>(t) * nvec;
    for (int v = threadIdx.x; v < nvec; v += 256) {
      V val = src[v];
      for (int j = 0; j < k; ++j) {
        int d = dp[j];
        if (d >= 0) xp[static_cast<size_t>(d) * nvec + v] = val;
      }
    }
  }
}

inline int disp_blocks(int T) { return (T + kDsTok - 1) / kDsTok; }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_dispatch_workspace_size(int T, int k, int E) {
  (void)k;
  if (T < 0 || E < 1) return 0;
  return align_up(static_cast<size_t>(disp_blocks(T) > 0 ? disp_blocks(T) : 1) * E * sizeof(int32_t), kWsAlign);
}

int moe_dispatch_permute(const int32_t* topk_idx, int T, int k, int E, int capacity, const void* x, int x_dt,
                         int d, void* x_perm, int32_t* counts_routed, int32_t* counts_kept, int32_t* offsets,
                         int32_t* dest_pos, int32_t* perm_token, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (T < 0 || k < 1 || E < 1 || k > E || capacity < -1) return MOE_ERR_INVALID_ARG;
  if (E > kDsMaxE) return MOE_ERR_UNSUPPORTED;
  if (!counts_routed || !counts_kept || !offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_idx || !dest_pos || !perm_token)) return MOE_ERR_INVALID_ARG;
  const bool copy_rows = T > 0 && (x != nullptr || x_perm != nullptr);
  if (copy_rows) {
    if (!x || !x_perm || d < 1) return MOE_ERR_INVALID_ARG;
    if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  }
  const void* ptrs[] = {topk_idx, counts_routed, counts_kept, offsets, dest_pos, perm_token};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_dispatch_workspace_size(T, k, E);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MOE_ERR_WORKSPACE;

  const int nb = disp_blocks(T);
  int32_t* bc = static_cast<int32_t*>(workspace);
  if (nb == 0) {
    hipLaunchKernelGGL(dispatch_empty_kernel, dim3(1), dim3(256), 0, stream, E, counts_routed, counts_kept, offsets);
    return check_launch();
  }
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(nb), dim3(kDsTok), 0, stream, topk_idx, T, k, E, bc);
  int st = check_launch();
  if (st != MOE_OK) return st;
  const size_t lds = static_cast<size_t>(kDsWaves) * E * sizeof(unsigned long long) + 2 * E * sizeof(int);
  hipLaunchKernelGGL(dispatch_rank_kernel, dim3(nb), dim3(kDsTok), lds, stream, topk_idx, T, k, E, capacity, nb,
                     static_cast<const int32_t*>(bc), counts_routed, counts_kept, offsets, dest_pos, perm_token);
  st = check_launch();
  if (st != MOE_OK) return st;
  if (!copy_rows) return MOE_OK;

  const size_t row_bytes = static_cast<size_t>(d) * dtype_bytes(x_dt);
  // about 2048 blocks, at least one token each
  int rows = (T + 2047) / 2048;
  if (rows < 1) rows = 1;
  const int nblk = (T + rows - 1) / rows;
  if (row_bytes % 16 == 0) {
    hipLaunchKernelGGL(permute_rows_kernel<uint4>, dim3(nblk), dim3(256), 0, stream,
                       static_cast<const uint4*>(x), static_cast<const int32_t*>(dest_pos), T, k,
                       static_cast<int>(row_bytes / 16), rows, static_cast<uint4*>(x_perm));
  } else if (row_bytes % 4 == 0) {
    hipLaunchKernelGGL(permute_rows_kernel<uint32_t>, dim3(nblk), dim3(256), 0, stream,
                       static_cast<const uint32_t*>(x), static_cast<const int32_t*>(dest_pos), T, k,
                       static_cast<int>(row_bytes / 4), rows, static_cast<uint32_t*>(x_perm));
  } else {
    hipLaunchKernelGGL(permute_rows_kernel<uint16_t>, dim3(nblk), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<const int32_t*>(dest_pos), T, k,
                       static_cast<int>(row_bytes / 2), rows, static_cast<uint16_t*>(x_perm));
  }
  return check_launch();
}

}  // extern "C"
