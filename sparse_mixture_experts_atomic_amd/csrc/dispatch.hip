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

// ---------------------------------------------------------------------------
// One-launch dispatch for T*k <= kFusedMaxEntries.  Every block reads all
// T*k expert ids (a few tens of KB, from L2) and derives from them what it
// needs: the expert totals, their kept counts and exclusive scan (offsets),
// and the assignments to each expert from tokens before its own range.  No
// block depends on another, so there is no second launch and no inter-block
// wait.  The block's rows of x are loaded into registers first, so their HBM
// latency overlaps the index work; each row is then stored to its kept
// slots.  Same outputs as the count/rank/permute path, bit for bit.
// PRE: for more than 8 experts, where counting every id in every block
// takes an LDS atomic per id, the per-256-token-block counts come from
// dispatch_count_kernel (one launch before) and a block sums those, counting
// only the ids of its own 256-token block that precede its tokens.
// at most 63 int4 loads + 1 tail id = 253 ids per thread, so the packed 8-bit
// per-thread counts below cannot overflow
// Sum of v over the 64 lanes of a wavefront, valid in lane 63: quad
// permutes, row shifts by 4 and 8, then the row-15 and row-31 broadcasts
// (gfx9 DPP; lanes whose source is outside the row read 0).
__device__ __forceinline__ uint32_t wave_sum_dpp(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0xb1, 0xf, 0xf, true);    // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0u, v, 0x4e, 0xf, 0xf, true);    // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xf, 0xf, true);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xf, 0xf, true);   // row_bcast:31
  return v;
}

constexpr int kFusedMaxEntries = 63 * 4 * 256;
constexpr int kPackedE = 8;                    // register-packed counting for E <= 8
constexpr int kIdPre = 8;                      // int4 id loads per thread issued before the rows
constexpr int kFusedThreads = 256;
constexpr int kFusedMaxVec = 16;               // row vectors per thread (the largest NQ instance)

template <int NQ, bool PRE>
__global__ __launch_bounds__(kFusedThreads) void dispatch_fused_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int C, int tpb, const uint4* __restrict__ x, int nvec,
    uint4* __restrict__ xp, int32_t* __restrict__ counts_routed, int32_t* __restrict__ counts_kept,
    int32_t* __restrict__ offsets, int32_t* __restrict__ dest_pos, int32_t* __restrict__ perm_token,
    const int32_t* __restrict__ block_counts, int nbc) {
  __shared__ int before[kDsMaxE];
  __shared__ int total[kDsMaxE];
  __shared__ int off[kDsMaxE];
  __shared__ int ent[kFusedThreads];      // expert of the block's entries
  __shared__ int dst[kFusedThreads];      // their destination row (-1: none)
  __shared__ int wsum[kFusedThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * tpb;
  const int t1 = min(T, t0 + tpb);
  const int nrow_vec = (t1 - t0) * nvec;  // 16-byte vectors of the block's rows

  // 1. the first ids (loads complete in issue order, so the ids are loaded
  //    before the rows: the counting below then waits only for them)
  const int n_all = T * k;
  const int n_before = t0 * k;
  const int n4 = n_all / 4;
  // every block reads all ids; starting each block at a different place
  // spreads the reads of one cache line over time (counting is order-free)
  const int rot = n4 > 0 ? static_cast<int>((static_cast<long>(blockIdx.x) * 1031) % n4) : 0;
  int4 iv[kIdPre];
#pragma unroll
  for (int u = 0; u < kIdPre; ++u) {
    const int j = tid + kFusedThreads * u;
    int i4 = j + rot;
    if (i4 >= n4) i4 -= n4;
    iv[u] = (!PRE && j < n4) ? reinterpret_cast<const int4*>(idx)[i4] : make_int4(-1, -1, -1, -1);
  }
  const int nb_ent = (t1 - t0) * k;
  const int my_ent = tid < nb_ent ? idx[static_cast<size_t>(t0) * k + tid] : -1;

  // 2. the block's rows, into registers (vector q = tid + 256 u of the rows)
  uint4 rv[NQ];
#pragma unroll
  for (int u = 0; u < NQ; ++u) rv[u] = make_uint4(0u, 0u, 0u, 0u);
  if (x) {
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int q = tid + kFusedThreads * u;
      if (q < nrow_vec) rv[u] = x[static_cast<size_t>(t0) * nvec + q];
    }
  }

  // 3. expert totals and counts before t0, from all T*k ids (PRE: from the
  //    per-256-token-block counts and the ids of t0's block before t0)
  if constexpr (PRE) {
    const int cb = t0 / kDsTok;
    for (int e = tid; e < E; e += kFusedThreads) {
      int tot = 0, bef = 0;
      for (int b = 0; b < nbc; ++b) {
        const int c = block_counts[static_cast<size_t>(b) * E + e];
        tot += c;
        bef += b < cb ? c : 0;
      }
      total[e] = tot;
      before[e] = bef;
    }
    __syncthreads();
    for (int i = cb * kDsTok * k + tid; i < n_before; i += kFusedThreads) {
      const int e = idx[i];
      if (e >= 0 && e < E) atomicAdd(&before[e], 1);
    }
  } else {
  for (int e = tid; e < E; e += kFusedThreads) {
    before[e] = 0;
    total[e] = 0;
  }
  __syncthreads();
  if (E <= kPackedE) {
    // per-thread counts in 8-bit fields of one 64-bit word (at most 255 ids
    // per thread), widened to 16-bit fields for the wavefront sum
    unsigned long long tot = 0, bef = 0;
    auto count = [&](int i, int e) __attribute__((always_inline)) {
      const unsigned long long one = (e >= 0 && e < E) ? (1ull << (8 * e)) : 0ull;
      tot += one;
      bef += i < n_before ? one : 0ull;
    };
#pragma unroll
    for (int u = 0; u < kIdPre; ++u) {
      const int j = tid + kFusedThreads * u;
      if (j < n4) {
        int i4 = j + rot;
        if (i4 >= n4) i4 -= n4;
        count(4 * i4, iv[u].x);
        count(4 * i4 + 1, iv[u].y);
        count(4 * i4 + 2, iv[u].z);
        count(4 * i4 + 3, iv[u].w);
      }
    }
    for (int j = tid + kFusedThreads * kIdPre; j < n4; j += kFusedThreads) {
      int i4 = j + rot;
      if (i4 >= n4) i4 -= n4;
      const int4 v = reinterpret_cast<const int4*>(idx)[i4];
      count(4 * i4, v.x);
      count(4 * i4 + 1, v.y);
      count(4 * i4 + 2, v.z);
      count(4 * i4 + 3, v.w);
    }
    for (int i = 4 * n4 + tid; i < n_all; i += kFusedThreads) count(i, idx[i]);
    // fields 0..3 and 4..7 as 16-bit lanes of two words each
    constexpr unsigned long long m8 = 0x00ff00ff00ff00ffull;
    auto widen_lo = [](unsigned long long w) __attribute__((always_inline)) {
      // bytes 0..3 -> 16-bit fields 0..3
      unsigned long long x = w & 0xffffffffull;
      x = (x | (x << 16)) & 0x0000ffff0000ffffull;
      x = (x | (x << 8)) & m8;
      return x;
    };
    const unsigned long long c64[4] = {widen_lo(tot), widen_lo(tot >> 32), widen_lo(bef), widen_lo(bef >> 32)};
    // eight 32-bit words of two 16-bit fields each, summed over the wavefront
    uint32_t c[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      c[2 * r] = wave_sum_dpp(static_cast<uint32_t>(c64[r]));
      c[2 * r + 1] = wave_sum_dpp(static_cast<uint32_t>(c64[r] >> 32));
    }
    if (lane == 63) {
#pragma unroll
      for (int e = 0; e < kPackedE; ++e) {
        if (e < E) {
          // expert e: word (e >> 1) of the totals (words 4.. of the counts before)
          atomicAdd(&total[e], static_cast<int>((c[e >> 1] >> (16 * (e & 1))) & 0xffff));
          atomicAdd(&before[e], static_cast<int>((c[4 + (e >> 1)] >> (16 * (e & 1))) & 0xffff));
        }
      }
    }
  } else {
    auto count = [&](int i, int e) __attribute__((always_inline)) {
      if (e >= 0 && e < E) {
        atomicAdd(&total[e], 1);
        if (i < n_before) atomicAdd(&before[e], 1);
      }
    };
#pragma unroll
    for (int u = 0; u < kIdPre; ++u) {
      const int j = tid + kFusedThreads * u;
      if (j < n4) {
        int i4 = j + rot;
        if (i4 >= n4) i4 -= n4;
        count(4 * i4, iv[u].x);
        count(4 * i4 + 1, iv[u].y);
        count(4 * i4 + 2, iv[u].z);
        count(4 * i4 + 3, iv[u].w);
      }
    }
    for (int j = tid + kFusedThreads * kIdPre; j < n4; j += kFusedThreads) {
      int i4 = j + rot;
      if (i4 >= n4) i4 -= n4;
      const int4 v = reinterpret_cast<const int4*>(idx)[i4];
      count(4 * i4, v.x);
      count(4 * i4 + 1, v.y);
      count(4 * i4 + 2, v.z);
      count(4 * i4 + 3, v.w);
    }
    for (int i = 4 * n4 + tid; i < n_all; i += kFusedThreads) count(i, idx[i]);
  }
  }
  if (tid < nb_ent) ent[tid] = my_ent;
  __syncthreads();

  // 3. kept counts and their exclusive scan over experts (offsets)
  if (E <= 64) {
    // one wavefront, lane e = expert e: kept counts, then an inclusive scan
    // by shuffles (exclusive = inclusive - own)
    if (wave == 0) {
      const int tot = lane < E ? total[lane] : 0;
      const int kept = C < 0 ? tot : min(tot, C);
      int incl = kept;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      if (lane < E) {
        off[lane] = incl - kept;
        if (blockIdx.x == 0) {
          counts_routed[lane] = tot;
          counts_kept[lane] = kept;
          offsets[lane] = incl - kept;
        }
      }
      if (blockIdx.x == 0 && lane == E - 1) offsets[E] = incl;
    }
  } else {
  const int per = (E + kFusedThreads - 1) / kFusedThreads;
  const int e0 = tid * per, e1 = min(E, e0 + per);
  int run = 0;
  for (int e = e0; e < e1; ++e) {
    const int kept = C < 0 ? total[e] : min(total[e], C);
    off[e] = kept;
    run += kept;
    if (blockIdx.x == 0) {
      counts_routed[e] = total[e];
      counts_kept[e] = kept;
    }
  }
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
  if (blockIdx.x == 0 && e0 < E && e1 == E) offsets[E] = prefix;
  }
  __syncthreads();

  // 4. ranks of the block's entries: assignments to the same expert from
  //    earlier tokens (before the block, then inside it)
  if (tid < nb_ent) {
    const int e = ent[tid];
    int d = -1;
    if (e >= 0 && e < E) {
      int r = before[e];
      const int first_of_token = (tid / k) * k;
      for (int i = 0; i < first_of_token; ++i) r += ent[i] == e ? 1 : 0;
      if (C < 0 || r < C) {
        d = off[e] + r;
        // never true when the counts are consistent; keeps any fault out
        if (d >= n_all) d = -1;
        else perm_token[d] = t0 + tid / k;
      }
    }
    dest_pos[static_cast<size_t>(t0) * k + tid] = d;
    dst[tid] = d;
  }
  __syncthreads();

  // 5. store each row to its kept slots
  if (x) {
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int q = tid + kFusedThreads * u;
      if (q < nrow_vec) {
        const int ti = q / nvec;
        const int v = q - ti * nvec;
        for (int j = 0; j < k; ++j) {
          const int d = dst[ti * k + j];
          if (d >= 0) xp[static_cast<size_t>(d) * nvec + v] = rv[u];
        }
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
  const size_t row_bytes = copy_rows ? static_cast<size_t>(d) * dtype_bytes(x_dt) : 0;
  // The one-launch kernel holds one entry per thread (so at most kFusedThreads
  // slots of one token) and at most kFusedMaxVec 16-byte vectors of rows per
  // thread (so one row of at most kFusedMaxVec * kFusedThreads vectors); wider
  // rows or more slots per token take the count/rank/permute launches.
  if (static_cast<long>(T) * k <= kFusedMaxEntries && row_bytes % 16 == 0 && k <= kFusedThreads &&
      row_bytes / 16 <= static_cast<size_t>(kFusedMaxVec) * kFusedThreads) {
    // tokens per block: at most 16 row vectors per thread, at most 256 entries,
    // and about 1024 blocks when T allows (four per CU: the row loads of one
    // block overlap the index work and stores of the others)
    const int nvec = static_cast<int>(row_bytes / 16);
    int tpb = nvec > 0 ? (kFusedMaxVec * kFusedThreads) / nvec : kFusedThreads;
    tpb = min(tpb, kFusedThreads / k);
    tpb = min(tpb, max(1, (T + 1023) / 1024));
    tpb = max(tpb, 1);
    const int nq = (tpb * nvec + kFusedThreads - 1) / kFusedThreads;
    const int nblk = (T + tpb - 1) / tpb;
    const uint4* xv = copy_rows ? static_cast<const uint4*>(x) : nullptr;
    uint4* xpv = copy_rows ? static_cast<uint4*>(x_perm) : nullptr;
    // more than 8 experts and more than 4096 ids: count once per 256-token
    // block first (dispatch_count_kernel) instead of every id in every block
    const bool pre = E > kPackedE && static_cast<long>(T) * k > 4096;
    if (pre) {
      hipLaunchKernelGGL(dispatch_count_kernel, dim3(nb), dim3(kDsTok), 0, stream, topk_idx, T, k, E, bc);
      const int st = check_launch();
      if (st != MOE_OK) return st;
    }
#define MOE_FUSED(NQ, PRE)                                                                                       \
  hipLaunchKernelGGL((dispatch_fused_kernel<NQ, PRE>), dim3(nblk), dim3(kFusedThreads), 0, stream, topk_idx, T, \
                     k, E, capacity, tpb, xv, nvec, xpv, counts_routed, counts_kept, offsets, dest_pos,          \
                     perm_token, static_cast<const int32_t*>(bc), nb)
    if (pre) {
      if (nq <= 4) MOE_FUSED(4, true);
      else if (nq <= 8) MOE_FUSED(8, true);
      else MOE_FUSED(16, true);
    } else {
      if (nq <= 4) MOE_FUSED(4, false);
      else if (nq <= 8) MOE_FUSED(8, false);
      else MOE_FUSED(16, false);
    }
#undef MOE_FUSED
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
