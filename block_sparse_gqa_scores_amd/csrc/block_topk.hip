// Index branch, selection step: for every (query, group) row keep the local
// block plus the k-1 best earlier blocks by block score, lower block index
// first on equal scores, and emit them in ascending block order, padded with
// -1 (Sparse Attention Part II, section 3.2: one slot reserved for the local
// block; section 4.2: exact top-k with a consistent tie rule; MiniMax Sparse
// Attention blog: the Top-k works on raw scores, with no exponential).
//
// One wavefront per row.  Scores are compared as order-preserving unsigned
// keys.  A cutoff is taken first: the (k-1)-th largest of the 64 per-lane
// maxima.  It cannot exceed the row's (k-1)-th largest score (the conservative
// filter of section 4.2), so every block of the answer passes it and the exact
// threshold is found among the few survivors.  Both order statistics come
// from a bitonic sort across the wave's 64 lanes (vector work only); when more
// than 64 blocks survive, the threshold is found by a most-significant-bit
// first search whose counts are wave ballots, over the survivor buffer or,
// past its capacity (massive ties), over the whole row.
#include "device_common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr int kThreads = 256;  // 4 rows per workgroup
constexpr int kCap = 256;      // survivor buffer per row (4 per lane)

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// The wave's 64 values (one per lane) sorted in descending order: lane l
// returns the l-th largest.  A bitonic network; every step is one cross-lane
// exchange, a compare and a select.
__device__ __forceinline__ uint32_t wave_sort_desc(uint32_t v, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)v, j, 64);
      const bool desc = (lane & k) == 0;  // direction of this lane's k-run
      const bool low = (lane & j) == 0;   // lower lane of the exchanged pair
      v = (low == desc) ? max(v, o) : min(v, o);
    }
  }
  return v;
}

__device__ __forceinline__ uint32_t lane_value(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Largest T with #{x >= T} >= kk over the values the callback exposes.
// count(cand) must return the wave-wide number of values >= cand.
template <class Count>
__device__ __forceinline__ uint32_t kth_largest(int kk, Count count) {
  uint32_t prefix = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    if (count(cand) >= kk) prefix = cand;
  }
  return prefix;
}

__global__ __launch_bounds__(kThreads) void block_topk_kernel(const float* __restrict__ bm,
                                                              int32_t* __restrict__ out_idx,
                                                              int n_rows, int S_q, int S_k,
                                                              int n_blk, int topk) {
  __shared__ uint32_t cand_x[4][kCap];
  __shared__ int32_t cand_j[4][kCap];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const long row = (long)blockIdx.x * 4 + wave;
  if (row >= n_rows) return;  // wave-uniform; no workgroup barrier below
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  const int i = (int)(row % S_q);
  const int local = (i + S_k - S_q) / 128;
  const int kk = topk - 1;      // slots the indexer fills
  const int n_c = local;        // candidates 0 .. local-1
  const float* x = bm + row * (long)n_blk;
  int32_t* out = out_idx + row * (long)topk;

  if (kk == 0) {  // k = 1: the local block alone
    if (lane == 0) out[0] = local;
    return;
  }
  if (n_c <= kk) {  // every earlier block fits: keep them all
    for (int e = lane; e < topk; e += 64) out[e] = e <= local ? e : -1;
    return;
  }

  // Cutoff: the kk-th largest of the per-lane maxima (kk <= 63).
  uint32_t lmax = 0;
  {
    int j = lane;
    for (; j + 192 < n_c; j += 256) {  // four loads in flight
      const float a0 = x[j], a1 = x[j + 64], a2 = x[j + 128], a3 = x[j + 192];
      lmax = max(max(lmax, max(order_key(a0), order_key(a1))), max(order_key(a2), order_key(a3)));
    }
    for (; j < n_c; j += 64) lmax = max(lmax, order_key(x[j]));
  }
  const uint32_t cut = lane_value(wave_sort_desc(lmax, lane), kk - 1);

  // Survivors >= cut, compacted in index order.
  int total = 0;
  for (int base = 0; base < n_c; base += 64) {
    const int j = base + lane;
    const uint32_t key = j < n_c ? order_key(x[j]) : 0u;
    const bool keep = j < n_c && key >= cut;
    const uint64_t m = ballot(keep);
    if (keep) {
      const int pos = total + __popcll(m & lt);
      if (pos < kCap) {
        cand_x[wave][pos] = key;
        cand_j[wave][pos] = j;
      }
    }
    total += __popcll(m);
  }

  uint32_t T;
  int need_eq;
  int written = 0;
  if (total <= 64) {
    // One survivor per lane: the threshold by sorting them.
    const uint32_t key = lane < total ? cand_x[wave][lane] : 0u;
    T = lane_value(wave_sort_desc(key, lane), kk - 1);
    need_eq = kk - __popcll(ballot(lane < total && key > T));
    const bool is_gt = lane < total && key > T;
    const bool is_eq = lane < total && key == T;
    const uint64_t em = ballot(is_eq);
    const bool sel = is_gt || (is_eq && __popcll(em & lt) < need_eq);
    const uint64_t sm = ballot(sel);
    if (sel) out[__popcll(sm & lt)] = cand_j[wave][lane];
  } else if (total <= kCap) {
    uint32_t reg[kCap / 64];
#pragma unroll
    for (int q = 0; q < kCap / 64; ++q) {
      const int p = q * 64 + lane;
      reg[q] = p < total ? cand_x[wave][p] : 0u;
    }
    auto count_ge = [&](uint32_t c) {
      int s = 0;
#pragma unroll
      for (int q = 0; q < kCap / 64; ++q) s += __popcll(ballot(reg[q] >= c));
      return s;
    };
    T = kth_largest(kk, count_ge);
    const int gt = (T == 0xFFFFFFFFu) ? 0 : count_ge(T + 1);
    need_eq = kk - gt;
    int seen_eq = 0;
    for (int base = 0; base < total && written < kk; base += 64) {
      const int p = base + lane;
      const uint32_t key = p < total ? cand_x[wave][p] : 0u;
      const bool is_gt = p < total && key > T;
      const bool is_eq = p < total && key == T;
      const uint64_t em = ballot(is_eq);
      const bool sel = is_gt || (is_eq && seen_eq + __popcll(em & lt) < need_eq);
      const uint64_t sm = ballot(sel);
      if (sel) out[written + __popcll(sm & lt)] = cand_j[wave][p];
      seen_eq += __popcll(em);
      written += __popcll(sm);
    }
  } else {
    // Massive ties: exact search and selection over the whole row.
    auto count_ge = [&](uint32_t c) {
      int s = 0;
      for (int base = 0; base < n_c; base += 64) {
        const int j = base + lane;
        s += __popcll(ballot(j < n_c && order_key(x[j]) >= c));
      }
      return s;
    };
    T = kth_largest(kk, count_ge);
    const int gt = (T == 0xFFFFFFFFu) ? 0 : count_ge(T + 1);
    need_eq = kk - gt;
    int seen_eq = 0;
    for (int base = 0; base < n_c && written < kk; base += 64) {
      const int j = base + lane;
      const uint32_t key = j < n_c ? order_key(x[j]) : 0u;
      const bool is_gt = j < n_c && key > T;
      const bool is_eq = j < n_c && key == T;
      const uint64_t em = ballot(is_eq);
      const bool sel = is_gt || (is_eq && seen_eq + __popcll(em & lt) < need_eq);
      const uint64_t sm = ballot(sel);
      if (sel) out[written + __popcll(sm & lt)] = j;
      seen_eq += __popcll(em);
      written += __popcll(sm);
    }
  }
  if (lane == 0) out[kk] = local;  // the local block is the largest index
}

}  // namespace

hipError_t launch_block_topk(const float* bm, int32_t* idx, int batch, int S_q, int S_k,
                             int H_kv, int n_blk, int topk, hipStream_t stream) {
  const long n_rows = (long)batch * H_kv * S_q;
  const long grid = (n_rows + 3) / 4;
  hipLaunchKernelGGL(block_topk_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, bm, idx,
                     (int)n_rows, S_q, S_k, n_blk, topk);
  return hipGetLastError();
}

}  // namespace msa
