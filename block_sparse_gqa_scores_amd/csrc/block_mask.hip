// Block-mask form of a selection (Sparse Attention Part II, section 4.3): the
// blocks a (query, group) row visits become flags packed 32 to an unsigned
// word, block j at bit j mod 32 of word floor(j / 32), bits past the last
// block left zero; a traversal recovers the blocks from each word's popcount
// and the position of its rank-th set bit.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr int kThreads = 256;

// One thread per (row, word): OR in the row's entries that fall in the word.
// Entries outside [0, n_blk) (the -1 padding, or anything else) are skipped,
// so no bit past the last block is ever set.
__global__ __launch_bounds__(kThreads) void block_mask_kernel(const int32_t* __restrict__ sel,
                                                              uint32_t* __restrict__ mask,
                                                              long n_rows, int topk, int n_blk,
                                                              int n_words) {
  const long x = (long)blockIdx.x * kThreads + threadIdx.x;
  if (x >= n_rows * n_words) return;
  const long row = x / n_words;
  const int w = (int)(x - row * n_words);
  const int32_t* s = sel + row * topk;
  uint32_t word = 0;
  for (int e = 0; e < topk; ++e) {
    const int j = s[e];
    if (j >= 0 && j < n_blk && (j >> 5) == w) word |= 1u << (j & 31);
  }
  mask[x] = word;
}

// A wave takes 64 / SEG rows of at most SEG words each (SEG a power of two
// <= 64; rows wider than 64 words loop over 64-word chunks with SEG = 64).
// Inside a row's segment, lane l takes word l (then l + SEG, ...); a prefix
// sum of the words' popcounts across the segment gives each word's first
// output position, and the lane then emits its word's set bits in rank order
// (the lowest set bit, then clear it: the rank-th pass finds the rank-th set
// bit).  Positions past `cap` are dropped; the rest of the row is padded with
// -1.  Bits past the last block are ignored.
template <int SEG>
__global__ __launch_bounds__(kThreads) void mask_blocks_kernel(const uint32_t* __restrict__ mask,
                                                               int32_t* __restrict__ sel,
                                                               long n_rows, int n_blk, int n_words, int cap) {
  constexpr int RPW = 64 / SEG;  // rows per wave
  const int lane = threadIdx.x & 63;
  const int sl = lane % SEG;     // lane within the row's segment
  const long row = ((long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * RPW + lane / SEG;
  const bool live = row < n_rows;
  const uint32_t* m = mask + (live ? row : 0) * n_words;
  int32_t* out = sel + (live ? row : 0) * cap;
  int base = 0;  // set bits in the words already handled (the same in the whole segment)
  for (int w0 = 0; w0 < n_words; w0 += SEG) {
    const int w = w0 + sl;
    uint32_t word = (live && w < n_words) ? m[w] : 0u;
    if (w == n_words - 1 && (n_blk & 31)) word &= (1u << (n_blk & 31)) - 1u;  // bits past the last block
    const int cnt = __popc(word);
    int incl = cnt;  // inclusive prefix sum over the segment
#pragma unroll
    for (int o = 1; o < SEG; o <<= 1) {
      const int t = __shfl_up(incl, o, SEG);
      if (sl >= o) incl += t;
    }
    int pos = base + incl - cnt;
    while (word != 0u && pos < cap) {
      const int bit = __ffs(word) - 1;
      out[pos++] = 32 * w + bit;
      word &= word - 1u;
    }
    base += __shfl(incl, SEG - 1, SEG);
  }
  if (live)
    for (int e = min(base, cap) + sl; e < cap; e += SEG) out[e] = -1;
}

}  // namespace

hipError_t launch_block_mask(const int32_t* sel, uint32_t* mask, long n_rows, int topk, int n_blk,
                             hipStream_t stream) {
  const int n_words = (n_blk + 31) / 32;
  const long n = n_rows * n_words;
  hipLaunchKernelGGL(block_mask_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     stream, sel, mask, n_rows, topk, n_blk, n_words);
  return hipGetLastError();
}

hipError_t launch_mask_blocks(const uint32_t* mask, int32_t* sel, long n_rows, int n_blk, int cap,
                              hipStream_t stream) {
  const int n_words = (n_blk + 31) / 32;
  auto go = [&](auto seg) {
    constexpr int SEG = decltype(seg)::value;
    const long rows_per_wg = (kThreads / 64) * (64 / SEG);
    hipLaunchKernelGGL(mask_blocks_kernel<SEG>, dim3((unsigned)((n_rows + rows_per_wg - 1) / rows_per_wg)),
                       dim3(kThreads), 0, stream, mask, sel, n_rows, n_blk, n_words, cap);
  };
  if (n_words <= 4) go(std::integral_constant<int, 4>{});
  else if (n_words <= 8) go(std::integral_constant<int, 8>{});
  else if (n_words <= 16) go(std::integral_constant<int, 16>{});
  else if (n_words <= 32) go(std::integral_constant<int, 32>{});
  else go(std::integral_constant<int, 64>{});
  return hipGetLastError();
}

}  // namespace msa
