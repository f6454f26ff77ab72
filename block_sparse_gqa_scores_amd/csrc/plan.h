// Host-side planning of the KV-stationary entry points: the workspace layout
// of each (bucket arrays, per-edge records, cross-chunk sums) and the query
// chunk that fits a caller's workspace.  Host code only, so it builds with
// any C++17 compiler (the sanitizer builds of the tests use g++); the
// kernels that fill these arrays are in the .hip files.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "kernels.h"

namespace msa {
namespace edges {

constexpr int kThreads = 256;  // threads per workgroup of the edge kernels
constexpr int kD = 128;         // head dim
constexpr int kBlock = 128;     // keys per block
constexpr int kSubTiles = 16;   // 4-wave sub-tiles per work item of the backward kernels
// 4-wave sub-tiles per forward work item: twice the backward's, so a bucket's
// K/V tiles are loaded for up to 512 edges (G = 8); measured 1.7 % faster for
// the partial kernel on 32K than 256, 128 was 3 % slower.
constexpr int kSubTilesFwd = 2 * kSubTiles;
constexpr int kScanPerWg = 1024;
// Bytes of per-edge records per designed chunk: a 128K prefill runs every
// entry point in one chunk (each further chunk rebuilds the buckets and
// reloads K/V; 16 GiB took 2-3 chunks there, measured 3-9 % slower), while
// the workspace stays a small part of 288 GB of HBM.
constexpr size_t kPartBudget = size_t(48) << 30;
constexpr int kBuildQueries = 256;   // queries per bucket-build workgroup
constexpr int kHistBins = 8192;      // widest row whose histogram lives in LDS
constexpr int kMinWindow = 2048;     // smallest query window (a multiple of kBuildQueries)
constexpr int kMaxWindow = 16384;    // largest query window (bounds a bucket's edge count)

// Byte offsets inside a workspace, and the bucket geometry of one chunk.
struct Layout {
  int Qc, QT, n_scan_wg;
  long NB, E, T;
  int W, n_win;
  size_t counts, cursor, offsets, tile_off, blk_sums, edges, work, part_stat, part_o, total;
  size_t kl_rec, kl_wsum, lse_t;  // alignment-loss layout only
  int n_kl_wg;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int grid_cap(long n, int per) {
  long g = (n + per - 1) / per;
  return (int)std::max(1L, std::min(g, 65536L));
}

// Default query chunk: the largest multiple of 128 queries (or all of them)
// whose per-edge records, `per_query` bytes for each query, fit kPartBudget.
inline int default_chunk(int S_q, size_t per_query) {
  long qc = (long)(kPartBudget / std::max<size_t>(per_query, 1));
  if (qc >= 128) qc -= qc % 128;
  return (int)std::max(1L, std::min<long>(qc, S_q));
}

// The query chunk used with a caller workspace of `budget` bytes: qc_max when
// total(qc_max) fits, otherwise the largest Qc < qc_max that fits, rounded
// down to whole 128-query blocks once it reaches 128; 0 when not even one
// query fits.  total(Qc) is the workspace of chunks of Qc queries; it does
// not decrease with Qc below qc_max (a one-chunk layout may drop the
// cross-chunk sums, which is why qc_max is tried first).
template <class Total>
int fit_chunk(int qc_max, size_t budget, Total total) {
  if (total(qc_max) <= budget) return qc_max;
  int lo = 0, hi = qc_max - 1;
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (total(mid) <= budget) lo = mid;
    else hi = mid - 1;
  }
  if (lo >= 128) lo -= lo % 128;
  return lo;
}

// Bucket geometry and the build arrays for a chunk of L.Qc queries (L.QT set
// by the caller); returns the offset past them.
size_t layout_build(Layout& L, const AttnShape& s);

}  // namespace edges

// The fused index scan keeps this many earlier blocks per row in registers
// (the selection kernel of the index scan), so it covers topk <= kSelectKeep + 1.
constexpr int kSelectKeep = 15;

// Attention forward: bucket arrays, then per-edge partial records.
edges::Layout make_fwd_layout(const AttnShape& s, int Qc);
int fwd_chunk(const AttnShape& s, size_t ws_bytes);

// Main backward: bucket arrays, per-row statistics, per-edge dq records, and
// fp32 dk / dv sums when there is more than one chunk.
// A (group, block) with more than `seg` sub-tiles in a chunk is split into
// segments whose fp32 dK / dV parts are summed afterwards: seg is the
// chunk's expected sub-tiles spread over kSegSpread work items, at least
// kSegMin.
constexpr long kSegSpread = 4096;
constexpr long kSegMin = 512;
struct BwdLayout {
  edges::Layout L;
  size_t stat, dq_rec, dq_sc, dk_acc, dv_acc, blk_t, blk_item, blk_part, items, part, total;
  int chunks, seg;
  bool seg_on;           // some block of a chunk can hold more than seg sub-tiles
  long n_items, n_part;  // bounds on work items and on partial slots
};
BwdLayout make_bwd_layout(const AttnShape& s, int Qc);
int bwd_chunk(const AttnShape& s, size_t ws_bytes);

// Alignment-loss backward: bucket arrays, per-edge dq_idx records and g rows,
// per-group fp32 dk_idx parts and their flags, grouped main-branch LSE.
struct KlBwdLayout {
  edges::Layout L;
  size_t rec, rec_sc, g_rec, dk_part, dk_flag, lse_t, total;
};
KlBwdLayout make_kl_bwd_layout(const AttnShape& s, int D_idx, int Qc);
int kl_bwd_chunk(const AttnShape& s, int D_idx, size_t ws_bytes);

// Both backward passes in one call (msa_backward), on the same query chunks
// and edge buckets: the main backward's layout, then the loss backward's
// dq_idx records, g rows, per-group fp32 dk_idx parts and their flags, and
// the grouped main-branch LSE.
struct FusedBwdLayout {
  BwdLayout B;
  size_t rec, rec_sc, g_rec, dk_part, dk_flag, lse_t, total;
};
FusedBwdLayout make_fused_bwd_layout(const AttnShape& s, int D_idx, int Qc);
int fused_bwd_chunk(const AttnShape& s, int D_idx, size_t ws_bytes);

// Alignment-loss forward: one chunk (32 bytes of records per edge).
edges::Layout make_kl_layout(const AttnShape& s);

}  // namespace msa
