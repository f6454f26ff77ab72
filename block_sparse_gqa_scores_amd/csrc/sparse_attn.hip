// Main branch: exact block-sparse causal GQA attention over the selected
// blocks (Sparse Attention Part II, section 3.2: every query head of a group
// attends to the visible tokens of the kept blocks with its own weights;
// section 2: the softmax is normalised inside the selection; section 4.1:
// scores and weights stay on chip, only statistics and the output leave).
//
// Schedule.  Neighbouring queries pick largely unrelated blocks, so a kernel
// that walks each query's own 16 blocks re-reads every KV block once per
// (query, group).  Here the edges (query i, group g, selected block j) are
// bucketed by (b, g, j) instead: one workgroup loads K_j and V_j of group g
// into LDS once and runs every query of its bucket against them, all G heads
// of a query sharing the load (section 3.2: fixed-size blocks allow the group's
// heads share KV loads).  Each edge leaves a partial result: the output
// normalised over the block's visible keys and its log-sum-exp.  A merge
// kernel then combines each query's partials, which is exactly the softmax
// over the union of its blocks.  Decode (one query per sequence) is the same
// computation with one query per bucket, i.e. split-KV.
//
// Buckets are further split by query window: bucket (b, g, w, j) holds the
// edges of queries in window w of the chunk, and work items run in bucket
// order, so the workgroups in flight at any time gather the Q rows of one or
// two windows, which stay in L2, instead of Q rows from the whole sequence.
// The window is sized so that a bucket still averages about QT edges.
//
// Work-list construction: counts per bucket, exclusive scans of edges and of
// work items, edge scatter (atomics choose positions inside a bucket only;
// every edge's arithmetic is independent of its position, so results do not
// depend on that order), and one work item per up-to-QT edges of a bucket.
#include "edge_buckets.h"

namespace msa {
using namespace edges;
namespace {

constexpr int kVStride = kBlock + 4;  // bf16 per row of the transposed V tile
constexpr long kMergePairRows = 1 << 16;  // from this many rows on, two merge rows per wave

// Record of one slot: its query's G x D partial outputs O_e / l_e as 12-bit
// codes (q12_code: each head's row scaled by its own largest magnitude), 1.5
// bytes a value, plus the row's LSE and scale in part_stat.
//
// The MFMA output puts O[hh][d] of a query in lane (row hh, half h) at
// register v = 4 rq + c of tile dt, with d = 32 dt + 8 rq + 4 h + c.  Piece
// f = (dt G + hh) 2 + h is the 16 values of one lane's tile, 24 bytes: codes
// 0..7 and 8..15 packed by q12_pack8 into dwords d0 d1 d2 and d3 d4 d5;
// d0..d3 go to area A of the record (16 bytes per piece) and d4 d5 to area B
// (8 bytes per piece).  The 2 G lanes of one query write 32 G contiguous
// bytes of A and 16 G of B per store instruction.
__device__ __forceinline__ int piece_of(int G, int dt, int hh, int h) { return (dt * G + hh) * 2 + h; }

__global__ void zero_kernel(int32_t* a, long n) {
  for (long x = (long)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (long)gridDim.x * blockDim.x)
    a[x] = 0;
}

// Bucket build with per-workgroup LDS histograms: a workgroup takes
// kBuildQueries queries of one (b, g), counts their edges per block in LDS and
// touches global memory once per distinct block.  Used when the histogram of
// n_blk bins fits in LDS; count_kernel / fill_kernel below cover wider rows.
// Rows below p.dense_q are attended by the dense tiles (dense_tile) and get no edges.
__device__ __forceinline__ bool edge_ok(const Params& p, int i, int j) {
  return i >= p.dense_q && j >= 0 && j <= (i + p.S_k - p.S_q) / kBlock;
}

__global__ __launch_bounds__(256) void bucket_count_kernel(Params p) {
  extern __shared__ int32_t hist[];  // n_blk
  const int tiles = (p.Qc + kBuildQueries - 1) / kBuildQueries;
  const int bg = blockIdx.x / tiles;
  const int il0 = (blockIdx.x - bg * tiles) * kBuildQueries;
  const int nq = min(min(kBuildQueries, p.Qc - il0), p.S_q - (p.q0 + il0));
  if (nq <= 0) return;  // uniform
  for (int x = threadIdx.x; x < p.n_blk; x += 256) hist[x] = 0;
  __syncthreads();
  const int32_t* sel = p.idx + ((long)bg * p.S_q + p.q0 + il0) * p.topk;
  for (int s = threadIdx.x; s < nq * p.topk; s += 256) {
    const int j = sel[s];
    if (edge_ok(p, p.q0 + il0 + s / p.topk, j)) atomicAdd(&hist[j], 1);
  }
  __syncthreads();
  int32_t* cnt = p.counts + ((long)bg * p.n_win + il0 / p.W) * p.n_blk;
  for (int x = threadIdx.x; x < p.n_blk; x += 256)
    if (hist[x]) atomicAdd(&cnt[x], hist[x]);
}

__global__ __launch_bounds__(256) void bucket_fill_kernel(Params p) {
  extern __shared__ int32_t lds[];  // hist[n_blk], base[n_blk]
  int32_t* hist = lds;
  int32_t* base = lds + p.n_blk;
  const int tiles = (p.Qc + kBuildQueries - 1) / kBuildQueries;
  const int bg = blockIdx.x / tiles;
  const int il0 = (blockIdx.x - bg * tiles) * kBuildQueries;
  const int nq = min(min(kBuildQueries, p.Qc - il0), p.S_q - (p.q0 + il0));
  if (nq <= 0) return;  // uniform
  for (int x = threadIdx.x; x < p.n_blk; x += 256) hist[x] = 0;
  __syncthreads();
  const int32_t* sel = p.idx + ((long)bg * p.S_q + p.q0 + il0) * p.topk;
  for (int s = threadIdx.x; s < nq * p.topk; s += 256) {
    const int j = sel[s];
    if (edge_ok(p, p.q0 + il0 + s / p.topk, j)) atomicAdd(&hist[j], 1);
  }
  __syncthreads();
  const long b0 = ((long)bg * p.n_win + il0 / p.W) * p.n_blk;
  for (int x = threadIdx.x; x < p.n_blk; x += 256) {
    const int c = hist[x];
    if (c) base[x] = p.offsets[b0 + x] + atomicAdd(&p.cursor[b0 + x], c);
    hist[x] = 0;
  }
  __syncthreads();
  for (int s = threadIdx.x; s < nq * p.topk; s += 256) {
    const int j = sel[s];
    if (edge_ok(p, p.q0 + il0 + s / p.topk, j)) {
      const int pos = base[j] + atomicAdd(&hist[j], 1);
      p.edges[pos] = (int32_t)slot_of(p, bg, il0 + s / p.topk, s % p.topk);
    }
  }
}

__global__ void count_kernel(Params p) {
  const long n = (long)p.B * p.H_kv * p.Qc * p.topk;
  for (long s = (long)blockIdx.x * blockDim.x + threadIdx.x; s < n; s += (long)gridDim.x * blockDim.x) {
    const int e = (int)(s % p.topk);
    const long r = s / p.topk;
    const int il = (int)(r % p.Qc);
    const int bg = (int)(r / p.Qc);
    const int i = p.q0 + il;
    if (i >= p.S_q) continue;
    const int j = p.idx[((long)bg * p.S_q + i) * p.topk + e];
    if (edge_ok(p, i, j))
      atomicAdd(&p.counts[((long)bg * p.n_win + il / p.W) * p.n_blk + j], 1);
  }
}

// Exclusive scans of edges and work items per bucket, stage 1: per-workgroup.
__global__ __launch_bounds__(256) void scan_local_kernel(Params p) {
  __shared__ int32_t se[256], st[256];
  const int tid = threadIdx.x;
  const long base = (long)blockIdx.x * kScanPerWg + tid * 4;
  int ce[4], ct[4], sum_e = 0, sum_t = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const long x = base + u;
    const int c = x < p.NB ? p.counts[x] : 0;
    ce[u] = sum_e;
    ct[u] = sum_t;
    sum_e += c;
    sum_t += (c + p.QT - 1) / p.QT;
  }
  se[tid] = sum_e;
  st[tid] = sum_t;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {  // Hillis-Steele inclusive scan
    const int ae = tid >= d ? se[tid - d] : 0;
    const int at = tid >= d ? st[tid - d] : 0;
    __syncthreads();
    se[tid] += ae;
    st[tid] += at;
    __syncthreads();
  }
  const int pe = se[tid] - sum_e, pt = st[tid] - sum_t;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const long x = base + u;
    if (x < p.NB) {
      p.offsets[x] = pe + ce[u];
      p.tile_off[x] = pt + ct[u];
    }
  }
  if (tid == 255) {
    p.blk_sums[2 * blockIdx.x] = se[255];
    p.blk_sums[2 * blockIdx.x + 1] = st[255];
  }
}

// Stage 2: one workgroup scans the per-workgroup totals (exclusive, in place)
// and writes the grand totals at offsets[NB], tile_off[NB].
__global__ __launch_bounds__(256) void scan_blocks_kernel(Params p, int n_wg) {
  __shared__ int32_t se[256], st[256];
  __shared__ int32_t carry[2];
  const int tid = threadIdx.x;
  if (tid == 0) carry[0] = carry[1] = 0;
  __syncthreads();
  for (int base = 0; base < n_wg; base += 256) {
    const int x = base + tid;
    const int ve = x < n_wg ? p.blk_sums[2 * x] : 0;
    const int vt = x < n_wg ? p.blk_sums[2 * x + 1] : 0;
    se[tid] = ve;
    st[tid] = vt;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int ae = tid >= d ? se[tid - d] : 0;
      const int at = tid >= d ? st[tid - d] : 0;
      __syncthreads();
      se[tid] += ae;
      st[tid] += at;
      __syncthreads();
    }
    const int ce = carry[0], ct = carry[1];
    if (x < n_wg) {
      p.blk_sums[2 * x] = ce + se[tid] - ve;
      p.blk_sums[2 * x + 1] = ct + st[tid] - vt;
    }
    __syncthreads();
    if (tid == 255) {
      carry[0] = ce + se[255];
      carry[1] = ct + st[255];
    }
    __syncthreads();
  }
  if (tid == 0) {
    p.offsets[p.NB] = carry[0];
    p.tile_off[p.NB] = carry[1];
  }
}

// Stage 3: add the workgroup prefix; also emits the work items of each bucket.
__global__ __launch_bounds__(256) void scan_add_kernel(Params p) {
  const long base = (long)blockIdx.x * kScanPerWg;
  const int add_e = p.blk_sums[2 * blockIdx.x];
  const int add_t = p.blk_sums[2 * blockIdx.x + 1];
  for (int u = threadIdx.x; u < kScanPerWg; u += 256) {
    const long x = base + u;
    if (x >= p.NB) break;
    const int oe = p.offsets[x] + add_e;
    const int ot = p.tile_off[x] + add_t;
    p.offsets[x] = oe;
    p.tile_off[x] = ot;
    const int c = p.counts[x];
    for (int t = 0, s = 0; s < c; ++t, s += p.QT) p.work[ot + t] = make_int2((int)x, s);
  }
}

__global__ void fill_kernel(Params p) {
  const long n = (long)p.B * p.H_kv * p.Qc * p.topk;
  for (long s = (long)blockIdx.x * blockDim.x + threadIdx.x; s < n; s += (long)gridDim.x * blockDim.x) {
    const int e = (int)(s % p.topk);
    const long r = s / p.topk;
    const int il = (int)(r % p.Qc);
    const int bg = (int)(r / p.Qc);
    const int i = p.q0 + il;
    if (i >= p.S_q) continue;
    const int j = p.idx[((long)bg * p.S_q + i) * p.topk + e];
    if (edge_ok(p, i, j)) {
      const long bucket = ((long)bg * p.n_win + il / p.W) * p.n_blk + j;
      const int pos = p.offsets[bucket] + atomicAdd(&p.cursor[bucket], 1);
      p.edges[pos] = (int32_t)s;
    }
  }
}

// K_j and V_j of (b, g) into LDS: K row-major [key][16 chunks], chunk c of
// key r at c ^ (r & 15); V transposed to [d][key] with padded rows (both the
// transposing writes and the operand reads are free of bank conflicts).  Keys
// past S_k are masked for every query (their weight is exactly 0), so a
// clamped row is read instead of branching.
__device__ __forceinline__ void load_kv_tile(const Params& p, int b, int g, int j, u32x4* ktile, uint32_t* vt,
                                             int tid) {
  const size_t row_stride = (size_t)p.H_kv * kD;
  const uint16_t* kb = p.k + ((size_t)b * p.S_k * p.H_kv + g) * kD;
  const uint16_t* vb = p.v + ((size_t)b * p.S_k * p.H_kv + g) * kD;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int qd = it * kThreads + tid;
    const int row = qd >> 4, c = qd & 15;
    const int s = min(j * kBlock + row, p.S_k - 1);
    ktile[row * 16 + (c ^ (row & 15))] = *reinterpret_cast<const u32x4*>(kb + (size_t)s * row_stride + 8 * c);
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int u = it * kThreads + tid;
    const int kp = (u & 15) + 16 * ((u >> 6) & 3);
    const int d0 = ((u >> 4) & 3) + 4 * ((u >> 8) & 3);
    const int s0 = min(j * kBlock + 2 * kp, p.S_k - 1);
    const int s1 = min(j * kBlock + 2 * kp + 1, p.S_k - 1);
    const u32x4 lo = *reinterpret_cast<const u32x4*>(vb + (size_t)s0 * row_stride + 8 * d0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(vb + (size_t)s1 * row_stride + 8 * d0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = (e & 1) ? (lo[e >> 1] >> 16) : (lo[e >> 1] & 0xFFFFu);
      const uint32_t c2 = (e & 1) ? (hi[e >> 1] & 0xFFFF0000u) : (hi[e >> 1] << 16);
      vt[((8 * d0 + e) * kVStride + 2 * kp) >> 1] = a | c2;
    }
  }
}

// S^T = K Q^T of one 32-row sub-tile (Q rows in qb, this lane's row n, half
// h) against the block in ktile, as a software pipeline: one MFMA per step
// (step st = 8 mt + ks: K rows 32 mt + n, k-step ks) with a scheduling
// barrier between steps, each K fragment read three steps ahead into a ring
// of four, and the row maximum of a finished 32-key chunk taken during the
// next chunk's MFMAs.  Register r of chunk mt holds key 32 mt + 8 (r / 4) +
// 4 h + r % 4; when need_mask (wave-uniform), keys above lim are set to
// -inf (one branch per finished chunk).  Returns the row's maximum.
__device__ __forceinline__ float s_block(const u32x4* ktile, const u32x4 (&qb)[8], int n, int h, bool need_mask,
                                         int lim, f32x16 (&sacc)[4]) {
  auto mask_chunk = [&](auto MT) {
    constexpr int mt = decltype(MT)::value;
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (mt * 32 + 8 * (r >> 2) + (r & 3) > lim) sacc[mt][r] = neg_inf();
    }
  };
  float mx = neg_inf();
  auto max2 = [&](auto MT, auto R) {
    constexpr int mt = decltype(MT)::value, r = decltype(R)::value;
    mx = max3f(sacc[mt][r], sacc[mt][r + 1], mx);
  };
  // Row 32 mt + n keeps its 16-byte chunks swizzled by n & 15.
  const u32x4* klane = ktile + n * 16;
  auto kfrag = [&](int st) { return klane[(st >> 3) * 512 + ((2 * (st & 7) + h) ^ (n & 15))]; };
  u32x4 ring[4];
  static_for<0, 3>([&](auto P) { ring[P] = kfrag(P); });
  static_for<0, 32>([&](auto S) {
    constexpr int st = decltype(S)::value, mt = st / 8, ks = st % 8;
    if constexpr (st + 3 < 32) ring[(st + 3) % 4] = kfrag(st + 3);
    sacc[mt] = mfma32x32x16(ring[st % 4], qb[ks], ks == 0 ? zero16() : sacc[mt]);
    if constexpr (mt >= 1 && ks == 0) mask_chunk(std::integral_constant<int, mt - 1>{});
    if constexpr (mt >= 1) max2(std::integral_constant<int, mt - 1>{}, std::integral_constant<int, 2 * ks>{});
    __builtin_amdgcn_sched_barrier(0);
  });
  mask_chunk(std::integral_constant<int, 3>{});
  static_for<0, 8>([&](auto K) { max2(std::integral_constant<int, 3>{}, std::integral_constant<int, 2 * K>{}); });
  return halves_max(mx);
}

// P = 2^(S c + bias) in bf16 as the B operand of O^T = V^T P^T, and O^T added
// into oacc (from zero when ZERO): a software pipeline like s_block's, step
// st = 8 mt + 4 qq + dt over V^T[d][key] with d = 32 dt + n, keys 32 mt + 16 qq
// + 4 h + 0..3 and + 8..11 (one lane base plus compile-time offsets), the
// exponentials of chunk mt + 1 issued two values a step during chunk mt's
// MFMAs.  l gains this lane half's fp32 weights.
template <bool ZERO>
__device__ __forceinline__ void pv_block(const uint32_t* vt, const f32x16 (&sacc)[4], float c, float bias, int n,
                                         int h, float& l, f32x16 (&oacc)[4]) {
  u32x4 pb[4][2];
  auto exp2v = [&](auto MT, auto R) {
    constexpr int mt = decltype(MT)::value, r = decltype(R)::value;
    const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][r], c, bias));
    const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][r + 1], c, bias));
    l += e0;
    l += e1;
    pb[mt][r / 8][(r % 8) / 2] = pack_bf16x2(e0, e1);
  };
  static_for<0, 8>([&](auto K) { exp2v(std::integral_constant<int, 0>{}, std::integral_constant<int, 2 * K>{}); });
  const uint32_t* vlane = vt + n * (kVStride / 2) + 2 * h;
  auto vfrag = [&](int st) {
    const uint32_t* va = vlane + (st & 3) * 16 * kVStride + (st >> 3) * 16 + 8 * ((st >> 2) & 1);
    const uint2 a0 = *reinterpret_cast<const uint2*>(va);
    const uint2 a1 = *reinterpret_cast<const uint2*>(va + 4);
    return u32x4{a0.x, a0.y, a1.x, a1.y};
  };
  u32x4 ring[4];
  static_for<0, 3>([&](auto P) { ring[P] = vfrag(P); });
  static_for<0, 32>([&](auto S) {
    constexpr int st = decltype(S)::value, mt = st / 8, qq = (st / 4) % 2, dt = st % 4;
    if constexpr (st + 3 < 32) ring[(st + 3) % 4] = vfrag(st + 3);
    oacc[dt] = mfma32x32x16(ring[st % 4], pb[mt][qq], ZERO && mt == 0 && qq == 0 ? zero16() : oacc[dt]);
    if constexpr (mt < 3) exp2v(std::integral_constant<int, mt + 1>{}, std::integral_constant<int, 2 * (st % 8)>{});
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Rows whose local block is below topk (t < 128 topk): under the selection
// rule such a row takes every block of its causal prefix, so neighbouring
// queries share one union of at most topk blocks.  Their attention runs
// query-stationary, in the flash form of Sparse Attention Part II section
// 4.1: a workgroup takes 4 QW consecutive queries of one (b, g), each wave
// 32 MFMA rows (QW queries x G heads) with its Q rows in registers, and walks
// the blocks 0 .. (local block of the tile's last query) in order.  Each
// block's K and V pass through LDS once for the four waves (the group's heads
// share the load), and every row keeps its running max, sum and output in
// registers (online softmax), so O and the LSE are written directly, with no
// per-edge record and no merge.  A row takes only the blocks its own
// selection names (a caller's selection may be any subset holding the local
// block) and the causal mask on its own block; a wave skips a block none of
// its rows takes.  Rows past the dense range repeat the last one and store
// nothing.  The matrix phases are the partial kernel's pipelines.
template <int G>
__device__ __forceinline__ void dense_tile(const Params& p, int n_dense, int with_lse, int wg, u32x4* ktile,
                                           uint32_t* vt) {
  constexpr int QW = 32 / G;   // queries per wave
  constexpr int QWG = 4 * QW;  // queries per workgroup

  const int tiles = (n_dense + QWG - 1) / QWG;
  const int bg = wg / tiles;
  const int il0 = (wg - bg * tiles) * QWG;  // first query of the tile, in the chunk
  const int b = bg / p.H_kv;
  const int g = bg - b * p.H_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int n = lane & 31;  // MFMA row of this lane
  const int qi = n / G, hh = n - (n / G) * G;
  const int off = p.S_k - p.S_q;
  const int il = il0 + wave * QW + qi;
  const bool row_ok = il < n_dense;
  const int i = p.q0 + min(il, n_dense - 1);
  const int t = i + off;
  const int lrow = t / kBlock;
  uint64_t selm = 0;  // blocks this row's selection names (all below topk <= 64)
  {
    const int32_t* sel = p.idx + ((long)bg * p.S_q + i) * p.topk;
    for (int e = 0; e < p.topk; ++e) {
      const int j = sel[e];
      if (j >= 0 && j <= lrow) selm |= 1ull << j;
    }
  }
  const int jmax = (p.q0 + min(il0 + QWG, n_dense) - 1 + off) / kBlock;  // uniform
  u32x4 qb[8];
  {
    const uint16_t* qrow = p.q + ((size_t)b * p.S_q + i) * p.H_q * kD + (size_t)(g * G + hh) * kD + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qb[ks] = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
  }
  const float c = p.scale_log2;
  float m = neg_inf(), l = 0.f;  // running raw-score max and (per half) weight sum
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = zero16();

  for (int j = 0; j <= jmax; ++j) {
    __syncthreads();  // the previous block's LDS reads are done
    load_kv_tile(p, b, g, j, ktile, vt, tid);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const bool mine = (selm >> j) & 1;
    if (__builtin_amdgcn_ballot_w64(mine) == 0) continue;  // uniform: no row of this wave takes j
    // A row that does not take j has every key masked, its own block the
    // keys past t.
    const bool need_mask = __builtin_amdgcn_ballot_w64(!mine || j * kBlock + kBlock - 1 > t) != 0;
    f32x16 sacc[4];
    const float mx = s_block(ktile, qb, n, h, need_mask, mine ? t - j * kBlock - 4 * h : -1, sacc);
    // Online softmax: rescale what the earlier blocks left by 2^((m - m') c).
    const float m_new = __builtin_fmaxf(m, mx);
    const bool none = m_new == neg_inf();  // nothing visible yet for this row
    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f((m - m_new) * c);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    pv_block<false>(vt, sacc, c, none ? 0.f : -m_new * c, n, h, l, oacc);
  }
  l = halves_sum(l);
  if (!row_ok) return;
  // Register r of tile dt holds d = 32 dt + 8 (r / 4) + 4 h + r % 4 of the row.
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* orow = p.out + (((size_t)b * p.S_q + i) * p.H_q + g * G + hh) * kD + 4 * h;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      uint2 w;
      w.x = pack_bf16x2(oacc[dt][4 * r4] * inv, oacc[dt][4 * r4 + 1] * inv);
      w.y = pack_bf16x2(oacc[dt][4 * r4 + 2] * inv, oacc[dt][4 * r4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * r4) = w;
    }
  if (with_lse && h == 0)
    p.lse[((size_t)b * p.H_q + g * G + hh) * p.S_q + i] =
        (m * c + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f;
}

// One work item: (bucket (b, g, j), up to QT of its edges).
//
// Each wave takes QW queries x G heads = 32 MFMA rows per sub-tile.  Rows past
// the item's last edge are clamped onto that edge: they recompute and rewrite
// exactly the same values, which keeps every load and store unconditional (a
// fixed number of memory operations in flight, no exec-skip branches).  The Q
// rows of the next sub-tile are loaded while the current one computes.
//
// The first n_dense_wg workgroups of the launch are instead the dense tiles
// (dense_tile above): they are the longest, so they start first and the
// work items fill in around them.
template <int G>
__global__ __launch_bounds__(kThreads, 2) void attn_partial_kernel(Params p, int n_dense, int n_dense_wg,
                                                                   int with_lse) {
  constexpr int QW = 32 / G;  // queries per wave (32 MFMA rows = QW queries x G heads)
  constexpr int QT = kSubTilesFwd * 4 * QW;            // edges per work item
  __shared__ u32x4 ktile[kBlock * 16];                 // [key][16 chunks], swizzled
  __shared__ uint32_t vt[kD * kVStride / 2];           // [d][key] bf16, padded rows
  __shared__ int32_t s_slot[QT];                       // this item's edge slots

  if ((int)blockIdx.x < n_dense_wg) {  // uniform
    dense_tile<G>(p, n_dense, with_lse, blockIdx.x, ktile, vt);
    return;
  }
  const int w = blockIdx.x - n_dense_wg;
  if (w >= p.tile_off[p.NB]) return;  // uniform: past the last work item
  const int2 item = p.work[w];
  const int bucket = item.x;
  const int start = item.y;
  const int n_here = min(p.QT, p.counts[bucket] - start);
  const int ebase = p.offsets[bucket] + start;
  const int bgw = bucket / p.n_blk;
  const int j = bucket - bgw * p.n_blk;
  const int bg = bgw / p.n_win;
  const int b = bg / p.H_kv;
  const int g = bg - b * p.H_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;

  for (int x = tid; x < n_here; x += kThreads) s_slot[x] = p.edges[ebase + x];
  load_kv_tile(p, b, g, j, ktile, vt, tid);  // K_j, V_j of group g
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int off = p.S_k - p.S_q;
  const int n = lane & 31;          // MFMA row of this lane
  const int qi = n / G, hh = n - (n / G) * G;
  const size_t q_head_off = (size_t)(g * G + hh) * kD + 8 * h;

  // Row geometry of sub-tile `sub` for this lane (clamped onto the last edge).
  auto row_slot = [&](int sub) { return s_slot[min(sub + wave * QW + qi, n_here - 1)]; };
  auto q_of_slot = [&](int slot) { return p.q0 + (int)((slot / p.topk) % p.Qc); };
  auto load_q = [&](u32x4* dst, int i) {
    const uint16_t* qrow = p.q + ((size_t)b * p.S_q + i) * p.H_q * kD + q_head_off;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) dst[ks] = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
  };

  int slot = row_slot(0);
  int i = q_of_slot(slot);
  // One sub-tile on the Q rows in qb while the next sub-tile's Q rows load
  // into qn; false when this wave has no rows left (wave-uniform).  The loop
  // below alternates the two register sets instead of copying qn to qb.
  auto sub_tile = [&](int sub, const u32x4 (&qb)[8], u32x4 (&qn)[8]) -> bool {
    if (sub + wave * QW >= n_here) return false;
    const int slot_n = row_slot(sub + 4 * QW);
    const int i_n = q_of_slot(slot_n);
    load_q(qn, i_n);
    asm volatile("" ::: "memory");

    // The two matrix phases are the software pipelines of s_block and
    // pv_block.  Causal mask only where the block reaches past some row's
    // position (the query's own block); raw scores are ranked, the scale is
    // applied inside the exponent: p = 2^(s * c - m * c) with
    // c = scale * log2(e).
    const int t = i + off;
    const bool need_mask = __builtin_amdgcn_ballot_w64(j * kBlock + kBlock - 1 > t) != 0;
    f32x16 sacc[4];
    const float mx = s_block(ktile, qb, n, h, need_mask, t - j * kBlock - 4 * h, sacc);
    const float c = p.scale_log2;
    // l sums the fp32 weights: the LSE it gives feeds the alignment loss,
    // whose teacher probabilities need it to a few 1e-6.
    float l = 0.f;
    f32x16 oacc[4];
    pv_block<true>(vt, sacc, c, -mx * c, n, h, l, oacc);
    l = halves_sum(l);
    float amax = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) amax = max3abs(oacc[dt][r], oacc[dt][r + 1], amax);
    amax = halves_max(amax);
    {
      const float s = 2047.f * rec_inv(amax);
      u32x4* rec = p.part_o + (size_t)slot * (kRecBytes<G> / 16);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) store_piece<G, true>(rec, piece_of(G, dt, hh, h), oacc[dt], s);
      // Both wave halves hold the same row statistics; both store them.
      p.part_stat[(size_t)slot * G + hh] = f32x2{mx * c + __builtin_amdgcn_logf(l), amax * __builtin_amdgcn_rcpf(2047.f * l)};
    }
    asm volatile("" ::: "memory");
    slot = slot_n;
    i = i_n;
    return true;
  };
  u32x4 q0[8], q1[8];
  load_q(q0, i);
  for (int sub = 0;; sub += 8 * QW) {
    if (!sub_tile(sub, q0, q1)) break;
    if (!sub_tile(sub + 4 * QW, q1, q0)) break;
  }
}

// Decode form of the partial (one query per (b, g) row, S_q = 1): every
// selected block is its own work item, so no bucket build is needed; one
// workgroup per (b, g, entry e) writes the record of slot (b H_kv + g) k + e,
// in the layout of attn_partial_kernel's records.  K and V are both read with
// whole 256-byte rows per 16 lanes and staged through one LDS tile in turn:
// K first, read back as the MFMA A operand (loading the operand fragments
// straight from memory touches 32 bytes of 32 rows per instruction, 0.116
// against 0.094 ms on 64 x 256K), then V, read back transposed
// (ds_read_b64_tr_b16).  S^T = K q^T puts this wave's 32 keys
// on registers and the heads on lanes; the block's per-head max and sum are
// exchanged across the four waves in LDS; P goes to LDS as [head][key]; wave w
// then forms O^T for head dims 32 w .. 32 w + 31 over all 128 keys.
constexpr int kPStride = kBlock + 8;  // bf16 per head row of P

template <int G>
__global__ __launch_bounds__(kThreads) void attn_decode_kernel(Params p) {
  __shared__ u32x4 vtile[kBlock * 16];                  // K_j, then V_j [key][chunk ^ rsw(key)]
  __shared__ __align__(16) uint16_t sp[G * kPStride];   // P [head][key] bf16
  __shared__ float s_m[4][32], s_l[4][32], s_a[4][32];  // per-wave max, sum, max |O|

  const int e = blockIdx.x % p.topk;
  const int bg = blockIdx.x / p.topk;
  const int b = bg / p.H_kv, g = bg - b * p.H_kv;
  const int t = p.S_k - 1;                              // the query's position
  const int jj = p.idx[(long)bg * p.topk + e];
  if (jj < 0 || jj > t / kBlock) return;  // uniform; the merge skips this entry too
  const long slot = (long)bg * p.topk + e;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, n = lane & 31;
  const float c = p.scale_log2;

  // Every load first: the K and V tile pieces (row qd / 16, chunk qd % 16),
  // and q of head n (the last head repeated past G).  Both tiles are read
  // once and only staged through LDS, so they are loaded non-temporally
  // (0.12 -> 0.11 ms on 64 x 256K for V).
  const size_t row_stride = (size_t)p.H_kv * kD;
  const uint16_t* kb = p.k + ((size_t)b * p.S_k * p.H_kv + g) * kD;
  const uint16_t* vb = p.v + ((size_t)b * p.S_k * p.H_kv + g) * kD;
  u32x4 vr[8], kq[8], qr[8];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int qd = it * kThreads + tid;
    const int s = min(jj * kBlock + (qd >> 4), p.S_k - 1);  // rows past S_k: masked below
    kq[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (size_t)s * row_stride + 8 * (qd & 15)));
    vr[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + (size_t)s * row_stride + 8 * (qd & 15)));
  }
  {
    const uint16_t* qrow = p.q + ((size_t)b * p.H_q + g * G + min(n, G - 1)) * kD + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qr[ks] = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
  }
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int qd = it * kThreads + tid;
    const int row = qd >> 4;
    vtile[row * 16 + ((qd & 15) ^ rsw(row))] = kq[it];
  }
  __syncthreads();  // the K tile
  u32x4 kr[8];  // this lane's K row (key 32 w + n), chunks 2 ks + h
  {
    const int krow = 32 * wave + n;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kr[ks] = vtile[krow * 16 + ((2 * ks + h) ^ rsw(krow))];
  }

  // S^T[key 32 w + 8 (r / 4) + 4 h + r % 4][head n].
  f32x16 sacc = zero16();
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) sacc = mfma32x32x16(kr[ks], qr[ks], sacc);
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (jj * kBlock + 32 * wave + mfma32_row(r, lane) > t) sacc[r] = neg_inf();
  float mx = max16(neg_inf(), sacc);
  mx = __builtin_fmaxf(mx, swap_halves(mx));
  if (h == 0) s_m[wave][n] = mx;
  __syncthreads();  // every wave has its K operands: the tile takes V now
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int qd = it * kThreads + tid;
    const int row = qd >> 4;
    vtile[row * 16 + ((qd & 15) ^ rsw(row))] = vr[it];
  }
  mx = __builtin_fmaxf(__builtin_fmaxf(s_m[0][n], s_m[1][n]), __builtin_fmaxf(s_m[2][n], s_m[3][n]));
  const float bias = -mx * c;
  float l = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sacc[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, bias));
    l += sacc[r];
  }
  l += swap_halves(l);
  if (h == 0) s_l[wave][n] = l;
  if (n < G) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      uint2 v2;
      v2.x = pack_bf16x2(sacc[4 * r4], sacc[4 * r4 + 1]);
      v2.y = pack_bf16x2(sacc[4 * r4 + 2], sacc[4 * r4 + 3]);
      *reinterpret_cast<uint2*>(&sp[n * kPStride + 32 * wave + 8 * r4 + 4 * h]) = v2;
    }
  }
  __syncthreads();
  l = (s_l[0][n] + s_l[1][n]) + (s_l[2][n] + s_l[3][n]);

  // O^T[dim 32 w + 8 (r / 4) + 4 h + r % 4][head n] over keys 16 kk + 8 h + 0..7.
  f32x16 oacc = zero16();
  {
    const int lr = lane & 15;
    const int hn = min(n, G - 1);
    const int c0 = 32 * wave + 16 * (n >> 4) + 4 * (lr & 3);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int r0 = 16 * kk + 8 * h + (lr >> 2), r1 = r0 + 4;
      const uint2 a0 = lds_read_tr16(reinterpret_cast<const char*>(vtile) + lds_tile_off(r0, c0, rsw(r0)));
      const uint2 a1 = lds_read_tr16(reinterpret_cast<const char*>(vtile) + lds_tile_off(r1, c0, rsw(r1)));
      const u32x4 pb = *reinterpret_cast<const u32x4*>(&sp[hn * kPStride + 16 * kk + 8 * h]);
      oacc = mfma32x32x16(u32x4{a0.x, a0.y, a1.x, a1.y}, pb, oacc);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) amax = max3abs(oacc[r], oacc[r + 1], amax);
  amax = __builtin_fmaxf(amax, swap_halves(amax));
  if (h == 0) s_a[wave][n] = amax;
  __syncthreads();
  amax = __builtin_fmaxf(__builtin_fmaxf(s_a[0][n], s_a[1][n]), __builtin_fmaxf(s_a[2][n], s_a[3][n]));
  if (n < G) {
    const float s = 2047.f * rec_inv(amax);
    store_piece<G, true>(p.part_o + (size_t)slot * (kRecBytes<G> / 16), piece_of(G, wave, n, h), oacc, s);
    if (wave == 0 && h == 0) {
      p.part_stat[(size_t)slot * G + n] = f32x2{mx * c + __builtin_amdgcn_logf(l), amax * __builtin_amdgcn_rcpf(2047.f * l)};
    }
  }
}

// Combines the partials of each (query, group): one wave per row.
// O = sum_e 2^(lse_e - M) sc_e (y_e - 2048) / sum_e 2^(lse_e - M) over the
// records' 12-bit codes y_e, LSE = M + log2(sum).  Every record shares one
// element order, so the sums run in record order and the order is undone
// once, when O is written.  Lane l reads piece l (+ 64 u) of every record,
// all of one head, (l / 2) mod G; the offset 2048 is taken off once, as
// 2048 sum_e 2^(lse_e - M) sc_e.
//
// The entries that count form a wave-uniform bit mask (one ballot).  Records
// are read kBatch at a time with unconditional loads (an entry that does not
// count reads its own slot, which lies inside the workspace, and is skipped
// after the load), so a lane keeps kBatch x F x 2 loads in flight.
//
// Records are read once and the output is written once, both non-temporal,
// so neither stream displaces what is still to be read (32K workload:
// 1.85 -> 1.66 ms).
template <int G>
__global__ __launch_bounds__(kThreads) void merge_kernel(Params p, int with_lse, int rows_per_wave) {
  constexpr int NP = 8 * G;                  // pieces per record
  constexpr int F = (NP + 63) / 64;          // pieces per lane
  constexpr int kBatch = F >= 4 ? 4 : (F >= 2 ? 8 : 16);  // records per batch of loads
  const int lane = threadIdx.x & 63;
  // rows_per_wave consecutive rows per wave: the next row's loads start while
  // the previous row's output stores drain.
  for (int rk = 0; rk < rows_per_wave; ++rk) {
    const long r = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * rows_per_wave + rk;
    if (r >= (long)p.B * p.H_kv * p.Qc) break;
    const int il = (int)(r % p.Qc);
    const int bg = (int)(r / p.Qc);
    const int i = p.q0 + il;
    if (i >= p.S_q) continue;  // past the end of this (b, g); the next row may be valid
    if (i < p.dense_q) continue;  // written by its dense tile
    const int b = bg / p.H_kv, g = bg - (bg / p.H_kv) * p.H_kv;
    const int32_t* sel = p.idx + ((long)bg * p.S_q + i) * p.topk;
    const int local = (i + p.S_k - p.S_q) / kBlock;  // entries past it are ignored
    const long slot0 = slot_of(p, bg, il, 0);        // the row's topk slots are consecutive

    // The validity mask, statistics and records of a batch are all requested
    // before any of them is used; the softmax max is kept online, one rescale
    // per batch, so no pass over the statistics precedes the records.
    const int je = lane < p.topk ? sel[lane] : -1;
    const int hh = (lane >> 1) % G;
    float M = neg_inf(), L = 0.f, W = 0.f, acc[F][16];
#pragma unroll
    for (int u = 0; u < F; ++u)
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[u][c] = 0.f;
    unsigned long long valid = 0;
    for (int e0 = 0; e0 < p.topk; e0 += kBatch) {
      u32x4 xa[kBatch][F];
      uint64_t xb[kBatch][F];
      float lse[kBatch], sc[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const long slot = slot0 + min(e0 + k, p.topk - 1);
        const f32x2 st = p.part_stat[slot * G + hh];
        lse[k] = st[0];
        sc[k] = st[1];
        const u32x4* rec = p.part_o + (size_t)slot * (kRecBytes<G> / 16);
#pragma unroll
        for (int u = 0; u < F; ++u) load_piece<G>(rec, min(lane + 64 * u, NP - 1), xa[k][u], xb[k][u]);
      }
      asm volatile("" ::: "memory");  // keep the loads above together
      if (e0 == 0) valid = __builtin_amdgcn_ballot_w64(je >= 0 && je <= local);
      // Entry e counts when its bit is set (wave-uniform); e past topk never is.
      const unsigned bits = (unsigned)(valid >> e0) & ((1u << kBatch) - 1u);  // e0 < topk <= 64
      if (bits == 0) continue;
      float mb = neg_inf();
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if ((bits >> k) & 1u) mb = __builtin_fmaxf(mb, lse[k]);
      const float m_new = __builtin_fmaxf(M, mb);
      const float alpha = __builtin_amdgcn_exp2f(M - m_new);  // 0 while M = -inf
      M = m_new;
      L *= alpha;
      W *= alpha;
#pragma unroll
      for (int u = 0; u < F; ++u)
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[u][c] *= alpha;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        if (!((bits >> k) & 1u)) continue;  // wave-uniform
        const float wl = __builtin_amdgcn_exp2f(lse[k] - M);
        const float wx = wl * sc[k];
        L += wl;
        W += wx;
#pragma unroll
        for (int u = 0; u < F; ++u) add_piece(xa[k][u], xb[k][u], wx, acc[u]);
      }
    }
    const float inv = 1.f / L;
    const float off = 2048.f * W;
    uint16_t* orow = p.out + (((size_t)b * p.S_q + i) * p.H_q + g * G + hh) * kD;
#pragma unroll
    for (int u = 0; u < F; ++u) {
      const int f = lane + 64 * u;
      if (f >= NP) continue;  // NP is even: lanes f and f ^ 1 skip together
      // Piece f = (dt G + hh) 2 + h holds d = 32 dt + 8 rq + 4 h + 0..3 at
      // values 4 rq + 0..3.  Lanes f and f ^ 1 (h = 0, 1) trade halves so
      // that lane h writes the 16 consecutive d = 32 dt + 16 h + 0..15 (two
      // 16-byte stores; whole 64-byte segments per lane pair): h = 0 sends
      // its rq = 2, 3 values and h = 1 its rq = 0, 1.
      const int dt = (f >> 1) / G, h = f & 1;
      float v[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) v[c] = (acc[u][c] - off) * inv;
      store_run32<true>(orow + 32 * dt, h, v);
      if (with_lse && dt == 0 && h == 0)
        p.lse[((size_t)b * p.H_q + g * G + hh) * p.S_q + i] =
            (M + __builtin_amdgcn_logf(L)) * 0.69314718055994530942f;
    }
  }
}

}  // namespace

namespace edges {

// Edge buckets of the chunk starting at p.q0: counts, scans, scatter.
void launch_build(const AttnShape& s, const Layout& L, const Params& p, hipStream_t st) {
  const long slots = (long)s.batch * s.H_kv * L.Qc * s.topk;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_cap(L.NB, 256)), dim3(256), 0, st, p.counts, L.NB);
  hipLaunchKernelGGL(zero_kernel, dim3(grid_cap(L.NB, 256)), dim3(256), 0, st, p.cursor, L.NB);
  const bool lds_hist = s.n_blk <= kHistBins;
  const long build_grid = (long)s.batch * s.H_kv * ((L.Qc + kBuildQueries - 1) / kBuildQueries);
  if (lds_hist)
    hipLaunchKernelGGL(bucket_count_kernel, dim3((unsigned)build_grid), dim3(256), s.n_blk * 4, st, p);
  else
    hipLaunchKernelGGL(count_kernel, dim3(grid_cap(slots, 256)), dim3(256), 0, st, p);
  hipLaunchKernelGGL(scan_local_kernel, dim3(L.n_scan_wg), dim3(256), 0, st, p);
  hipLaunchKernelGGL(scan_blocks_kernel, dim3(1), dim3(256), 0, st, p, L.n_scan_wg);
  hipLaunchKernelGGL(scan_add_kernel, dim3(L.n_scan_wg), dim3(256), 0, st, p);
  if (lds_hist)
    hipLaunchKernelGGL(bucket_fill_kernel, dim3((unsigned)build_grid), dim3(256), s.n_blk * 8, st, p);
  else
    hipLaunchKernelGGL(fill_kernel, dim3(grid_cap(slots, 256)), dim3(256), 0, st, p);
}

Params base_params(const AttnShape& s, const Layout& L, char* base, const int32_t* idx) {
  Params p{};
  p.idx = idx;
  p.B = s.batch; p.S_q = s.S_q; p.S_k = s.S_k; p.H_q = s.H_q; p.H_kv = s.H_kv;
  p.G = s.H_q / s.H_kv; p.n_blk = s.n_blk; p.topk = s.topk;
  p.Qc = L.Qc; p.NB = (int)L.NB; p.QT = L.QT; p.scale_log2 = s.scale_log2;
  p.W = L.W; p.n_win = L.n_win;
  set_topk_divisor(p);
  p.counts = reinterpret_cast<int32_t*>(base + L.counts);
  p.cursor = reinterpret_cast<int32_t*>(base + L.cursor);
  p.offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  p.tile_off = reinterpret_cast<int32_t*>(base + L.tile_off);
  p.blk_sums = reinterpret_cast<int32_t*>(base + L.blk_sums);
  p.edges = reinterpret_cast<int32_t*>(base + L.edges);
  p.work = reinterpret_cast<int2*>(base + L.work);
  return p;
}

}  // namespace edges

template <int G>
static hipError_t launch_g(const AttnShape& s, const Layout& L, Params p, bool with_lse, hipStream_t st,
                           const StageEvents* ev) {
  // Chunk c's stage m (0 = build, 1 = partial, 2 = merge) is bracketed by
  // events 4 + 6 c + 2 m and 4 + 6 c + 2 m + 1 (see StageEvents).
  auto mark = [&](int c, int m, int after) {
    const int x = 4 + 6 * c + 2 * m + after;
    if (ev && x < ev->n) (void)hipEventRecord(ev->ev[x], st);
  };
  for (int q0 = 0, c = 0; q0 < s.S_q; q0 += L.Qc, ++c) {
    p.q0 = q0;
    mark(c, 0, 0);
    if (s.S_q > 1) launch_build(s, L, p, st);
    mark(c, 0, 1);
    mark(c, 1, 0);
    const int n_dense = std::min(std::min(L.Qc, s.S_q - q0), std::max(0, p.dense_q - q0));
    constexpr int QWG = 4 * (32 / G);  // queries per dense tile
    const int n_dense_wg = n_dense > 0 ? s.batch * s.H_kv * ((n_dense + QWG - 1) / QWG) : 0;
    if (s.S_q > 1)
      hipLaunchKernelGGL(attn_partial_kernel<G>, dim3((unsigned)(L.T + n_dense_wg)), dim3(kThreads), 0, st, p,
                         n_dense, n_dense_wg, with_lse ? 1 : 0);
    else  // one query per row: every selected block is its own work item
      hipLaunchKernelGGL(attn_decode_kernel<G>, dim3((unsigned)(s.batch * s.H_kv * s.topk)), dim3(kThreads), 0, st, p);
    mark(c, 1, 1);
    const long rows = (long)s.batch * s.H_kv * L.Qc;
    mark(c, 2, 0);
    const int rpw = rows >= kMergePairRows ? 2 : 1;
    hipLaunchKernelGGL(merge_kernel<G>, dim3((unsigned)((rows + 4 * rpw - 1) / (4 * rpw))), dim3(kThreads), 0,
                       st, p, with_lse ? 1 : 0, rpw);
    mark(c, 2, 1);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_sparse_attn(const AttnShape& s, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int32_t* idx, uint16_t* out, float* lse,
                              void* ws, size_t ws_bytes, hipStream_t stream,
                              const StageEvents* events) {
  const int qc = fwd_chunk(s, ws_bytes);
  if (qc <= 0) return hipErrorInvalidValue;
  const Layout L = make_fwd_layout(s, qc);
  char* base = static_cast<char*>(ws);
  Params p = base_params(s, L, base, idx);
  p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse;
  // Rows whose local block is below topk take their whole causal prefix
  // (query-stationary kernel); decode keeps its own kernel for every row.
  p.dense_q = s.S_q > 1 ? std::min(s.S_q, std::max(0, s.topk * kBlock - (s.S_k - s.S_q))) : 0;
  p.part_stat = reinterpret_cast<f32x2*>(base + L.part_stat);
  p.part_o = reinterpret_cast<u32x4*>(base + L.part_o);
  const bool with_lse = lse != nullptr;
  switch (p.G) {
    case 1: return launch_g<1>(s, L, p, with_lse, stream, events);
    case 2: return launch_g<2>(s, L, p, with_lse, stream, events);
    case 4: return launch_g<4>(s, L, p, with_lse, stream, events);
    case 8: return launch_g<8>(s, L, p, with_lse, stream, events);
    case 16: return launch_g<16>(s, L, p, with_lse, stream, events);
    case 32: return launch_g<32>(s, L, p, with_lse, stream, events);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
