// Index branch, scoring step: token scores of each (query, group) index query
// against the shared index key, max-pooled over each block of 128 keys
// (Sparse Attention Part II, section 3.2).  The token-score matrix lives only
// in MFMA accumulators and never reaches memory (same page, section 4.4).
//
// The score matrix is computed transposed, S^T[key][row] = k_idx[key] . q_idx[row],
// with keys on the MFMA M axis: in the 32x32 output layout each lane then holds
// 16 keys of one row in registers, so the max over a block's 128 keys is 64
// in-register maxima per lane plus one exchange between the two wave halves.
//
// Rows are r = i * H_kv + g: q_idx[b] is one contiguous [S_q * H_kv][D_idx]
// matrix, and 256 consecutive rows (32 queries when H_kv = 8) share one
// 128-block window of causal positions.
//
// Selection (index_select_kernel, the forward path with k <= 16): one
// workgroup sweeps every key block before its rows' local blocks and keeps,
// per row, the running best k-1 blocks in registers, so neither the block
// scores nor a separate Top-k pass touch memory (the streaming form of the exact top-k of Sparse
// Attention Part II, sections 4.2 and 4.4).  Blocks arrive in ascending index
// order, so a new block displaces the current worst kept block only when its
// score is strictly higher: equal scores keep the lower index, as the
// selection rule requires.
#include <climits>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace msa {
namespace {

constexpr int kBlock = 128;        // keys per block (the pages' block size)
constexpr int kThreads = 256;      // 4 waves
constexpr int kChunk = 32;         // key blocks per workgroup
constexpr int kStageStride = kChunk + 1;  // padded: conflict-free stage writes

struct ScanArgs {
  const uint16_t* q_idx;
  const uint16_t* k_idx;
  float* bm;
  int S_q, S_k, H_kv, n_blk;
  int n_qtiles;   // ceil(S_q * H_kv / rows per workgroup)
  int batch;
  int32_t* sel;   // selection: [B][H_kv][S_q][topk] output
  int topk;
};

constexpr int kKeep = kSelectKeep;  // selection: earlier blocks kept per row (k <= 16)

// 16-byte chunk position inside an LDS row of the key tile, XOR-swizzled so
// that the 16 lanes reading one chunk column of 16 consecutive rows hit 16
// different 16-byte bank groups.
template <int DIDX>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (DIDX == 128) return chunk ^ (row & 15);
  else return chunk ^ ((row >> 1) & 7);
}

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4):
// lane l of the wave writes them at wave_base + l.  wave_base is the same in
// every lane.  A device function, so the host pass never sees the builtin.
__device__ __forceinline__ void load_lds16(const uint16_t* src, u32x4* wave_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)wave_base, 16, 0, 0);
}

// Block scores of many rows (prefill): a workgroup of WAVES waves covers
// WAVES * 32 * NT rows and kChunk key blocks.  NT 32-row MFMA N tiles per
// wave: every 16-byte key fragment read from LDS feeds NT matrix
// instructions.
template <int DIDX, int NT, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void index_scan_prefill(ScanArgs a) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int KS = DIDX / 16;           // MFMA k-steps
  constexpr int CPR = DIDX / 8;           // 16-byte chunks per key row
  constexpr int TILE_CHUNKS = kBlock * CPR;
  constexpr int LOADS = TILE_CHUNKS / kThreads;  // 16-byte loads per thread
  constexpr int ROWS_W = 32 * NT;
  constexpr int ROWS_WG = WAVES * ROWS_W;
  __shared__ u32x4 ktile[2][TILE_CHUNKS];
  __shared__ float stage[ROWS_WG * kStageStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int per_chunk = a.batch * a.n_qtiles;
  const int chunk = blockIdx.x / per_chunk;
  const int rem = blockIdx.x - chunk * per_chunk;
  const int b = rem / a.n_qtiles;
  const int qt = rem - b * a.n_qtiles;

  const int R = a.S_q * a.H_kv;
  const int off = a.S_k - a.S_q;        // position of query i is i + off
  const int wg_r0 = qt * ROWS_WG;
  const int wg_r1 = min(wg_r0 + ROWS_WG, R) - 1;  // last valid row
  const int j0 = chunk * kChunk;
  const int nj = min(kChunk, a.n_blk - j0);
  const int wg_lmax = (wg_r1 / a.H_kv + off) / kBlock;  // largest local block
  const int nj_live = max(0, min(nj, wg_lmax - j0 + 1));

  // The wave's rows and their causal positions.
  const int w_r0 = wg_r0 + wave * ROWS_W;
  const int w_t_min = (min(w_r0, R - 1) / a.H_kv) + off;
  const int w_t_max = (min(w_r0 + ROWS_W - 1, R - 1) / a.H_kv) + off;
  int t_col[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int r = w_r0 + 32 * n + (lane & 31);
    t_col[n] = r < R ? r / a.H_kv + off : -1;
  }

  // Stationary B operand: this wave's index-query rows.
  u32x4 qb[NT][KS];
  {
    const uint16_t* qbase = a.q_idx + (size_t)b * R * DIDX;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int r = min(w_r0 + 32 * n + (lane & 31), R - 1);  // rows past R are never stored
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qb[n][ks] = *reinterpret_cast<const u32x4*>(qbase + (size_t)r * DIDX + 16 * ks + 8 * (lane >> 5));
    }
  }

  const uint16_t* kbase = a.k_idx + (size_t)b * a.S_k * DIDX;
  // Key tiles go from memory straight into LDS (global_load_lds_dwordx4: lane
  // l of a wave writes the 16 bytes at the wave's LDS base + 16 l), so no
  // registers stage them.  LDS piece q = it * kThreads + tid is key row
  // q / CPR, stored chunk q % CPR, which holds the row's chunk
  // swz(row, q % CPR) (the swizzle is its own inverse): its element offset
  // inside a key block is kofs[it].  A block that lies inside S_k is then a
  // uniform base plus kofs; for the last, partial block the rows past S_k
  // (causally masked for every query) read the last key row instead, which
  // keeps the loads unconditional.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  int kofs[LOADS];
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int q = it * kThreads + tid;
    kofs[it] = (q / CPR) * DIDX + 8 * swz<DIDX>(q / CPR, q % CPR);
  }
#define MSA_LOAD_TILE(J, BUF)                                                              \
  {                                                                                        \
    const int j_ = (J);                                                                    \
    const uint16_t* kb_ = kbase + (size_t)j_ * kBlock * DIDX;                              \
    if (j_ * kBlock + kBlock <= a.S_k) {                                                   \
      _Pragma("unroll") for (int it = 0; it < LOADS; ++it)                                 \
        load_lds16(kb_ + kofs[it], &ktile[BUF][it * kThreads + wave_s * 64]);              \
    } else {                                                                               \
      _Pragma("unroll") for (int it = 0; it < LOADS; ++it) {                               \
        const int row_ = kofs[it] / DIDX;                                                  \
        const int s_ = min(j_ * kBlock + row_, a.S_k - 1);                                 \
        load_lds16(kbase + (size_t)s_ * DIDX + (kofs[it] - row_ * DIDX),                   \
                   &ktile[BUF][it * kThreads + wave_s * 64]);                              \
      }                                                                                    \
    }                                                                                      \
  }

  if (nj_live > 0) { MSA_LOAD_TILE(j0, 0) }
  // Everything loaded so far (index queries, first tile) has landed; saying so
  // explicitly keeps the loop's MFMAs from waiting on the next tile's loads.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const bool lo = lane < 32;
  // Block max of block j for this lane's rows (tile kt in LDS).
  auto block_max = [&](int j, const u32x4* kt, float (&best)[NT / 2]) {
    if (j * kBlock > w_t_max) {
#pragma unroll
      for (int p2 = 0; p2 < NT / 2; ++p2) best[p2] = neg_inf();  // nothing visible to this wave
    } else {
      const bool need_mask = j * kBlock + kBlock - 1 > w_t_min;
      float m[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) m[n] = neg_inf();
      // Operand fragments of tile row mt + 1 are read from LDS while the MFMAs
      // of tile row mt run.
      u32x4 ka[KS], kn[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int krow = (lane & 31);
        ka[ks] = kt[krow * CPR + swz<DIDX>(krow, 2 * ks + (lane >> 5))];
      }
      // All eight first-row fragments land before the first MFMA (one LDS
      // round trip instead of one per k-step).
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < 3) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int krow = (mt + 1) * 32 + (lane & 31);
            kn[ks] = kt[krow * CPR + swz<DIDX>(krow, 2 * ks + (lane >> 5))];
          }
        }
        f32x16 acc[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = mfma32x32x16(ka[0], qb[n][0], zero16());
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) {
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[n] = mfma32x32x16(ka[ks], qb[n][ks], acc[n]);
        }
        if (need_mask) {
#pragma unroll
          for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int s = j * kBlock + mt * 32 + mfma32_row(r, lane);
              if (s > t_col[n]) acc[n][r] = neg_inf();
            }
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) m[n] = max16(m[n], acc[n]);
        // The maxima of this tile row may overlap the next row's MFMAs (two
        // rows of accumulators live): with the key tiles loaded straight into
        // LDS the registers allow it, and it measured 3 % faster.
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ka[ks] = kn[ks];
      }
      // Tile pair (2p, 2p+1): lanes < 32 finish tile 2p, lanes >= 32 tile 2p+1,
      // so lane l ends with row w_r0 + 64 p + l.
#pragma unroll
      for (int p2 = 0; p2 < NT / 2; ++p2) {
        const float give = lo ? m[2 * p2 + 1] : m[2 * p2];
        const float got = swap_halves(give);
        best[p2] = __builtin_fmaxf(lo ? m[2 * p2] : m[2 * p2 + 1], got);
      }
    }
  };
  for (int jj = 0; jj < nj_live; ++jj) {
    const int j = j0 + jj;
    // The other buffer was last read before the previous barrier.
    if (jj + 1 < nj_live) { MSA_LOAD_TILE(j + 1, (jj & 1) ^ 1) }
    // Compiler-only fence: keep the next tile's loads before the compute,
    // so they fly during the MFMAs.
    asm volatile("" ::: "memory");
    float best[NT / 2];
    block_max(j, ktile[jj & 1], best);
#pragma unroll
    for (int p2 = 0; p2 < NT / 2; ++p2)
      stage[(wave * ROWS_W + 64 * p2 + lane) * kStageStride + jj] = best[p2];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

#undef MSA_LOAD_TILE

  // Each row's nj block scores are contiguous in memory.
  for (int rr = tid; rr < ROWS_WG; rr += kThreads) {
    const int r = wg_r0 + rr;
    if (r >= R || nj <= 0) continue;
    const int i = r / a.H_kv, g = r - (r / a.H_kv) * a.H_kv;
    float* dst = a.bm + (((size_t)b * a.H_kv + g) * a.S_q + i) * a.n_blk + j0;
    const float* src = stage + rr * kStageStride;
    if ((a.n_blk & 3) == 0) {
      for (int q = 0; q < nj; q += 4) {
        float4 v;
        v.x = q + 0 < nj_live ? src[q + 0] : neg_inf();
        v.y = q + 1 < nj_live ? src[q + 1] : neg_inf();
        v.z = q + 2 < nj_live ? src[q + 2] : neg_inf();
        v.w = q + 3 < nj_live ? src[q + 3] : neg_inf();
        *reinterpret_cast<float4*>(dst + q) = v;
      }
    } else {
      for (int q = 0; q < nj; ++q) dst[q] = q < nj_live ? src[q] : neg_inf();
    }
  }
}

// Selection (scores + Top-k in one pass, k <= 16): one workgroup of
// eight waves per 512-row tile sweeps the key blocks 0 .. (its largest local
// block - 1), two blocks per barrier, the next two blocks' tiles loading
// straight into the other half of the LDS meanwhile.  Each wave owns 64 rows
// (two 32-row MFMA N tiles) and keeps their index queries in registers.
//
// The instruction stream of a block is one software pipeline, so the matrix
// pipe does not drain between 32-key tile rows:
//   - tile rows alternate between two accumulator sets: the maxima of row mt
//     are taken while the MFMAs of row mt + 1 run (the last row's during the
//     next block's first row);
//   - the operand fragments are read from LDS three MFMA pairs ahead;
//   - the previous block's maximum is finished (one lane-half swap) during
//     the next block's first row and its Top-k offer during the rows after;
//   - the MFMAs, LDS reads and vector instructions are placed step by step
//     (one MFMA pair per step, a scheduling barrier between steps), and the
//     only branches in a block are wave-uniform: a block whose key no lane
//     would keep skips the offer slots.
// A row's kept blocks are 64-bit keys (order-preserving score << 32 |
// ~index: larger is better), ascending, keep[0] the worst; a key that beats
// keep[0] enters and keep[0] drops out.  Blocks arrive in ascending order,
// keys are distinct, so the kept set after the last offer is the exact
// top-(k-1) with ties to the lower index, whatever the offers' order.
// Anchors in the instruction stream (empty statements, no instruction is
// emitted; statements with side effects keep their order): pin(v) makes v be
// computed before this point, launder(v) makes whatever uses v after it wait
// for this point.  Together they hold a computation between two points.
__device__ __forceinline__ void pin(float v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void pin(uint64_t v) {
  asm volatile("" ::"v"((uint32_t)v), "v"((uint32_t)(v >> 32)));
}
__device__ __forceinline__ void launder(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void launder(uint64_t& v) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  asm volatile("" : "+v"(lo), "+v"(hi));
  v = ((uint64_t)hi << 32) | lo;
}

// Key of block j for this lane's row from the block's maxima m[0], m[1] of
// the wave's two N tiles: lanes < 32 own a row of tile 0 and lanes >= 32 a row
// of tile 1, and each 32-key group of the block sits in the two lane halves,
// so one swap of halves gives every lane its row's maximum over 128 keys.
// Blocks at or past the row's local block (and j = INT_MAX) give 0, which
// enters nowhere.  No branch: the compiler would otherwise split the block's
// instruction stream at a divergent one.
__device__ __forceinline__ uint64_t offer_key(const float (&m)[2], int j, int my_l) {
  float lo_half = m[0], hi_half = m[1];
  swap32(lo_half, hi_half);
  const uint32_t u = __float_as_uint(__builtin_fmaxf(lo_half, hi_half));
  const uint32_t score = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);  // order_key(max)
  const uint32_t ok = 0u - (uint32_t)(j < my_l);
  return ((uint64_t)(score & ok) << 32) | (uint32_t)(~(uint32_t)j & ok);
}

template <int DIDX>
__global__ __launch_bounds__(512, 1) void index_select_kernel(ScanArgs a) {
  constexpr int WAVES = 8;
  constexpr int kThr = 64 * WAVES;
  constexpr int KS = DIDX / 16;                  // MFMA k-steps per tile row
  constexpr int CPR = DIDX / 8;                  // 16-byte chunks per key row
  constexpr int TILE_CHUNKS = kBlock * CPR;
  constexpr int TILE_BYTES = TILE_CHUNKS * 16;
  constexpr int ROW_BYTES = 32 * CPR * 16;       // one 32-key tile row
  constexpr int LOADS = TILE_CHUNKS / kThr;      // 16-byte loads per thread per tile
  constexpr int STEPS = 4 * KS;                  // MFMA pairs per block
  constexpr int PF = 3;                          // fragment prefetch distance (pairs)
  constexpr int ROWS_WG = WAVES * 64;
  __shared__ u32x4 ktile[4 * TILE_CHUNKS];       // two pairs of key tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.x / a.n_qtiles;
  const int qt = a.n_qtiles - 1 - (blockIdx.x - b * a.n_qtiles);  // longest rows first

  const int R = a.S_q * a.H_kv;
  const int off = a.S_k - a.S_q;                 // position of query i is i + off
  const int wg_r0 = qt * ROWS_WG;
  const int wg_r1 = min(wg_r0 + ROWS_WG, R) - 1;
  const int nj = max(0, (wg_r1 / a.H_kv + off) / kBlock);  // blocks before the largest local block
  const int w_r0 = wg_r0 + wave * 64;

  // Stationary B operand: this wave's 64 index-query rows (rows past R read
  // the last row; they are never stored).
  u32x4 qb[2][KS];
  {
    const uint16_t* qbase = a.q_idx + (size_t)b * R * DIDX;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int r = min(w_r0 + 32 * n + (lane & 31), R - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qb[n][ks] = *reinterpret_cast<const u32x4*>(qbase + (size_t)r * DIDX + 16 * ks + 8 * (lane >> 5));
    }
  }

  // Key tiles go from memory straight into LDS (global_load_lds_dwordx4:
  // lane l of a wave writes the 16 bytes at the wave's LDS base + 16 l); LDS
  // piece q = it * kThr + tid is key row q / CPR, stored chunk q % CPR, which
  // holds the row's chunk swz(row, q % CPR) (the swizzle is its own inverse).
  // Rows past S_k (only in the last block; masked for every row, since only
  // blocks before a row's local block are ranked) read the last key row.
  const uint16_t* kbase = a.k_idx + (size_t)b * a.S_k * DIDX;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  int kofs[LOADS];
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int q = it * kThr + tid;
    kofs[it] = (q / CPR) * DIDX + 8 * swz<DIDX>(q / CPR, q % CPR);
  }
  auto load_tile = [&](int j, int buf) {
    const uint16_t* kb = kbase + (size_t)j * kBlock * DIDX;
    if (j * kBlock + kBlock <= a.S_k) {
#pragma unroll
      for (int it = 0; it < LOADS; ++it)
        load_lds16(kb + kofs[it], &ktile[buf * TILE_CHUNKS + it * kThr + wave_s * 64]);
    } else {
#pragma unroll
      for (int it = 0; it < LOADS; ++it) {
        const int row = kofs[it] / DIDX;
        const int s = min(j * kBlock + row, a.S_k - 1);
        load_lds16(kbase + (size_t)s * DIDX + (kofs[it] - row * DIDX),
                   &ktile[buf * TILE_CHUNKS + it * kThr + wave_s * 64]);
      }
    }
  };

  // Byte offset of this lane's operand fragment for k-step ks inside a tile
  // row (key row lane % 32, chunk 2 ks + lane / 32, swizzled); a row mt of
  // block slot s of pair half h adds h * 2 TILE_BYTES + s * TILE_BYTES +
  // mt * ROW_BYTES, which fits the instruction's immediate offset but for h.
  int fb[KS];  // of pair half 0; moved to the other half and back pair by pair
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    fb[ks] = ((lane & 31) * CPR + swz<DIDX>(lane & 31, 2 * ks + (lane >> 5))) * 16;
  const char* lds = reinterpret_cast<const char*>(ktile);

  if (nj > 0) {
    load_tile(0, 0);
    load_tile(min(1, nj - 1), 1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int my_r = w_r0 + lane;
  const int my_l = my_r < R ? (my_r / a.H_kv + off) / kBlock : -1;
  uint64_t keep[kKeep];
#pragma unroll
  for (int t = 0; t < kKeep; ++t) keep[t] = t < a.topk - 1 ? 0ull : ~0ull;

  f32x16 acc[2][2];  // [set][n tile]; set 1 starts as -inf: no block before the first
#pragma unroll
  for (int n = 0; n < 2; ++n) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[1][n][r] = neg_inf();
  }
  float mlast[2] = {neg_inf(), neg_inf()};  // previous block's maxima (rows 0..2 taken)
  int jlast = INT_MAX;                       // previous block (INT_MAX: none, offers nothing)

  // Row maxima as micro-ops, so that each MFMA step carries a fixed share:
  // op k of max16 for one N tile (k = 0..7): five maxima of three
  // accumulators, two of those, then the running maximum.  Each result is
  // pinned to its step (an empty asm statement that takes it as an input):
  // otherwise the optimizer sinks the maxima of the later rows to their first
  // use, at the block's end, where they would run without any MFMA beside them.
  struct RowMax {
    float t[5], u[2];
  };
  auto max_op = [](RowMax& rm, const f32x16& x, float& m, auto K) {
    constexpr int k = decltype(K)::value;
    if constexpr (k < 5) {
      float a = x[3 * k], b = x[3 * k + 1], c = x[3 * k + 2];
      launder(a);
      launder(b);
      launder(c);
      rm.t[k] = max3f(a, b, c);
      pin(rm.t[k]);
    } else if constexpr (k == 5) {
      rm.u[0] = max3f(rm.t[0], rm.t[1], rm.t[2]);
      pin(rm.u[0]);
    } else if constexpr (k == 6) {
      float c = x[15];
      launder(c);
      rm.u[1] = max3f(rm.t[3], rm.t[4], c);
      pin(rm.u[1]);
    } else {
      m = max3f(rm.u[0], rm.u[1], m);
      pin(m);
    }
  };

  // One block: the MFMAs of its 4 tile rows (row mt into accumulator set
  // mt & 1), each step (one MFMA pair) with a fixed share of vector work on
  // earlier rows:
  //   row 0: the previous block's last row maxima (set 1), then its key x;
  //   rows 1..3: the maxima of rows 0..2, and the kept keys offered x one
  //   slot at a time (the ones below x move down one slot, x takes the slot
  //   above them).
  // Each step is its own scheduling region (sched_barrier), so the LDS read
  // for three steps ahead stays where it is written and the vector work stays
  // between this step's MFMAs.  Steps are a compile-time loop, so every index
  // into the register arrays is a constant.  `fb` holds the per-k-step
  // fragment addresses of the pair half, `slot` the block's place in the
  // pair, `jo` the block index its offer will carry (INT_MAX for a repeated
  // last block).
  constexpr int OPS = 16 / KS;  // max16 micro-ops per N tile per step (2 at D_idx 128)
  auto block = [&](const int (&fb)[KS], const int slot, const int jo) {
    u32x4 ring[4];
    static_for<0, PF>([&](auto S) {
      constexpr int sp = decltype(S)::value;
      ring[sp] = *reinterpret_cast<const u32x4*>(lds + fb[sp % KS] + slot * TILE_BYTES + (sp / KS) * ROW_BYTES);
    });
    float mrow[2] = {neg_inf(), neg_inf()};
    RowMax rm[2];
    uint64_t x = 0;
    bool above0 = false;  // x beats keep[t] for the next slot t to update
    // Whether some lane's key beats its worst kept key: when none does (the
    // common case once many blocks have been seen), nothing can enter and
    // rows 1..3 skip the offer slots (a wave-uniform branch per slot).
    bool any = false;
    // Step s of the block; rows 1..3 carry the offer slots.
    auto step = [&](auto S) {
      constexpr int s = decltype(S)::value;
      constexpr int mt = s / KS, ks = s % KS, set = mt & 1;
      if constexpr (s + PF < STEPS) {
        constexpr int sp = s + PF;
        ring[sp % 4] = *reinterpret_cast<const u32x4*>(lds + fb[sp % KS] + slot * TILE_BYTES + (sp / KS) * ROW_BYTES);
      }
      const u32x4 fa = ring[s % 4];
      // Maxima of the previous row (of the previous block's last row in row 0).
      auto row_ops = [&](int n) {
        static_for<0, OPS>([&](auto O) {
          constexpr int k = ks * OPS + decltype(O)::value;
          if constexpr (k < 8) {
            if constexpr (mt == 0) max_op(rm[n], acc[1][n], mlast[n], std::integral_constant<int, k>{});
            else max_op(rm[n], acc[set ^ 1][n], mrow[n], std::integral_constant<int, k>{});
          }
        });
      };
      acc[set][0] = mfma32x32x16(fa, qb[0][ks], ks == 0 ? zero16() : acc[set][0]);
      row_ops(0);
      acc[set][1] = mfma32x32x16(fa, qb[1][ks], ks == 0 ? zero16() : acc[set][1]);
      row_ops(1);
      if constexpr (mt == 0 && ks == KS - 1) {
        x = offer_key(mlast, jlast, my_l);
        above0 = x > keep[0];
        any = __builtin_amdgcn_ballot_w64(above0) != 0;
        pin(x);
      }
      if constexpr (mt >= 1) {
        // Slots in ascending order over rows 1..3: slot t compares x with
        // keep[t + 1] before that one moves, so two flags are live at a time.
        static_for<0, kKeep>([&](auto T) {
          constexpr int t = decltype(T)::value;
          if constexpr (t * 3 * KS / kKeep == (mt - 1) * KS + ks) if (any) {
            // The kept keys ascend, so above1 implies above0.
            const bool above1 = t + 1 < kKeep && x > keep[t + 1 < kKeep ? t + 1 : t];
            const uint64_t up = above1 ? keep[t + 1 < kKeep ? t + 1 : t] : x;
            keep[t] = above0 ? up : keep[t];
            pin(keep[t]);
            above0 = above1;
          }
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<0, STEPS>(step);
    mlast[0] = mrow[0];
    mlast[1] = mrow[1];
    jlast = jo;
  };

  for (int jj = 0; jj < nj; jj += 2) {
    const int h = (jj >> 1) & 1;  // pair half of blocks jj, jj + 1
    // The other half was last read before the previous barrier.
    if (jj + 2 < nj) {
      load_tile(jj + 2, 2 * (h ^ 1));
      load_tile(min(jj + 3, nj - 1), 2 * (h ^ 1) + 1);
    }
    // A pair past the last block repeats it (its tile was loaded clamped)
    // and offers nothing for the repeat.
    block(fb, 0, jj);
    block(fb, 1, jj + 1 < nj ? jj + 1 : INT_MAX);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) fb[ks] += h ? -2 * TILE_BYTES : 2 * TILE_BYTES;
    // This wave's tile loads have landed before anyone reads them.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  // The last block's last row and its offer.
  {
#pragma unroll
    for (int n = 0; n < 2; ++n) mlast[n] = max16(mlast[n], acc[1][n]);
    const uint64_t x = offer_key(mlast, jlast, my_l);
    bool above[kKeep];
#pragma unroll
    for (int t = 0; t < kKeep; ++t) above[t] = x > keep[t];
#pragma unroll
    for (int t = 0; t < kKeep; ++t) {
      const bool up = t + 1 < kKeep && above[t + 1];
      keep[t] = up ? keep[t + 1] : (above[t] ? x : keep[t]);
    }
  }

  // Kept blocks in ascending order, then the local block, then -1 padding.
  if (my_r < R) {
    int js[16];
#pragma unroll
    for (int t = 0; t < kKeep; ++t)
      js[t] = (keep[t] != 0ull && keep[t] != ~0ull) ? (int)~(uint32_t)keep[t] : INT_MAX;
    js[15] = INT_MAX;
#pragma unroll
    for (int k2 = 2; k2 <= 16; k2 <<= 1)
#pragma unroll
      for (int h2 = k2 >> 1; h2 > 0; h2 >>= 1)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int u = t ^ h2;
          if (u > t) {
            const int mn = min(js[t], js[u]), mx = max(js[t], js[u]);
            const bool up = (t & k2) == 0;
            js[t] = up ? mn : mx;
            js[u] = up ? mx : mn;
          }
        }
    int n = 0;
#pragma unroll
    for (int t = 0; t < 16; ++t) n += js[t] != INT_MAX;
    const int i = my_r / a.H_kv, g = my_r - (my_r / a.H_kv) * a.H_kv;
    int32_t* out = a.sel + (((size_t)b * a.H_kv + g) * a.S_q + i) * a.topk;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (e < a.topk) out[e] = e < n ? js[e] : (e == n ? my_l : -1);
  }
}

// Few rows per sequence (decode): one wave covers every row of a sequence
// (at most 32), so the waves of a workgroup split the key blocks between them
// and need no barrier.  A wave reads its key block with fully coalesced loads
// (each instruction takes 1 KiB: four whole 256-byte rows at D_idx = 128) into
// its own LDS tile, then reads the MFMA operands from there (XOR-swizzled,
// conflict-free); the next block's loads are in flight meanwhile.  Loading
// the operands straight from memory instead takes 32 bytes of 32 different
// rows per instruction and streams about 6 % slower.  Every key row is read
// exactly once, so the loads are non-temporal (64 x 256K keys: 0.71 ->
// 0.64 ms, 6.0 -> 6.7 TB/s).
constexpr int kDecodeBlocksPerWave = 4;

template <int DIDX>
__global__ __launch_bounds__(kThreads, 1) void index_scan_decode(ScanArgs a) {
  constexpr int KS = DIDX / 16;
  constexpr int CPR = DIDX / 8;                  // 16-byte chunks per key row
  constexpr int PIECES = kBlock * CPR / 64;      // 16-byte pieces per lane per block
  __shared__ u32x4 tile[4][kBlock * CPR];        // one key block per wave
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int blocks_per_wg = 4 * kDecodeBlocksPerWave;
  const int n_wg_per_seq = (a.n_blk + blocks_per_wg - 1) / blocks_per_wg;
  const int b = blockIdx.x / n_wg_per_seq;
  const int jw = (blockIdx.x - b * n_wg_per_seq) * blocks_per_wg;

  const int R = a.S_q * a.H_kv;  // <= 32
  const int off = a.S_k - a.S_q;
  const int r = lane & 31;
  const int t_col = r < R ? r / a.H_kv + off : -1;
  const int t_min = off;
  const int t_max = (R - 1) / a.H_kv + off;

  u32x4 qb[KS];
  {
    const uint16_t* qbase = a.q_idx + (size_t)b * R * DIDX;
    const int rc = min(r, R - 1);  // rows past R are never stored
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = *reinterpret_cast<const u32x4*>(qbase + (size_t)rc * DIDX + 16 * ks + 8 * (lane >> 5));
  }
  const uint16_t* kbase = a.k_idx + (size_t)b * a.S_k * DIDX;
  u32x4* my = tile[wave];
  u32x4 buf[PIECES];
  // Piece p of this lane: chunk c = 64 p + lane of the block, i.e. key row
  // c / CPR, 16-byte column c % CPR (the same column for every p).  Rows past
  // S_k are read clamped: they are causally masked for every row.
#define MSA_DEC_LOAD(J)                                                                    \
  _Pragma("unroll") for (int p = 0; p < PIECES; ++p) {                                     \
    const int s_ = min((J) * kBlock + (64 * p + lane) / CPR, a.S_k - 1);                   \
    buf[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + (size_t)s_ * DIDX + 8 * (lane % CPR))); \
  }

  const int j_first = jw + wave;
  if (j_first < a.n_blk) { MSA_DEC_LOAD(j_first) }
  for (int q = 0; q < kDecodeBlocksPerWave; ++q) {
    const int j = jw + q * 4 + wave;
    if (j >= a.n_blk) break;  // wave-uniform
    // This block's pieces into the wave's tile (loads of the previous step).
#pragma unroll
    for (int p = 0; p < PIECES; ++p) {
      const int row = (64 * p + lane) / CPR;
      my[row * CPR + swz<DIDX>(row, lane % CPR)] = buf[p];
    }
    asm volatile("" ::: "memory");
    // The next block's loads fly during this block's MFMAs.
    const int jn = jw + (q + 1) * 4 + wave;
    if (q + 1 < kDecodeBlocksPerWave && jn < a.n_blk) { MSA_DEC_LOAD(jn) }
    asm volatile("" ::: "memory");
    float best;
    if (j * kBlock > t_max) {
      best = neg_inf();
    } else {
      const bool need_mask = j * kBlock + kBlock - 1 > t_min;
      float m = neg_inf();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int krow = mt * 32 + (lane & 31);
        u32x4 ka[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ka[ks] = my[krow * CPR + swz<DIDX>(krow, 2 * ks + (lane >> 5))];
        f32x16 acc = mfma32x32x16(ka[0], qb[0], zero16());
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) acc = mfma32x32x16(ka[ks], qb[ks], acc);
        if (need_mask) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int s = j * kBlock + mt * 32 + mfma32_row(rr, lane);
            if (s > t_col) acc[rr] = neg_inf();
          }
        }
        m = max16(m, acc);
      }
      best = __builtin_fmaxf(m, swap_halves(m));
    }
    asm volatile("" ::: "memory");  // this block's tile reads stay before the next stores
    if (lane < R) {
      const int i = lane / a.H_kv, g = lane - (lane / a.H_kv) * a.H_kv;
      a.bm[(((size_t)b * a.H_kv + g) * a.S_q + i) * a.n_blk + j] = best;
    }
  }
#undef MSA_DEC_LOAD
}

}  // namespace

// N tiles per wave and waves per workgroup of the prefill scores kernel; the
// selection kernel uses the same row tile (8 waves of 64 rows).
constexpr int kNT = 2;
constexpr int kWaves = 8;
constexpr int kRowsPerWg = kWaves * 32 * kNT;

hipError_t launch_index_scores(const uint16_t* q_idx, const uint16_t* k_idx, float* bm,
                               int batch, int S_q, int S_k, int H_kv, int D_idx, int n_blk,
                               hipStream_t stream) {
  ScanArgs a{q_idx, k_idx, bm, S_q, S_k, H_kv, n_blk, 0, batch, nullptr, 0};
  const int R = S_q * H_kv;
  if (R <= 32) {
    const int blocks_per_wg = 4 * kDecodeBlocksPerWave;
    const long grid = (long)batch * ((n_blk + blocks_per_wg - 1) / blocks_per_wg);
    if (D_idx == 128)
      hipLaunchKernelGGL(index_scan_decode<128>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(index_scan_decode<64>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  }
  a.n_qtiles = (R + kRowsPerWg - 1) / kRowsPerWg;
  const long n_chunks = (n_blk + kChunk - 1) / kChunk;
  const long grid = n_chunks * batch * a.n_qtiles;
  if (D_idx == 128)
    hipLaunchKernelGGL((index_scan_prefill<128, kNT, kWaves>), dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((index_scan_prefill<64, kNT, kWaves>), dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_index_select(const uint16_t* q_idx, const uint16_t* k_idx, int32_t* sel,
                               int batch, int S_q, int S_k, int H_kv, int D_idx, int n_blk,
                               int topk, hipStream_t stream) {
  if (!index_select_fused(S_q, H_kv, topk)) return hipErrorInvalidValue;
  ScanArgs a{q_idx, k_idx, nullptr, S_q, S_k, H_kv, n_blk, 0, batch, sel, topk};
  const int R = S_q * H_kv;
  a.n_qtiles = (R + kRowsPerWg - 1) / kRowsPerWg;
  const long grid = (long)batch * a.n_qtiles;
  if (D_idx == 128)
    hipLaunchKernelGGL(index_select_kernel<128>, dim3((unsigned)grid), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(index_select_kernel<64>, dim3((unsigned)grid), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace msa
