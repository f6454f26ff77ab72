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
#include "device_common.h"
#include "kernels.h"

namespace msa {
namespace {

constexpr int kBlock = 128;        // keys per block (the pages' block size)
constexpr int kThreads = 256;      // 4 waves
constexpr int kRowsPerWave = 64;   // two 32-row MFMA N tiles
constexpr int kRowsPerWg = 256;
constexpr int kChunk = 16;         // key blocks per workgroup

struct ScanArgs {
  const uint16_t* q_idx;
  const uint16_t* k_idx;
  float* bm;
  int S_q, S_k, H_kv, n_blk;
  int n_qtiles;   // ceil(S_q * H_kv / 256)
  int batch;
};

// 16-byte chunk position inside an LDS row of the key tile, XOR-swizzled so
// that the 16 lanes reading one chunk column of 16 consecutive rows hit 16
// different 16-byte bank groups.
template <int DIDX>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (DIDX == 128) return chunk ^ (row & 15);
  else return chunk ^ ((row >> 1) & 7);
}

template <int DIDX>
__global__ __launch_bounds__(kThreads, 2) void index_scan_prefill(ScanArgs a) {
  constexpr int KS = DIDX / 16;           // MFMA k-steps
  constexpr int CPR = DIDX / 8;           // 16-byte chunks per key row
  constexpr int TILE_CHUNKS = kBlock * CPR;
  constexpr int LOADS = TILE_CHUNKS / kThreads;  // 16-byte loads per thread
  __shared__ uint4 ktile[2][TILE_CHUNKS];
  __shared__ float stage[kRowsPerWg * kChunk];

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
  const int wg_r0 = qt * kRowsPerWg;
  const int wg_r1 = min(wg_r0 + kRowsPerWg, R) - 1;  // last valid row
  const int j0 = chunk * kChunk;
  const int nj = min(kChunk, a.n_blk - j0);
  const int wg_lmax = (wg_r1 / a.H_kv + off) / kBlock;  // largest local block
  const int nj_live = max(0, min(nj, wg_lmax - j0 + 1));

  // The wave's rows and their causal positions.
  const int w_r0 = wg_r0 + wave * kRowsPerWave;
  const int w_t_min = (min(w_r0, R - 1) / a.H_kv) + off;
  const int w_t_max = (min(w_r0 + kRowsPerWave - 1, R - 1) / a.H_kv) + off;
  int t_col[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int r = w_r0 + 32 * n + (lane & 31);
    t_col[n] = r < R ? r / a.H_kv + off : -1;
  }

  // Stationary B operand: this wave's 64 index-query rows.
  uint4 qb[2][KS];
  {
    const uint16_t* qbase = a.q_idx + (size_t)b * R * DIDX;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int r = w_r0 + 32 * n + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (r < R)
          qb[n][ks] = *reinterpret_cast<const uint4*>(qbase + (size_t)r * DIDX + 16 * ks + 8 * (lane >> 5));
        else
          qb[n][ks] = make_uint4(0, 0, 0, 0);
      }
    }
  }

  const uint16_t* kbase = a.k_idx + (size_t)b * a.S_k * DIDX;
  uint4 pre[LOADS];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int q = it * kThreads + tid;
      const int row = q / CPR, c = q % CPR;
      const int s = j * kBlock + row;
      pre[it] = s < a.S_k ? *reinterpret_cast<const uint4*>(kbase + (size_t)s * DIDX + 8 * c)
                          : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int q = it * kThreads + tid;
      const int row = q / CPR, c = q % CPR;
      ktile[buf][row * CPR + swz<DIDX>(row, c)] = pre[it];
    }
  };

  if (nj_live > 0) {
    load_tile(j0);
    store_tile(0);
  }
  __syncthreads();

  for (int jj = 0; jj < nj_live; ++jj) {
    const int j = j0 + jj;
    if (jj + 1 < nj_live) load_tile(j + 1);
    const int buf = jj & 1;
    float best;
    if (j * kBlock > w_t_max) {
      best = neg_inf();  // nothing visible to any row of this wave
    } else {
      const bool need_mask = j * kBlock + kBlock - 1 > w_t_min;
      float m[2] = {neg_inf(), neg_inf()};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x16 acc[2];
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
        const int krow = mt * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 av = ktile[buf][krow * CPR + swz<DIDX>(krow, 2 * ks + (lane >> 5))];
          acc[0] = mfma32x32x16(av, qb[0][ks], acc[0]);
          acc[1] = mfma32x32x16(av, qb[1][ks], acc[1]);
        }
        if (need_mask) {
#pragma unroll
          for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int s = j * kBlock + mt * 32 + mfma32_row(r, lane);
              if (s > t_col[n]) acc[n][r] = neg_inf();
            }
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          float x = m[n];
#pragma unroll
          for (int r = 0; r < 16; r += 2) x = max3f(x, acc[n][r], acc[n][r + 1]);
          m[n] = x;
        }
      }
      // Lanes < 32 finish rows of tile 0, lanes >= 32 rows of tile 1.
      const bool lo = lane < 32;
      const float give = lo ? m[1] : m[0];
      const float got = swap_halves(give);
      best = __builtin_fmaxf(lo ? m[0] : m[1], got);
    }
    stage[(wave * kRowsPerWave + lane) * kChunk + jj] = best;
    if (jj + 1 < nj_live) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Each thread writes one row's nj block scores (contiguous in memory).
  const int r = wg_r0 + tid;
  if (r < R && nj > 0) {
    const int i = r / a.H_kv, g = r - (r / a.H_kv) * a.H_kv;
    float* dst = a.bm + (((size_t)b * a.H_kv + g) * a.S_q + i) * a.n_blk + j0;
    const float* src = stage + tid * kChunk;
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

// Few rows per sequence (decode): one wave covers every row of a sequence
// (at most 32), so the waves of a workgroup split the key blocks between them
// and read their key tiles straight from memory into MFMA operands.
constexpr int kDecodeBlocksPerWave = 4;

template <int DIDX>
__global__ __launch_bounds__(kThreads, 2) void index_scan_decode(ScanArgs a) {
  constexpr int KS = DIDX / 16;
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

  uint4 qb[KS];
  {
    const uint16_t* qbase = a.q_idx + (size_t)b * R * DIDX;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = r < R ? *reinterpret_cast<const uint4*>(qbase + (size_t)r * DIDX + 16 * ks + 8 * (lane >> 5))
                     : make_uint4(0, 0, 0, 0);
  }
  const uint16_t* kbase = a.k_idx + (size_t)b * a.S_k * DIDX;

  for (int q = 0; q < kDecodeBlocksPerWave; ++q) {
    const int j = jw + q * 4 + wave;
    if (j >= a.n_blk) break;
    float best;
    if (j * kBlock > t_max) {
      best = neg_inf();
    } else {
      // All 4 x KS operand loads of the block are issued before any MFMA.
      uint4 av[4][KS];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int s = j * kBlock + mt * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          av[mt][ks] = s < a.S_k ? load_nt16(kbase + (size_t)s * DIDX + 16 * ks + 8 * (lane >> 5))
                                 : make_uint4(0, 0, 0, 0);
      }
      const bool need_mask = j * kBlock + kBlock - 1 > t_min;
      float m = neg_inf();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x16 acc;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) acc[rr] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma32x32x16(av[mt][ks], qb[ks], acc);
        if (need_mask) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int s = j * kBlock + mt * 32 + mfma32_row(rr, lane);
            if (s > t_col) acc[rr] = neg_inf();
          }
        }
#pragma unroll
        for (int rr = 0; rr < 16; rr += 2) m = max3f(m, acc[rr], acc[rr + 1]);
      }
      best = __builtin_fmaxf(m, swap_halves(m));
    }
    if (lane < R) {
      const int i = lane / a.H_kv, g = lane - (lane / a.H_kv) * a.H_kv;
      a.bm[(((size_t)b * a.H_kv + g) * a.S_q + i) * a.n_blk + j] = best;
    }
  }
}

}  // namespace

hipError_t launch_index_scores(const uint16_t* q_idx, const uint16_t* k_idx, float* bm,
                               int batch, int S_q, int S_k, int H_kv, int D_idx, int n_blk,
                               hipStream_t stream) {
  ScanArgs a{q_idx, k_idx, bm, S_q, S_k, H_kv, n_blk, 0, batch};
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
    hipLaunchKernelGGL(index_scan_prefill<128>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(index_scan_prefill<64>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

long index_scores_grid(int batch, int S_q, int H_kv, int n_blk) {
  const int R = S_q * H_kv;
  if (R <= 32) return (long)batch * ((n_blk + 4 * kDecodeBlocksPerWave - 1) / (4 * kDecodeBlocksPerWave));
  return (long)((n_blk + kChunk - 1) / kChunk) * batch * ((R + kRowsPerWg - 1) / kRowsPerWg);
}

}  // namespace msa
