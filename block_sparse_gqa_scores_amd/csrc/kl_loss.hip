// Alignment loss of the index branch, forward value: the per-row KL terms and
// their mean, on the edge buckets of the attention (see the kernel notes).
#include "edge_buckets.h"

namespace msa {
using namespace edges;
namespace {

// ------------------------------------------------------------------------
// Alignment loss of the index branch, forward value (Sparse Attention Part
// II, section 3.2): for row (b, i, g) with token set T (the visible tokens of
// its selected blocks),
//   KL_row = sum_{x in T} P(x) ln(P(x) / Pidx(x)),
//   P(x) = (1/G) sum_h exp(scale q_h . k_x - lse_h)   (each head normalised on T),
//   Pidx = softmax over T of z(x) = q_idx . k_idx_x   (raw index scores),
// and the loss is the mean of KL_row over the B * S_q * H_kv rows.  With
// S = sum P, A = sum P ln P and, for any shift m, C = sum P (z - m) and
// L = sum exp(z - m), the row term is A - C + S (m + ln L - ... ) rearranged
// per block below; neither distribution is ever written out (the expansion
// of the KL term the MSA kernel notes describe).
//
// The same edge buckets as the attention: a work item loads K_j and the index
// keys of block j into LDS once and runs all its edges against them.  For an
// edge (query i, block j) it leaves the record (S_j, A_j, C_j, m_j) and L_j
// with m_j = max z over the block's visible tokens; a merge per row combines
//   M = max m_j, L = sum_j L_j e^(m_j - M), LSE = M + ln L,
//   KL_row = sum_j (A_j - C_j + S_j (LSE - m_j)).
//
// Scores are formed as S = Q K^T (query heads on MFMA rows, keys on lanes),
// so the G heads of a query sit in registers of one lane (and of its partner
// in the other half of the wave for G >= 8): the group mean of the teacher is
// an in-lane sum.  The index scores must land in the lanes that hold the
// teacher for (query, key): for G >= 8 (at most 4 queries per sub-tile) they
// come from 16x16x32 tiles whose A row m carries query m % 4 (see the kernel);
// for G < 8 the A operand holds the query's index row once per head (G
// copies), in the teacher's own layout.
template <int G, int DIDX>
__global__ __launch_bounds__(kThreads, 2) void kl_partial_kernel(Params p) {
  constexpr int QW = 32 / G;                 // queries per wave sub-tile
  constexpr int QT = kSubTiles * 4 * QW;     // edges per work item
  constexpr int ICH = DIDX / 8;              // 16-byte chunks per index key
  constexpr int RPS = G >= 8 ? G / 2 : G;    // registers per (query, key) in a lane
  constexpr int NL = 16 / RPS;               // queries per lane
  __shared__ u32x4 ktile[kBlock * 16];       // [key][16 chunks], swizzled
  __shared__ u32x4 itile[kBlock * ICH];      // [key][ICH chunks], swizzled
  __shared__ __align__(16) float s_lse[QT * G];  // log2(e) * lse of (edge, head)
  __shared__ int32_t s_slot[QT];
  __shared__ int32_t s_i[QT];

  const int w = blockIdx.x;
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
  constexpr float kLog2e = 1.4426950408889634f;

  // Edges past n_here repeat the last one (same inputs, same record).
  for (int x = tid; x < QT; x += kThreads) {
    const int sl = p.edges[ebase + min(x, n_here - 1)];
    s_slot[x] = sl;
    s_i[x] = p.q0 + (int)((sl / p.topk) % p.Qc);
  }
  __syncthreads();
  {  // each edge's G head LSEs are one contiguous run of lse_t
    const float* lq = p.lse_t + (size_t)bg * p.S_q * G;
    for (int x = tid; x < QT * G; x += kThreads) s_lse[x] = lq[(size_t)s_i[x / G] * G + x % G];
  }
  {
    const size_t row_stride = (size_t)p.H_kv * kD;
    const uint16_t* kb = p.k + ((size_t)b * p.S_k * p.H_kv + g) * kD;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int qd = it * kThreads + tid;
      const int row = qd >> 4, c = qd & 15;
      // Keys past S_k are masked for every query; a clamped row is read.
      const int s = min(j * kBlock + row, p.S_k - 1);
      ktile[row * 16 + (c ^ (row & 15))] = *reinterpret_cast<const u32x4*>(kb + (size_t)s * row_stride + 8 * c);
    }
    const uint16_t* ib = p.k_idx + (size_t)b * p.S_k * DIDX;
#pragma unroll
    for (int it = 0; it < kBlock * ICH / kThreads; ++it) {
      const int qd = it * kThreads + tid;
      const int row = qd / ICH, c = qd % ICH;
      const int s = min(j * kBlock + row, p.S_k - 1);
      itile[row * ICH + (c ^ (row & (ICH - 1)))] = *reinterpret_cast<const u32x4*>(ib + (size_t)s * DIDX + 8 * c);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int off = p.S_k - p.S_q;
  const int n = lane & 31;                       // key column of this lane / A row
  const int qm = n / G, hm = n - (n / G) * G;    // A row: query qm of the sub-tile, head hm
  const float c = p.scale_log2;
  const float invG = 1.f / G;

  // Query (within the sub-tile) of query slot l of this lane: the D rows
  // 8 (r / 4) + 4 h + r % 4 for r = l RPS .. l RPS + RPS - 1.
  auto q_of = [&](int l) {
    const int r0 = l * RPS;
    return (8 * (r0 >> 2) + 4 * h + (r0 & 3)) / G;
  };
  auto load_q = [&](u32x4* dq, int i) {
    const uint16_t* qrow = p.q + (((size_t)b * p.S_q + i) * p.H_q + g * G + hm) * kD + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) dq[ks] = *reinterpret_cast<const u32x4*>(qrow + 16 * ks);
  };
  auto load_qi = [&](u32x4* di, int i) {
    const uint16_t* irow = p.q_idx + (((size_t)b * p.S_q + i) * p.H_kv + g) * DIDX + 8 * h;
#pragma unroll
    for (int ks = 0; ks < DIDX / 16; ++ks) di[ks] = *reinterpret_cast<const u32x4*>(irow + 16 * ks);
  };

  // With G >= 8 a sub-tile has at most 4 queries, and z (one value per query
  // and key) takes 16x16x32 instructions whose A row m carries query m % 4
  // (the last query repeated past QW): every 16-lane group of the result then
  // holds all the queries, in register order, for its 16 keys.
  constexpr bool kZ16 = G >= 8;
  constexpr int ZKS = DIDX / 32;
  const int qz = min(lane & 3, QW - 1);
  auto load_qz = [&](u32x4* dz, int i) {
    const uint16_t* irow = p.q_idx + (((size_t)b * p.S_q + i) * p.H_kv + g) * DIDX + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < ZKS; ++ks) dz[ks] = *reinterpret_cast<const u32x4*>(irow + 32 * ks);
  };

  u32x4 qb[8], ib[kZ16 ? 1 : DIDX / 16], iz[kZ16 ? ZKS : 1];
  load_q(qb, s_i[wave * QW + qm]);
  if constexpr (kZ16) load_qz(iz, s_i[wave * QW + qz]);
  else load_qi(ib, s_i[wave * QW + qm]);
  for (int sub = 0; sub < n_here; sub += 4 * QW) {
    const int e0 = sub + wave * QW;  // first edge of this wave's sub-tile
    if (e0 >= n_here) break;         // wave-uniform
    const int i_next = s_i[min(e0 + 4 * QW, QT - QW) + qm];
    const int iz_next = s_i[min(e0 + 4 * QW, QT - QW) + qz];

    float lse2[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 v = *reinterpret_cast<const float4*>(&s_lse[e0 * G + 8 * r4 + 4 * h]);
      lse2[4 * r4 + 0] = v.x; lse2[4 * r4 + 1] = v.y; lse2[4 * r4 + 2] = v.z; lse2[4 * r4 + 3] = v.w;
    }
    int tq[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) tq[l] = s_i[e0 + q_of(l)] + off;

    // Index scores first; the index rows of the next sub-tile load meanwhile.
    float pt[4][NL], zv[4][NL];
    if constexpr (kZ16) {
      // Key tiles 2 nt and 2 nt + 1 (16 keys each); lane n (= lane % 32)
      // takes key 32 nt + n from the first for n < 16, else from the second,
      // and register l is query l (= q_of(l) for G >= 8).
      const bool upper = (lane >> 4) & 1;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int k0 = nt * 32 + (lane & 15), k1 = k0 + 16;
        f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < ZKS; ++ks) {
          const int ch = 4 * ks + (lane >> 4);
          z0 = mfma16x16x32(iz[ks], itile[k0 * ICH + (ch ^ (k0 & (ICH - 1)))], z0);
          z1 = mfma16x16x32(iz[ks], itile[k1 * ICH + (ch ^ (k1 & (ICH - 1)))], z1);
        }
#pragma unroll
        for (int l = 0; l < NL; ++l) zv[nt][l] = upper ? z1[l] : z0[l];
      }
      load_qz(iz, iz_next);
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int krow = nt * 32 + n;
        f32x16 za = zero16();
#pragma unroll
        for (int ks = 0; ks < DIDX / 16; ++ks)
          za = mfma32x32x16(ib[ks], itile[krow * ICH + ((2 * ks + h) ^ (krow & (ICH - 1)))], za);
#pragma unroll
        for (int l = 0; l < NL; ++l) zv[nt][l] = za[l * RPS];
        __builtin_amdgcn_sched_barrier(0);
      }
      load_qi(ib, i_next);
    }
    // S = Q K^T as a software pipeline, one MFMA per step (step st = 8 nt +
    // ks, key tile nt) with a scheduling barrier between steps: each K
    // fragment is read three steps ahead into a ring of four, and the
    // teacher sums of tile nt - 1 run two values a step during tile nt's
    // MFMAs (in the same order as one pass would add them).  Keys past a
    // query are dropped after the head sum (the same keys for every head of
    // the query), where vis is applied.  G = 1 keeps 64 teacher values per
    // lane and has no registers for the ring: one tile at a time there.
    if constexpr (G == 1) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int krow = nt * 32 + n;
        f32x16 sa = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          sa = mfma32x32x16(qb[ks], ktile[krow * 16 + ((2 * ks + h) ^ (krow & 15))], sa);
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          float acc = 0.f;
#pragma unroll
          for (int rr = 0; rr < RPS; ++rr) {
            const int r = l * RPS + rr;
            acc += __builtin_amdgcn_exp2f(__builtin_fmaf(sa[r], c, -lse2[r]));
          }
          pt[nt][l] = acc;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      const u32x4* klane = ktile + n * 16;  // row 32 nt + n keeps its chunks swizzled by n & 15
      auto kfrag = [&](int st) { return klane[(st >> 3) * 512 + ((2 * (st & 7) + h) ^ (n & 15))]; };
      f32x16 sa[2];
      // Values r, r + 1 of tile NT (accumulator sa[NT & 1]) into pt[NT].
      auto teach2 = [&](auto NT, auto R) {
        constexpr int nt = decltype(NT)::value, r = decltype(R)::value;
#pragma unroll
        for (int x = r; x < r + 2; ++x) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[nt & 1][x], c, -lse2[x]));
          if (x % RPS == 0) pt[nt][x / RPS] = 0.f;
          pt[nt][x / RPS] += e;
        }
      };
      u32x4 ring[4];
      static_for<0, 3>([&](auto P) { ring[P] = kfrag(P); });
      static_for<0, 32>([&](auto S) {
        constexpr int st = decltype(S)::value, nt = st / 8, ks = st % 8;
        if constexpr (st + 3 < 32) ring[(st + 3) % 4] = kfrag(st + 3);
        sa[nt & 1] = mfma32x32x16(qb[ks], ring[st % 4], ks == 0 ? zero16() : sa[nt & 1]);
        if constexpr (nt >= 1) teach2(std::integral_constant<int, nt - 1>{}, std::integral_constant<int, 2 * ks>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      static_for<0, 8>([&](auto K) { teach2(std::integral_constant<int, 3>{}, std::integral_constant<int, 2 * K>{}); });
    }
    // Teacher and index score of each (query slot l, key tile u) of this
    // lane.  For G >= 8 the halves hold head partial sums of the same queries:
    // one swap32 per pair of key tiles completes the head sums and leaves
    // tiles 0, 1 in half 0 and tiles 2, 3 in half 1 (sums then run over all 64
    // lanes); for G <= 4 each half has its own queries and all four tiles.
    constexpr int NT = G >= 8 ? 2 : 4;
    float P[NL][NT], Z[NL][NT];
    bool vis[NL][NT];
#pragma unroll
    for (int l = 0; l < NL; ++l)
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        float pv;
        if constexpr (G >= 8) {
          float a = pt[u][l], bq = pt[2 + u][l];
          swap32(a, bq);
          pv = (a + bq) * invG;
          float za = zv[u][l], zb = zv[2 + u][l];
          swap32(za, zb);
          Z[l][u] = za;
        } else {
          pv = pt[u][l] * invG;
          Z[l][u] = zv[u][l];
        }
        const int nt = G >= 8 ? 2 * h + u : u;
        vis[l][u] = j * kBlock + nt * 32 + n <= tq[l];
        P[l][u] = vis[l][u] ? pv : 0.f;
      }
    load_q(qb, i_next);  // lands while the statistics below are reduced

    // m_l = max of z over the visible keys of query slot l, in every lane;
    // mown = the maximum of the slot whose sums this lane's row writes below.
    float mz[NL], mown;
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      float m = neg_inf();
#pragma unroll
      for (int u = 0; u < NT; ++u) m = vis[l][u] ? __builtin_fmaxf(m, Z[l][u]) : m;
      mz[l] = m;
    }
    float mw[NL > 1 ? NL / 2 : 1];  // row-held maxima of the G <= 4 split
    if constexpr (G >= 8) {
      if constexpr (NL == 4) {
        scatter32<4, true>(mz);
        scatter16<2, true>(mz);
        mz[0] = row_max16(mz[0]);
        mown = mz[0];
        gather16<2>(mz);
        gather32<4>(mz);
      } else if constexpr (NL == 2) {
        scatter32<2, true>(mz);
        mz[0] = row_max16(allred16<true>(mz[0]));
        mown = mz[0];
        gather32<2>(mz);
      } else {
        mz[0] = row_max16(allred16<true>(allred32<true>(mz[0])));
        mown = mz[0];
      }
    } else {
      scatter16<NL, true>(mz);
#pragma unroll
      for (int x = 0; x < NL / 2; ++x) mw[x] = mz[x] = row_max16(mz[x]);
      gather16<NL>(mz);
      mown = 0.f;
    }

    // Sums per slot: S = sum P, A = sum P ln P, C = sum P (z - m), L = sum e^(z - m).
    constexpr int V0 = 4 * NL;
    float sums[V0];
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      float sS = 0.f, sA = 0.f, sC = 0.f, sL = 0.f;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const float pv = P[l][u];
        const float d = Z[l][u] - mz[l];
        sS += pv;
        sA += pv > 1e-30f ? pv * __builtin_amdgcn_logf(pv) : 0.f;
        sC += pv > 0.f ? pv * d : 0.f;
        sL += vis[l][u] ? __builtin_amdgcn_exp2f(d * kLog2e) : 0.f;
      }
      sums[4 * l + 0] = sS;
      sums[4 * l + 1] = sA * 0.69314718055994530942f;
      sums[4 * l + 2] = sC;
      sums[4 * l + 3] = sL;
    }
    // Reduce-scatter: lanes of row rho (of half h) end with VR totals.
    constexpr int VR = G >= 8 ? V0 / 4 : V0 / 2;
    if constexpr (G >= 8) {
      scatter32<V0, false>(sums);
      scatter16<V0 / 2, false>(sums);
    } else {
      scatter16<V0, false>(sums);
    }
#pragma unroll
    for (int x = 0; x < VR; ++x) sums[x] = row_sum16(sums[x]);
    if ((lane & 15) == 0) {
      const int rho = (lane >> 4) & 1;
#pragma unroll
      for (int x = 0; x < VR; ++x) {
        const int orig = G >= 8 ? x + VR * rho + 2 * VR * h : x + VR * rho;
        const int l = orig >> 2, qq = orig & 3;
        const int sl = s_slot[e0 + q_of(l)];
        p.kl_rec[(size_t)sl * 8 + qq] = sums[x];
        if (qq == 0) p.kl_rec[(size_t)sl * 8 + 4] = G >= 8 ? mown : mw[x >> 2];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Row terms and the loss.  One thread per row (b, g, i); the records of its
// selected blocks are requested 16 at a time (an entry that does not count
// reads its own slot, inside the record array, and is skipped; 32K:
// 2.20 -> 2.12 ms for the loss against one entry's loads at a time) and
// combined online, in entry order:
//   M running max of m_j, L = sum L_j e^(m_j - M), U = sum S_j (m_j - M),
//   KL_row = sum (A_j - C_j) - U + (sum S_j) ln L.
// Each workgroup leaves the sum of its rows' terms; kl_total_kernel adds those
// in a fixed order, so the loss is identical from run to run.
__global__ __launch_bounds__(256) void kl_merge_kernel(Params p) {
  __shared__ float red[256];
  const long r = (long)blockIdx.x * 256 + threadIdx.x;
  const long rows = (long)p.B * p.H_kv * p.S_q;
  float kl = 0.f;
  if (r < rows) {
    const int i = (int)(r % p.S_q);
    const int local = (i + p.S_k - p.S_q) / kBlock;
    const int32_t* sel = p.idx + r * p.topk;
    float M = neg_inf(), L = 0.f, U = 0.f, S = 0.f, AC = 0.f;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr int kB = 16;
    for (int e0 = 0; e0 < p.topk; e0 += kB) {
      float4 recs[kB];
      float mjs[kB];
      int js[kB];
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const long e = r * p.topk + min(e0 + k, p.topk - 1);
        js[k] = sel[min(e0 + k, p.topk - 1)];
        recs[k] = *reinterpret_cast<const float4*>(p.kl_rec + e * 8);
        mjs[k] = p.kl_rec[e * 8 + 4];
      }
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        if (e0 + k >= p.topk || js[k] < 0 || js[k] > local) continue;
        const float4 rec = recs[k];
        const float mj = mjs[k];
        if (mj > M) {  // rescale what was summed against the old maximum
          if (M != neg_inf()) {
            L *= __builtin_amdgcn_exp2f((M - mj) * kLog2e);
            U += S * (M - mj);
          }
          M = mj;
        }
        const float dm = mj - M;
        L += rec.w * __builtin_amdgcn_exp2f(dm * kLog2e);
        U += rec.x * dm;
        S += rec.x;
        AC += rec.y - rec.z;
      }
    }
    const float lnL = __builtin_amdgcn_logf(L) * 0.69314718055994530942f;
    kl = AC - U + S * lnL;
    if (p.kl_rows) p.kl_rows[r] = kl;
    if (p.kl_lse) p.kl_lse[r] = M + lnL;
  }
  red[threadIdx.x] = kl;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.kl_wsum[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void kl_total_kernel(Params p, int n_wg, float inv_rows) {
  __shared__ float red[256];
  float s = 0.f;
  for (int x = threadIdx.x; x < n_wg; x += 256) s += p.kl_wsum[x];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *p.loss = red[0] * inv_rows;
}

__global__ void lse_group_kernel(const float* lse, float* lse_t, int H_q, int G, int S_q, long n) {
  for (long x = (long)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (long)gridDim.x * blockDim.x) {
    // x = ((b H_q + h) S_q + i): reads in order, writes to (b, h / G, i, h % G).
    const int i = (int)(x % S_q);
    const long bh = x / S_q;
    const int h = (int)(bh % H_q);
    const long b = bh / H_q;
    lse_t[((b * (H_q / G) + h / G) * S_q + i) * G + h % G] = lse[x] * 1.4426950408889634f;
  }
}

__global__ void fill_zero_kernel(float* a, long n) {
  for (long x = (long)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (long)gridDim.x * blockDim.x)
    a[x] = 0.f;
}
}  // namespace

namespace edges {
void launch_lse_group(const AttnShape& s, const float* lse, float* lse_t, hipStream_t st) {
  const long n = (long)s.batch * s.H_q * s.S_q;
  hipLaunchKernelGGL(lse_group_kernel, dim3(grid_cap(n, 256)), dim3(256), 0, st, lse, lse_t, s.H_q,
                     s.H_q / s.H_kv, s.S_q, n);
}
}  // namespace edges

hipError_t launch_fill_zero(float* dst, long n, hipStream_t stream) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_cap(n, 256)), dim3(256), 0, stream, dst, n);
  return hipGetLastError();
}

namespace {
template <int G, int DIDX>
hipError_t launch_kl_g(const AttnShape& s, const Layout& L, const Params& p, hipStream_t st) {
  launch_build(s, L, p, st);
  hipLaunchKernelGGL((kl_partial_kernel<G, DIDX>), dim3((unsigned)L.T), dim3(kThreads), 0, st, p);
  hipLaunchKernelGGL(kl_merge_kernel, dim3((unsigned)L.n_kl_wg), dim3(256), 0, st, p);
  if (p.loss) {
    const double rows = (double)s.batch * s.H_kv * s.S_q;
    hipLaunchKernelGGL(kl_total_kernel, dim3(1), dim3(256), 0, st, p, L.n_kl_wg, (float)(1.0 / rows));
  }
  return hipGetLastError();
}

template <int DIDX>
hipError_t launch_kl_d(const AttnShape& s, const Layout& L, const Params& p, hipStream_t st) {
  switch (p.G) {
    case 1: return launch_kl_g<1, DIDX>(s, L, p, st);
    case 2: return launch_kl_g<2, DIDX>(s, L, p, st);
    case 4: return launch_kl_g<4, DIDX>(s, L, p, st);
    case 8: return launch_kl_g<8, DIDX>(s, L, p, st);
    case 16: return launch_kl_g<16, DIDX>(s, L, p, st);
    case 32: return launch_kl_g<32, DIDX>(s, L, p, st);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_kl_loss(const AttnShape& s, int D_idx, const uint16_t* q, const uint16_t* k,
                          const uint16_t* q_idx, const uint16_t* k_idx, const int32_t* idx,
                          const float* lse, float* kl_rows, float* loss, float* lse_idx, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  const Layout L = make_kl_layout(s);
  if (ws_bytes < L.total) return hipErrorInvalidValue;
  char* base = static_cast<char*>(ws);
  Params p = base_params(s, L, base, idx);
  p.q = q; p.k = k; p.q_idx = q_idx; p.k_idx = k_idx; p.lse_in = lse;
  p.kl_rec = reinterpret_cast<float*>(base + L.kl_rec);
  p.kl_wsum = reinterpret_cast<float*>(base + L.kl_wsum);
  float* lse_t = reinterpret_cast<float*>(base + L.lse_t);
  p.lse_t = lse_t;
  launch_lse_group(s, lse, lse_t, stream);
  p.kl_rows = kl_rows;
  p.kl_lse = lse_idx;
  p.loss = loss;
  switch (D_idx) {
    case 64: return launch_kl_d<64>(s, L, p, stream);
    case 128: return launch_kl_d<128>(s, L, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
