// Alignment loss, backward: gradients of c * sum_rows KL_row with respect to
// the index inputs q_idx and k_idx (Sparse Attention Part II, section 3.2:
// the teacher is detached, so nothing flows into the main branch; the
// indexer's input is detached too, so these are the gradients the index
// projections receive).  For row (b, g, i) over its tokens T,
//   d KL_row / d z_s = Pidx_s - P_s,   Pidx_s = exp(z_s - LSE_z),
//   P_s = (1/G) sum_h exp(scale q_h . k_s - lse_h)   (the teacher),
// so with g_s = c (Pidx_s - P_s):
//   dq_idx[b][i][g] = sum_s g_s k_idx[b][s],
//   dk_idx[b][s] = sum over rows (b, g, i) with s in T of g_s q_idx[b][i][g].
// c is the caller's gradient of the loss divided by B * S_q * H_kv (the loss
// is the mean of the row terms).
//
// Schedule, per query chunk, on the attention's edge buckets: kl_grad_kernel
// runs the work items (a bucket's K_j and index keys loaded once, up to QT
// of its edges, two workgroups per CU) and leaves per edge g as a bf16 row
// and dq_idx as an fp16 record (added per row by kl_dq_merge_kernel);
// kl_dk_kernel then reduces each (batch, group, block)'s dk_idx over the
// block's edges in sorted order from those g rows, and after the last chunk
// kl_dk_reduce_kernel adds the groups (all share one index key head) in a
// fixed order.  Splitting the two sums this way lets the heavy pass run on
// independent work items instead of one long walk per block.
#include "bwd_common.h"

namespace msa {
using namespace edges;
namespace {



// Per-edge gradients on the attention's work items (the loss forward's
// schedule, kl_loss.hip: a work item loads K_j and the index keys of block j
// once and runs up to QT of its edges, two workgroups per CU): per edge the
// teacher P (head mean of the main branch's probabilities, from S = Q K^T and
// the forward's LSE), the index scores z and P_idx = 2^(z log2(e) - LSE_z),
// then g = c (P_idx - P) on the visible keys.  g leaves as a bf16 row per
// edge (for the dk_idx reduction, kl_dk_kernel) and, through this wave's LDS
// rows, gives dq_idx = sum_key g k_idx, one fp16 record per edge (per 32-dim
// quarter scaled by its largest magnitude, in the order the merge reads).
template <int G, int DIDX>
__global__ __launch_bounds__(kThreads, 2) void kl_grad_kernel(KlBwdParams kp) {
  const Params& p = kp.e;
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
  __shared__ float s_lsez[QT];                   // log2(e) * index-score LSE of the edge's row
  constexpr int GS = kBlock + 8;                 // bf16 per g row (padded)
  __shared__ __align__(16) uint16_t sg[4][QW][GS];  // per wave: g of its sub-tile [query][key]

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
    const float* lz = kp.lse_idx + (size_t)bg * p.S_q;
    for (int x = tid; x < QT; x += kThreads) s_lsez[x] = lz[s_i[x]] * kLog2e;
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

    // g = c (P_idx - P) on visible keys, P_idx = 2^(z log2(e) - LSE_z).
    // Stored as bf16 per (edge, key) for the dk_idx reduction and into this
    // wave's LDS rows for dq_idx; each (query, key) is held by one lane.
    const int wg = wave;
    float lsz[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) lsz[l] = s_lsez[e0 + q_of(l)];
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const int q = q_of(l);
      uint16_t* grow = kp.g_rec + (size_t)s_slot[e0 + q] * kBlock;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const float pidx = __builtin_amdgcn_exp2f(__builtin_fmaf(Z[l][u], kLog2e, -lsz[l]));
        const float gv = vis[l][u] ? kp.coef * (pidx - P[l][u]) : 0.f;
        const uint16_t gb = (uint16_t)(pack_bf16x2(gv, 0.f) & 0xFFFFu);
        const int key = (G >= 8 ? 2 * h + u : u) * 32 + n;
        grow[key] = gb;
        sg[wg][q][key] = gb;
      }
    }

    // dq_idx^T[d][q] = sum_key k_idx^T[d][key] g[q][key], 16x16x32 tiles: A
    // = k_idx^T (transposing reads of the row-major index tile: lane i of
    // each 16-lane group takes dim 16 t + i, keys 32 ks + 8 (lane / 16) + 0..7),
    // B = g rows of the wave's queries (query 16 qg + lane % 16, clamped past
    // QW).  Lane L then holds dims 16 t + 4 (L / 16) + 0..3 of that query.
    constexpr int NDQ = DIDX / 16;
    const int i16 = lane & 15, g16 = lane >> 4;
    // Queries 16 qg + i16 (a 16-column MFMA per 16 queries of the sub-tile).
#pragma unroll
    for (int qg = 0; qg < (QW + 15) / 16; ++qg) {
      f32x4 dqa[NDQ];
#pragma unroll
      for (int t = 0; t < NDQ; ++t) dqa[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int qcol = 16 * qg + i16;
      const uint16_t* gq = &sg[wg][min(qcol, QW - 1)][0];
#pragma unroll
      for (int ks = 0; ks < kBlock / 32; ++ks) {
        const u32x4 gbv = *reinterpret_cast<const u32x4*>(gq + 32 * ks + 8 * g16);
        const int ra = 32 * ks + 8 * g16 + (i16 >> 2), rb = ra + 4;
#pragma unroll
        for (int t = 0; t < NDQ; ++t) {
          const int c0 = 16 * t + 4 * (i16 & 3);
          const uint2 a0 = lds_read_tr16(reinterpret_cast<const char*>(itile) + lds_tile_off<ICH>(ra, c0, ra & (ICH - 1)));
          const uint2 a1 = lds_read_tr16(reinterpret_cast<const char*>(itile) + lds_tile_off<ICH>(rb, c0, rb & (ICH - 1)));
          dqa[t] = mfma16x16x32(u32x4{a0.x, a0.y, a1.x, a1.y}, gbv, dqa[t]);
        }
      }
      // The record of query qcol (lanes with qcol < QW): per 32-dim quarter
      // the largest magnitude m (over the quarter's two tiles and the four
      // lanes of the query), the values / m as fp16 at the record positions
      // the merge reads (rec_dim order: dim 16 (t % 2) + 4 g16 + x of the
      // quarter at 16 (g16 % 2) + 8 (t % 2) + 4 (g16 / 2) + x).
      const long slot = s_slot[e0 + min(qcol, QW - 1)];
#pragma unroll
      for (int qq = 0; qq < DIDX / 32; ++qq) {
        float m = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) m = max3abs(dqa[2 * qq][x], dqa[2 * qq + 1][x], m);
        m = __builtin_fmaxf(m, __shfl_xor(m, 16, 64));
        m = __builtin_fmaxf(m, __shfl_xor(m, 32, 64));
        const float inv = rec_inv(m);
        if (qcol < QW) {
          uint16_t* rec = kp.rec + slot * DIDX + 32 * qq;
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            const f32x4 v = dqa[2 * qq + t2];
            uint2 w2;
            w2.x = pack_f16x2(v[0] * inv, v[1] * inv);
            w2.y = pack_f16x2(v[2] * inv, v[3] * inv);
            *reinterpret_cast<uint2*>(rec + 16 * (g16 & 1) + 8 * t2 + 4 * (g16 >> 1)) = w2;
          }
          if (g16 == 0) kp.rec_sc[slot * (DIDX / 32) + qq] = m;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// dk_idx of block j for group (b, g): the sum over the block's edges (every
// query window of the chunk, each bucket in its sorted order) of
// g_e[key] q_idx[query(e)][g][:], with g from kl_grad_kernel.  Edges go
// through LDS 32 at a time (g rows and index-query rows, row-swizzled);
// wave w takes keys 32 w .. 32 w + 31 and all index dims, A = g^T and
// B = q_idx^T both from transposing reads (lane (n, h) takes edges
// 16 kk + 4 h + 0..3 and + 8..11 of step kk), the sums in registers.  This
// group's part is stored (fp32, added across chunks) and
// kl_dk_reduce_kernel adds the groups in a fixed order.
template <int DIDX>
__global__ __launch_bounds__(kThreads, 2) void kl_dk_kernel(KlBwdParams kp) {
  const Params& p = kp.e;
  constexpr int ICH = DIDX / 8;   // 16-byte chunks per index row
  constexpr int NDT = DIDX / 32;  // 32-dim tiles
  constexpr int EB = 32;          // edges per batch
  __shared__ u32x4 sgb[EB * 16];  // g rows [edge][128 keys], chunk c at c ^ rsw(edge)
  __shared__ u32x4 sqb[EB * ICH]; // index-query rows [edge][DIDX], chunk c at c ^ (rsw(edge) & (ICH - 1))
  const int BG = p.B * p.H_kv;
  const int j = blockIdx.x / BG;  // early (busier) blocks first
  const int bg = blockIdx.x - j * BG;
  const int b = bg / p.H_kv;
  const int g = bg - b * p.H_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, n = lane & 31;
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = zero16();
  const long flag_at = (long)bg * p.n_blk + j;
  const bool had = !kp.first && kp.dk_flag[flag_at] != 0;
  const int lr = lane & 15;
  // Batches of up to EB edges of one window's bucket, windows ascending.
  // Advances to the next batch; past the last one it returns false and
  // leaves the cursor on the last batch, so its addresses stay valid.
  struct Cursor {
    int w, e0, cnt;
    const int32_t* ed;
  };
  auto next = [&](Cursor& cu) {  // uniform
    Cursor t = cu;
    t.e0 += EB;
    while (t.e0 >= t.cnt) {
      if (++t.w >= p.n_win) return false;
      const long bucket = ((long)bg * p.n_win + t.w) * p.n_blk + j;
      t.cnt = __builtin_amdgcn_readfirstlane(p.counts[bucket]);
      t.ed = p.edges + __builtin_amdgcn_readfirstlane(p.offsets[bucket]);
      t.e0 = 0;
    }
    cu = t;
    return true;
  };
  // This thread's rows of a batch: g rows r = tid / 16 + 16 y (chunk
  // tid % 16) and index-query rows (tid + 256 y) / ICH.  A row past the
  // bucket's end repeats its last edge (loaded, in bounds) and is flagged
  // invalid, so it is staged as zeros.
  constexpr int NQ = EB * ICH / kThreads;
  struct Ids {
    int eg[2], eq[NQ];
    int valid;  // bit y: g row y; bit 2 + y: index-query row y
  };
  auto load_ids = [&](const Cursor& cu, Ids& d) {
    int v = 0;
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int r = (tid >> 4) + 16 * y;
      d.eg[y] = cu.ed[min(cu.e0 + r, cu.cnt - 1)];
      v |= (cu.e0 + r < cu.cnt) << y;
    }
#pragma unroll
    for (int y = 0; y < NQ; ++y) {
      const int r = (tid + kThreads * y) / ICH;
      d.eq[y] = cu.ed[min(cu.e0 + r, cu.cnt - 1)];
      v |= (cu.e0 + r < cu.cnt) << (2 + y);
    }
    d.valid = v;
  };
  struct Rows {
    u32x4 g[2], q[NQ];
    int valid;
  };
  auto fetch = [&](const Ids& d, Rows& f) {
#pragma unroll
    for (int y = 0; y < 2; ++y) f.g[y] = *reinterpret_cast<const u32x4*>(kp.g_rec + (size_t)d.eg[y] * kBlock + 8 * (tid & 15));
#pragma unroll
    for (int y = 0; y < NQ; ++y) {
      const int i = slot_query(p, bg, d.eq[y]);
      const int cc = (tid + kThreads * y) % ICH;
      f.q[y] = *reinterpret_cast<const u32x4*>(p.q_idx + (((size_t)b * p.S_q + i) * p.H_kv + g) * DIDX + 8 * cc);
    }
    f.valid = d.valid;
  };
  auto stage = [&](const Rows& f) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int r = (tid >> 4) + 16 * y, cc = tid & 15;
      sgb[r * 16 + (cc ^ rsw(r))] = (f.valid >> y) & 1 ? f.g[y] : z;
    }
#pragma unroll
    for (int y = 0; y < NQ; ++y) {
      const int x = tid + kThreads * y, r = x / ICH, cc = x % ICH;
      sqb[r * ICH + (cc ^ (rsw(r) & (ICH - 1)))] = (f.valid >> (2 + y)) & 1 ? f.q[y] : z;
    }
  };
  // Pipeline: batch n stages the rows fetched during n - 2, then requests
  // the ids of n + 3 and the rows of n + 2 before its products, so two
  // batches of loads are in flight behind each batch's barrier and MFMAs
  // (a block chosen by most queries walks thousands of batches).
  Cursor cur{-1, -EB, 0, nullptr};
  bool h0 = next(cur), h1 = false, h2 = false;
  const bool any = h0;  // some edge of this chunk selects the block
  Rows fx, fy;
  Ids ide, ido;  // ids of the even and of the odd batches
  if (h0) {
    Ids i0;
    load_ids(cur, i0);
    h1 = next(cur);
    load_ids(cur, ido);
    fetch(i0, fx);
    h2 = h1 && next(cur);
    load_ids(cur, ide);
    fetch(ido, fy);
  }
  auto step = [&](Rows& f, const Ids& use, Ids& load) {
    __syncthreads();  // the previous batch's LDS reads are done
    stage(f);
    __syncthreads();
    {
      const bool h3 = h2 && next(cur);
      load_ids(cur, load);
      fetch(use, f);
      h2 = h3;
    }
#pragma unroll
    for (int kk = 0; kk < EB / 16; ++kk) {
      const int r0 = 16 * kk + 4 * h;
      const int ra = r0 + (lr >> 2), rb = r0 + 8 + (lr >> 2);
      const int ck = 32 * wave + 16 * (n >> 4) + 4 * (lr & 3);
      const uint2 a0 = lds_read_tr16(reinterpret_cast<const char*>(sgb) + lds_tile_off(ra, ck, rsw(ra)));
      const uint2 a1 = lds_read_tr16(reinterpret_cast<const char*>(sgb) + lds_tile_off(rb, ck, rsw(rb)));
      const u32x4 ga = {a0.x, a0.y, a1.x, a1.y};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int cd = 32 * dt + 16 * (n >> 4) + 4 * (lr & 3);
        const uint2 b0 = lds_read_tr16(reinterpret_cast<const char*>(sqb) + lds_tile_off<ICH>(ra, cd, rsw(ra) & (ICH - 1)));
        const uint2 b1 = lds_read_tr16(reinterpret_cast<const char*>(sqb) + lds_tile_off<ICH>(rb, cd, rsw(rb) & (ICH - 1)));
        acc[dt] = mfma32x32x16(ga, u32x4{b0.x, b0.y, b1.x, b1.y}, acc[dt]);
      }
    }
  };
  while (h0) {  // uniform
    bool hb = h2;
    step(fx, ide, ido);
    h0 = h1;
    h1 = hb;
    if (!h0) break;
    hb = h2;
    step(fy, ido, ide);
    h0 = h1;
    h1 = hb;
  }
  // This group's part of the wave's keys (fp32, summed over chunks); a block
  // no edge of the chunk selects stores nothing, and its flag tells the
  // reduce whether the rows hold anything.
  if (any) {  // uniform
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int dcol = 32 * dt + n;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j * kBlock + 32 * wave + mfma32_row(r, lane);
        if (key >= p.S_k) continue;
        float* o = kp.dk_part + (((size_t)b * p.H_kv + g) * p.S_k + key) * DIDX + dcol;
        *o = had ? *o + acc[dt][r] : acc[dt][r];
      }
    }
  }
  if (tid == 0 && (kp.first || any)) kp.dk_flag[flag_at] = had || any;
}

// dq_idx of each row: the sum of its edges' records; 16 lanes per row, 8
// index dims each.  Every entry's selection, scale and record piece of a
// batch are requested before any is used (an entry that does not count
// reads its own slot, which lies inside the record array, and is skipped),
// and the sums still run in entry order.  Records are read once and dq_idx
// is written once, both non-temporal (32K loss backward: 3.56 -> 3.46 ms
// against one entry's loads at a time).
template <int DIDX>
__global__ __launch_bounds__(256) void kl_dq_merge_kernel(KlBwdParams kp) {
  constexpr int NDT = DIDX / 32;
  constexpr int NP = DIDX / 8;  // 16-byte pieces per record
  const Params& p = kp.e;
  const long r = ((long)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int f = threadIdx.x & 15;
  if (r >= (long)p.B * p.H_kv * p.Qc || f >= NP) return;
  const int il = (int)(r % p.Qc);
  const int bg = (int)(r / p.Qc);
  const int i = p.q0 + il;
  if (i >= p.S_q) return;
  const int b = bg / p.H_kv, g = bg - (bg / p.H_kv) * p.H_kv;
  const int32_t* sel = p.idx + ((long)bg * p.S_q + i) * p.topk;
  const int local = (i + p.S_k - p.S_q) / kBlock;
  const long slot0 = ((long)bg * p.Qc + il) * p.topk;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr int kB = 16;
  for (int e0 = 0; e0 < p.topk; e0 += kB) {
    u32x4 xs[kB];
    float scs[kB];
    int js[kB];
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int e = min(e0 + k, p.topk - 1);
      const long slot = slot0 + e;
      js[k] = sel[e];
      scs[k] = kp.rec_sc[slot * NDT + f / 4];
      xs[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp.rec + slot * DIDX + 8 * f));
    }
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      if (e0 + k >= p.topk || js[k] < 0 || js[k] > local) continue;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        acc[2 * y] += scs[k] * f16_lo(xs[k][y]);
        acc[2 * y + 1] += scs[k] * f16_hi(xs[k][y]);
      }
    }
  }
  uint16_t* o = kp.dq_idx + (((size_t)b * p.S_q + i) * p.H_kv + g) * DIDX;
  const int quarter = f / 4, pos = 8 * (f % 4);
  uint2 lo, hi;
  lo.x = pack_bf16x2(acc[0], acc[1]);
  lo.y = pack_bf16x2(acc[2], acc[3]);
  hi.x = pack_bf16x2(acc[4], acc[5]);
  hi.y = pack_bf16x2(acc[6], acc[7]);
  __builtin_nontemporal_store(((uint64_t)lo.y << 32) | lo.x, reinterpret_cast<uint64_t*>(o + rec_dim(quarter, pos)));
  __builtin_nontemporal_store(((uint64_t)hi.y << 32) | hi.x, reinterpret_cast<uint64_t*>(o + rec_dim(quarter, pos + 4)));
}

// dk_idx = the sum of the groups' parts, in group order, over the groups
// whose part of the key's block holds data (the others are zero).  Four
// workgroups per (batch, key block); four index dims per thread and step.
// Eight groups' flags and parts are requested before any is added (a part
// whose flag is clear is read, inside its buffer, and skipped).  Each part
// is read once and dk_idx written once, both non-temporal (32K loss
// backward: 3.56 -> 3.43 ms against one workgroup per block and one group's
// loads at a time).
template <int DIDX>
__global__ __launch_bounds__(256) void kl_dk_reduce_kernel(KlBwdParams kp) {
  const Params& p = kp.e;
  constexpr int kSplit = 4;
  const int bj = blockIdx.x / kSplit;
  const int part = blockIdx.x - bj * kSplit;
  const int b = bj / p.n_blk;
  const int j = bj - b * p.n_blk;
  const int keys = min(kBlock, p.S_k - j * kBlock);
  const int n4 = keys * DIDX / 4;
  const size_t row0 = (size_t)j * kBlock * DIDX;  // the block's first element in a [S_k][D_idx] plane
  for (int x = part * 256 + threadIdx.x; x < n4; x += 256 * kSplit) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int g0 = 0; g0 < p.H_kv; g0 += 8) {
      f32x4 v[8];
      int fl[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const long bg = (long)b * p.H_kv + min(g0 + k, p.H_kv - 1);
        fl[k] = kp.dk_flag[bg * p.n_blk + j];
        v[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kp.dk_part + bg * p.S_k * DIDX + row0 + 4 * x));
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (g0 + k >= p.H_kv || fl[k] == 0) continue;  // uniform
        acc.x += v[k].x; acc.y += v[k].y; acc.z += v[k].z; acc.w += v[k].w;
      }
    }
    const uint64_t o = ((uint64_t)pack_bf16x2(acc.z, acc.w) << 32) | pack_bf16x2(acc.x, acc.y);
    __builtin_nontemporal_store(o, reinterpret_cast<uint64_t*>(kp.dk_idx + (size_t)b * p.S_k * DIDX + row0 + 4 * x));
  }
}

template <int G, int DIDX>
void launch_kl_chunk_g(const AttnShape& s, const Layout& L, const KlBwdParams& kp, hipStream_t st) {
  hipLaunchKernelGGL((kl_grad_kernel<G, DIDX>), dim3((unsigned)L.T), dim3(kThreads), 0, st, kp);
  const long rows = (long)s.batch * s.H_kv * L.Qc;
  hipLaunchKernelGGL(kl_dq_merge_kernel<DIDX>, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, st, kp);
  hipLaunchKernelGGL(kl_dk_kernel<DIDX>, dim3((unsigned)(s.batch * s.H_kv * s.n_blk)), dim3(kThreads), 0, st, kp);
}

template <int DIDX>
hipError_t launch_kl_chunk_d(const AttnShape& s, const Layout& L, const KlBwdParams& kp, hipStream_t st) {
  switch (kp.e.G) {
    case 1: launch_kl_chunk_g<1, DIDX>(s, L, kp, st); break;
    case 2: launch_kl_chunk_g<2, DIDX>(s, L, kp, st); break;
    case 4: launch_kl_chunk_g<4, DIDX>(s, L, kp, st); break;
    case 8: launch_kl_chunk_g<8, DIDX>(s, L, kp, st); break;
    case 16: launch_kl_chunk_g<16, DIDX>(s, L, kp, st); break;
    case 32: launch_kl_chunk_g<32, DIDX>(s, L, kp, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

namespace edges {
hipError_t launch_kl_chunk(const AttnShape& s, const Layout& L, const KlBwdParams& kp, hipStream_t st) {
  switch (kp.D_idx) {
    case 64: return launch_kl_chunk_d<64>(s, L, kp, st);
    case 128: return launch_kl_chunk_d<128>(s, L, kp, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_kl_dk_reduce(const KlBwdParams& kp, int D_idx, long blocks, hipStream_t st) {
  if (D_idx == 64) hipLaunchKernelGGL(kl_dk_reduce_kernel<64>, dim3((unsigned)(4 * blocks)), dim3(256), 0, st, kp);
  else hipLaunchKernelGGL(kl_dk_reduce_kernel<128>, dim3((unsigned)(4 * blocks)), dim3(256), 0, st, kp);
  return hipGetLastError();
}
}  // namespace edges

hipError_t launch_kl_loss_bwd(const AttnShape& s, int D_idx, const uint16_t* q, const uint16_t* k,
                              const uint16_t* q_idx, const uint16_t* k_idx, const int32_t* idx,
                              const float* lse, const float* lse_idx, float coef, uint16_t* dq_idx,
                              uint16_t* dk_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int qc = kl_bwd_chunk(s, D_idx, ws_bytes);
  if (qc <= 0) return hipErrorInvalidValue;
  const KlBwdLayout K = make_kl_bwd_layout(s, D_idx, qc);
  char* base = static_cast<char*>(ws);
  KlBwdParams kp{};
  kp.e = base_params(s, K.L, base, idx);
  kp.e.q = q; kp.e.k = k; kp.e.q_idx = q_idx; kp.e.k_idx = k_idx;
  kp.lse_idx = lse_idx; kp.coef = coef;
  float* lse_t = reinterpret_cast<float*>(base + K.lse_t);
  kp.e.lse_t = lse_t;
  launch_lse_group(s, lse, lse_t, stream);
  kp.rec = reinterpret_cast<uint16_t*>(base + K.rec);
  kp.rec_sc = reinterpret_cast<float*>(base + K.rec_sc);
  kp.g_rec = reinterpret_cast<uint16_t*>(base + K.g_rec);
  kp.sink = K.L.E;
  kp.dk_part = reinterpret_cast<float*>(base + K.dk_part);
  kp.dk_flag = reinterpret_cast<int32_t*>(base + K.dk_flag);
  kp.dq_idx = dq_idx; kp.dk_idx = dk_idx; kp.D_idx = D_idx;
  const Layout& L = K.L;
  for (int q0 = 0, ci = 0; q0 < s.S_q; q0 += L.Qc, ++ci) {
    kp.e.q0 = q0;
    kp.first = ci == 0;
    launch_build(s, L, kp.e, stream);
    launch_bucket_sort(L, kp.e, stream);
    const hipError_t err = launch_kl_chunk(s, L, kp, stream);
    if (err != hipSuccess) return err;
  }
  return launch_kl_dk_reduce(kp, D_idx, (long)s.batch * s.n_blk, stream);
}

}  // namespace msa
