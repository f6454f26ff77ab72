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
// Schedule: as the main-branch backward (attn_bwd.hip).  One workgroup per
// (batch, group, block) runs every edge of the block in sorted order; its four
// waves split the block's keys.  Per 32-row sub-tile (32 / G queries x G
// heads) it recomputes the teacher from S = Q K^T and the forward's LSE (the
// head mean is an in-lane sum plus one half-wave exchange), the index scores
// z (16x16x32 tiles with the sub-tile's queries on every 16-lane group for
// G >= 8, else the query's index row repeated on its heads' rows), then g.  The
// block's dk_idx accumulates in registers (per group; the groups are added in
// a fixed order at the end, since all groups share one index key head);
// dq_idx of each edge goes through LDS and a per-edge fp16 record, added per
// row by a merge.
#include "bwd_common.h"

namespace msa {
using namespace edges;
namespace {



template <int G, int DIDX>
__global__ __launch_bounds__(kThreads, 1) void kl_bwd_kernel(KlBwdParams kp) {
  constexpr int QW = 32 / G;
  constexpr int ICH = DIDX / 8;             // 16-byte chunks per index row
  constexpr int NDT = DIDX / 32;            // 32-dim tiles of the index dims
  constexpr int RPS = G >= 8 ? G / 2 : G;   // registers of one query in a lane
  constexpr int NL = 16 / RPS;              // queries per lane
  const Params& p = kp.e;
  __shared__ u32x4 ktile[kBlock * 16];      // K_j rows, chunk c at c ^ (key & 15)
  __shared__ u32x4 itile[kBlock * ICH];     // k_idx rows, chunk c at c ^ (key & (ICH - 1))
  __shared__ u32x4 sq[32 * 16];             // Q rows of the sub-tile, chunk c at c ^ rsw(row)
  __shared__ u32x4 sqi[32 * ICH];           // q_idx row of each row's query, chunk c at c ^ (rsw(row) & (ICH - 1))
  __shared__ __align__(16) uint16_t sg[32 * kGStride];  // g [row][key] bf16
  __shared__ __align__(16) float s_lse[32];
  __shared__ float s_lsez[QW];
  __shared__ int s_t[QW];
  __shared__ int s_slot[QW];

  const int BG = p.B * p.H_kv;
  const int j = blockIdx.x / BG;
  const int bg = blockIdx.x - j * BG;
  const int b = bg / p.H_kv;
  const int g = bg - b * p.H_kv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int n = lane & 31;
  const int off = p.S_k - p.S_q;
  constexpr float kLog2e = 1.4426950408889634f;
  const float c = p.scale_log2;
  const float invG = 1.f / G;


  f32x16 dk_acc[NDT];  // [key row][index-dim tile]: this wave's 32 keys
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dk_acc[dt] = zero16();
  const int key0 = 32 * wave;
  const int key_abs = j * kBlock + key0 + n;

  struct Cursor {
    int w, base, cnt;
    const int32_t* ed;
  };
  // Advances to the next sub-tile; past the last one it returns false and
  // leaves the cursor on the last sub-tile, so its addresses stay valid.
  auto next = [&](Cursor& cu) {  // uniform
    Cursor t = cu;
    t.base += QW;
    while (t.base >= t.cnt) {
      if (++t.w >= p.n_win) return false;
      const long bucket = ((long)bg * p.n_win + t.w) * p.n_blk + j;
      t.cnt = __builtin_amdgcn_readfirstlane(p.counts[bucket]);
      t.ed = p.edges + __builtin_amdgcn_readfirstlane(p.offsets[bucket]);
      t.base = 0;
    }
    cu = t;
    return true;
  };
  const int pr = tid & 15, cc = tid >> 4;  // staging role: rows (2 pr, 2 pr + 1), chunk cc
  // Edge ids one sub-tile ahead of the rows: e for this thread's staging
  // rows (one query unless G = 1), e2 for the statistics of row tid % 32;
  // validity flags come from the cursor alone.
  constexpr int NI = G >= 2 ? 1 : 2;
  struct Ids {
    int e[NI];
    int e2;
    int valid;  // bit y: e[y]; bit 2: e2
  };
  auto load_ids = [&](const Cursor& cu, Ids& d) {
    int v = 0;
#pragma unroll
    for (int y = 0; y < NI; ++y) {
      const int q = (2 * pr + y) / G;
      d.e[y] = cu.ed[min(cu.base + q, cu.cnt - 1)];
      v |= (cu.base + q < cu.cnt) << y;
    }
    const int q2 = (tid & 31) / G;
    d.e2 = cu.ed[min(cu.base + q2, cu.cnt - 1)];
    d.valid = v | (cu.base + q2 < cu.cnt) << 2;
  };
  // The rows of one sub-tile as fetched by this thread (two sets alternate):
  // Q rows, the query's index row (chunk cc % ICH; threads past ICH repeat
  // a chunk and do not stage it), and for the first 32 threads the row's
  // main-branch LSE and its query's index-score LSE.
  struct Fetched {
    u32x4 qa[2], qi[2];
    float lse, lsez;
    Ids id;
  };
  auto fetch = [&](const Ids& d, Fetched& f) {
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int r = 2 * pr + y, hh = r % G;
      const int i = slot_query(p, bg, d.e[y % NI]);
      f.qa[y] = *reinterpret_cast<const u32x4*>(p.q + (((size_t)b * p.S_q + i) * p.H_q + g * G + hh) * kD + 8 * cc);
      f.qi[y] = *reinterpret_cast<const u32x4*>(p.q_idx + (((size_t)b * p.S_q + i) * p.H_kv + g) * DIDX +
                                                8 * (cc % ICH));
    }
    if (tid < 32) {
      const int hh = tid % G;
      const int i = slot_query(p, bg, d.e2);
      f.lse = p.lse_t[((size_t)bg * p.S_q + i) * G + hh];
      f.lsez = kp.lse_idx[((size_t)b * p.H_kv + g) * p.S_q + i];
    }
    f.id = d;
  };
  // Pipeline, in issue order: sub-tile n stages rows fetched during n - 2,
  // requests the ids of n + 3 and then the rows of n + 2, computes, and
  // stores its dq_idx records.  Every request but the statistics is
  // unconditional (past the end the cursor repeats the last sub-tile, and
  // rows that store no record write the sink), so the memory counter's
  // order is the same on every iteration and its waits stay tight.
  Cursor cur{-1, -QW, 0, nullptr};
  // The block's tiles, loaded only when some edge selects the block (a
  // workgroup without edges just writes zero gradients).
  auto load_tiles = [&]() {  // K_j and k_idx of block j (rows past S_k clamped: never visible)
    const size_t row_stride = (size_t)p.H_kv * kD;
    const uint16_t* kb = p.k + ((size_t)b * p.S_k * p.H_kv + g) * kD;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int qd = it * kThreads + tid;
      const int row = qd >> 4, cc = qd & 15;
      const int s = min(j * kBlock + row, p.S_k - 1);
      ktile[row * 16 + (cc ^ (row & 15))] = *reinterpret_cast<const u32x4*>(kb + (size_t)s * row_stride + 8 * cc);
    }
    const uint16_t* ib = p.k_idx + (size_t)b * p.S_k * DIDX;
#pragma unroll
    for (int it = 0; it < kBlock * ICH / kThreads; ++it) {
      const int qd = it * kThreads + tid;
      const int row = qd / ICH, cc = qd % ICH;
      const int s = min(j * kBlock + row, p.S_k - 1);
      itile[row * ICH + (cc ^ (row & (ICH - 1)))] = *reinterpret_cast<const u32x4*>(ib + (size_t)s * DIDX + 8 * cc);
    }
  };
  bool h0 = next(cur), h1 = false, h2 = false;
  if (h0) load_tiles();  // uniform
  // Whether this group's dk_part rows of the block already hold an earlier
  // chunk's sums; read before the loop's barriers, written after them.
  const bool any = h0;
  const long flag_at = (long)bg * p.n_blk + j;
  const bool had = !kp.first && kp.dk_flag[flag_at] != 0;
  Fetched fx, fy;
  Ids ide, ido;  // ids of the even and of the odd sub-tiles

  // The dq_idx record of each query of a sub-tile, written by the lanes of
  // its first row (the other rows hold the same values); every other lane,
  // and the dummy stores of the prologue, write the sink.
  auto store_records = [&](const f32x16& qacc, bool dummy) {
    const int q = n / G, hh = n - (n / G) * G;
    const int sl = dummy ? -1 : s_slot[q];
    const long slot = hh == 0 && sl >= 0 ? sl : kp.sink;
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) m = max3abs(qacc[r], qacc[r], m);
    m = __builtin_fmaxf(m, swap_halves(m));
    const float inv = m > 0.f ? __builtin_amdgcn_rcpf(m) : 0.f;
    u32x4* rec = reinterpret_cast<u32x4*>(kp.rec + (slot * NDT + wave) * 32 + 16 * h);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 v4;
#pragma unroll
      for (int x = 0; x < 4; ++x)
        v4[x] = pack_f16x2(qacc[8 * half + 2 * x] * inv, qacc[8 * half + 2 * x + 1] * inv);
      rec[half] = v4;
    }
    kp.rec_sc[slot * NDT + wave] = m;  // both halves store the same m
  };

  // The block's operands that are the same for every sub-tile stay in
  // registers once loaded (K_j rows of the wave's keys for S, their k_idx
  // rows for z, k_idx^T of the wave's index dims for dq_idx), which takes
  // three quarters of the LDS reads of a sub-tile off the LDS.
  constexpr int NZ = G >= 8 ? 2 * (DIDX / 32) : DIDX / 16;
  u32x4 kf[8], zf[NZ], qf[8];
  auto load_frags = [&]() {
    const int krow = key0 + n;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kf[ks] = ktile[krow * 16 + ((2 * ks + h) ^ (krow & 15))];
    if constexpr (G >= 8) {
      const int k0 = key0 + (lane & 15), k1 = k0 + 16;
#pragma unroll
      for (int ks = 0; ks < DIDX / 32; ++ks) {
        const int ch = 4 * ks + (lane >> 4);
        zf[2 * ks] = itile[k0 * ICH + (ch ^ (k0 & (ICH - 1)))];
        zf[2 * ks + 1] = itile[k1 * ICH + (ch ^ (k1 & (ICH - 1)))];
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < DIDX / 16; ++ks) {
        const int ch = 2 * ks + h;
        zf[ks] = itile[krow * ICH + (ch ^ (krow & (ICH - 1)))];
      }
    }
    if (wave < NDT) {
      const int lr = lane & 15;
      const int c0 = 32 * wave + 16 * (n >> 4) + 4 * (lr & 3);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int k0 = 16 * ks + 8 * h + (lr >> 2), k1 = k0 + 4;
        const uint2 a0 = lds_read_tr16(reinterpret_cast<const char*>(itile) + lds_tile_off<ICH>(k0, c0, k0 & (ICH - 1)));
        const uint2 a1 = lds_read_tr16(reinterpret_cast<const char*>(itile) + lds_tile_off<ICH>(k1, c0, k1 & (ICH - 1)));
        qf[ks] = u32x4{a0.x, a0.y, a1.x, a1.y};
      }
    }
  };

  auto step = [&](Fetched& f, const Ids& use, Ids& load) {
    __syncthreads();  // the previous sub-tile's LDS reads are done
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int r = 2 * pr + y;
      sq[r * 16 + (cc ^ rsw(r))] = f.qa[y];
      if (cc < ICH) sqi[r * ICH + (cc ^ (rsw(r) & (ICH - 1)))] = f.qi[y];
    }
    if (tid < 32) {
      const int x = f.id.e2;
      const bool valid = (f.id.valid >> 2) & 1;
      s_lse[tid] = valid ? f.lse : __builtin_inff();
      if (tid % G == 0) {
        const int i = slot_query(p, bg, x);
        s_lsez[tid / G] = valid ? f.lsez * kLog2e : __builtin_inff();
        s_t[tid / G] = valid ? i + off : -1;
        s_slot[tid / G] = valid ? x : -1;
      }
    }
    __syncthreads();
    {
      const bool h3 = h2 && next(cur);
      load_ids(cur, load);
      fetch(use, f);
      h2 = h3;
    }
    asm volatile("" ::: "memory");

    // S and z for this wave's 32 keys: rows on registers, keys on lanes.
    f32x16 sacc = zero16();
    const int krow = key0 + n;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int ch = 2 * ks + h;
      sacc = mfma32x32x16(sq[n * 16 + (ch ^ rsw(n))], kf[ks], sacc);
    }
    // z of query slot l at key key0 + n.  With G >= 8 a sub-tile has at most
    // 4 queries: 16x16x32 tiles whose A row m is query m % 4 (the last one
    // repeated past QW), keys key0 .. + 15 and key0 + 16 .. + 31; lane n takes
    // the tile holding its key, and register l is query l (= the query of
    // slot l).  Otherwise z repeats each query's index row on its heads' rows.
    float zv[NL];
    if constexpr (G >= 8) {
      const int qr = min(lane & 3, QW - 1) * G;  // a row of query qr / G in sqi
      const int k0 = key0 + (lane & 15), k1 = k0 + 16;
      f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DIDX / 32; ++ks) {
        const int ch = 4 * ks + (lane >> 4);
        const u32x4 a = sqi[qr * ICH + (ch ^ (rsw(qr) & (ICH - 1)))];
        z0 = mfma16x16x32(a, zf[2 * ks], z0);
        z1 = mfma16x16x32(a, zf[2 * ks + 1], z1);
      }
      const bool upper = (lane >> 4) & 1;
#pragma unroll
      for (int l = 0; l < NL; ++l) zv[l] = upper ? z1[l] : z0[l];
    } else {
      f32x16 zacc = zero16();
#pragma unroll
      for (int ks = 0; ks < DIDX / 16; ++ks) {
        const int ch = 2 * ks + h;
        zacc = mfma32x32x16(sqi[n * ICH + (ch ^ (rsw(n) & (ICH - 1)))], zf[ks], zacc);
      }
#pragma unroll
      for (int l = 0; l < NL; ++l) zv[l] = zacc[l * RPS];
    }
    // Teacher per (query slot l, key): the mean over the query's heads.
    float lse4[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 a = *reinterpret_cast<const float4*>(&s_lse[8 * r4 + 4 * h]);
      lse4[4 * r4] = a.x; lse4[4 * r4 + 1] = a.y; lse4[4 * r4 + 2] = a.z; lse4[4 * r4 + 3] = a.w;
    }
    float gq[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      float acc = 0.f;
#pragma unroll
      for (int rr = 0; rr < RPS; ++rr) {
        const int r = l * RPS + rr;
        acc += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -lse4[r]));
      }
      if constexpr (G >= 8) acc += swap_halves(acc);
      const int q = mfma32_row(l * RPS, lane) / G;
      const bool vis = key_abs <= s_t[q];
      const float pidx = __builtin_amdgcn_exp2f(__builtin_fmaf(zv[l], kLog2e, -s_lsez[q]));
      gq[l] = vis ? kp.coef * (pidx - acc * invG) : 0.f;
    }
    // dk_idx += g^T q_idx: A = g of each register's row (a query's value on
    // each of its G rows, times 1/G), B = the rows' index rows, transposed.
    {
      const int lr = lane & 15;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 ga;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r0 = 8 * kk + 2 * x;
          ga[x] = pack_bf16x2(gq[r0 / RPS] * invG, gq[(r0 + 1) / RPS] * invG);
        }
        const int rbase = 16 * kk + 4 * h;
        const int ra = rbase + (lr >> 2), rb = rbase + 8 + (lr >> 2);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int c0 = 32 * dt + 16 * (n >> 4) + 4 * (lr & 3);
          const uint2 b0 = lds_read_tr16(reinterpret_cast<const char*>(sqi) + lds_tile_off<ICH>(ra, c0, rsw(ra) & (ICH - 1)));
          const uint2 b1 = lds_read_tr16(reinterpret_cast<const char*>(sqi) + lds_tile_off<ICH>(rb, c0, rsw(rb) & (ICH - 1)));
          const u32x4 bb = {b0.x, b0.y, b1.x, b1.y};
          dk_acc[dt] = mfma32x32x16(ga, bb, dk_acc[dt]);
        }
      }
    }
    // g to LDS as [row][key] for dq_idx (each row carries its query's g).
#pragma unroll
    for (int r = 0; r < 16; ++r)
      sg[mfma32_row(r, lane) * kGStride + key0 + n] = (uint16_t)(pack_bf16x2(gq[r / RPS], 0.f) & 0xFFFFu);
    __syncthreads();

    // dq_idx^T[c'][row] = sum_key k_idx^T[c'][key] g[row][key] for index dims
    // 32 wave .. 32 wave + 31 (waves past D_idx / 32 idle); one record per query.
    if (wave < NDT) {
      f32x16 qacc = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 gb = *reinterpret_cast<const u32x4*>(&sg[n * kGStride + 16 * ks + 8 * h]);
        qacc = mfma32x32x16(qf[ks], gb, qacc);
      }
      store_records(qacc, false);
    }
  };
  if (h0) {  // uniform
    Ids i0;
    load_ids(cur, i0);
    h1 = next(cur);
    load_ids(cur, ido);
    fetch(i0, fx);
    if (wave < NDT) store_records(zero16(), true);
    h2 = h1 && next(cur);
    load_ids(cur, ide);
    fetch(ido, fy);
    if (wave < NDT) store_records(zero16(), true);
  }
  if (h0) {  // uniform
    __syncthreads();  // the tiles are in LDS
    load_frags();
  }
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

  // This group's dk_idx for the wave's keys (fp32, summed over chunks).  A
  // block that no edge of the chunk selects stores nothing: its flag tells
  // the reduce whether the rows hold anything (on a decode-shaped problem
  // nearly every block is such a block).
  if (any) {  // uniform
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int dcol = 32 * dt + n;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j * kBlock + key0 + mfma32_row(r, lane);
        if (key >= p.S_k) continue;
        float* o = kp.dk_part + (((size_t)b * p.H_kv + g) * p.S_k + key) * DIDX + dcol;
        *o = had ? *o + dk_acc[dt][r] : dk_acc[dt][r];
      }
    }
  }
  if (tid == 0 && (kp.first || any)) kp.dk_flag[flag_at] = had || any;
}

// dq_idx of each row: the sum of its edges' records; 16 lanes per row, 8
// index dims each.
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
  for (int e = 0; e < p.topk; ++e) {
    const int jj = sel[e];
    if (jj < 0 || jj > local) continue;
    const long slot = slot0 + e;
    const float sc = kp.rec_sc[slot * NDT + f / 4];
    const u32x4 x = *reinterpret_cast<const u32x4*>(kp.rec + slot * DIDX + 8 * f);
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      acc[2 * y] += sc * f16_lo(x[y]);
      acc[2 * y + 1] += sc * f16_hi(x[y]);
    }
  }
  uint16_t* o = kp.dq_idx + (((size_t)b * p.S_q + i) * p.H_kv + g) * DIDX;
  const int quarter = f / 4, pos = 8 * (f % 4);
  uint2 lo, hi;
  lo.x = pack_bf16x2(acc[0], acc[1]);
  lo.y = pack_bf16x2(acc[2], acc[3]);
  hi.x = pack_bf16x2(acc[4], acc[5]);
  hi.y = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint2*>(o + rec_dim(quarter, pos)) = lo;
  *reinterpret_cast<uint2*>(o + rec_dim(quarter, pos + 4)) = hi;
}

// dk_idx = the sum of the groups' parts, in group order, over the groups
// whose part of the key's block holds data (the others are zero).  One
// workgroup per (batch, key block); four index dims per thread and step.
template <int DIDX>
__global__ __launch_bounds__(256) void kl_dk_reduce_kernel(KlBwdParams kp) {
  const Params& p = kp.e;
  const int b = blockIdx.x / p.n_blk;
  const int j = blockIdx.x - b * p.n_blk;
  const int keys = min(kBlock, p.S_k - j * kBlock);
  const int n4 = keys * DIDX / 4;
  const size_t row0 = (size_t)j * kBlock * DIDX;  // the block's first element in a [S_k][D_idx] plane
  for (int x = threadIdx.x; x < n4; x += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int g = 0; g < p.H_kv; ++g) {
      const long bg = (long)b * p.H_kv + g;
      if (kp.dk_flag[bg * p.n_blk + j] == 0) continue;  // uniform
      const float4 v = *reinterpret_cast<const float4*>(kp.dk_part + bg * p.S_k * DIDX + row0 + 4 * x);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    uint2 o;
    o.x = pack_bf16x2(acc.x, acc.y);
    o.y = pack_bf16x2(acc.z, acc.w);
    *reinterpret_cast<uint2*>(kp.dk_idx + (size_t)b * p.S_k * DIDX + row0 + 4 * x) = o;
  }
}

}  // namespace

namespace edges {
hipError_t launch_kl_dq_merge(const KlBwdParams& kp, int D_idx, long rows, hipStream_t st) {
  const dim3 grid((unsigned)((rows * 16 + 255) / 256));
  if (D_idx == 64) hipLaunchKernelGGL(kl_dq_merge_kernel<64>, grid, dim3(256), 0, st, kp);
  else hipLaunchKernelGGL(kl_dq_merge_kernel<128>, grid, dim3(256), 0, st, kp);
  return hipGetLastError();
}

hipError_t launch_kl_dk_reduce(const KlBwdParams& kp, int D_idx, long blocks, hipStream_t st) {
  if (D_idx == 64) hipLaunchKernelGGL(kl_dk_reduce_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, st, kp);
  else hipLaunchKernelGGL(kl_dk_reduce_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, st, kp);
  return hipGetLastError();
}
}  // namespace edges

namespace {

template <int G, int DIDX>
hipError_t launch_kl_bwd_g(const AttnShape& s, const KlBwdLayout& K, KlBwdParams kp, hipStream_t st) {
  const Layout& L = K.L;
  for (int q0 = 0, ci = 0; q0 < s.S_q; q0 += L.Qc, ++ci) {
    kp.e.q0 = q0;
    kp.first = ci == 0;
    launch_build(s, L, kp.e, st);
    launch_bucket_sort(L, kp.e, st);
    hipLaunchKernelGGL((kl_bwd_kernel<G, DIDX>), dim3((unsigned)(s.batch * s.H_kv * s.n_blk)), dim3(kThreads), 0, st, kp);
    const long rows = (long)s.batch * s.H_kv * L.Qc;
    hipLaunchKernelGGL(kl_dq_merge_kernel<DIDX>, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, st, kp);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(kl_dk_reduce_kernel<DIDX>, dim3((unsigned)((long)s.batch * s.n_blk)), dim3(256), 0, st, kp);
  return hipGetLastError();
}

template <int DIDX>
hipError_t launch_kl_bwd_d(const AttnShape& s, const KlBwdLayout& K, const KlBwdParams& kp, hipStream_t st) {
  switch (kp.e.G) {
    case 1: return launch_kl_bwd_g<1, DIDX>(s, K, kp, st);
    case 2: return launch_kl_bwd_g<2, DIDX>(s, K, kp, st);
    case 4: return launch_kl_bwd_g<4, DIDX>(s, K, kp, st);
    case 8: return launch_kl_bwd_g<8, DIDX>(s, K, kp, st);
    case 16: return launch_kl_bwd_g<16, DIDX>(s, K, kp, st);
    case 32: return launch_kl_bwd_g<32, DIDX>(s, K, kp, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

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
  kp.sink = K.L.E;
  kp.dk_part = reinterpret_cast<float*>(base + K.dk_part);
  kp.dk_flag = reinterpret_cast<int32_t*>(base + K.dk_flag);
  kp.dq_idx = dq_idx; kp.dk_idx = dk_idx; kp.D_idx = D_idx;
  switch (D_idx) {
    case 64: return launch_kl_bwd_d<64>(s, K, kp, stream);
    case 128: return launch_kl_bwd_d<128>(s, K, kp, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
