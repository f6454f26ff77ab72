// Main branch, backward: dQ, dK, dV of the block-sparse causal GQA attention
// from the upstream gradient dO.  The selection is a discrete choice and
// carries no gradient; inside it the attention is a softmax attention over
// the visible tokens of the selected blocks (Sparse Attention Part II,
// section 2), differentiated the usual way.  With P the probabilities of a
// head over its tokens and Delta = sum_d dO O (= sum_s P_s dP_s):
//   dP_s = dO . v_s,  dS_s = P_s (dP_s - Delta),
//   dV_s += P_s dO,  dK_s += scale dS_s q,  dq = scale sum_s dS_s k_s.
//
// Schedule (the re-parameterisation of block-sparse attention as a
// variable-length attention over key blocks that the MSA notes credit to
// MoBA): the forward's edge buckets, walked KV-stationary.  One workgroup owns
// one (batch, group, block): it loads K_j and V_j into LDS once and
// runs every edge of the block (all query windows of the chunk), so dK_j and
// dV_j accumulate in registers and are written once, with no atomics.  A
// block that far more queries select than the rest is cut into segments of
// its sub-tiles, one workgroup each, whose fp32 parts are added afterwards in
// segment order (seg_count / seg_scan / seg_reduce below).  Its
// four waves split the block's 128 keys; the edges go through in sub-tiles of
// 32 MFMA rows (32 / G queries x G heads) staged in LDS, in a fixed order
// (windows ascending, slots sorted inside each bucket), so the sums and the
// results are identical from run to run.  Transposed operands (K^T, dO^T,
// Q^T) come from the row-major tiles through transposing LDS reads.  dq of an
// edge needs all 128 keys: dS goes through LDS and each wave then forms a
// quarter of the head dims, written as a per-edge fp16 record; a merge adds a
// query's records.
#include "bwd_common.h"

namespace msa {
using namespace edges;
namespace {

constexpr int kSStride = kBlock + 8;  // bf16 per row of dS [row][key]
constexpr int kSortSmall = 1024;      // buckets up to this size sort in a small workgroup


// Delta = sum_d dO O per (b, h, i): 16 lanes per row, one 16-byte chunk each.
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams bp) {
  const Params& p = bp.e;
  const long row = ((long)blockIdx.x * 256 + threadIdx.x) >> 4;  // (b, i, h), h fastest
  const int c = threadIdx.x & 15;
  const long rows = (long)p.B * p.S_q * p.H_q;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(bp.dout + row * kD + 8 * c);
    const u32x4 o = *reinterpret_cast<const u32x4*>(bp.out + row * kD + 8 * c);
#pragma unroll
    for (int x = 0; x < 4; ++x) acc += bf16_lo(a[x]) * bf16_lo(o[x]) + bf16_hi(a[x]) * bf16_hi(o[x]);
  }
  acc = row_sum16(acc);
  if (row < rows && c == 0) {
    const int h = (int)(row % p.H_q);
    const long bi = row / p.H_q;
    const int i = (int)(bi % p.S_q);
    const int b = (int)(bi / p.S_q);
    const long li = ((long)b * p.H_q + h) * p.S_q + i;
    const int G = p.H_q / p.H_kv;
    bp.stat[(((long)b * p.H_kv + h / G) * p.S_q + i) * G + h % G] = make_float2(bp.lse[li] * 1.4426950408889634f, acc);
  }
}

// Sorts each bucket's edge slots ascending (the fill scatters them in an
// order that depends on scheduling).  Bitonic network in LDS over the next
// power of two of the bucket's size; SIZE bounds the buckets this instance
// takes (the other instance skips them).
//
// Large buckets first try a counting sort: slot = row * topk + e with row =
// bg * Qc + il, and a bucket (bg, window w, block j) holds at most one entry
// per query of the window unless a row repeats a block.  One bit per query
// of the window marks the bucket's rows and the entry index e is kept
// beside it; the set bits, taken in order, give the slots in ascending
// order.  A repeated row (a bit found set) leaves the bucket to the network.
template <int SIZE, bool LARGE>
__global__ __launch_bounds__(256) void bucket_sort_kernel(Params p) {
  __shared__ int32_t v[SIZE];
  __shared__ int32_t scan[256];
  __shared__ int dup;
  const long bucket = blockIdx.x;
  const int n = p.counts[bucket];
  if (n <= 1 || (LARGE ? n <= kSortSmall : n > kSortSmall)) return;  // uniform
  int32_t* e = p.edges + p.offsets[bucket];
  const int tid = threadIdx.x;
  if constexpr (LARGE) {
    static_assert(SIZE >= kMaxWindow / 32 + kMaxWindow / 4, "bit set and entry bytes must fit in v");
    const int w = (int)((bucket / p.n_blk) % p.n_win);
    const int bg = (int)(bucket / ((long)p.n_win * p.n_blk));
    const int row0 = bg * p.Qc + w * p.W;  // the window's first row
    const int nw = (p.W + 31) / 32;        // words of the bit set (W <= kMaxWindow)
    uint32_t* bits = reinterpret_cast<uint32_t*>(v);
    uint8_t* ent = reinterpret_cast<uint8_t*>(v + kMaxWindow / 32);
    for (int x = tid; x < nw; x += 256) bits[x] = 0u;
    if (tid == 0) dup = 0;
    __syncthreads();
    for (int x = tid; x < n; x += 256) {
      const int slot = e[x];
      const int row = slot_row(p, slot);
      const int r = row - row0;  // 0 <= r < W for every slot of the bucket
      if ((unsigned)r >= (unsigned)p.W) {
        dup = 1;
        continue;
      }
      const uint32_t bit = 1u << (r & 31);
      if (atomicOr(&bits[r >> 5], bit) & bit) dup = 1;
      ent[r] = (uint8_t)(slot - row * p.topk);  // topk <= 64
    }
    __syncthreads();
    if (!dup) {  // uniform
      // Exclusive prefix of the words' popcounts: thread t holds words 2t, 2t + 1.
      const int w0 = 2 * tid;
      const int c0 = w0 < nw ? __popc(bits[w0]) : 0;
      const int c1 = w0 + 1 < nw ? __popc(bits[w0 + 1]) : 0;
      scan[tid] = c0 + c1;
      __syncthreads();
      for (int d = 1; d < 256; d <<= 1) {  // Hillis-Steele inclusive scan
        const int a = tid >= d ? scan[tid - d] : 0;
        __syncthreads();
        scan[tid] += a;
        __syncthreads();
      }
      int pos = scan[tid] - c0 - c1;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (w0 + k >= nw) break;
        uint32_t m = bits[w0 + k];
        while (m) {
          const int r = 32 * (w0 + k) + __builtin_ctz(m);
          m &= m - 1u;
          e[pos++] = (row0 + r) * p.topk + ent[r];
        }
      }
      return;
    }
    __syncthreads();  // v is reused below
  }
  if (n > SIZE) return;  // more edges than queries in a window: repeated blocks in a row
  int P = 2;
  while (P < n) P <<= 1;
  for (int x = threadIdx.x; x < P; x += 256) v[x] = x < n ? e[x] : 0x7FFFFFFF;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int x = threadIdx.x; x < P; x += 256) {
        const int y = x ^ jj;
        if (y > x) {
          const int32_t a = v[x], c = v[y];
          const bool up = (x & k) == 0;
          if ((a > c) == up) {
            v[x] = c;
            v[y] = a;
          }
        }
      }
      __syncthreads();
    }
  for (int x = threadIdx.x; x < n; x += 256) e[x] = v[x];
}

template <int G>
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_kernel(BwdParams bp) {
  constexpr int QW = 32 / G;                // queries per sub-tile
  const Params& p = bp.e;
  __shared__ u32x4 ktile[kBlock * 16];      // K_j [key][16 chunks], swizzled
  __shared__ u32x4 vtile[kBlock * 16];      // V_j, same
  __shared__ u32x4 sq[32 * 16];             // Q rows of the sub-tile [row][chunk], swizzled
  __shared__ u32x4 sdo[32 * 16];            // dO rows, same
  __shared__ __align__(16) uint16_t sds[32 * kSStride];  // dS [row][key] bf16
  __shared__ __align__(16) float2 s_stat[32];  // (LSE log2, delta) of each row
  __shared__ int s_t[QW];                   // position of each query (-1: no edge)
  __shared__ int s_slot[QW];

  const int BG = p.B * p.H_kv;
  const long nblk = (long)BG * p.n_blk;
  // Work item: segment sg of the sub-tiles of block x = (j, bg), early
  // (busier) blocks first; a block with one segment is walked whole.  When
  // no block can be split, work item x is block x.
  int x = blockIdx.x, sg = 0, nseg = 1, n_tiles = 0x7FFFFFFF;
  if (bp.seg_on) {  // uniform
    if ((long)blockIdx.x >= bp.blk_item[nblk]) return;  // past the last work item
    const int2 item = bp.items[blockIdx.x];
    x = item.x;
    sg = item.y;
    nseg = bp.blk_item[x + 1] - bp.blk_item[x];
    n_tiles = bp.blk_t[x];
  }
  const int j = x / BG;
  const int bg = x - j * BG;
  const int b = bg / p.H_kv;
  const int g = bg - b * p.H_kv;
  const int seg_len = nseg == 1 ? n_tiles : (n_tiles + nseg - 1) / nseg;
  const int first_tile = sg * seg_len;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int n = lane & 31;
  const int off = p.S_k - p.S_q;
  const float c = p.scale_log2;


  f32x16 dk_acc[4], dv_acc[4];  // [key row][d tile]: this wave's 32 keys x 128 dims
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) dk_acc[dt] = dv_acc[dt] = zero16();

  const int key0 = 32 * wave;          // this wave's keys within the block
  const int key_abs = j * kBlock + key0 + n;
  // Sub-tiles in a fixed order: windows ascending, QW edges at a time (the
  // fetch pipeline below keeps two sub-tiles of rows in flight); rows of
  // queries past a bucket's end repeat its last edge with dO = 0 and
  // LSE = +inf, so they add nothing.
  struct Cursor {
    int w, base, cnt;
    const int32_t* ed;
    int left;  // sub-tiles of the segment still to come
  };
  // Advances to the next sub-tile; past the segment's last one it returns
  // false and leaves the cursor on that sub-tile, so its addresses stay valid.
  auto next = [&](Cursor& cu) {  // uniform
    if (cu.left <= 0) return false;
    Cursor t = cu;
    --t.left;
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
  // rows (one query unless G = 1), e2 for the statistics of row tid % 32.  A
  // row past a bucket's end repeats the bucket's last edge and is flagged
  // invalid; the flags come from the cursor alone, so nothing waits for the
  // ids before they are used.
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
  // The rows of one sub-tile as fetched by this thread (two sets alternate).
  struct Fetched {
    u32x4 qa[2], da[2];
    float2 st;
    Ids id;
  };
  auto fetch = [&](const Ids& d, Fetched& f) {
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int r = 2 * pr + y, hh = r % G;
      const int i = slot_query(p, bg, d.e[y % NI]);
      const size_t rowoff = (((size_t)b * p.S_q + i) * p.H_q + g * G + hh) * kD + 8 * cc;
      f.qa[y] = *reinterpret_cast<const u32x4*>(p.q + rowoff);
      f.da[y] = *reinterpret_cast<const u32x4*>(bp.dout + rowoff);
    }
    if (tid < 32) {  // (loading it in every thread costs registers)
      const int hh = tid % G;
      const int i = slot_query(p, bg, d.e2);
      f.st = bp.stat[((size_t)bg * p.S_q + i) * G + hh];
    }
    f.id = d;
  };
  // The dq records of one sub-tile (rows without an edge, and the dummy
  // stores of the prologue, write the sink): this wave's quarter of the head
  // dims, a piece per lane, as 12-bit codes scaled by the quarter's largest
  // magnitude.  Cached stores: non-temporal ones measured 5 % slower here.
  auto store_records = [&](const f32x16& qacc, bool dummy) {
    const int q = n / G, hh = n - (n / G) * G;
    const int sl = dummy ? -1 : s_slot[q];
    const long slot = sl >= 0 ? sl : bp.sink;
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) m = max3abs(qacc[r], qacc[r + 1], m);
    m = halves_max(m);
    const float s = 2047.f * rec_inv(m);
    store_piece<G, false>(bp.dq_rec + slot * (kRecBytes<G> / 16), (wave * G + hh) * 2 + h, qacc, s);
    bp.dq_sc[(slot * 4 + wave) * G + hh] = m * bp.scale * (1.f / 2047.f);  // both halves store the same value
  };
  // Pipeline, in issue order: sub-tile n stages rows fetched during n - 2,
  // requests the ids of n + 3 and then the rows of n + 2, computes, and
  // stores its dq records.  Every request is unconditional (past the end
  // the cursor repeats the last sub-tile), so the memory counter's order is
  // the same on every iteration and the waits stay exact: the rows of n + 1
  // and the records of n - 1 stay in flight while n stages.  The prologue
  // issues the same sequence, with two dummy record stores.
  Cursor cur{-1, -QW, 0, nullptr, nseg == 1 ? n_tiles : max(0, min(seg_len, n_tiles - first_tile))};
  if (first_tile > 0) {  // uniform: start at the segment's first sub-tile
    int skip = first_tile;
    for (int w = 0; w < p.n_win; ++w) {
      const long bucket = ((long)bg * p.n_win + w) * p.n_blk + j;
      const int cnt = __builtin_amdgcn_readfirstlane(p.counts[bucket]);
      const int t = (cnt + QW - 1) / QW;
      if (skip < t) {
        cur.w = w;
        cur.base = (skip - 1) * QW;  // next() moves to sub-tile `skip` of this bucket
        cur.cnt = cnt;
        cur.ed = p.edges + __builtin_amdgcn_readfirstlane(p.offsets[bucket]);
        break;
      }
      skip -= t;
    }
  }
  // The block's tiles, loaded only when some edge selects the block (a
  // workgroup without edges just writes zero gradients).
  auto load_tiles = [&]() {  // K_j, V_j row-major into LDS (rows past S_k clamped: masked for every query)
    const size_t row_stride = (size_t)p.H_kv * kD;
    const uint16_t* kb = p.k + ((size_t)b * p.S_k * p.H_kv + g) * kD;
    const uint16_t* vb = p.v + ((size_t)b * p.S_k * p.H_kv + g) * kD;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int qd = it * kThreads + tid;
      const int row = qd >> 4, cc = qd & 15;
      const int s = min(j * kBlock + row, p.S_k - 1);
      ktile[row * 16 + (cc ^ (row & 15))] = *reinterpret_cast<const u32x4*>(kb + (size_t)s * row_stride + 8 * cc);
      vtile[row * 16 + (cc ^ (row & 15))] = *reinterpret_cast<const u32x4*>(vb + (size_t)s * row_stride + 8 * cc);
    }
  };
  bool h0 = next(cur), h1 = false, h2 = false;
  const bool any = h0;   // some edge of this chunk selects the block
  if (h0) load_tiles();  // uniform
  Fetched fx, fy;
  Ids ide, ido;  // ids of the even and of the odd sub-tiles
  if (h0) {
    Ids i0;
    load_ids(cur, i0);
    h1 = next(cur);
    load_ids(cur, ido);
    fetch(i0, fx);
    store_records(zero16(), true);
    h2 = h1 && next(cur);
    load_ids(cur, ide);
    fetch(ido, fy);
    store_records(zero16(), true);
  }

  // Operands that are the same for every sub-tile stay in registers once
  // loaded instead of being read from LDS each sub-tile: the K_j and V_j rows
  // of the wave's keys (S, dP) and K^T of the wave's head dims (dq), 96
  // registers (one wave per SIMD leaves room).
  u32x4 kf[8], vf[8], ktf[8];
  auto load_frags = [&]() {
    const int krow = key0 + n;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kf[ks] = ktile[krow * 16 + ((2 * ks + h) ^ (krow & 15))];
      vf[ks] = vtile[krow * 16 + ((2 * ks + h) ^ (krow & 15))];
    }
    const int lr = lane & 15;
    const int c0 = 32 * wave + 16 * (n >> 4) + 4 * (lr & 3);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int k0 = 16 * ks + 8 * h + (lr >> 2), k1 = k0 + 4;
      const uint2 a0 = lds_read_tr16(reinterpret_cast<const char*>(ktile) + lds_tile_off(k0, c0, k0 & 15));
      const uint2 a1 = lds_read_tr16(reinterpret_cast<const char*>(ktile) + lds_tile_off(k1, c0, k1 & 15));
      ktf[ks] = u32x4{a0.x, a0.y, a1.x, a1.y};
    }
  };

  auto step = [&](Fetched& f, const Ids& use, Ids& load) {
    __syncthreads();  // the previous sub-tile's LDS reads are done
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int r = 2 * pr + y;
      const u32x4 z = {0u, 0u, 0u, 0u};
      sq[r * 16 + (cc ^ rsw(r))] = f.qa[y];
      sdo[r * 16 + (cc ^ rsw(r))] = (f.id.valid >> (y % NI)) & 1 ? f.da[y] : z;
    }
    if (tid < 32) {
      const int x = f.id.e2;
      const bool valid = (f.id.valid >> 2) & 1;
      s_stat[tid] = valid ? f.st : make_float2(__builtin_inff(), 0.f);
      if (tid % G == 0) {
        s_t[tid / G] = valid ? slot_query(p, bg, x) + off : -1;
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

      // S = Q K^T and dP = dO V^T for this wave's 32 keys: rows on registers,
      // keys on lanes (D[row][key]).
      f32x16 sacc = zero16(), pacc = zero16();
      const int krow = key0 + n;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int ch = 2 * ks + h;
        sacc = mfma32x32x16(sq[n * 16 + (ch ^ rsw(n))], kf[ks], sacc);
        pacc = mfma32x32x16(sdo[n * 16 + (ch ^ rsw(n))], vf[ks], pacc);
      }
      // P and dS; rows r -> 8 (r / 4) + 4 h + r % 4.
      float lse4[16], del4[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 a = *reinterpret_cast<const float4*>(&s_stat[8 * r4 + 4 * h]);
        const float4 d = *reinterpret_cast<const float4*>(&s_stat[8 * r4 + 4 * h + 2]);
        lse4[4 * r4] = a.x; lse4[4 * r4 + 1] = a.z; lse4[4 * r4 + 2] = d.x; lse4[4 * r4 + 3] = d.z;
        del4[4 * r4] = a.y; del4[4 * r4 + 1] = a.w; del4[4 * r4 + 2] = d.y; del4[4 * r4 + 3] = d.w;
      }
      float pv[16], dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mfma32_row(r, lane);
        const bool vis = key_abs <= s_t[row / G];
        const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, -lse4[r]));
        pv[r] = vis ? e2 : 0.f;
        dsv[r] = pv[r] * (pacc[r] - del4[r]);
      }
      // dV += P^T dO and dK += dS^T Q: A = this lane's P / dS (row = key,
      // k = the 8 rows of registers 8 kk .. 8 kk + 7), B = dO^T / Q^T rows of
      // the same 8 rows: 8 (e / 4) + 4 h + e % 4 + 16 kk.
      u32x4 ds_bf[2];  // the bf16 dS of this lane's rows, also staged for dq below
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        u32x4 pa, sa;
        pa[0] = pack_bf16x2(pv[8 * kk + 0], pv[8 * kk + 1]);
        pa[1] = pack_bf16x2(pv[8 * kk + 2], pv[8 * kk + 3]);
        pa[2] = pack_bf16x2(pv[8 * kk + 4], pv[8 * kk + 5]);
        pa[3] = pack_bf16x2(pv[8 * kk + 6], pv[8 * kk + 7]);
        sa[0] = pack_bf16x2(dsv[8 * kk + 0], dsv[8 * kk + 1]);
        sa[1] = pack_bf16x2(dsv[8 * kk + 2], dsv[8 * kk + 3]);
        sa[2] = pack_bf16x2(dsv[8 * kk + 4], dsv[8 * kk + 5]);
        sa[3] = pack_bf16x2(dsv[8 * kk + 6], dsv[8 * kk + 7]);
        ds_bf[kk] = sa;
        // Lane (d = 32 dt + n, h) needs rows r0 .. r0 + 3 and r0 + 8 .. r0 + 11
        // of column d: two transposing reads of the row-major staged tiles.
        const int r0 = 16 * kk + 4 * h;
        const int lr = lane & 15;
        const int ra = r0 + (lr >> 2), rb = r0 + 8 + (lr >> 2);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int c0 = 32 * dt + 16 * (n >> 4) + 4 * (lr & 3);
          const uint2 o0 = lds_read_tr16(reinterpret_cast<const char*>(sdo) + lds_tile_off(ra, c0, rsw(ra)));
          const uint2 o1 = lds_read_tr16(reinterpret_cast<const char*>(sdo) + lds_tile_off(rb, c0, rsw(rb)));
          const uint2 q0 = lds_read_tr16(reinterpret_cast<const char*>(sq) + lds_tile_off(ra, c0, rsw(ra)));
          const uint2 q1 = lds_read_tr16(reinterpret_cast<const char*>(sq) + lds_tile_off(rb, c0, rsw(rb)));
          const u32x4 ob = {o0.x, o0.y, o1.x, o1.y};
          const u32x4 qb = {q0.x, q0.y, q1.x, q1.y};
          dv_acc[dt] = mfma32x32x16(pa, ob, dv_acc[dt]);
          dk_acc[dt] = mfma32x32x16(sa, qb, dk_acc[dt]);
        }
      }
      // dS to LDS as [row][key] for dq: the halves of the dK operand above.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t w2 = ds_bf[r >> 3][(r & 7) >> 1];
        sds[mfma32_row(r, lane) * kSStride + key0 + n] = (uint16_t)((r & 1) ? (w2 >> 16) : (w2 & 0xFFFFu));
      }
      __syncthreads();

      // dq for head dims 32 wave .. 32 wave + 31 over all 128 keys, as
      // dq^T[d][row] = sum_key K^T[d][key] dS[row][key]: rows on lanes, each
      // lane holding 16 dims of its row (4 runs of 4 consecutive dims).
      f32x16 qacc = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        // K^T operand (keys 16 ks + 8 h .. + 7 of column 32 wave + n): ktf.
        const u32x4 sb = *reinterpret_cast<const u32x4*>(&sds[n * kSStride + 16 * ks + 8 * h]);
        qacc = mfma32x32x16(ktf[ks], sb, qacc);
      }
      store_records(qacc, false);
  };
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

  // A segment of a split block leaves its fp32 part, summed in segment order
  // with the other segments' by seg_reduce_kernel.
  if (nseg > 1) {  // uniform
    float* pk = bp.part + (size_t)(bp.blk_part[x] + sg) * 2 * kBlock * kD;
    float* pv = pk + kBlock * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = (key0 + mfma32_row(r, lane)) * kD + 32 * dt + n;
        pk[o] = dk_acc[dt][r] * bp.scale;
        pv[o] = dv_acc[dt][r];
      }
    }
    return;
  }

  // A block that no edge of the chunk selects adds nothing: in a middle chunk
  // the running sums stay as they are, and a one-chunk problem writes zero
  // rows 16 bytes at a time (on a decode-shaped problem nearly every block is
  // such a block).  First and last chunks of several take the path below.
  if (!any) {  // uniform
    if (!bp.first && !bp.last) return;
    if (bp.first && bp.last) {
      const int keys = min(kBlock, p.S_k - j * kBlock);
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int x = tid; x < keys * 16; x += kThreads) {  // 16 pieces of 16 bytes per row
        const size_t o = (((size_t)b * p.S_k + j * kBlock + (x >> 4)) * p.H_kv + g) * kD + 8 * (x & 15);
        *reinterpret_cast<u32x4*>(bp.dk + o) = z;
        *reinterpret_cast<u32x4*>(bp.dv + o) = z;
      }
      return;
    }
  }

  // dK (times the softmax scale) and dV of this wave's keys.
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int d = 32 * dt + n;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j * kBlock + key0 + mfma32_row(r, lane);
      if (key >= p.S_k) continue;
      const size_t o = (((size_t)b * p.S_k + key) * p.H_kv + g) * kD + d;
      float kv = dk_acc[dt][r] * bp.scale, vv = dv_acc[dt][r];
      if (!bp.first) {
        kv += bp.dk_acc[o];
        vv += bp.dv_acc[o];
      }
      if (bp.last) {
        bp.dk[o] = (uint16_t)(pack_bf16x2(kv, 0.f) & 0xFFFFu);
        bp.dv[o] = (uint16_t)(pack_bf16x2(vv, 0.f) & 0xFFFFu);
      } else {
        bp.dk_acc[o] = kv;
        bp.dv_acc[o] = vv;
      }
    }
  }
}

// dq of each (query, group): the sum of its edges' records.  One wave per
// row; lane l takes piece l (+ 64 u) of every record, i.e. (quarter, head,
// half) = ((f / 2) / G, (f / 2) % G, f % 2), and adds sc (code - 2048) of its
// 16 values, the offset taken off once.  All entries of the row are
// requested together with unconditional loads (an entry that does not count
// reads its own slot, inside the workspace, and is skipped), 16 at a time.
// dq is written once and not read back here, so its stores are non-temporal
// (32K: 10.49 -> 10.41 ms for the main backward; two rows per wave, as in the
// forward merge, measured no faster).
template <int G>
__global__ __launch_bounds__(256) void dq_merge_kernel(BwdParams bp) {
  constexpr int NP = 8 * G;          // pieces per record
  constexpr int F = (NP + 63) / 64;  // pieces per lane
  constexpr int kBatch = F >= 4 ? 4 : (F >= 2 ? 8 : 16);
  const Params& p = bp.e;
  const int lane = threadIdx.x & 63;
  const long r = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= (long)p.B * p.H_kv * p.Qc) return;
  const int il = (int)(r % p.Qc);
  const int bg = (int)(r / p.Qc);
  const int i = p.q0 + il;
  if (i >= p.S_q) return;
  const int b = bg / p.H_kv, g = bg - (bg / p.H_kv) * p.H_kv;
  const int32_t* sel = p.idx + ((long)bg * p.S_q + i) * p.topk;
  const int local = (i + p.S_k - p.S_q) / kBlock;
  const long slot0 = ((long)bg * p.Qc + il) * p.topk;
  const int je = lane < p.topk ? sel[lane] : -1;
  const unsigned long long valid = __builtin_amdgcn_ballot_w64(je >= 0 && je <= local);
  float acc[F][16], W[F];
#pragma unroll
  for (int u = 0; u < F; ++u) {
    W[u] = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[u][c] = 0.f;
  }
  for (int e0 = 0; e0 < p.topk; e0 += kBatch) {
    u32x4 xa[kBatch][F];
    uint64_t xb[kBatch][F];
    float sc[kBatch][F];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const long slot = slot0 + min(e0 + k, p.topk - 1);
      const u32x4* rec = bp.dq_rec + slot * (kRecBytes<G> / 16);
#pragma unroll
      for (int u = 0; u < F; ++u) {
        const int f = min(lane + 64 * u, NP - 1);
        load_piece<G>(rec, f, xa[k][u], xb[k][u]);
        sc[k][u] = bp.dq_sc[slot * 4 * G + (f >> 1)];  // (quarter, head) = f / 2
      }
    }
    const unsigned bits = (unsigned)(valid >> e0) & ((1u << kBatch) - 1u);  // e0 < topk <= 64
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (!((bits >> k) & 1u)) continue;  // wave-uniform
#pragma unroll
      for (int u = 0; u < F; ++u) {
        add_piece(xa[k][u], xb[k][u], sc[k][u], acc[u]);
        W[u] += sc[k][u];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < F; ++u) {
    const int f = lane + 64 * u;
    if (f >= NP) continue;  // NP is even: lanes f and f ^ 1 skip together
    const int quarter = (f >> 1) / G, hh = (f >> 1) % G, h = f & 1;
    float v[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) v[c] = acc[u][c] - 2048.f * W[u];
    store_run32<true>(bp.dq + (((size_t)b * p.S_q + i) * p.H_q + g * G + hh) * kD + 32 * quarter, h, v);
  }
}

// Sub-tiles of each (group, block) in the chunk, and its number of work
// items: max(1, ceil(T / seg)), kept in blk_item until the scan.
__global__ __launch_bounds__(256) void seg_count_kernel(BwdParams bp, int QW) {
  const Params& p = bp.e;
  const int BG = p.B * p.H_kv;
  const long x = (long)blockIdx.x * 256 + threadIdx.x;
  if (x >= (long)BG * p.n_blk) return;
  const int j = (int)(x / BG), bg = (int)(x % BG);
  int T = 0;
  for (int w = 0; w < p.n_win; ++w) T += (p.counts[((long)bg * p.n_win + w) * p.n_blk + j] + QW - 1) / QW;
  bp.blk_t[x] = T;
  bp.blk_item[x] = T > bp.seg ? (T + bp.seg - 1) / bp.seg : 1;
}

// One workgroup: exclusive scans of the work items and of the partial slots
// (split blocks only) in x order, the totals at blk_item[nblk], and the
// work-item list: the segments of split blocks first (the longest items, so
// none of them starts last), then the other blocks in x order.  Each thread
// takes a contiguous run of x.
__global__ __launch_bounds__(256) void seg_scan_kernel(BwdParams bp, long nblk) {
  __shared__ int32_t sa[256], sb[256];
  const int tid = threadIdx.x;
  const long per = (nblk + 255) / 256;
  const long x0 = min(nblk, tid * per), x1 = min(nblk, x0 + per);
  int na = 0, nb = 0;
  for (long x = x0; x < x1; x += 8) {  // eight independent loads in flight
    int k[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) k[u] = x + u < x1 ? bp.blk_item[x + u] : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      na += k[u];
      nb += k[u] > 1 ? k[u] : 0;
    }
  }
  sa[tid] = na;
  sb[tid] = nb;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {  // Hillis-Steele inclusive scan
    const int a = tid >= d ? sa[tid - d] : 0;
    const int c = tid >= d ? sb[tid - d] : 0;
    __syncthreads();
    sa[tid] += a;
    sb[tid] += c;
    __syncthreads();
  }
  int oa = sa[tid] - na, ob = sb[tid] - nb;
  const int n_split = sb[255];  // work items of split blocks
  for (long x = x0; x < x1; ++x) {
    const int k = bp.blk_item[x];
    bp.blk_item[x] = oa;
    bp.blk_part[x] = ob;
    if (k > 1) {
      for (int u = 0; u < k; ++u) bp.items[ob + u] = make_int2((int)x, u);
    } else {
      bp.items[n_split + oa - ob] = make_int2((int)x, 0);  // oa - ob: unsplit blocks before x
    }
    oa += k;
    ob += k > 1 ? k : 0;
  }
  if (tid == 255) bp.blk_item[nblk] = sa[255];
}

// dK, dV of each split (group, block): its segments' fp32 parts added in
// segment order, then what the unsplit path does (the earlier chunks' sums
// added, bf16 out after the last chunk, fp32 sums kept before it).
__global__ __launch_bounds__(256) void seg_reduce_kernel(BwdParams bp) {
  const Params& p = bp.e;
  const int BG = p.B * p.H_kv;
  const long x = blockIdx.x;
  const int nseg = bp.blk_item[x + 1] - bp.blk_item[x];
  if (nseg <= 1) return;  // uniform
  const int j = (int)(x / BG), bg = (int)(x % BG);
  const int b = bg / p.H_kv, g = bg - (bg / p.H_kv) * p.H_kv;
  const float* base = bp.part + (size_t)bp.blk_part[x] * 2 * kBlock * kD;
  constexpr int kSlot = 2 * kBlock * kD;
  for (int c = threadIdx.x; c < kBlock * kD / 4; c += 256) {  // 4 values of one key row
    const int key = j * kBlock + c / (kD / 4);
    if (key >= p.S_k) break;  // rows past S_k come last
    float4 sk = *reinterpret_cast<const float4*>(base + 4 * c);
    float4 sv = *reinterpret_cast<const float4*>(base + kBlock * kD + 4 * c);
    for (int u = 1; u < nseg; ++u) {
      const float4 ak = *reinterpret_cast<const float4*>(base + (size_t)u * kSlot + 4 * c);
      const float4 av = *reinterpret_cast<const float4*>(base + (size_t)u * kSlot + kBlock * kD + 4 * c);
      sk.x += ak.x; sk.y += ak.y; sk.z += ak.z; sk.w += ak.w;
      sv.x += av.x; sv.y += av.y; sv.z += av.z; sv.w += av.w;
    }
    const size_t o = (((size_t)b * p.S_k + key) * p.H_kv + g) * kD + 4 * (c % (kD / 4));
    if (!bp.first) {
      const float4 ak = *reinterpret_cast<const float4*>(bp.dk_acc + o);
      const float4 av = *reinterpret_cast<const float4*>(bp.dv_acc + o);
      sk.x += ak.x; sk.y += ak.y; sk.z += ak.z; sk.w += ak.w;
      sv.x += av.x; sv.y += av.y; sv.z += av.z; sv.w += av.w;
    }
    if (bp.last) {
      *reinterpret_cast<uint2*>(bp.dk + o) = make_uint2(pack_bf16x2(sk.x, sk.y), pack_bf16x2(sk.z, sk.w));
      *reinterpret_cast<uint2*>(bp.dv + o) = make_uint2(pack_bf16x2(sv.x, sv.y), pack_bf16x2(sv.z, sv.w));
    } else {
      *reinterpret_cast<float4*>(bp.dk_acc + o) = sk;
      *reinterpret_cast<float4*>(bp.dv_acc + o) = sv;
    }
  }
}

}  // namespace

namespace edges {
void launch_bucket_sort(const Layout& L, const Params& p, hipStream_t st) {
  hipLaunchKernelGGL((bucket_sort_kernel<kSortSmall, false>), dim3((unsigned)L.NB), dim3(256), 0, st, p);
  hipLaunchKernelGGL((bucket_sort_kernel<kMaxWindow, true>), dim3((unsigned)L.NB), dim3(256), 0, st, p);
}
}  // namespace edges

namespace {

// The main backward of one chunk, after the chunk's bucket build and sort.
template <int G>
void launch_main_chunk(const AttnShape& s, const Layout& L, const BwdParams& bp, long n_items, hipStream_t st) {
  const long nblk = (long)s.batch * s.H_kv * s.n_blk;
  if (bp.seg_on) {
    hipLaunchKernelGGL(seg_count_kernel, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, st, bp, 32 / G);
    hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(256), 0, st, bp, nblk);
    hipLaunchKernelGGL((attn_bwd_kernel<G>), dim3((unsigned)n_items), dim3(kThreads), 0, st, bp);
    hipLaunchKernelGGL(seg_reduce_kernel, dim3((unsigned)nblk), dim3(256), 0, st, bp);
  } else {
    hipLaunchKernelGGL((attn_bwd_kernel<G>), dim3((unsigned)nblk), dim3(kThreads), 0, st, bp);
  }
  const long mrows = (long)s.batch * s.H_kv * L.Qc;
  hipLaunchKernelGGL(dq_merge_kernel<G>, dim3((unsigned)((mrows + 3) / 4)), dim3(256), 0, st, bp);
}

template <int G>
hipError_t launch_bwd_g(const AttnShape& s, const BwdLayout& BL, BwdParams bp, hipStream_t st) {
  const Layout& L = BL.L;
  const long rows = (long)s.batch * s.S_q * s.H_q;
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, st, bp);
  for (int q0 = 0, ci = 0; q0 < s.S_q; q0 += L.Qc, ++ci) {
    bp.e.q0 = q0;
    bp.first = ci == 0;
    bp.last = q0 + L.Qc >= s.S_q;
    launch_build(s, L, bp.e, st);
    launch_bucket_sort(L, bp.e, st);
    launch_main_chunk<G>(s, L, bp, BL.n_items, st);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

// Both backward passes on the same query chunks: one bucket build and sort
// per chunk serves the main-branch kernels and the loss backward's.
template <int G>
hipError_t launch_both_g(const AttnShape& s, const FusedBwdLayout& FL, BwdParams bp, KlBwdParams kp,
                         hipStream_t st) {
  const Layout& L = FL.B.L;
  const long rows = (long)s.batch * s.S_q * s.H_q;
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, st, bp);
  for (int q0 = 0, ci = 0; q0 < s.S_q; q0 += L.Qc, ++ci) {
    bp.e.q0 = q0;
    bp.first = ci == 0;
    bp.last = q0 + L.Qc >= s.S_q;
    kp.first = ci == 0;
    launch_build(s, L, bp.e, st);
    launch_bucket_sort(L, bp.e, st);
    launch_main_chunk<G>(s, L, bp, FL.B.n_items, st);
    kp.e = bp.e;
    const hipError_t err = launch_kl_chunk(s, L, kp, st);
    if (err != hipSuccess) return err;
  }
  return launch_kl_dk_reduce(kp, kp.D_idx, (long)s.batch * s.n_blk, st);
}

}  // namespace

// The work-item arrays of the main backward in a workspace laid out by BL.
static void set_segments(BwdParams& bp, const BwdLayout& BL, char* base) {
  bp.seg = BL.seg;
  bp.seg_on = BL.seg_on;
  bp.blk_t = reinterpret_cast<int32_t*>(base + BL.blk_t);
  bp.blk_item = reinterpret_cast<int32_t*>(base + BL.blk_item);
  bp.blk_part = reinterpret_cast<int32_t*>(base + BL.blk_part);
  bp.items = reinterpret_cast<int2*>(base + BL.items);
  bp.part = reinterpret_cast<float*>(base + BL.part);
}

hipError_t launch_backward(const AttnShape& s, int D_idx, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint16_t* q_idx, const uint16_t* k_idx,
                           const int32_t* idx, const uint16_t* out, const float* lse,
                           const float* lse_idx, const uint16_t* dout, float coef, uint16_t* dq,
                           uint16_t* dk, uint16_t* dv, uint16_t* dq_idx, uint16_t* dk_idx, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  const int qc = fused_bwd_chunk(s, D_idx, ws_bytes);
  if (qc <= 0) return hipErrorInvalidValue;
  const FusedBwdLayout FL = make_fused_bwd_layout(s, D_idx, qc);
  const BwdLayout& BL = FL.B;
  char* base = static_cast<char*>(ws);
  BwdParams bp{};
  bp.e = base_params(s, BL.L, base, idx);
  bp.e.q = q; bp.e.k = k; bp.e.v = v; bp.e.q_idx = q_idx; bp.e.k_idx = k_idx;
  bp.dout = dout; bp.out = out; bp.lse = lse;
  bp.stat = reinterpret_cast<float2*>(base + BL.stat);
  bp.sink = BL.L.E;
  bp.dq_rec = reinterpret_cast<u32x4*>(base + BL.dq_rec);
  bp.dq_sc = reinterpret_cast<float*>(base + BL.dq_sc);
  bp.dk_acc = reinterpret_cast<float*>(base + BL.dk_acc);
  bp.dv_acc = reinterpret_cast<float*>(base + BL.dv_acc);
  set_segments(bp, BL, base);
  bp.dq = dq; bp.dk = dk; bp.dv = dv;
  bp.scale = s.scale;
  float* lse_t = reinterpret_cast<float*>(base + FL.lse_t);
  bp.e.lse_t = lse_t;
  launch_lse_group(s, lse, lse_t, stream);
  KlBwdParams kp{};
  kp.e = bp.e;
  kp.lse_idx = lse_idx; kp.coef = coef;
  kp.rec = reinterpret_cast<uint16_t*>(base + FL.rec);
  kp.rec_sc = reinterpret_cast<float*>(base + FL.rec_sc);
  kp.g_rec = reinterpret_cast<uint16_t*>(base + FL.g_rec);
  kp.sink = BL.L.E;
  kp.dk_part = reinterpret_cast<float*>(base + FL.dk_part);
  kp.dk_flag = reinterpret_cast<int32_t*>(base + FL.dk_flag);
  kp.dq_idx = dq_idx; kp.dk_idx = dk_idx; kp.D_idx = D_idx;
  switch (bp.e.G) {
    case 1: return launch_both_g<1>(s, FL, bp, kp, stream);
    case 2: return launch_both_g<2>(s, FL, bp, kp, stream);
    case 4: return launch_both_g<4>(s, FL, bp, kp, stream);
    case 8: return launch_both_g<8>(s, FL, bp, kp, stream);
    case 16: return launch_both_g<16>(s, FL, bp, kp, stream);
    case 32: return launch_both_g<32>(s, FL, bp, kp, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sparse_attn_bwd(const AttnShape& s, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const int32_t* idx, const uint16_t* out,
                                  const float* lse, const uint16_t* dout, uint16_t* dq,
                                  uint16_t* dk, uint16_t* dv, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  const int qc = bwd_chunk(s, ws_bytes);
  if (qc <= 0) return hipErrorInvalidValue;
  const BwdLayout BL = make_bwd_layout(s, qc);
  char* base = static_cast<char*>(ws);
  BwdParams bp{};
  bp.e = base_params(s, BL.L, base, idx);
  bp.e.q = q; bp.e.k = k; bp.e.v = v;
  bp.dout = dout; bp.out = out; bp.lse = lse;
  bp.stat = reinterpret_cast<float2*>(base + BL.stat);
  bp.sink = BL.L.E;
  bp.dq_rec = reinterpret_cast<u32x4*>(base + BL.dq_rec);
  bp.dq_sc = reinterpret_cast<float*>(base + BL.dq_sc);
  bp.dk_acc = reinterpret_cast<float*>(base + BL.dk_acc);
  bp.dv_acc = reinterpret_cast<float*>(base + BL.dv_acc);
  set_segments(bp, BL, base);
  bp.dq = dq; bp.dk = dk; bp.dv = dv;
  bp.scale = s.scale;
  switch (bp.e.G) {
    case 1: return launch_bwd_g<1>(s, BL, bp, stream);
    case 2: return launch_bwd_g<2>(s, BL, bp, stream);
    case 4: return launch_bwd_g<4>(s, BL, bp, stream);
    case 8: return launch_bwd_g<8>(s, BL, bp, stream);
    case 16: return launch_bwd_g<16>(s, BL, bp, stream);
    case 32: return launch_bwd_g<32>(s, BL, bp, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
