// Edge buckets: the work lists shared by the kernels that run KV-stationary
// over a selection (attention forward, alignment loss).
//
// An edge is (query i, group g, selected block j) of a query chunk; its slot
// is ((b * H_kv + g) * Qc + il) * topk + e for entry e of row (b, g, i).
// Buckets group edges by (b, g, query window w, block j), bucket index
// ((b * H_kv + g) * n_win + w) * n_blk + j; work items are (bucket, first
// edge) with at most QT edges each.  The build (sparse_attn.hip) counts edges
// per bucket, scans the counts and scatters the slots.
#pragma once

#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace msa {
namespace edges {

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  uint16_t* out;
  float* lse;
  int B, S_q, S_k, H_q, H_kv, G, n_blk, topk;
  int q0, Qc;            // this chunk's queries: [q0, q0 + Qc) clipped to S_q
  int NB;                // buckets = B * H_kv * n_win * n_blk
  int W, n_win;          // queries per window (a multiple of kBuildQueries unless
                         // it is the whole chunk), windows per chunk
  int QT;                // edges per work item
  int dense_q;           // forward only: queries below this take no edges (dense tiles); else 0
  uint32_t topk_m;       // slot / topk == (slot * topk_m) >> topk_s (set_topk_divisor)
  int topk_s;
  float scale_log2;
  int32_t* counts;
  int32_t* cursor;
  int32_t* offsets;      // NB + 1
  int32_t* tile_off;     // NB + 1
  int32_t* blk_sums;     // 2 * n_scan_wg
  int32_t* edges;        // slot ids grouped by bucket
  int2* work;            // (bucket, first edge in bucket)
  f32x2* part_stat;      // [slot][G]: log2-sum-exp of the block's visible logits, and
                         // the scale of the row's codes (value = (code - 2048) scale)
  u32x4* part_o;         // [slot][kRecBytes(G)]: O_e / l_e as 12-bit codes (sparse_attn.hip)
  // Alignment loss (kl_* kernels below).
  const uint16_t* q_idx;
  const uint16_t* k_idx;
  const float* lse_in;   // [B][H_q][S_q] natural-log LSE of the main branch
  const float* lse_t;    // [B][H_kv][S_q][G]: the same in log2 units, grouped per query
  float* kl_rec;         // [slot][8]: sum P, sum P ln P, sum P (z - m), sum e^(z - m), m
  float* kl_rows;        // [B][H_kv][S_q] or null
  float* kl_lse;         // [B][H_kv][S_q]: log-sum-exp of the index scores over T, or null
  float* kl_wsum;        // per merge workgroup: sum of its rows' terms
  float* loss;           // or null
};

// Slot of edge (b, g, il, e) inside the chunk.
__device__ __forceinline__ long slot_of(const Params& p, int bg, int il, int e) {
  return ((long)bg * p.Qc + il) * p.topk + e;
}

// Division of a slot by topk as a multiply and a shift (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// with l = ceil(log2 topk) and m = ceil(2^(31 + l) / topk) < 2^32,
// n / topk == (n * m) >> (31 + l) for every 0 <= n < 2^31.  Slots are int32.
inline void set_topk_divisor(Params& p) {
  int l = 0;
  while ((1 << l) < p.topk) ++l;
  const uint64_t num = uint64_t(1) << (31 + l);
  p.topk_m = (uint32_t)((num + (uint64_t)p.topk - 1) / (uint64_t)p.topk);
  p.topk_s = 31 + l;
}
__device__ __forceinline__ int slot_row(const Params& p, int slot) {
  return (int)(((uint64_t)(uint32_t)slot * p.topk_m) >> p.topk_s);
}
// Query of a slot of group row bg: slot / topk = bg * Qc + (query - q0).
__device__ __forceinline__ int slot_query(const Params& p, int bg, int slot) {
  return p.q0 + slot_row(p, slot) - bg * p.Qc;
}

// Records of 12-bit codes (q12_code in device_common.h).  A piece is the 16
// values one lane holds of a 32 x 32 MFMA output tile, its register r at
// position 8 (r / 4) + 4 h + r % 4 of the tile's 32-row run (h = lane / 32);
// it takes 24 bytes: codes 0..7 and 8..15 packed by q12_pack8 into dwords
// d0 d1 d2 and d3 d4 d5, with d0..d3 in area A of the record (16 bytes per
// piece) and d4 d5 in area B (8 bytes per piece).  A record holds 8 G pieces.
template <int G> constexpr int kRecBytes = 8 * G * 24;
template <int G> constexpr int kRecA = 8 * G * 16;  // area B starts here

// Stores the 16 values x, scaled by s, as piece f of the record at rec
// (non-temporally when NT).
template <int G, bool NT>
__device__ __forceinline__ void store_piece(u32x4* rec, int f, const f32x16& x, float s) {
  uint32_t c0[8], c1[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    c0[v] = q12_code(x[v], s);
    c1[v] = q12_code(x[8 + v], s);
  }
  uint32_t a0, a1, a2, a3, b0, b1;
  q12_pack8(c0, a0, a1, a2);
  q12_pack8(c1, a3, b0, b1);
  const u32x4 a = {a0, a1, a2, a3};
  const uint64_t bb = (uint64_t)b0 | ((uint64_t)b1 << 32);
  uint64_t* rb = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(rec) + kRecA<G>) + f;
  if constexpr (NT) {
    __builtin_nontemporal_store(a, rec + f);
    __builtin_nontemporal_store(bb, rb);
  } else {
    rec[f] = a;
    *rb = bb;
  }
}

// Piece f of the record at rec (non-temporal loads: a record is read once).
template <int G>
__device__ __forceinline__ void load_piece(const u32x4* rec, int f, u32x4& a, uint64_t& b) {
  a = __builtin_nontemporal_load(rec + f);
  b = __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(reinterpret_cast<const char*>(rec) + kRecA<G>) + f);
}

// acc[v] += w * code v of a loaded piece (the offset 2048 is left in).
__device__ __forceinline__ void add_piece(const u32x4& a, uint64_t b, float w, float (&acc)[16]) {
  float y[8];
  q12_unpack8(a[0], a[1], a[2], y);
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = __builtin_fmaf(w, y[c], acc[c]);
  q12_unpack8(a[3], (uint32_t)b, (uint32_t)(b >> 32), y);
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[8 + c] = __builtin_fmaf(w, y[c], acc[8 + c]);
}

// Value of x held by lane l ^ 1 (DPP quad_perm [1, 0, 3, 2]).
__device__ __forceinline__ float swap_adjacent(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}

// Writes a piece's 16 values, as bf16, into the 32-value run `row` (the values
// at positions 8 (c / 4) + 4 h + c % 4).  Lanes l and l ^ 1, holding h = 0 and
// h = 1 of the same run, trade halves so that lane h writes positions
// 16 h .. 16 h + 15 as two 16-byte stores: whole 64-byte segments per lane
// pair.  Both lanes of a pair must be active.
template <bool NT>
__device__ __forceinline__ void store_run32(uint16_t* row, int h, const float (&v)[16]) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = swap_adjacent(h ? v[k] : v[8 + k]);
  float o[16];  // positions 16 h + 0..15
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[k] = h ? x[k] : v[k];
    o[4 + k] = h ? v[8 + k] : x[k];
    o[8 + k] = h ? x[4 + k] : v[4 + k];
    o[12 + k] = h ? v[12 + k] : x[4 + k];
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const u32x4 w4 = {pack_bf16x2(o[8 * q], o[8 * q + 1]), pack_bf16x2(o[8 * q + 2], o[8 * q + 3]),
                      pack_bf16x2(o[8 * q + 4], o[8 * q + 5]), pack_bf16x2(o[8 * q + 6], o[8 * q + 7])};
    u32x4* dst = reinterpret_cast<u32x4*>(row + 16 * h + 8 * q);
    if constexpr (NT) __builtin_nontemporal_store(w4, dst);
    else *dst = w4;
  }
}

// Gradient records of the backward kernels: per slot, quarters of 32 dims
// (x heads) of 32 values each, in the order a transposed MFMA tile holds
// them: position p = 16 h + r for MFMA register r of lane half h, which is
// dim 32 quarter + 8 (r / 4) + 4 h + r % 4.
__device__ __forceinline__ int rec_dim(int quarter, int pos) {
  const int h = pos >> 4, r = pos & 15;
  return 32 * quarter + 8 * (r >> 2) + 4 * h + (r & 3);
}

// Edge buckets of the chunk starting at p.q0: counts, scans, scatter.
void launch_build(const AttnShape& s, const Layout& L, const Params& p, hipStream_t st);
// Sorts each bucket's edge slots ascending, so that work that sums over a
// bucket's edges does so in a fixed order (attn_bwd.hip).
void launch_bucket_sort(const Layout& L, const Params& p, hipStream_t st);
// lse_t[b][g][i][hh] = log2(e) * lse[b][g G + hh][i]: the main branch's LSE of
// a query's G heads in 4 G contiguous bytes (kl_loss.hip).
void launch_lse_group(const AttnShape& s, const float* lse, float* lse_t, hipStream_t st);
// Params with the shape, the layout and the build arrays of `base` filled in.
Params base_params(const AttnShape& s, const Layout& L, char* base, const int32_t* idx);

}  // namespace edges
}  // namespace msa
