// Host-side planning of the KV-stationary entry points (declarations and
// the chunking rule in plan.h): workspace layouts, default and smallest
// workspaces, and the query chunk that fits a caller's workspace.
#include "plan.h"

namespace msa {
using namespace edges;

namespace edges {

// Bucket geometry and the build arrays for a chunk of Qc queries; returns the
// offset past them.
size_t layout_build(Layout& L, const AttnShape& s) {
  // Window: about QT edges per (window, block) bucket at the chunk's mean
  // number of visible blocks, between kMinWindow and kMaxWindow queries; the
  // whole chunk when that exceeds it.
  const long vis = std::max(1L, ((long)s.S_k - s.S_q + s.S_q / 2) / kBlock);
  long w = ((long)L.QT * vis / std::max(1, s.topk) + kBuildQueries - 1) / kBuildQueries * kBuildQueries;
  w = std::min<long>(std::max<long>(w, kMinWindow), kMaxWindow);
  L.W = w < L.Qc ? (int)w : L.Qc;
  L.n_win = (L.Qc + L.W - 1) / L.W;
  L.NB = (long)s.batch * s.H_kv * L.n_win * s.n_blk;
  L.E = (long)s.batch * s.H_kv * L.Qc * s.topk;
  L.T = (L.E + L.QT - 1) / L.QT + std::min(L.NB, L.E);
  L.n_scan_wg = (int)((L.NB + kScanPerWg - 1) / kScanPerWg);
  size_t o = 0;
  L.counts = o;   o = align256(o + L.NB * 4);
  L.cursor = o;   o = align256(o + L.NB * 4);
  L.offsets = o;  o = align256(o + (L.NB + 1) * 4);
  L.tile_off = o; o = align256(o + (L.NB + 1) * 4);
  L.blk_sums = o; o = align256(o + (size_t)L.n_scan_wg * 8);
  L.edges = o;    o = align256(o + L.E * 4);
  L.work = o;     o = align256(o + L.T * 8);
  return o;
}

}  // namespace edges

// ---------------------------------------------------------------- index branch
// One pass scores and selects when there are more rows than the decode kernel
// covers (32 per sequence) and the kept blocks fit the scan's registers.
bool index_select_fused(int S_q, int H_kv, int topk) {
  return S_q * H_kv > 32 && topk <= kSelectKeep + 1;
}

// ---------------------------------------------------------------- forward
// Bytes of per-edge records per query: G partial rows (12-bit output codes, log2-sum-exp,
// scale) and the edge slot, for each (b, g) row's topk entries.
static size_t fwd_per_query(const AttnShape& s) {
  const int G = s.H_q / s.H_kv;
  return (size_t)s.batch * s.H_kv * s.topk * ((size_t)G * (kD * 3 / 2 + 8) + 8 + 4);
}

// Workspace layout for query chunks of Qc queries.
Layout make_fwd_layout(const AttnShape& s, int Qc) {
  Layout L{};
  const int G = s.H_q / s.H_kv;
  L.QT = kSubTilesFwd * 4 * (32 / G);
  L.Qc = Qc;
  size_t o = layout_build(L, s);
  L.part_stat = o; o = align256(o + (size_t)L.E * G * 8);
  L.part_o = o;   o = align256(o + (size_t)L.E * G * kD * 3 / 2);  // 12-bit codes
  L.total = o;
  return L;
}

int fwd_chunk(const AttnShape& s, size_t ws_bytes) {
  return fit_chunk(default_chunk(s.S_q, fwd_per_query(s)), ws_bytes,
                   [&](int qc) { return make_fwd_layout(s, qc).total; });
}

size_t sparse_attn_workspace(const AttnShape& s) {
  return make_fwd_layout(s, default_chunk(s.S_q, fwd_per_query(s))).total;
}

size_t sparse_attn_workspace_min(const AttnShape& s) { return make_fwd_layout(s, 1).total; }

int sparse_attn_chunks(const AttnShape& s, size_t ws_bytes) {
  const int qc = fwd_chunk(s, ws_bytes);
  return qc > 0 ? (s.S_q + qc - 1) / qc : 0;
}

// ---------------------------------------------------------------- main backward
// Bytes of per-edge records per query: each (b, g) row's topk dq records
// (G x D fp16 values and 4 scales per head) and edge slots.
static size_t bwd_per_query(const AttnShape& s) {
  const int G = s.H_q / s.H_kv;
  return (size_t)s.batch * s.H_kv * s.topk * ((size_t)G * (kD * 3 / 2 + 16) + 4);
}

// Workspace layout for query chunks of Qc queries; with more than one chunk
// the key gradients are summed across chunks in fp32.
BwdLayout make_bwd_layout(const AttnShape& s, int Qc) {
  BwdLayout B{};
  Layout& L = B.L;
  const int G = s.H_q / s.H_kv;
  L.QT = kSubTiles * 4 * (32 / G);
  L.Qc = Qc;
  size_t o = layout_build(L, s);
  B.chunks = (s.S_q + L.Qc - 1) / L.Qc;
  B.stat = o;   o = align256(o + (size_t)s.batch * s.H_q * s.S_q * 8);
  // One record past the chunk's edges takes the stores of padding rows.
  B.dq_rec = o; o = align256(o + (size_t)(L.E + 1) * G * kD * 3 / 2);  // 12-bit codes
  B.dq_sc = o;  o = align256(o + (size_t)(L.E + 1) * G * 16);
  const size_t kv = (size_t)s.batch * s.S_k * s.H_kv * kD * 4;
  B.dk_acc = o; o = align256(o + (B.chunks > 1 ? kv : 0));
  B.dv_acc = o; o = align256(o + (B.chunks > 1 ? kv : 0));
  // Segments: `sub` bounds the chunk's sub-tiles (a bucket adds at most one
  // partial one).  A block of T sub-tiles takes max(1, ceil(T / seg)) work
  // items, at most 1 + T / seg, and when split (T > seg) at most 2 T / seg
  // partial slots.
  const int QW = 32 / G;
  const long nblk = (long)s.batch * s.H_kv * s.n_blk;
  const long sub = (L.E + QW - 1) / QW + std::min(L.NB, L.E);
  B.seg = (int)std::max(kSegMin, (L.E / QW + kSegSpread - 1) / kSegSpread);
  // A block holds at most one edge per query of the chunk (selections are
  // distinct), so at most Qc / QW + n_win sub-tiles.
  B.seg_on = (long)L.Qc / QW + L.n_win > B.seg;
  B.n_items = nblk + sub / B.seg + 1;
  B.n_part = 2 * sub / B.seg + 1;
  B.blk_t = o;    o = align256(o + (size_t)nblk * 4);
  B.blk_item = o; o = align256(o + (size_t)(nblk + 1) * 4);
  B.blk_part = o; o = align256(o + (size_t)nblk * 4);
  B.items = o;    o = align256(o + (size_t)B.n_items * 8);
  B.part = o;     o = align256(o + (size_t)B.n_part * 2 * kBlock * kD * 4);
  B.total = o;
  L.total = o;
  return B;
}

int bwd_chunk(const AttnShape& s, size_t ws_bytes) {
  return fit_chunk(default_chunk(s.S_q, bwd_per_query(s)), ws_bytes,
                   [&](int qc) { return make_bwd_layout(s, qc).total; });
}

size_t sparse_attn_bwd_workspace(const AttnShape& s) {
  return make_bwd_layout(s, default_chunk(s.S_q, bwd_per_query(s))).total;
}

size_t sparse_attn_bwd_workspace_min(const AttnShape& s) {
  // One query per chunk, or the default chunk when that is smaller (a
  // one-chunk layout keeps no cross-chunk sums).
  return std::min(make_bwd_layout(s, 1).total,
                  make_bwd_layout(s, default_chunk(s.S_q, bwd_per_query(s))).total);
}

int sparse_attn_bwd_chunks(const AttnShape& s, size_t ws_bytes) {
  const int qc = bwd_chunk(s, ws_bytes);
  return qc > 0 ? (s.S_q + qc - 1) / qc : 0;
}

// ---------------------------------------------------------------- both backward passes
static size_t kl_bwd_per_query(const AttnShape& s, int D_idx);

// Bytes of per-edge records per query: the main backward's and the loss
// backward's (the edge slot once).
static size_t fused_bwd_per_query(const AttnShape& s, int D_idx) {
  return bwd_per_query(s) + kl_bwd_per_query(s, D_idx) - (size_t)s.batch * s.H_kv * s.topk * 4;
}

FusedBwdLayout make_fused_bwd_layout(const AttnShape& s, int D_idx, int Qc) {
  FusedBwdLayout F{};
  F.B = make_bwd_layout(s, Qc);
  const edges::Layout& L = F.B.L;
  size_t o = F.B.total;
  // One record past the chunk's edges takes the stores of padding rows.
  F.rec = o;     o = align256(o + (size_t)(L.E + 1) * D_idx * 2);
  F.rec_sc = o;  o = align256(o + (size_t)(L.E + 1) * (D_idx / 32) * 4);
  F.g_rec = o;   o = align256(o + (size_t)(L.E + 1) * kBlock * 2);
  F.dk_part = o; o = align256(o + (size_t)s.batch * s.H_kv * s.S_k * D_idx * 4);
  F.dk_flag = o; o = align256(o + (size_t)s.batch * s.H_kv * s.n_blk * 4);
  F.lse_t = o;   o = align256(o + (size_t)s.batch * s.H_q * s.S_q * 4);
  F.total = o;
  return F;
}

int fused_bwd_chunk(const AttnShape& s, int D_idx, size_t ws_bytes) {
  return fit_chunk(default_chunk(s.S_q, fused_bwd_per_query(s, D_idx)), ws_bytes,
                   [&](int qc) { return make_fused_bwd_layout(s, D_idx, qc).total; });
}

size_t backward_workspace(const AttnShape& s, int D_idx) {
  return make_fused_bwd_layout(s, D_idx, default_chunk(s.S_q, fused_bwd_per_query(s, D_idx))).total;
}

size_t backward_workspace_min(const AttnShape& s, int D_idx) {
  return std::min(make_fused_bwd_layout(s, D_idx, 1).total,
                  make_fused_bwd_layout(s, D_idx, default_chunk(s.S_q, fused_bwd_per_query(s, D_idx))).total);
}

int backward_chunks(const AttnShape& s, int D_idx, size_t ws_bytes) {
  const int qc = fused_bwd_chunk(s, D_idx, ws_bytes);
  return qc > 0 ? (s.S_q + qc - 1) / qc : 0;
}

// ---------------------------------------------------------------- alignment loss
// The alignment loss keeps 32 bytes per edge, so one chunk covers all queries.
Layout make_kl_layout(const AttnShape& s) {
  Layout L{};
  const int G = s.H_q / s.H_kv;
  L.QT = kSubTiles * 4 * (32 / G);
  L.Qc = s.S_q;
  size_t o = layout_build(L, s);
  const long rows = (long)s.batch * s.H_kv * s.S_q;
  L.n_kl_wg = (int)((rows + 255) / 256);
  L.kl_rec = o;  o = align256(o + (size_t)L.E * 32);
  L.kl_wsum = o; o = align256(o + (size_t)L.n_kl_wg * 4);
  L.lse_t = o;   o = align256(o + (size_t)s.batch * s.H_q * s.S_q * 4);
  L.total = o;
  return L;
}

size_t kl_loss_workspace(const AttnShape& s) { return make_kl_layout(s).total; }

// Bytes of per-edge records per query: each (b, g) row's topk dq_idx records
// (D_idx fp16 values and one scale per 32 dims), g rows (128 bf16) and edge
// slots.
static size_t kl_bwd_per_query(const AttnShape& s, int D_idx) {
  return (size_t)s.batch * s.H_kv * s.topk * ((size_t)D_idx * 2 + 16 + kBlock * 2 + 4);
}

// Workspace layout for query chunks of Qc queries.
KlBwdLayout make_kl_bwd_layout(const AttnShape& s, int D_idx, int Qc) {
  KlBwdLayout K{};
  Layout& L = K.L;
  const int G = s.H_q / s.H_kv;
  L.QT = kSubTiles * 4 * (32 / G);
  L.Qc = Qc;
  size_t o = layout_build(L, s);
  // One record past the chunk's edges takes the stores of padding rows.
  K.rec = o;     o = align256(o + (size_t)(L.E + 1) * D_idx * 2);
  K.rec_sc = o;  o = align256(o + (size_t)(L.E + 1) * (D_idx / 32) * 4);
  K.g_rec = o;   o = align256(o + (size_t)(L.E + 1) * kBlock * 2);
  K.dk_part = o; o = align256(o + (size_t)s.batch * s.H_kv * s.S_k * D_idx * 4);
  K.dk_flag = o; o = align256(o + (size_t)s.batch * s.H_kv * s.n_blk * 4);
  K.lse_t = o;   o = align256(o + (size_t)s.batch * s.H_q * s.S_q * 4);
  K.total = o;
  L.total = o;
  return K;
}

int kl_bwd_chunk(const AttnShape& s, int D_idx, size_t ws_bytes) {
  return fit_chunk(default_chunk(s.S_q, kl_bwd_per_query(s, D_idx)), ws_bytes,
                   [&](int qc) { return make_kl_bwd_layout(s, D_idx, qc).total; });
}

size_t kl_loss_bwd_workspace(const AttnShape& s, int D_idx) {
  return make_kl_bwd_layout(s, D_idx, default_chunk(s.S_q, kl_bwd_per_query(s, D_idx))).total;
}

size_t kl_loss_bwd_workspace_min(const AttnShape& s, int D_idx) {
  return make_kl_bwd_layout(s, D_idx, 1).total;
}

int kl_loss_bwd_chunks(const AttnShape& s, int D_idx, size_t ws_bytes) {
  const int qc = kl_bwd_chunk(s, D_idx, ws_bytes);
  return qc > 0 ? (s.S_q + qc - 1) / qc : 0;
}

}  // namespace msa
