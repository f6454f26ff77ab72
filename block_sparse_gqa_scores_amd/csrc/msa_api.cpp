// C ABI of the MSA forward path: argument checks on the host, workspace
// layout, and the launch order index scores -> Top-k -> sparse attention on
// the caller's stream.  Declarations and the contract are in include/msa.h.
#include "msa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.h"

namespace {

constexpr int kBlockSize = 128;
constexpr int kHeadDim = 128;
constexpr int kMaxTopk = 64;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t n_blocks(const msa_dims& d) { return (int64_t(d.seqlen_k) + d.block_size - 1) / d.block_size; }

bool is_empty(const msa_dims& d) { return d.batch == 0 || d.seqlen_q == 0; }

// Structural checks common to every entry point.
msa_status check_dims(const msa_dims* d, bool uses_index, bool uses_main) {
  if (!d) return MSA_ERR_NULL_PTR;
  if (d->batch < 0 || d->seqlen_q < 0 || d->seqlen_k < 0) return MSA_ERR_INVALID_DIMS;
  if (d->seqlen_k < d->seqlen_q) return MSA_ERR_INVALID_DIMS;
  if (d->num_heads_kv <= 0 || d->block_size <= 0 || d->topk <= 0) return MSA_ERR_INVALID_DIMS;
  if (uses_main) {
    if (d->num_heads_q <= 0 || d->head_dim <= 0) return MSA_ERR_INVALID_DIMS;
    if (d->num_heads_q % d->num_heads_kv != 0) return MSA_ERR_INVALID_DIMS;
    if (!std::isfinite(d->softmax_scale) || d->softmax_scale < 0.f) return MSA_ERR_INVALID_DIMS;
  }
  if (uses_index && d->index_dim <= 0) return MSA_ERR_INVALID_DIMS;
  if (d->causal != 1) return MSA_ERR_UNSUPPORTED;
  if (d->block_size != kBlockSize) return MSA_ERR_UNSUPPORTED;
  if (d->topk > kMaxTopk) return MSA_ERR_UNSUPPORTED;
  if (uses_index && d->index_dim != 64 && d->index_dim != 128) return MSA_ERR_UNSUPPORTED;
  if (uses_main) {
    if (d->head_dim != kHeadDim) return MSA_ERR_UNSUPPORTED;
    const int G = d->num_heads_q / d->num_heads_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16 && G != 32) return MSA_ERR_UNSUPPORTED;
  }
  if (is_empty(*d)) return MSA_OK;
  if (d->seqlen_k == 0) return MSA_ERR_INVALID_DIMS;
  // Index arithmetic inside the kernels is 32-bit where it counts rows/slots.
  const int64_t rows = int64_t(d->batch) * d->num_heads_kv * d->seqlen_q;
  if (rows * d->topk >= (int64_t(1) << 31)) return MSA_ERR_UNSUPPORTED;
  if (int64_t(d->batch) * d->num_heads_kv * n_blocks(*d) >= (int64_t(1) << 31)) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

msa::AttnShape attn_shape(const msa_dims& d) {
  msa::AttnShape s;
  s.batch = d.batch;
  s.S_q = d.seqlen_q;
  s.S_k = d.seqlen_k;
  s.H_q = d.num_heads_q;
  s.H_kv = d.num_heads_kv;
  s.n_blk = int(n_blocks(d));
  s.topk = d.topk;
  s.scale = d.softmax_scale != 0.f ? d.softmax_scale : 1.f / std::sqrt(float(d.head_dim));
  s.scale_log2 = s.scale * 1.4426950408889634f;
  return s;
}

size_t bm_bytes(const msa_dims& d) {
  return size_t(d.batch) * d.num_heads_kv * d.seqlen_q * n_blocks(d) * sizeof(float);
}
size_t idx_bytes(const msa_dims& d) {
  return size_t(d.batch) * d.num_heads_kv * d.seqlen_q * d.topk * sizeof(int32_t);
}

// msa_forward scores and selects in one pass (no block scores in memory) when
// the fused kernel covers the shape.
bool fused_select(const msa_dims& d) {
  return msa::index_select_fused(d.seqlen_q, d.num_heads_kv, d.topk);
}

size_t forward_bm_bytes(const msa_dims& d) { return fused_select(d) ? 0 : align256(bm_bytes(d)); }

msa_status from_hip(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_HIP; }

// Default (`min` false) or smallest (`min` true) workspace of an entry point;
// (size_t)-1 when the dims are not valid for it.
size_t workspace_of(const msa_dims* d, int entry, bool min) {
  const size_t bad = ~size_t(0);
  switch (entry) {
    case MSA_ENTRY_INDEX_SCORES:
      return check_dims(d, true, false) == MSA_OK ? 0 : bad;
    case MSA_ENTRY_BLOCK_TOPK:
      return check_dims(d, false, false) == MSA_OK ? 0 : bad;
    case MSA_ENTRY_SPARSE_ATTN_FWD:
      if (check_dims(d, false, true) != MSA_OK) return bad;
      if (is_empty(*d)) return 0;
      return min ? msa::sparse_attn_workspace_min(attn_shape(*d)) : msa::sparse_attn_workspace(attn_shape(*d));
    case MSA_ENTRY_FORWARD:
      if (check_dims(d, true, true) != MSA_OK) return bad;
      if (is_empty(*d)) return 0;
      return forward_bm_bytes(*d) + align256(idx_bytes(*d)) +
             (min ? msa::sparse_attn_workspace_min(attn_shape(*d)) : msa::sparse_attn_workspace(attn_shape(*d)));
    case MSA_ENTRY_KL_LOSS_FWD:
      if (check_dims(d, true, true) != MSA_OK) return bad;
      return is_empty(*d) ? 0 : msa::kl_loss_workspace(attn_shape(*d));
    case MSA_ENTRY_SPARSE_ATTN_BWD:
      if (check_dims(d, false, true) != MSA_OK) return bad;
      if (is_empty(*d)) return 0;
      return min ? msa::sparse_attn_bwd_workspace_min(attn_shape(*d))
                 : msa::sparse_attn_bwd_workspace(attn_shape(*d));
    case MSA_ENTRY_KL_LOSS_BWD:
      if (check_dims(d, true, true) != MSA_OK) return bad;
      if (is_empty(*d)) return 0;
      return min ? msa::kl_loss_bwd_workspace_min(attn_shape(*d), d->index_dim)
                 : msa::kl_loss_bwd_workspace(attn_shape(*d), d->index_dim);
    case MSA_ENTRY_BACKWARD:
      if (check_dims(d, true, true) != MSA_OK) return bad;
      if (is_empty(*d)) return 0;
      return min ? msa::backward_workspace_min(attn_shape(*d), d->index_dim)
                 : msa::backward_workspace(attn_shape(*d), d->index_dim);
    default:
      return bad;
  }
}

}  // namespace

namespace msa {

msa_status forward_checks(const msa_dims* d, const void* q, const void* k, const void* v,
                          const void* q_idx, const void* k_idx, const void* out, const float* lse,
                          const int32_t* block_idx_out) {
  msa_status st = check_dims(d, true, true);
  if (st != MSA_OK || is_empty(*d)) return st;
  if (!q || !k || !v || !q_idx || !k_idx || !out) return MSA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_idx) || !aligned16(k_idx) ||
      !aligned16(out) || (lse && !aligned16(lse)) || (block_idx_out && !aligned16(block_idx_out)))
    return MSA_ERR_MISALIGNED;
  return MSA_OK;
}

}  // namespace msa

extern "C" {

const char* msa_status_str(msa_status s) {
  switch (s) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_NULL_PTR: return "MSA_ERR_NULL_PTR";
    case MSA_ERR_INVALID_DIMS: return "MSA_ERR_INVALID_DIMS";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_MISALIGNED: return "MSA_ERR_MISALIGNED";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

size_t msa_workspace_bytes(const msa_dims* d, int entry) { return workspace_of(d, entry, false); }

size_t msa_workspace_min_bytes(const msa_dims* d, int entry) { return workspace_of(d, entry, true); }

int msa_attn_chunks(const msa_dims* d, int entry, size_t ws_bytes) {
  const size_t need = workspace_of(d, entry, true);
  if (need == ~size_t(0) || ws_bytes < need || is_empty(*d)) return 0;
  const msa::AttnShape s = attn_shape(*d);
  switch (entry) {
    case MSA_ENTRY_SPARSE_ATTN_FWD:
      return msa::sparse_attn_chunks(s, ws_bytes);
    case MSA_ENTRY_FORWARD:
      return msa::sparse_attn_chunks(s, ws_bytes - forward_bm_bytes(*d) - align256(idx_bytes(*d)));
    case MSA_ENTRY_KL_LOSS_FWD:
      return 1;
    case MSA_ENTRY_SPARSE_ATTN_BWD:
      return msa::sparse_attn_bwd_chunks(s, ws_bytes);
    case MSA_ENTRY_KL_LOSS_BWD:
      return msa::kl_loss_bwd_chunks(s, d->index_dim, ws_bytes);
    case MSA_ENTRY_BACKWARD:
      return msa::backward_chunks(s, d->index_dim, ws_bytes);
    default:
      return 0;
  }
}

msa_status msa_index_scores(const msa_dims* d, const void* q_idx, const void* k_idx,
                            float* block_scores, void* stream) {
  msa_status st = check_dims(d, true, false);
  if (st != MSA_OK || is_empty(*d)) return st;
  if (!q_idx || !k_idx || !block_scores) return MSA_ERR_NULL_PTR;
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(block_scores)) return MSA_ERR_MISALIGNED;
  return from_hip(msa::launch_index_scores(
      static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx), block_scores,
      d->batch, d->seqlen_q, d->seqlen_k, d->num_heads_kv, d->index_dim, int(n_blocks(*d)),
      static_cast<hipStream_t>(stream)));
}

msa_status msa_block_topk(const msa_dims* d, const float* block_scores, int32_t* block_idx,
                          void* stream) {
  msa_status st = check_dims(d, false, false);
  if (st != MSA_OK || is_empty(*d)) return st;
  if (!block_scores || !block_idx) return MSA_ERR_NULL_PTR;
  if (!aligned16(block_scores) || !aligned16(block_idx)) return MSA_ERR_MISALIGNED;
  return from_hip(msa::launch_block_topk(block_scores, block_idx, d->batch, d->seqlen_q,
                                         d->seqlen_k, d->num_heads_kv, int(n_blocks(*d)),
                                         d->topk, static_cast<hipStream_t>(stream)));
}

msa_status msa_block_mask(const msa_dims* d, const int32_t* block_idx, uint32_t* mask,
                          void* stream) {
  msa_status st = check_dims(d, false, false);
  if (st != MSA_OK || is_empty(*d)) return st;
  if (!block_idx || !mask) return MSA_ERR_NULL_PTR;
  if (!aligned16(block_idx) || !aligned16(mask)) return MSA_ERR_MISALIGNED;
  const long rows = long(d->batch) * d->num_heads_kv * d->seqlen_q;
  return from_hip(msa::launch_block_mask(block_idx, mask, rows, d->topk, int(n_blocks(*d)),
                                         static_cast<hipStream_t>(stream)));
}

msa_status msa_mask_blocks(const msa_dims* d, const uint32_t* mask, int32_t* block_idx,
                           void* stream) {
  msa_status st = check_dims(d, false, false);
  if (st != MSA_OK || is_empty(*d)) return st;
  if (!block_idx || !mask) return MSA_ERR_NULL_PTR;
  if (!aligned16(block_idx) || !aligned16(mask)) return MSA_ERR_MISALIGNED;
  const long rows = long(d->batch) * d->num_heads_kv * d->seqlen_q;
  return from_hip(msa::launch_mask_blocks(mask, block_idx, rows, int(n_blocks(*d)), d->topk,
                                          static_cast<hipStream_t>(stream)));
}

msa_status msa_sparse_attn_fwd(const msa_dims* d, const void* q, const void* k, const void* v,
                               const int32_t* block_idx, void* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream) {
  msa_status st = check_dims(d, false, true);
  if (st != MSA_OK || is_empty(*d)) return st;
  if (!q || !k || !v || !block_idx || !out) return MSA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(block_idx) ||
      !aligned16(out) || (lse && !aligned16(lse)))
    return MSA_ERR_MISALIGNED;
  const msa::AttnShape s = attn_shape(*d);
  const size_t need = msa::sparse_attn_workspace_min(s);
  if (!ws || ws_bytes < need) return ws ? MSA_ERR_WORKSPACE_TOO_SMALL : MSA_ERR_NULL_PTR;
  if (!aligned16(ws)) return MSA_ERR_MISALIGNED;
  return from_hip(msa::launch_sparse_attn(
      s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), block_idx, static_cast<uint16_t*>(out), lse, ws, ws_bytes,
      static_cast<hipStream_t>(stream)));
}

msa_status msa_sparse_attn_bwd(const msa_dims* d, const void* q, const void* k, const void* v,
                               const int32_t* block_idx, const void* out, const float* lse,
                               const void* dout, void* dq, void* dk, void* dv, void* ws,
                               size_t ws_bytes, void* stream) {
  msa_status st = check_dims(d, false, true);
  if (st != MSA_OK) return st;
  if (is_empty(*d)) {  // no query: zero key gradients
    if (d->batch == 0 || d->seqlen_k == 0) return MSA_OK;
    if (!dk || !dv) return MSA_ERR_NULL_PTR;
    if (!aligned16(dk) || !aligned16(dv)) return MSA_ERR_MISALIGNED;
    const long n = long(d->batch) * d->seqlen_k * d->num_heads_kv * d->head_dim / 2;
    hipStream_t strm = static_cast<hipStream_t>(stream);
    if (msa::launch_fill_zero(static_cast<float*>(dk), n, strm) != hipSuccess) return MSA_ERR_HIP;
    return from_hip(msa::launch_fill_zero(static_cast<float*>(dv), n, strm));
  }
  if (!q || !k || !v || !block_idx || !out || !lse || !dout || !dq || !dk || !dv)
    return MSA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(block_idx) ||
      !aligned16(out) || !aligned16(lse) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return MSA_ERR_MISALIGNED;
  const msa::AttnShape s = attn_shape(*d);
  const size_t need = msa::sparse_attn_bwd_workspace_min(s);
  if (!ws || ws_bytes < need) return ws ? MSA_ERR_WORKSPACE_TOO_SMALL : MSA_ERR_NULL_PTR;
  if (!aligned16(ws)) return MSA_ERR_MISALIGNED;
  return from_hip(msa::launch_sparse_attn_bwd(
      s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), block_idx, static_cast<const uint16_t*>(out), lse,
      static_cast<const uint16_t*>(dout), static_cast<uint16_t*>(dq), static_cast<uint16_t*>(dk),
      static_cast<uint16_t*>(dv), ws, ws_bytes, static_cast<hipStream_t>(stream)));
}

msa_status msa_kl_loss_bwd(const msa_dims* d, const void* q, const void* k, const void* q_idx,
                           const void* k_idx, const int32_t* block_idx, const float* lse,
                           const float* lse_idx, float grad_loss, void* dq_idx, void* dk_idx,
                           void* ws, size_t ws_bytes, void* stream) {
  msa_status st = check_dims(d, true, true);
  if (st != MSA_OK) return st;
  if (!std::isfinite(grad_loss)) return MSA_ERR_INVALID_DIMS;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  if (is_empty(*d)) {  // no row: zero index-key gradient
    if (d->batch == 0 || d->seqlen_k == 0) return MSA_OK;
    if (!dk_idx) return MSA_ERR_NULL_PTR;
    if (!aligned16(dk_idx)) return MSA_ERR_MISALIGNED;
    const long n = long(d->batch) * d->seqlen_k * d->index_dim / 2;
    return from_hip(msa::launch_fill_zero(static_cast<float*>(dk_idx), n, strm));
  }
  if (!q || !k || !q_idx || !k_idx || !block_idx || !lse || !lse_idx || !dq_idx || !dk_idx)
    return MSA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_idx) || !aligned16(k_idx) ||
      !aligned16(block_idx) || !aligned16(lse) || !aligned16(lse_idx) || !aligned16(dq_idx) ||
      !aligned16(dk_idx))
    return MSA_ERR_MISALIGNED;
  const msa::AttnShape s = attn_shape(*d);
  const size_t need = msa::kl_loss_bwd_workspace_min(s, d->index_dim);
  if (!ws || ws_bytes < need) return ws ? MSA_ERR_WORKSPACE_TOO_SMALL : MSA_ERR_NULL_PTR;
  if (!aligned16(ws)) return MSA_ERR_MISALIGNED;
  const float coef = float(double(grad_loss) / (double(d->batch) * d->seqlen_q * d->num_heads_kv));
  return from_hip(msa::launch_kl_loss_bwd(
      s, d->index_dim, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx), block_idx, lse,
      lse_idx, coef, static_cast<uint16_t*>(dq_idx), static_cast<uint16_t*>(dk_idx), ws, ws_bytes,
      strm));
}

msa_status msa_backward(const msa_dims* d, const void* q, const void* k, const void* v,
                        const void* q_idx, const void* k_idx, const int32_t* block_idx,
                        const void* out, const float* lse, const float* lse_idx,
                        const void* dout, float grad_loss, void* dq, void* dk, void* dv,
                        void* dq_idx, void* dk_idx, void* ws, size_t ws_bytes, void* stream) {
  msa_status st = check_dims(d, true, true);
  if (st != MSA_OK) return st;
  if (!std::isfinite(grad_loss)) return MSA_ERR_INVALID_DIMS;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  if (is_empty(*d)) {  // no query: zero key gradients
    if (d->batch == 0 || d->seqlen_k == 0) return MSA_OK;
    if (!dk || !dv || !dk_idx) return MSA_ERR_NULL_PTR;
    if (!aligned16(dk) || !aligned16(dv) || !aligned16(dk_idx)) return MSA_ERR_MISALIGNED;
    const long n = long(d->batch) * d->seqlen_k * d->num_heads_kv * d->head_dim / 2;
    if (msa::launch_fill_zero(static_cast<float*>(dk), n, strm) != hipSuccess) return MSA_ERR_HIP;
    if (msa::launch_fill_zero(static_cast<float*>(dv), n, strm) != hipSuccess) return MSA_ERR_HIP;
    const long ni = long(d->batch) * d->seqlen_k * d->index_dim / 2;
    return from_hip(msa::launch_fill_zero(static_cast<float*>(dk_idx), ni, strm));
  }
  if (!q || !k || !v || !q_idx || !k_idx || !block_idx || !out || !lse || !lse_idx || !dout || !dq ||
      !dk || !dv || !dq_idx || !dk_idx)
    return MSA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_idx) || !aligned16(k_idx) ||
      !aligned16(block_idx) || !aligned16(out) || !aligned16(lse) || !aligned16(lse_idx) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dq_idx) ||
      !aligned16(dk_idx))
    return MSA_ERR_MISALIGNED;
  const msa::AttnShape s = attn_shape(*d);
  const size_t need = msa::backward_workspace_min(s, d->index_dim);
  if (!ws || ws_bytes < need) return ws ? MSA_ERR_WORKSPACE_TOO_SMALL : MSA_ERR_NULL_PTR;
  if (!aligned16(ws)) return MSA_ERR_MISALIGNED;
  const float coef = float(double(grad_loss) / (double(d->batch) * d->seqlen_q * d->num_heads_kv));
  return from_hip(msa::launch_backward(
      s, d->index_dim, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(q_idx),
      static_cast<const uint16_t*>(k_idx), block_idx, static_cast<const uint16_t*>(out), lse, lse_idx,
      static_cast<const uint16_t*>(dout), coef, static_cast<uint16_t*>(dq), static_cast<uint16_t*>(dk),
      static_cast<uint16_t*>(dv), static_cast<uint16_t*>(dq_idx), static_cast<uint16_t*>(dk_idx), ws,
      ws_bytes, strm));
}

msa_status msa_kl_loss_fwd(const msa_dims* d, const void* q, const void* k, const void* q_idx,
                           const void* k_idx, const int32_t* block_idx, const float* lse,
                           float* kl_rows, float* loss, float* lse_idx, void* ws, size_t ws_bytes,
                           void* stream) {
  msa_status st = check_dims(d, true, true);
  if (st != MSA_OK) return st;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  if (is_empty(*d)) {
    if (!loss) return MSA_OK;
    if (!aligned16(loss)) return MSA_ERR_MISALIGNED;
    return from_hip(msa::launch_fill_zero(loss, 1, strm));
  }
  if (!q || !k || !q_idx || !k_idx || !block_idx || !lse) return MSA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_idx) || !aligned16(k_idx) ||
      !aligned16(block_idx) || !aligned16(lse) || (kl_rows && !aligned16(kl_rows)) ||
      (loss && !aligned16(loss)) || (lse_idx && !aligned16(lse_idx)))
    return MSA_ERR_MISALIGNED;
  const msa::AttnShape s = attn_shape(*d);
  const size_t need = msa::kl_loss_workspace(s);
  if (!ws || ws_bytes < need) return ws ? MSA_ERR_WORKSPACE_TOO_SMALL : MSA_ERR_NULL_PTR;
  if (!aligned16(ws)) return MSA_ERR_MISALIGNED;
  return from_hip(msa::launch_kl_loss(
      s, d->index_dim, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx), block_idx, lse,
      kl_rows, loss, lse_idx, ws, ws_bytes, strm));
}

namespace {

msa_status forward_impl(const msa_dims* d, const void* q, const void* k, const void* v,
                        const void* q_idx, const void* k_idx, void* out, float* lse,
                        int32_t* block_idx_out, void* ws, size_t ws_bytes, void* stream,
                        const msa::StageEvents* ev) {
  msa_status st = msa::forward_checks(d, q, k, v, q_idx, k_idx, out, lse, block_idx_out);
  if (st != MSA_OK || is_empty(*d)) return st;
  const msa::AttnShape s = attn_shape(*d);
  const size_t bm_sz = forward_bm_bytes(*d);
  const size_t idx_sz = align256(idx_bytes(*d));
  const size_t need = bm_sz + idx_sz + msa::sparse_attn_workspace_min(s);
  if (!ws || ws_bytes < need) return ws ? MSA_ERR_WORKSPACE_TOO_SMALL : MSA_ERR_NULL_PTR;
  if (ev && ev->n < 4 + 6 * msa::sparse_attn_chunks(s, ws_bytes - bm_sz - idx_sz)) return MSA_ERR_INVALID_DIMS;
  const size_t attn_sz = ws_bytes - bm_sz - idx_sz;
  if (!aligned16(ws)) return MSA_ERR_MISALIGNED;
  char* base = static_cast<char*>(ws);
  float* bm = reinterpret_cast<float*>(base);
  int32_t* idx = block_idx_out ? block_idx_out : reinterpret_cast<int32_t*>(base + bm_sz);
  void* attn_ws = base + bm_sz + idx_sz;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (ev) (void)hipEventRecord(ev->ev[0], strm);
  if (fused_select(*d)) {
    // One kernel scores and selects; the Top-k stage is empty.
    e = msa::launch_index_select(static_cast<const uint16_t*>(q_idx),
                                 static_cast<const uint16_t*>(k_idx), idx, d->batch, d->seqlen_q,
                                 d->seqlen_k, d->num_heads_kv, d->index_dim, s.n_blk, d->topk,
                                 strm);
    if (e != hipSuccess) return MSA_ERR_HIP;
    if (ev) (void)hipEventRecord(ev->ev[1], strm);
    if (ev) (void)hipEventRecord(ev->ev[2], strm);
  } else {
    e = msa::launch_index_scores(static_cast<const uint16_t*>(q_idx),
                                 static_cast<const uint16_t*>(k_idx), bm, d->batch, d->seqlen_q,
                                 d->seqlen_k, d->num_heads_kv, d->index_dim, s.n_blk, strm);
    if (e != hipSuccess) return MSA_ERR_HIP;
    if (ev) (void)hipEventRecord(ev->ev[1], strm);
    if (ev) (void)hipEventRecord(ev->ev[2], strm);
    e = msa::launch_block_topk(bm, idx, d->batch, d->seqlen_q, d->seqlen_k, d->num_heads_kv,
                               s.n_blk, d->topk, strm);
    if (e != hipSuccess) return MSA_ERR_HIP;
  }
  if (ev) (void)hipEventRecord(ev->ev[3], strm);
  e = msa::launch_sparse_attn(s, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                              static_cast<const uint16_t*>(v), idx, static_cast<uint16_t*>(out),
                              lse, attn_ws, attn_sz, strm, ev);
  return from_hip(e);
}

}  // namespace

msa_status msa_forward(const msa_dims* d, const void* q, const void* k, const void* v,
                       const void* q_idx, const void* k_idx, void* out, float* lse,
                       int32_t* block_idx_out, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(d, q, k, v, q_idx, k_idx, out, lse, block_idx_out, ws, ws_bytes, stream,
                      nullptr);
}

msa_status msa_forward_profiled(const msa_dims* d, const void* q, const void* k, const void* v,
                                const void* q_idx, const void* k_idx, void* out, float* lse,
                                int32_t* block_idx_out, void* ws, size_t ws_bytes, void* stream,
                                void* const* events, int n_events) {
  if (!events) return MSA_ERR_NULL_PTR;
  if (n_events < 4) return MSA_ERR_INVALID_DIMS;
  for (int x = 0; x < n_events; ++x)
    if (!events[x]) return MSA_ERR_NULL_PTR;
  msa::StageEvents ev{reinterpret_cast<const hipEvent_t*>(events), n_events};
  return forward_impl(d, q, k, v, q_idx, k_idx, out, lse, block_idx_out, ws, ws_bytes, stream, &ev);
}

}  // extern "C"
