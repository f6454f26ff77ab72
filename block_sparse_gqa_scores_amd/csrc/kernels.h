// Internal launch interface between the C-ABI layer (msa_api.cpp) and the
// gfx950 kernels.  Shapes reaching these functions are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

// Block scores (see index_scan.hip).
hipError_t launch_index_scores(const uint16_t* q_idx, const uint16_t* k_idx, float* bm,
                               int batch, int S_q, int S_k, int H_kv, int D_idx, int n_blk,
                               hipStream_t stream);

// Block scores and Top-k in one pass, no block scores in memory (see
// index_scan.hip); only for the shapes index_select_fused accepts.
bool index_select_fused(int S_q, int H_kv, int topk);
hipError_t launch_index_select(const uint16_t* q_idx, const uint16_t* k_idx, int32_t* sel,
                               int batch, int S_q, int S_k, int H_kv, int D_idx, int n_blk,
                               int topk, hipStream_t stream);

// Top-k selection (see block_topk.hip).
hipError_t launch_block_topk(const float* bm, int32_t* idx, int batch, int S_q, int S_k,
                             int H_kv, int n_blk, int topk, hipStream_t stream);

// Block-mask form of selections (see block_mask.hip).
hipError_t launch_block_mask(const int32_t* sel, uint32_t* mask, long n_rows, int topk, int n_blk,
                             hipStream_t stream);
hipError_t launch_mask_blocks(const uint32_t* mask, int32_t* sel, long n_rows, int n_blk, int cap,
                              hipStream_t stream);

// Sparse attention (see sparse_attn.hip).
struct AttnShape {
  int batch, S_q, S_k, H_q, H_kv, n_blk, topk;
  float scale_log2;  // softmax scale * log2(e)
  float scale;       // softmax scale
};
// Workspace of the attention forward: the default size (query chunks whose
// per-edge records fit 16 GiB) and the smallest it accepts (one query per
// chunk).  A launch runs in the largest query chunks that fit its ws_bytes
// (never larger than the default ones); sparse_attn_chunks counts them, 0
// when ws_bytes is below the minimum.
size_t sparse_attn_workspace(const AttnShape& s);
size_t sparse_attn_workspace_min(const AttnShape& s);
int sparse_attn_chunks(const AttnShape& s, size_t ws_bytes);

// Optional stage events of msa_forward_profiled: ev[0..1] bracket the index
// scores, ev[2..3] the Top-k, and chunk c's attention stages take
// ev[4 + 6 c + 2 m] (before) and ev[4 + 6 c + 2 m + 1] (after) for m = 0
// (bucket build), 1 (partial), 2 (merge).  n >= 4 + 6 * chunks.
struct StageEvents {
  const hipEvent_t* ev;
  int n;
};
hipError_t launch_sparse_attn(const AttnShape& s, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int32_t* idx, uint16_t* out, float* lse,
                              void* ws, size_t ws_bytes, hipStream_t stream,
                              const StageEvents* events = nullptr);

// Main branch, backward (see attn_bwd.hip).
size_t sparse_attn_bwd_workspace(const AttnShape& s);
size_t sparse_attn_bwd_workspace_min(const AttnShape& s);
int sparse_attn_bwd_chunks(const AttnShape& s, size_t ws_bytes);
hipError_t launch_sparse_attn_bwd(const AttnShape& s, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const int32_t* idx, const uint16_t* out,
                                  const float* lse, const uint16_t* dout, uint16_t* dq,
                                  uint16_t* dk, uint16_t* dv, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

// Alignment loss, backward (see kl_bwd.hip).
size_t kl_loss_bwd_workspace(const AttnShape& s, int D_idx);
size_t kl_loss_bwd_workspace_min(const AttnShape& s, int D_idx);
int kl_loss_bwd_chunks(const AttnShape& s, int D_idx, size_t ws_bytes);
hipError_t launch_kl_loss_bwd(const AttnShape& s, int D_idx, const uint16_t* q, const uint16_t* k,
                              const uint16_t* q_idx, const uint16_t* k_idx, const int32_t* idx,
                              const float* lse, const float* lse_idx, float coef, uint16_t* dq_idx,
                              uint16_t* dk_idx, void* ws, size_t ws_bytes, hipStream_t stream);

// Both backward passes in one call: per query chunk, one bucket build and sort,
// then the main backward's kernels and the loss backward's.
size_t backward_workspace(const AttnShape& s, int D_idx);
size_t backward_workspace_min(const AttnShape& s, int D_idx);
int backward_chunks(const AttnShape& s, int D_idx, size_t ws_bytes);
hipError_t launch_backward(const AttnShape& s, int D_idx, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint16_t* q_idx, const uint16_t* k_idx,
                           const int32_t* idx, const uint16_t* out, const float* lse,
                           const float* lse_idx, const uint16_t* dout, float coef, uint16_t* dq,
                           uint16_t* dk, uint16_t* dv, uint16_t* dq_idx, uint16_t* dk_idx, void* ws,
                           size_t ws_bytes, hipStream_t stream);

// The host checks msa_forward makes before anything else (dims, then the
// pointers' presence and alignment); MSA_OK for an empty problem as well.
msa_status forward_checks(const msa_dims* d, const void* q, const void* k, const void* v,
                          const void* q_idx, const void* k_idx, const void* out, const float* lse,
                          const int32_t* block_idx_out);

// Writes n zero floats (a kernel, so the call can sit inside a graph capture).
hipError_t launch_fill_zero(float* dst, long n, hipStream_t stream);

// Alignment loss of the index branch, forward value (see sparse_attn.hip).
size_t kl_loss_workspace(const AttnShape& s);
hipError_t launch_kl_loss(const AttnShape& s, int D_idx, const uint16_t* q, const uint16_t* k,
                          const uint16_t* q_idx, const uint16_t* k_idx, const int32_t* idx,
                          const float* lse, float* kl_rows, float* loss, float* lse_idx, void* ws,
                          size_t ws_bytes, hipStream_t stream);

}  // namespace msa
