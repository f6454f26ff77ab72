// Parameters shared by the backward kernels: the main branch's
// (attn_bwd.hip) and the alignment loss's (kl_bwd.hip).  The combined
// backward (launch_backward, attn_bwd.hip) runs both on the same query chunks,
// one bucket build and sort per chunk serving the two.
#pragma once

#include "edge_buckets.h"

namespace msa {
namespace edges {

constexpr int kGStride = kBlock + 8;  // bf16 per row of the loss backward's g tile [row][key]

struct BwdParams {
  Params e;              // edge buckets, q, k, v, idx and shapes of the chunk
  const uint16_t* dout;  // [B][S_q][H_q][D] bf16
  const uint16_t* out;   // forward output, same layout
  const float* lse;      // forward LSE [B][H_q][S_q] (natural log)
  float2* stat;          // [B][H_kv][S_q][G]: (LSE in log2 units, sum_d dO O), a query's heads together
  u32x4* dq_rec;         // [slot][kRecBytes(G)]: the edge's dq as 12-bit codes, piece (quarter G + head) 2 + half
  float* dq_sc;          // [slot][4][G]: scale of each quarter's codes (dq = (code - 2048) scale)
  long sink;             // record slot written by padding rows (never read)
  uint16_t* dq;          // [B][S_q][H_q][D] bf16
  uint16_t* dk;          // [B][S_k][H_kv][D] bf16
  uint16_t* dv;
  float* dk_acc;         // fp32 sums of earlier chunks (several chunks only)
  float* dv_acc;
  float scale;           // softmax scale
  int first, last;       // this chunk is the first / the last
  // Work items of attn_bwd_kernel: the sub-tiles of a (group, block) in
  // segments of about `seg`, so that a block most queries select spreads
  // over several workgroups.  Index x = j * B * H_kv + b * H_kv + g.
  int seg;               // sub-tiles per segment; a block with more is split
  int seg_on;            // 0: no block of the chunk can exceed seg (one work item per block)
  int32_t* blk_t;        // [x]: the block's sub-tiles in this chunk
  int32_t* blk_item;     // [x]: first work item of x (NBLK + 1, total at the end)
  int32_t* blk_part;     // [x]: first partial slot of a split x
  int2* items;           // (x, segment)
  float* part;           // [slot][2][kBlock][kD]: one segment's fp32 dK (times scale), dV
};

struct KlBwdParams {
  Params e;
  const float* lse_idx;  // [B][H_kv][S_q]: log-sum-exp of z over T (natural log)
  float coef;            // gradient of the loss / (B * S_q * H_kv)
  uint16_t* rec;         // [slot][D_idx / 32][32] fp16 (rec_dim order) / scale
  float* rec_sc;         // [slot][D_idx / 32]
  uint16_t* g_rec;       // [slot][128] bf16: g of each (edge, key) (kl_grad_kernel), read by kl_dk_kernel
  long sink;             // record slot written by padding rows (never read)
  float* dk_part;        // [B][H_kv][S_k][D_idx] fp32, per group
  int32_t* dk_flag;      // [B][H_kv][n_blk]: 1 if the group's dk_part rows of the block hold data
  uint16_t* dq_idx;      // [B][S_q][H_kv][D_idx] bf16
  uint16_t* dk_idx;      // [B][S_k][D_idx] bf16
  int D_idx;
  int first;             // this chunk is the first (dk_part is stored, not added)
};

// The loss backward's kernels of one query chunk (kp.e.q0; its bucket build
// and sort done): g rows and dq_idx records, their per-row merge, and the
// per-group dk_idx parts; then, after the last chunk, the reduce of the
// groups' parts (kl_bwd.hip; D_idx = 64 or 128).
hipError_t launch_kl_chunk(const AttnShape& s, const Layout& L, const KlBwdParams& kp, hipStream_t st);
hipError_t launch_kl_dk_reduce(const KlBwdParams& kp, int D_idx, long blocks, hipStream_t st);

}  // namespace edges
}  // namespace msa
