// Host check of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer:
// every argument check of include/msa.h on the failure paths, the workspace
// and chunk planning over a sweep of shapes (including the large ones, where
// size arithmetic would overflow first), and valid calls that reach the
// (stubbed) launchers.  Pointers are fake addresses that are never
// dereferenced.  Exits 0 when every expectation holds.
#include <cstdio>
#include <cstdlib>

#include "msa.h"

extern int g_launches;

namespace {

int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, \
                   __LINE__, #cond);                                   \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

void* const A = reinterpret_cast<void*>(0x10000);    // aligned, never dereferenced
void* const MIS = reinterpret_cast<void*>(0x10008);  // misaligned

msa_dims dims(int B, int Sq, int Sk, int Hq, int Hkv, int topk = 16, int Didx = 128) {
  msa_dims d{};
  d.batch = B; d.seqlen_q = Sq; d.seqlen_k = Sk; d.num_heads_q = Hq; d.num_heads_kv = Hkv;
  d.head_dim = 128; d.index_dim = Didx; d.block_size = 128; d.topk = topk; d.causal = 1;
  d.softmax_scale = 0.f;
  return d;
}

const size_t kHuge = size_t(1) << 40;
const size_t kBad = ~size_t(0);

void check_dims_rejections() {
  msa_dims d = dims(1, 256, 512, 8, 2);
  auto fwd = [&](const msa_dims* x) {
    return msa_forward(x, A, A, A, A, A, A, nullptr, nullptr, A, kHuge, nullptr);
  };
  EXPECT(fwd(nullptr) == MSA_ERR_NULL_PTR);
  msa_dims x = d; x.batch = -1; EXPECT(fwd(&x) == MSA_ERR_INVALID_DIMS);
  x = d; x.seqlen_q = 600; EXPECT(fwd(&x) == MSA_ERR_INVALID_DIMS);
  x = d; x.num_heads_q = 7; EXPECT(fwd(&x) == MSA_ERR_INVALID_DIMS);
  x = d; x.topk = 0; EXPECT(fwd(&x) == MSA_ERR_INVALID_DIMS);
  x = d; x.softmax_scale = -1.f; EXPECT(fwd(&x) == MSA_ERR_INVALID_DIMS);
  x = d; x.causal = 0; EXPECT(fwd(&x) == MSA_ERR_UNSUPPORTED);
  x = d; x.head_dim = 64; EXPECT(fwd(&x) == MSA_ERR_UNSUPPORTED);
  x = d; x.index_dim = 96; EXPECT(fwd(&x) == MSA_ERR_UNSUPPORTED);
  x = d; x.topk = 65; EXPECT(fwd(&x) == MSA_ERR_UNSUPPORTED);
  x = d; x.num_heads_q = 6; EXPECT(fwd(&x) == MSA_ERR_UNSUPPORTED);
  // 32-bit slot ids: rows * topk must stay below 2^31
  x = dims(1 << 10, 1 << 17, 1 << 17, 8, 2); EXPECT(fwd(&x) == MSA_ERR_UNSUPPORTED);
  x = dims(1 << 14, 1 << 17, 1 << 17, 8, 8); EXPECT(msa_workspace_bytes(&x, MSA_ENTRY_FORWARD) == kBad);
}

void check_pointers() {
  msa_dims d = dims(1, 256, 512, 8, 2);
  EXPECT(msa_forward(&d, nullptr, A, A, A, A, A, nullptr, nullptr, A, kHuge, nullptr) == MSA_ERR_NULL_PTR);
  EXPECT(msa_forward(&d, A, A, MIS, A, A, A, nullptr, nullptr, A, kHuge, nullptr) == MSA_ERR_MISALIGNED);
  EXPECT(msa_forward(&d, A, A, A, A, A, A, nullptr, nullptr, nullptr, 0, nullptr) == MSA_ERR_NULL_PTR);
  EXPECT(msa_sparse_attn_fwd(&d, A, A, A, nullptr, A, nullptr, A, kHuge, nullptr) == MSA_ERR_NULL_PTR);
  EXPECT(msa_sparse_attn_fwd(&d, A, A, A, static_cast<const int32_t*>(A), MIS, nullptr, A, kHuge, nullptr) ==
         MSA_ERR_MISALIGNED);
  EXPECT(msa_index_scores(&d, A, A, nullptr, nullptr) == MSA_ERR_NULL_PTR);
  EXPECT(msa_block_topk(&d, static_cast<const float*>(MIS), static_cast<int32_t*>(A), nullptr) ==
         MSA_ERR_MISALIGNED);
  EXPECT(msa_block_mask(&d, nullptr, static_cast<uint32_t*>(A), nullptr) == MSA_ERR_NULL_PTR);
  EXPECT(msa_mask_blocks(&d, static_cast<const uint32_t*>(A), nullptr, nullptr) == MSA_ERR_NULL_PTR);
  const float* F = static_cast<const float*>(A);
  EXPECT(msa_kl_loss_fwd(&d, A, A, A, A, nullptr, F, nullptr, nullptr, nullptr, A, kHuge, nullptr) ==
         MSA_ERR_NULL_PTR);
  EXPECT(msa_kl_loss_bwd(&d, A, A, A, A, static_cast<const int32_t*>(A), F, F, 1.f, A, MIS, A, kHuge,
                         nullptr) == MSA_ERR_MISALIGNED);
  EXPECT(msa_sparse_attn_bwd(&d, A, A, A, static_cast<const int32_t*>(A), A, F, A, A, A, nullptr, A, kHuge,
                             nullptr) == MSA_ERR_NULL_PTR);
  void* ev[10];
  for (auto& e : ev) e = A;
  EXPECT(msa_forward_profiled(&d, A, A, A, A, A, A, nullptr, nullptr, A, kHuge, nullptr, nullptr, 10) ==
         MSA_ERR_NULL_PTR);
  EXPECT(msa_forward_profiled(&d, A, A, A, A, A, A, nullptr, nullptr, A, kHuge, nullptr, ev, 9) ==
         MSA_ERR_INVALID_DIMS);
}

// Workspace planning over a sweep of shapes: min <= designed, chunk counts
// non-increasing in ws_bytes, 1 chunk at the designed size (or the designed
// count), 0 below the minimum, and the size check of each entry point.
void check_planning() {
  const int entries[] = {MSA_ENTRY_SPARSE_ATTN_FWD, MSA_ENTRY_FORWARD, MSA_ENTRY_SPARSE_ATTN_BWD,
                         MSA_ENTRY_KL_LOSS_BWD};
  const msa_dims shapes[] = {dims(1, 256, 512, 8, 2),          dims(2, 1000, 1300, 16, 2, 6),
                             dims(1, 4096, 4096, 8, 2, 16, 64), dims(1, 32768, 32768, 64, 8),
                             dims(1, 131072, 131072, 64, 8),    dims(64, 1, 262144, 64, 8),
                             dims(1, 16384, 1048576, 64, 8),    dims(3, 1, 5000, 16, 2, 16, 64),
                             dims(1, 130, 9000, 4, 1, 64),      dims(2, 300, 300, 32, 1, 4, 64)};
  for (const msa_dims& d : shapes) {
    for (int e : entries) {
      const size_t full = msa_workspace_bytes(&d, e), low = msa_workspace_min_bytes(&d, e);
      EXPECT(full != kBad && low != kBad && low <= full && low > 0);
      const int n_full = msa_attn_chunks(&d, e, full);
      EXPECT(n_full >= 1);
      EXPECT(msa_attn_chunks(&d, e, low) >= n_full);
      EXPECT(msa_attn_chunks(&d, e, low - 1) == 0);
      int prev = msa_attn_chunks(&d, e, low);
      for (int s = 1; s <= 16; ++s) {
        const size_t ws = low + (full - low) / 16 * s;
        const int n = msa_attn_chunks(&d, e, ws);
        EXPECT(n >= 1 && n <= prev);
        prev = n;
      }
    }
    const size_t lf = msa_workspace_min_bytes(&d, MSA_ENTRY_FORWARD);
    EXPECT(msa_forward(&d, A, A, A, A, A, A, nullptr, nullptr, A, lf - 1, nullptr) ==
           MSA_ERR_WORKSPACE_TOO_SMALL);
    const size_t la = msa_workspace_min_bytes(&d, MSA_ENTRY_SPARSE_ATTN_FWD);
    EXPECT(msa_sparse_attn_fwd(&d, A, A, A, static_cast<const int32_t*>(A), A, nullptr, A, la - 1, nullptr) ==
           MSA_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(msa_workspace_bytes(&d, MSA_ENTRY_INDEX_SCORES) == 0);
    EXPECT(msa_workspace_bytes(&d, 17) == kBad);
  }
}

// Calls that pass every host check reach the launchers (stubbed: each
// reports a launch failure), with workspaces at the minimum, in between and
// at the designed size.
void check_valid_calls_reach_launch() {
  const msa_dims shapes[] = {dims(2, 1000, 1300, 16, 2, 6), dims(3, 1, 5000, 16, 2, 16, 64),
                             dims(1, 16384, 1048576, 64, 8)};
  const float* F = static_cast<const float*>(A);
  const int32_t* I = static_cast<const int32_t*>(A);
  for (const msa_dims& d : shapes) {
    for (int which = 0; which < 3; ++which) {
      const size_t low = msa_workspace_min_bytes(&d, MSA_ENTRY_FORWARD);
      const size_t full = msa_workspace_bytes(&d, MSA_ENTRY_FORWARD);
      const size_t ws = which == 0 ? low : (which == 1 ? (low + full) / 2 : full);
      int before = g_launches;
      EXPECT(msa_forward(&d, A, A, A, A, A, A, nullptr, nullptr, A, ws, nullptr) == MSA_ERR_HIP);
      EXPECT(g_launches == before + 1);
      void* ev[4 + 6 * 1024];
      for (auto& e : ev) e = A;
      const int chunks = msa_attn_chunks(&d, MSA_ENTRY_FORWARD, ws);
      if (4 + 6 * chunks <= 4 + 6 * 1024)
        EXPECT(msa_forward_profiled(&d, A, A, A, A, A, A, nullptr, nullptr, A, ws, nullptr, ev,
                                    4 + 6 * chunks) == MSA_ERR_HIP);
    }
    EXPECT(msa_sparse_attn_fwd(&d, A, A, A, I, A, nullptr, A, kHuge, nullptr) == MSA_ERR_HIP);
    EXPECT(msa_sparse_attn_bwd(&d, A, A, A, I, A, F, A, A, A, A, A, kHuge, nullptr) == MSA_ERR_HIP);
    EXPECT(msa_kl_loss_bwd(&d, A, A, A, A, I, F, F, 1.f, A, A, A, kHuge, nullptr) == MSA_ERR_HIP);
    EXPECT(msa_kl_loss_fwd(&d, A, A, A, A, I, F, nullptr, nullptr, nullptr, A, kHuge, nullptr) == MSA_ERR_HIP);
    EXPECT(msa_index_scores(&d, A, A, static_cast<float*>(A), nullptr) == MSA_ERR_HIP);
  }
  // empty problems launch nothing (except the zero fills that the backward
  // and loss entries write for their key gradients and loss)
  msa_dims e = dims(0, 0, 0, 8, 2);
  const int before = g_launches;
  EXPECT(msa_forward(&e, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                     nullptr) == MSA_OK);
  EXPECT(g_launches == before);
}

}  // namespace

int main() {
  check_dims_rejections();
  check_pointers();
  check_planning();
  check_valid_calls_reach_launch();
  for (int s = 0; s < 8; ++s) EXPECT(msa_status_str(static_cast<msa_status>(s)) != nullptr);
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("abi host check ok\n");
  return 0;
}
