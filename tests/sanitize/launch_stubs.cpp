// Host-only stand-ins for the device launchers of libmsa, for the sanitizer
// build of the C-ABI host code (msa_api.cpp + plan.cpp, built with g++ and
// -fsanitize=address,undefined).  Test infrastructure: nothing is launched;
// each stub counts its call and reports a launch failure, so a call that
// passes every host check returns MSA_ERR_HIP.  hipEventRecord is stubbed
// too, so the check needs no HIP runtime and no GPU.
#include <hip/hip_runtime.h>

#include "kernels.h"

int g_launches = 0;

namespace msa {

hipError_t launch_index_scores(const uint16_t*, const uint16_t*, float*, int, int, int, int, int, int,
                               hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_index_select(const uint16_t*, const uint16_t*, int32_t*, int, int, int, int, int, int,
                               int, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_block_topk(const float*, int32_t*, int, int, int, int, int, int, hipStream_t) {
  ++g_launches;
  return hipErrorInvalidValue;
}
hipError_t launch_block_mask(const int32_t*, uint32_t*, long, int, int, hipStream_t) {
  ++g_launches;
  return hipErrorInvalidValue;
}
hipError_t launch_mask_blocks(const uint32_t*, int32_t*, long, int, int, hipStream_t) {
  ++g_launches;
  return hipErrorInvalidValue;
}
hipError_t launch_sparse_attn(const AttnShape&, const uint16_t*, const uint16_t*, const uint16_t*,
                              const int32_t*, uint16_t*, float*, void*, size_t, hipStream_t,
                              const StageEvents*) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_sparse_attn_bwd(const AttnShape&, const uint16_t*, const uint16_t*, const uint16_t*,
                                  const int32_t*, const uint16_t*, const float*, const uint16_t*, uint16_t*,
                                  uint16_t*, uint16_t*, void*, size_t, hipStream_t) {
  ++g_launches;
  return hipErrorInvalidValue;
}
hipError_t launch_kl_loss_bwd(const AttnShape&, int, const uint16_t*, const uint16_t*, const uint16_t*,
                              const uint16_t*, const int32_t*, const float*, const float*, float, uint16_t*,
                              uint16_t*, void*, size_t, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_backward(const AttnShape&, int, const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                           const uint16_t*, const int32_t*, const uint16_t*, const float*, const float*,
                           const uint16_t*, float, uint16_t*, uint16_t*, uint16_t*, uint16_t*, uint16_t*, void*,
                           size_t, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_fill_zero(float*, long, hipStream_t) { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_kl_loss(const AttnShape&, int, const uint16_t*, const uint16_t*, const uint16_t*,
                          const uint16_t*, const int32_t*, const float*, float*, float*, float*, void*, size_t,
                          hipStream_t) { ++g_launches; return hipErrorInvalidValue; }

}  // namespace msa

extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
