// msa_forward for callers that cannot allocate (include/msa.h): the
// workspace is the library's own file-scope device array `scratch`.
//
// In host code `scratch` names a host-side stand-in, not device memory, so
// its device address is taken once per device with hipGetSymbolAddress
// (with that device current) and kept; only that address is ever passed to
// the kernels.  Each GPU holds its own copy of the array from the first call
// on it until the process ends.  Calls that overlap on one GPU share the
// array and race; every stage clears what it needs with its own kernels, so
// consecutive calls do not depend on what the last one left there.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "msa.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once known

// Device address of the current device's scratch array.
msa_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MSA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MSA_OK;
}

}  // namespace

extern "C" msa_status msa_forward_noalloc(const msa_dims* dims, const void* q, const void* k,
                                          const void* v, const void* q_idx, const void* k_idx,
                                          void* out, float* lse, int32_t* block_idx_out,
                                          void* stream) {
  // Every host check before the first HIP call, as for msa_forward.
  const msa_status st = msa::forward_checks(dims, q, k, v, q_idx, k_idx, out, lse, block_idx_out);
  if (st != MSA_OK) return st;
  if (dims->batch == 0 || dims->seqlen_q == 0) return MSA_OK;
  if (msa_workspace_min_bytes(dims, MSA_ENTRY_FORWARD) > MSA_NOALLOC_SCRATCH_BYTES)
    return MSA_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  const msa_status sst = scratch_of_current_device(&ws);
  if (sst != MSA_OK) return sst;
  return msa_forward(dims, q, k, v, q_idx, k_idx, out, lse, block_idx_out, ws,
                     MSA_NOALLOC_SCRATCH_BYTES, stream);
}
