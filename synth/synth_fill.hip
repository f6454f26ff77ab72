// Device fill kernels of the seeded synthetic inputs.
//
// This file holds no part of the attention method: it only writes the
// pseudo-random test tensors, so that the 68 GiB decode cache and the 1M-token
// prefix never have to cross PCIe.  It is an independent implementation of
// the same generator that synth/__init__.py implements on the host with
// numpy; the two share no code.
//
// Generator (both sides implement it from these published definitions):
//   counter(e)  = seed XOR (tensor_id << 40) XOR e             (64-bit)
//   x           = splitmix64(counter)   -- Steele, Lea and Flood, "Fast
//                 splittable pseudorandom number generators" (OOPSLA 2014),
//                 finaliser constants as published with Vigna's splitmix64.c
//   u(e)        = (x >> 11) * 2^-53                             in [0, 1)
//   integer     = floor(7 u) - 3                                in {-3..3}
//   normal(e)   = Box-Muller (Box and Muller, 1958) on the pair (2m, 2m+1),
//                 m = e >> 1:  r = sqrt(-2 ln(1 - u(2m))), th = 2 pi u(2m+1);
//                 r cos th for even e, r sin th for odd e      (fp64)
//   stored bf16 = round-to-nearest-even of the fp32 value (float)z.
//   Optional per-block gain (uneven block scores): g_j = exp(0.5 normal_6(j))
//   for key block j; a normal element becomes (float)(g_j z); an integer
//   element becomes rint_half_even(g_j * integer).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ double uniform01(uint64_t seed, uint32_t tid,
                                            uint64_t e) {
  uint64_t c = seed ^ ((uint64_t)tid << 40) ^ e;
  return (double)(splitmix64(c) >> 11) * 0x1.0p-53;
}

__device__ __forceinline__ double normal_at(uint64_t seed, uint32_t tid,
                                            uint64_t e) {
  uint64_t m = e >> 1;
  double u1 = uniform01(seed, tid, 2 * m);
  double u2 = uniform01(seed, tid, 2 * m + 1);
  double r = sqrt(-2.0 * log(1.0 - u1));
  double th = 6.283185307179586476925286766559 * u2;
  return (e & 1) ? r * sin(th) : r * cos(th);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  uint32_t lsb = (b >> 16) & 1u;
  b += 0x7FFFu + lsb;
  return (uint16_t)(b >> 16);
}

constexpr uint32_t kGainTensor = 6;

struct Geometry {
  int64_t elems_per_token;  // elements of one token row (H * D)
  int64_t tokens_per_seq;   // S
  int64_t block;            // tokens per gain block (0: no gain)
};

__device__ __forceinline__ double gain_of(uint64_t seed, Geometry g,
                                          uint64_t e) {
  int64_t tok = (int64_t)(e / (uint64_t)g.elems_per_token) % g.tokens_per_seq;
  int64_t j = tok / g.block;
  return exp(0.5 * normal_at(seed, kGainTensor, (uint64_t)j));
}

__global__ void fill_normal_kernel(uint16_t* __restrict__ dst, int64_t n,
                                   uint64_t seed, uint32_t tid, Geometry geo) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += stride) {
    double z = normal_at(seed, tid, (uint64_t)e);
    if (geo.block > 0) z *= gain_of(seed, geo, (uint64_t)e);
    dst[e] = f32_to_bf16_rne((float)z);
  }
}

__global__ void fill_int_kernel(uint16_t* __restrict__ dst, int64_t n,
                                uint64_t seed, uint32_t tid, Geometry geo) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += stride) {
    double u = uniform01(seed, tid, (uint64_t)e);
    double v = floor(7.0 * u) - 3.0;
    if (geo.block > 0) v = rint(v * gain_of(seed, geo, (uint64_t)e));
    dst[e] = f32_to_bf16_rne((float)v);
  }
}

// Plain copy of n16 16-byte words (a known-size memory stream used to
// calibrate hardware traffic counters).
__global__ void copy16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n16) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n16; e += stride)
    dst[e] = src[e];
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" {

// Fill dst[0 .. n) with bf16 N(0,1) draws of tensor `tensor_id`.  When
// gain_block > 0, element e is scaled by the gain of key block
// ((e / elems_per_token) % tokens_per_seq) / gain_block.  Returns 0 or the
// hipError_t of the launch.
int synth_fill_normal_bf16(void* dst, int64_t n, uint64_t seed,
                           uint32_t tensor_id, int64_t elems_per_token,
                           int64_t tokens_per_seq, int64_t gain_block,
                           void* stream) {
  if (n <= 0) return 0;
  Geometry geo{elems_per_token > 0 ? elems_per_token : 1,
               tokens_per_seq > 0 ? tokens_per_seq : 1, gain_block};
  hipLaunchKernelGGL(fill_normal_kernel, dim3(grid_for(n)), dim3(256), 0,
                     (hipStream_t)stream, (uint16_t*)dst, n, seed, tensor_id,
                     geo);
  return (int)hipGetLastError();
}

// Fill dst[0 .. n) with bf16 integers uniform in {-3..3} of tensor
// `tensor_id`, optionally scaled by the block gain and rounded half-to-even.
int synth_fill_int_bf16(void* dst, int64_t n, uint64_t seed, uint32_t tensor_id,
                        int64_t elems_per_token, int64_t tokens_per_seq,
                        int64_t gain_block, void* stream) {
  if (n <= 0) return 0;
  Geometry geo{elems_per_token > 0 ? elems_per_token : 1,
               tokens_per_seq > 0 ? tokens_per_seq : 1, gain_block};
  hipLaunchKernelGGL(fill_int_kernel, dim3(grid_for(n)), dim3(256), 0,
                     (hipStream_t)stream, (uint16_t*)dst, n, seed, tensor_id,
                     geo);
  return (int)hipGetLastError();
}

// Copy `bytes` (a multiple of 16) from src to dst on `stream`: a plain
// streaming kernel that reads and writes exactly `bytes` each.
int synth_copy_bytes(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes <= 0 || (bytes & 15)) return bytes == 0 ? 0 : -1;
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(copy16_kernel, dim3(grid_for(n16)), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, (uint4*)dst, n16);
  return (int)hipGetLastError();
}

}  // extern "C"
