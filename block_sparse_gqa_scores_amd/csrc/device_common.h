// Device-side helpers shared by the gfx950 kernels of the MSA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// D = A * B + C on a 32x32 tile with K = 16 (v_mfma_f32_32x32x16_bf16).
// Lane l supplies A[m = l % 32][k = 8 * (l / 32) + e] and
// B[k = 8 * (l / 32) + e][n = l % 32] for e = 0..7; it receives
// D[m = 8 * (r / 4) + 4 * (l / 32) + (r % 4)][n = l % 32] in register r.
// Only the pairing of A and B along k matters for the result, so any
// consistent assignment of k to (lane half, e) on both operands is valid.
__device__ __forceinline__ f32x16 mfma32x32x16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Row index (within a 32x32 MFMA output tile) held by register r of lane l.
__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// max(a, b, c): the compiler fuses the two maxima into one v_max3_f32.  This
// is written with the compiler's max, not inline assembly: the compiler then
// sees where the operands come from and inserts the wait states that a vector
// ALU read of a fresh MFMA result requires (it cannot do so for an assembly
// operand, and a read too early returns the register's previous contents).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// Max of the 16 values of an MFMA 32x32 output register block and `m`.
__device__ __forceinline__ float max16(float m, const f32x16& x) {
  const float a = max3f(x[0], x[1], x[2]);
  const float b = max3f(x[3], x[4], x[5]);
  const float c = max3f(x[6], x[7], x[8]);
  const float d = max3f(x[9], x[10], x[11]);
  const float e = max3f(x[12], x[13], x[14]);
  return max3f(max3f(a, b, c), max3f(d, e, x[15]), m);
}

// max(|a|, |b|, c): one v_max3_f32 with abs source modifiers (see max3f).
__device__ __forceinline__ float max3abs(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a), __builtin_fabsf(b)), c);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z = {};
  return z;
}

// Value of `x` held by lane (l ^ 32).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest-even bf16, packed low|high
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Two fp32 values rounded to nearest-even fp16, packed low|high
// (one v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Order-preserving unsigned key of a float: a < b (non-NaN) iff key(a) < key(b).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace msa
