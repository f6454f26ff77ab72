// Device-side helpers shared by the gfx950 kernels of the MSA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// D = A * B + C on a 16x16 tile with K = 32 (v_mfma_f32_16x16x32_bf16).
// Lane l supplies A[m = l % 16][k = 8 * (l / 16) + e] and
// B[k = 8 * (l / 16) + e][n = l % 16] for e = 0..7; it receives
// D[m = 4 * (l / 16) + r][n = l % 16] in register r (checked on the device).
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
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

// Calls f(std::integral_constant<int, i>) for i = B .. E - 1 in order: a
// loop whose every index is a compile-time constant.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
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
// Reciprocal of a record's scale m (its largest magnitude): the values are
// stored as fractions or codes of m.  Below 2^-100 they are stored as zero:
// 1 / m of a subnormal m overflows fp32 (and 2047 / m even earlier), which
// would turn the record into inf or NaN, and values this small vanish next to
// any other contribution to a bf16 result.
__device__ __forceinline__ float rec_inv(float m) { return m >= 0x1p-100f ? __builtin_amdgcn_rcpf(m) : 0.f; }

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

// 12-bit codes.  A value x of a row whose largest magnitude is amax is stored
// as round(x * s) + 2048 with s = 2047 / amax, an integer in 1 .. 4095; it
// reads back as (code - 2048) / s, within amax / 4094 of x.
//
// q12_code: fma(x, s, 2^23 + 2048) rounds x * s + 2048 to the nearest integer
// (from 2^23 to 2^24 floats are spaced by 1) and leaves it in the low 12 bits
// of the result; the bits above are the exponent field of 2^23, 0x4B000000,
// which any left shift by 8 or more moves out of the word.
__device__ __forceinline__ uint32_t q12_code(float x, float s) {
  return __float_as_uint(__builtin_fmaf(x, s, 8390656.0f));
}
// Eight codes (from q12_code) into three dwords, code v at bits 12 v .. 12 v + 11
// of the 96-bit word d0 | d1 << 32 | d2 << 64.
__device__ __forceinline__ void q12_pack8(const uint32_t (&c)[8], uint32_t& d0, uint32_t& d1, uint32_t& d2) {
  d0 = (c[0] & 0xFFFu) | (c[1] << 12) | (c[2] << 24);
  d1 = ((c[2] >> 8) & 0xFu) | ((c[3] & 0xFFFu) << 4) | (c[4] << 16) | (c[5] << 28);
  d2 = ((c[5] >> 4) & 0xFFu) | (c[6] << 8) | (c[7] << 20);
}
// The eight codes of d0, d1, d2 (q12_pack8) as floats.
__device__ __forceinline__ void q12_unpack8(uint32_t d0, uint32_t d1, uint32_t d2, float (&y)[8]) {
  const uint32_t c2 = (uint32_t)((((uint64_t)d1 << 32) | d0) >> 24);
  const uint32_t c5 = (uint32_t)((((uint64_t)d2 << 32) | d1) >> 28);
  y[0] = (float)(d0 & 0xFFFu);
  y[1] = (float)((d0 >> 12) & 0xFFFu);
  y[2] = (float)(c2 & 0xFFFu);
  y[3] = (float)((d1 >> 4) & 0xFFFu);
  y[4] = (float)((d1 >> 16) & 0xFFFu);
  y[5] = (float)(c5 & 0xFFFu);
  y[6] = (float)((d2 >> 8) & 0xFFFu);
  y[7] = (float)(d2 >> 20);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Cross-lane exchanges without LDS traffic.
//
// swap32(a, b): lanes 32..63 of a trade places with lanes 0..31 of b
// (v_permlane32_swap): afterwards a = (a[0..31], b[0..31]) and
// b = (a[32..63], b[32..63]).  So a + b holds the two halves' sum of the old a
// in lanes 0..31 and of the old b in lanes 32..63.
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// max and sum of x over lanes l and l ^ 32, in every lane (one
// v_permlane32_swap instead of a ds_bpermute round trip).
__device__ __forceinline__ float halves_max(float x) {
  float a = x, b = x;
  swap32(a, b);
  return __builtin_fmaxf(a, b);
}
__device__ __forceinline__ float halves_sum(float x) {
  float a = x, b = x;
  swap32(a, b);
  return a + b;
}

// swap16(a, b): the odd 16-lane rows of a trade places with the even rows of
// b (v_permlane16_swap): afterwards a = (a.r0, b.r0, a.r2, b.r2) and
// b = (a.r1, b.r1, a.r3, b.r3).
__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Value of x in the lane that the DPP control `ctl` selects (within a row).
template <int ctl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctl, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7 - i within each 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15 - i within each row

// Sum / max over the 16 lanes of each row, in every lane of the row.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v + dpp<kDppMirror>(v);
}
__device__ __forceinline__ float row_max16(float v) {
  v = __builtin_fmaxf(v, dpp<kDppXor1>(v));
  v = __builtin_fmaxf(v, dpp<kDppXor2>(v));
  v = __builtin_fmaxf(v, dpp<kDppHalfMirror>(v));
  return __builtin_fmaxf(v, dpp<kDppMirror>(v));
}

// Reductions of several values at once over 32 or 64 lanes, built from the
// swaps above.  scatter32<N>: element i < N/2 becomes the two halves' total
// (sum, or max when MAX) of element i in lanes 0..31 and of element i + N/2
// in lanes 32..63.  scatter16<N>: the same across each pair of rows (rows 0, 1
// and rows 2, 3): element i + (N/2) * (row & 1) in the result.  gather32 and
// gather16 undo the split of an already reduced vector, so every lane holds
// all N elements.  allred32 / allred16 combine one value across the halves /
// row pairs.
template <bool MAX>
__device__ __forceinline__ float combine(float a, float b) { return MAX ? __builtin_fmaxf(a, b) : a + b; }

template <int N, bool MAX>
__device__ __forceinline__ void scatter32(float* v) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    float a = v[i], b = v[i + N / 2];
    swap32(a, b);
    v[i] = combine<MAX>(a, b);
  }
}
template <int N, bool MAX>
__device__ __forceinline__ void scatter16(float* v) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    float a = v[i], b = v[i + N / 2];
    swap16(a, b);
    v[i] = combine<MAX>(a, b);
  }
}
template <int N>
__device__ __forceinline__ void gather32(float* v) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    float a = v[i], b = v[i];
    swap32(a, b);
    v[i] = a;
    v[i + N / 2] = b;
  }
}
template <int N>
__device__ __forceinline__ void gather16(float* v) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    float a = v[i], b = v[i];
    swap16(a, b);
    v[i] = a;
    v[i + N / 2] = b;
  }
}
template <bool MAX>
__device__ __forceinline__ float allred32(float x) {
  float a = x, b = x;
  swap32(a, b);
  return combine<MAX>(a, b);
}
template <bool MAX>
__device__ __forceinline__ float allred16(float x) {
  float a = x, b = x;
  swap16(a, b);
  return combine<MAX>(a, b);
}

// Chunk swizzle of the staged rows: distinct chunks both for 16 consecutive
// rows (the MFMA operand reads) and for 16 rows of one parity (the staging
// writes), so neither conflicts on LDS banks.
__device__ __forceinline__ int rsw(int r) { return ((r >> 1) ^ ((r & 1) << 3)) & 15; }

// Transposing LDS read (ds_read_b64_tr_b16): each lane names 4 consecutive
// bf16 values; within each group of 16 lanes, lane i receives, as element e,
// value i % 4 of those named by lane 4 e + i / 4.  So when lane i of a group
// names row r0 + i / 4, columns c0 + 4 (i % 4) .. + 3 of a row-major tile,
// lane i receives rows r0 .. r0 + 3 of column c0 + i: a 4 x 16 block read
// transposed (checked on the device: lane i gets elements i, i + 16, i + 32,
// i + 48 of a 64-element run).
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const void* lds_addr) {
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)lds_addr);
  return __builtin_bit_cast(uint2, r);
}

// Byte offset of element (row, col) in a row-major bf16 tile of CH 16-byte
// chunks per row (CH * 8 columns), chunk c of a row stored at c ^ sw.
template <int CH = 16>
__device__ __forceinline__ int lds_tile_off(int row, int col, int sw) {
  return row * (16 * CH) + 16 * ((col >> 3) ^ sw) + 2 * (col & 7);
}

// Order-preserving unsigned key of a float: a < b (non-NaN) iff key(a) < key(b).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace msa
