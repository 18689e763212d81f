// Device helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D = A(32x16) * B(16x32) + C on the matrix cores, bf16 in, fp32 accumulate.
// Lane l (r = l % 32, g = l / 32) supplies A[r][8g .. 8g+7] and B[8g .. 8g+7][r];
// result element j of lane l is C[8*(j/4) + 4*g + j%4][r].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS transposing read of four 16-bit values.  Within each group of 16 lanes,
// element e of lane i comes from the 8-byte chunk addressed by lane 4*e + i/4,
// at position i % 4.  Four lanes pointing at consecutive 4-element chunks of
// one row therefore hand out that row's 16 values one per lane.
__device__ __forceinline__ i16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// Two transposing reads forming one 8-value MFMA operand.
__device__ __forceinline__ bf16x8 lds_read_tr8(const uint16_t* p0, const uint16_t* p1) {
  i16x4 a = lds_read_tr(p0);
  i16x4 b = lds_read_tr(p1);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Combine a per-lane value with the one held 32 lanes away (the other half of
// the wavefront).  permlane32_swap(x, x) returns {own, other} in the lower half
// and {other, own} in the upper half, so any symmetric operation of the pair
// is the cross-half result in every lane.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float from_bf16(uint16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                        float a6, float a7) {
  u32x4 u = {pack_bf16x2(a0, a1), pack_bf16x2(a2, a3), pack_bf16x2(a4, a5), pack_bf16x2(a6, a7)};
  return __builtin_bit_cast(bf16x8, u);
}

// Workgroups are handed to the 8 XCDs round-robin (id % 8).  This maps the
// hardware id to a logical id so that consecutive logical ids run on the same
// XCD and share its L2.  Identity when the grid is not a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  constexpr int X = 8;
  if (nwg % X) return bid;
  return (bid % X) * (nwg / X) + bid / X;
}

}  // namespace mi355
