// Device-side helpers shared by the layout and row kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// One 16-byte chunk of a row: 4 fp32 or 8 bf16 elements.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum : int { kF32 = 0, kBF16 = 1 };

template <int DT>
struct Elems {
  static constexpr int kPerChunk = DT == kF32 ? 4 : 8;  // elements per 16-byte chunk
};

// bfloat16 -> float32 is exact: bf16 is the upper half of a binary32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bfloat16 bits, round to nearest, ties to even.  Adds 0x7FFF plus
// the lowest kept bit, then drops the low half; NaNs are made quiet and keep
// their sign and top payload bits.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (b >> 16) | 0x40u;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Unpack a chunk into its float32 elements (in memory order).
template <int DT>
__device__ __forceinline__ void unpack(const u32x4 c, float* f) {
  if constexpr (DT == kF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(c[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(c[i]);
      f[2 * i + 1] = bf16_hi(c[i]);
    }
  }
}

// Pack float32 elements into a chunk, rounding to the row type.
template <int DT>
__device__ __forceinline__ u32x4 pack(const float* f) {
  u32x4 c;
  if constexpr (DT == kF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = __float_as_uint(f[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  }
  return c;
}

template <bool NT>
__device__ __forceinline__ void store_chunk(u32x4* p, const u32x4 v) {
  if constexpr (NT) {
    __builtin_nontemporal_store(v, p);
  } else {
    *p = v;
  }
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ int read_lane_i(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}

__device__ __forceinline__ float read_lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Fold the 64 lane partials: for s = 32, 16, ..., 1 every lane adds the
// partial of lane (l xor s).  float32 addition is commutative, so every lane
// ends with the same value, the one partial 0 holds.
__device__ __forceinline__ float fold64(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    float o = __shfl_xor(v, s, kWave);
    v = __fadd_rn(v, o);
  }
  return v;
}

}  // namespace moe
