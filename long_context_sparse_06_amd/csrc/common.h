// Device helpers shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4bf lds_v4bf;

constexpr int WAVE = 64;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

// Number of set bits of a 64-bit wave mask strictly below this lane.
__device__ __forceinline__ int mask_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Order-preserving map fp32 -> u32 (larger float -> larger key); -0.0 is mapped like +0.0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// bf16 bits -> fp32 and fp32 -> bf16 bits (round to nearest even; inputs are finite).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP e4m3fn code -> fp32 (bias 7, subnormals, max 448).  Codes 0x7F/0xFF (NaN) never occur.
__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  const uint32_t e = (c >> 3) & 0xF, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80) ? -mag : mag;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Address of logical row s of sequence b in a contiguous or paged cache (width in elements).
template <typename T>
__device__ __forceinline__ const T* cache_row(const T* base, const int32_t* table, int max_pages,
                                              int page_size, int64_t seq_stride, int b, int64_t s,
                                              int width) {
  int64_t row;
  if (table) {
    const int32_t page = table[(int64_t)b * max_pages + s / page_size];
    row = (int64_t)page * page_size + s % page_size;
  } else {
    row = (int64_t)b * seq_stride + s;
  }
  return base + row * width;
}

}  // namespace dsa
