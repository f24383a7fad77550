// Cache append: each row's new token goes into the indexer-key and latent caches before a
// step reads them (decode reads position n - 1 as the query's own token).
//
// The pages give the indexer's keys only as "FP8" (MarkTechPost, "DeepSeek V3.2-Exp Cuts
// Long-Context Costs with DeepSeek Sparse Attention (DSA) ...", the two-tier pipeline whose
// first tier indexes in FP8); the storage is this library's
// reading: OCP e4m3 codes with one fp32 scale per token, scale = amax / 448 (1 for an
// all-zero key), codes = the key divided by the scale, clamped to +-448 and rounded to
// nearest even.  The latent row (the joint K/V entry of MLA, same article,
// "Instantiation") is stored as given, bf16.
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kAppendRowsPerWg = 4;  // one wave per row

// e4m3 code of a finite |y| <= 448, rounded to nearest with ties to the even code.
// Normal range: the top three fraction bits of the fp32 value, rounded on the 20 bits
// below them (a carry out of the mantissa moves to the next exponent, which is the next
// code).  Below 2^-6 the codes are the multiples of 2^-9, so the code is y * 512 rounded
// to the nearest even integer (8 is the smallest normal, code 0x08).
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  const uint32_t b = __float_as_uint(a);
  const uint32_t e = (b >> 23) - 127u + 7u;
  const uint32_t rem = b & 0xFFFFFu;
  uint32_t code = (e << 3) | ((b >> 20) & 7u);
  if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1;
  return sign | code;
}

__device__ __forceinline__ int64_t cache_row(const int32_t* table, int page_size, int max_pages,
                                             int64_t seq_stride, int seq, int pos) {
  if (table) return (int64_t)table[(int64_t)seq * max_pages + pos / page_size] * page_size + pos % page_size;
  return (int64_t)seq * seq_stride + pos;
}

__global__ __launch_bounds__(kAppendRowsPerWg * WAVE) void cache_append_kernel(
    const float* __restrict__ k_new, const uint16_t* __restrict__ kv_new,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos, int R, int dI,
    int Dqk, uint8_t* __restrict__ kdata, float* __restrict__ kscale, const int32_t* __restrict__ ktable,
    int kps, int kmp, int64_t kstride, uint16_t* __restrict__ vdata,
    const int32_t* __restrict__ vtable, int vps, int vmp, int64_t vstride) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int r = blockIdx.x * kAppendRowsPerWg + (int)(threadIdx.x / WAVE);
  if (r >= R) return;
  const int seq = row_seq[r], pos = row_pos[r];
  const float* x = k_new + (int64_t)r * dI;
  // amax over the key (wave reduction), then the scale in fp32.
  float amax = 0.0f;
  for (int i = lane; i < dI; i += WAVE) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
  const int64_t krow = cache_row(ktable, kps, kmp, kstride, seq, pos);
  uint8_t* kd = kdata + krow * dI;
  for (int i = lane; i < dI; i += WAVE) {
    const float y = fminf(fmaxf(x[i] / scale, -448.0f), 448.0f);
    kd[i] = (uint8_t)e4m3_rne(y);
  }
  if (lane == 0) kscale[krow] = scale;
  // Latent row: 16-byte pieces when the row allows, else 2-byte elements.
  const int64_t vrow = cache_row(vtable, vps, vmp, vstride, seq, pos);
  const uint16_t* src = kv_new + (int64_t)r * Dqk;
  uint16_t* dst = vdata + vrow * Dqk;
  if ((Dqk & 7) == 0) {
    for (int i = lane; i < Dqk / 8; i += WAVE)
      reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
  } else {
    for (int i = lane; i < Dqk; i += WAVE) dst[i] = src[i];
  }
}

}  // namespace

hipError_t launch_cache_append(const float* k_new, const uint16_t* kv_new, const int32_t* row_seq,
                               const int32_t* row_pos, int R, int dI, int Dqk, const CacheView& keys,
                               const CacheView& kv, hipStream_t s) {
  const unsigned grid = (unsigned)((R + kAppendRowsPerWg - 1) / kAppendRowsPerWg);
  cache_append_kernel<<<grid, kAppendRowsPerWg * WAVE, 0, s>>>(
      k_new, kv_new, row_seq, row_pos, R, dI, Dqk,
      static_cast<uint8_t*>(const_cast<void*>(keys.data)), const_cast<float*>(keys.scale), keys.table,
      keys.page_size, keys.max_pages, keys.seq_stride,
      static_cast<uint16_t*>(const_cast<void*>(kv.data)), kv.table, kv.page_size, kv.max_pages,
      kv.seq_stride);
  return hipGetLastError();
}

}  // namespace dsa
