// dsa_read_probe: a streaming-read measurement, not a step of the path.  It reads a device
// buffer once and folds it into one XOR word per workgroup, so the caller can time how fast
// this GPU streams a buffer of a given size -- the practical ceiling that the bandwidth-bound
// indexer scan is compared with -- and check on the host that every byte was read.
//
// Access pattern: every load instruction of a wave reads one contiguous 1 KB (16 bytes per
// lane, non-temporal), eight of them in flight per wave, each wave walking its own contiguous
// stretch of the buffer.  512 workgroups of 512 threads: two per CU, the residency of the
// decode indexer.
#include <hip/hip_runtime.h>

#include "../../include/dsa.h"

namespace {

constexpr int kProbeWgs = 512;
constexpr int kProbeThreads = 512;
constexpr int kProbeWaves = kProbeThreads / 64;
constexpr int kProbeBatch = 8;  // 1 KB loads in flight per wave
typedef int v4i __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const v4i* __restrict__ buf, int64_t nblk,
                                                                   uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Wave g of the grid reads 1 KB blocks [g * per, min((g + 1) * per, nblk)).
  const int64_t nwaves = (int64_t)gridDim.x * kProbeWaves;
  const int64_t per = (nblk + nwaves - 1) / nwaves;
  const int64_t g = (int64_t)blockIdx.x * kProbeWaves + wave;
  const int64_t b0 = g * per;
  const int64_t b1 = b0 + per < nblk ? b0 + per : nblk;
  uint32_t acc = 0;
  for (int64_t b = b0; b < b1; b += kProbeBatch) {
    v4i a[kProbeBatch];
#pragma unroll
    for (int u = 0; u < kProbeBatch; ++u) {
      const int64_t bu = b + u < b1 ? b + u : b1 - 1;  // every load issues; repeats are dropped below
      a[u] = __builtin_nontemporal_load(buf + bu * 64 + lane);
    }
#pragma unroll
    for (int u = 0; u < kProbeBatch; ++u)
      if (b + u < b1) acc ^= (uint32_t)(a[u][0] ^ a[u][1] ^ a[u][2] ^ a[u][3]);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
  __shared__ uint32_t part[kProbeWaves];
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < kProbeWaves; ++i) x ^= part[i];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

extern "C" int dsa_read_probe_sink_words(void) { return kProbeWgs; }

extern "C" dsa_status dsa_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink) return DSA_ERR_NULL;
  if (bytes <= 0 || bytes % 1024 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0) return DSA_ERR_SHAPE;
  read_probe_kernel<<<kProbeWgs, kProbeThreads, 0, stream>>>(static_cast<const v4i*>(buf), bytes / 1024, sink);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}
