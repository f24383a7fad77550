// dsa_sparse_mla_decode_noalloc: the decode attention with its split partials in a static
// device array instead of a caller workspace, for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this file; host code never passes its name to a kernel (on the host the
// name is only a stand-in): each device's address of it is looked up once, with that device
// current, and kept in a per-device table.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dsa.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per device
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// This device's address of `scratch` (nullptr and an error code if the lookup failed).
void* scratch_ptr(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *err = g_err[dev];
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t dsa_noalloc_scratch_bytes(void) { return kScratchBytes; }

dsa_status dsa_sparse_mla_decode_noalloc(dsa_dtype dt, const void* q, const dsa_cache* kv,
                                         const int32_t* idx, int B, int H, int Dqk, int Dv, int k,
                                         float softmax_scale, void* out, float* lse,
                                         hipStream_t stream) {
  if (!q || !kv || !kv->data || !idx || !out) return DSA_ERR_NULL;
  if (B <= 0 || H <= 0 || Dqk <= 0 || Dv <= 0 || k <= 0) return DSA_ERR_SHAPE;
  const size_t need = dsa_sparse_mla_decode_workspace_size(B, H, Dv, k);
  if (need > kScratchBytes) return DSA_ERR_WORKSPACE;
  hipError_t e = hipSuccess;
  void* ws = scratch_ptr(&e);
  if (!ws) return DSA_ERR_LAUNCH;
  return dsa_sparse_mla_decode(dt, q, kv, idx, B, H, Dqk, Dv, k, softmax_scale, out, lse, ws,
                               kScratchBytes, stream);
}

}  // extern "C"
