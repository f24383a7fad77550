// Host-side launchers of the DSA kernels (internal; the public ABI is include/dsa.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct CacheView {
  const void* data;
  const float* scale;
  const int32_t* table;
  int page_size;
  int max_pages;
  int64_t seq_stride;
};

// ---- indexer
// samp (optional): rows longer than samp_min_n also store their 2048 evenly spaced sample
// scores contiguously in samp[R, 2048] (positions (i * n) / 2048); the rows kernel for many
// rows is not used then.
// Calls with at least this many rows (and no sample wanted) use the many-rows kernel.
int index_rows_kernel_min();
hipError_t launch_index_fp8_h64d128(const uint8_t* q, const float* q_scale, const float* w,
                                    const CacheView& keys, const int32_t* row_seq,
                                    const int32_t* row_pos, int R, int64_t n_bound, float* scores,
                                    int64_t ld, hipStream_t s, float* samp = nullptr,
                                    int samp_min_n = 0);
hipError_t launch_index_generic(bool fp8, const void* q, const float* q_scale, const float* w,
                                const CacheView& keys, const int32_t* row_seq, const int32_t* row_pos,
                                int R, int HI, int dI, int64_t n_bound, float* scores, int64_t ld,
                                hipStream_t s);

// ---- top-k
size_t topk_workspace_bytes(int R, int64_t ld, int k);
// False when R rows of length ld need more blocks than one launch can take.
bool topk_shape_ok(int R, int64_t ld);
// samp (optional): each long row's 2048 sample scores, contiguous (see the indexer);
// the rows' lengths are n_valid[r] + n_off.
hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* n_valid, int R, int k,
                       int32_t* idx, void* ws, hipStream_t s, const float* samp = nullptr,
                       int n_off = 0);
// Rows longer than this use the sampled compaction (and so want the indexer's sample), for
// score rows of leading dimension ld.
int topk_long_row_min(int64_t ld);

// ---- sparse MLA
size_t mla_decode_workspace_bytes(int B, int H, int Dv, int k);
int mla_max_tokens_per_wg();  // longest kept set one bf16 workgroup holds (prefill: k limit)
hipError_t launch_mla_bf16(const uint16_t* q, const CacheView& kv, const int32_t* idx, int R,
                           int H, int k, bool decode, float scale, uint16_t* out, float* lse,
                           void* ws, size_t ws_bytes, hipStream_t s);
// Prefill attention in its dense "masked" form: row t over positions 0..t, masked to idx[t, :].
hipError_t launch_mla_bf16_masked(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int T,
                                  int H, int k, float scale, uint16_t* out, float* lse, hipStream_t s);
hipError_t launch_mla_generic(bool bf16, const void* q, const CacheView& kv, const int32_t* idx,
                              int R, int H, int Dqk, int Dv, int k, bool decode, float scale,
                              void* out, float* lse, hipStream_t s);

// ---- cache append (writes through keys.data / keys.scale / kv.data)
hipError_t launch_cache_append(const float* k_new, const uint16_t* kv_new, const int32_t* row_seq,
                               const int32_t* row_pos, int R, int dI, int Dqk, const CacheView& keys,
                               const CacheView& kv, hipStream_t s);

// ---- indexer-quality diagnostic
size_t quality_workspace_bytes(int R, int H, int64_t ld);
hipError_t launch_indexer_quality(const uint16_t* q, const CacheView& kv, const float* scores,
                                  int64_t sld, const int32_t* idx, int k, const int32_t* row_seq,
                                  const int32_t* row_pos, int R, int H, int Dqk, int64_t ld,
                                  float scale, float* kl, float* recall, float* kl_rev, void* ws,
                                  hipStream_t s);

}  // namespace dsa
