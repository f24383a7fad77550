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

// Hand-off of the sampled long-row top-k between its passes (and from the compacting indexer).
struct RowHeader {
  uint32_t theta;  // sample threshold key of a long row
  uint32_t shift;  // survivor bin of key = min((key - theta) >> shift, 4095)
};
struct ChunkCount {
  uint32_t gt;     // survivors of a chunk above theta
  uint32_t eq;     // survivors of a chunk equal to theta
  uint32_t theta;  // the threshold the chunk was compacted with
  uint32_t pad;
};
// A row threshold published inside the compacting indexer: (kThetaReady << 32) | theta.
constexpr uint32_t kThetaReady = 0x7E7A5EEDu;

// ---- indexer
// Calls with at least this many rows use the many-rows kernel.
int index_rows_kernel_min();
// Keys per workgroup (the compaction chunk) of the one-row-per-workgroup indexer for R rows
// of at most n_bound keys.
int index_keys_per_wg(int R, int64_t n_bound);
hipError_t launch_index_fp8_h64d128(const uint8_t* q, const float* q_scale, const float* w,
                                    const CacheView& keys, const int32_t* row_seq,
                                    const int32_t* row_pos, int R, int64_t n_bound, float* scores,
                                    int64_t ld, hipStream_t s);
// Chunks per row of the compacting indexer for R rows of at most n_bound keys; chunk c starts
// at key 64 * (c * tb / nc), tb = ceil(n_bound / 64).
int index_compact_chunks(int R, int64_t n_bound);
// Scores rows longer than min_n without storing them.  R extra workgroups score each row's
// sample and publish its threshold (hdr[r], and the word ready[r] the scoring workgroups poll);
// the survivors of that threshold go to the chunk slots of cand [R, ld] with per-chunk counts
// [R, index_compact_chunks(R, n_bound)].  ready[r] must not hold a published word of an earlier call
// (the resolve clears it); if it does, chunks may be compacted with a stale threshold, which
// the resolve detects (ChunkCount::theta) and answers by rescoring the row.
hipError_t launch_index_fp8_compact(const uint8_t* q, const float* q_scale, const float* w,
                                    const CacheView& keys, const int32_t* row_seq,
                                    const int32_t* row_pos, int R, int64_t n_bound, int64_t ld,
                                    RowHeader* hdr, uint64_t* ready, ChunkCount* counts, uint2* cand,
                                    int min_n, hipStream_t s);
hipError_t launch_index_generic(bool fp8, const void* q, const float* q_scale, const float* w,
                                const CacheView& keys, const int32_t* row_seq, const int32_t* row_pos,
                                int R, int HI, int dI, int64_t n_bound, float* scores, int64_t ld,
                                hipStream_t s);

// ---- top-k
size_t topk_workspace_bytes(int R, int64_t ld, int k);
// False when R rows of length ld need more blocks than one launch can take.
bool topk_shape_ok(int R, int64_t ld);
// Row r has n_valid[r] + n_off scores.
hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* n_valid, int R, int k,
                       int32_t* idx, void* ws, hipStream_t s, int n_off = 0);
// Rows longer than this use the sampled compaction, for score rows of leading dimension ld.
int topk_long_row_min(int64_t ld);

// ---- fused index + top-k, fast indexer shape (64 heads x 128, e4m3): sample pass, compacting
// indexer, resolve -- no score row is stored.  Rows are row_pos[r] + 1 keys long, ld >= each.
size_t index_topk_fused_bytes(int R, int64_t ld);
bool index_topk_fused_ok(int R, int64_t ld);
hipError_t launch_index_topk_fused(const uint8_t* q, const float* q_scale, const float* w, const CacheView& keys,
                                   const int32_t* row_seq, const int32_t* row_pos, int R, int64_t ld, int k,
                                   int32_t* idx, void* ws, hipStream_t s);

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
