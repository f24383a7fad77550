// C ABI of the DSA hot path (declared in include/dsa.h): host-side validation and
// dispatch to the gfx950 kernels.  Nothing here allocates, frees or synchronises.
#include "../../include/dsa.h"

#include "kernels.h"

namespace {

dsa::CacheView view(const dsa_cache* c) {
  return dsa::CacheView{c->data, c->scale, c->block_table, c->page_size, c->max_pages, c->seq_stride};
}

// Longest sequence a cache can hold; 0 if the descriptor is malformed.
int64_t cache_capacity(const dsa_cache* c) {
  if (c->block_table) {
    if (c->page_size <= 0 || c->max_pages <= 0) return 0;
    return (int64_t)c->page_size * c->max_pages;
  }
  return c->seq_stride > 0 ? c->seq_stride : 0;
}

dsa_status launched(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE";
    case DSA_ERR_DTYPE: return "DSA_ERR_DTYPE";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_LAUNCH: return "DSA_ERR_LAUNCH";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_RANGE: return "DSA_ERR_RANGE";
  }
  return "DSA_ERR_UNKNOWN";
}

dsa_status dsa_index_scores(dsa_dtype dt, const void* q, const float* q_scale, const float* w,
                            const dsa_cache* keys, const int32_t* row_seq, const int32_t* row_pos,
                            int R, int H_I, int d_I, float* scores, int64_t ld, hipStream_t stream) {
  if (!q || !w || !keys || !keys->data || !row_seq || !row_pos || !scores) return DSA_ERR_NULL;
  if (dt != DSA_E4M3 && dt != DSA_F32) return DSA_ERR_DTYPE;
  if (R <= 0 || H_I <= 0 || d_I <= 0 || R > 65535) return DSA_ERR_SHAPE;
  const int64_t cap = cache_capacity(keys);
  if (cap <= 0 || ld < cap) return DSA_ERR_SHAPE;
  if ((int64_t)H_I * d_I > 16384) return DSA_ERR_UNSUPPORTED;
  const dsa::CacheView kv = view(keys);
  if (dt == DSA_E4M3 && H_I == 64 && d_I == 128)
    return launched(dsa::launch_index_fp8_h64d128(static_cast<const uint8_t*>(q), q_scale, w, kv,
                                                  row_seq, row_pos, R, cap, scores, ld, stream));
  return launched(dsa::launch_index_generic(dt == DSA_E4M3, q, q_scale, w, kv, row_seq, row_pos, R,
                                            H_I, d_I, cap, scores, ld, stream));
}

size_t dsa_topk_workspace_size(int R, int64_t ld, int k) {
  if (R <= 0 || ld <= 0 || k <= 0) return 0;
  return dsa::topk_workspace_bytes(R, ld, k);
}

dsa_status dsa_topk(const float* scores, int64_t ld, const int32_t* n_valid, int R, int k,
                    int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!scores || !n_valid || !idx) return DSA_ERR_NULL;
  if (R <= 0 || k <= 0 || ld <= 0 || k > 16384 || ld > (int64_t(1) << 24) || R > 2147483647 / 2 ||
      !dsa::topk_shape_ok(R, ld))
    return DSA_ERR_SHAPE;
  const size_t need = dsa::topk_workspace_bytes(R, ld, k);
  if (need > 0 && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
  return launched(dsa::launch_topk(scores, ld, n_valid, R, k, idx, ws, stream));
}

size_t dsa_sparse_mla_decode_workspace_size(int B, int H, int Dv, int k) {
  if (B <= 0 || H <= 0 || Dv <= 0 || k <= 0) return 0;
  return dsa::mla_decode_workspace_bytes(B, H, Dv, k);
}

static dsa_status mla_check(dsa_dtype dt, const void* q, const void* kv, const int32_t* idx, int R,
                            int H, int Dqk, int Dv, int k, void* out) {
  if (!q || !kv || !idx || !out) return DSA_ERR_NULL;
  if (dt != DSA_BF16 && dt != DSA_F32) return DSA_ERR_DTYPE;
  if (R <= 0 || H <= 0 || Dqk <= 0 || Dv <= 0 || k <= 0 || Dv > Dqk) return DSA_ERR_SHAPE;
  if ((int64_t)R * H > 2147483647LL) return DSA_ERR_SHAPE;
  return DSA_OK;
}

static bool mla_fast(dsa_dtype dt, int H, int Dqk, int Dv) {
  return dt == DSA_BF16 && Dqk == 576 && Dv == 512 && H % 64 == 0;
}

static dsa_status mla_generic_ok(int Dqk, int k) {
  // logits of one (row, head) and the query row sit in LDS
  return ((size_t)Dqk + k + 8) * sizeof(float) <= 64 * 1024 && Dqk <= 1024 ? DSA_OK : DSA_ERR_UNSUPPORTED;
}

dsa_status dsa_sparse_mla_decode(dsa_dtype dt, const void* q, const dsa_cache* kv, const int32_t* idx,
                                 int B, int H, int Dqk, int Dv, int k, float softmax_scale, void* out,
                                 float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!kv) return DSA_ERR_NULL;
  dsa_status st = mla_check(dt, q, kv->data, idx, B, H, Dqk, Dv, k, out);
  if (st != DSA_OK) return st;
  if (cache_capacity(kv) <= 0) return DSA_ERR_SHAPE;
  const dsa::CacheView v = view(kv);
  if (mla_fast(dt, H, Dqk, Dv)) {
    const size_t need = dsa::mla_decode_workspace_bytes(B, H, Dv, k);
    if (need > 0 && (!ws || ws_bytes < need)) return DSA_ERR_WORKSPACE;
    return launched(dsa::launch_mla_bf16(static_cast<const uint16_t*>(q), v, idx, B, H, k, true,
                                         softmax_scale, static_cast<uint16_t*>(out), lse, ws, ws_bytes,
                                         stream));
  }
  if ((st = mla_generic_ok(Dqk, k)) != DSA_OK) return st;
  return launched(dsa::launch_mla_generic(dt == DSA_BF16, q, v, idx, B, H, Dqk, Dv, k, true,
                                          softmax_scale, out, lse, stream));
}

dsa_status dsa_sparse_mla_prefill(dsa_dtype dt, const void* q, const void* kv, const int32_t* idx,
                                  int T, int H, int Dqk, int Dv, int k, float softmax_scale, void* out,
                                  float* lse, hipStream_t stream) {
  dsa_status st = mla_check(dt, q, kv, idx, T, H, Dqk, Dv, k, out);
  if (st != DSA_OK) return st;
  const dsa::CacheView v{kv, nullptr, nullptr, 0, 0, (int64_t)T};
  if (mla_fast(dt, H, Dqk, Dv)) {
    if (k > dsa::mla_max_tokens_per_wg()) return DSA_ERR_UNSUPPORTED;
    return launched(dsa::launch_mla_bf16(static_cast<const uint16_t*>(q), v, idx, T, H, k, false,
                                         softmax_scale, static_cast<uint16_t*>(out), lse, nullptr, 0,
                                         stream));
  }
  if ((st = mla_generic_ok(Dqk, k)) != DSA_OK) return st;
  return launched(dsa::launch_mla_generic(dt == DSA_BF16, q, v, idx, T, H, Dqk, Dv, k, false,
                                          softmax_scale, out, lse, stream));
}

namespace {
// The fused call on the fast indexer shape with few, long rows (decode) stores no score row:
// the compacting indexer with its sample workgroups, then the resolve
// (dsa::launch_index_topk_fused).  Other calls (many rows: prefill; capacities up to 32768;
// other shapes) score a block of rows into the workspace and select from it, block after
// block, so the score buffer is bounded by kScoreBlockBytes instead of growing with R x n_max.
constexpr size_t kScoreBlockBytes = size_t(256) << 20;
constexpr int kRowGroup = 7;  // rows per workgroup of the many-rows indexer: blocks keep its groups whole

bool fused_fast(dsa_dtype dt, int H_I, int d_I) { return dt == DSA_E4M3 && H_I == 64 && d_I == 128; }
// Rows up to 32768 keys are selected by one workgroup each straight from their score row (no
// compaction pass), which measured faster than the sampled compaction at that length: the
// sample workgroup's latency is longer than the short chunks' scoring.
constexpr int64_t kFusedMinCapacity = 32768;
bool fused_decode(int R, int64_t cap) {
  return R < dsa::index_rows_kernel_min() && cap > kFusedMinCapacity && dsa::index_topk_fused_ok(R, cap);
}

int block_rows(int R, int64_t cap) {
  int64_t rb = (int64_t)(kScoreBlockBytes / (sizeof(float) * (size_t)cap)) / kRowGroup * kRowGroup;
  rb = rb < kRowGroup ? kRowGroup : rb;
  return (int)(rb < R ? rb : R);
}

struct BlockWs {
  int rows;
  size_t scores, topk, total;
};
BlockWs block_ws(int R, int64_t cap, int k) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  BlockWs L{};
  L.rows = block_rows(R, cap);
  L.scores = 0;
  L.topk = up(sizeof(float) * (size_t)L.rows * (size_t)cap);
  L.total = L.topk + up(dsa::topk_workspace_bytes(L.rows, cap, k));
  return L;
}
}  // namespace

size_t dsa_index_topk_workspace_size(int R, int64_t n_max, int k) {
  if (R <= 0 || n_max <= 0 || k <= 0) return 0;
  size_t need = block_ws(R, n_max, k).total;
  if (fused_decode(R, n_max)) {
    const size_t f = dsa::index_topk_fused_bytes(R, n_max);
    need = f > need ? f : need;
  }
  return need;
}

dsa_status dsa_index_topk(dsa_dtype dt, const void* q, const float* q_scale, const float* w,
                          const dsa_cache* keys, const int32_t* row_seq, const int32_t* row_pos,
                          int R, int H_I, int d_I, int k, int32_t* idx, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  if (!q || !w || !keys || !keys->data || !row_seq || !row_pos || !idx) return DSA_ERR_NULL;
  if (dt != DSA_E4M3 && dt != DSA_F32) return DSA_ERR_DTYPE;
  if (R <= 0 || H_I <= 0 || d_I <= 0 || R > 65535 || k <= 0 || k > 16384) return DSA_ERR_SHAPE;
  const int64_t cap = cache_capacity(keys);
  if (cap <= 0 || cap > (int64_t(1) << 24) || !dsa::topk_shape_ok(R, cap)) return DSA_ERR_SHAPE;
  if ((int64_t)H_I * d_I > 16384) return DSA_ERR_UNSUPPORTED;
  if (!ws) return DSA_ERR_WORKSPACE;
  const dsa::CacheView kv = view(keys);
  const bool fast = fused_fast(dt, H_I, d_I);
  if (fast && fused_decode(R, cap)) {
    if (ws_bytes < dsa::index_topk_fused_bytes(R, cap)) return DSA_ERR_WORKSPACE;
    return launched(dsa::launch_index_topk_fused(static_cast<const uint8_t*>(q), q_scale, w, kv, row_seq,
                                                 row_pos, R, cap, k, idx, ws, stream));
  }
  const BlockWs L = block_ws(R, cap, k);
  if (ws_bytes < L.total) return DSA_ERR_WORKSPACE;
  char* b = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(b + L.scores);
  void* tws = b + L.topk;
  const size_t qrow = (size_t)H_I * d_I * (dt == DSA_E4M3 ? 1 : sizeof(float));
  for (int r0 = 0; r0 < R; r0 += L.rows) {
    const int nb = R - r0 < L.rows ? R - r0 : L.rows;
    const void* qb = static_cast<const char*>(q) + (size_t)r0 * qrow;
    const float* qsb = q_scale ? q_scale + r0 : nullptr;
    const float* wb = w + (size_t)r0 * H_I;
    hipError_t e;
    if (fast)
      e = dsa::launch_index_fp8_h64d128(static_cast<const uint8_t*>(qb), qsb, wb, kv, row_seq + r0, row_pos + r0,
                                        nb, cap, scores, cap, stream);
    else
      e = dsa::launch_index_generic(dt == DSA_E4M3, qb, qsb, wb, kv, row_seq + r0, row_pos + r0, nb, H_I, d_I,
                                    cap, scores, cap, stream);
    if (e != hipSuccess) return DSA_ERR_LAUNCH;
    e = dsa::launch_topk(scores, cap, row_pos + r0, nb, k, idx + (size_t)r0 * k, tws, stream, 1);
    if (e != hipSuccess) return DSA_ERR_LAUNCH;
  }
  return DSA_OK;
}

size_t dsa_indexer_quality_workspace_size(int R, int H, int64_t ld) {
  if (R <= 0 || H <= 0 || ld <= 0) return 0;
  return dsa::quality_workspace_bytes(R, H, ld);
}

dsa_status dsa_indexer_quality(const void* q, const dsa_cache* kv, const float* scores, int64_t ld,
                               const int32_t* idx, const int32_t* row_seq, const int32_t* row_pos,
                               int R, int H, int Dqk, int k, float softmax_scale, float* kl,
                               float* recall, float* kl_rev, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  if (!q || !kv || !kv->data || !scores || !idx || !row_seq || !row_pos || !kl || !recall)
    return DSA_ERR_NULL;
  if (R <= 0 || H <= 0 || Dqk <= 0 || k <= 0 || ld <= 0 || R > 65535) return DSA_ERR_SHAPE;
  const int64_t cap = cache_capacity(kv);
  if (cap <= 0 || ld < cap) return DSA_ERR_SHAPE;
  if (H % 16 != 0 || H > 128 || Dqk % 32 != 0 || Dqk > 576) return DSA_ERR_UNSUPPORTED;
  if ((int64_t)R * ((ld + 63) / 64) > 2147483647LL) return DSA_ERR_SHAPE;
  if (!ws || ws_bytes < dsa::quality_workspace_bytes(R, H, ld)) return DSA_ERR_WORKSPACE;
  return launched(dsa::launch_indexer_quality(static_cast<const uint16_t*>(q), view(kv), scores, ld, idx, k,
                                              row_seq, row_pos, R, H, Dqk, ld, softmax_scale, kl, recall,
                                              kl_rev, ws, stream));
}

dsa_status dsa_masked_mla_prefill(dsa_dtype dt, const void* q, const void* kv, const int32_t* idx,
                                  int T, int H, int Dqk, int Dv, int k, float softmax_scale, void* out,
                                  float* lse, hipStream_t stream) {
  dsa_status st = mla_check(dt, q, kv, idx, T, H, Dqk, Dv, k, out);
  if (st != DSA_OK) return st;
  if (T > 65536) return DSA_ERR_SHAPE;
  if (mla_fast(dt, H, Dqk, Dv))
    return launched(dsa::launch_mla_bf16_masked(static_cast<const uint16_t*>(q),
                                                static_cast<const uint16_t*>(kv), idx, T, H, k,
                                                softmax_scale, static_cast<uint16_t*>(out), lse, stream));
  // Other shapes: the generic kernel computes the same attention from the index list.
  const dsa::CacheView v{kv, nullptr, nullptr, 0, 0, (int64_t)T};
  if ((st = mla_generic_ok(Dqk, k)) != DSA_OK) return st;
  return launched(dsa::launch_mla_generic(dt == DSA_BF16, q, v, idx, T, H, Dqk, Dv, k, false,
                                          softmax_scale, out, lse, stream));
}

dsa_status dsa_cache_append(const float* k_new, const void* kv_new, const int32_t* row_seq,
                            const int32_t* row_pos, int R, int d_I, int Dqk, const dsa_cache* keys,
                            const dsa_cache* kv, hipStream_t stream) {
  if (!k_new || !kv_new || !row_seq || !row_pos || !keys || !kv || !keys->data || !keys->scale || !kv->data)
    return DSA_ERR_NULL;
  if (R <= 0 || d_I <= 0 || Dqk <= 0 || d_I > 4096 || Dqk > 4096) return DSA_ERR_SHAPE;
  if (cache_capacity(keys) <= 0 || cache_capacity(kv) <= 0) return DSA_ERR_SHAPE;
  return launched(dsa::launch_cache_append(k_new, static_cast<const uint16_t*>(kv_new), row_seq, row_pos,
                                           R, d_I, Dqk, view(keys), view(kv), stream));
}

dsa_status dsa_check_indices(const int32_t* idx, int R, int k, const int32_t* n_valid, int strict,
                             int64_t* first_bad) {
  if (!idx || !n_valid || !first_bad) return DSA_ERR_NULL;
  *first_bad = -1;
  if (R <= 0 || k <= 0) return DSA_ERR_SHAPE;
  for (int r = 0; r < R; ++r) {
    const int32_t n = n_valid[r];
    const int32_t* row = idx + (int64_t)r * k;
    if (n < 0) {
      *first_bad = (int64_t)r * k;
      return DSA_ERR_RANGE;
    }
    bool padding = false;  // strict: a -1 was seen, only -1 may follow
    int32_t prev = -1;
    for (int j = 0; j < k; ++j) {
      const int32_t v = row[j];
      bool bad = v < -1 || v >= n;
      if (strict && !bad) bad = (v >= 0 && (padding || v <= prev));
      if (bad) {
        *first_bad = (int64_t)r * k + j;
        return DSA_ERR_RANGE;
      }
      if (v < 0) padding = true;
      else prev = v;
    }
  }
  return DSA_OK;
}

dsa_status dsa_check_block_table(const int32_t* table, int B, int max_pages, const int32_t* lengths,
                                 int page_size, int64_t pool_pages, int64_t* first_bad) {
  if (!table || !lengths || !first_bad) return DSA_ERR_NULL;
  *first_bad = -1;
  if (B <= 0 || max_pages <= 0 || page_size <= 0 || pool_pages <= 0) return DSA_ERR_SHAPE;
  for (int b = 0; b < B; ++b) {
    const int64_t len = lengths[b];
    if (len < 0 || len > (int64_t)max_pages * page_size) {
      *first_bad = -1 - (int64_t)b;
      return DSA_ERR_RANGE;
    }
    const int64_t used = (len + page_size - 1) / page_size;
    for (int64_t p = 0; p < used; ++p) {
      const int32_t e = table[(int64_t)b * max_pages + p];
      if (e < 0 || e >= pool_pages) {
        *first_bad = (int64_t)b * max_pages + p;
        return DSA_ERR_RANGE;
      }
    }
  }
  return DSA_OK;
}

}  // extern "C"
