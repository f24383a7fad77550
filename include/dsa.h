/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) hot path for MI355X (gfx950).
 *
 * The path, as the pages state the problem (MarkTechPost, "DeepSeek V3.2-Exp Cuts
 * Long-Context Costs with DeepSeek Sparse Attention (DSA) While Maintaining
 * Benchmark Parity": a two-tier pipeline -- an FP8 indexer, then top-k, then core
 * attention over the kept tokens; maplevalley.com.cn news 1594152, section "1. 细粒度稀疏架构": a
 * lightning indexer scores every preceding token and each query keeps only k
 * key/value pairs, O(L^2) -> O(Lk)):
 *
 *   1. dsa_index_scores       I[r, s] for every query row r and candidate s < n_r
 *   2. dsa_topk               the k best s per row (ties -> lower s), -1 padded
 *   3. dsa_sparse_mla_decode  MLA in MQA mode over the kept latent rows, one query
 *      dsa_sparse_mla_prefill token per sequence (decode) or every token (prefill)
 *   and, before them, dsa_cache_append: the new token's FP8 indexer key and latent row
 *   written into the caches; dsa_index_topk: steps 1 and 2 in one call;
 *   dsa_masked_mla_prefill: step 3 of a prefill in dense masked form, for short sequences;
 *   dsa_indexer_quality: a forward-only diagnostic of the indexer against dense attention.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, 16-byte aligned,
 *     densely packed in the documented layout (row-major, last index fastest).
 *   - The library never allocates, frees or synchronises.  Every call only enqueues
 *     kernels on `stream` and returns; results are valid once the stream reaches them.
 *   - Arguments are validated on the host before anything is launched; a validation
 *     error returns its status and enqueues nothing.  Device-side values (indices,
 *     lengths, page-table entries) are not validated: out-of-range values are
 *     undefined behaviour.  A failed launch returns DSA_ERR_LAUNCH.
 *   - Calls are stateless and thread-safe.  Two calls that share a workspace must
 *     not overlap in time (same stream, or synchronised).
 *   - Dtypes: DSA_E4M3 is OCP FP8 E4M3 ("e4m3fn": bias 7, max 448, no inf);
 *     DSA_BF16 is bfloat16; DSA_F32 is IEEE binary32.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,        /* a required pointer is NULL                              */
  DSA_ERR_SHAPE = 2,       /* a size is <= 0, inconsistent, or exceeds a stated limit  */
  DSA_ERR_DTYPE = 3,       /* dtype not accepted by this entry point                   */
  DSA_ERR_WORKSPACE = 4,   /* workspace pointer NULL or smaller than required          */
  DSA_ERR_LAUNCH = 5,      /* the HIP runtime reported an error after launching        */
  DSA_ERR_UNSUPPORTED = 6, /* valid but unsupported combination (e.g. an fp32 shape
                              beyond the generic kernel's LDS)                         */
  DSA_ERR_RANGE = 7        /* a validator found an index or page entry out of range    */
} dsa_status;

typedef enum { DSA_F32 = 0, DSA_BF16 = 1, DSA_E4M3 = 2 } dsa_dtype;

/*
 * A per-token cache of one tensor (indexer keys, or MLA latent rows), either
 *   contiguous: row (b, s) at  data + (b * seq_stride + s) * D          (block_table == NULL)
 *   paged:      row (b, s) at  data + (block_table[b * max_pages + s / page_size] * page_size
 *                                      + s % page_size) * D
 * D is the row width given to the call.  `scale` (indexer keys only) is the per-token
 * fp32 dequantisation scale with the same addressing and a width of one float; NULL
 * means 1.  Any page size >= 1 is accepted; the paged workloads use 64-token pages (the
 * pages do not fix a size).
 */
typedef struct {
  const void* data;
  const float* scale;
  const int32_t* block_table;
  int32_t page_size;
  int32_t max_pages;
  int64_t seq_stride;
} dsa_cache;

/*
 * dsa_index_scores -- lightning-indexer scores (first tier of the DSA pipeline:
 * an FP8 indexer, MarkTechPost article above; the lightning indexer, maplevalley article
 * section 1).  The pages do not print the formula; this library computes
 *
 *   scores[r * ld + s] = k_scale[seq, s] * q_scale[r] * sum_{j < H_I} w[r, j] * max(0, q[r, j, :] . k[seq, s, :])
 *
 * for seq = row_seq[r] and every s in [0, n_r), n_r = row_pos[r] + 1 (the query's own
 * token is a candidate).  Entries s >= n_r of a score row are left untouched.
 *
 *   dt        DSA_E4M3: q and keys are e4m3 codes (fast path: H_I == 64, d_I == 128, any
 *             page size); DSA_F32: q and keys are fp32 (any shape).
 *   q         [R, H_I, d_I]          q_scale [R] or NULL (= 1)     w [R, H_I] fp32
 *   keys      cache of rows of width d_I (+ per-token scale)
 *   row_seq   [R] int32 sequence of each row      row_pos [R] int32 position of each row
 *   scores    [R, ld] fp32 output; ld >= the cache's longest sequence
 *             (seq_stride, or max_pages * page_size when paged)
 * Decode: row r = sequence r, row_pos = L_r - 1.  Prefill of one sequence: row_seq = 0,
 * row_pos = t.
 */
dsa_status dsa_index_scores(dsa_dtype dt, const void* q, const float* q_scale, const float* w,
                            const dsa_cache* keys, const int32_t* row_seq, const int32_t* row_pos,
                            int R, int H_I, int d_I, float* scores, int64_t ld, hipStream_t stream);

/*
 * dsa_topk -- per-row top-k token selection (maplevalley article section 1: "Top-k
 * Token Selection", each query keeps k key/value pairs; tellworld "What happened":
 * token-level selection; MarkTechPost "Training signal": k = 2048).
 *
 * For row r with n = n_valid[r] candidates (scores[r * ld + s], s < n): if n <= k all
 * n indices are kept; otherwise the k largest, ties broken towards the lower index
 * (-0.0 ties with +0.0; NaN scores are undefined behaviour).  idx[r * k + j] holds the
 * kept indices in ascending order in slots j < min(k, n) and -1 in the rest.
 *
 *   scores [R, ld] fp32      n_valid [R] int32, 0 <= n_valid[r] <= ld
 *   idx    [R, k] int32 output
 *   ws     device workspace of at least dsa_topk_workspace_size(R, ld, k) bytes
 * Limits: k <= 16384, ld <= 2^24, and for ld > 32768 R * ceil(ld / 4096) <= 2^31 - 1
 * (DSA_ERR_SHAPE otherwise).
 */
size_t dsa_topk_workspace_size(int R, int64_t ld, int k);
dsa_status dsa_topk(const float* scores, int64_t ld, const int32_t* n_valid, int R, int k,
                    int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * dsa_sparse_mla_decode -- sparse core attention for one new token per sequence:
 * MLA in MQA mode (MarkTechPost "Instantiation": one latent KV row serves every query
 * head).  For sequence b and head h, over S_b = { idx[b, j] : idx[b, j] >= 0 }:
 *
 *   z_s = softmax_scale * q[b, h, :] . kv[b, s, :]          (all Dqk columns)
 *   out[b, h, :] = sum_s softmax(z)_s * kv[b, s, :Dv]        (value = first Dv columns)
 *   lse[b, h]    = log sum_s exp(z_s)                         (natural log)
 * An empty S_b gives out = 0 and lse = -inf.
 *
 *   dt     DSA_BF16: q, kv, out bf16 (fast path: H % 64 == 0, Dqk == 576, Dv == 512,
 *          paged page_size any); DSA_F32: fp32 (any shape with Dv <= Dqk <= 1024)
 *   q      [B, H, Dqk]     kv cache of rows of width Dqk      idx [B, k] int32
 *   out    [B, H, Dv]      lse [B, H] fp32 or NULL
 *   ws     device workspace of at least dsa_sparse_mla_decode_workspace_size(...) bytes
 *          (split-KV partials); may be NULL when that size is 0
 * Limits: B * H <= 2^31 - 1; off the bf16 fast path (DSA_F32 or other shapes) the
 * generic kernel needs (Dqk + k + 8) * 4 <= 65536 bytes and Dqk <= 1024, else
 * DSA_ERR_UNSUPPORTED.  The fast path takes any k (a workgroup holds at most 8192 kept
 * tokens; longer sets are split further).
 */
size_t dsa_sparse_mla_decode_workspace_size(int B, int H, int Dv, int k);
dsa_status dsa_sparse_mla_decode(dsa_dtype dt, const void* q, const dsa_cache* kv,
                                 const int32_t* idx, int B, int H, int Dqk, int Dv, int k,
                                 float softmax_scale, void* out, float* lse, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/*
 * dsa_sparse_mla_decode_noalloc -- dsa_sparse_mla_decode for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without a workspace, the same kernels and the same result bit for bit.  The
 * split-KV partials go to a static device array of dsa_noalloc_scratch_bytes() bytes (32 MiB),
 * one per GPU, held until the process ends.  It calls no allocator.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, or two threads without ordering) race and give undefined results; serialise them.
 * The array keeps the last call's contents; nothing in it needs clearing (every partial a
 * call reads is written by the same call first).
 * Errors: as dsa_sparse_mla_decode, plus DSA_ERR_WORKSPACE when the partials this call needs
 * (dsa_sparse_mla_decode_workspace_size) exceed the array, and DSA_ERR_LAUNCH when the
 * array's device address cannot be looked up.  The lookup runs once per device, on the
 * first call with that device current.
 */
size_t dsa_noalloc_scratch_bytes(void);
dsa_status dsa_sparse_mla_decode_noalloc(dsa_dtype dt, const void* q, const dsa_cache* kv,
                                         const int32_t* idx, int B, int H, int Dqk, int Dv, int k,
                                         float softmax_scale, void* out, float* lse,
                                         hipStream_t stream);

/*
 * dsa_sparse_mla_prefill -- the same attention for every token t of one sequence,
 * each over its own kept set S_t = { idx[t, j] >= 0 } (causal selection is the
 * caller's: dsa_topk with n_valid[t] = t + 1 keeps only s <= t).
 *
 *   q [T, H, Dqk]   kv [T, Dqk] (contiguous latent rows of the sequence)   idx [T, k]
 *   out [T, H, Dv]  lse [T, H] fp32 or NULL
 * dt and shape rules as for dsa_sparse_mla_decode.  Limits: as there, and k <= 8192 on the
 * bf16 fast path (one workgroup holds a row's whole kept set; else DSA_ERR_UNSUPPORTED).
 */
dsa_status dsa_sparse_mla_prefill(dsa_dtype dt, const void* q, const void* kv, const int32_t* idx,
                                  int T, int H, int Dqk, int Dv, int k, float softmax_scale,
                                  void* out, float* lse, hipStream_t stream);

/*
 * dsa_index_topk -- dsa_index_scores followed by dsa_topk in one call (the pages' first two
 * steps, indexing then selection, as one stage), with n_valid[r] = row_pos[r] + 1.  The result is exactly
 * that of the two calls (same scores, same selection rule).
 *
 * On the fast indexer shape (e4m3, H_I = 64, d_I = 128) with fewer than 512 rows (decode) and
 * a capacity above 32768 no score row is stored: inside the indexer's launch, one workgroup
 * per row scores 1024 evenly spaced sample keys and publishes a threshold expected to keep
 * about 3k keys, while the other workgroups score the row and write only the keys at or above
 * it (with their positions) to `ws`; a second launch selects the top k among them.  Where the
 * sample misleads (fewer than k keys reach the threshold, or more than 12288 with at least k
 * above it) that launch scores the row again and selects from all of it: the result never
 * depends on the sample.  The threshold hand-off uses words in `ws` that each call clears for
 * the next: any contents are correct, but a workspace that starts zeroed avoids the slow path
 * on its first call.  Otherwise (prefill-sized calls; capacities up to 32768, where one
 * workgroup per row selects from the score row faster than the compaction; other shapes) the
 * rows are scored into `ws` a block at a time (at most 256 MiB of scores per block) and each
 * block is selected before the next is scored, so the workspace does not grow with
 * R x capacity.
 *
 *   arguments as dsa_index_scores (the keys cache's capacity plays the role of ld) and dsa_topk
 *   idx [R, k] int32 output, as dsa_topk
 *   ws    device workspace of at least dsa_index_topk_workspace_size(R, capacity, k) bytes;
 *         calls that share one workspace must not overlap in time
 * Limits: as the two calls; capacity <= 2^24.
 */
size_t dsa_index_topk_workspace_size(int R, int64_t n_max, int k);
dsa_status dsa_index_topk(dsa_dtype dt, const void* q, const float* q_scale, const float* w,
                          const dsa_cache* keys, const int32_t* row_seq, const int32_t* row_pos,
                          int R, int H_I, int d_I, int k, int32_t* idx, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * dsa_indexer_quality -- forward-only diagnostic of how well the index scores imitate dense
 * attention, the quantity the pages say the indexer is trained on (MarkTechPost article
 * above, "Training signal": a KL loss pulls the indexer towards the dense attention
 * summed over heads).  For row r with n = row_pos[r] + 1 candidates:
 *   p[s]      = (1/H) sum_h softmax_s(softmax_scale * q[r, h, :] . kv[s, :])   (all s < n)
 *   kl[r]     = sum_s p[s] * (ln p[s] - ln softmax_s(scores[r, s]))   (nats, the dense
 *               distribution as the target)
 *   kl_rev[r] = sum_s q[s] * (ln q[s] - ln p[s]), q = softmax_s(scores[r, s])   (the other
 *               order: the pages do not fix it; +inf where p underflows to 0)
 *   recall[r] = sum of p[s] over the kept set { idx[r, j] : 0 <= idx[r, j] < n }
 *
 *   q [R, H, Dqk] bf16     kv  bf16 latent cache, contiguous or paged (as the decode call)
 *   scores [R, ld] fp32 (as dsa_index_scores wrote them)   idx [R, k] int32 (as dsa_topk)
 *   kl, recall [R] fp32 outputs      kl_rev [R] fp32 output or NULL
 *   ws  device workspace of at least dsa_indexer_quality_workspace_size(R, H, ld) bytes (it
 *       holds every head's logits: R * H * ld fp32)
 * Limits: H a multiple of 16 and <= 128, Dqk a multiple of 32 and <= 576 (else
 * DSA_ERR_UNSUPPORTED); ld >= the cache's capacity.
 */
size_t dsa_indexer_quality_workspace_size(int R, int H, int64_t ld);
dsa_status dsa_indexer_quality(const void* q, const dsa_cache* kv, const float* scores, int64_t ld,
                               const int32_t* idx, const int32_t* row_seq, const int32_t* row_pos,
                               int R, int H, int Dqk, int k, float softmax_scale, float* kl,
                               float* recall, float* kl_rev, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/*
 * dsa_masked_mla_prefill -- the same result as dsa_sparse_mla_prefill, computed in the
 * dense "masked" form the pages name for short prefill (MarkTechPost article above, "Costs
 * vs. position (128k)": short prefills run attention densely under a mask):
 * row t runs over the contiguous positions 0..t in 32-row tiles and masks every position
 * not in its kept set S_t = { idx[t, j] : 0 <= idx[t, j] <= t } (other entries are ignored).
 * No row gather, but the cost grows with t rather than |S_t|: it pays while t + 1 is
 * within a small multiple of k.
 *
 *   arguments, layouts and dtypes as dsa_sparse_mla_prefill; T <= 65536, any k on the bf16
 *   fast path (the kept set only sets mask bits), the generic kernel's limit otherwise.
 * Shapes off the bf16 fast path are served by the same generic kernel as the sparse call.
 */
dsa_status dsa_masked_mla_prefill(dsa_dtype dt, const void* q, const void* kv, const int32_t* idx,
                                  int T, int H, int Dqk, int Dv, int k, float softmax_scale,
                                  void* out, float* lse, hipStream_t stream);

/*
 * dsa_cache_append -- store each row's new token in the two caches before a step reads
 * them: the indexer key (FP8, as the pages' indexer runs, MarkTechPost article above, two-tier
 * pipeline) and the latent row (the joint K/V entry MLA attends over, same article,
 * "Instantiation").  For row r the cache slot is (row_seq[r], row_pos[r]); decode writes
 * the new token at n_valid - 1, the position dsa_index_scores and the attention read as
 * the query's own token.
 *
 *   k_new  [R, d_I] fp32   the new token's indexer key, before quantisation
 *   kv_new [R, Dqk] bf16   the new token's latent row
 *   keys   e4m3 key cache of row width d_I with a non-NULL per-token fp32 `scale`;
 *          WRITTEN through keys->data and keys->scale
 *   kv     bf16 latent cache of row width Dqk; WRITTEN through kv->data
 * Quantisation (this library's reading of "FP8"): scale = max_i |k_new[r, i]| / 448 in
 * fp32 (1 when the key is all zero); code_i = e4m3(clamp(k_new[r, i] / scale, -448, 448))
 * rounded to nearest, ties to even.  Rows must name distinct slots (two rows writing one
 * slot leave either).  Limits: d_I <= 4096, Dqk <= 4096.
 */
dsa_status dsa_cache_append(const float* k_new, const void* kv_new, const int32_t* row_seq,
                            const int32_t* row_pos, int R, int d_I, int Dqk, const dsa_cache* keys,
                            const dsa_cache* kv, hipStream_t stream);

/*
 * dsa_read_probe -- a measurement, not a step of the path: reads `bytes` bytes at `buf` once
 * and writes to sink[w], for each of its dsa_read_probe_sink_words() workgroups w, the XOR of
 * the 32-bit words that workgroup read.  The XOR of all sink words is the XOR of every 32-bit
 * word of the buffer, so a host check shows that all of it was read.  Timing launches of it
 * gives the rate at which this GPU streams a buffer of that size: every load instruction reads
 * one contiguous 1 KB (non-temporal), eight in flight per wave, two 512-thread workgroups per
 * CU.  It is the practical ceiling that the bandwidth-bound indexer scan is compared with.
 *
 *   buf   device, 16-byte aligned, `bytes` a positive multiple of 1024; only read
 *   sink  device uint32 [dsa_read_probe_sink_words()], fully overwritten
 *
 * Errors: DSA_ERR_NULL (buf or sink NULL), DSA_ERR_SHAPE (size or alignment), DSA_ERR_LAUNCH.
 */
int dsa_read_probe_sink_words(void);
dsa_status dsa_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);

/* Static text for a status code ("DSA_OK", ...); never NULL. */
const char* dsa_status_string(dsa_status status);

/*
 * dsa_check_indices, dsa_check_block_table -- host-side validators of the device-side values
 * the kernels trust (see the conventions above: out-of-range indices or page-table entries are
 * undefined behaviour, they read outside the caches).  They do no GPU work and touch only HOST
 * memory: the caller copies the arrays to the host first, e.g. in a debug build or before the
 * first launch on new tables.  Setting DSA_DEBUG_CHECKS=1 makes the Python step classes run
 * them on every step.  Both return DSA_OK, DSA_ERR_NULL, DSA_ERR_SHAPE (a size <= 0) or
 * DSA_ERR_RANGE with *first_bad set to the flat index of the first offending entry (else -1).
 *
 * dsa_check_indices: idx [R, k] int32 (host), n_valid [R] int32 (host), as dsa_topk writes and
 *   the attention calls read them: every entry is -1 or in [0, n_valid[r]).  strict != 0 also
 *   requires the form dsa_topk produces -- the valid entries ascending without repeats, then
 *   only -1 (the attention kernels count a repeated index twice).  A negative n_valid[r] is
 *   reported at index r * k.
 * dsa_check_block_table: table [B, max_pages] int32 (host), lengths [B] int32 (host, tokens
 *   cached per sequence): every length lies in [0, max_pages * page_size] (else *first_bad =
 *   -1 - b) and every page a sequence uses, p < ceil(lengths[b] / page_size), maps into the
 *   pool: 0 <= table[b * max_pages + p] < pool_pages (else *first_bad = b * max_pages + p).
 */
dsa_status dsa_check_indices(const int32_t* idx, int R, int k, const int32_t* n_valid, int strict,
                             int64_t* first_bad);
dsa_status dsa_check_block_table(const int32_t* table, int B, int max_pages, const int32_t* lengths,
                                 int page_size, int64_t pool_pages, int64_t* first_bad);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
