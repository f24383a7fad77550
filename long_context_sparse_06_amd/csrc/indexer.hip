// Lightning indexer: I[r,s] = k_scale[s] * q_scale[r] * sum_j w[r,j] * ReLU(q[r,j,:] . k[s,:]).
//
// The pages give the indexer only as the lightweight FP8 first tier of the pipeline that
// then keeps the top-k tokens and attends over them (MarkTechPost, "DeepSeek V3.2-Exp Cuts
// Long-Context Costs with DeepSeek Sparse Attention (DSA) ...") and as the "Lightning
// Indexer" that computes lightweight index scores (maplevalley.com.cn news 1594152,
// section 1); the ReLU-of-per-head-dots form above is this library's reading.
//
// Fast path (H_I = 64, d_I = 128, e4m3): one gfx950 v_mfma_scale_f32_16x16x128_f8f6f4
// per 16 heads x 16 keys covers the whole 128-byte key row, so a key is read from HBM
// exactly once and multiplied against all 64 query heads held in registers.  The
// ReLU / w-weighted head sum / per-token scale run in fp32 on the MFMA results
// (score_core.h).
#include "common.h"
#include "kernels.h"
#include "score_core.h"
#include "select_core.h"

namespace dsa {
namespace {

constexpr int kIdxWaves = 8;
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kCompactTrips = 8;  // most trips per wave of the compacting indexer (4096 keys per workgroup)

// Score of 64 keys per loop trip and wave.  Lane (col, grp) feeds key s0 + 16*u + col, bytes
// 32*grp .. 32*grp+31, to the MFMA of column group u; the result layout leaves the lane with
// 16 of the 64 heads of that key, which are ReLU'd, weighted and summed in-lane.  A two-stage
// butterfly of gfx950 lane swaps (v_permlane32_swap, v_permlane16_swap) then adds the four
// partial sums of each group and leaves group g's totals in lanes 16*g .. 16*g+15, so the 64
// scores of the trip leave in one coalesced 256-byte store.
//
// Chunks of the compacting indexer: the row bound's tb 64-key trips split as evenly as the
// trips allow, chunk c starting at key chunk_start(c, tb, nc).
__device__ __forceinline__ int64_t chunk_start(int c, int tb, int nc) {
  return (int64_t)kIdxBatch * (((int64_t)c * tb) / nc);
}

// COMPACT (the fused index + top-k call): no score is stored.  The grid has R extra blocks
// in front: block r scores row r's kCompactSample evenly spaced keys (positions
// (i * n) / kCompactSample) and publishes the row's threshold theta -- about 3k survivors
// expected -- in hdr[r] and in the word ready[r].  Every other block scores its chunk, parks
// the keys in LDS and only then reads ready[r] (by then the sample block, dispatched first
// and far less work, has long published it); it writes only the survivors (key >= theta) as
// (key, position) pairs, in position order, to the chunk's slot of the candidate buffer, with
// the chunk's counts of keys above theta and equal to it and the theta it used.  The wait is
// bounded: a chunk that finds no threshold keeps nothing and records so, and the resolve
// rescores such a row.  Rows of at most min_n keys are skipped (their selection needs no
// scores).
constexpr int kCompactSample = 1024;  // 8 waves x 2 trips
constexpr int kThetaPolls = 2048;     // ~2 ms of polling (s_sleep 32 between reads)
constexpr int kSampleWords = kCompactSample + kPassMax * kHistBins + (int)(sizeof(SelState) + 3) / 4;
constexpr int kParkWords = kIdxWaves * kCompactTrips * kIdxBatch;
constexpr int kPoolWords = kSampleWords > kParkWords ? kSampleWords : kParkWords;

// The sample block of row r (all threads of the block).
__device__ void compact_sample_block(int r, const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
                                     const float* __restrict__ w, const uint8_t* __restrict__ kdata,
                                     const float* __restrict__ kscale, const KeyRows& kr,
                                     const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos,
                                     int min_n, RowHeader* __restrict__ hdr, uint64_t* __restrict__ ready,
                                     uint8_t* sq, float* sw, uint32_t* pool) {
  const int64_t n = (int64_t)row_pos[r] + 1;
  if (n <= min_n) return;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int col = lane & 15, grp = lane >> 4;
  const int seq = row_seq[r];
  // Cache rows of this lane's sampled keys (four per trip) and of the key whose scale it
  // applies (one per trip), for both trips, found before the query is staged: with a
  // paged cache each is a block-table read, and issuing them all at once keeps them to one
  // round trip instead of a table read ahead of every trip's key loads.
  int64_t krow[2][4], srow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j0 = (2 * wave + t) * kIdxBatch;
#pragma unroll
    for (int u = 0; u < 4; ++u) krow[t][u] = kr.row(seq, (int64_t)(j0 + 16 * u + col) * n / kCompactSample);
    srow[t] = kr.row(seq, (int64_t)(j0 + lane) * n / kCompactSample);
  }
  for (int i = tid; i < 64 * 128 / 16; i += kIdxWaves * WAVE)
    reinterpret_cast<uint4*>(sq)[i] = reinterpret_cast<const uint4*>(q + (int64_t)r * (64 * 128))[i];
  if (tid < 64) sw[tid] = w[(int64_t)r * 64 + tid];
  __syncthreads();
  v8i qa[4];
  float wr[4][4];
  load_query(sq, sw, col, grp, qa, wr);
  const float qs = q_scale ? q_scale[r] : 1.0f;
  uint32_t* samp = pool;
  int* hist = reinterpret_cast<int*>(pool + kCompactSample);
  SelState& st = *reinterpret_cast<SelState*>(pool + kCompactSample + kPassMax * kHistBins);
  uint32_t lmn = 0xFFFFFFFFu, lmx = 0u;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j0 = (2 * wave + t) * kIdxBatch;
    v8i kb[4];
    load_rows(kdata, krow[t], grp, kb);
    const float ks = kscale ? kscale[srow[t]] : 1.0f;
    const uint32_t key = float_key(scaled_score(trip_scores(qa, wr, kb), ks, qs));
    samp[j0 + lane] = key;
    lmn = min(lmn, key);
    lmx = max(lmx, key);
  }
  const RowHeader rh = sample_header<kIdxWaves * WAVE>(samp, kCompactSample, 3, lmn, lmx, n, min_n, hist, st);
  if (tid == 0) {
    hdr[r] = rh;
    __hip_atomic_store(&ready[r], ((uint64_t)kThetaReady << 32) | rh.theta, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool PAGED, bool COMPACT = false>
__global__ __launch_bounds__(kIdxWaves * WAVE) void index_fp8_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ kdata, const float* __restrict__ kscale,
    const int32_t* __restrict__ table, int max_pages, int page_size, int page_shift,
    int64_t seq_stride, const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos,
    float* __restrict__ scores, int64_t ld, int keys_per_wg, int n_chunks,
    RowHeader* __restrict__ hdr = nullptr, uint64_t* __restrict__ ready = nullptr,
    ChunkCount* __restrict__ counts = nullptr, uint2* __restrict__ cand = nullptr, int min_n = 0,
    int n_rows = 0) {
  // The row's query (8 KB) and head weights go to LDS once; every wave reads its fragments
  // there instead of fetching its own copy through L2.
  __shared__ __attribute__((aligned(16))) uint8_t sq[64 * 128];
  __shared__ __attribute__((aligned(16))) float sw[64];
  __shared__ __attribute__((aligned(16))) uint32_t pool[COMPACT ? kPoolWords : 1];
  if (COMPACT && (int)blockIdx.x < n_rows) {
    compact_sample_block(blockIdx.x, q, q_scale, w, kdata, kscale,
                         KeyRows{PAGED ? table : nullptr, max_pages, page_size, page_shift, seq_stride}, row_seq,
                         row_pos, min_n, hdr, ready, sq, sw, pool);
    return;
  }
  const int blk = COMPACT ? (int)blockIdx.x - n_rows : (int)blockIdx.x;
  extern __shared__ int spage[];  // paged: physical page of each logical page of this range
  // Block b takes chunk b % n_chunks of row b / n_chunks: consecutive blocks (which the
  // dispatcher deals round-robin to the eight XCDs) walk along a row, so rows of different
  // lengths still spread their work evenly over the XCDs.
  const int r = blk / n_chunks;
  const int chunk = blk % n_chunks;
  const int64_t n = (int64_t)row_pos[r] + 1;
  // COMPACT: keys_per_wg is the row bound's trip count tb and chunk c covers trips
  // [c * tb / n_chunks, (c + 1) * tb / n_chunks) (chunk_start).
  int64_t wg_begin, wg_full;
  if (COMPACT) {
    wg_begin = chunk_start(chunk, keys_per_wg, n_chunks);
    wg_full = chunk_start(chunk + 1, keys_per_wg, n_chunks);
  } else {
    wg_begin = (int64_t)chunk * keys_per_wg;
    wg_full = wg_begin + keys_per_wg;
  }
  if (wg_begin >= n || (COMPACT && n <= min_n)) return;
  const int64_t wg_end = min(wg_full, n);
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wave = tid / WAVE;
  const int col = lane & 15;  // key (B column) / head row (A row) within a 16-tile
  const int grp = lane >> 4;  // 32-byte k-slice of the 128-byte row
  const int seq = row_seq[r];

  int64_t p_first = 0;
  if (PAGED) {
    p_first = page_shift >= 0 ? (wg_begin >> page_shift) : wg_begin / page_size;
    const int64_t p_last = page_shift >= 0 ? ((wg_end - 1) >> page_shift) : (wg_end - 1) / page_size;
    const int np = (int)(p_last - p_first + 1);
    for (int i = tid; i < np; i += kIdxWaves * WAVE) spage[i] = table[(int64_t)seq * max_pages + p_first + i];
    __syncthreads();
  }

  // A operand: q[r, 16*ht + col, 32*grp .. 32*grp+31] (e4m3 bytes); result rows held by
  // this lane are heads 16*ht + 4*grp + i.
  for (int i = tid; i < 64 * 128 / 16; i += kIdxWaves * WAVE)
    reinterpret_cast<uint4*>(sq)[i] = reinterpret_cast<const uint4*>(q + (int64_t)r * (64 * 128))[i];
  if (tid < 64) sw[tid] = w[(int64_t)r * 64 + tid];
  __syncthreads();
  v8i qa[4];
  float wr[4][4];
  load_query(sq, sw, col, grp, qa, wr);
  const float qs = q_scale ? q_scale[r] : 1.0f;
  int64_t wbeg, wend;
  if (COMPACT) {  // wave w of a chunk of nt trips: trips [w * nt / 8, (w + 1) * nt / 8)
    const int nt = (int)((wg_full - wg_begin) / kIdxBatch);
    wbeg = wg_begin + (int64_t)kIdxBatch * (wave * nt / kIdxWaves);
    wend = min(wg_begin + (int64_t)kIdxBatch * ((wave + 1) * nt / kIdxWaves), n);
  } else {
    const int per_wave = keys_per_wg / kIdxWaves;
    wbeg = wg_begin + (int64_t)wave * per_wave;
    wend = min(wbeg + per_wave, n);
  }

  auto row_of = [&](int64_t s) -> int64_t {
    if (PAGED) {
      const int64_t pg = page_shift >= 0 ? (s >> page_shift) : s / page_size;
      const int64_t off = page_shift >= 0 ? (s & (page_size - 1)) : s % page_size;
      return (int64_t)spage[pg - p_first] * page_size + off;
    }
    return (int64_t)seq * seq_stride + s;
  };

  // The score of key s0 + lane (s0 < wend; lanes past wend return the last key's score).
  auto trip = [&](int64_t s0) -> float {
    // Addresses are clamped to the last valid key instead of branching, so every load issues.
    // Keys are read once per call.  Contiguous caches stream them with non-temporal loads
    // (faster here, and the later kernels of the step run faster too); paged caches, whose
    // keys come in 8 KB pages scattered over the pool, measured slower that way and use
    // ordinary loads.
    v8i kb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t row = row_of(min(s0 + 16 * u + col, wend - 1));
      const v4i* p = reinterpret_cast<const v4i*>(kdata + row * 128 + 32 * grp);
      v4i a, b;
      if (PAGED) {
        a = p[0];
        b = p[1];
      } else {
        a = __builtin_nontemporal_load(p);
        b = __builtin_nontemporal_load(p + 1);
      }
      kb[u] = v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
    const float ks = kscale ? kscale[row_of(min(s0 + lane, wend - 1))] : 1.0f;
    return scaled_score(trip_scores(qa, wr, kb), ks, qs);
  };

  if (!COMPACT) {
    float* srow = scores + (int64_t)r * ld;
    for (int64_t s0 = wbeg; s0 < wend; s0 += kIdxBatch) {
      const float score = trip(s0);
      if (s0 + lane < wend) srow[s0 + lane] = score;
    }
    return;
  }

  // ---- compaction.  The trips' keys are parked in LDS (registers are what limits this kernel
  // to two workgroups per CU); 0 stands for "no key" and is below every real score's key.
  uint32_t* s_key = pool;  // [wave][trip][lane]
  int nt = 0;
  for (int64_t s0 = wbeg; s0 < wend; s0 += kIdxBatch, ++nt) {
    const float score = trip(s0);
    s_key[(wave * kCompactTrips + nt) * kIdxBatch + lane] = s0 + lane < wend ? float_key(score) : 0u;
  }
  __shared__ uint32_t s_theta;
  if (tid == 0) {
    uint64_t v = 0;
    bool ok = false;
    for (int it = 0; it < kThetaPolls && !ok; ++it) {
      v = __hip_atomic_load(&ready[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = (uint32_t)(v >> 32) == kThetaReady;
      if (!ok) __builtin_amdgcn_s_sleep(32);
    }
    // No threshold: keep nothing; the recorded theta cannot match the row's, so the resolve
    // rescores the row.
    s_theta = ok ? (uint32_t)v : 0xFFFFFFFFu;
  }
  __syncthreads();
  const uint32_t theta = s_theta;
  __shared__ int s_cnt[2][kIdxWaves];
  int lgt = 0, leq = 0;  // per-lane counts, summed over the wave once
  for (int t = 0; t < nt; ++t) {
    const uint32_t key = s_key[(wave * kCompactTrips + t) * kIdxBatch + lane];
    lgt += key > theta ? 1 : 0;
    leq += key == theta ? 1 : 0;
  }
  const int gt = (int)wave_reduce((uint32_t)lgt, UAdd{}), eq = (int)wave_reduce((uint32_t)leq, UAdd{});
  if (lane == 0) {
    s_cnt[0][wave] = gt;
    s_cnt[1][wave] = eq;
  }
  __syncthreads();
  int off, G, E;
  wave_offsets<kIdxWaves>(s_cnt[0], s_cnt[1], wave, off, G, E);
  uint2* cr = cand + (int64_t)r * ld + wg_begin;
  for (int t = 0; t < nt; ++t) {
    const uint32_t key = s_key[(wave * kCompactTrips + t) * kIdxBatch + lane];
    const bool keep = key >= theta;
    const uint64_t km = ballot(keep);
    if (keep) cr[off + mask_rank(km)] = make_uint2(key, (uint32_t)(wbeg + (int64_t)t * kIdxBatch + lane));
    off += __popcll(km);
  }
  if (tid == 0) counts[(int64_t)r * n_chunks + chunk] = ChunkCount{(uint32_t)G, (uint32_t)E, theta, 0u};
}

// Many rows (prefill): one workgroup scores kRowsPerWg consecutive rows against one key range.
// When the rows share a sequence (prefill rows do) a copy wave stages each 64-key trip once in
// LDS with global_load_lds and every compute wave (one row each) reads it from there, so a key
// crosses the vector-memory path once per workgroup instead of once per row; rows of
// different sequences fall back to loading their own keys.  Trip layout: block 2*u + h
// (1 KB) holds, at lane position col + 16*grp, bytes 32*grp + 16*h .. +15 of key 16*u + col --
// the k-slice load_query gives the query operand -- so a 64-lane ds_read_b128 of a block is
// one contiguous, conflict-free 1 KB; the 64 key scales follow.  Ring of three trips, two in flight; the slots are separate LDS variables and the
// loop is unrolled by three so every slot is a compile-time variable (the copy wave never
// reads the ring, the compute waves issue no copies).
// Seven rows plus the copy wave make eight waves, so two workgroups fit a CU at this kernel's
// register use (eight rows and nine waves allowed only one).
constexpr int kRowsPerWg = 7;
constexpr int kRowsKernelMin = 512;  // calls with at least this many rows use the kernel below
constexpr int kRowsThreads = (kRowsPerWg + 1) * WAVE;
constexpr int kTripBytes = kIdxBatch * 128 + kIdxBatch * 4;
constexpr int kKeyRing = 3;
__shared__ __attribute__((aligned(16))) char g_kring0[kTripBytes];
__shared__ __attribute__((aligned(16))) char g_kring1[kTripBytes];
__shared__ __attribute__((aligned(16))) char g_kring2[kTripBytes];
template <int S>
__device__ __forceinline__ char* key_slot() {
  return S == 0 ? g_kring0 : (S == 1 ? g_kring1 : g_kring2);
}
template <int S>
struct KeySlot {
  static constexpr int value = S;
};
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ uint32_t lds_offset(const void* p) { return (uint32_t)(uintptr_t)p; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <bool PAGED>
__global__ __launch_bounds__(kRowsThreads) void index_fp8_rows_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ kdata, const float* __restrict__ kscale,
    const int32_t* __restrict__ table, int max_pages, int page_size, int page_shift,
    int64_t seq_stride, const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos,
    int R, float* __restrict__ scores, int64_t ld, int keys_per_wg) {
  extern __shared__ int spage[];  // paged, shared rows: physical page of each logical page
  const int r0 = blockIdx.x * kRowsPerWg;
  const int nrows = min(kRowsPerWg, R - r0);
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
  const int col = lane & 15, grp = lane >> 4;
  // Every thread reads the workgroup's row list (uniform values).
  int seq0 = row_seq[r0];
  bool shared = true;
  int64_t n_max = 0;
  for (int i = 0; i < nrows; ++i) {
    shared = shared && row_seq[r0 + i] == seq0;
    n_max = max(n_max, (int64_t)row_pos[r0 + i] + 1);
  }
  const int64_t c0 = (int64_t)blockIdx.y * keys_per_wg;
  if (c0 >= n_max) return;
  const int64_t c1 = min(c0 + keys_per_wg, n_max);  // keys scored by this workgroup
  const int my_r = r0 + min(wv, nrows - 1);
  const bool my_valid = wv < nrows;
  const int64_t my_n = my_valid ? (int64_t)row_pos[my_r] + 1 : 0;

  auto row_in = [&](int seq, int64_t s, const int* pages, int64_t p_first) -> int64_t {
    if (PAGED) {
      const int64_t pg = page_shift >= 0 ? (s >> page_shift) : s / page_size;
      const int64_t off = page_shift >= 0 ? (s & (page_size - 1)) : s % page_size;
      const int phys = pages ? pages[pg - p_first] : table[(int64_t)seq * max_pages + pg];
      return (int64_t)phys * page_size + off;
    }
    return (int64_t)seq * seq_stride + s;
  };

  if (!shared) {
    // Rows of different sequences: wave wv scores its own row over [c0, min(c1, n_w)) with
    // direct key loads.
    if (wv >= kRowsPerWg || !my_valid) return;
    const int seq = row_seq[my_r];
    const int64_t end = min(c1, my_n);
    if (c0 >= end) return;
    v8i qa[4];
    float wr[4][4];
    load_query(q + (int64_t)my_r * (64 * 128), w + (int64_t)my_r * 64, col, grp, qa, wr);
    const float qs = q_scale ? q_scale[my_r] : 1.0f;
    float* srow = scores + (int64_t)my_r * ld;
    for (int64_t s0 = c0; s0 < end; s0 += kIdxBatch) {
      v8i kb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t row = row_in(seq, min(s0 + 16 * u + col, end - 1), nullptr, 0);
        const uint4* p = reinterpret_cast<const uint4*>(kdata + row * 128 + 32 * grp);
        const uint4 a = p[0], b = p[1];
        kb[u] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
      }
      const int64_t s_out = s0 + lane;
      const float ks = kscale ? kscale[row_in(seq, min(s_out, end - 1), nullptr, 0)] : 1.0f;
      const float tot = trip_scores(qa, wr, kb);
      if (s_out < end) srow[s_out] = scaled_score(tot, ks, qs);
    }
    return;
  }

  // Shared sequence.  Paged: the workgroup's page-table slice goes to LDS first.
  int64_t p_first = 0;
  if (PAGED) {
    p_first = page_shift >= 0 ? (c0 >> page_shift) : c0 / page_size;
    const int64_t p_last = page_shift >= 0 ? ((c1 - 1) >> page_shift) : (c1 - 1) / page_size;
    for (int i = tid; i <= (int)(p_last - p_first); i += kRowsThreads)
      spage[i] = table[(int64_t)seq0 * max_pages + p_first + i];
    __syncthreads();
  }
  const int ntrips = (int)((c1 - c0 + kIdxBatch - 1) / kIdxBatch);

  if (wv == kRowsPerWg) {
    // ---------------------------------------------------------------- copy wave
    // Lane (col, grp) of block 2u + h fetches bytes 32*grp + 16*h of key 16u + col; lane l
    // of the scale copy fetches key l's scale (4 bytes).
    auto issue = [&](int t, char* dst) {
      const int64_t s0 = c0 + (int64_t)t * kIdxBatch;
      const uint32_t d = lds_offset(dst);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t row = row_in(seq0, min(s0 + 16 * u + col, c1 - 1), PAGED ? spage : nullptr, p_first);
        const uint8_t* src = kdata + row * 128 + 32 * grp;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          __builtin_amdgcn_global_load_lds((const void*)(src + 16 * h), (lds_void*)(uintptr_t)(d + (2 * u + h) * 1024), 16, 0, 0);
      }
      if (kscale) {
        const int64_t row = row_in(seq0, min(s0 + lane, c1 - 1), PAGED ? spage : nullptr, p_first);
        __builtin_amdgcn_global_load_lds((const void*)(kscale + row), (lds_void*)(uintptr_t)(d + 8192), 4, 0, 0);
      }
    };
    if (ntrips > 0) issue(0, key_slot<0>());
    if (ntrips > 1) issue(1, key_slot<1>());
    auto hand = [&](auto slot, int t) {
      constexpr int S = decltype(slot)::value;
      if (t + 1 < ntrips) {  // trip t landed, t+1 may be in flight
        if (kscale) wait_vmcnt<9>(); else wait_vmcnt<8>();
      } else {
        wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_barrier();
      if (t + 2 < ntrips) issue(t + 2, key_slot<(S + 2) % kKeyRing>());
    };
    for (int t = 0; t < ntrips; t += kKeyRing) {
      hand(KeySlot<0>{}, t);
      if (t + 1 < ntrips) hand(KeySlot<1>{}, t + 1);
      if (t + 2 < ntrips) hand(KeySlot<2>{}, t + 2);
    }
    return;
  }

  // ------------------------------------------------------------------ compute waves
  v8i qa[4];
  float wr[4][4];
  load_query(q + (int64_t)my_r * (64 * 128), w + (int64_t)my_r * 64, col, grp, qa, wr);
  const float qs = (q_scale && my_valid) ? q_scale[my_r] : 1.0f;
  const int64_t end = min(c1, my_n);
  float* srow = scores + (int64_t)my_r * ld;
  auto step = [&](auto slot, int t) {
    constexpr int S = decltype(slot)::value;
    __builtin_amdgcn_s_barrier();  // trip t is in slot S
    const char* tb = key_slot<S>();
    v8i kb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 a = *reinterpret_cast<const uint4*>(tb + (2 * u) * 1024 + 16 * lane);
      const uint4 b = *reinterpret_cast<const uint4*>(tb + (2 * u + 1) * 1024 + 16 * lane);
      kb[u] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    }
    const float ks = kscale ? *reinterpret_cast<const float*>(tb + 8192 + 4 * lane) : 1.0f;
    const float tot = trip_scores(qa, wr, kb);
    const int64_t s_out = c0 + (int64_t)t * kIdxBatch + lane;
    if (s_out < end) srow[s_out] = scaled_score(tot, ks, qs);
  };
  for (int t = 0; t < ntrips; t += kKeyRing) {
    step(KeySlot<0>{}, t);
    if (t + 1 < ntrips) step(KeySlot<1>{}, t + 1);
    if (t + 2 < ntrips) step(KeySlot<2>{}, t + 2);
  }
}

// Any H_I, d_I; fp32 or e4m3 operands.  One thread per key; the query row sits in LDS.
template <bool FP8>
__global__ __launch_bounds__(256) void index_generic_kernel(
    const void* __restrict__ qv, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ kv, const float* __restrict__ kscale, const int32_t* __restrict__ table,
    int max_pages, int page_size, int64_t seq_stride, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int HI, int dI, float* __restrict__ scores, int64_t ld) {
  extern __shared__ float sq[];  // [HI*dI] query row, then [HI] weights
  const int r = blockIdx.x;
  const int64_t n = (int64_t)row_pos[r] + 1;
  const int64_t base = (int64_t)blockIdx.y * blockDim.x;
  if (base >= n) return;
  for (int i = threadIdx.x; i < HI * dI; i += blockDim.x) {
    const int64_t o = (int64_t)r * HI * dI + i;
    sq[i] = FP8 ? e4m3_to_f32(static_cast<const uint8_t*>(qv)[o]) : static_cast<const float*>(qv)[o];
  }
  for (int j = threadIdx.x; j < HI; j += blockDim.x) sq[HI * dI + j] = w[(int64_t)r * HI + j];
  __syncthreads();
  const int64_t s = base + threadIdx.x;
  if (s >= n) return;
  const int seq = row_seq[r];
  int64_t row;
  if (table) {
    row = (int64_t)table[(int64_t)seq * max_pages + s / page_size] * page_size + s % page_size;
  } else {
    row = (int64_t)seq * seq_stride + s;
  }
  float acc = 0.0f;
  for (int j = 0; j < HI; ++j) {
    float dot = 0.0f;
    for (int d = 0; d < dI; ++d) {
      const float kd = FP8 ? e4m3_to_f32(static_cast<const uint8_t*>(kv)[row * dI + d])
                           : static_cast<const float*>(kv)[row * dI + d];
      dot = fmaf(sq[j * dI + d], kd, dot);
    }
    acc = fmaf(sq[HI * dI + j], fmaxf(dot, 0.0f), acc);
  }
  const float ks = kscale ? kscale[row] : 1.0f;
  const float qs = q_scale ? q_scale[r] : 1.0f;
  scores[(int64_t)r * ld + s] = acc * ks * qs;
}

}  // namespace

int index_rows_kernel_min() { return kRowsKernelMin; }

// Keys per workgroup of the one-row-per-workgroup indexer: ~512 workgroups of 8 waves (two
// per CU at its register use); each wave's share is a multiple of the 64-key trip.
int index_keys_per_wg(int R, int64_t n_bound) {
  const int64_t total = (int64_t)R * n_bound;
  int64_t kpw = 512;
  while (kpw < 64 * kIdxWaves * kCompactTrips && total / (kpw * 2) >= 512) kpw *= 2;
  return (int)kpw;
}

hipError_t launch_index_fp8_h64d128(const uint8_t* q, const float* q_scale, const float* w,
                                    const CacheView& keys, const int32_t* row_seq,
                                    const int32_t* row_pos, int R, int64_t n_bound, float* scores,
                                    int64_t ld, hipStream_t s) {
  const uint8_t* kd = static_cast<const uint8_t*>(keys.data);
  if (R >= kRowsKernelMin) {
    // Many rows: seven rows per workgroup sharing staged key trips; 4096 keys per workgroup.
    const int64_t kpw = 4096;
    const dim3 grid((unsigned)((R + kRowsPerWg - 1) / kRowsPerWg), (unsigned)((n_bound + kpw - 1) / kpw));
    if (keys.table) {
      const int ps = keys.page_size;
      const int shift = (ps & (ps - 1)) == 0 ? __builtin_ctz(ps) : -1;
      const size_t lds = sizeof(int) * (size_t)(kpw / ps + 2);
      index_fp8_rows_kernel<true><<<grid, kRowsThreads, lds, s>>>(
          q, q_scale, w, kd, keys.scale, keys.table, keys.max_pages, ps, shift, 0, row_seq, row_pos,
          R, scores, ld, (int)kpw);
    } else {
      index_fp8_rows_kernel<false><<<grid, kRowsThreads, 0, s>>>(
          q, q_scale, w, kd, keys.scale, nullptr, 0, 1, 0, keys.seq_stride, row_seq, row_pos, R,
          scores, ld, (int)kpw);
    }
    return hipGetLastError();
  }
  const int kpw = index_keys_per_wg(R, n_bound);
  const int n_chunks = (int)((n_bound + kpw - 1) / kpw);
  const unsigned grid = (unsigned)R * (unsigned)n_chunks;
  if (keys.table) {
    const int ps = keys.page_size;
    const int shift = (ps & (ps - 1)) == 0 ? __builtin_ctz(ps) : -1;
    const size_t lds = sizeof(int) * (size_t)(kpw / ps + 2);
    index_fp8_kernel<true><<<grid, kIdxWaves * WAVE, lds, s>>>(
        q, q_scale, w, kd, keys.scale, keys.table, keys.max_pages, ps, shift, 0, row_seq, row_pos,
        scores, ld, kpw, n_chunks);
  } else {
    index_fp8_kernel<false><<<grid, kIdxWaves * WAVE, 0, s>>>(
        q, q_scale, w, kd, keys.scale, nullptr, 0, 1, 0, keys.seq_stride, row_seq, row_pos, scores,
        ld, kpw, n_chunks);
  }
  return hipGetLastError();
}

// Resident workgroups of this kernel on the chip: two per CU (its register use) x 256 CUs.
constexpr int kIndexSlots = 512;

int index_compact_chunks(int R, int64_t n_bound) {
  const int64_t tb = (n_bound + kIdxBatch - 1) / kIdxBatch;
  const int64_t nc_min = (tb + kIdxWaves * kCompactTrips - 1) / (kIdxWaves * kCompactTrips);  // <= 8 trips per wave
  const int64_t nc_max = tb / kIdxWaves > 1 ? tb / kIdxWaves : 1;                              // >= 1 trip per wave
  // The sample blocks and every chunk of every row in one resident round, when they fit.
  const int64_t fill = R < kIndexSlots ? (kIndexSlots - R) / R : 1;
  const int64_t nc = fill < nc_max ? fill : nc_max;
  return (int)(nc > nc_min ? nc : nc_min);
}

hipError_t launch_index_fp8_compact(const uint8_t* q, const float* q_scale, const float* w,
                                    const CacheView& keys, const int32_t* row_seq,
                                    const int32_t* row_pos, int R, int64_t n_bound, int64_t ld,
                                    RowHeader* hdr, uint64_t* ready, ChunkCount* counts, uint2* cand,
                                    int min_n, hipStream_t s) {
  const uint8_t* kd = static_cast<const uint8_t*>(keys.data);
  const int tb = (int)((n_bound + kIdxBatch - 1) / kIdxBatch);
  const int n_chunks = index_compact_chunks(R, n_bound);
  const int max_keys = kIdxBatch * ((tb + n_chunks - 1) / n_chunks);  // longest chunk
  const unsigned grid = (unsigned)R + (unsigned)R * (unsigned)n_chunks;  // sample blocks first
  if (keys.table) {
    const int ps = keys.page_size;
    const int shift = (ps & (ps - 1)) == 0 ? __builtin_ctz(ps) : -1;
    const size_t lds = sizeof(int) * (size_t)(max_keys / ps + 2);
    index_fp8_kernel<true, true><<<grid, kIdxWaves * WAVE, lds, s>>>(
        q, q_scale, w, kd, keys.scale, keys.table, keys.max_pages, ps, shift, 0, row_seq, row_pos,
        nullptr, ld, tb, n_chunks, hdr, ready, counts, cand, min_n, R);
  } else {
    index_fp8_kernel<false, true><<<grid, kIdxWaves * WAVE, 0, s>>>(
        q, q_scale, w, kd, keys.scale, nullptr, 0, 1, 0, keys.seq_stride, row_seq, row_pos, nullptr,
        ld, tb, n_chunks, hdr, ready, counts, cand, min_n, R);
  }
  return hipGetLastError();
}

hipError_t launch_index_generic(bool fp8, const void* q, const float* q_scale, const float* w,
                                const CacheView& keys, const int32_t* row_seq, const int32_t* row_pos,
                                int R, int HI, int dI, int64_t n_bound, float* scores, int64_t ld,
                                hipStream_t s) {
  const dim3 grid((unsigned)R, (unsigned)((n_bound + 255) / 256));
  const size_t lds = sizeof(float) * ((size_t)HI * dI + HI);
  if (fp8)
    index_generic_kernel<true><<<grid, 256, lds, s>>>(q, q_scale, w, keys.data, keys.scale, keys.table,
                                                      keys.max_pages, keys.page_size, keys.seq_stride,
                                                      row_seq, row_pos, HI, dI, scores, ld);
  else
    index_generic_kernel<false><<<grid, 256, lds, s>>>(q, q_scale, w, keys.data, keys.scale, keys.table,
                                                       keys.max_pages, keys.page_size, keys.seq_stride,
                                                       row_seq, row_pos, HI, dI, scores, ld);
  return hipGetLastError();
}

}  // namespace dsa
