// Exact per-row top-k token selection (ties -> lower index) for the DSA pipeline.
//
// The pages fix that each query keeps k key/value pairs chosen from the indexer's
// scores at token granularity (maplevalley.com.cn news 1594152, section 1 "Top-k
// Token Selection"; tellworld.net "What happened": fine-grained, not blocks; k = 2048
// in MarkTechPost's "Training signal" paragraph).  The tie rule and the output order
// (ascending index, -1 padded) are this library's.
//
// Method: the radix select and ordered emit of select_core.h.
//
// Rows up to kRowMax scores (up to kLongMinWs when the call's rows are longer than kRowMax, so
// the compaction workspace exists) are selected by one workgroup that holds the row in
// registers (read from memory once) and keeps only the histograms in LDS.  Longer rows
// (decode at 128k context) take a sampled compaction: a threshold theta whose expected
// survivor count is ~2k comes from an evenly spaced sample of 2048 scores; many workgroups
// per row compact the survivors (in index order, counting those above theta and those equal
// to it per chunk); one workgroup per row then resolves them.  The hand-offs are kernel
// boundaries: an in-kernel device-scope fence costs a whole-L2 writeback and invalidate on
// this chip.  The resolve has three cases:
//   * theta is the threshold itself (fewer than k keys above it, at least k at or above it,
//     as on a row of equal scores): every key above theta and the first keys equal to it
//     are taken, copied straight from the chunks' candidate slots;
//   * up to 12288 survivors: they are gathered into LDS, histogrammed into 4096 bins above
//     theta on the way, so the bin holding the k-th largest is known after one block scan,
//     and the few keys of that bin are ranked by direct comparison;
//   * otherwise (fewer than k survivors, or too many with at least k above theta): the
//     radix select over the whole row in global memory.
// Correctness never depends on the sample, only the speed does.
//
// The fused index + top-k call runs the same resolve without any score row: the compacting
// indexer (indexer.hip, COMPACT) scores each row's sample in workgroups of its own and
// compacts the survivors as it scores; the resolve checks that every chunk used the row's
// threshold, and its last case rescores the row into the candidate buffer first.
#include "common.h"
#include "kernels.h"
#include "score_core.h"
#include "select_core.h"

namespace dsa {
namespace {

constexpr int kRowMax = 32768;     // longest row selected by one workgroup (32 keys per thread)
constexpr int kSample = 2048;      // sample size for longer rows (from stored score rows)
constexpr int kChunk = 4096;       // scores per workgroup in the long-row compaction pass
// When the call has a candidate workspace (ld > kRowMax), rows longer than this already take
// the sampled compaction: a single workgroup's multi-pass radix select over 8k..32k scores
// is slower than the compaction and resolve.
constexpr int kLongMinWs = 8192;
constexpr int kCandCap = 12288;    // survivors resolvable in LDS (96 KiB of key/index pairs)
constexpr int kTieMax = 256;       // largest boundary bin ranked by pairwise comparison
constexpr int kFusedMaxChunks = 4096;  // chunk offsets of a fused call's row that fit the resolve's LDS
constexpr int kRowThreads = 1024;
constexpr int kLongThreads = 256;  // compaction workgroups
constexpr int kResolveThreads = 1024;


// Long rows, pass 1 (R x chunks workgroups): every workgroup of a row derives the same
// sample threshold theta (about 2k survivors expected) from kSample evenly spaced scores
// (positions (i * n) / kSample)
// while the loads of its own 4096-score chunk are in flight, then compacts the chunk's
// survivors (key >= theta) in index order into the chunk's slot of the candidate buffer and
// records how many of them lie above theta and how many equal it.  Chunk 0 also records the
// row header for the resolve.  n = n_valid[r] + n_off.
__global__ __launch_bounds__(kLongThreads) void topk_prep_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ n_valid, int k,
    RowHeader* __restrict__ hdr, ChunkCount* __restrict__ counts, int max_chunks,
    uint2* __restrict__ cand, int n_off, int long_min) {
  __shared__ uint32_t samp[kSample];
  __shared__ __attribute__((aligned(16))) int hist[kPassMax * kHistBins];
  __shared__ SelState st;
  constexpr int NW = kLongThreads / WAVE;
  // Block b takes chunk b % max_chunks of row b / max_chunks, so consecutive blocks (dealt
  // round-robin to the eight XCDs) walk along a row and rows of different lengths spread
  // evenly over the XCDs.
  const int r = blockIdx.x / max_chunks;
  const int c = blockIdx.x % max_chunks;
  int64_t n64 = (int64_t)n_valid[r] + n_off;
  n64 = n64 < 0 ? 0 : (n64 > ld ? ld : n64);
  const int n = (int)n64;
  if (n <= long_min || n <= k) return;
  const int nch = (n + kChunk - 1) / kChunk;
  if (c >= nch) return;
  const float* row = scores + (int64_t)r * ld;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int base = c * kChunk;
  const int end = min(n, base + kChunk);
  constexpr int per = kChunk / NW;
  constexpr int kIter = per / WAVE;
  const int wb = base + w * per;
  // The chunk's keys stay in registers from here to the compaction.
  uint32_t key[kIter];
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int e = wb + it * WAVE + lane;
    key[it] = float_key(row[min(e, end - 1)]);  // unconditional: all loads in flight at once
  }
  uint32_t lmn = 0xFFFFFFFFu, lmx = 0u;
  {
    constexpr int kPer = kSample / kLongThreads;
    uint32_t kv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) kv[u] = float_key(row[(int64_t)(tid + u * kLongThreads) * n / kSample]);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      samp[tid + u * kLongThreads] = kv[u];
      lmn = min(lmn, kv[u]);
      lmx = max(lmx, kv[u]);
    }
  }
  const RowHeader rh = sample_header<kLongThreads>(samp, kSample, 2, lmn, lmx, n, k, hist, st);
  const uint32_t theta = rh.theta;
  if (c == 0 && tid == 0) hdr[r] = rh;
  int lgt = 0, leq = 0;  // per-lane counts, summed over the wave once
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const bool in = wb + it * WAVE + lane < end;
    lgt += (in & (key[it] > theta)) ? 1 : 0;
    leq += (in & (key[it] == theta)) ? 1 : 0;
  }
  const int gt = (int)wave_reduce((uint32_t)lgt, UAdd{}), eq = (int)wave_reduce((uint32_t)leq, UAdd{});
  if (lane == 0) {
    st.wtot[0][w] = gt;
    st.wtot[1][w] = eq;
  }
  __syncthreads();
  int off, G, E;
  wave_offsets<NW>(st.wtot[0], st.wtot[1], w, off, G, E);
  uint2* cr = cand + (int64_t)r * ld + base;
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int e = wb + it * WAVE + lane;
    const bool keep = e < end && key[it] >= theta;
    const uint64_t km = ballot(keep);
    if (keep) cr[off + mask_rank(km)] = make_uint2(key[it], (uint32_t)e);
    off += __popcll(km);
  }
  if (tid == 0) counts[(int64_t)r * max_chunks + c] = ChunkCount{(uint32_t)G, (uint32_t)E, theta, 0u};
}

// Exact top-k among `total` survivors (keys/ids in LDS, in index order) that all lie at or
// above theta and have been histogrammed into kSurvBins bins of 2^shift keys above theta
// (the last bin open-ended).  One block scan finds the bin b* holding the k-th largest;
// its keys are then ranked directly, or by the radix select when there are too many.  The
// caller has passed a barrier since the histogram was complete and has cleared st.ntie.
__device__ __forceinline__ void select_survivors(const uint32_t* keys, const int* ids, int total, uint32_t theta,
                                 uint32_t shift, int k, int* hist, uint2* ties, SelState& st,
                                 int32_t* __restrict__ out) {
  constexpr int NW = kResolveThreads / WAVE;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  // Bin b* of the k-th largest survivor: thread t holds bins 4095-4t .. 4092-4t (top down);
  // every wave then finds the crossing wave from the per-wave totals and rescans its bins.
  const int4 hv = reinterpret_cast<const int4*>(hist)[kResolveThreads - 1 - tid];
  const int incl = wave_incl_scan(hv.x + hv.y + hv.z + hv.w);
  if (lane == WAVE - 1) st.wscan[w] = incl;
  __syncthreads();
  int before, vc;
  crossing_wave<NW>(st.wscan, k, vc, before);
  const int4 hc = reinterpret_cast<const int4*>(hist)[kResolveThreads - 1 - (vc * WAVE + lane)];
  const int cb[4] = {hc.w, hc.z, hc.y, hc.x};
  int bstar, above, bcnt;
  wave_crossing<4>(cb, kSurvBins - 1 - 4 * (vc * WAVE + lane), before, k, bstar, above, bcnt);
  const int need = k - above;
  const uint32_t t_lo = theta + ((uint32_t)bstar << shift);  // first key of bin b*
  const LdsPairs src{keys, ids};
  Threshold th;
  if (bcnt == need) {
    th = Threshold{t_lo, 0, true, 0u};  // all of bin b* and above: { key >= t_lo }
  } else if (bcnt <= kTieMax) {
    // Rank the keys of bin b* by (key descending, position ascending); the one of rank
    // need-1 is the threshold T, and need - (keys of the bin above T) of those equal to T
    // are taken, lowest position first -- the same rule as emit_selected.  The pass that
    // gathers the bin's keys already walks the survivors in the emit pass's wave ranges and
    // counts each range's keys above the bin, and the bin's own keys are all in `ties`, so
    // the emit needs no counting pass and no barrier of its own.
    const uint64_t bin_end = (uint64_t)t_lo + ((uint64_t)1 << shift) - 1;  // may pass 2^32
    const uint32_t t_hi = (bstar == kSurvBins - 1 || bin_end > 0xFFFFFFFFull) ? 0xFFFFFFFFu : (uint32_t)bin_end;
    const int per = ((total + NW - 1) / NW + WAVE - 1) / WAVE * WAVE;
    const int beg = w * per;
    const int end = min(total, beg + per);
    int above_l = 0;  // this lane's count, summed over the wave after the pass
    for (int i0 = beg; i0 < end; i0 += 4 * WAVE) {
      uint32_t kv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) kv[u] = keys[min(i0 + u * WAVE + lane, end - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * WAVE + lane;
        const bool ok = i < end;
        above_l += (ok & (kv[u] > t_hi)) ? 1 : 0;
        const bool in = ok & (kv[u] >= t_lo) & (kv[u] <= t_hi);
        const uint64_t im = ballot(in);
        if (im) {  // one slot reservation per wave and round
          int slot = 0;
          if (lane == 0) slot = atomicAdd(&st.ntie, __popcll(im));
          slot = readlane(slot, 0);
          if (in) ties[slot + mask_rank(im)] = make_uint2(kv[u], (uint32_t)i);
        }
      }
    }
    const int above_w = (int)wave_reduce((uint32_t)above_l, UAdd{});
    if (lane == 0) st.wtot[0][w] = above_w;
    __syncthreads();
    if (tid < bcnt) {
      const uint2 me = ties[tid];
      int gt = 0, eq_before = 0;
      for (int j = 0; j < bcnt; ++j) {
        const uint2 o = ties[j];
        gt += o.x > me.x;
        eq_before += (o.x == me.x) & (o.y < me.y);
      }
      if (gt + eq_before == need - 1) {
        st.tie_T = me.x;
        st.tie_need = need - gt;
      }
    }
    __syncthreads();
    const uint32_t T = st.tie_T;
    const int tneed = st.tie_need;
    // Selected before this wave's range: every range's keys above the bin, the bin's keys
    // above T at lower positions, and the first of those equal to T (up to tneed).
    int g = 0, b = 0;
    for (int e0 = 0; e0 < bcnt; e0 += WAVE) {
      const int e = e0 + lane;
      const uint2 o = ties[min(e, bcnt - 1)];
      const bool ok = (e < bcnt) & ((int)o.y < beg);
      g += __popcll(ballot(ok & (o.x > T)));
      b += __popcll(ballot(ok & (o.x == T)));
    }
    const int ab_v = lane < NW ? st.wtot[0][lane] : 0;
    const int ab_before = readlane(wave_incl_scan(ab_v) - ab_v, w);
    int sel_run = ab_before + g + min(b, tneed);
    int eq_run = b;
    for (int i0 = beg; i0 < end; i0 += 4 * WAVE) {
      uint32_t kv[4];
      int iv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = min(i0 + u * WAVE + lane, end - 1);
        kv[u] = keys[e];
        iv[u] = ids[e];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = i0 + u * WAVE + lane < end;
        const bool eq = ok & (kv[u] == T);
        const uint64_t eqm = ballot(eq);
        const bool sel = (ok & (kv[u] > T)) | (eq & (eq_run + mask_rank(eqm) < tneed));
        const uint64_t selm = ballot(sel);
        if (sel) out[sel_run + mask_rank(selm)] = iv[u];
        eq_run += __popcll(eqm);
        sel_run += __popcll(selm);
      }
    }
    return;
  } else {
    __syncthreads();  // every wave has read the survivor histogram before the radix select clears it
    th = find_threshold<kResolveThreads>(src, total, k, hist, st);
  }
  emit_selected<kResolveThreads>(src, total, th, st, out);
}

// Rows of at most kRowMax scores (one workgroup each): the radix select and the emit pass
// above with the row held in registers -- wave w holds the contiguous index range
// [w*per, w*per + per) in rounds of 64, KPT keys per thread -- so the row is read from
// memory once and only the histograms live in LDS.  The loads are unconditional (clamped
// to the last element) so they all issue back to back; a branch around each would make the
// compiler wait for each in turn.
template <int KPT>
__device__ __forceinline__ void select_mid_row(const float* __restrict__ row, int n, int k, int32_t* __restrict__ out,
                               int* hist, SelState& st) {
  constexpr int NT = kRowThreads, NW = NT / WAVE;
  static_assert(KPT * NT <= kRowMax, "keys per thread");
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int per = ((n + NW - 1) / NW + WAVE - 1) / WAVE * WAVE;  // <= KPT * WAVE
  const int beg = w * per;
  const int end = min(n, beg + per);
  // Positions past the wave's range get key 0, below every non-NaN score's key (the key of
  // -inf is 0x007FFFFF), so no later pass needs a range test: they never reach a histogram
  // range or the threshold.
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) key[j] = float_key(row[min(beg + j * WAVE + lane, n - 1)]);
#pragma unroll
  for (int j = 0; j < KPT; ++j) key[j] = beg + j * WAVE + lane < end ? key[j] : 0u;
  uint32_t lmn = 0xFFFFFFFFu, lmx = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    lmn = min(lmn, key[j] ? key[j] : 0xFFFFFFFFu);
    lmx = max(lmx, key[j]);
  }
  publish_range<NT>(lmn, lmx, hist, st);
  __syncthreads();
  const uint32_t lo = block_min<NW>(st.wmin), hi = block_max<NW>(st.wmax);
  const Threshold th = radix_threshold<NT>(lo, hi, k, hist, st, 0, [&](uint32_t a, uint32_t b, int s, int* h) {
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if ((key[j] >= a) & (key[j] <= b)) atomicAdd(&h[(key[j] - a) >> s], 1);
  });
  // Emit: per-wave counts of keys above T and equal to T, then the waves' offsets from two
  // DPP scans (ties taken in wave order, lowest index first), then the ballot-ranked writes.
  const uint32_t T = th.T;
  const bool ex = th.exact;
  const int need = ex ? 0 : th.need;
  int lgt = 0, leq = 0;  // per-lane counts, summed over the wave once
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    lgt += ((key[j] > T) | (ex & (key[j] == T))) ? 1 : 0;
    leq += (!ex & (key[j] == T)) ? 1 : 0;
  }
  const int cgt = (int)wave_reduce((uint32_t)lgt, UAdd{}), ceq = (int)wave_reduce((uint32_t)leq, UAdd{});
  if (lane == 0) {
    st.wtot[0][w] = cgt;
    st.wtot[1][w] = ceq;
    st.wred[w] = T;
  }
  __syncthreads();
  // T comes back through LDS so the compiler recomputes the comparisons below instead of
  // keeping the count pass's 2 x KPT lane masks alive (in spilled scalar registers).
  const uint32_t T2 = st.wred[w];
  const int gt_v = lane < NW ? st.wtot[0][lane] : 0;
  const int eq_v = lane < NW ? st.wtot[1][lane] : 0;
  const int eq_before_v = wave_incl_scan(eq_v) - eq_v;
  const int take_v = min(max(need - eq_before_v, 0), eq_v);
  const int sel_v = gt_v + take_v;
  const int sel_before_v = wave_incl_scan(sel_v) - sel_v;
  const int eq_before = readlane(eq_before_v, w);
  int sel_run = readlane(sel_before_v, w);
  if (ex) {  // the selection is { key >= T }: no tie bookkeeping (the usual case)
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool sel = key[j] >= T2;
      const uint64_t selm = ballot(sel);
      if (sel) out[sel_run + mask_rank(selm)] = beg + j * WAVE + lane;
      sel_run += __popcll(selm);
    }
    return;
  }
  int eq_run = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool gt = key[j] > T2;
    const bool eq = key[j] == T2;
    const uint64_t eqm = ballot(eq);
    const bool sel = gt | (eq & (eq_before + eq_run + mask_rank(eqm) < need));
    const uint64_t selm = ballot(sel);
    if (sel) out[sel_run + mask_rank(selm)] = beg + j * WAVE + lane;
    eq_run += __popcll(eqm);
    sel_run += __popcll(selm);
  }
}

// Inputs of the indexer's fast shape, for the fused call's sample pass and its rescoring
// fallback (the same scoring core as the indexer: score_core.h).
struct Rescore {
  const uint8_t* q;        // [R, 64, 128] e4m3 codes
  const float* q_scale;    // [R] or null
  const float* w;          // [R, 64]
  const uint8_t* kdata;    // key cache, 128 bytes per row
  const float* kscale;     // per-row key scale or null
  KeyRows kr;
  const int32_t* row_seq;  // [R]
};

// Candidate-slot chunks of a row: the row bound's tb 64-key trips split into nc chunks,
// chunk j starting at position 64 * (j * tb / nc) (uniform 4096-position chunks: tb = 64 nc).
struct Chunks {
  int tb, nc;
  __device__ int start(int j) const {
    const uint64_t p = (uint64_t)(uint32_t)j * (uint32_t)tb;  // 32-bit division when it fits
    return 64 * (int)(p >> 32 ? p / (uint32_t)nc : (uint32_t)p / (uint32_t)nc);
  }
  // chunks holding positions below n
  __device__ int count(int n) const { return (int)((((int64_t)n + 63) / 64 * nc + tb - 1) / tb); }
};

// Scores positions 0 .. n-1 of row r into order-preserving keys keys_out[0 .. n) (all threads
// of the block; the caller publishes them with a barrier).
__device__ void rescore_row(const Rescore& rs, int r, int n, uint32_t* __restrict__ keys_out) {
  constexpr int NW = kResolveThreads / WAVE;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int col = lane & 15, grp = lane >> 4;
  v8i qa[4];
  float wr[4][4];
  load_query(rs.q + (int64_t)r * (64 * 128), rs.w + (int64_t)r * 64, col, grp, qa, wr);
  const float qs = rs.q_scale ? rs.q_scale[r] : 1.0f;
  const int seq = rs.row_seq[r];
  const int ntrips = (n + kIdxBatch - 1) / kIdxBatch;
  for (int t = w; t < ntrips; t += NW) {
    const int s0 = t * kIdxBatch;
    v8i kb[4];
    load_trip(rs.kdata, rs.kr, seq, col, grp, [&](int j) { return (int64_t)min(s0 + j, n - 1); }, kb);
    const float ks = rs.kscale ? rs.kscale[rs.kr.row(seq, min(s0 + lane, n - 1))] : 1.0f;
    const float sc = scaled_score(trip_scores(qa, wr, kb), ks, qs);
    if (s0 + lane < n) keys_out[s0 + lane] = float_key(sc);
  }
}

// Theta is the threshold itself: fewer than k keys above theta (G of them) and at least k at
// or above it.  Every key above theta is kept, and the first k - G keys equal to theta in
// position order.  Chunk j keeps its keys above theta and eqt_j of its keys equal to theta
// (those before it have taken pe[j]), from output offset pg[j] + min(pe[j], k - G).  When a
// chunk keeps a prefix of its slot -- it has no key equal to theta, or keeps all of them, or
// has only such keys -- its ids are copied straight out: output position p finds its chunk
// by binary search over the offsets.  Any other chunk is walked by one wave with ballots.
__device__ void emit_theta_boundary(const uint2* __restrict__ rcand, const Chunks& C, int nch, const int* pg,
                                    const int* pe, uint32_t theta, int k, int32_t* __restrict__ out) {
  constexpr int NW = kResolveThreads / WAVE;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int G = pg[nch];
  const int take = k - G;
  auto sb = [&](int j) { return pg[j] + min(pe[j], take); };
  auto eqt = [&](int j) { return min(max(take - pe[j], 0), pe[j + 1] - pe[j]); };
  auto direct = [&](int j) {
    const int g = pg[j + 1] - pg[j], e = pe[j + 1] - pe[j];
    return g == 0 || e == 0 || eqt(j) == e;
  };
  constexpr int U = 4;
  for (int p0 = 0; p0 < k; p0 += U * kResolveThreads) {
    int src[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * kResolveThreads + tid;
      src[u] = -1;
      if (p < k) {
        int lo = 0, hi = nch - 1;  // the last chunk whose offset is <= p
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (sb(mid) <= p) lo = mid; else hi = mid - 1;
        }
        if (direct(lo)) src[u] = C.start(lo) + (p - sb(lo));
      }
    }
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[u] >= 0 ? (int)rcand[src[u]].y : 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (src[u] >= 0) out[p0 + u * kResolveThreads + tid] = v[u];
  }
  for (int j = w; j < nch; j += NW) {
    const int g = pg[j + 1] - pg[j];
    const int et = eqt(j);
    if (direct(j) || g + et == 0) continue;
    const int cnt = g + (pe[j + 1] - pe[j]);
    const uint2* cj = rcand + C.start(j);
    int eq_run = 0, sel_run = sb(j);
    for (int i0 = 0; i0 < cnt; i0 += U * WAVE) {
      uint2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = cj[min(i0 + u * WAVE + lane, cnt - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = i0 + u * WAVE + lane < cnt;
        const bool eq = ok & (v[u].x == theta);
        const uint64_t eqm = ballot(eq);
        const bool sel = (ok & (v[u].x > theta)) | (eq & (eq_run + mask_rank(eqm) < et));
        const uint64_t selm = ballot(sel);
        if (sel) out[sel_run + mask_rank(selm)] = (int)v[u].y;
        eq_run += __popcll(eqm);
        sel_run += __popcll(selm);
      }
    }
  }
}

// Long rows, pass 2 (one workgroup per row).  The chunks' survivor counts give, by one scan,
// how many keys lie above theta (G) and at it (E); then the three cases of the file comment.
// C is the chunk length of the candidate slots; `row` is the score row, or null in the fused
// call, whose fallback rescores the row (through rs) into its candidate slots first.
// kPre x U: chunks per wave and slot rounds per chunk loaded before the counts are known
// (sized to the launch's chunks: ~4k survivors in 32 chunks of 4096 positions, or ~6k in the
// fused call's 63 chunks of ~2080 at 8 x 131072).
template <int kPre, int U>
__device__ void resolve_long_row(const float* __restrict__ row, const Rescore& rs, int64_t ld, int n, int k,
                                 int r, int32_t* __restrict__ out, const RowHeader* __restrict__ hdr,
                                 const ChunkCount* __restrict__ counts, int max_chunks, const Chunks& C,
                                 uint2* __restrict__ cand, uint64_t* __restrict__ ready, uint32_t* smem,
                                 int* hist, uint2* ties, SelState& st) {
  static_assert(kSurvBins <= kPassMax * kHistBins, "the survivor histogram reuses the radix buffers");
  static_assert(kSurvBins == 4 * kResolveThreads, "four survivor bins per thread");
  constexpr int NW = kResolveThreads / WAVE;
  const int nch = C.count(n);
  uint32_t* keys = smem;
  int* ids = reinterpret_cast<int*>(smem + kCandCap);
  int* pg = reinterpret_cast<int*>(smem + 2 * kCandCap);  // [nch + 1] survivors above theta before chunk j
  int* pe = pg + max_chunks + 1;                          // [nch + 1] survivors equal to theta before chunk j
  const ChunkCount* rc = counts + (int64_t)r * max_chunks;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const RowHeader rh = hdr[r];
  // The first 64 chunk counts (wave 0), then -- before any count is known -- the first
  // U * WAVE candidate slots of this wave's first kPre chunks (slots past a chunk's count
  // hold stale pairs and are dropped below).  The count load goes first, so waiting for it
  // leaves the candidate loads in flight, and a typical row's gather costs the one round
  // trip these loads share.
  uint2* rcand = cand + (int64_t)r * ld;
  const ChunkCount c0 = (w == 0 && lane < nch) ? rc[lane] : ChunkCount{0u, 0u, rh.theta, 0u};
  if (ready && tid == 0) ready[r] = 0;  // the next call's scoring blocks wait for a fresh threshold
  uint2 pre[kPre][U];
  // Starts of those chunks and of the chunks after them, lane 2m (+1) for the m-th: divisions
  // in parallel on the vector unit rather than one scalar division per chunk in every wave.
  static_assert(2 * kPre <= WAVE, "one lane per chunk start");
  const int jm = w + (lane >> 1) * NW;
  const int cs = C.start((lane < 2 * kPre && jm < nch ? jm : 0) + (lane & 1));
#pragma unroll
  for (int m = 0; m < kPre; ++m) {
    const int c0j = readlane(cs, 2 * m);
    const int cl = min(readlane(cs, 2 * m + 1), n) - c0j;  // the chunk's length: slots stay in the row
#pragma unroll
    for (int u = 0; u < U; ++u) pre[m][u] = rcand[c0j + min(u * WAVE + lane, cl - 1)];
  }
  // Survivors past the preloaded slots are gathered by all waves together as one flat range:
  // rf[j] counts those of the chunks before j.  It lives in the survivor histogram's unused
  // tail (the radix select clears the whole buffer before it uses it), so rows of more
  // chunks than that tail holds keep the gather of one wave per chunk.
  int* rf = hist + kSurvBins;
  const bool flat = nch < kPassMax * kHistBins - kSurvBins;
  if (w == 0) {  // exclusive prefixes of the survivor counts, 64 chunks per step
    int cg = 0, ce = 0, cr = 0;
    bool stale = false;  // a chunk compacted with another threshold than the row's
    for (int j0 = 0; j0 < nch; j0 += WAVE) {
      const int j = j0 + lane;
      const ChunkCount cj = j0 == 0 ? c0 : (j < nch ? rc[j] : ChunkCount{0u, 0u, rh.theta, 0u});
      stale = stale || cj.theta != rh.theta;
      const int ig = wave_incl_scan((int)cj.gt), ie = wave_incl_scan((int)cj.eq);
      const int cnt = (int)(cj.gt + cj.eq);
      const int rj = cnt - (j < kPre * NW ? min(cnt, U * WAVE) : 0);
      const int ir = wave_incl_scan(rj);
      if (j < nch) {
        pg[j] = cg + ig - (int)cj.gt;
        pe[j] = ce + ie - (int)cj.eq;
        if (flat) rf[j] = cr + ir - rj;
      }
      cg += __shfl(ig, WAVE - 1);
      ce += __shfl(ie, WAVE - 1);
      cr += __shfl(ir, WAVE - 1);
    }
    if (lane == 0) {
      pg[nch] = ballot(stale) ? -1 : cg;  // -1: the survivors are not one threshold's
      pe[nch] = ce;
      if (flat) rf[nch] = cr;
    }
  }
  reinterpret_cast<int4*>(hist)[tid] = make_int4(0, 0, 0, 0);
  if (tid == 0) st.ntie = 0;
  __syncthreads();
  const int G = pg[nch];
  const int total = G < 0 ? -1 : G + pe[nch];
  if (G >= 0 && G < k && k <= total) {
    emit_theta_boundary(rcand, C, nch, pg, pe, rh.theta, k, out);
    return;
  }
  if (total < k || total > kCandCap) {
    if (row) {
      const GlobalRow src{row};
      const Threshold th = find_threshold<kResolveThreads>(src, n, k, hist, st);
      emit_selected<kResolveThreads>(src, n, th, st, out);
    } else {
      // The row's candidate slots (8 bytes per position) hold its n keys from here on.
      uint32_t* rk = reinterpret_cast<uint32_t*>(rcand);
      rescore_row(rs, r, n, rk);
      __syncthreads();
      const GlobalKeys src{rk};
      const Threshold th = find_threshold<kResolveThreads>(src, n, k, hist, st);
      emit_selected<kResolveThreads>(src, n, th, st, out);
    }
    return;
  }
  {
    // Wave w copies the preloaded slots of chunks w, w + NW, ... (its first kPre); the rest --
    // survivors past those slots, and chunks beyond the first kPre per wave -- follows below.
    auto off = [&](int j) { return pg[j] + pe[j]; };
    // Offsets and survivor counts of this wave's first kPre chunks, lane m for the m-th (one
    // LDS read per lane instead of scalar reads of every chunk in every wave).
    const int jl = w + lane * NW;
    const bool lv = lane < kPre && jl < nch;
    const int o_l = lv ? off(jl) : 0;
    const int c_l = lv ? off(jl + 1) - o_l : 0;
#pragma unroll
    for (int m = 0; m < kPre; ++m) {
      const int o = readlane(o_l, m), cj = min(readlane(c_l, m), U * WAVE);  // 0: no such chunk
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = u * WAVE + lane;
        if (i < cj) {
          keys[o + i] = pre[m][u].x;
          ids[o + i] = (int)pre[m][u].y;
          atomicAdd(&hist[min((pre[m][u].x - rh.theta) >> rh.shift, (uint32_t)(kSurvBins - 1))], 1);
        }
      }
    }
    // The rest: survivors past the preloaded slots, and chunks past the first kPre.  Thread t
    // takes flat positions t, t + 1024, ... of the rest and finds its chunk by binary search
    // over rf, so a row whose survivors crowd into a few chunks (a short row keeps nearly
    // every key) still gathers them with every wave instead of one wave per chunk.
    if (flat) {
      const int rest = rf[nch];
      for (int i0 = 0; i0 < rest; i0 += U * kResolveThreads) {
        uint2 v[U];
        int dst[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          // Positions past the rest load the last one (so every load issues) and are dropped.
          const int i = i0 + u * kResolveThreads + tid;
          const int ic = min(i, rest - 1);
          int lo = 0, hi = nch - 1;  // the last chunk whose rest starts at or before ic
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (rf[mid] <= ic) lo = mid; else hi = mid - 1;
          }
          const int o = off(lo);
          const int e = (lo < kPre * NW ? min(off(lo + 1) - o, U * WAVE) : 0) + (ic - rf[lo]);
          v[u] = rcand[C.start(lo) + e];
          dst[u] = i < rest ? o + e : -1;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (dst[u] >= 0) {
            keys[dst[u]] = v[u].x;
            ids[dst[u]] = (int)v[u].y;
            atomicAdd(&hist[min((v[u].x - rh.theta) >> rh.shift, (uint32_t)(kSurvBins - 1))], 1);
          }
        }
      }
    } else if (ballot(c_l > U * WAVE) || w + kPre * NW < nch) {
      for (int j = w; j < nch; j += NW) {
        const int o = off(j), cj = off(j + 1) - o;
        for (int i0 = j < w + kPre * NW ? U * WAVE : 0; i0 < cj; i0 += U * WAVE) {
          uint2 v[U];
#pragma unroll
          for (int u = 0; u < U; ++u) v[u] = rcand[C.start(j) + min(i0 + u * WAVE + lane, cj - 1)];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int i = i0 + u * WAVE + lane;
            if (i < cj) {
              keys[o + i] = v[u].x;
              ids[o + i] = (int)v[u].y;
              atomicAdd(&hist[min((v[u].x - rh.theta) >> rh.shift, (uint32_t)(kSurvBins - 1))], 1);
            }
          }
        }
      }
    }
  }
  __syncthreads();
  select_survivors(keys, ids, total, rh.theta, rh.shift, k, hist, ties, st, out);
}

// One workgroup per row: trivial rows, LDS-resident rows, or the resolve of long rows.
// scores == null (the fused call): every row longer than k takes the resolve.
template <int kPre, int U>
__global__ __launch_bounds__(kRowThreads) void topk_finish_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ n_valid, int k,
    int32_t* __restrict__ idx, const RowHeader* __restrict__ hdr, const ChunkCount* __restrict__ counts,
    int max_chunks, int tb, uint2* __restrict__ cand, uint64_t* __restrict__ ready, int n_off, int long_min,
    Rescore rs) {
  static_assert(kRowThreads == kResolveThreads, "one kernel serves both paths");
  extern __shared__ uint32_t smem[];  // long rows: survivor keys, ids and chunk offsets
  __shared__ __attribute__((aligned(16))) int hist[kPassMax * kHistBins];
  __shared__ uint2 ties[kTieMax];
  __shared__ SelState st;
  const int r = blockIdx.x;
  int64_t n64 = (int64_t)n_valid[r] + n_off;
  n64 = n64 < 0 ? 0 : (n64 > ld ? ld : n64);
  const int n = (int)n64;
  int32_t* out = idx + (int64_t)r * k;
  const float* row = scores ? scores + (int64_t)r * ld : nullptr;
  if (n <= k) {
    for (int i = threadIdx.x; i < k; i += kRowThreads) out[i] = i < n ? i : -1;
    return;
  }
  if (row && n <= long_min) {
    if (n <= kRowMax / 4) select_mid_row<kRowMax / 4 / kRowThreads>(row, n, k, out, hist, st);
    else if (n <= kRowMax / 2) select_mid_row<kRowMax / 2 / kRowThreads>(row, n, k, out, hist, st);
    else select_mid_row<kRowMax / kRowThreads>(row, n, k, out, hist, st);
    return;
  }
  resolve_long_row<kPre, U>(row, rs, ld, n, k, r, out, hdr, counts, max_chunks, Chunks{tb, max_chunks}, cand,
                            ready, smem, hist, ties, st);
}

struct WsLayout {
  size_t ready, hdr, counts, cand, total;
  int max_chunks;
};

// [ready [R] (fused call only)], hdr [R], counts [R, max_chunks], cand [R, ld] (one 8-byte
// slot per position).
WsLayout long_ws(int R, int64_t ld, int max_chunks, bool fused) {
  WsLayout L{};
  L.max_chunks = max_chunks;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  L.ready = 0;
  L.hdr = fused ? up(sizeof(uint64_t) * (size_t)R) : 0;
  L.counts = L.hdr + up(sizeof(RowHeader) * (size_t)R);
  L.cand = L.counts + up(sizeof(ChunkCount) * (size_t)R * L.max_chunks);
  L.total = L.cand + up(sizeof(uint2) * (size_t)R * (size_t)ld);
  return L;
}

WsLayout ws_layout(int R, int64_t ld) {
  if (ld <= kRowMax) return WsLayout{};
  return long_ws(R, ld, (int)((ld + kChunk - 1) / kChunk), false);
}

size_t finish_lds_bytes(int max_chunks) {
  return sizeof(uint32_t) * (2 * (size_t)kCandCap + 2 * ((size_t)max_chunks + 1));
}

}  // namespace

int topk_long_row_min(int64_t ld) { return ld > kRowMax ? kLongMinWs : kRowMax; }

bool topk_shape_ok(int R, int64_t ld) {
  return (int64_t)R * ws_layout(1, ld).max_chunks <= 2147483647LL;
}

size_t topk_workspace_bytes(int R, int64_t ld, int k) {
  (void)k;
  return ws_layout(R, ld).total;
}

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* n_valid, int R, int k,
                       int32_t* idx, void* ws, hipStream_t s, int n_off) {
  const WsLayout L = ws_layout(R, ld);
  const int long_min = topk_long_row_min(ld);
  char* wsb = static_cast<char*>(ws);
  RowHeader* hdr = L.total ? reinterpret_cast<RowHeader*>(wsb + L.hdr) : nullptr;
  ChunkCount* counts = L.total ? reinterpret_cast<ChunkCount*>(wsb + L.counts) : nullptr;
  uint2* cand = L.total ? reinterpret_cast<uint2*>(wsb + L.cand) : nullptr;
  if (L.total) {
    topk_prep_kernel<<<(unsigned)R * (unsigned)L.max_chunks, kLongThreads, 0, s>>>(
        scores, ld, n_valid, k, hdr, counts, L.max_chunks, cand, n_off, long_min);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Long rows: survivor keys and ids, then the chunk offsets (rows up to kRowMax need none).
  const size_t lds = L.total ? finish_lds_bytes(L.max_chunks) : 0;
  topk_finish_kernel<2, 4><<<R, kRowThreads, lds, s>>>(scores, ld, n_valid, k, idx, hdr, counts, L.max_chunks,
                                                       kChunk / 64 * L.max_chunks, cand, nullptr, n_off,
                                                       long_min, Rescore{});
  return hipGetLastError();
}

// ---- fused index + top-k (fast indexer shape)

size_t index_topk_fused_bytes(int R, int64_t ld) { return long_ws(R, ld, index_compact_chunks(R, ld), true).total; }

bool index_topk_fused_ok(int R, int64_t ld) {
  const int mc = index_compact_chunks(R, ld);
  return mc <= kFusedMaxChunks && (int64_t)R * (mc + 1) <= 2147483647LL;
}

hipError_t launch_index_topk_fused(const uint8_t* q, const float* q_scale, const float* w, const CacheView& keys,
                                   const int32_t* row_seq, const int32_t* row_pos, int R, int64_t ld, int k,
                                   int32_t* idx, void* ws, hipStream_t s) {
  const WsLayout L = long_ws(R, ld, index_compact_chunks(R, ld), true);
  const int tb = (int)((ld + 63) / 64);
  char* wsb = static_cast<char*>(ws);
  uint64_t* ready = reinterpret_cast<uint64_t*>(wsb + L.ready);
  RowHeader* hdr = reinterpret_cast<RowHeader*>(wsb + L.hdr);
  ChunkCount* counts = reinterpret_cast<ChunkCount*>(wsb + L.counts);
  uint2* cand = reinterpret_cast<uint2*>(wsb + L.cand);
  const int ps = keys.table ? keys.page_size : 1;
  const int shift = keys.table && (ps & (ps - 1)) == 0 ? __builtin_ctz(ps) : -1;
  const Rescore rs{q, q_scale, w, static_cast<const uint8_t*>(keys.data), keys.scale,
                   KeyRows{keys.table, keys.max_pages, ps, shift, keys.seq_stride}, row_seq};
  hipError_t e = launch_index_fp8_compact(q, q_scale, w, keys, row_seq, row_pos, R, ld, ld, hdr, ready, counts, cand,
                                          k, s);
  if (e != hipSuccess) return e;
  topk_finish_kernel<4, 3><<<R, kRowThreads, finish_lds_bytes(L.max_chunks), s>>>(
      nullptr, ld, row_pos, k, idx, hdr, counts, L.max_chunks, tb, cand, ready, 1, 0, rs);
  return hipGetLastError();
}

}  // namespace dsa
