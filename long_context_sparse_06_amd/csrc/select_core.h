// Exact top-k selection primitives on order-preserving 32-bit keys (block-parallel radix
// select, ordered emit), shared by the top-k kernels and the compacting indexer's sample
// workgroups.  The tie rule (equal keys: lower position first) and the output order
// (ascending position) are this library's; the pages fix only that each query keeps its k
// best-scored tokens (maplevalley.com.cn news 1594152, section 1 "Top-k Token Selection").
//
// Method: radix select on keys held in LDS or registers.  A min/max pass first strips the
// bits all keys share, so the 11-bit histogram digits land where the keys actually differ;
// each digit pass narrows to one bin until either that bin holds exactly the elements still
// needed or the full key (the threshold T) is known.  Every search step is block-parallel
// (DPP wave scans, per-wave totals through LDS); no phase runs on a single wave.  The emit
// pass walks each wave's contiguous index range with ballots, so the elements equal to T are
// taken lowest index first and the output comes out sorted.
#pragma once
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kHistBins = 2048;    // 11-bit digits
constexpr int kPassMax = 3;        // range-relative 11-bit digits resolve 32-bit keys in 3 passes
constexpr int kSurvBins = 4096;    // survivor histogram of a long row (the row header's bins)

// Block-shared scratch of the selection routines.
struct SelState {
  uint32_t wmin[16], wmax[16];      // per-wave key range
  uint32_t wred[16];                // per-wave partials of a caller's final reduction
  alignas(16) int wscan[16];        // per-wave bin totals of a crossing search
  alignas(16) int wtot[2][16];      // per-wave counts of the emit pass
  int digit, above, cnt;            // result of a crossing search
  uint32_t tie_T;                   // result of the boundary-bin ranking
  int tie_need;
  int ntie;
};

// ---- element sources --------------------------------------------------------------
struct LdsKeys {  // keys in LDS, ids = position + base
  const uint32_t* keys;
  int base;
  __device__ uint32_t key(int i) const { return keys[i]; }
  __device__ int id(int i) const { return base + i; }
};
struct LdsPairs {  // keys and ids in LDS
  const uint32_t* keys;
  const int* ids;
  __device__ uint32_t key(int i) const { return keys[i]; }
  __device__ int id(int i) const { return ids[i]; }
};
struct GlobalRow {  // a score row in global memory
  const float* row;
  __device__ uint32_t key(int i) const { return float_key(row[i]); }
  __device__ int id(int i) const { return i; }
};

struct GlobalKeys {  // order-preserving keys in global memory, ids = position
  const uint32_t* keys;
  __device__ uint32_t key(int i) const { return keys[i]; }
  __device__ int id(int i) const { return i; }
};

// Visits elements i = tid, tid + NT, ... of [0, m) in batches of U per thread: all U keys of a
// batch are read before any is used, so global-memory sources have U loads in flight
// instead of one round trip per element.
template <int NT, int U, class Src, class F>
__device__ __forceinline__ void for_each_key(const Src& src, int m, F&& f) {
  for (int base = 0; base < m; base += NT * U) {
    uint32_t kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NT + (int)threadIdx.x;
      kv[u] = src.key(min(i, m - 1));  // unconditional: the batch's loads issue back to back
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NT + (int)threadIdx.x;
      if (i < m) f(i, kv[u]);
    }
  }
}

// ---- wave primitives: DPP row shifts/rotations and gfx950 lane swaps (no LDS traffic) ----
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp<0x111>(v);        // row_shr:1
  v += dpp<0x112>(v);        // row_shr:2
  v += dpp<0x114>(v);        // row_shr:4
  v += dpp<0x118>(v);        // row_shr:8  -> inclusive within rows of 16
  v += dpp<0x142, 0xA>(v);   // row_bcast:15 -> rows 1 and 3 add the previous row's total
  v += dpp<0x143, 0xC>(v);   // row_bcast:31 -> rows 2 and 3 add rows 0-1
  return v;
}
// All-lane reductions: rotations within rows of 16, then swaps across rows and halves.
template <class F>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, F op) {
  v = op(v, (uint32_t)dpp<0x128>((int)v));  // row_ror:8
  v = op(v, (uint32_t)dpp<0x124>((int)v));  // row_ror:4
  v = op(v, (uint32_t)dpp<0x122>((int)v));  // row_ror:2
  v = op(v, (uint32_t)dpp<0x121>((int)v));  // row_ror:1
  const v2i a = __builtin_amdgcn_permlane16_swap((int)v, (int)v, false, false);
  v = op((uint32_t)a[0], (uint32_t)a[1]);
  const v2i b = __builtin_amdgcn_permlane32_swap((int)v, (int)v, false, false);
  return op((uint32_t)b[0], (uint32_t)b[1]);
}
struct UMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };
struct UAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct UMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// Block-level reductions over the NW per-wave values in LDS, done with lane v standing for wave
// v (one LDS load, a DPP scan or reduce, a ballot).  Every wave of the block computes them; a
// scalar walk over the NW values costs each wave ~10 scalar instructions per value, and the CU
// issues one scalar instruction per SIMD every fourth cycle, so with four waves per SIMD those
// walks, not the data, set the time of the selection's short phases.
//
// Crossing wave of a search from the per-wave totals t[0..NW): the first wave v whose running
// total reaches `need` (vc = -1 when none does), and the total of the waves before it (of all
// of them when none does).
template <int NW>
__device__ __forceinline__ void crossing_wave(const int* t, int need, int& vc, int& before) {
  static_assert(NW <= WAVE, "one lane per wave");
  const int lane = threadIdx.x & (WAVE - 1);
  const int tv = lane < NW ? t[lane] : 0;
  const int incl = wave_incl_scan(tv);
  const uint64_t hit = ballot((lane < NW) & (incl >= need));
  vc = hit ? (int)__builtin_ctzll(hit) : -1;
  before = hit ? readlane(incl - tv, vc) : readlane(incl, NW - 1);
}
// Minimum (and maximum) of the per-wave values v[0..NW), in every lane.
template <int NW>
__device__ __forceinline__ uint32_t block_min(const uint32_t* v) {
  static_assert(NW <= WAVE, "one lane per wave");
  const int lane = threadIdx.x & (WAVE - 1);
  return wave_reduce(lane < NW ? v[lane] : 0xFFFFFFFFu, UMin{});
}
template <int NW>
__device__ __forceinline__ uint32_t block_max(const uint32_t* v) {
  static_assert(NW <= WAVE, "one lane per wave");
  const int lane = threadIdx.x & (WAVE - 1);
  return wave_reduce(lane < NW ? v[lane] : 0u, UMax{});
}
// Per-wave counts a[0..NW) and b[0..NW): their totals, and the sum of a + b over the waves
// before wave w (a compaction's output offset), in every lane.
template <int NW>
__device__ __forceinline__ void wave_offsets(const int* a, const int* b, int w, int& off, int& ta, int& tb) {
  static_assert(NW <= WAVE, "one lane per wave");
  const int lane = threadIdx.x & (WAVE - 1);
  const int av = lane < NW ? a[lane] : 0, bv = lane < NW ? b[lane] : 0;
  const int ia = wave_incl_scan(av), ib = wave_incl_scan(bv);
  off = readlane(ia - av + ib - bv, w);
  ta = readlane(ia, NW - 1);
  tb = readlane(ib, NW - 1);
}

// The top-k threshold: the selection is { key > T } plus the `need` lowest-index elements
// equal to T, or exactly { key >= T } when `exact`.  `top` is the largest key seen.
struct Threshold {
  uint32_t T;
  int need;
  bool exact;
  uint32_t top;
};

// Given one thread's PER bin counts cb[0..PER) (its bins in descending order, the first
// being bin `first`), finds the bin where the count from the top reaches `need` within the
// wave whose bins these are; `before` counts everything above the wave.  Returns the
// crossing (bin, count above it, its count), the same in every lane.  The caller
// guarantees the crossing lies in this wave.
template <int PER>
__device__ __forceinline__ void wave_crossing(const int (&cb)[PER], int first, int before, int need,
                                              int& digit, int& above, int& cnt) {
  int local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) local += cb[j];
  const int incl = wave_incl_scan(local);
  int run = before + incl - local;
  const bool mine = run < need && run + local >= need;
  int dj = 0, ab = 0, cn = 0;
  bool found = false;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool hit = !found && run + cb[j] >= need;
    dj = hit ? j : dj;
    ab = hit ? run : ab;
    cn = hit ? cb[j] : cn;
    found = found || hit;
    run += cb[j];
  }
  const int cl = (int)__builtin_ctzll(ballot(mine));
  digit = readlane(first - dj, cl);
  above = readlane(ab, cl);
  cnt = readlane(cn, cl);
}

// Publishes the block's key range for find_threshold (each thread passes the min and max of
// its own keys) and clears the histogram buffers; the caller's next barrier publishes both.
template <int NT>
__device__ __forceinline__ void publish_range(uint32_t lmn, uint32_t lmx, int* hist, SelState& st) {
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  lmn = wave_reduce(lmn, UMin{});
  lmx = wave_reduce(lmx, UMax{});
  if (lane == 0) {
    st.wmin[w] = lmn;
    st.wmax[w] = lmx;
  }
  for (int i = tid; i < kPassMax * kHistBins / 4; i += NT) reinterpret_cast<int4*>(hist)[i] = make_int4(0, 0, 0, 0);
}

// Finds the selection threshold of the top-k (1 <= k <= m) among m elements with
// range-relative radix digits: the threshold lies in the key interval [lo, hi]; each pass
// splits it into at most 2048 equal bins of 2^s keys (s chosen from its width), so the
// histogram resolves wherever the keys actually are, in at most three passes.  Each pass
// has two barriers: after the histogram, and after the per-wave totals; every wave then
// finds the crossing wave from the totals and rescans that wave's bins itself, so the
// result needs no broadcast.  Each pass has its own histogram buffer (cleared up front),
// so no clearing races a slower wave's rescan.  All NT threads must call it.
//
// RANGED: the caller has already run publish_range (and a barrier) with every thread's key
// range, typically while it loaded the keys, which saves a pass and a barrier.  `slack`
// lets the search stop early, with `exact` set, once the bin holds at most `slack` more
// elements than needed -- only for callers content with up to k + slack elements >= T.
// The digit passes of find_threshold on the key interval [lo, hi]; fill(lo, hi, s, h) adds
// every element whose key lies in [lo, hi] to bin (key - lo) >> s of h.
template <int NT, class Fill>
__device__ Threshold radix_threshold(uint32_t lo, uint32_t hi, int k, int* hist, SelState& st, int slack,
                                     Fill&& fill) {
  constexpr int NW = NT / WAVE;
  constexpr int PER = kHistBins / NT;
  static_assert(PER * NT == kHistBins, "bins per thread");
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int w = tid / WAVE;
  const uint32_t top = hi;
  int need = k;
  bool exact = false;
  for (int pass = 0; pass < kPassMax && hi != lo; ++pass) {
    const uint32_t width = hi - lo;
    const int s = max(0, 32 - __builtin_clz(width) - 11);
    const int nb = (int)(width >> s) + 1;
    int* h = hist + pass * kHistBins;
    fill(lo, hi, s, h);
    __syncthreads();
    // Thread t owns bins nb-1-PER*t-j (j < PER): bins counted from the top.
    int cb[PER];
    int local = 0;
    const int first = nb - 1 - PER * tid;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int b = first - j;
      const int v = h[max(b, 0)];
      cb[j] = b >= 0 ? v : 0;
      local += cb[j];
    }
    const int incl = wave_incl_scan(local);
    if (lane == WAVE - 1) st.wscan[w] = incl;
    __syncthreads();
    int before, vc;
    crossing_wave<NW>(st.wscan, need, vc, before);
    // Rescan the crossing wave's bins (the same PER per lane that wave read).
    const int first2 = nb - 1 - PER * (vc * WAVE + lane);
    int cb2[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int b = first2 - j;
      const int v = h[max(b, 0)];
      cb2[j] = b >= 0 ? v : 0;
    }
    int d, above, cnt;
    wave_crossing<PER>(cb2, first2, before, need, d, above, cnt);
    need -= above;
    const uint32_t new_lo = lo + ((uint32_t)d << s);
    const uint64_t top_of_bin = (uint64_t)new_lo + ((uint64_t)1 << s) - 1;
    hi = top_of_bin < (uint64_t)hi ? (uint32_t)top_of_bin : hi;
    lo = new_lo;
    if (cnt - need <= slack) {  // every key of the bin is taken: the selection is { key >= lo }
      exact = true;
      break;
    }
  }
  return Threshold{lo, need, exact, top};
}

// Finds the selection threshold of the top-k (1 <= k <= m) among m elements with
// range-relative radix digits: the threshold lies in the key interval [lo, hi]; each pass
// splits it into at most 2048 equal bins of 2^s keys (s chosen from its width), so the
// histogram resolves wherever the keys actually are, in at most three passes.  Each pass
// has two barriers: after the histogram, and after the per-wave totals; every wave then
// finds the crossing wave from the totals and rescans that wave's bins itself, so the
// result needs no broadcast.  Each pass has its own histogram buffer (cleared up front),
// so no clearing races a slower wave's rescan.  All NT threads must call it.
//
// RANGED: the caller has already run publish_range (and a barrier) with every thread's key
// range, typically while it loaded the keys, which saves a pass and a barrier.  `slack`
// lets the search stop early, with `exact` set, once the bin holds at most `slack` more
// elements than needed -- only for callers content with up to k + slack elements >= T.
template <int NT, bool RANGED = false, class Src>
__device__ Threshold find_threshold(const Src& src, int m, int k, int* hist, SelState& st,
                                    int slack = 0) {
  constexpr int NW = NT / WAVE;
  if (!RANGED) {
    uint32_t lmn = 0xFFFFFFFFu, lmx = 0u;
    for_each_key<NT, 8>(src, m, [&](int, uint32_t key) {
      lmn = min(lmn, key);
      lmx = max(lmx, key);
    });
    publish_range<NT>(lmn, lmx, hist, st);
    __syncthreads();
  }
  const uint32_t lo = block_min<NW>(st.wmin), hi = block_max<NW>(st.wmax);
  return radix_threshold<NT>(lo, hi, k, hist, st, slack, [&](uint32_t a, uint32_t b, int s, int* h) {
    for_each_key<NT, 8>(src, m, [&](int, uint32_t key) {
      if (key >= a && key <= b) atomicAdd(&h[(key - a) >> s], 1);
    });
  });
}

// Writes the ids of the selected elements, in ascending position order, to out[0..k).
// Each wave walks a contiguous position range with ballots, so elements equal to T are
// taken lowest position first; the waves' output offsets come from two DPP scans over
// the per-wave counts.  Predicates combine with bitwise operators so the element loop is
// straight-line mask arithmetic, and ids are read together with keys, before any is used.
template <int NT, class Src>
__device__ void emit_selected(const Src& src, int m, const Threshold& th, SelState& st,
                              int32_t* __restrict__ out) {
  constexpr int NW = NT / WAVE;
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  const uint32_t T = th.T;
  const bool ex = th.exact;
  const int need = ex ? 0 : th.need;
  const int per = ((m + NW - 1) / NW + WAVE - 1) / WAVE * WAVE;
  const int beg = w * per;
  const int end = min(m, beg + per);
  constexpr int U = 8;  // rounds of 64 whose keys are read before they are used
  // Per-lane counts, summed over the wave once (a ballot count per round is scalar work)
  int lgt = 0, leq = 0;
  for (int i0 = beg; i0 < end; i0 += U * WAVE) {
    uint32_t kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kv[u] = src.key(min(i0 + u * WAVE + lane, end - 1));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = i0 + u * WAVE + lane < end;
      lgt += (in & ((kv[u] > T) | (ex & (kv[u] == T)))) ? 1 : 0;
      leq += (in & !ex & (kv[u] == T)) ? 1 : 0;
    }
  }
  const int cgt = (int)wave_reduce((uint32_t)lgt, UAdd{}), ceq = (int)wave_reduce((uint32_t)leq, UAdd{});
  if (lane == 0) {
    st.wtot[0][w] = cgt;
    st.wtot[1][w] = ceq;
  }
  __syncthreads();
  // Lane v < NW stands for wave v: ties are taken in wave order until `need` is met.
  const int gt_v = lane < NW ? st.wtot[0][lane] : 0;
  const int eq_v = lane < NW ? st.wtot[1][lane] : 0;
  const int eq_before_v = wave_incl_scan(eq_v) - eq_v;
  const int take_v = min(max(need - eq_before_v, 0), eq_v);
  const int sel_v = gt_v + take_v;
  const int sel_before_v = wave_incl_scan(sel_v) - sel_v;
  const int eq_before = readlane(eq_before_v, w);
  const int sel_before = readlane(sel_before_v, w);
  int eq_run = 0, sel_run = 0;
  if (ex) {  // the selection is { key >= T }: no tie bookkeeping
    for (int i0 = beg; i0 < end; i0 += U * WAVE) {
      uint32_t kv[U];
      int iv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = min(i0 + u * WAVE + lane, end - 1);
        kv[u] = src.key(e);
        iv[u] = src.id(e);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool sel = (i0 + u * WAVE + lane < end) & (kv[u] >= T);
        const uint64_t selm = ballot(sel);
        if (sel) out[sel_before + sel_run + mask_rank(selm)] = iv[u];
        sel_run += __popcll(selm);
      }
    }
    return;
  }
  for (int i0 = beg; i0 < end; i0 += U * WAVE) {
    uint32_t kv[U];
    int iv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = min(i0 + u * WAVE + lane, end - 1);
      kv[u] = src.key(e);
      iv[u] = src.id(e);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = i0 + u * WAVE + lane < end;
      const bool gt = in & ((kv[u] > T) | (ex & (kv[u] == T)));
      const bool eq = in & !ex & (kv[u] == T);
      const uint64_t eqm = ballot(eq);
      const bool sel = gt | (eq & (eq_before + eq_run + mask_rank(eqm) < need));
      const uint64_t selm = ballot(sel);
      if (sel) out[sel_before + sel_run + mask_rank(selm)] = iv[u];
      eq_run += __popcll(eqm);
      sel_run += __popcll(selm);
    }
  }
}

// The sample threshold of a long row of n scores: the ks-th largest of the ns sample keys in
// LDS (ks chosen so that about `over` x k scores of the row are expected to reach it), or any
// sample key of rank ks .. ks + ks/4 -- the search stops at the first bin that close, usually
// after one pass -- raised to the smallest sample key at or above the search's bound.  (When
// the search stops early its bound is only that bin's lower edge, and the row can hold many
// more scores between it and the smallest sample in the bin.)  Each thread passes the range of
// the sample keys it stored; the caller's stores to `samp` need no barrier before the call.
// Returns the row header (theta and the survivor-bin shift), the same in every thread.  All NT
// threads must call it.
template <int NT>
__device__ RowHeader sample_header(const uint32_t* samp, int ns, int over, uint32_t lmn, uint32_t lmx, int64_t n,
                                   int k, int* hist, SelState& st) {
  constexpr int NW = NT / WAVE;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  publish_range<NT>(lmn, lmx, hist, st);
  __syncthreads();
  int ks = (int)(((int64_t)over * k * ns + n - 1) / n);
  ks = ks < 1 ? 1 : (ks > ns ? ns : ks);
  const Threshold th = find_threshold<NT, true>(LdsKeys{samp, 0}, ns, ks, hist, st, ks / 4);
  uint32_t theta = th.T;
  if (th.exact) {
    uint32_t mn = 0xFFFFFFFFu;
    for (int i = tid; i < ns; i += NT) {
      const uint32_t sk = samp[i];
      if (sk >= th.T) mn = min(mn, sk);
    }
    mn = wave_reduce(mn, UMin{});
    if (lane == 0) st.wred[w] = mn;  // not wmin: slower waves may still read that
    __syncthreads();
    theta = block_min<NW>(st.wred);
  }
  // Survivor bins span [theta, largest sample] in at most kSurvBins steps of 2^shift;
  // scores above the largest sample land in the last bin.
  const uint32_t width = th.top - theta;
  const int shift = width ? max(0, 32 - __builtin_clz(width) - 12) : 0;
  return RowHeader{theta, (uint32_t)shift};
}

}  // namespace dsa
