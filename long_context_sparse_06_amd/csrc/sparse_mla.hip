// Sparse core attention: MLA in MQA mode over the kept latent rows.
//
// The pages fix the instantiation: DSA runs under MLA in MQA mode so that every latent
// KV entry is shared by all query heads, the kernel-level requirement being that a KV
// entry is reused across queries (MarkTechPost, "DeepSeek V3.2-Exp Cuts Long-Context Costs
// with DeepSeek Sparse Attention (DSA) ...", "Instantiation"); attention runs only over
// the selected tokens (same article, two-tier pipeline; maplevalley.com.cn news 1594152,
// section 1).  Row layout (576 = 512 value + 64 rope columns, value = first 512) and the
// explicit softmax scale are this library's readings.
//
// bf16 fast path (Dqk = 576, Dv = 512, 64 heads per workgroup: four 16-head blocks, each
// computed by a pair of waves, plus one copy wave):
//   * 32 selected rows are gathered into LDS once per tile and used by all 64 heads;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = K rows from LDS (ds_read_b128),
//     B = the block's 16 query heads held in registers for the whole kernel (each wave of
//     the pair holds half of the 576 columns; the two partial logit tiles are summed
//     through LDS); the result layout puts one head per lane column, so the
//     online-softmax row statistics of a head live in one lane column and need two
//     cross-lane steps;
//   * O^T += V^T P^T: A = V^T fragments read from the row-major LDS tile with the gfx950
//     transposing LDS load (ds_read_b64_tr_b16), B = P^T straight from the S^T
//     registers (the token order inside the 32-wide K step is permuted identically on
//     both operands, so no data moves between lanes);
//   * decode splits each sequence's kept set over several workgroups and merges the
//     partials (each split's normalized output in bf16, its max and sum in fp32) with a
//     log-sum-exp combine kernel.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace dsa {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kTok = 32;                        // rows per LDS tile
constexpr int kRowChunks = kDqk * 2 / 16;       // 72 16-byte chunks per latent row
constexpr int kDmaPerTile = kRowChunks / 2;     // 36 wave-wide 1 KB copies per tile
// Tile layout (chunk-major): copy j fills block j with chunk j of rows 0..31 (lanes 0-31,
// "side 0") and chunk j + 36 (lanes 32-63, "side 1"), 16 bytes per lane.  With 1024-byte
// blocks the logit-fragment reads (16 rows of one chunk per 16 lanes, four chunks per
// wave) are free of bank conflicts on gfx950; the transposing value reads run at their
// own rate with either this or a padded stride (both measured).
constexpr int kBlock = 1024;
constexpr int kBufBytes = kDmaPerTile * kBlock;  // 36864
constexpr int kNBuf = 3;                        // ring depth: two tiles in flight during compute
constexpr int kMlaWaves = 8;                    // compute waves: two per 16-head block
constexpr int kMlaThreads = (kMlaWaves + 1) * WAVE;  // + one copy wave
constexpr int kHeadsPerWg = 64;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleLog2 = 64.0f;  // wide kernel: largest lead of a logit over its reference max

// Byte offset of (row, 16-byte chunk c) inside a tile.
__device__ __forceinline__ int tile_off(int row, int c) {
  return (c < kDmaPerTile ? c * kBlock : (c - kDmaPerTile) * kBlock + 512) + row * 16;
}

typedef __attribute__((address_space(3))) void lds_void;

// LDS pointers are formed from the byte offset, which a flat pointer into LDS carries in
// its low 32 bits: a flat-to-LDS pointer cast would add a null check per use.
__device__ __forceinline__ uint32_t lds_offset(const void* p) { return (uint32_t)(uintptr_t)p; }

__device__ __forceinline__ v4bf lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(uintptr_t)lds_offset(p));
}

// s_waitcnt with only the vector-memory counter constrained (expcnt, lgkmcnt left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The ring's three slots are separate LDS variables, so the compiler can tell that a copy
// into one slot never aliases the reads of another and puts no wait between them.
__shared__ __attribute__((aligned(16))) char g_ring0[kBufBytes];
__shared__ __attribute__((aligned(16))) char g_ring1[kBufBytes];
__shared__ __attribute__((aligned(16))) char g_ring2[kBufBytes];
// Partial logits exchanged between the two waves of a head block (8 floats per lane).
__shared__ __attribute__((aligned(16))) float g_xchg[kMlaWaves][WAVE * 8];
// Tiles this workgroup actually runs: up to the last kept token of its range (index lists
// are -1 padded at the end when a row has fewer than k candidates); set by the copy wave
// before the first hand-over.
__shared__ int g_ntiles;

// Max / sum over lanes l and l ^ 16, and over l and l ^ 32, with the gfx950 lane-swap
// instructions (VALU; a ds_bpermute shuffle would be an LDS round trip).
__device__ __forceinline__ float max_x16(float v) {
  const v2i y = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(y[0]), __int_as_float(y[1]));
}
__device__ __forceinline__ float max_x32(float v) {
  const v2i y = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(y[0]), __int_as_float(y[1]));
}
__device__ __forceinline__ float sum_x16(float v) {
  const v2i y = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(y[0]) + __int_as_float(y[1]);
}
__device__ __forceinline__ float sum_x32(float v) {
  const v2i y = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(y[0]) + __int_as_float(y[1]);
}

template <int S>
__device__ __forceinline__ char* ring_slot() {
  static_assert(S >= 0 && S < kNBuf, "ring slot");
  return S == 0 ? g_ring0 : (S == 1 ? g_ring1 : g_ring2);
}
template <int S>
struct Slot {
  static constexpr int value = S;
};
// One wide LDS-DMA copy: every lane loads 16 bytes from its global address and the wave's
// 64 pieces land contiguously at LDS byte address `lds` (M0) + 16 * lane.  Written as asm so
// the compiler's wait-count pass, which cannot tell a ring slot being filled from one being
// read, does not make every LDS read wait for every copy in flight; the caller orders copies
// and reads itself (s_waitcnt vmcnt + barrier).  No VGPR is written.  M0 is a reserved
// register the compiler does not let asm clobber; the kernels that use this copy make no
// other use of M0 (a CPU test compiles them and checks the generated code).
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "memory");
}
typedef __attribute__((address_space(3))) char lds_char;
// The same slot as an LDS-address-space pointer: an address-space cast of the variable itself
// (folded by the compiler, no null check), so alias analysis still sees which slot a read uses
// and the wait-count pass does not make it wait for copies into the other slots.
template <int S>
__device__ __forceinline__ lds_char* ring_lds() {
  return (lds_char*)ring_slot<S>();
}

// One workgroup = (row r, 64 heads, a range of the kept set): eight compute waves and one
// copy wave.  Compute waves w and w+4 share head block w&3 (16 heads): for S^T = K Q^T each
// takes one half of the 576 latent columns and the two partial logit tiles are summed
// through LDS (both waves then hold identical logits and run identical softmax
// statistics); for O^T += V^T P^T each takes one half of the 512 value columns.  Per wave
// that is half the query fragments and half the output accumulators of a whole-head-block
// wave, which leaves registers for LDS prefetch at three waves per SIMD.
//
// The copy wave streams each 32-row tile straight from global memory into a 3-deep LDS
// ring with global_load_lds_dwordx4 (a row is gathered once and shared by all 64 heads),
// two tiles ahead of the one being computed, and hands a tile over by waiting for its
// copies and one barrier (it also takes part in the compute waves' second barrier of each
// tile, the logit exchange, so the two sides' barriers pair up).  It starts the first two
// tiles from the split's first 64 indices before building the rest of the row list, so
// the first gather overlaps the query loads.  It never reads the ring (its only LDS reads
// are the row list, a different variable), so the compiler never waits on copies in
// flight; the compute waves issue no copies.  The tile loop is unrolled by the ring depth
// so every slot is a compile-time LDS variable.
//
// MASKED (prefill only): row t attends over the contiguous positions 0..t, each tile's live
// mask set from the bits of the kept set idx[t, :] -- the dense "masked" form of the same
// attention (no row-list gather; contiguous tiles).
template <bool PAGED, bool SPLIT, bool MASKED = false>
__global__ __launch_bounds__(kMlaThreads) void mla_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ table, int max_pages, int page_size, int64_t seq_stride,
    const int32_t* __restrict__ idx, int k, int H, int decode, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o,
    float* __restrict__ part_ml, int n_split, int tok_per_split) {
  extern __shared__ int srow[];  // [tok_per_split] cache row of each kept token, -1 = none;
                                 // then [tiles] bit mask of each tile's live tokens (MASKED:
                                 // the masks only)
  const int HG = H / kHeadsPerWg;
  // The head blocks of one unit (row, token range) read the same latent rows.  The dispatcher
  // deals consecutive blocks round-robin to the eight XCDs, so blocks b and b + 8 (same XCD)
  // take two head blocks of one unit while consecutive units still go to consecutive XCDs:
  // the second workgroup's gathers hit the XCD's L2, and ragged units stay spread evenly.
  int unit, hg;
  {
    const int b = (int)blockIdx.x, full = ((int)gridDim.x / HG) / 8 * 8 * HG;
    if (b < full) {
      unit = b / (8 * HG) * 8 + b % 8;
      hg = (b / 8) % HG;
    } else {  // the last units when their count is not a multiple of 8
      unit = full / HG + (b - full) / HG;
      hg = (b - full) % HG;
    }
  }
  const int sp = unit % n_split;
  const int r = unit / n_split;
  const int t_begin = MASKED ? 0 : sp * tok_per_split;
  const int t_end = MASKED ? r + 1 : min(k, t_begin + tok_per_split);
  const int n_tok = t_end > t_begin ? t_end - t_begin : 0;
  const int ntiles = (n_tok + kTok - 1) / kTok;
  const int seq = decode ? r : 0;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  uint32_t* smask = reinterpret_cast<uint32_t*>(MASKED ? srow : srow + tok_per_split);

  if (w == kMlaWaves) {
    // ---------------------------------------------------------------- copy wave
    const int32_t* irow = idx + (int64_t)r * k + t_begin;
    // Rows are addressed relative to `base`: the sequence's first row (contiguous) or the
    // pool (paged: the page table is resolved here, once per kept token).
    const uint16_t* base = PAGED ? kv : kv + (int64_t)seq * seq_stride * kDqk;
    auto resolve = [&](int id) -> int {  // cache row of a token index (-1 stays -1)
      if (!PAGED) return id;
      const int pg = table[(int64_t)seq * max_pages + (id >= 0 ? id : 0) / page_size];
      return id >= 0 ? pg * page_size + id % page_size : -1;
    };
    // Dead rows (past the range or index -1) copy this row's first query row, which is
    // finite, so masked tokens never inject NaN into the value products.
    const uint16_t* dummy = q + (int64_t)r * H * kDqk;
    const int half = lane >> 5;  // lanes 32-63 copy the row's second half (chunks 36..71)
    auto issue_row = [&](int row, char* dst) {
      const uint16_t* src = (row >= 0 ? base + (int64_t)row * kDqk : dummy) + half * (kDqk / 2);
#pragma unroll
      for (int j = 0; j < kDmaPerTile; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(src + 8 * j),
                                         (lds_void*)(uintptr_t)(lds_offset(dst) + j * kBlock), 16, 0, 0);
    };
    int last = MASKED ? n_tok - 1 : -1;  // last kept token of the range (uniform)
    if (MASKED) {
      // Live masks from the kept set (positions outside 0..r are ignored), then tiles 0
      // and 1 of the contiguous positions.
      for (int i = lane; i < ntiles; i += WAVE) smask[i] = 0u;
      const int32_t* krow = idx + (int64_t)r * k;
      constexpr int U = 8;
      for (int j0 = 0; j0 < k; j0 += U * WAVE) {
        int id[U];
#pragma unroll
        for (int u = 0; u < U; ++u) id[u] = krow[min(j0 + u * WAVE + lane, k - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int s = id[u];
          if (j0 + u * WAVE + lane < k && s >= 0 && s < n_tok) atomicOr(&smask[s >> 5], 1u << (s & 31));
        }
      }
      if (ntiles > 0) issue_row((lane & 31) < n_tok ? (lane & 31) : -1, g_ring0);
      if (ntiles > 1) issue_row(32 + (lane & 31) < n_tok ? 32 + (lane & 31) : -1, g_ring1);
    } else {
      // The first batch of the row list (tokens 0 .. U * 64 - 1) is loaded before any copy goes
      // out: loads and copies retire in issue order, so list loads issued after the 72 copies of
      // tiles 0 and 1 could only be waited for once both tiles had landed, which held tile 0's
      // hand-over back until tile 1 was in LDS too.
      constexpr int U = 8;
      int id[U];
#pragma unroll
      for (int u = 0; u < U; ++u) id[u] = u * WAVE < n_tok ? irow[min(u * WAVE + lane, n_tok - 1)] : -1;
      __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of the copies
      // Tiles 0 and 1 straight from the first 64 indices (token = lane).
      {
        const int v = lane < n_tok ? id[0] : -1;
        const int row = resolve(v);
        const uint64_t live = ballot(row >= 0);
        if (live) last = 63 - (int)__builtin_clzll(live);
        if (lane < n_tok) srow[lane] = row;
        if (lane == 0) {
          if (ntiles > 0) smask[0] = (uint32_t)live;
          if (ntiles > 1) smask[1] = (uint32_t)(live >> 32);
        }
        // lane l needs token l & 31 (tile 0) and 32 + (l & 31) (tile 1)
        const v2i sw = __builtin_amdgcn_permlane32_swap(row, row, false, false);
        if (ntiles > 0) issue_row(sw[0], g_ring0);
        if (ntiles > 1) issue_row(sw[1], g_ring1);
      }
      // Row list entries of tokens i0 + 64 u + lane (u >= u0) from id[].
      auto list = [&](int i0, auto u0) {
#pragma unroll
        for (int u = decltype(u0)::value; u < U; ++u) {
          const int i = i0 + u * WAVE + lane;
          const int row = resolve(i < n_tok ? id[u] : -1);
          const uint64_t live = ballot(row >= 0);
          if (live) last = i0 + u * WAVE + 63 - (int)__builtin_clzll(live);
          if (i < n_tok) srow[i] = row;
          const int t0 = (i0 + u * WAVE) / kTok;
          if (lane == 0 && t0 < ntiles) smask[t0] = (uint32_t)live;
          if (lane == 0 && t0 + 1 < ntiles) smask[t0 + 1] = (uint32_t)(live >> 32);
        }
      };
      list(0, std::integral_constant<int, 1>{});
      // Later batches (splits of more than U * 64 tokens), 8 tokens per lane per batch.
      for (int i0 = U * WAVE; i0 < n_tok; i0 += U * WAVE) {
#pragma unroll
        for (int u = 0; u < U; ++u) id[u] = irow[min(i0 + u * WAVE + lane, n_tok - 1)];  // unconditional: no wait between batch members
        list(i0, std::integral_constant<int, 0>{});
      }
    }
    // Tiles run: through the last kept token, at least one (tiles 0 and 1 are already in
    // flight; the last hand-over drains whatever was issued).
    const int nt = ntiles == 0 ? 0 : max(1, min(ntiles, (last + kTok) / kTok));
    if (lane == 0) g_ntiles = nt;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the count is in LDS before the barrier
    auto row_of_tile = [&](int t) {
      const int tok = t * kTok + (lane & 31);
      return tok < n_tok ? (MASKED ? tok : srow[tok]) : -1;
    };
    auto hand = [&](auto slot, int t) {
      constexpr int S = decltype(slot)::value;
      if (t + 1 < nt) wait_vmcnt<kDmaPerTile>();  // tile t landed, t+1 may be in flight
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();                    // hand tile t to the compute waves
      if (t + 2 < nt) issue_row(row_of_tile(t + 2), ring_slot<(S + 2) % kNBuf>());
      __builtin_amdgcn_s_barrier();  // the compute waves' logit exchange (barriers must pair up)
    };
    for (int t = 0; t < nt; t += kNBuf) {
      hand(Slot<0>{}, t);
      if (t + 1 < nt) hand(Slot<1>{}, t + 1);
      if (t + 2 < nt) hand(Slot<2>{}, t + 2);
    }
    return;
  }

  // ------------------------------------------------------------------ compute waves
  const int hb = w & 3;     // head block
  const int half = w >> 2;  // latent-column half (logits) and value-column half (output)
  // Query fragments of this wave's column half: B[k = dim][n = head col] =
  // q[r, h, 288*half + 32*kk + 8*grp + j].
  constexpr int kKK = kDqk / 64;  // 9 steps of 32 columns per half
  const int col = lane & 15, grp = lane >> 4;
  const int h = hg * kHeadsPerWg + 16 * hb + col;
  const uint16_t* qrow = q + ((int64_t)r * H + h) * kDqk + (kDqk / 2) * half;
  v8bf qf[kKK];
  {
    // Each quad of lanes (4 hh .. 4 hh + 3) loads one head's 64-byte piece of a k-step, so a
    // load makes 16 cache-line requests instead of 64 (at start-up every workgroup loads its
    // queries at once, beside the first gathers); a lane permute then moves piece grp of head
    // col to lane col + 16 grp, the operand layout.
    const int hh = lane >> 2, g = lane & 3;
    const uint4* qp = reinterpret_cast<const uint4*>(qrow + (int64_t)(hh - col) * kDqk) + g;
    uint4 raw[kKK];
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) raw[kk] = qp[4 * kk];
    const int src = 4 * col + grp;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      const uint4 t = make_uint4((uint32_t)__shfl((int)raw[kk].x, src), (uint32_t)__shfl((int)raw[kk].y, src),
                                 (uint32_t)__shfl((int)raw[kk].z, src), (uint32_t)__shfl((int)raw[kk].w, src));
      qf[kk] = __builtin_bit_cast(v8bf, t);
    }
  }
  constexpr int kVSide1 = 14;  // half 1: value tiles below this are on side 1
  v4f acc_o[kDv / 32];         // value tile dt of this half (columns in the epilogue), head col
#pragma unroll
  for (int dt = 0; dt < kDv / 32; ++dt) acc_o[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // reference max of scaled logits (log2 domain), per head = col
  float l_run = 0.0f;       // this lane's share of the running sum
  // Logit fragments: chunk 36*half + 4*kk + grp of row 16*st + col sits in block 4*kk + grp,
  // side `half` (tile layout above), so every fragment is this lane base plus a constant.
  const int qk_lane = grp * kBlock + 512 * half + 16 * col;
  // Value fragments.  Value-column tile dt (16 columns, chunks 2dt' and 2dt'+1 of the row)
  // is read by a transposing load where lane (col, grp) supplies row 4*grp + col/4 (+16),
  // columns +4*(col&3) .. +3: chunk +(col&3)/2, byte 8*(col&1).  Half 0 takes chunks 0..31
  // (side 0, blocks 0..31); half 1 takes chunks 36..63 (side 1, blocks 0..27) as its tiles
  // 0..13 and chunks 32..35 (side 0, blocks 32..35) as tiles 14 and 15.  Both are a lane
  // base plus a constant per tile.
  const int pv_lane = ((col & 3) >> 1) * kBlock + 16 * (4 * grp + (col >> 2)) + 8 * (col & 1);
  const int pv_lane_a = pv_lane + 512 * half;            // tiles 0..13
  const int pv_lane_b = pv_lane + (half ? 4 * kBlock : 0);  // tiles 14, 15
  float* xmine = &g_xchg[w][lane * 8];
  const float* xpart = &g_xchg[w ^ 4][lane * 8];

  auto step = [&](auto slot, int t) {
    constexpr int S = decltype(slot)::value;
    __builtin_amdgcn_s_barrier();  // tile t is in ring slot S
    const char* tb = ring_slot<S>();
    // ---- partial S^T over this wave's 288 columns: tokens 16*st + row, two accumulation
    // chains (one per token half), KD K fragments in flight.
    constexpr int NF = 2 * kKK;
    constexpr int KD = 4;
    const char* kb = tb + qk_lane;
    auto kfrag = [&](int i) {
      return *reinterpret_cast<const v8bf*>(kb + (i >> 1) * 4 * kBlock + (i & 1) * 256);
    };
    v8bf kf[KD];
#pragma unroll
    for (int i = 0; i < KD; ++i) kf[i] = kfrag(i);
    v4f as[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const v8bf a = kf[i % KD];
      if (i + KD < NF) kf[i % KD] = kfrag(i + KD);
      as[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[i >> 1], as[i & 1], 0, 0, 0);
    }
    // (Compute waves issue no copies, so these stores wait on nothing in flight.)
    *reinterpret_cast<v4f*>(xmine) = as[0];
    *reinterpret_cast<v4f*>(xmine + 4) = as[1];
    // First value fragments, read while the partner's logits arrive.
    constexpr int VD = 3;
    v4bf vlo[VD], vhi[VD];
    auto vfrag = [&](int dt, v4bf& lo, v4bf& hi) {
      const char* vb = tb + (dt < kVSide1 ? pv_lane_a : pv_lane_b) + dt * 2 * kBlock;
      lo = lds_read_tr16(vb);
      hi = lds_read_tr16(vb + 16 * 16);
    };
#pragma unroll
    for (int d = 0; d < VD; ++d) vfrag(d, vlo[d], vhi[d]);
    const uint32_t live = smask[t];
    __syncthreads();  // both halves of every logit tile are in LDS
    const v4f p0 = *reinterpret_cast<const v4f*>(xpart);
    const v4f p1 = *reinterpret_cast<const v4f*>(xpart + 4);
    // Both waves of a pair add the same two halves (a + b == b + a), so their logits agree.
    const v4f sf[2] = {as[0] + p0, as[1] + p1};
    // ---- online softmax (lane holds tokens 16*st + 4*grp + i of head col)
    float s[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = (live >> (16 * st + 4 * grp + i)) & 1u;
        s[st][i] = ok ? sf[st][i] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[st][i]);
      }
    }
    mx = max_x32(max_x16(mx));
    // Lazy rescaling: the reference max only moves when a logit exceeds it by more than
    // 2^8 (or on the first valid tile), so p <= 256 and the accumulators rarely rescale.
    float m_ref = m_run;
    if (__ballot(mx > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDv / 32; ++dt) acc_o[dt] *= alpha;
      m_ref = m_new;
    }
    m_run = m_ref;
    const float m_use = m_ref == -INFINITY ? 0.0f : m_ref;  // no valid token yet: p = 0
    float p[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[st][i] = __builtin_amdgcn_exp2f(s[st][i] - m_use);
        psum += p[st][i];
      }
    }
    l_run += psum;
    // P^T fragment: k-slot 8*grp + j <-> token 4*grp + j (j < 4) or 16 + 4*grp + (j - 4).
    v8bf pf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pf[i] = (__bf16)p[0][i];
      pf[4 + i] = (__bf16)p[1][i];
    }
    // ---- O^T += V^T P^T over this wave's 16 tiles of 16 value columns
#pragma unroll
    for (int dt = 0; dt < kDv / 32; ++dt) {
      const v8bf a = __builtin_shufflevector(vlo[dt % VD], vhi[dt % VD], 0, 1, 2, 3, 4, 5, 6, 7);
      if (dt + VD < kDv / 32) vfrag(dt + VD, vlo[dt % VD], vhi[dt % VD]);
      acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, acc_o[dt], 0, 0, 0);
    }
  };

  if (ntiles > 0) {
    step(Slot<0>{}, 0);
    const int nt = g_ntiles;  // written by the copy wave before the first hand-over
    if (1 < nt) step(Slot<1>{}, 1);
    if (2 < nt) step(Slot<2>{}, 2);
    for (int t = kNBuf; t < nt; t += kNBuf) {
      step(Slot<0>{}, t);
      if (t + 1 < nt) step(Slot<1>{}, t + 1);
      if (t + 2 < nt) step(Slot<2>{}, t + 2);
    }
  }

  const float l = sum_x32(sum_x16(l_run));
  // First value column of this lane in tile dt: half 0 tile dt = columns 16*dt; half 1
  // tiles 0..13 = columns 288 + 16*dt, tiles 14, 15 = columns 256 + 16*(dt - 14).
  auto vcol = [&](int dt) {
    return 4 * grp + (half == 0 ? 16 * dt : (dt < kVSide1 ? 288 + 16 * dt : 256 + 16 * (dt - kVSide1)));
  };
  // Split partials hold this split's own normalized output (bf16, like the final output)
  // and its (max, sum) in fp32; the merge weights each by sum * 2^(max - overall max).
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  // The 64 head rows go out through the idle ring: each wave writes its bf16 pieces into the
  // head's row (rows 0..31 in slot 0, 32..63 in slot 1, padded to 1040 bytes), then every
  // store instruction writes one whole 1 KB row.  Storing from the accumulator layout would
  // spread each instruction's 8-byte pieces over 16 head rows.
  constexpr int ROWB = kDv * 2 + 16;
  static_assert(32 * ROWB <= kBufBytes, "32 head rows fit one slot");
  __syncthreads();  // every compute wave is done with the ring (the copy wave has left)
  {
    char* srow_h = (hb >> 1 ? g_ring1 : g_ring0) + (16 * (hb & 1) + col) * ROWB;
#pragma unroll
    for (int dt = 0; dt < kDv / 32; ++dt) {
      const uint32_t lo = f32_to_bf16(acc_o[dt][0] * inv) | ((uint32_t)f32_to_bf16(acc_o[dt][1] * inv) << 16);
      const uint32_t hi = f32_to_bf16(acc_o[dt][2] * inv) | ((uint32_t)f32_to_bf16(acc_o[dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(srow_h + 2 * vcol(dt)) = make_uint2(lo, hi);
    }
  }
  if (grp == 0 && half == 0) {
    if (SPLIT) {
      const int64_t pr = ((int64_t)r * n_split + sp) * H + h;
      part_ml[2 * pr] = m_run;
      part_ml[2 * pr + 1] = l;
    } else if (lse) {
      lse[(int64_t)r * H + h] = l > 0.0f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kHeadsPerWg / kMlaWaves; ++i) {  // row rr of the workgroup's 64 heads
    const int rr = w + kMlaWaves * i;
    const int hd = hg * kHeadsPerWg + rr;
    uint16_t* dst = SPLIT ? part_o + (((int64_t)r * n_split + sp) * H + hd) * kDv : out + ((int64_t)r * H + hd) * kDv;
    const uint4 v = *reinterpret_cast<const uint4*>((rr >> 5 ? g_ring1 : g_ring0) + (rr & 31) * ROWB + 16 * lane);
    *reinterpret_cast<uint4*>(dst + 8 * lane) = v;
  }
}

// Wide variant: one workgroup = (row, 32 * NW heads, a range of the kept set), NW waves and no
// copy wave.  Per 32-row tile:
//   * logits: wave w owns 32 heads over all 576 latent columns: S^T (32 tokens x 32 heads)
//     = K Q^T with v_mfma_f32_32x32x16_bf16 (36 k-steps, one accumulation chain), so its
//     logits need no exchange.  Softmax statistics of those heads live in wave w only.
//   * P exchange: the 32x32 result layout leaves each lane 16 tokens of one head, which are
//     exactly the B operand (P^T, two 16-token k-steps) of the value product; each wave
//     publishes its heads' bf16 probabilities in LDS (2 KB); one barrier.
//   * values: wave w accumulates O^T for ALL heads of the workgroup over its 512 / NW value
//     columns (32x32x16 tiles), so each transposing V^T read from LDS feeds NW MFMAs and a
//     tile's V^T crosses LDS once in total.
// One wave issues 32x32x16 bf16 MFMAs at about 2.1 PFLOP/s chip-wide against about 1.4 for
// 16x16x32 (own measurement, one wave per SIMD), hence this shape.  The accumulators (NW head
// blocks x 16 / NW value blocks x 16 = 256 per lane) sit in AGPRs and the 32 heads' query
// fragments in 144 VGPRs: one wave per SIMD.
//
// Tile layout in LDS (this variant): 36 blocks of 1 KB; block b holds rows 16 * (b & 1) .. + 15
// and 16-byte chunks 4 * (b >> 1) .. + 3 of those rows, chunk-major with a row swizzle: chunk
// cc of row rr at byte 256 * cc + 16 * (rr ^ 4 * cc).  One wide LDS-DMA copy fills one block
// (lane l loads chunk l >> 4 of row (l & 15) ^ 4 * (l >> 4)), so a copy touches 16 rows'
// 64-byte pieces -- 16 cache lines rather than the 64 of a copy taking 16 bytes from each of
// 64 rows, which the memory path handles several times slower.  The swizzle makes both the K
// fragment reads (16 rows of one chunk per 16 lanes) and the transposing V^T reads (4 rows x 2
// chunks per 16 lanes) cover every LDS bank evenly: neither has bank conflicts.
//
// Gathers: every wave issues its share (36 / NW) of each tile's copies -- all in the same
// 16-row half -- into a three-slot ring, two tiles ahead, spread over the logit MFMAs; the
// first barrier of a tile both publishes tile t (each wave first waits for its own copies of
// it) and retires tile t - 1, whose slot then takes tile t + 2.  The row list (cache row of
// each kept token, -1 for none) and each tile's live-token mask are built by all waves before
// the first copy.
template <int NW, bool PAGED, bool SPLIT, bool MASKED = false>
__global__ __launch_bounds__(NW * WAVE) void mla_wide_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ table, int max_pages, int page_size, int64_t seq_stride,
    const int32_t* __restrict__ idx, int k, int H, int decode, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o,
    float* __restrict__ part_ml, int n_split, int tok_per_split) {
  static_assert(NW == 2 || NW == 4, "32 heads per wave, 64 or 128 per workgroup");
  constexpr int HPW = 32 * NW;              // heads per workgroup
  constexpr int CPW = kDmaPerTile / NW;     // copies per wave per tile
  constexpr int KS = kDqk / 16;             // 36 k-steps of 16 latent columns
  constexpr int CB = kDv / 32 / NW;         // 32-column value blocks per wave
  extern __shared__ int srow[];  // [tok_per_split] cache row of each kept token (-1 = none),
                                 // then [tiles] live-token mask of each tile (MASKED: masks only)
  __shared__ int s_last[NW];
  __shared__ __attribute__((aligned(16))) v8bf s_p[NW][2][WAVE];  // P^T fragments per head block
  __shared__ float s_alpha[NW][32];                                // rescale factor per head
  __shared__ int s_flag[2];                                        // a head rescaled (parity)
  __shared__ float s_fin[NW][32];                                  // 1 / sum per head (epilogue)
  const int HG = H / HPW;
  int unit, hg;
  {
    const int b = (int)blockIdx.x, full = ((int)gridDim.x / HG) / 8 * 8 * HG;
    if (b < full) {
      unit = b / (8 * HG) * 8 + b % 8;
      hg = (b / 8) % HG;
    } else {
      unit = full / HG + (b - full) / HG;
      hg = (b - full) % HG;
    }
  }
  const int sp = unit % n_split;
  const int r = unit / n_split;
  const int t_begin = MASKED ? 0 : sp * tok_per_split;
  const int t_end = MASKED ? r + 1 : min(k, t_begin + tok_per_split);
  const int n_tok = t_end > t_begin ? t_end - t_begin : 0;
  const int ntiles = (n_tok + kTok - 1) / kTok;
  const int seq = decode ? r : 0;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);  // wave-uniform (scalar)
  const int n = lane & 31, h = lane >> 5;  // 32x32 MFMA lane coordinates
  uint32_t* smask = reinterpret_cast<uint32_t*>(MASKED ? srow : srow + tok_per_split);

  // The first batch of this wave's row-list indices goes out before the query loads, whose
  // issue alone takes thousands of cycles (each touches 32 cache lines): the index round trip
  // then overlaps it instead of following it.
  const int32_t* irow = idx + (int64_t)r * k + t_begin;
  int v_first = -1;
  if (!MASKED && 64 * w < n_tok) v_first = irow[min(64 * w + lane, n_tok - 1)];
  __builtin_amdgcn_sched_barrier(0);
  // ---- query fragments (B operand of S^T = K Q^T): lane (n, h) holds, for k-step ks,
  // q[r, head n of this wave, 16 * ks + 8 * h .. + 7].  Issued before the row list is built
  // so their latency overlaps it.
  v8bf qf[KS];
  {
    const int hd = hg * HPW + 32 * w + n;
    const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)r * H + hd) * kDqk + 8 * h);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(v8bf, qp[2 * ks]);
  }

  // ---- row list and live masks
  const uint16_t* base = PAGED ? kv : kv + (int64_t)seq * seq_stride * kDqk;
  const uint16_t* dummy = q + (int64_t)r * H * kDqk;  // finite stand-in for dead rows
  int last = -1;                                      // last live token this wave saw
  if (tid < 2) s_flag[tid] = 0;
  if (tid < NW * 32) s_alpha[tid / 32][tid % 32] = 1.0f;
  if (MASKED) {
    for (int i = tid; i < ntiles; i += NW * WAVE) smask[i] = 0u;
    __syncthreads();
    const int32_t* krow = idx + (int64_t)r * k;
    for (int j = tid; j < k; j += NW * WAVE) {
      const int s = krow[j];
      if (s >= 0 && s < n_tok) {
        atomicOr(&smask[s >> 5], 1u << (s & 31));
        last = max(last, s);
      }
    }
  } else {
    for (int i0 = 64 * w; i0 < n_tok; i0 += 64 * NW) {
      const int i = i0 + lane;
      const int v = i < n_tok ? (i0 == 64 * w ? v_first : irow[i]) : -1;
      int row = v;
      if (PAGED && v >= 0) row = table[(int64_t)seq * max_pages + v / page_size] * page_size + v % page_size;
      const uint64_t live = ballot(row >= 0);
      if (live) last = i0 + 63 - (int)__builtin_clzll(live);
      if (i < n_tok) srow[i] = row;
      if (lane == 0) {
        const int t0 = i0 / kTok;
        if (t0 < ntiles) smask[t0] = (uint32_t)live;
        if (t0 + 1 < ntiles) smask[t0 + 1] = (uint32_t)(live >> 32);
      }
    }
  }
  {
    int m = last;
    for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o));
    if (lane == 0) s_last[w] = m;
  }
  __syncthreads();
  int lst = -1;
#pragma unroll
  for (int i = 0; i < NW; ++i) lst = max(lst, s_last[i]);
  // tiles run: through the last kept token (at least one when the range is not empty, so an
  // all-dead range still writes its zero output and -inf statistics)
  const int nt = ntiles == 0 ? 0 : max(1, min(ntiles, (lst + kTok) / kTok));

  // This wave's copies are blocks j = w + NW * c: all in row half w & 1 (NW is even).  Lane
  // l loads chunk 4 * (j >> 1) + (l >> 4) of tile row 16 * (w & 1) + ((l & 15) ^ 4 * (l >> 4)).
  const int crow = 16 * (w & 1) + ((lane & 15) ^ (4 * (lane >> 4)));
  // Cache row of this lane's copy row in tile t; tiles past the last one and dead tokens
  // use the finite dummy row (-1).
  auto tile_row = [&](int t) {
    const int tok = t * kTok + crow;
    return (t < nt && tok < n_tok) ? (MASKED ? tok : srow[tok]) : -1;
  };
  auto row_src = [&](int row) {
    return (row >= 0 ? base + (int64_t)row * kDqk : dummy) + 8 * (lane >> 4);
  };
  // Copy c (of this wave's CPW) of a tile into block j = w + NW * c of the slot.
  auto copy = [&](auto slot, const uint16_t* src, int c) {
    constexpr int S = decltype(slot)::value;
    const int j = w + NW * c;
    lds_dma16(src + 32 * (j >> 1), __builtin_amdgcn_readfirstlane(lds_offset(ring_slot<S>()) + j * kBlock));
  };
  auto issue = [&](auto slot, int t) {
    const uint16_t* src = row_src(tile_row(t));
#pragma unroll
    for (int c = 0; c < CPW; ++c) copy(slot, src, c);
  };
  // The query fragments have landed (they were issued before the index loads the row list
  // waited for); waiting here tells the compiler so, and no wait inside the tile loop is
  // left to count them among the copies in flight.
  wait_vmcnt<0>();
  // Every step issues a full tile of copies (tiles past the last one copy the dummy row into
  // the free slot), so each wave always has exactly one tile of copies in flight behind the
  // one it waits for.
  if (nt > 0) {
    issue(Slot<0>{}, 0);
    issue(Slot<1>{}, 1);
  }
  int next_row = tile_row(2);  // copy row of the tile two ahead, read one step early

  v16f acc[CB][NW];  // value block x head block; lane (n, h): columns 8 j + 4 h + i, head n
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int b = 0; b < NW; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[cb][b][e] = 0.0f;
  float m_run = -INFINITY;  // reference max of head n (log2 domain)
  float l_run = 0.0f;       // this lane's share of the running sum
  // K fragment (A operand) of k-step ks: lane (n, h) = row n, chunk 2 ks + h -> block
  // 2 (ks >> 1) + (n >> 4), chunk-in-block cc = 2 (ks & 1) + h, at 256 cc + 16 ((n & 15) ^ 4 cc).
  int k_lane[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int cc = 2 * p + h;
    k_lane[p] = (n >> 4) * kBlock + 256 * cc + 16 * ((n & 15) ^ (4 * cc));
  }
  // V^T fragment (A operand) of value block CBg, k-step ks': lane (n, h) = value column
  // 32 CBg + n, tokens 16 ks' + 4 h + 0..3 (lo) and 16 ks' + 8 + 4 h + 0..3 (hi).  The
  // transposing read: in 16-lane group g = lane >> 4, lane i points at token row
  // 16 ks' + 4 (g >> 1) + (i >> 2) (+ 8 for hi), columns 16 (g & 1) + 4 (i & 3) .. + 3 of the
  // block = chunk 4 CBg + cc, cc = 2 (g & 1) + (i & 3) / 2, byte 8 (i & 1).
  int v_lane[2];
  {
    const int g = lane >> 4, i = lane & 15;
    const int cc = 2 * (g & 1) + ((i & 3) >> 1);
    const int rr = 4 * (g >> 1) + (i >> 2);
    v_lane[0] = 256 * cc + 16 * (rr ^ (4 * cc)) + 8 * (i & 1);
    v_lane[1] = 256 * cc + 16 * ((rr + 8) ^ (4 * cc)) + 8 * (i & 1);
  }

  auto step = [&](auto slot, int t) {
    constexpr int S = decltype(slot)::value;
    constexpr int SN = (S + 2) % kNBuf;
    // This wave's copies of tile t landed (those of t + 1 may be in flight) and its LDS
    // writes of the previous tile (flag clear, rescale factors) completed.
    __builtin_amdgcn_s_waitcnt((CPW & 15) | (0 << 8) | (7 << 4) | ((CPW >> 4) << 14));
    // Every wave's copies of tile t landed; tile t - 1 (and its P) retired.  A bare barrier: a
    // workgroup fence here would also wait for tile t + 1's copies.  The empty asm keeps the
    // compiler from moving LDS accesses across it.
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Clear the other parity's rescale flag for tile t + 1: every wave read it at tile t - 1
    // and has passed the barrier above since.
    if (tid == 0) s_flag[(t + 1) & 1] = 0;
    const uint16_t* nsrc = row_src(next_row);
    const char* tb = ring_slot<S>();
    const uint32_t live = smask[t];
    // ---- S^T = K Q^T for the own 32 heads, one accumulation chain (a second chain's 16
    // registers push query fragments out of registers and costs more than it gains).  Tile
    // t + 2's copies go out one every KS / CPW k-steps, behind the MFMAs.
    constexpr int KD = 3;
    constexpr int CSTEP = KS / CPW;
    auto kfrag = [&](int ks) {
      return *reinterpret_cast<const v8bf*>(tb + (ks >> 1) * 2 * kBlock + k_lane[ks & 1]);
    };
    v8bf kf[KD];
#pragma unroll
    for (int i = 0; i < KD; ++i) kf[i] = kfrag(i);
    v16f sc[1];
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[0][e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const v8bf a = kf[ks % KD];
      if (ks + KD < KS) kf[ks % KD] = kfrag(ks + KD);
      sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sc[0], 0, 0, 0);
      if (ks % CSTEP == 0 && ks / CSTEP < CPW) copy(Slot<SN>{}, nsrc, ks / CSTEP);
    }
    // ---- online softmax of head n: register 4 j + i holds token 8 j + 4 h + i
    // Dead tokens' logits become -inf (their probability exp2(-inf) = 0); a fully live tile
    // (the usual case; uniform) skips the per-token test.
    if (live != 0xFFFFFFFFu) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (!((live >> (8 * (e >> 2) + 4 * h + (e & 3))) & 1u)) sc[0][e] = -INFINITY;
    }
    float mx = -INFINITY;  // this lane's max scaled logit (the head's max needs lane n + 32 too)
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[0][e]);
    mx *= scale_log2;  // scale_log2 > 0
    // Reference max: the first tile with a live token sets it (the accumulators are still
    // zero); afterwards it moves only when a logit exceeds it by more than 2^64 (log2 domain),
    // so p <= 2^64 and sums of 2^13 such terms stay far inside the fp32 and bf16 ranges.  Such
    // a move (rare) rescales every wave's accumulators of the head, through s_alpha; no VALU
    // instruction otherwise takes an accumulator as an operand, so they stay in AGPRs.  Both
    // lanes of a head hold the same reference, so testing each lane's own max finds every
    // head that needs a move.
    float m_ref = m_run;
    float alpha = 1.0f;
    bool resc = false;
    if (__ballot(m_ref == -INFINITY)) {  // a head with no live token yet (first tiles only)
      mx = max_x32(mx);
      if (m_ref == -INFINITY) m_ref = mx;  // stays -inf while the head has no live token
    } else if (__ballot(mx > m_ref + kRescaleLog2)) {
      mx = max_x32(mx);
      const float m_new = fmaxf(m_ref, mx);
      alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      l_run *= alpha;
      m_ref = m_new;
      resc = true;
    }
    m_run = m_ref;
    const float m_use = m_ref == -INFINITY ? 0.0f : m_ref;
    float psum = 0.0f;
    v8bf pf[2];  // P^T of k-step ks': slot 8 h + e' <-> token 16 ks' + 8 (e' >> 2) + 4 h + (e' & 3)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[0][e], scale_log2, -m_use));
      psum += p;
      pf[e >> 3][e & 7] = (__bf16)p;
    }
    l_run += psum;
    s_p[w][0][lane] = pf[0];
    s_p[w][1][lane] = pf[1];
    if (resc) {
      if (h == 0) s_alpha[w][n] = alpha;
      if (lane == 0) s_flag[t & 1] = 1;
    }
    next_row = tile_row(t + 3);  // for the next step's copies; its LDS latency hides here
    // Every head's probabilities are in LDS: this wave's writes have completed (lgkmcnt(0);
    // the bare barrier does not wait for them) before any wave passes the barrier.
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (s_flag[t & 1]) {  // rare: some head's reference max moved; rescale its accumulators
      volatile v16f tmp;
#pragma unroll
      for (int b = 0; b < NW; ++b) {
        const float a = s_alpha[b][n];
        if (__ballot(a != 1.0f)) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            tmp = acc[cb][b];
            v16f x = tmp;
            tmp = x * a;
            acc[cb][b] = tmp;
          }
        }
      }
    }
    // ---- O^T += V^T P^T over this wave's value blocks, every head block of the workgroup;
    // one 16-token k-step at a time (half the P fragments live at once)
    auto vfrag = [&](int cb, int ks2) {
      lds_char* vb = ring_lds<S>() + (2 * (CB * w + cb) + ks2) * kBlock;
      const v4bf lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(vb + v_lane[0]));
      const v4bf hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(vb + v_lane[1]));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    constexpr int VD = 2;
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      v8bf pb[NW];
#pragma unroll
      for (int b = 0; b < NW; ++b) pb[b] = s_p[b][ks2][lane];
      v8bf vf[VD];
#pragma unroll
      for (int d = 0; d < VD; ++d) vf[d] = vfrag(d, ks2);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const v8bf a = vf[cb % VD];
        if (cb + VD < CB) vf[cb % VD] = vfrag(cb + VD, ks2);
#pragma unroll
        for (int b = 0; b < NW; ++b)
          acc[cb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[b], acc[cb][b], 0, 0, 0);
      }
    }
    if (resc && h == 0) s_alpha[w][n] = 1.0f;
  };
  __syncthreads();  // the rescale factors and flags are set

  for (int t = 0; t < nt; t += kNBuf) {
    step(Slot<0>{}, t);
    if (t + 1 < nt) step(Slot<1>{}, t + 1);
    if (t + 2 < nt) step(Slot<2>{}, t + 2);
  }
  wait_vmcnt<0>();  // the copies issued past the last tile land before the LDS is released

  // ---- epilogue: statistics of the own heads, then every wave's value columns of all heads
  {
    const int hd = hg * HPW + 32 * w + n;
    const float l = sum_x32(l_run);
    if (h == 0) {
      s_fin[w][n] = l > 0.0f ? 1.0f / l : 0.0f;
      if (SPLIT) {
        const int64_t pr = ((int64_t)r * n_split + sp) * H + hd;
        part_ml[2 * pr] = m_run;
        part_ml[2 * pr + 1] = l;
      } else if (lse) {
        lse[(int64_t)r * H + hd] = l > 0.0f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
      }
    }
  }
  // The output (or this split's partial) rows go out through LDS: every wave scales its
  // accumulators and writes them as bf16 into the (now idle) ring, then each store
  // instruction writes one head's whole 1 KB row.  Storing straight from the accumulator
  // layout would spread every instruction's 8-byte pieces over 32 head rows.  Two rounds of
  // NW / 2 head blocks; block bb of a round goes to ring slot bb, its 32 head rows padded to
  // 1040 bytes (33,280 bytes per slot), so every staging address is a lane base plus a
  // constant.
  __syncthreads();  // s_fin visible; every wave is done with the ring
  constexpr int RH = HPW / 2;         // head rows per round
  constexpr int ROWB = kDv * 2 + 16;  // padded LDS row: 2-way bank conflicts at most
  static_assert(32 * ROWB <= kBufBytes && NW / 2 <= kNBuf, "a head block's rows fit one slot");
  auto slot_base = [](int bb) -> char* { return bb == 0 ? g_ring0 : (bb == 1 ? g_ring1 : g_ring2); };
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
#pragma unroll
    for (int bb = 0; bb < NW / 2; ++bb) {
      const int b = rd * (NW / 2) + bb;
      const float inv = s_fin[b][n];
      char* srow_b = slot_base(bb) + n * ROWB + 2 * (32 * CB * w + 4 * h);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v16f& x = acc[cb][b];
          const v4bf o4 = {(__bf16)(x[4 * j] * inv), (__bf16)(x[4 * j + 1] * inv), (__bf16)(x[4 * j + 2] * inv),
                           (__bf16)(x[4 * j + 3] * inv)};
          *reinterpret_cast<v4bf*>(srow_b + 2 * (32 * cb + 8 * j)) = o4;
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RH / NW; ++i) {  // row rr: head block rr >> 5 of the round, head rr & 31
      const int rr = w + NW * i;
      const int hd = hg * HPW + rd * RH + rr;
      uint16_t* dst = SPLIT ? part_o + (((int64_t)r * n_split + sp) * H + hd) * kDv
                            : out + ((int64_t)r * H + hd) * kDv;
      const uint4 v = *reinterpret_cast<const uint4*>(slot_base(rr >> 5) + (rr & 31) * ROWB + 16 * lane);
      *reinterpret_cast<uint4*>(dst + 8 * lane) = v;
    }
    if (rd == 0) __syncthreads();  // round 0's rows are read before round 1 overwrites them
  }
}

// Log-sum-exp merge of the split partials: one wave per (row, head), 8 value columns per
// lane (16-byte loads and stores).  Split s contributes its normalized output u_s with
// weight l_s * 2^(m_s - M).  Splits are taken NB at a time (NB = the split count rounded up
// to a power of two, at most 16) with every load of a batch -- values and the (max, sum)
// pairs alike -- issued before any is used, so a typical merge is one round trip; batches
// after the first rescale the running sums to the new maximum.
constexpr int kCombinePairs = 4;  // (row, head) pairs per 256-thread workgroup
template <int NB>
__global__ __launch_bounds__(256) void mla_combine_kernel(const uint16_t* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int RH, int H, int n_split,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int pair = blockIdx.x * kCombinePairs + threadIdx.x / WAVE;
  if (pair >= RH) return;
  const int r = pair / H, h = pair % H;
  const int t = threadIdx.x & (WAVE - 1);
  const int64_t p0 = (int64_t)r * n_split * H + h;  // partial of split s at p0 + s * H
  float M = -INFINITY, L = 0.0f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_split; s0 += NB) {
    float2 ml[NB];
    uint4 v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int64_t pr = p0 + (int64_t)min(s0 + u, n_split - 1) * H;
      ml[u] = *reinterpret_cast<const float2*>(part_ml + 2 * pr);
      v[u] = *reinterpret_cast<const uint4*>(part_o + pr * kDv + 8 * t);
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (s0 + u < n_split && ml[u].y > 0.0f) Mb = fmaxf(Mb, ml[u].x);
    const float c = M == -INFINITY ? 0.0f : exp2f(M - Mb);
    L *= c;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= c;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const bool valid = s0 + u < n_split && ml[u].y > 0.0f;
      const float f = valid ? ml[u].y * exp2f(ml[u].x - Mb) : 0.0f;
      L += f;
      const uint32_t wv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += __uint_as_float(wv[j] << 16) * f;
        acc[2 * j + 1] += __uint_as_float(wv[j] & 0xFFFF0000u) * f;
      }
    }
    M = Mb;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = f32_to_bf16(acc[2 * j] * inv) | ((uint32_t)f32_to_bf16(acc[2 * j + 1] * inv) << 16);
  *reinterpret_cast<uint4*>(out + ((int64_t)r * H + h) * kDv + 8 * t) = make_uint4(o[0], o[1], o[2], o[3]);
  if (lse && t == 0) lse[(int64_t)r * H + h] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// Any shape, fp32 or bf16: one workgroup per (row, head), logits staged in LDS.
template <bool BF16>
__global__ __launch_bounds__(256) void mla_generic_kernel(
    const void* __restrict__ qv, const void* __restrict__ kvv, const int32_t* __restrict__ table,
    int max_pages, int page_size, int64_t seq_stride, const int32_t* __restrict__ idx, int k, int H,
    int Dqk, int Dv, int decode, float scale, void* __restrict__ outv, float* __restrict__ lse) {
  extern __shared__ float sm[];  // [Dqk] query, [k] logits / weights, [8] reduction scratch
  float* sq = sm;
  float* sz = sm + Dqk;
  float* red = sz + k;
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  const int seq = decode ? r : 0;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  auto ld = [&](const void* p, int64_t i) -> float {
    return BF16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
  };
  auto row_of = [&](int id) -> int64_t {
    if (table) return (int64_t)table[(int64_t)seq * max_pages + id / page_size] * page_size + id % page_size;
    return (int64_t)seq * seq_stride + id;
  };
  for (int d = tid; d < Dqk; d += 256) sq[d] = ld(qv, ((int64_t)r * H + h) * Dqk + d);
  __syncthreads();
  float mx = -INFINITY;
  for (int j = tid; j < k; j += 256) {
    const int id = idx[(int64_t)r * k + j];
    float z = -INFINITY;
    if (id >= 0) {
      const int64_t row = row_of(id) * Dqk;
      float dot = 0.0f;
      for (int d = 0; d < Dqk; ++d) dot = fmaf(sq[d], ld(kvv, row + d), dot);
      z = dot * scale;
    }
    sz[j] = z;
    mx = fmaxf(mx, z);
  }
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.0f;
  for (int j = tid; j < k; j += 256) {
    const float pj = M == -INFINITY ? 0.0f : expf(sz[j] - M);
    sz[j] = pj;
    sum += pj;
  }
  sum = wave_sum(sum);
  if (lane == 0) red[w] = sum;
  __syncthreads();
  const float L = red[0] + red[1] + red[2] + red[3];
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  for (int d = tid; d < Dv; d += 256) {
    float o = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int id = idx[(int64_t)r * k + j];
      if (id >= 0) o = fmaf(sz[j], ld(kvv, row_of(id) * Dqk + d), o);
    }
    o *= inv;
    const int64_t oi = ((int64_t)r * H + h) * Dv + d;
    if (BF16) static_cast<uint16_t*>(outv)[oi] = f32_to_bf16(o);
    else static_cast<float*>(outv)[oi] = o;
  }
  if (lse && tid == 0) lse[(int64_t)r * H + h] = L > 0.0f ? M + logf(L) : -INFINITY;
}

// Dynamic LDS of the bf16 kernel: the row list and one live-token mask per tile.  The
// static part (ring, logit exchange) takes 124 KB of the 160 KB, which leaves room for the
// list of kMaxTokPerWg tokens.
size_t mla_lds_bytes(int tok_per_split) {
  return sizeof(int) * ((size_t)tok_per_split + (tok_per_split + kTok - 1) / kTok);
}

constexpr int kMaxTokPerWg = 8192;  // kept tokens one workgroup of the bf16 kernel can hold

struct SplitPlan {
  int n_split, tok_per_split;
};

SplitPlan split_plan(int B, int H, int k) {
  // One workgroup per CU (the LDS ring allows no second one): split each sequence's kept
  // set until ~256 workgroups exist, keeping at least 4 tiles (128 rows) per workgroup and
  // at most kMaxTokPerWg tokens (the row list sits in LDS beside the ring).
  const int groups = B * (H / kHeadsPerWg);
  int ns = (256 + groups - 1) / groups;
  const int max_ns = (k + 4 * kTok - 1) / (4 * kTok);
  ns = ns < 1 ? 1 : (ns > max_ns ? max_ns : ns);
  const int min_ns = (k + kMaxTokPerWg - 1) / kMaxTokPerWg;
  ns = ns < min_ns ? min_ns : ns;
  int tps = (k + ns - 1) / ns;
  tps = (tps + kTok - 1) / kTok * kTok;
  ns = (k + tps - 1) / tps;
  return {ns, tps};
}

hipError_t launch_combine(const uint16_t* part_o, const float* part_ml, int R, int H, int n_split,
                          uint16_t* out, float* lse, hipStream_t s) {
  const int RH = R * H;
  const unsigned cgrid = (unsigned)((RH + kCombinePairs - 1) / kCombinePairs);
  if (n_split <= 2)
    mla_combine_kernel<2><<<cgrid, 256, 0, s>>>(part_o, part_ml, RH, H, n_split, out, lse);
  else if (n_split <= 4)
    mla_combine_kernel<4><<<cgrid, 256, 0, s>>>(part_o, part_ml, RH, H, n_split, out, lse);
  else if (n_split <= 8)
    mla_combine_kernel<8><<<cgrid, 256, 0, s>>>(part_o, part_ml, RH, H, n_split, out, lse);
  else
    mla_combine_kernel<16><<<cgrid, 256, 0, s>>>(part_o, part_ml, RH, H, n_split, out, lse);
  return hipGetLastError();
}

// Decode dispatch.  The wide kernel (128 heads per workgroup) processes a tile with fewer,
// larger MFMAs but carries more fixed cost per workgroup (query fragments of 128 heads, 128
// KB of output or partials); it wins once the batch alone gives many (row, 128-head) groups,
// so every split holds many tiles.  Below that the 64-head kernel, whose workgroups start and
// finish faster, is quicker (measured at 8 x 131072 and 32 x 8192 against 64 x 20000).
constexpr int kWideMinGroups = 64;

bool decode_wide(int B, int H) { return H % 128 == 0 && B * (H / 128) >= kWideMinGroups; }

// Waves (32 heads each) per workgroup of the wide kernel.
int wide_nw(int H) { return H % 128 == 0 ? 4 : 2; }

SplitPlan split_plan_wide(int B, int H, int k) {
  // ~256 workgroups (one per CU: the ring leaves no LDS for a second), at least 4 tiles and
  // at most kMaxTokPerWg kept tokens per workgroup
  const int groups = B * (H / (32 * wide_nw(H)));
  int ns = (256 + groups - 1) / groups;
  const int max_ns = (k + 4 * kTok - 1) / (4 * kTok);
  ns = ns < 1 ? 1 : (ns > max_ns ? max_ns : ns);
  const int min_ns = (k + kMaxTokPerWg - 1) / kMaxTokPerWg;
  ns = ns < min_ns ? min_ns : ns;
  int tps = (k + ns - 1) / ns;
  tps = (tps + kTok - 1) / kTok * kTok;
  ns = (k + tps - 1) / tps;
  return {ns, tps};
}

SplitPlan decode_plan(int B, int H, int k) {
  return decode_wide(B, H) ? split_plan_wide(B, H, k) : split_plan(B, H, k);
}

template <int NW>
hipError_t launch_wide(const uint16_t* q, const CacheView& kv, const int32_t* idx, int R, int H,
                       int k, bool decode, bool masked, float scale_log2, uint16_t* out, float* lse,
                       uint16_t* part_o, float* part_ml, SplitPlan p, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)R * (H / (32 * NW)) * p.n_split);
  const uint16_t* kvp = static_cast<const uint16_t*>(kv.data);
  if (masked) {
    const size_t lds = sizeof(uint32_t) * (size_t)((R + kTok - 1) / kTok);
    mla_wide_kernel<NW, false, false, true><<<grid, NW * WAVE, lds, s>>>(
        q, kvp, nullptr, 0, 1, (int64_t)R, idx, k, H, 0, scale_log2, out, lse, nullptr, nullptr, 1, 0);
    return hipGetLastError();
  }
  const size_t lds = mla_lds_bytes(p.tok_per_split);
#define DSA_WIDE_LAUNCH(PG, SP)                                                                   \
  mla_wide_kernel<NW, PG, SP><<<grid, NW * WAVE, lds, s>>>(q, kvp, kv.table, kv.max_pages,          \
                                                           kv.page_size, kv.seq_stride, idx, k, H,   \
                                                           decode ? 1 : 0, scale_log2, out, lse,     \
                                                           part_o, part_ml, p.n_split, p.tok_per_split)
  if (kv.table) {
    if (p.n_split > 1) DSA_WIDE_LAUNCH(true, true); else DSA_WIDE_LAUNCH(true, false);
  } else {
    if (p.n_split > 1) DSA_WIDE_LAUNCH(false, true); else DSA_WIDE_LAUNCH(false, false);
  }
#undef DSA_WIDE_LAUNCH
  return hipGetLastError();
}

}  // namespace

int mla_max_tokens_per_wg() { return kMaxTokPerWg; }

size_t mla_decode_workspace_bytes(int B, int H, int Dv, int k) {
  if (Dv != kDv || H % kHeadsPerWg != 0) return 0;  // generic path needs no workspace
  const SplitPlan p = decode_plan(B, H, k);
  if (p.n_split <= 1) return 0;
  const size_t pairs = (size_t)B * p.n_split * H;
  return pairs * kDv * sizeof(uint16_t) + pairs * 2 * sizeof(float);
}

hipError_t launch_mla_bf16(const uint16_t* q, const CacheView& kv, const int32_t* idx, int R,
                           int H, int k, bool decode, float scale, uint16_t* out, float* lse,
                           void* ws, size_t ws_bytes, hipStream_t s) {
  if (!decode || decode_wide(R, H)) {
    const float scale_log2 = scale * 1.44269504088896340736f;
    SplitPlan p = decode ? split_plan_wide(R, H, k) : SplitPlan{1, k};
    if (p.n_split > 1 && ws_bytes < mla_decode_workspace_bytes(R, H, kDv, k)) return hipErrorInvalidValue;
    if (p.n_split <= 1) p = SplitPlan{1, k};
    uint16_t* part_o = static_cast<uint16_t*>(ws);
    float* part_ml = part_o ? reinterpret_cast<float*>(part_o + (size_t)R * p.n_split * H * kDv) : nullptr;
    hipError_t e = wide_nw(H) == 4
                       ? launch_wide<4>(q, kv, idx, R, H, k, decode, false, scale_log2, out, lse, part_o, part_ml, p, s)
                       : launch_wide<2>(q, kv, idx, R, H, k, decode, false, scale_log2, out, lse, part_o, part_ml, p, s);
    if (e != hipSuccess || p.n_split <= 1) return e;
    return launch_combine(part_o, part_ml, R, H, p.n_split, out, lse, s);
  }
  const float scale_log2 = scale * 1.44269504088896340736f;
  const uint16_t* kvp = static_cast<const uint16_t*>(kv.data);
  const int HG = H / kHeadsPerWg;
  SplitPlan p = decode ? split_plan(R, H, k) : SplitPlan{1, k};
  if (p.n_split > 1 && ws_bytes < mla_decode_workspace_bytes(R, H, kDv, k)) return hipErrorInvalidValue;
  if (p.n_split <= 1) p = SplitPlan{1, k};
  const unsigned grid = (unsigned)((int64_t)R * HG * p.n_split);
  uint16_t* part_o = static_cast<uint16_t*>(ws);
  float* part_ml = part_o ? reinterpret_cast<float*>(part_o + (size_t)R * p.n_split * H * kDv) : nullptr;
#define DSA_MLA_LAUNCH(PG, SP)                                                                   \
  mla_bf16_kernel<PG, SP><<<grid, kMlaThreads, mla_lds_bytes(p.tok_per_split), s>>>(q, kvp, kv.table, kv.max_pages,             \
                                                        kv.page_size, kv.seq_stride, idx, k, H,     \
                                                        decode ? 1 : 0, scale_log2, out, lse,       \
                                                        part_o, part_ml, p.n_split, p.tok_per_split)
  if (kv.table) {
    if (p.n_split > 1) DSA_MLA_LAUNCH(true, true); else DSA_MLA_LAUNCH(true, false);
  } else {
    if (p.n_split > 1) DSA_MLA_LAUNCH(false, true); else DSA_MLA_LAUNCH(false, false);
  }
#undef DSA_MLA_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split <= 1) return e;
  return launch_combine(part_o, part_ml, R, H, p.n_split, out, lse, s);
}

hipError_t launch_mla_bf16_masked(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int T,
                                  int H, int k, float scale, uint16_t* out, float* lse, hipStream_t s) {
  const float scale_log2 = scale * 1.44269504088896340736f;
  {
    const CacheView v{kv, nullptr, nullptr, 0, 0, (int64_t)T};
    return wide_nw(H) == 4
               ? launch_wide<4>(q, v, idx, T, H, k, false, true, scale_log2, out, lse, nullptr, nullptr, SplitPlan{1, k}, s)
               : launch_wide<2>(q, v, idx, T, H, k, false, true, scale_log2, out, lse, nullptr, nullptr, SplitPlan{1, k}, s);
  }
  const unsigned grid = (unsigned)((int64_t)T * (H / kHeadsPerWg));
  const size_t lds = sizeof(uint32_t) * (size_t)((T + kTok - 1) / kTok);  // one live mask per tile
  mla_bf16_kernel<false, false, true><<<grid, kMlaThreads, lds, s>>>(
      q, kv, nullptr, 0, 1, (int64_t)T, idx, k, H, 0, scale_log2, out, lse, nullptr, nullptr, 1, 0);
  return hipGetLastError();
}

hipError_t launch_mla_generic(bool bf16, const void* q, const CacheView& kv, const int32_t* idx,
                              int R, int H, int Dqk, int Dv, int k, bool decode, float scale,
                              void* out, float* lse, hipStream_t s) {
  const size_t lds = sizeof(float) * ((size_t)Dqk + k + 8);
  const unsigned grid = (unsigned)((int64_t)R * H);
  if (bf16)
    mla_generic_kernel<true><<<grid, 256, lds, s>>>(q, kv.data, kv.table, kv.max_pages, kv.page_size,
                                                    kv.seq_stride, idx, k, H, Dqk, Dv, decode ? 1 : 0,
                                                    scale, out, lse);
  else
    mla_generic_kernel<false><<<grid, 256, lds, s>>>(q, kv.data, kv.table, kv.max_pages, kv.page_size,
                                                     kv.seq_stride, idx, k, H, Dqk, Dv, decode ? 1 : 0,
                                                     scale, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
