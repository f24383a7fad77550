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
// bf16 fast path (Dqk = 576, Dv = 512, 64 heads per workgroup, 4 waves x 16 heads):
//   * 32 selected rows are gathered into LDS once per tile and used by all 64 heads;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = K rows from LDS (ds_read_b128),
//     B = the wave's 16 query heads held in registers for the whole kernel;
//     the result layout puts one head per lane column, so the online-softmax row
//     statistics of a head live in one lane column and need two cross-lane steps;
//   * O^T += V^T P^T: A = V^T fragments read from the row-major LDS tile with the gfx950
//     transposing LDS load (ds_read_b64_tr_b16), B = P^T straight from the S^T
//     registers (the token order inside the 32-wide K step is permuted identically on
//     both operands, so no data moves between lanes);
//   * decode splits each sequence's kept set over several workgroups and merges the
//     partial (o, max, sum) triples with a log-sum-exp combine kernel.
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kTok = 32;                        // rows per LDS tile
constexpr int kRowChunks = kDqk * 2 / 16;       // 72 16-byte chunks per latent row
constexpr int kDmaPerTile = kRowChunks / 2;     // 36 wave-wide 1 KB copies per tile
// Tile layout (chunk-major): copy j fills block j with chunk j of rows 0..31 (lanes 0-31)
// and chunk j + 36 (lanes 32-63), 16 bytes per lane.  Blocks are 1088 bytes apart so
// chunks 2d and 2d+1 (one 16-column value slice) sit 16 banks apart for the transposing
// reads; a 16-lane read of one chunk covers 256 contiguous bytes (all 64 banks).
constexpr int kBlock = 1024 + 64;
constexpr int kBufBytes = kDmaPerTile * kBlock;  // 39168
constexpr int kNBuf = 3;                        // ring depth: two tiles in flight during compute
constexpr int kMlaWaves = 4;                    // compute waves, 16 heads each
constexpr int kMlaThreads = (kMlaWaves + 1) * WAVE;          // + one loader wave
constexpr int kHeadsPerWg = 16 * kMlaWaves;
constexpr float kLn2 = 0.69314718055994530942f;

// Byte offset of (row, 16-byte chunk c) inside a tile.
__device__ __forceinline__ int tile_off(int row, int c) {
  return (c < kDmaPerTile ? c * kBlock : (c - kDmaPerTile) * kBlock + 512) + row * 16;
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ v4bf lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(p));
}

// s_waitcnt with only the vector-memory counter constrained (expcnt, lgkmcnt left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__shared__ __attribute__((aligned(16))) char g_ring[kNBuf][kBufBytes];

// One workgroup = (row r, 64 heads, a range of the kept set).  Wave 4 is the loader: it
// streams each 32-row tile straight from global memory into a 3-deep LDS ring with
// global_load_lds_dwordx4 (a row is gathered once and shared by all 64 heads) and never
// reads the ring, so its copies stay in flight across the tile barriers; waves 0-3
// compute.  The loader's only LDS reads are the row list `srow`, a different LDS array,
// which keeps the compiler from waiting on the copies before them.
template <bool PAGED, bool SPLIT>
__global__ __launch_bounds__(kMlaThreads) void mla_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ table, int max_pages, int page_size, int64_t seq_stride,
    const int32_t* __restrict__ idx, int k, int H, int decode, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml, int n_split, int tok_per_split) {
  extern __shared__ int srow[];  // [tok_per_split] cache row of each kept token, -1 = none

  const int HG = H / kHeadsPerWg;
  int bid = blockIdx.x;
  const int sp = bid % n_split;
  bid /= n_split;
  const int hg = bid % HG;
  const int r = bid / HG;
  const int t_begin = sp * tok_per_split;
  const int t_end = min(k, t_begin + tok_per_split);
  const int n_tok = t_end > t_begin ? t_end - t_begin : 0;
  const int seq = decode ? r : 0;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int32_t* irow = idx + (int64_t)r * k + t_begin;
  // Rows are addressed relative to `base`: the sequence's first row (contiguous) or the
  // pool (paged: the page table is resolved here, once per kept token).
  const uint16_t* base = PAGED ? kv : kv + (int64_t)seq * seq_stride * kDqk;
  // Query fragments of the compute waves, issued before the row list is built so the two
  // latencies overlap: B[k = dim][n = head col] = q[r, h, 32*kk + 8*grp + j].
  const int col = lane & 15, grp = lane >> 4;
  const int h = hg * kHeadsPerWg + 16 * min(w, kMlaWaves - 1) + col;
  const uint16_t* qrow = q + ((int64_t)r * H + h) * kDqk;
  v8bf qf[kDqk / 32];
  if (w < kMlaWaves) {
    const uint4* qp = reinterpret_cast<const uint4*>(qrow + 8 * grp);
#pragma unroll
    for (int kk = 0; kk < kDqk / 32; ++kk) {
      const uint4 x = qp[4 * kk];
      qf[kk] = __builtin_bit_cast(v8bf, x);
    }
  }
  {
    constexpr int U = 8;  // ids (and their page-table entries) read in batches
    for (int i0 = 0; i0 < n_tok; i0 += U * kMlaThreads) {
      int id[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * kMlaThreads + tid;
        const int v = irow[min(i, n_tok - 1)];  // unconditional load: no wait between batch members
        id[u] = i < n_tok ? v : -1;
      }
      if (PAGED) {
        int pg[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          pg[u] = table[(int64_t)seq * max_pages + (id[u] >= 0 ? id[u] : 0) / page_size];
#pragma unroll
        for (int u = 0; u < U; ++u) id[u] = id[u] >= 0 ? pg[u] * page_size + id[u] % page_size : -1;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * kMlaThreads + tid;
        if (i < n_tok) srow[i] = id[u] >= 0 ? id[u] : -1;
      }
    }
  }
  __syncthreads();
  const int ntiles = (n_tok + kTok - 1) / kTok;

  if (w == kMlaWaves) {
    // ---------------------------------------------------------------- loader wave
    // Dead rows (past the range or index -1) copy this row's first query row, which is
    // finite, so masked tokens never inject NaN into the value products.
    const uint16_t* dummy = q + (int64_t)r * H * kDqk;
    const int half = lane >> 5;  // lanes 32-63 copy the row's second half (chunks 36..71)
    auto issue = [&](int t) {
      char* dst = g_ring[t % kNBuf];
      const int tok = t * kTok + (lane & 31);
      const int row = tok < n_tok ? srow[tok] : -1;
      const uint16_t* src = (row >= 0 ? base + (int64_t)row * kDqk : dummy) + half * (kDqk / 2);
#pragma unroll
      for (int j = 0; j < kDmaPerTile; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(src + 8 * j), (lds_void*)(dst + j * kBlock), 16, 0, 0);
    };
    if (ntiles > 0) issue(0);
    if (ntiles > 1) issue(1);
    for (int t = 0; t < ntiles; ++t) {
      if (t + 1 < ntiles) wait_vmcnt<kDmaPerTile>();  // tile t landed, t+1 may be in flight
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();                    // hand tile t to the compute waves
      if (t + 2 < ntiles) issue(t + 2);                // its buffer was freed by tile t-1
    }
    return;
  }

  // ------------------------------------------------------------------ compute waves
  v4f acc_o[kDv / 16];
#pragma unroll
  for (int dt = 0; dt < kDv / 16; ++dt) acc_o[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // reference max of scaled logits (log2 domain), per head = col
  float l_run = 0.0f;       // this lane's share of the running sum

  for (int t = 0; t < ntiles; ++t) {
    __builtin_amdgcn_s_barrier();  // tile t is in g_ring[t % kNBuf]
    const char* tb = g_ring[t % kNBuf];
    // ---- S^T = K Q^T for tokens 0..15 (st = 0) and 16..31 (st = 1)
    v4f acc_s[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < kDqk / 32; ++kk) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const v8bf a = *reinterpret_cast<const v8bf*>(tb + tile_off(16 * st + col, 4 * kk + grp));
        acc_s[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk], acc_s[st], 0, 0, 0);
      }
    }
    // ---- online softmax (lane holds tokens 16*st + 4*grp + i of head col)
    float s[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t * kTok + 16 * st + 4 * grp + i;
        const bool ok = tok < n_tok && srow[tok] >= 0;
        s[st][i] = ok ? acc_s[st][i] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[st][i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescaling: the reference max only moves when a logit exceeds it by more than
    // 2^8 (or on the first valid tile), so p <= 256 and the accumulators rarely rescale.
    float m_ref = m_run;
    if (__ballot(mx > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_run == -INFINITY ? 0.0f : exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDv / 16; ++dt) acc_o[dt] *= alpha;
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
        p[st][i] = exp2f(s[st][i] - m_use);
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
    // ---- O^T += V^T P^T, 32 tiles of 16 value columns
    // lane (col, grp) of a transposing read supplies row 4*grp + col/4 (+16), value columns
    // 16*dt + 4*(col&3) .. +3: chunk 2*dt + (col&3)/2, byte 8*(col&1) within it.
    const int vrow = 4 * grp + (col >> 2);
    const int vsub = 8 * (col & 1);
#pragma unroll
    for (int dt = 0; dt < kDv / 16; ++dt) {
      const int c = 2 * dt + ((col & 3) >> 1);
      const v4bf lo = lds_read_tr16(tb + tile_off(vrow, c) + vsub);
      const v4bf hi = lds_read_tr16(tb + tile_off(vrow + 16, c) + vsub);
      const v8bf a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, acc_o[dt], 0, 0, 0);
    }
  }

  float l = l_run + __shfl_xor(l_run, 16);
  l += __shfl_xor(l, 32);
  if (SPLIT) {
    const int64_t pr = ((int64_t)r * n_split + sp) * H + h;
    float* po = part_o + pr * kDv + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < kDv / 16; ++dt)
      *reinterpret_cast<float4*>(po + 16 * dt) = make_float4(acc_o[dt][0], acc_o[dt][1], acc_o[dt][2], acc_o[dt][3]);
    if (grp == 0) {
      part_ml[2 * pr] = m_run;
      part_ml[2 * pr + 1] = l;
    }
  } else {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* op = out + ((int64_t)r * H + h) * kDv + 4 * grp;
#pragma unroll
    for (int dt = 0; dt < kDv / 16; ++dt) {
      const uint32_t lo = f32_to_bf16(acc_o[dt][0] * inv) | ((uint32_t)f32_to_bf16(acc_o[dt][1] * inv) << 16);
      const uint32_t hi = f32_to_bf16(acc_o[dt][2] * inv) | ((uint32_t)f32_to_bf16(acc_o[dt][3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + 16 * dt) = make_uint2(lo, hi);
    }
    if (lse && grp == 0) lse[(int64_t)r * H + h] = l > 0.0f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
  }
}

// Log-sum-exp merge of the split partials: 128 threads per (row, head), 4 value columns
// per thread.  Splits are taken 16 at a time with every load of a batch (values and the
// (max, sum) pairs alike) issued before any is used, so a typical merge is one round trip;
// batches after the first rescale the running sums to the new maximum.
constexpr int kCombineBatch = 16;
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int RH, int H, int n_split,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int pair = blockIdx.x * 2 + threadIdx.x / 128;
  if (pair >= RH) return;
  const int r = pair / H, h = pair % H;
  const int t = threadIdx.x & 127;
  const int64_t p0 = (int64_t)r * n_split * H + h;  // partial of split s at p0 + s * H
  float M = -INFINITY, L = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = 0; s0 < n_split; s0 += kCombineBatch) {
    float2 ml[kCombineBatch];
    float4 v[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int64_t pr = p0 + (int64_t)min(s0 + u, n_split - 1) * H;
      ml[u] = *reinterpret_cast<const float2*>(part_ml + 2 * pr);
      v[u] = *reinterpret_cast<const float4*>(part_o + pr * kDv + 4 * t);
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      if (s0 + u < n_split && ml[u].y > 0.0f) Mb = fmaxf(Mb, ml[u].x);
    const float c = M == -INFINITY ? 0.0f : exp2f(M - Mb);
    L *= c;
    acc.x *= c; acc.y *= c; acc.z *= c; acc.w *= c;
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const bool valid = s0 + u < n_split && ml[u].y > 0.0f;
      const float f = valid ? exp2f(ml[u].x - Mb) : 0.0f;
      L += valid ? ml[u].y * f : 0.0f;
      acc.x += v[u].x * f; acc.y += v[u].y * f; acc.z += v[u].z * f; acc.w += v[u].w * f;
    }
    M = Mb;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const uint32_t lo = f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16);
  const uint32_t hi = f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16);
  *reinterpret_cast<uint2*>(out + ((int64_t)r * H + h) * kDv + 4 * t) = make_uint2(lo, hi);
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

struct SplitPlan {
  int n_split, tok_per_split;
};

SplitPlan split_plan(int B, int H, int k) {
  // One workgroup per CU (the LDS ring allows no second one): split each sequence's kept
  // set until ~256 workgroups exist, keeping at least 4 tiles (128 rows) per workgroup.
  const int groups = B * (H / kHeadsPerWg);
  int ns = (256 + groups - 1) / groups;
  const int max_ns = (k + 4 * kTok - 1) / (4 * kTok);
  ns = ns < 1 ? 1 : (ns > max_ns ? max_ns : ns);
  int tps = (k + ns - 1) / ns;
  tps = (tps + kTok - 1) / kTok * kTok;
  ns = (k + tps - 1) / tps;
  return {ns, tps};
}

}  // namespace

size_t mla_decode_workspace_bytes(int B, int H, int Dv, int k) {
  if (Dv != kDv || H % kHeadsPerWg != 0) return 0;  // generic path needs no workspace
  const SplitPlan p = split_plan(B, H, k);
  if (p.n_split <= 1) return 0;
  const size_t pairs = (size_t)B * p.n_split * H;
  return pairs * kDv * sizeof(float) + pairs * 2 * sizeof(float);
}

hipError_t launch_mla_bf16(const uint16_t* q, const CacheView& kv, const int32_t* idx, int R,
                           int H, int k, bool decode, float scale, uint16_t* out, float* lse,
                           void* ws, size_t ws_bytes, hipStream_t s) {
  const float scale_log2 = scale * 1.44269504088896340736f;
  const uint16_t* kvp = static_cast<const uint16_t*>(kv.data);
  const int HG = H / kHeadsPerWg;
  SplitPlan p = decode ? split_plan(R, H, k) : SplitPlan{1, k};
  if (p.n_split > 1 && ws_bytes < mla_decode_workspace_bytes(R, H, kDv, k)) return hipErrorInvalidValue;
  if (p.n_split <= 1) p = SplitPlan{1, k};
  const unsigned grid = (unsigned)((int64_t)R * HG * p.n_split);
  float* part_o = static_cast<float*>(ws);
  float* part_ml = part_o ? part_o + (size_t)R * p.n_split * H * kDv : nullptr;
#define DSA_MLA_LAUNCH(PG, SP)                                                                   \
  mla_bf16_kernel<PG, SP><<<grid, kMlaThreads, sizeof(int) * p.tok_per_split, s>>>(q, kvp, kv.table, kv.max_pages,             \
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
  const int RH = R * H;
  mla_combine_kernel<<<(RH + 1) / 2, 256, 0, s>>>(part_o, part_ml, RH, H, p.n_split, out, lse);
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
