// Indexer-quality diagnostic: how well the indexer's distribution imitates dense attention.
//
// In the pages the indexer learns by matching, under a KL loss, the distribution of the
// dense attention summed over heads (MarkTechPost, "DeepSeek V3.2-Exp Cuts Long-Context
// Costs with DeepSeek Sparse Attention (DSA) ...", "Training signal").  For each query row
// this computes, over its n candidates,
//   p[s]   = (1/H) sum_h softmax_s(scale * q_h . kv_s)          (dense, head-averaged)
//   KL     = sum_s p[s] * (ln p[s] - ln softmax_s(I[s]))          (nats; target first)
//   KL_rev = sum_s q[s] * (ln q[s] - ln p[s]), q = softmax(I)     (the other order; optional)
//   recall = sum_{s in kept set} p[s]
// Forward only: no gradients, nothing here is on the decode path.
//
// Four launches: logits (MFMA, each 32-row tile staged once in LDS for all head blocks)
// with each span's per-head softmax statistics, their merge per row (and the index scores'
// own statistics), per-chunk KL / recall partial sums, and the per-row totals.  Logits are
// kept in fp32 in the workspace (log2 domain).
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kQTile = 32;          // latent rows per LDS tile of the logits kernel
constexpr int kQSpan = 1024;        // tokens per logits workgroup (32 tiles)
constexpr int kQComputeWaves = 8;   // logits workgroup: eight compute waves + one copy wave
constexpr int kQThreads = (kQComputeWaves + 1) * WAVE;
constexpr int kQMaxDqk = 576;
constexpr int kQDmaPerTile = kQMaxDqk / 16;  // 1 KB LDS DMA blocks per tile (36)
constexpr int kQTileBytes = kQDmaPerTile * 1024;

typedef __attribute__((address_space(3))) void q_lds_void;
// LDS pointers are formed from the byte offset a flat pointer into LDS carries in its low
// 32 bits.
__device__ __forceinline__ uint32_t q_lds_offset(const void* p) { return (uint32_t)(uintptr_t)p; }
// s_waitcnt with only the vector-memory counter constrained (expcnt, lgkmcnt left at max).
template <int N>
__device__ __forceinline__ void q_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Three ring slots as separate LDS variables, so the compiler can tell a copy into one slot
// never aliases reads of another.
__shared__ __attribute__((aligned(16))) char g_qring0[kQTileBytes];
__shared__ __attribute__((aligned(16))) char g_qring1[kQTileBytes];
__shared__ __attribute__((aligned(16))) char g_qring2[kQTileBytes];
// Paged caches: the physical page of each logical page of the logits workgroup's span.
__shared__ int g_qpage[kQSpan];
template <int S>
__device__ __forceinline__ char* qring_slot() {
  return S == 0 ? g_qring0 : (S == 1 ? g_qring1 : g_qring2);
}
template <int S>
struct QSlot {
  static constexpr int value = S;
};
constexpr int kQSumChunk = 1024;    // tokens per partial-sum workgroup
constexpr int kQScoreChunk = 4096;  // index scores per statistics workgroup
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2f = 0.69314718055994530942f;

// z2[r, h, s] = scale * log2(e) * q[r, h, :] . kv[s, :] for the kQSpan tokens of this
// workgroup, plus each head's (max, sum of 2^(z2 - max)) over them.  Nine waves: a copy wave
// streams 32-row tiles of latent rows into a three-slot LDS ring with LDS DMA
// (global_load_lds_dwordx4, two tiles ahead) and eight compute waves read them; wave w < H/16
// takes heads 16w .. 16w+15 (S^T tiles of 16 tokens x 16 heads, v_mfma_f32_16x16x32_bf16,
// A = rows from LDS, B = the heads' query held in registers).  Tile layout: DMA j writes
// 1 KB block j -- 16-byte piece j of rows 0..31 (lanes 0..31), then piece j + 36 (lanes
// 32..63) -- so a 16-lane MFMA fragment read is 256 contiguous bytes, the four lane groups
// sit 1 KB apart (no bank conflicts), and every fragment is a lane base plus a constant.
// Rows narrower than 576 columns copy their last piece into the unused places.
__device__ __forceinline__ constexpr int qtile_off(int pc) {
  return pc < kQDmaPerTile ? pc * 1024 : (pc - kQDmaPerTile) * 1024 + 512;
}

__global__ __launch_bounds__(kQThreads) void quality_logits_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ table,
    int page_size, int max_pages, int64_t seq_stride, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int H, int Dqk, int n_spans, float scale_log2,
    float* __restrict__ z2, int64_t ld, float2* __restrict__ span_stats) {
  const int r = blockIdx.x / n_spans;
  const int span = blockIdx.x % n_spans;
  const int64_t n = (int64_t)row_pos[r] + 1;
  const int64_t sp0 = (int64_t)span * kQSpan;
  if (sp0 >= n) return;
  const int nt = (int)((min(n - sp0, (int64_t)kQSpan) + kQTile - 1) / kQTile);
  const int seq = row_seq[r];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int pieces = Dqk / 8;  // 16-byte pieces per row

  if (w == kQComputeWaves) {
    // ---------------------------------------------------------------- copy wave
    const int pbase = kQDmaPerTile * (lane >> 5);  // lanes 32..63: the row's pieces 36..71
    // Paged: this span's slice of the block table goes to LDS first, so resolving a row never
    // waits on a global load issued behind DMA in flight.
    int64_t p_first = 0;
    if (table) {
      p_first = sp0 / page_size;
      const int np = (int)((min(n, sp0 + kQSpan) - 1) / page_size - p_first + 1);
      for (int i = lane; i < np; i += WAVE) g_qpage[i] = table[(int64_t)seq * max_pages + p_first + i];
    }
    auto issue = [&](int t, char* dst) {
      const int64_t s = min(sp0 + (int64_t)t * kQTile + (lane & 31), n - 1);
      const int64_t row = table ? (int64_t)g_qpage[s / page_size - p_first] * page_size + s % page_size
                                : (int64_t)seq * seq_stride + s;
      const uint16_t* src = kv + row * Dqk;
#pragma unroll
      for (int j = 0; j < kQDmaPerTile; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(src + 8 * min(pbase + j, pieces - 1)),
                                         (q_lds_void*)(uintptr_t)(q_lds_offset(dst) + j * 1024), 16, 0, 0);
    };
    issue(0, g_qring0);
    if (nt > 1) issue(1, g_qring1);
    auto hand = [&](auto slot, int t) {
      constexpr int S = decltype(slot)::value;
      if (t + 1 < nt) q_wait_vmcnt<kQDmaPerTile>();  // tile t landed, t+1 may be in flight
      else q_wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();  // hand tile t to the compute waves
      if (t + 2 < nt) issue(t + 2, qring_slot<(S + 2) % 3>());
    };
    for (int t = 0; t < nt; t += 3) {
      hand(QSlot<0>{}, t);
      if (t + 1 < nt) hand(QSlot<1>{}, t + 1);
      if (t + 2 < nt) hand(QSlot<2>{}, t + 2);
    }
    return;
  }

  // ------------------------------------------------------------------ compute waves
  const bool computes = w < H / 16;
  const int col = lane & 15, grp = lane >> 4;
  // Query fragments: B[k = dim][n = head col] = q[r, 16w + col, 32*kk + 8*grp + j].
  const int nk = Dqk / 32;
  v8bf qf[kQMaxDqk / 32];
  if (computes) {
    const uint16_t* qrow = q + ((int64_t)r * H + 16 * w + col) * Dqk + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < kQMaxDqk / 32; ++kk)
      if (kk < nk) qf[kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(qrow + 32 * kk));
  }
  float* zr = z2 + ((int64_t)r * H + 16 * w + col) * ld;
  float m_run = -INFINITY, l_run = 0.0f;  // this lane's tokens of head 16w + col
  const bool vec_store = (ld & 3) == 0;

  auto step = [&](auto slot, int t) {
    constexpr int S = decltype(slot)::value;
    __builtin_amdgcn_s_barrier();  // tile t is in ring slot S
    if (!computes) return;
    const char* tb_base = qring_slot<S>() + grp * 1024 + col * 16;
    const int64_t s0 = sp0 + (int64_t)t * kQTile;
    v4f acc[kQTile / 16];
#pragma unroll
    for (int tb = 0; tb < kQTile / 16; ++tb) {
      acc[tb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kQMaxDqk / 32; ++kk)
        if (kk < nk)
          acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *reinterpret_cast<const v8bf*>(tb_base + qtile_off(4 * kk) + 256 * tb), qf[kk],
              acc[tb], 0, 0, 0);
    }
    // lane holds tokens s0 + 16*tb + 4*grp + i of head 16w + col
    float cm = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < kQTile / 16; ++tb) {
      const int64_t s = s0 + 16 * tb + 4 * grp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[tb][i] *= scale_log2;
        if (s + i < n) cm = fmaxf(cm, acc[tb][i]);
      }
      if (vec_store && s + 3 < n) {
        *reinterpret_cast<float4*>(zr + s) = make_float4(acc[tb][0], acc[tb][1], acc[tb][2], acc[tb][3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (s + i < n) zr[s + i] = acc[tb][i];
      }
    }
    if (cm > -INFINITY) {
      const float nm = fmaxf(m_run, cm);
      float acc_l = l_run > 0.0f ? l_run * exp2f(m_run - nm) : 0.0f;
#pragma unroll
      for (int tb = 0; tb < kQTile / 16; ++tb) {
        const int64_t s = s0 + 16 * tb + 4 * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (s + i < n) acc_l += exp2f(acc[tb][i] - nm);
      }
      m_run = nm;
      l_run = acc_l;
    }
  };
  for (int t = 0; t < nt; t += 3) {
    step(QSlot<0>{}, t);
    if (t + 1 < nt) step(QSlot<1>{}, t + 1);
    if (t + 2 < nt) step(QSlot<2>{}, t + 2);
  }
  if (!computes) return;
  // Merge the four lanes (grp = 0..3) that hold head col's tokens.
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    const float m2 = __shfl_xor(m_run, off), l2 = __shfl_xor(l_run, off);
    const float mm = fmaxf(m_run, m2);
    l_run = (l_run > 0.0f ? l_run * exp2f(m_run - mm) : 0.0f) + (l2 > 0.0f ? l2 * exp2f(m2 - mm) : 0.0f);
    m_run = mm;
  }
  if (grp == 0) span_stats[((int64_t)r * H + 16 * w + col) * n_spans + span] = make_float2(m_run, l_run);
}

// Online merge of (max, sum of 2^(x - max)) pairs.
__device__ __forceinline__ void merge_ml(float& m1, float& l1, float m2, float l2) {
  const float mm = fmaxf(m1, m2);
  l1 = (l1 > 0.0f ? l1 * exp2f(m1 - mm) : 0.0f) + (l2 > 0.0f ? l2 * exp2f(m2 - mm) : 0.0f);
  m1 = mm;
}

// Block-wide merge of every thread's (m, l); the result is valid in thread 0.
__device__ __forceinline__ void block_merge_ml(float& m, float& l, float* sm, float* sl) {
  sm[threadIdx.x] = m;
  sl[threadIdx.x] = l;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      float m1 = sm[threadIdx.x], l1 = sl[threadIdx.x];
      merge_ml(m1, l1, sm[threadIdx.x + o], sl[threadIdx.x + o]);
      sm[threadIdx.x] = m1;
      sl[threadIdx.x] = l1;
    }
    __syncthreads();
  }
  m = sm[0];
  l = sl[0];
}

// Workgroup (r, j): j < H merges head j's span statistics over all n tokens of row r into
// stats[r, j]; j >= H takes chunk c = j - H of the row's index scores (scaled to log2) and
// writes its (max, sum) to score_stats[r, c].
__global__ __launch_bounds__(256) void quality_stats_kernel(const float2* __restrict__ span_stats,
                                                            int n_spans, const float* __restrict__ scores,
                                                            int64_t sld, const int32_t* __restrict__ row_pos,
                                                            int H, int n_sc, float2* __restrict__ stats,
                                                            float2* __restrict__ score_stats) {
  __shared__ float sm[256], sl[256];
  const int r = blockIdx.x / (H + n_sc), j = blockIdx.x % (H + n_sc);
  const int64_t n = (int64_t)row_pos[r] + 1;
  float m = -INFINITY, l = 0.0f;
  if (j < H) {
    const int used = (int)((n + kQSpan - 1) / kQSpan);
    const float2* st = span_stats + ((int64_t)r * H + j) * n_spans;
    for (int i = threadIdx.x; i < used; i += 256) merge_ml(m, l, st[i].x, st[i].y);
  } else {
    const int64_t c0 = (int64_t)(j - H) * kQScoreChunk;
    const float* x = scores + (int64_t)r * sld;
    float v[kQScoreChunk / 256];
#pragma unroll
    for (int u = 0; u < kQScoreChunk / 256; ++u) {
      const int64_t s = c0 + 256 * u + threadIdx.x;
      v[u] = s < n ? x[s] * kLog2e : -INFINITY;
      m = fmaxf(m, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kQScoreChunk / 256; ++u) l += v[u] == -INFINITY ? 0.0f : exp2f(v[u] - m);
  }
  block_merge_ml(m, l, sm, sl);
  if (threadIdx.x == 0) {
    if (j < H) stats[(int64_t)r * H + j] = make_float2(m, l);
    else score_stats[(int64_t)r * n_sc + (j - H)] = make_float2(m, l);
  }
}

// Partial sums over one chunk of tokens: KL terms p (ln p - ln q) and q (ln q - ln p), and the
// kept set's mass.
__global__ __launch_bounds__(256) void quality_partial_kernel(
    const float* __restrict__ z2, const float* __restrict__ scores, int64_t sld,
    const int32_t* __restrict__ idx, int k, const int32_t* __restrict__ row_pos, int H, int64_t ld,
    const float2* __restrict__ stats, const float2* __restrict__ score_stats, int n_sc, int n_chunks,
    float4* __restrict__ partial) {
  __shared__ uint32_t kept[kQSumChunk / 32];
  __shared__ float2 hst[129];  // per head: (max, 1 / sum); then the index scores' (max, sum)
  __shared__ float red_kl[256], red_rc[256], red_kr[256];
  const int r = blockIdx.x / n_chunks;
  const int64_t c0 = (int64_t)(blockIdx.x % n_chunks) * kQSumChunk;
  const int64_t n = (int64_t)row_pos[r] + 1;
  float kl = 0.0f, rc = 0.0f, kr = 0.0f;
  if (c0 < n) {
    for (int i = threadIdx.x; i < kQSumChunk / 32; i += 256) kept[i] = 0u;
    for (int h = threadIdx.x; h < H; h += 256) {
      const float2 v = stats[(int64_t)r * H + h];
      hst[h] = make_float2(v.x, 1.0f / v.y);
    }
    {  // the index scores' (max, sum) from their chunks
      float m = -INFINITY, l = 0.0f;
      for (int c = threadIdx.x; c < n_sc; c += 256) {
        const float2 v = score_stats[(int64_t)r * n_sc + c];
        merge_ml(m, l, v.x, v.y);
      }
      block_merge_ml(m, l, red_kl, red_rc);
      if (threadIdx.x == 0) hst[H] = make_float2(m, l);
    }
    __syncthreads();
    for (int j = threadIdx.x; j < k; j += 256) {
      const int64_t s = idx[(int64_t)r * k + j];
      if (s >= c0 && s < c0 + kQSumChunk && s < n) atomicOr(&kept[(s - c0) >> 5], 1u << ((s - c0) & 31));
    }
    __syncthreads();
    const float2 si = hst[H];
    const float ln_li = logf(si.y);
    const float* zr = z2 + (int64_t)r * H * ld;
    for (int64_t s = c0 + threadIdx.x; s < min(c0 + kQSumChunk, n); s += 256) {
      // 16 heads' logits in flight at a time (the head loop would otherwise wait on each load)
      float p = 0.0f;
      for (int h0 = 0; h0 < H; h0 += 16) {
        float zv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) zv[u] = zr[(int64_t)(h0 + u) * ld + s];
#pragma unroll
        for (int u = 0; u < 16; ++u) p += exp2f(zv[u] - hst[h0 + u].x) * hst[h0 + u].y;
      }
      p *= 1.0f / (float)H;
      const float log_q = (scores[(int64_t)r * sld + s] * kLog2e - si.x) * kLn2f - ln_li;
      const float q = expf(log_q);
      if (p > 0.0f) {
        const float ln_p = logf(p);
        kl += p * (ln_p - log_q);
        kr += q * (log_q - ln_p);
      } else if (q > 0.0f) {
        kr = INFINITY;  // the dense target has a zero the indexer does not
      }
      if ((kept[(s - c0) >> 5] >> ((s - c0) & 31)) & 1u) rc += p;
    }
  }
  red_kl[threadIdx.x] = kl;
  red_rc[threadIdx.x] = rc;
  red_kr[threadIdx.x] = kr;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      red_kl[threadIdx.x] += red_kl[threadIdx.x + o];
      red_rc[threadIdx.x] += red_rc[threadIdx.x + o];
      red_kr[threadIdx.x] += red_kr[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = make_float4(red_kl[0], red_rc[0], red_kr[0], 0.0f);
}

__global__ __launch_bounds__(256) void quality_finish_kernel(const float4* __restrict__ partial,
                                                             int n_chunks, float* __restrict__ kl,
                                                             float* __restrict__ recall,
                                                             float* __restrict__ kl_rev) {
  __shared__ float a[256], b[256], c3[256];
  const int r = blockIdx.x;
  float x = 0.0f, y = 0.0f, z = 0.0f;
  for (int c = threadIdx.x; c < n_chunks; c += 256) {
    const float4 v = partial[(int64_t)r * n_chunks + c];
    x += v.x;
    y += v.y;
    z += v.z;
  }
  a[threadIdx.x] = x;
  b[threadIdx.x] = y;
  c3[threadIdx.x] = z;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      a[threadIdx.x] += a[threadIdx.x + o];
      b[threadIdx.x] += b[threadIdx.x + o];
      c3[threadIdx.x] += c3[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    kl[r] = a[0];
    recall[r] = b[0];
    if (kl_rev) kl_rev[r] = c3[0];
  }
}

struct QualityWs {
  size_t z2, span_stats, stats, score_stats, partial, total;
};
QualityWs quality_ws(int R, int H, int64_t ld) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  QualityWs L{};
  L.z2 = 0;
  L.span_stats = up(sizeof(float) * (size_t)R * H * (size_t)ld);
  L.stats = L.span_stats + up(sizeof(float2) * (size_t)R * H * (size_t)((ld + kQSpan - 1) / kQSpan));
  L.score_stats = L.stats + up(sizeof(float2) * (size_t)R * H);
  L.partial = L.score_stats + up(sizeof(float2) * (size_t)R * (size_t)((ld + kQScoreChunk - 1) / kQScoreChunk));
  L.total = L.partial + up(sizeof(float4) * (size_t)R * (size_t)((ld + kQSumChunk - 1) / kQSumChunk));
  return L;
}

}  // namespace

size_t quality_workspace_bytes(int R, int H, int64_t ld) { return quality_ws(R, H, ld).total; }

hipError_t launch_indexer_quality(const uint16_t* q, const CacheView& kv, const float* scores,
                                  int64_t sld, const int32_t* idx, int k, const int32_t* row_seq,
                                  const int32_t* row_pos, int R, int H, int Dqk, int64_t ld,
                                  float scale, float* kl, float* recall, float* kl_rev, void* ws,
                                  hipStream_t s) {
  const QualityWs L = quality_ws(R, H, ld);
  char* b = static_cast<char*>(ws);
  float* z2 = reinterpret_cast<float*>(b + L.z2);
  float2* span_stats = reinterpret_cast<float2*>(b + L.span_stats);
  float2* stats = reinterpret_cast<float2*>(b + L.stats);
  float2* score_stats = reinterpret_cast<float2*>(b + L.score_stats);
  float4* partial = reinterpret_cast<float4*>(b + L.partial);
  const int nsp = (int)((ld + kQSpan - 1) / kQSpan);
  quality_logits_kernel<<<(unsigned)R * (unsigned)nsp, kQThreads, 0, s>>>(
      q, static_cast<const uint16_t*>(kv.data), kv.table, kv.page_size, kv.max_pages, kv.seq_stride,
      row_seq, row_pos, H, Dqk, nsp, scale * kLog2e, z2, ld, span_stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nsc = (int)((ld + kQScoreChunk - 1) / kQScoreChunk);
  quality_stats_kernel<<<(unsigned)R * (unsigned)(H + nsc), 256, 0, s>>>(span_stats, nsp, scores, sld, row_pos,
                                                                        H, nsc, stats, score_stats);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int ns = (int)((ld + kQSumChunk - 1) / kQSumChunk);
  quality_partial_kernel<<<(unsigned)R * (unsigned)ns, 256, 0, s>>>(z2, scores, sld, idx, k, row_pos, H, ld,
                                                                   stats, score_stats, nsc, ns, partial);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  quality_finish_kernel<<<R, 256, 0, s>>>(partial, ns, kl, recall, kl_rev);
  return hipGetLastError();
}

}  // namespace dsa
