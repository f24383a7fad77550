// Indexer-quality diagnostic: how well the indexer's distribution imitates dense attention.
//
// The pages say the indexer is trained to imitate the dense model's head-summed attention
// distribution through a KL divergence (MarkTechPost, "DeepSeek V3.2-Exp Cuts Long-Context
// Costs with DeepSeek Sparse Attention (DSA) ...", "Training signal").  For each query row
// this computes, over its n candidates,
//   p[s]   = (1/H) sum_h softmax_s(scale * q_h . kv_s)          (dense, head-averaged)
//   KL     = sum_s p[s] * (ln p[s] - ln softmax_s(I[s]))          (nats; target first)
//   recall = sum_{s in kept set} p[s]
// Forward only: no gradients, nothing here is on the decode path.
//
// Four launches: logits (MFMA, the 64-row chunk staged once in LDS for all head blocks),
// per-head and per-row softmax statistics, per-chunk KL / recall partial sums, and the
// per-row totals.  Logits are kept in fp32 in the workspace (log2 domain).
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kQChunk = 64;         // tokens per logits workgroup
constexpr int kQRowStride = 1168;   // LDS bytes per staged row (1152 + 16: conflict-free reads)
constexpr int kQMaxDqk = 576;
constexpr int kQSumChunk = 1024;    // tokens per partial-sum workgroup
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2f = 0.69314718055994530942f;

__device__ __forceinline__ int64_t kv_row(const int32_t* table, int page_size, int max_pages,
                                          int64_t seq_stride, int seq, int64_t s) {
  if (table) return (int64_t)table[(int64_t)seq * max_pages + s / page_size] * page_size + s % page_size;
  return (int64_t)seq * seq_stride + s;
}

// z2[r, h, s] = scale * log2(e) * q[r, h, :] . kv[s, :] for s in this workgroup's chunk.
// Wave w takes heads 16w .. 16w+15: S^T tiles (16 tokens x 16 heads) with
// v_mfma_f32_16x16x32_bf16, A = rows from LDS, B = the heads' query held in registers.
__global__ __launch_bounds__(512) void quality_logits_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ table,
    int page_size, int max_pages, int64_t seq_stride, const int32_t* __restrict__ row_seq,
    const int32_t* __restrict__ row_pos, int H, int Dqk, int n_chunks, float scale_log2,
    float* __restrict__ z2, int64_t ld) {
  __shared__ __attribute__((aligned(16))) char rows[kQChunk * kQRowStride];
  const int r = blockIdx.x / n_chunks;
  const int64_t s0 = (int64_t)(blockIdx.x % n_chunks) * kQChunk;
  const int64_t n = (int64_t)row_pos[r] + 1;
  if (s0 >= n) return;
  const int seq = row_seq[r];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int nthreads = blockDim.x;
  // Stage the chunk's rows (dead rows past n copy the last live row: finite values).
  const int pieces = Dqk / 8;  // 16-byte pieces per row
  for (int i = tid; i < kQChunk * pieces; i += nthreads) {
    const int t = i / pieces, c = i % pieces;
    const int64_t row = kv_row(table, page_size, max_pages, seq_stride, seq, min(s0 + t, n - 1));
    *reinterpret_cast<uint4*>(rows + t * kQRowStride + 16 * c) =
        reinterpret_cast<const uint4*>(kv + row * Dqk)[c];
  }
  // Query fragments: B[k = dim][n = head col] = q[r, 16w + col, 32*kk + 8*grp + j].
  const int col = lane & 15, grp = lane >> 4;
  const int nk = Dqk / 32;
  v8bf qf[kQMaxDqk / 32];
  const uint16_t* qrow = q + ((int64_t)r * H + 16 * w + col) * Dqk + 8 * grp;
#pragma unroll
  for (int kk = 0; kk < kQMaxDqk / 32; ++kk)
    if (kk < nk) qf[kk] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(qrow + 32 * kk));
  __syncthreads();
  float* zr = z2 + ((int64_t)r * H + 16 * w + col) * ld;
#pragma unroll
  for (int tb = 0; tb < kQChunk / 16; ++tb) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    const char* kb = rows + (16 * tb + col) * kQRowStride + 16 * grp;
#pragma unroll
    for (int kk = 0; kk < kQMaxDqk / 32; ++kk)
      if (kk < nk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const v8bf*>(kb + 64 * kk), qf[kk],
                                                      acc, 0, 0, 0);
    // lane holds tokens 16*tb + 4*grp + i of head col
    const int64_t s = s0 + 16 * tb + 4 * grp;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (s + i < n) zr[s + i] = acc[i] * scale_log2;
  }
}

// Online (max, sum of 2^(x - max)) over one row of n values; x = z2[r, h, :] for h < H, or
// the index scores scaled to log2 for h == H.  One workgroup per (row, h).
__global__ __launch_bounds__(256) void quality_stats_kernel(const float* __restrict__ z2,
                                                            const float* __restrict__ scores,
                                                            int64_t sld, const int32_t* __restrict__ row_pos,
                                                            int H, int64_t ld, float2* __restrict__ stats) {
  __shared__ float sm[256], sl[256];
  const int r = blockIdx.x / (H + 1), h = blockIdx.x % (H + 1);
  const int64_t n = (int64_t)row_pos[r] + 1;
  const float* x = h < H ? z2 + ((int64_t)r * H + h) * ld : scores + (int64_t)r * sld;
  const float mul = h < H ? 1.0f : kLog2e;
  // Eight loads in flight per step; the chunk's max is folded in before its sum.
  float m = -INFINITY, l = 0.0f;
  for (int64_t s0 = threadIdx.x; s0 < n; s0 += 256 * 8) {
    float v[8];
    float cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t s = s0 + 256 * u;
      v[u] = s < n ? x[s] * mul : -INFINITY;
      cm = fmaxf(cm, v[u]);
    }
    const float nm = fmaxf(m, cm);
    float acc = l > 0.0f ? l * exp2f(m - nm) : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u] == -INFINITY ? 0.0f : exp2f(v[u] - nm);
    m = nm;
    l = acc;
  }
  sm[threadIdx.x] = m;
  sl[threadIdx.x] = l;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      const float m2 = sm[threadIdx.x + o], l2 = sl[threadIdx.x + o];
      const float m1 = sm[threadIdx.x], l1 = sl[threadIdx.x];
      const float mm = fmaxf(m1, m2);
      sm[threadIdx.x] = mm;
      sl[threadIdx.x] = (l1 > 0.0f ? l1 * exp2f(m1 - mm) : 0.0f) + (l2 > 0.0f ? l2 * exp2f(m2 - mm) : 0.0f);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) stats[(int64_t)r * (H + 1) + h] = make_float2(sm[0], sl[0]);
}

// Partial sums over one chunk of tokens: KL terms p (ln p - ln q) and the kept set's mass.
__global__ __launch_bounds__(256) void quality_partial_kernel(
    const float* __restrict__ z2, const float* __restrict__ scores, int64_t sld,
    const int32_t* __restrict__ idx, int k, const int32_t* __restrict__ row_pos, int H, int64_t ld,
    const float2* __restrict__ stats, int n_chunks, float2* __restrict__ partial) {
  __shared__ uint32_t kept[kQSumChunk / 32];
  __shared__ float2 hst[129];  // per head: (max, 1 / sum); then the index scores' (max, sum)
  __shared__ float red_kl[256], red_rc[256];
  const int r = blockIdx.x / n_chunks;
  const int64_t c0 = (int64_t)(blockIdx.x % n_chunks) * kQSumChunk;
  const int64_t n = (int64_t)row_pos[r] + 1;
  float kl = 0.0f, rc = 0.0f;
  if (c0 < n) {
    for (int i = threadIdx.x; i < kQSumChunk / 32; i += 256) kept[i] = 0u;
    for (int h = threadIdx.x; h <= H; h += 256) {
      const float2 v = stats[(int64_t)r * (H + 1) + h];
      hst[h] = h < H ? make_float2(v.x, 1.0f / v.y) : v;
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
      if (p > 0.0f) kl += p * (logf(p) - log_q);
      if ((kept[(s - c0) >> 5] >> ((s - c0) & 31)) & 1u) rc += p;
    }
  }
  red_kl[threadIdx.x] = kl;
  red_rc[threadIdx.x] = rc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      red_kl[threadIdx.x] += red_kl[threadIdx.x + o];
      red_rc[threadIdx.x] += red_rc[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = make_float2(red_kl[0], red_rc[0]);
}

__global__ __launch_bounds__(256) void quality_finish_kernel(const float2* __restrict__ partial,
                                                             int n_chunks, float* __restrict__ kl,
                                                             float* __restrict__ recall) {
  __shared__ float a[256], b[256];
  const int r = blockIdx.x;
  float x = 0.0f, y = 0.0f;
  for (int c = threadIdx.x; c < n_chunks; c += 256) {
    const float2 v = partial[(int64_t)r * n_chunks + c];
    x += v.x;
    y += v.y;
  }
  a[threadIdx.x] = x;
  b[threadIdx.x] = y;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      a[threadIdx.x] += a[threadIdx.x + o];
      b[threadIdx.x] += b[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    kl[r] = a[0];
    recall[r] = b[0];
  }
}

struct QualityWs {
  size_t z2, stats, partial, total;
};
QualityWs quality_ws(int R, int H, int64_t ld) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  QualityWs L{};
  L.z2 = 0;
  L.stats = up(sizeof(float) * (size_t)R * H * (size_t)ld);
  L.partial = L.stats + up(sizeof(float2) * (size_t)R * (H + 1));
  L.total = L.partial + up(sizeof(float2) * (size_t)R * (size_t)((ld + kQSumChunk - 1) / kQSumChunk));
  return L;
}

}  // namespace

size_t quality_workspace_bytes(int R, int H, int64_t ld) { return quality_ws(R, H, ld).total; }

hipError_t launch_indexer_quality(const uint16_t* q, const CacheView& kv, const float* scores,
                                  int64_t sld, const int32_t* idx, int k, const int32_t* row_seq,
                                  const int32_t* row_pos, int R, int H, int Dqk, int64_t ld,
                                  float scale, float* kl, float* recall, void* ws, hipStream_t s) {
  const QualityWs L = quality_ws(R, H, ld);
  char* b = static_cast<char*>(ws);
  float* z2 = reinterpret_cast<float*>(b + L.z2);
  float2* stats = reinterpret_cast<float2*>(b + L.stats);
  float2* partial = reinterpret_cast<float2*>(b + L.partial);
  const int nc = (int)((ld + kQChunk - 1) / kQChunk);
  quality_logits_kernel<<<(unsigned)R * (unsigned)nc, (H / 16) * WAVE, 0, s>>>(
      q, static_cast<const uint16_t*>(kv.data), kv.table, kv.page_size, kv.max_pages, kv.seq_stride,
      row_seq, row_pos, H, Dqk, nc, scale * kLog2e, z2, ld);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  quality_stats_kernel<<<(unsigned)R * (unsigned)(H + 1), 256, 0, s>>>(z2, scores, sld, row_pos, H, ld, stats);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int ns = (int)((ld + kQSumChunk - 1) / kQSumChunk);
  quality_partial_kernel<<<(unsigned)R * (unsigned)ns, 256, 0, s>>>(z2, scores, sld, idx, k, row_pos, H, ld,
                                                                   stats, ns, partial);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  quality_finish_kernel<<<R, 256, 0, s>>>(partial, ns, kl, recall);
  return hipGetLastError();
}

}  // namespace dsa
