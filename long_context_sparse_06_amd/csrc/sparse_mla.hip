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
constexpr int kTok = 32;                       // rows per LDS tile
constexpr int kRowChunks = kDqk * 2 / 16;      // 72 16-byte chunks per latent row
constexpr int kRS = kDqk * 2 + 16;             // padded LDS row stride (bytes)
constexpr int kTileBytes = kTok * kRS;
constexpr int kMlaWaves = 4;
constexpr int kMlaThreads = kMlaWaves * WAVE;
constexpr int kHeadsPerWg = 16 * kMlaWaves;
constexpr int kPrefetch = (kTok * kRowChunks + kMlaThreads - 1) / kMlaThreads;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ v4bf lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(p));
}

template <bool PAGED, bool SPLIT>
__global__ __launch_bounds__(kMlaThreads) void mla_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ table, int max_pages, int page_size, int64_t seq_stride,
    const int32_t* __restrict__ idx, int k, int H, int decode, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml, int n_split, int tok_per_split) {
  __shared__ __attribute__((aligned(16))) char tile[2][kTileBytes];
  __shared__ int tidx[2][kTok];

  const int HG = H / kHeadsPerWg;
  int bid = blockIdx.x;
  const int sp = bid % n_split;
  bid /= n_split;
  const int hg = bid % HG;
  const int r = bid / HG;
  const int t_begin = sp * tok_per_split;
  const int t_end = min(k, t_begin + tok_per_split);
  const int seq = decode ? r : 0;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int col = lane & 15, grp = lane >> 4;
  const int h = hg * kHeadsPerWg + 16 * w + col;
  const int32_t* irow = idx + (int64_t)r * k;

  // Query fragments: B[k = dim][n = head col] = q[r, h, 32*kk + 8*grp + j].
  v8bf qf[kDqk / 32];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)r * H + h) * kDqk + 8 * grp);
#pragma unroll
    for (int kk = 0; kk < kDqk / 32; ++kk) {
      const uint4 x = qp[4 * kk];
      qf[kk] = __builtin_bit_cast(v8bf, x);
    }
  }

  v4f acc_o[kDv / 16];
#pragma unroll
  for (int dt = 0; dt < kDv / 16; ++dt) acc_o[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of scaled logits (log2 domain), per head = col
  float l_run = 0.0f;       // this lane's share of the running sum

  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTok - 1) / kTok : 0;
  uint4 pre[kPrefetch];
  int pre_id = -1;

  auto row_ptr = [&](int id) -> const uint16_t* {
    int64_t row;
    if (PAGED) {
      row = (int64_t)table[(int64_t)seq * max_pages + id / page_size] * page_size + id % page_size;
    } else {
      row = (int64_t)seq * seq_stride + id;
    }
    return kv + row * kDqk;
  };
  auto prefetch = [&](int t0) {
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) {
      const int c = tid + i * kMlaThreads;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < kTok * kRowChunks) {
        const int j = c / kRowChunks, ch = c % kRowChunks;
        const int t = t0 + j;
        const int id = t < t_end ? irow[t] : -1;
        if (id >= 0) v = *reinterpret_cast<const uint4*>(row_ptr(id) + 8 * ch);
      }
      pre[i] = v;
    }
    pre_id = (tid < kTok && t0 + tid < t_end) ? irow[t0 + tid] : -1;
  };

  if (ntiles > 0) prefetch(t_begin);
  for (int it = 0; it < ntiles; ++it) {
    const int b = it & 1;
    char* tb = tile[b];
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) {
      const int c = tid + i * kMlaThreads;
      if (c < kTok * kRowChunks) {
        const int j = c / kRowChunks, ch = c % kRowChunks;
        *reinterpret_cast<uint4*>(tb + j * kRS + 16 * ch) = pre[i];
      }
    }
    if (tid < kTok) tidx[b][tid] = pre_id;
    __syncthreads();
    if (it + 1 < ntiles) prefetch(t_begin + (it + 1) * kTok);

    // ---- S^T = K Q^T for tokens 0..15 (st = 0) and 16..31 (st = 1)
    v4f acc_s[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < kDqk / 32; ++kk) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const v8bf a = *reinterpret_cast<const v8bf*>(tb + (16 * st + col) * kRS + 64 * kk + 16 * grp);
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
        const bool ok = tidx[b][16 * st + 4 * grp + i] >= 0;
        s[st][i] = ok ? acc_s[st][i] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[st][i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;  // no valid token yet: p = 0
    const float alpha = exp2f(m_run - m_use);               // m_run = -inf -> 0
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
    l_run = l_run * alpha + psum;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < kDv / 16; ++dt) acc_o[dt] *= alpha;
    }
    m_run = m_new;
    // P^T fragment: k-slot 8*grp + j <-> token 4*grp + j (j < 4) or 16 + 4*grp + (j - 4).
    v8bf pf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pf[i] = (__bf16)p[0][i];
      pf[4 + i] = (__bf16)p[1][i];
    }
    // ---- O^T += V^T P^T, 32 tiles of 16 value columns
    const char* v0 = tb + (4 * grp + (col >> 2)) * kRS + 8 * (col & 3);
    const char* v1 = v0 + 16 * kRS;
#pragma unroll
    for (int dt = 0; dt < kDv / 16; ++dt) {
      const v4bf lo = lds_read_tr16(v0 + 32 * dt);
      const v4bf hi = lds_read_tr16(v1 + 32 * dt);
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

// Log-sum-exp merge of the split partials: one 64-thread group per (row, head),
// 8 value columns per thread.
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int RH, int H, int n_split,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int pair = blockIdx.x * 4 + threadIdx.x / WAVE;
  if (pair >= RH) return;
  const int r = pair / H, h = pair % H;
  const int lane = threadIdx.x & (WAVE - 1);
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) {
    const int64_t pr = ((int64_t)r * n_split + s) * H + h;
    if (part_ml[2 * pr + 1] > 0.0f) M = fmaxf(M, part_ml[2 * pr]);
  }
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float L = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_split; ++s) {
      const int64_t pr = ((int64_t)r * n_split + s) * H + h;
      const float ls = part_ml[2 * pr + 1];
      if (!(ls > 0.0f)) continue;
      const float f = exp2f(part_ml[2 * pr] - M);
      L += ls * f;
      const float4* po = reinterpret_cast<const float4*>(part_o + pr * kDv + 8 * lane);
      const float4 a = po[0], b = po[1];
      o[0] += a.x * f; o[1] += a.y * f; o[2] += a.z * f; o[3] += a.w * f;
      o[4] += b.x * f; o[5] += b.y * f; o[6] += b.z * f; o[7] += b.w * f;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  uint32_t pk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    pk[i] = f32_to_bf16(o[2 * i] * inv) | ((uint32_t)f32_to_bf16(o[2 * i + 1] * inv) << 16);
  *reinterpret_cast<uint4*>(out + ((int64_t)r * H + h) * kDv + 8 * lane) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  if (lse && lane == 0) lse[(int64_t)r * H + h] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
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
  // Enough workgroups to cover the chip twice, but at least 256 kept rows per workgroup
  // so the partial (o, m, l) traffic stays below the gathered KV bytes.
  const int groups = B * (H / kHeadsPerWg);
  int ns = (512 + groups - 1) / groups;
  const int max_ns = (k + 255) / 256;
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
  mla_bf16_kernel<PG, SP><<<grid, kMlaThreads, 0, s>>>(q, kvp, kv.table, kv.max_pages,             \
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
  mla_combine_kernel<<<(RH + 3) / 4, 256, 0, s>>>(part_o, part_ml, RH, H, p.n_split, out, lse);
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
