// Scoring core of the lightning indexer's fast shape (64 heads x 128, e4m3 operands):
// I[r,s] = k_scale[s] * q_scale[r] * sum_j w[r,j] * ReLU(q[r,j,:] . k[s,:]).
//
// The pages give the indexer as the lightweight FP8 first tier that scores every cached token
// before the top-k choice (MarkTechPost, "DeepSeek V3.2-Exp Cuts Long-Context Costs with
// DeepSeek Sparse Attention (DSA) ..."; maplevalley.com.cn news 1594152, section 1 "Lightning
// Indexer"); the ReLU-of-per-head-dots form is this library's reading.
//
// Every kernel that scores keys of this shape -- the indexer proper, the fused top-k's sample
// pass and its rescoring fallback -- goes through trip_scores and the same scale products, so
// a key gets the same bits of score wherever it is computed.
#pragma once
#include "common.h"

namespace dsa {

constexpr int kIdxBatch = 64;  // keys per wave per trip: four 16-key MFMA column groups

// Scores of one trip of 64 keys for 64 heads.  kb[u] holds lane (col, grp)'s 32 key bytes of
// key 16*u + col (k-slice grp), qa[ht] the matching query bytes of heads 16*ht + col, wr the
// weights of the heads the result layout leaves in this lane (16*ht + 4*grp + i).  Returns,
// in lane l, the weighted ReLU head sum of key l of the trip (before the scales).
__device__ __forceinline__ float trip_scores(const v8i (&qa)[4], const float (&wr)[4][4], const v8i (&kb)[4]) {
  float part[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    // The four head groups' products go out back to back into separate accumulators, so the
    // ReLU-weight epilogue of one overlaps the MFMAs still in flight instead of waiting on each.
    v4f acc[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      // cbsz/blgp = 0: both operands OCP e4m3; scale exponent 127 = x1.
      acc[ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ht], kb[u], v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                                 0, 0, 0, 127, 0, 127);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the four MFMAs ahead of the epilogue
    float sum = 0.0f;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int i = 0; i < 4; ++i) sum = fmaf(wr[ht][i], __builtin_amdgcn_fmed3f(acc[ht][i], 0.0f, 3.0e38f), sum);
    part[u] = sum;
  }
  // Stage 1 (lanes l, l^32): lower half keeps groups 0/1, upper half 2/3.
  const v2i x02 = __builtin_amdgcn_permlane32_swap(__float_as_int(part[0]), __float_as_int(part[2]), false, false);
  const v2i x13 = __builtin_amdgcn_permlane32_swap(__float_as_int(part[1]), __float_as_int(part[3]), false, false);
  const float h02 = __int_as_float(x02[0]) + __int_as_float(x02[1]);
  const float h13 = __int_as_float(x13[0]) + __int_as_float(x13[1]);
  // Stage 2 (rows of 16 lanes, r and r^1): row g ends with group g's full sum.
  const v2i y = __builtin_amdgcn_permlane16_swap(__float_as_int(h02), __float_as_int(h13), false, false);
  return __int_as_float(y[0]) + __int_as_float(y[1]);
}

// The score of a trip's key: head sum x key scale x query scale, in this order everywhere.
__device__ __forceinline__ float scaled_score(float tot, float ks, float qs) { return tot * ks * qs; }

// Query fragments and head weights of one row in the lane layout trip_scores expects.
__device__ __forceinline__ void load_query(const uint8_t* __restrict__ qr, const float* __restrict__ wrow,
                                           int col, int grp, v8i (&qa)[4], float (&wr)[4][4]) {
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const uint4* p = reinterpret_cast<const uint4*>(qr + (16 * ht + col) * 128 + 32 * grp);
    const uint4 a = p[0], b = p[1];
    qa[ht] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const float4 v = *reinterpret_cast<const float4*>(wrow + 16 * ht + 4 * grp);
    wr[ht][0] = v.x; wr[ht][1] = v.y; wr[ht][2] = v.z; wr[ht][3] = v.w;
  }
}

// Physical row of logical key s of sequence `seq` in a contiguous or paged key cache
// (page_shift = log2(page_size) for power-of-two pages, else -1).
struct KeyRows {
  const int32_t* table;
  int max_pages, page_size, page_shift;
  int64_t seq_stride;
  __device__ __forceinline__ int64_t row(int seq, int64_t s) const {
    if (!table) return (int64_t)seq * seq_stride + s;
    const int64_t pg = page_shift >= 0 ? (s >> page_shift) : s / page_size;
    const int64_t off = page_shift >= 0 ? (s & (page_size - 1)) : s % page_size;
    return (int64_t)table[(int64_t)seq * max_pages + pg] * page_size + off;
  }
};

// Loads lane (col, grp)'s key operand of one trip from cache rows rows[u] (key 16*u + col).
__device__ __forceinline__ void load_rows(const uint8_t* __restrict__ kdata, const int64_t (&rows)[4], int grp,
                                          v8i (&kb)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint4* p = reinterpret_cast<const uint4*>(kdata + rows[u] * 128 + 32 * grp);
    const uint4 a = p[0], b = p[1];
    kb[u] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }
}

// Loads lane (col, grp)'s key operand of one trip whose keys are at logical positions pos(j),
// j = 16*u + col (u < 4); positions are the caller's, already clamped into the row.
template <class Pos>
__device__ __forceinline__ void load_trip(const uint8_t* __restrict__ kdata, const KeyRows& kr, int seq, int col,
                                          int grp, Pos&& pos, v8i (&kb)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t row = kr.row(seq, pos(16 * u + col));
    const uint4* p = reinterpret_cast<const uint4*>(kdata + row * 128 + 32 * grp);
    const uint4 a = p[0], b = p[1];
    kb[u] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }
}

}  // namespace dsa
