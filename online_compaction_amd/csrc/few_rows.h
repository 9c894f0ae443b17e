// Pieces shared by the kernels that score units with few proxy rows (score_valu.hip: float32 and
// the cached score pass; score_small.hip: bf16 on MFMA): the per-chunk LDS staging of block-table
// entries, slots and bias, key-row addressing, (max, sum) merging of LSE partials and the per-row
// exponent offsets. Logits are in log2 units throughout; see score_valu.hip for the passes.
#pragma once

#include <climits>

#include "kvc_internal.h"

namespace kvc {
namespace few {

constexpr int kThreads = 256;  // 4 waves
constexpr int kMaxChunk = kValuMaxChunk;

// (max, sum of 2^(y - max)) pairs; max = -inf with sum 0 when nothing has been seen
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  const float a = s > 0.0f ? s * __builtin_amdgcn_exp2f(m - mm) : 0.0f;
  const float b = s2 > 0.0f ? s2 * __builtin_amdgcn_exp2f(m2 - mm) : 0.0f;
  m = mm;
  s = a + b;
}

// Per-workgroup view of one unit's key chunk [kbeg, kend): the chunk's block-table entries
// (paged) or slots (slot map) and its per-key bias (times bias_scale) staged in LDS, so every key
// address and mask depends on LDS only.
struct ChunkLds {
  int32_t idx[kMaxChunk];
  float kts[kMaxChunk];
};

template <int LAYOUT>
__device__ __forceinline__ void stage_chunk(ChunkLds& L, const int32_t* __restrict__ table, int max_blocks,
                                            const float* __restrict__ bias, int64_t n_max, int s, int64_t unit,
                                            int ko, int kbeg, int kend, float bias_scale = kLog2e) {
  const int tid = threadIdx.x;
  if constexpr (LAYOUT == kPaged) {
    const int32_t* trow = table + (int64_t)s * max_blocks;
    const int blk0 = (ko + kbeg) >> 4;
    const int nb = ((ko + kend - 1) >> 4) - blk0 + 1;
    for (int b = tid; b < nb; b += kThreads) L.idx[b] = trow[blk0 + b];
  } else if constexpr (LAYOUT == kSlots) {
    const int32_t* srow = table + unit * n_max + ko;
    for (int j = tid; j < kend - kbeg; j += kThreads) L.idx[j] = srow[kbeg + j];
  }
  for (int j = tid; j < kend - kbeg; j += kThreads)
    L.kts[j] = bias ? bias_scale * bias[(int64_t)s * n_max + kbeg + j] : 0.0f;
}

template <bool F32, int LAYOUT>
__device__ __forceinline__ const void* chunk_key_row(const void* __restrict__ k, const ChunkLds& L, int H, int h,
                                               int64_t n_max, int64_t unit, int ko, int kbeg, int key) {
  constexpr int esz = F32 ? 4 : 2;
  const int pos = ko + key;
  int64_t row;
  if constexpr (LAYOUT == kPaged) {
    row = ((int64_t)L.idx[(pos >> 4) - ((ko + kbeg) >> 4)] * 16 + (pos & 15)) * H + h;
  } else if constexpr (LAYOUT == kSlots) {
    row = (int64_t)L.idx[key - kbeg] * H + h;
  } else {
    row = unit * n_max + pos;
  }
  return static_cast<const char*>(k) + row * (kHeadDim * esz);
}

// Every proxy row's exponent offset nb_r = kSqOffset - pw * L2_r (L2 = log2(e) * LSE) for rows
// [row0, row0 + nrows) into nbs[0 .. nrows): from the supplied LSE, or merged from the unit's nkc
// chunk partials by `lpr` lanes per row (a power of two <= 64, so a row's lanes share a wave;
// lpr * nrows <= kThreads), each with four partial loads in flight. A row whose keys are all
// masked gets +inf (its logits are all -inf, and those terms are skipped).
__device__ __forceinline__ void row_terms(const float* __restrict__ lse, const float2* __restrict__ parts, int nkc,
                                          int64_t unit, int R, int row0, int nrows, int lpr, float pw, float* nbs) {
  const int t = threadIdx.x;
  const int rr = t / lpr, sub = t % lpr;
  const int r = row0 + rr;
  const bool live = rr < nrows && r < R;
  if (lse) {
    if (live && sub == 0) nbs[rr] = kSqOffset - pw * kLog2e * lse[unit * R + r];
    return;
  }
  float m = -INFINITY, s = 0.0f;
  if (live) {
    const float2* p = parts + r;
    int kc = sub;
    for (; kc + 3 * lpr < nkc; kc += 4 * lpr) {
      const float2 a = p[(int64_t)kc * R], b = p[(int64_t)(kc + lpr) * R];
      const float2 c = p[(int64_t)(kc + 2 * lpr) * R], d = p[(int64_t)(kc + 3 * lpr) * R];
      merge_ms(m, s, a.x, a.y);
      merge_ms(m, s, b.x, b.y);
      merge_ms(m, s, c.x, c.y);
      merge_ms(m, s, d.x, d.y);
    }
    for (; kc < nkc; kc += lpr) {
      const float2 a = p[(int64_t)kc * R];
      merge_ms(m, s, a.x, a.y);
    }
  }
  for (int off = 1; off < lpr; off <<= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    merge_ms(m, s, m2, s2);
  }
  if (live && sub == 0) nbs[rr] = s > 0.0f ? kSqOffset - pw * (m + __builtin_log2f(s)) : INFINITY;
}

// Lanes per row for merging the partials of n rows: all 256 threads, at most one wave per row.
__device__ __forceinline__ int lanes_per_row(int n) {
  int l = 64;
  while (l > 1 && l * n > kThreads) l >>= 1;
  return l;
}

__device__ __forceinline__ float finish(float acc, int R, int pw) {
  return pw == 2 ? __builtin_sqrtf(acc / (float)R) * kSqUnscale : acc / (float)R * kMassUnscale;
}
}  // namespace few
}  // namespace kvc
