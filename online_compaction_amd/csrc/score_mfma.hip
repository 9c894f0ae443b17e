// Token Eviction scoring on MFMA (bf16 operands, float32 accumulate) for gfx950.
//
// Score of key j of one unit ("Practical Online KV Cache Compaction for LLM Agents", design-space
// section, TE score equation): s_j = sqrt((1/R) sum_r alpha_rj^2) with
// alpha_rj = exp(l_rj - LSE_r) (ActKV page, paged-memory paragraph: weights recovered from the
// LSE without gathering or materialising the attention matrix).
//
// Two kernels, mirror images of each other:
//   lse_partials_mfma  reduces over KEYS for every proxy row: the WG keeps 512 proxy rows in
//                      registers (MFMA B operand) and streams 64-key stages of K through LDS
//                      (A operand); online max/sum in the log2 domain; one (max, sum) partial
//                      per row and key chunk goes to the workspace.
//   score_mfma         reduces over ROWS for every key: the WG keeps 512 keys in registers and
//                      streams 64-row stages of Q (and the per-row LSE term) through LDS; each
//                      lane accumulates exp2(2 log2(alpha) + 100) for its key, and the 4 lane
//                      groups that share a key are summed with two cross-lane exchanges.
// The d = 128 contraction is 4 k-steps of v_mfma_f32_16x16x32_bf16. Within a k-step, lane
// group g = lane / 16 supplies d-chunk 4*kstep + g (8 bf16 = 16 bytes) of its row, the same
// d permutation on both operands. LDS rows are 256 bytes; 16-byte chunk c of row r is stored
// at chunk position c ^ (r & 15) so the 16 rows read by one MFMA operand hit distinct banks.
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int kThreads = 256;
constexpr int kSub = 8;                 // 16-wide subtiles per wave held in registers (LSE pass)
constexpr int kPerWave = 16 * kSub;     // 128 rows per wave (LSE pass)
constexpr int kPerBlock = 4 * kPerWave; // 512 per workgroup (LSE pass)
#ifndef KVC_SCORE_KSUB
#define KVC_SCORE_KSUB 8
#endif
#ifndef KVC_SCORE_OCC
#define KVC_SCORE_OCC 2
#endif
constexpr int kScoreSub = KVC_SCORE_KSUB;           // key subtiles per wave (score pass)
constexpr int kScoreKeys = 4 * 16 * kScoreSub;      // keys per workgroup (score pass)
constexpr int kStage = 64;              // rows / keys per LDS stage

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Pointer to the 256-byte stored row at cache position `pos` of unit (s, h).
template <bool PAGED>
__device__ __forceinline__ const u32x4* key_row(const uint16_t* __restrict__ k, const int32_t* __restrict__ trow,
                                                int H, int h, int64_t n_max, int64_t unit, int pos) {
  if constexpr (PAGED) {
    const int64_t blk = trow[pos >> 4];
    return reinterpret_cast<const u32x4*>(k + ((blk * 16 + (pos & 15)) * H + h) * kHeadDim);
  } else {
    return reinterpret_cast<const u32x4*>(k + (unit * n_max + pos) * kHeadDim);
  }
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

}  // namespace

// ------------------------------------------------------------------------------------------------
// Pass 2: scores. Work item = (sequence, KV head, 512-key tile).
// lse: natural-log LSE per proxy row, [S][H*G][q] == [unit][R].
// ------------------------------------------------------------------------------------------------
template <bool PAGED, bool BIAS>
__global__ __launch_bounds__(kThreads, KVC_SCORE_OCC) void score_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const int32_t* __restrict__ table,
    int max_blocks, const float* __restrict__ lse, const float* __restrict__ bias, float* __restrict__ scores,
    int H, int R, int64_t n_max, float scale, SeqTable T) {
  __shared__ __attribute__((aligned(16))) uint8_t qs[2][kStage * 256];
  __shared__ __attribute__((aligned(16))) float nbs[2][kStage];

  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int ko = T.kofs[i];
  const int tiles = (n + kScoreKeys - 1) / kScoreKeys;
  const int local = t - T.start[i];
  const int h = local / tiles;
  const int kt = local - h * tiles;
  const int64_t unit = (int64_t)s * H + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int32_t* trow = PAGED ? table + (int64_t)s * max_blocks : nullptr;

  // keys of this wave, held for the whole row sweep
  bf16x8 kb[kScoreSub][4];
  float bb[kScoreSub];
  const int key0 = kt * kScoreKeys + wave * (16 * kScoreSub);
#pragma unroll
  for (int sub = 0; sub < kScoreSub; ++sub) {
    const int key = key0 + sub * 16 + c16;
    if (key < n) {
      const u32x4* p = key_row<PAGED>(k, trow, H, h, n_max, unit, ko + key);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[sub][ks] = as_bf16x8(p[4 * ks + g]);
      if constexpr (BIAS) bb[sub] = 2.0f * kLog2e * bias[(int64_t)s * n_max + key];
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[sub][ks] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      if constexpr (BIAS) bb[sub] = 0.0f;
    }
  }

  const uint16_t* qu = q + unit * (int64_t)R * kHeadDim;
  const float* lu = lse + unit * (int64_t)R;
  const float a2 = 2.0f * kLog2e * scale;
  const int nst = (R + kStage - 1) / kStage;

  u32x4 pre[4];
  float prenb = 0.0f;
  auto load_stage = [&](int st) {
    const int r0 = st * kStage;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int id = tid + kThreads * j, row = id >> 4, c = id & 15;
      const int r = r0 + row;
      pre[j] = r < R ? reinterpret_cast<const u32x4*>(qu + (int64_t)r * kHeadDim)[c] : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < kStage) {
      const int r = r0 + tid;
      prenb = r < R ? kSqOffset - 2.0f * kLog2e * lu[r] : -INFINITY;
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int id = tid + kThreads * j, row = id >> 4, c = id & 15;
      *reinterpret_cast<u32x4*>(&qs[buf][swz(row, c)]) = pre[j];
    }
    if (tid < kStage) nbs[buf][tid] = prenb;
  };

  float ssum[kScoreSub];
#pragma unroll
  for (int sub = 0; sub < kScoreSub; ++sub) ssum[sub] = 0.0f;

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) load_stage(st + 1);
#pragma unroll 1
    for (int rt = 0; rt < kStage / 16; ++rt) {
      const int row = rt * 16 + c16;
      bf16x8 a[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) a[ks] = *reinterpret_cast<const bf16x8*>(&qs[buf][swz(row, 4 * ks + g)]);
      const f32x4 nb4 = *reinterpret_cast<const f32x4*>(&nbs[buf][rt * 16 + 4 * g]);
      f32x4 acc[kScoreSub];
#pragma unroll
      for (int sub = 0; sub < kScoreSub; ++sub) acc[sub] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int sub = 0; sub < kScoreSub; ++sub) acc[sub] = mfma16(a[ks], kb[sub][ks], acc[sub]);
#pragma unroll
      for (int sub = 0; sub < kScoreSub; ++sub) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = __builtin_fmaf(acc[sub][e], a2, nb4[e]);
          if constexpr (BIAS) x += bb[sub];
          ssum[sub] += __builtin_amdgcn_exp2f(x);
        }
      }
    }
    if (st + 1 < nst) store_stage(buf ^ 1);
    __syncthreads();
  }

  const float invR = 1.0f / (float)R;
#pragma unroll
  for (int sub = 0; sub < kScoreSub; ++sub) {
    float v = ssum[sub];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    const int key = key0 + sub * 16 + c16;
    if (g == 0 && key < n) scores[unit * n_max + key] = __builtin_sqrtf(v * invR) * kSqUnscale;
  }
}

// ------------------------------------------------------------------------------------------------
// Pass 1: per proxy row, partial (max, sum) of 2^(log2e * l_rj) over one key chunk, with the
// max kept lazily (rescale only when a new maximum exceeds the reference by more than 2^8).
// Work item = (sequence, KV head, key chunk kc, 512-row block rb), rb fastest so the blocks
// sharing a key chunk run together on one XCD.
// partials: float2 [T.off[i] + (h * nkc + kc) * R + row]
// ------------------------------------------------------------------------------------------------
template <bool PAGED, bool BIAS>
__global__ __launch_bounds__(kThreads, 2) void lse_partials_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const int32_t* __restrict__ table,
    int max_blocks, const float* __restrict__ bias, float2* __restrict__ partials, int H, int R,
    int64_t n_max, float scale, int kchunk, SeqTable T) {
  __shared__ __attribute__((aligned(16))) uint8_t ks_[2][kStage * 256];
  __shared__ __attribute__((aligned(16))) float kts[2][kStage];

  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int ko = T.kofs[i];
  const int nkc = (n + kchunk - 1) / kchunk;
  const int nrb = (R + kPerBlock - 1) / kPerBlock;
  int local = t - T.start[i];
  const int h = local / (nkc * nrb);
  local -= h * nkc * nrb;
  const int kc = local / nrb;
  const int rb = local - kc * nrb;
  const int64_t unit = (int64_t)s * H + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int32_t* trow = PAGED ? table + (int64_t)s * max_blocks : nullptr;

  // proxy rows of this wave, held for the whole key sweep
  const uint16_t* qu = q + unit * (int64_t)R * kHeadDim;
  const int row0 = rb * kPerBlock + wave * kPerWave;
  bf16x8 qb[kSub][4];
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    const int r = row0 + sub * 16 + c16;
    if (r < R) {
      const u32x4* p = reinterpret_cast<const u32x4*>(qu + (int64_t)r * kHeadDim);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qb[sub][kk] = as_bf16x8(p[4 * kk + g]);
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qb[sub][kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }

  const int kbeg = kc * kchunk;
  const int kend = min(n, kbeg + kchunk);
  const int nst = (kend - kbeg + kStage - 1) / kStage;
  const float c2 = kLog2e * scale;

  u32x4 pre[4];
  float prekt = 0.0f;
  auto load_stage = [&](int st) {
    const int k0 = kbeg + st * kStage;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int id = tid + kThreads * j, row = id >> 4, c = id & 15;
      const int key = k0 + row;
      pre[j] = key < kend ? key_row<PAGED>(k, trow, H, h, n_max, unit, ko + key)[c] : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < kStage) {
      const int key = k0 + tid;
      if (key < kend) {
        prekt = 0.0f;
        if constexpr (BIAS) prekt = kLog2e * bias[(int64_t)s * n_max + key];
      } else {
        prekt = -INFINITY;
      }
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int id = tid + kThreads * j, row = id >> 4, c = id & 15;
      *reinterpret_cast<u32x4*>(&ks_[buf][swz(row, c)]) = pre[j];
    }
    if (tid < kStage) kts[buf][tid] = prekt;
  };

  float mref[kSub], ssum[kSub];
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    mref[sub] = -1.0e30f;
    ssum[sub] = 0.0f;
  }

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) load_stage(st + 1);
#pragma unroll 1
    for (int kt = 0; kt < kStage / 16; ++kt) {
      const int row = kt * 16 + c16;
      bf16x8 a[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) a[kk] = *reinterpret_cast<const bf16x8*>(&ks_[buf][swz(row, 4 * kk + g)]);
      const f32x4 kt4 = *reinterpret_cast<const f32x4*>(&kts[buf][kt * 16 + 4 * g]);
      f32x4 acc[kSub];
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) acc[sub] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int sub = 0; sub < kSub; ++sub) acc[sub] = mfma16(a[kk], qb[sub][kk], acc[sub]);
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(acc[sub][e], c2, kt4[e]);
        const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        if (mx > mref[sub] + 8.0f) {
          ssum[sub] *= __builtin_amdgcn_exp2f(mref[sub] - mx);
          mref[sub] = mx;
        }
        const float mr = mref[sub];
        ssum[sub] += (__builtin_amdgcn_exp2f(x[0] - mr) + __builtin_amdgcn_exp2f(x[1] - mr)) +
                     (__builtin_amdgcn_exp2f(x[2] - mr) + __builtin_amdgcn_exp2f(x[3] - mr));
      }
    }
    if (st + 1 < nst) store_stage(buf ^ 1);
    __syncthreads();
  }

  const int64_t pbase = T.off[i] + ((int64_t)h * nkc + kc) * R;
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    float m1 = mref[sub], s1 = ssum[sub];
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float m2 = __shfl_xor(m1, off), s2 = __shfl_xor(s1, off);
      const float mm = fmaxf(m1, m2);
      s1 = s1 * __builtin_amdgcn_exp2f(m1 - mm) + s2 * __builtin_amdgcn_exp2f(m2 - mm);
      m1 = mm;
    }
    const int r = row0 + sub * 16 + c16;
    if (g == 0 && r < R) partials[pbase + r] = make_float2(m1, s1);
  }
}

// ------------------------------------------------------------------------------------------------
// Combine the per-chunk partials of every proxy row into its natural-log LSE.
// Work item = (sequence, KV head, 256-row block); partial chunk count per unit = nchunk(n).
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lse_combine(const float2* __restrict__ partials, float* __restrict__ lse_out,
                                                   int H, int R, int kchunk, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int nkc = (n + kchunk - 1) / kchunk;
  const int nrb = (R + 255) / 256;
  const int local = t - T.start[i];
  const int h = local / nrb;
  const int r = (local - h * nrb) * 256 + threadIdx.x;
  if (r >= R) return;
  const float2* p = partials + T.off[i] + (int64_t)h * nkc * R + r;
  float mm = -INFINITY;
  for (int c = 0; c < nkc; ++c) mm = fmaxf(mm, p[(int64_t)c * R].x);
  float sum = 0.0f;
  for (int c = 0; c < nkc; ++c) {
    const float2 v = p[(int64_t)c * R];
    sum += v.y * __builtin_amdgcn_exp2f(v.x - mm);
  }
  lse_out[((int64_t)s * H + h) * R + r] = (mm + __builtin_log2f(sum)) * kLn2;
}

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------
int score_mfma_tiles(int n) { return (n + kScoreKeys - 1) / kScoreKeys; }
int lse_mfma_row_blocks(int R) { return (R + kPerBlock - 1) / kPerBlock; }

hipError_t launch_score_mfma(bool paged, bool has_bias, const void* q, const void* k, const int32_t* table,
                             int max_blocks, const float* lse, const float* bias, float* scores, int H, int R,
                             int64_t n_max, float scale, const SeqTable& T, hipStream_t st) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  dim3 grid(T.total), block(kThreads);
  if (paged) {
    if (has_bias)
      score_mfma<true, true><<<grid, block, 0, st>>>(qq, kk, table, max_blocks, lse, bias, scores, H, R, n_max, scale, T);
    else
      score_mfma<true, false><<<grid, block, 0, st>>>(qq, kk, table, max_blocks, lse, bias, scores, H, R, n_max, scale, T);
  } else {
    if (has_bias)
      score_mfma<false, true><<<grid, block, 0, st>>>(qq, kk, table, max_blocks, lse, bias, scores, H, R, n_max, scale, T);
    else
      score_mfma<false, false><<<grid, block, 0, st>>>(qq, kk, table, max_blocks, lse, bias, scores, H, R, n_max, scale, T);
  }
  return hipGetLastError();
}

hipError_t launch_lse_partials_mfma(bool paged, bool has_bias, const void* q, const void* k, const int32_t* table,
                                    int max_blocks, const float* bias, float2* partials, int H, int R, int64_t n_max,
                                    float scale, int kchunk, const SeqTable& T, hipStream_t st) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  dim3 grid(T.total), block(kThreads);
  if (paged) {
    if (has_bias)
      lse_partials_mfma<true, true><<<grid, block, 0, st>>>(qq, kk, table, max_blocks, bias, partials, H, R, n_max, scale, kchunk, T);
    else
      lse_partials_mfma<true, false><<<grid, block, 0, st>>>(qq, kk, table, max_blocks, bias, partials, H, R, n_max, scale, kchunk, T);
  } else {
    if (has_bias)
      lse_partials_mfma<false, true><<<grid, block, 0, st>>>(qq, kk, table, max_blocks, bias, partials, H, R, n_max, scale, kchunk, T);
    else
      lse_partials_mfma<false, false><<<grid, block, 0, st>>>(qq, kk, table, max_blocks, bias, partials, H, R, n_max, scale, kchunk, T);
  }
  return hipGetLastError();
}

hipError_t launch_lse_combine(const float2* partials, float* lse_out, int H, int R, int kchunk, const SeqTable& T,
                              hipStream_t st) {
  lse_combine<<<dim3(T.total), dim3(256), 0, st>>>(partials, lse_out, H, R, kchunk, T);
  return hipGetLastError();
}

}  // namespace kvc
