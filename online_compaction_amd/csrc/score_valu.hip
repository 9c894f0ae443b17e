// Token Eviction scoring on the vector ALU, for float32 inputs and for bf16 units with so few
// proxy rows (R < 16) that the pass is bound by reading K, not by the dot products.
//
// Same two passes as the MFMA path (score equation of the design-space section of "Practical
// Online KV Cache Compaction for LLM Agents"; exp(logit - LSE) recovery from the ActKV page's
// paged-memory paragraph). One thread owns one key: its 128-element row is widened to float32
// in registers once, the proxy rows are staged as float32 in LDS (every lane reads the same
// address, a broadcast), and each logit is a 128-term FMA chain.
//   pass 1 (lse_partials_valu): per proxy row, (max, sum) of 2^(log2e * logit) over the
//           block's 256 keys -> workspace partials, combined by lse_combine.
//   pass 2 (score_valu): per key, sum over rows of exp2(2 log2(alpha) + 100) -> score, or of
//           exp2(log2(alpha) + 100) -> attention mass.
#include <climits>

#include "kvc_internal.h"

namespace kvc {

namespace {
constexpr int kThreads = 256;   // keys per block
constexpr int kRowsStage = 32;  // proxy rows per LDS stage (32 x 512 B = 16 KB)

// Stored row of key position `pos` of unit (s, h), widened to float32. `map` is the sequence's
// block table (kPaged) or the unit's slot-map row (kSlots).
template <int LAYOUT>
__device__ __forceinline__ int64_t key_row_index(const int32_t* __restrict__ map, int H, int h, int64_t n_max,
                                                 int64_t unit, int pos) {
  if constexpr (LAYOUT == kPaged) return ((int64_t)map[pos >> 4] * 16 + (pos & 15)) * H + h;
  else if constexpr (LAYOUT == kSlots) return (int64_t)map[pos] * H + h;
  else return unit * n_max + pos;
}

template <bool F32, int LAYOUT>
__device__ __forceinline__ void load_key_f32(const void* __restrict__ kbase, const int32_t* __restrict__ map, int H,
                                             int h, int64_t n_max, int64_t unit, int pos, float (&kr)[kHeadDim]) {
  const int64_t row = key_row_index<LAYOUT>(map, H, h, n_max, unit, pos);
  if constexpr (F32) {
    const float* p = static_cast<const float*>(kbase) + row * kHeadDim;
    const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int c = 0; c < kHeadDim / 4; ++c) {
      const float4 v = p4[c];
      kr[4 * c] = v.x; kr[4 * c + 1] = v.y; kr[4 * c + 2] = v.z; kr[4 * c + 3] = v.w;
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(kbase) + row * kHeadDim;
    const u32x4* p4 = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int c = 0; c < kHeadDim / 8; ++c) {
      const u32x4 v = p4[c];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kr[8 * c + 2 * e] = bf16_lo(w[e]);
        kr[8 * c + 2 * e + 1] = bf16_hi(w[e]);
      }
    }
  }
}

// Stage proxy rows [r0, r0 + kRowsStage) of the unit as float32 into LDS (zeros past R).
template <bool F32>
__device__ __forceinline__ void stage_rows(const void* __restrict__ qbase, int64_t unit, int R, int r0,
                                           float (*qs)[kHeadDim]) {
  for (int id = threadIdx.x; id < kRowsStage * (kHeadDim / 4); id += kThreads) {
    const int row = id / (kHeadDim / 4), c4 = id % (kHeadDim / 4);
    const int r = r0 + row;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < R) {
      if constexpr (F32) {
        v = reinterpret_cast<const float4*>(static_cast<const float*>(qbase) + (unit * R + r) * kHeadDim)[c4];
      } else {
        const uint2 w = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(qbase) + (unit * R + r) * kHeadDim)[c4];
        v = make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
      }
    }
    *reinterpret_cast<float4*>(&qs[row][4 * c4]) = v;
  }
}

__device__ __forceinline__ float dot_row(const float (&kr)[kHeadDim], const float* __restrict__ qrow) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int c = 0; c < kHeadDim / 4; ++c) {
    const float4 qv = *reinterpret_cast<const float4*>(qrow + 4 * c);
    a0 = __builtin_fmaf(kr[4 * c], qv.x, a0);
    a1 = __builtin_fmaf(kr[4 * c + 1], qv.y, a1);
    a2 = __builtin_fmaf(kr[4 * c + 2], qv.z, a2);
    a3 = __builtin_fmaf(kr[4 * c + 3], qv.w, a3);
  }
  return (a0 + a1) + (a2 + a3);
}
}  // namespace

// Work item = (sequence, KV head, 256-key tile).
template <bool F32, int LAYOUT, bool BIAS>
__global__ __launch_bounds__(kThreads) void score_valu(const void* __restrict__ q, const void* __restrict__ k,
                                                       const int32_t* __restrict__ table, int max_blocks,
                                                       const float* __restrict__ lse, const float* __restrict__ bias,
                                                       const int32_t* __restrict__ rpos, float* __restrict__ scores,
                                                       int H, int R, int64_t n_max, float scale, int pw, int dead,
                                                       SeqTable T) {
  __shared__ __attribute__((aligned(16))) float qs[kRowsStage][kHeadDim];
  __shared__ float nbs[kRowsStage];
  __shared__ int32_t pss[kRowsStage];  // causal: the rows' positions (INT32_MAX without a mask)
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int tiles = (n + kThreads - 1) / kThreads;
  const int local = t - T.start[i];
  const int h = local / tiles;
  const int key = (local - h * tiles) * kThreads + threadIdx.x;
  const int64_t unit = (int64_t)s * H + h;
  const int32_t* map = LAYOUT == kPaged ? table + (int64_t)s * max_blocks
                                        : (LAYOUT == kSlots ? table + unit * n_max : nullptr);
  const bool inrange = key < n;
  const bool isdead = LAYOUT == kSlots && inrange && map[T.kofs[i] + key] == dead;  // scored 0
  const bool valid = inrange && !isdead;

  float kr[kHeadDim];
  if (valid)
    load_key_f32<F32, LAYOUT>(k, map, H, h, n_max, unit, T.kofs[i] + key, kr);
  else
#pragma unroll
    for (int e = 0; e < kHeadDim; ++e) kr[e] = 0.f;
  // pw = 2: squared weights (the score); pw = 1: the weights themselves (attention mass)
  const float pl2 = (float)pw * kLog2e;
  float bb = 0.f;
  if constexpr (BIAS) bb = valid ? pl2 * bias[(int64_t)s * n_max + key] : 0.f;

  const float a2 = pl2 * scale;
  float acc = 0.f;
  for (int r0 = 0; r0 < R; r0 += kRowsStage) {
    __syncthreads();
    stage_rows<F32>(q, unit, R, r0, qs);
    if (threadIdx.x < kRowsStage) {
      const int r = r0 + threadIdx.x;
      nbs[threadIdx.x] = r < R ? kSqOffset - pl2 * lse[unit * R + r] : -INFINITY;
      pss[threadIdx.x] = (rpos && r < R) ? rpos[unit * R + r] : INT32_MAX;
    }
    __syncthreads();
    const int rows = min(kRowsStage, R - r0);
    for (int rr = 0; rr < rows; ++rr) {
      float x = __builtin_fmaf(dot_row(kr, qs[rr]), a2, nbs[rr]);
      if constexpr (BIAS) x += bb;
      if (key > pss[rr]) x = -INFINITY;  // causal: the row does not see this key
      acc += __builtin_amdgcn_exp2f(x);
    }
  }
  if (inrange)
    scores[unit * n_max + key] = isdead ? 0.0f
                                 : pw == 2 ? __builtin_sqrtf(acc / (float)R) * kSqUnscale : acc / (float)R * kMassUnscale;
}

// Work item = (sequence, KV head, 256-key tile); partial chunk = the tile.
// partials: float2 [T.off[i] + (h * ntiles + tile) * R + row]
template <bool F32, int LAYOUT, bool BIAS>
__global__ __launch_bounds__(kThreads) void lse_partials_valu(const void* __restrict__ q, const void* __restrict__ k,
                                                              const int32_t* __restrict__ table, int max_blocks,
                                                              const float* __restrict__ bias,
                                                              const int32_t* __restrict__ rpos,
                                                              float2* __restrict__ partials, int H, int R,
                                                              int64_t n_max, float scale, int dead, SeqTable T) {
  __shared__ __attribute__((aligned(16))) float qs[kRowsStage][kHeadDim];
  __shared__ float2 wred[kThreads / 64][kRowsStage];
  __shared__ int32_t pss[kRowsStage];  // causal: the rows' positions (INT32_MAX without a mask)
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int tiles = (n + kThreads - 1) / kThreads;
  const int local = t - T.start[i];
  const int h = local / tiles;
  const int tile = local - h * tiles;
  const int key = tile * kThreads + threadIdx.x;
  const int64_t unit = (int64_t)s * H + h;
  const int32_t* map = LAYOUT == kPaged ? table + (int64_t)s * max_blocks
                                        : (LAYOUT == kSlots ? table + unit * n_max : nullptr);
  // keys in the dead slot take no part in the softmax, like keys past n
  const bool valid = key < n && !(LAYOUT == kSlots && map[T.kofs[i] + key] == dead);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  float kr[kHeadDim];
  if (valid)
    load_key_f32<F32, LAYOUT>(k, map, H, h, n_max, unit, T.kofs[i] + key, kr);
  else
#pragma unroll
    for (int e = 0; e < kHeadDim; ++e) kr[e] = 0.f;
  float kt = valid ? 0.f : -INFINITY;
  if constexpr (BIAS) if (valid) kt = kLog2e * bias[(int64_t)s * n_max + key];

  const float c2 = kLog2e * scale;
  float2* pout = partials + T.off[i] + ((int64_t)h * tiles + tile) * R;
  for (int r0 = 0; r0 < R; r0 += kRowsStage) {
    __syncthreads();
    stage_rows<F32>(q, unit, R, r0, qs);
    if (threadIdx.x < kRowsStage) {
      const int r = r0 + threadIdx.x;
      pss[threadIdx.x] = (rpos && r < R) ? rpos[unit * R + r] : INT32_MAX;
    }
    __syncthreads();
    const int rows = min(kRowsStage, R - r0);
    for (int rr = 0; rr < rows; ++rr) {
      float x = __builtin_fmaf(dot_row(kr, qs[rr]), c2, kt);
      if (key > pss[rr]) x = -INFINITY;  // causal: the row does not see this key
      float mx = x;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      // every wave holds at least one valid key unless the whole wave is past n (or dead)
      float e = (mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x - mx);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) e += __shfl_xor(e, off);
      if (lane == 0) wred[wave][rr] = make_float2(mx, e);
    }
    __syncthreads();
    if (threadIdx.x < rows) {
      const int rr = threadIdx.x;
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) mm = fmaxf(mm, wred[w][rr].x);
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) {
        const float2 v = wred[w][rr];
        if (v.x != -INFINITY) sum += v.y * __builtin_amdgcn_exp2f(v.x - mm);
      }
      pout[r0 + rr] = make_float2(mm, sum);
    }
  }
}

int score_valu_tiles(int n) { return (n + kThreads - 1) / kThreads; }

#define KVC_VALU_DISPATCH_L(KERNEL, F, ...)                                                         \
  do {                                                                                            \
    if (layout == kPaged) {                                                                       \
      if (has_bias) KERNEL<F, kPaged, true><<<grid, block, 0, st>>>(__VA_ARGS__);                 \
      else KERNEL<F, kPaged, false><<<grid, block, 0, st>>>(__VA_ARGS__);                         \
    } else if (layout == kSlots) {                                                                \
      if (has_bias) KERNEL<F, kSlots, true><<<grid, block, 0, st>>>(__VA_ARGS__);                 \
      else KERNEL<F, kSlots, false><<<grid, block, 0, st>>>(__VA_ARGS__);                         \
    } else {                                                                                      \
      if (has_bias) KERNEL<F, kContig, true><<<grid, block, 0, st>>>(__VA_ARGS__);                \
      else KERNEL<F, kContig, false><<<grid, block, 0, st>>>(__VA_ARGS__);                        \
    }                                                                                             \
  } while (0)
#define KVC_VALU_DISPATCH(KERNEL, ...)                                                            \
  do {                                                                                          \
    if (f32) KVC_VALU_DISPATCH_L(KERNEL, true, __VA_ARGS__);                                    \
    else KVC_VALU_DISPATCH_L(KERNEL, false, __VA_ARGS__);                                       \
  } while (0)

hipError_t launch_score_valu(bool f32, int layout, bool has_bias, const void* q, const void* k, const int32_t* table,
                             int max_blocks, const float* lse, const float* bias, const int32_t* rpos, float* scores,
                             int H, int R, int64_t n_max, float scale, int pw, int dead, const SeqTable& T,
                             hipStream_t st) {
  dim3 grid(T.total), block(kThreads);
  KVC_VALU_DISPATCH(score_valu, q, k, table, max_blocks, lse, bias, rpos, scores, H, R, n_max, scale, pw, dead, T);
  return hipGetLastError();
}

hipError_t launch_lse_partials_valu(bool f32, int layout, bool has_bias, const void* q, const void* k,
                                    const int32_t* table, int max_blocks, const float* bias, const int32_t* rpos,
                                    float2* partials, int H, int R, int64_t n_max, float scale, int dead,
                                    const SeqTable& T, hipStream_t st) {
  dim3 grid(T.total), block(kThreads);
  KVC_VALU_DISPATCH(lse_partials_valu, q, k, table, max_blocks, bias, rpos, partials, H, R, n_max, scale, dead, T);
  return hipGetLastError();
}

}  // namespace kvc
