// Token Eviction scoring of float32 inputs on the vector ALU, and the score pass from cached logits
// that the few-row paths share.
//
// Score equation of the design-space section of "Practical Online KV Cache Compaction for LLM
// Agents", with alpha recovered as exp(logit - LSE) as in the ActKV page's paged-memory paragraph.
//
// Key rows are read cooperatively: the 16 lanes of a lane group each load 32 bytes of a 512-byte
// float32 row (two 16-byte pieces, each wave-wide load covering 256 contiguous bytes per group).
// Each lane forms the partial dot products of its 8 elements with the 8 matching elements of every
// proxy row of its row block; a group handles KB keys against RB rows at once (KB * RB = 16), and a
// 4-stage reduce-scatter over the group's 16 lanes (DPP row permutes) leaves every lane with one
// finished logit -- (key kb, row r) for lane c = kb * RB + r -- so the exponentials and stores that
// follow run once per logit.
//
// Logits are kept in log2 units, y = log2(e) * (scale * q.k + bias), -inf where a key is masked
// (past the sequence, a dead slot, or after a causal row's position).
//   valu_lse_pass     per (unit, key chunk, row block): every row's (max, sum 2^(y - max)) over the
//                     chunk -> partials; with R <= 32 it also stores every logit (the "logit
//                     cache", R floats per key instead of a second pass over the key rows).
//   valu_score_keys   per (unit, key chunk): sum_r 2^(pw * y + 100 - pw * L2_r) from a fresh pass over
//                     the key rows, with the LSE supplied or merged from the partials; rows in
//                     blocks of RB.
//   valu_score_cached per (unit, 512 keys): each row's LSE from its partials (the combine is fused:
//                     every workgroup merges the few partials of its unit's rows itself), then the
//                     same sum from the cached logits -- for this file's pass and score_small.hip's.
// pw = 2 gives the TE score (square root of the mean, offset 2^50 removed), pw = 1 the attention mass.
#include "few_rows.h"

namespace kvc {

using namespace few;

namespace {
constexpr int kCachedKeys = 2;                       // keys per thread of valu_score_cached
constexpr int kCachedTile = kThreads * kCachedKeys;  // keys per workgroup of valu_score_cached

// DPP permutations within each 16-lane row of a wave
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]: lane i <-> i ^ 1
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]: lane i <-> i ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each half-row of 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Reduce-scatter of 16 values over the 16 lanes of a row: lane c returns the row-wide sum of v[c].
// Stage k pairs every lane with a partner whose lane bit (8, 4, 2, 1) differs; both form the pair
// sums of the two halves of their values and keep the half their bit selects.
__device__ __forceinline__ float reduce_scatter16(const float (&v)[16], int c) {
  float w8[8], w4[4], w2[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float a = v[j] + dpp<kDppMirror>(v[j]), b = v[j + 8] + dpp<kDppMirror>(v[j + 8]);
    w8[j] = (c & 8) ? b : a;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = w8[j] + dpp<kDppHalfMirror>(w8[j]), b = w8[j + 4] + dpp<kDppHalfMirror>(w8[j + 4]);
    w4[j] = (c & 4) ? b : a;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float a = w4[j] + dpp<kDppXor2>(w4[j]), b = w4[j + 2] + dpp<kDppXor2>(w4[j + 2]);
    w2[j] = (c & 2) ? b : a;
  }
  const float a = w2[0] + dpp<kDppXor1>(w2[0]), b = w2[1] + dpp<kDppXor1>(w2[1]);
  return (c & 1) ? b : a;
}

// Sum over the RB consecutive lanes c = kb * RB + r, r < RB (all of them get it).
template <int RB>
__device__ __forceinline__ float segment_sum(float x) {
  if constexpr (RB >= 2) x += dpp<kDppXor1>(x);
  if constexpr (RB >= 4) x += dpp<kDppXor2>(x);
  if constexpr (RB >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (RB >= 16) x += dpp<kDppMirror>(x);
  return x;
}

// A lane's 8 elements of a 128-element float32 row: elements 4c .. 4c+3 and 64+4c .. 64+4c+3.
struct Frag {
  f32x4 a, b;
};

__device__ __forceinline__ void load_frag(const void* __restrict__ row, int c, Frag& f) {
  const f32x4* p = static_cast<const f32x4*>(row);
  f.a = p[c];
  f.b = p[16 + c];
}

__device__ __forceinline__ float dot8(const Frag& k, const Frag& q) {
  float a = k.a[0] * q.a[0], b = k.b[0] * q.b[0];
#pragma unroll
  for (int e = 1; e < 4; ++e) {
    a = __builtin_fmaf(k.a[e], q.a[e], a);
    b = __builtin_fmaf(k.b[e], q.b[e], b);
  }
  return a + b;
}

// Key-row iterations a lane group keeps in flight: a ring of P iterations of fragments (at most 64
// registers of key data per lane, at most 4 iterations). valu_min_chunk (below) keeps every
// workgroup's chunk a multiple of P iterations.
template <int RB>
constexpr int prefetch_depth() {
  constexpr int regs = (16 / RB) * 8;
  return regs >= 64 ? 1 : (64 / regs > 4 ? 4 : 64 / regs);
}

// Sweep of keys [kbeg, kend) against rows [row0, row0 + RB): per iteration every lane group takes
// KB consecutive keys, with the key rows of the next P - 1 iterations already loading; epi(key, y)
// runs on every lane with the lane's logit y (log2 units; -inf when masked). The loop runs a
// multiple of P iterations and loads unconditionally (straight-line code, so the compiler waits for
// exactly the loads it uses): keys past kend load the row of key kend - 1 and come out masked, and
// iterations past the chunk's last skip the epilogue. Requires kend - kbeg <= the chunk length,
// a multiple of P * kIter.
template <int LAYOUT, int RB, class Epi>
__device__ __forceinline__ void sweep(const void* __restrict__ q, const void* __restrict__ k, const ChunkLds& L,
                                      const int32_t* __restrict__ rpos, int H, int h, int R, int row0,
                                      int64_t n_max, int64_t unit, int ko, int kbeg, int kend, float c2, int dead,
                                      Epi&& epi) {
  constexpr int KB = 16 / RB;
  constexpr int kIter = 16 * KB;  // keys per workgroup per iteration
  constexpr int P = prefetch_depth<RB>();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, c = lane & 15;
  const int my_kb = c / RB, my_r = c % RB;
  const int row = row0 + my_r;
  const int niter = (kend - kbeg + kIter - 1) / kIter;
  const int nrun = (niter + P - 1) / P * P;
  const int lane_base = wave * (4 * KB) + grp * KB;  // first key of the group, relative to an iteration

  // the rows (rows past R repeat row R - 1; their logits are masked) and the lane's row position
  Frag qf[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
    load_frag(static_cast<const float*>(q) + (unit * R + min(row0 + r, R - 1)) * kHeadDim, c, qf[r]);
  const int rp = rpos ? rpos[unit * R + min(row, R - 1)] : INT_MAX;

  Frag buf[P][KB];
  auto load_keys = [&](int it, Frag (&f)[KB]) {
    const int key0 = kbeg + it * kIter + lane_base;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      load_frag(chunk_key_row<true, LAYOUT>(k, L, H, h, n_max, unit, ko, kbeg, min(key0 + kb, kend - 1)), c, f[kb]);
  };
  auto step = [&](int it, const Frag (&f)[KB]) {
    float v[16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < RB; ++r) v[kb * RB + r] = dot8(f[kb], qf[r]);
    const float d = reduce_scatter16(v, c);
    if (it < niter) {  // uniform
      const int key = kbeg + it * kIter + lane_base + my_kb;
      bool valid = key < kend && row < R && key <= rp;
      if constexpr (LAYOUT == kSlots) valid = valid && L.idx[key - kbeg] != dead;
      const float y = valid ? __builtin_fmaf(d, c2, L.kts[key - kbeg]) : -INFINITY;
      epi(key, y);
    }
  };
#pragma unroll
  for (int p = 0; p < P; ++p) load_keys(p, buf[p]);
  int it0 = 0;
  for (; it0 + P < nrun; it0 += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      step(it0 + p, buf[p]);
      load_keys(it0 + p + P, buf[p]);
    }
  }
#pragma unroll
  for (int p = 0; p < P; ++p) step(it0 + p, buf[p]);
}
}  // namespace

// Work item = (sequence, KV head, key chunk, row block); the sequence's region of the workspace
// starts at ws + T.off[i] (float2 units): partials [H][nkc][R], then (cache) the logits
// [H][R][nkc * kchunk] (float32, log2 units; -inf where masked).
template <int LAYOUT, int RB>
__global__ __launch_bounds__(kThreads) void valu_lse_pass(const void* __restrict__ q, const void* __restrict__ k,
                                                          const int32_t* __restrict__ table, int max_blocks,
                                                          const float* __restrict__ bias,
                                                          const int32_t* __restrict__ rpos, float2* __restrict__ ws,
                                                          int cache, int H, int R, int64_t n_max, float scale,
                                                          int kchunk, int dead, SeqTable T) {
  __shared__ ChunkLds L;
  __shared__ float2 red[4][RB];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int ko = T.kofs[i];
  const int nkc = (n + kchunk - 1) / kchunk;
  const int nrb = (R + RB - 1) / RB;
  int local = t - T.start[i];
  const int h = local / (nkc * nrb);
  local -= h * nkc * nrb;
  const int kc = local / nrb;
  const int rb = local - kc * nrb;
  const int64_t unit = (int64_t)s * H + h;
  const int kbeg = kc * kchunk, kend = min(n, kbeg + kchunk);

  stage_chunk<LAYOUT>(L, table, max_blocks, bias, n_max, s, unit, ko, kbeg, kend);
  __syncthreads();

  float2* region = ws + T.off[i];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int my_r = (lane & 15) % RB;
  const int row = rb * RB + my_r;
  const int64_t npad = (int64_t)nkc * kchunk;
  float* lrow = (cache && row < R)
                    ? reinterpret_cast<float*>(region + valu_partials_float2(H, R, n, kchunk)) + ((int64_t)h * R + row) * npad
                    : nullptr;
  float m = -INFINITY, sm = 0.0f;
  sweep<LAYOUT, RB>(q, k, L, rpos, H, h, R, rb * RB, n_max, unit, ko, kbeg, kend, kLog2e * scale, dead,
                    [&](int key, float y) {
                      if (lrow) lrow[key] = y;  // key < kbeg + kchunk <= npad
                      if (y > -INFINITY) {
                        const float mm = fmaxf(m, y);
                        sm = (sm > 0.0f ? sm * __builtin_amdgcn_exp2f(m - mm) : 0.0f) + __builtin_amdgcn_exp2f(y - mm);
                        m = mm;
                      }
                    });
  // lanes holding the same row: merge over the key bits of the group, then the groups, then the waves
#pragma unroll
  for (int off = RB; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(sm, off);
    merge_ms(m, sm, m2, s2);
  }
  if (lane < RB) red[wave][lane] = make_float2(m, sm);
  __syncthreads();
  if (threadIdx.x < RB && rb * RB + (int)threadIdx.x < R) {
    float mm = red[0][threadIdx.x].x, ss = red[0][threadIdx.x].y;
#pragma unroll
    for (int w = 1; w < 4; ++w) merge_ms(mm, ss, red[w][threadIdx.x].x, red[w][threadIdx.x].y);
    region[((int64_t)h * nkc + kc) * R + rb * RB + threadIdx.x] = make_float2(mm, ss);
  }
}

// Work item = (sequence, KV head, kCachedTile keys): thread t takes keys t + kThreads * j,
// j < kCachedKeys, their cached logits (layout [H][R][nkc * kchunk] after the partials) loaded
// before the row terms are merged. RC = R rounded up to a power of two (at most
// kValuMaxCacheRows); rows R .. RC - 1 load row R - 1 and are not summed, so every load is
// unconditional.
template <int RC>
__global__ __launch_bounds__(kThreads) void valu_score_cached(const float2* __restrict__ ws, float* __restrict__ out,
                                                              int H, int R, int64_t n_max, int kchunk, int pw,
                                                              SeqTable T) {
  __shared__ float nbs[kValuMaxCacheRows];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int tiles = (n + kCachedTile - 1) / kCachedTile;
  const int local = t - T.start[i];
  const int h = local / tiles;
  const int key0 = (local - h * tiles) * kCachedTile + threadIdx.x;
  const int64_t unit = (int64_t)s * H + h;
  const int nkc = (n + kchunk - 1) / kchunk;
  const int64_t npad = (int64_t)nkc * kchunk;
  const float2* region = ws + T.off[i];
  const float* logits =
      reinterpret_cast<const float*>(region + valu_partials_float2(H, R, n, kchunk)) + (int64_t)h * R * npad;
  // every key's cached logits first (independent of the row terms); keys past n read key n - 1's
  // and are not written
  float y[kCachedKeys][RC];
#pragma unroll
  for (int j = 0; j < kCachedKeys; ++j) {
    const int key = min(key0 + j * kThreads, n - 1);
#pragma unroll
    for (int r = 0; r < RC; ++r) y[j][r] = logits[(int64_t)min(r, R - 1) * npad + key];
  }
  row_terms(nullptr, region + (int64_t)h * nkc * R, nkc, unit, R, 0, R, lanes_per_row(R), (float)pw, nbs);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kCachedKeys; ++j) {
    float acc = 0.0f;
#pragma unroll
    for (int r = 0; r < RC; ++r)
      if (r < R && y[j][r] > -INFINITY) acc += __builtin_amdgcn_exp2f(__builtin_fmaf(y[j][r], (float)pw, nbs[r]));
    const int key = key0 + j * kThreads;
    if (key < n) out[unit * n_max + key] = finish(acc, R, pw);
  }
}

// Work item = (sequence, KV head, key chunk). The LSE is supplied (lse), or merged from the chunk
// partials that valu_lse_pass left at ws + T.off[i] (chunks of lse_kchunk keys).
template <int LAYOUT, int RB>
__global__ __launch_bounds__(kThreads) void valu_score_keys(const void* __restrict__ q, const void* __restrict__ k,
                                                            const int32_t* __restrict__ table, int max_blocks,
                                                            const float* __restrict__ lse,
                                                            const float2* __restrict__ ws,
                                                            const float* __restrict__ bias,
                                                            const int32_t* __restrict__ rpos, float* __restrict__ out,
                                                            int H, int R, int64_t n_max, float scale, int pw,
                                                            int lse_kchunk, int chunk, int dead, SeqTable T) {
  __shared__ ChunkLds L;
  __shared__ float sacc[kMaxChunk];
  __shared__ float nbs[RB];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int ko = T.kofs[i];
  const int nch = (n + chunk - 1) / chunk;
  const int local = t - T.start[i];
  const int h = local / nch;
  const int kbeg = (local - h * nch) * chunk, kend = min(n, kbeg + chunk);
  const int64_t unit = (int64_t)s * H + h;
  const int nkc = lse ? 0 : (n + lse_kchunk - 1) / lse_kchunk;
  const float2* parts = lse ? nullptr : ws + T.off[i] + (int64_t)h * nkc * R;

  stage_chunk<LAYOUT>(L, table, max_blocks, bias, n_max, s, unit, ko, kbeg, kend);
  for (int j = threadIdx.x; j < kend - kbeg; j += kThreads) sacc[j] = 0.0f;
  const int my_r = (threadIdx.x & 15) % RB;
  const float pwf = (float)pw;
  for (int row0 = 0; row0 < R; row0 += RB) {
    row_terms(lse, parts, nkc, unit, R, row0, RB, lanes_per_row(RB), pwf, nbs);
    __syncthreads();  // (also publishes the staged chunk and the cleared sums on the first block)
    const float nb = nbs[my_r];
    sweep<LAYOUT, RB>(q, k, L, rpos, H, h, R, row0, n_max, unit, ko, kbeg, kend, kLog2e * scale, dead,
                      [&](int key, float y) {
                        float e = y > -INFINITY ? __builtin_amdgcn_exp2f(__builtin_fmaf(y, pwf, nb)) : 0.0f;
                        e = segment_sum<RB>(e);
                        if (my_r == 0 && key < kend) sacc[key - kbeg] += e;
                      });
    __syncthreads();
  }
  for (int j = threadIdx.x; j < kend - kbeg; j += kThreads) out[unit * n_max + kbeg + j] = finish(sacc[j], R, pw);
}

int valu_row_block(int R) { return R <= 1 ? 1 : R <= 2 ? 2 : R <= 4 ? 4 : R <= 8 ? 8 : 16; }
int valu_cached_tiles(int n) { return (n + kCachedTile - 1) / kCachedTile; }

// Shortest key chunk of a float32 workgroup: P iterations of 256 / RB keys, at least 64 keys.
int valu_min_chunk_f32(int R) {
  int p = 1;
  switch (valu_row_block(R)) {
    case 1: p = prefetch_depth<1>(); break;
    case 2: p = prefetch_depth<2>(); break;
    case 4: p = prefetch_depth<4>(); break;
    case 8: p = prefetch_depth<8>(); break;
    default: p = prefetch_depth<16>(); break;
  }
  const int c = p * (256 / valu_row_block(R));
  return c < 64 ? 64 : c;
}

#define KVC_VALU_LAYOUT(K, RBV, ...)                                        \
  do {                                                                     \
    if (layout == kPaged) K<kPaged, RBV><<<grid, block, 0, st>>>(__VA_ARGS__); \
    else if (layout == kSlots) K<kSlots, RBV><<<grid, block, 0, st>>>(__VA_ARGS__); \
    else K<kContig, RBV><<<grid, block, 0, st>>>(__VA_ARGS__);            \
  } while (0)
#define KVC_VALU_RB(K, ...)                                   \
  switch (valu_row_block(R)) {                                \
    case 1: KVC_VALU_LAYOUT(K, 1, __VA_ARGS__); break;        \
    case 2: KVC_VALU_LAYOUT(K, 2, __VA_ARGS__); break;        \
    case 4: KVC_VALU_LAYOUT(K, 4, __VA_ARGS__); break;        \
    case 8: KVC_VALU_LAYOUT(K, 8, __VA_ARGS__); break;        \
    default: KVC_VALU_LAYOUT(K, 16, __VA_ARGS__); break;      \
  }

hipError_t launch_valu_lse_pass(int layout, const void* q, const void* k, const int32_t* table, int max_blocks,
                                const float* bias, const int32_t* rpos, float2* ws, bool cache, int H, int R,
                                int64_t n_max, float scale, int kchunk, int dead, const SeqTable& T, hipStream_t st) {
  dim3 grid(T.total), block(kThreads);
  KVC_VALU_RB(valu_lse_pass, q, k, table, max_blocks, bias, rpos, ws, cache ? 1 : 0, H, R, n_max, scale, kchunk, dead,
              T)
  return hipGetLastError();
}

hipError_t launch_valu_score_cached(const float2* ws, float* out, int H, int R, int64_t n_max, int kchunk, int pw,
                                    const SeqTable& T, hipStream_t st) {
  dim3 grid(T.total), block(kThreads);
#define KVC_C(RC) valu_score_cached<RC><<<grid, block, 0, st>>>(ws, out, H, R, n_max, kchunk, pw, T)
  if (R <= 1) KVC_C(1);
  else if (R <= 2) KVC_C(2);
  else if (R <= 4) KVC_C(4);
  else if (R <= 8) KVC_C(8);
  else if (R <= 16) KVC_C(16);
  else if (R <= kValuMaxCacheRows) KVC_C(32);
  else return hipErrorInvalidValue;
#undef KVC_C
  return hipGetLastError();
}

hipError_t launch_valu_score_keys(int layout, const void* q, const void* k, const int32_t* table, int max_blocks,
                                  const float* lse, const float2* ws, const float* bias, const int32_t* rpos,
                                  float* out, int H, int R, int64_t n_max, float scale, int pw, int lse_kchunk,
                                  int chunk, int dead, const SeqTable& T, hipStream_t st) {
  dim3 grid(T.total), block(kThreads);
  KVC_VALU_RB(valu_score_keys, q, k, table, max_blocks, lse, ws, bias, rpos, out, H, R, n_max, scale, pw, lse_kchunk,
              chunk, dead, T)
  return hipGetLastError();
}

#undef KVC_VALU_RB
#undef KVC_VALU_LAYOUT

}  // namespace kvc
