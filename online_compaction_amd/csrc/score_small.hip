// Token Eviction scoring of bf16 units with fewer than 16 proxy rows (boundary queries: one query
// per query head), on MFMA: the dot products of a key tile against the few rows are one
// v_mfma_f32_16x16x32_bf16 per 32 elements, with 16 keys as the M side and the rows (padded in
// effect to 16 columns) as the N side, so the vector ALU only applies the epilogue.
//
// Score equation of the design-space section of "Practical Online KV Cache Compaction for LLM
// Agents", with alpha recovered as exp(logit - LSE) as in the ActKV page's paged-memory paragraph.
//
// The pass is bound by reading the key rows, so they are read whole: a workgroup takes a chunk of
// kSmallChunk keys, each wave 64 consecutive keys, and every wave issues at once the 16 LDS-DMA
// loads (global_load_lds_dwordx4, 1 KB each: 4 key rows of 256 contiguous bytes) that bring its
// keys into a private LDS area, 16-byte chunks XOR-swizzled by row so that the MFMA operand reads
// that follow are free of bank conflicts. It then works through its 4 steps of 16 keys as the
// loads land (waiting for exactly the step's loads: no other vector-memory access is in flight
// meanwhile), with the proxy rows' operands, row positions, block-table entries and bias staged in
// LDS beforehand. After the 4 k-steps of a step, lane (g = lane / 16, c = lane % 16) holds the
// logits of keys 4g .. 4g+3 of the step for proxy row c; lanes with c < R carry the results.
//   small_lse_pass   per (unit, key chunk): every row's (max, sum 2^(y - max)) over the chunk ->
//                    partials, and (score calls) the logits, [H][R][keys] (16-byte stores after
//                    the last load has landed); valu_score_cached then forms the scores from them.
//   small_score_keys per (unit, key chunk): the score from a fresh pass over the key rows, with the
//                    LSE supplied or merged from the partials.
#include "few_rows.h"
#include "mfma_common.h"

namespace kvc {

using few::ChunkLds;

namespace {
constexpr int kThreads = few::kThreads;
constexpr int kWaveKeys = 64;                 // keys per wave: 4 steps of 16
constexpr int kSmallChunk = 4 * kWaveKeys;    // keys per workgroup

// Per-workgroup LDS: the chunk's table entries and bias, the proxy rows (16 rows, swizzled), the
// rows' positions and every wave's 64 key rows (swizzled).
struct SmallLds {
  ChunkLds chunk;
  uint8_t qs[16 * 256];
  int32_t pos[16];
  uint8_t ks[4][kWaveKeys * 256];
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() {
  if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else static_assert(N == 0, "unsupported count");
}
#pragma clang diagnostic pop

// Wait until at most 16 of this wave's vector-memory loads are outstanding, then a workgroup barrier.
__device__ __forceinline__ void vm_wait16_barrier() {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma clang diagnostic pop
}

// The wave's key rows kbeg + wave * 64 + [0, 64) (keys past kend load key kend - 1's row): 16
// LDS-DMA loads, 4 per step of 16 keys, issued in step order.
template <int LAYOUT>
__device__ __forceinline__ void issue_keys(SmallLds& S, const void* __restrict__ k, int H, int h, int64_t n_max,
                                           int64_t unit, int ko, int kbeg, int kend) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = 4 * (j & 3) + (lane >> 4);  // row within the step
    const int key = min(kbeg + wave * kWaveKeys + 16 * (j >> 2) + r, kend - 1);
    const u32x4* row = static_cast<const u32x4*>(few::chunk_key_row<false, LAYOUT>(k, S.chunk, H, h, n_max, unit, ko,
                                                                                  kbeg, key));
    mfma::dma16(row + ((lane & 15) ^ r), &S.ks[wave][j * 1024]);
  }
}

// Starts a workgroup's chunk [kbeg, kend): stages in LDS the proxy rows (rows past R repeat row
// R - 1; 16 rows, swizzled), their positions (rpos, or unused), the keys' bias (natural units, 0
// without bias) and, for paged keys and slot maps, the chunk's table entries or slots; then issues
// every wave's 16 key-row loads. On return the staged data is visible to every wave and exactly
// the 16 key-row loads of the wave are outstanding.
//   Contiguous keys: everything goes by LDS-DMA -- each wave loads 4 of the rows, the positions
//   and its 64 keys' bias, then its key rows -- and one wait for all but the last 16 loads plus a
//   barrier publishes the staging, so the key loads start without a round trip before them.
//   Paged keys and slot maps: the key addresses need the table, so the staging goes through
//   registers and a barrier first.
template <int LAYOUT>
__device__ __forceinline__ void begin_chunk(SmallLds& S, const uint16_t* __restrict__ q, const void* __restrict__ k,
                                            const int32_t* __restrict__ table, int max_blocks,
                                            const float* __restrict__ bias, const int32_t* __restrict__ rpos, int H,
                                            int h, int R, int64_t n_max, int s, int64_t unit, int ko, int kbeg,
                                            int kend) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if constexpr (LAYOUT == kContig) {
    const int r = 4 * wave + (lane >> 4);
    mfma::dma16(reinterpret_cast<const u32x4*>(q + (unit * R + min(r, R - 1)) * kHeadDim) + ((lane & 15) ^ r),
                &S.qs[4 * wave * 256]);
    // positions and bias come from a valid dummy address when absent (then they are not read)
    if (lane < 16)
      mfma::dma4(rpos ? reinterpret_cast<const float*>(rpos + unit * R + min(lane, R - 1)) : bias ? bias : reinterpret_cast<const float*>(q),
                 &S.pos[0]);
    const int key = min(kbeg + wave * kWaveKeys + lane, kend - 1);
    mfma::dma4(bias ? bias + (int64_t)s * n_max + key : reinterpret_cast<const float*>(q),
               &S.chunk.kts[wave * kWaveKeys]);
    issue_keys<LAYOUT>(S, k, H, h, n_max, unit, ko, kbeg, kend);
    vm_wait16_barrier();
  } else {
    few::stage_chunk<LAYOUT>(S.chunk, table, max_blocks, bias, n_max, s, unit, ko, kbeg, kend, 1.0f);
    const int row = t >> 4, ch = t & 15;  // (row, chunk) of the proxy rows
    const u32x4 v = reinterpret_cast<const u32x4*>(q + (unit * R + min(row, R - 1)) * kHeadDim)[ch];
    *reinterpret_cast<u32x4*>(&S.qs[mfma::swz(row, ch)]) = v;
    if (t < 16 && rpos) S.pos[t] = rpos[unit * R + min(t, R - 1)];
    __syncthreads();  // every staging load has landed (the compiler waits before the LDS stores)
    issue_keys<LAYOUT>(S, k, H, h, n_max, unit, ko, kbeg, kend);
  }
}

// Logits of step st (keys kbeg + wave * 64 + 16 st + 4g + e, e < 4) for the lane's row c, log2 units,
// -inf where masked; the caller has waited for the step's loads.
template <int LAYOUT>
__device__ __forceinline__ f32x4 step_logits(const SmallLds& S, const bf16x8 (&bq)[4], int st, int R, int kbeg,
                                             int kend, float c2, bool has_bias, int dead, int rp, int& key0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const uint8_t* kt = &S.ks[wave][st * 4096];
  f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = mfma::mfma16(*reinterpret_cast<const bf16x8*>(kt + mfma::swz(c, 4 * s + g)), bq[s], acc);
  key0 = kbeg + wave * kWaveKeys + 16 * st + 4 * g;
  f32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int key = key0 + e;
    bool valid = key < kend && c < R && key <= rp;
    if constexpr (LAYOUT == kSlots) valid = valid && S.chunk.idx[key - kbeg] != dead;
    const float b = has_bias ? kLog2e * S.chunk.kts[key - kbeg] : 0.0f;  // (unset without a bias)
    y[e] = valid ? __builtin_fmaf(acc[e], c2, b) : -INFINITY;
  }
  return y;
}

// The 4 steps of the wave, each after its loads have landed; epi(st, key0, y) per step.
template <int LAYOUT, class Epi>
__device__ __forceinline__ void small_steps(const SmallLds& S, const bf16x8 (&bq)[4], int R, int kbeg, int kend,
                                            float c2, bool has_bias, int dead, int rp, Epi&& epi) {
  int key0;
  vm_wait<12>();
  epi(0, key0, step_logits<LAYOUT>(S, bq, 0, R, kbeg, kend, c2, has_bias, dead, rp, key0));
  vm_wait<8>();
  epi(1, key0, step_logits<LAYOUT>(S, bq, 1, R, kbeg, kend, c2, has_bias, dead, rp, key0));
  vm_wait<4>();
  epi(2, key0, step_logits<LAYOUT>(S, bq, 2, R, kbeg, kend, c2, has_bias, dead, rp, key0));
  vm_wait<0>();
  epi(3, key0, step_logits<LAYOUT>(S, bq, 3, R, kbeg, kend, c2, has_bias, dead, rp, key0));
}
}  // namespace

// Work item = (sequence, KV head, chunk of kSmallChunk keys); the sequence's region of the
// workspace starts at ws + T.off[i] (float2 units): partials [H][nkc][R], then (cache) the logits
// [H][R][nkc * kSmallChunk].
template <int LAYOUT>
__global__ __launch_bounds__(kThreads) void small_lse_pass(const uint16_t* __restrict__ q, const void* __restrict__ k,
                                                           const int32_t* __restrict__ table, int max_blocks,
                                                           const float* __restrict__ bias,
                                                           const int32_t* __restrict__ rpos, float2* __restrict__ ws,
                                                           int cache, int H, int R, int64_t n_max, float scale,
                                                           int dead, SeqTable T) {
  __shared__ __attribute__((aligned(16))) SmallLds S;
  __shared__ float2 red[4][16];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int ko = T.kofs[i];
  const int nkc = (n + kSmallChunk - 1) / kSmallChunk;
  const int local = t - T.start[i];
  const int h = local / nkc;
  const int kc = local - h * nkc;
  const int64_t unit = (int64_t)s * H + h;
  const int kbeg = kc * kSmallChunk, kend = min(n, kbeg + kSmallChunk);

  begin_chunk<LAYOUT>(S, q, k, table, max_blocks, bias, rpos, H, h, R, n_max, s, unit, ko, kbeg, kend);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  bf16x8 bq[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) bq[st] = *reinterpret_cast<const bf16x8*>(&S.qs[mfma::swz(c, 4 * st + g)]);
  const int rp = rpos ? S.pos[c] : INT_MAX;

  float m = -INFINITY, sm = 0.0f;
  f32x4 ys[4];
  small_steps<LAYOUT>(S, bq, R, kbeg, kend, kLog2e * scale, bias != nullptr, dead, rp, [&](int st, int, const f32x4& y) {
    ys[st] = y;
    const float mm = fmaxf(fmaxf(m, fmaxf(y[0], y[1])), fmaxf(y[2], y[3]));
    if (mm > -INFINITY) {
      float acc = sm > 0.0f ? sm * __builtin_amdgcn_exp2f(m - mm) : 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (y[e] > -INFINITY) acc += __builtin_amdgcn_exp2f(y[e] - mm);
      sm = acc;
      m = mm;
    }
  });
  float2* region = ws + T.off[i];
  if (cache && c < R) {  // every load has landed: the stores do not mix into the waits above
    const int64_t npad = (int64_t)nkc * kSmallChunk;
    float* lrow = reinterpret_cast<float*>(region + valu_partials_float2(H, R, n, kSmallChunk)) +
                  ((int64_t)h * R + c) * npad + kbeg + wave * kWaveKeys + 4 * g;
#pragma unroll
    for (int st = 0; st < 4; ++st) *reinterpret_cast<f32x4*>(lrow + 16 * st) = ys[st];
  }
  // the four lane groups hold the same row for different keys: merge them, then the waves
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(sm, off);
    few::merge_ms(m, sm, m2, s2);
  }
  if (lane < 16) red[wave][lane] = make_float2(m, sm);
  __syncthreads();
  if ((int)threadIdx.x < R) {
    float mm = red[0][threadIdx.x].x, ss = red[0][threadIdx.x].y;
#pragma unroll
    for (int w = 1; w < 4; ++w) few::merge_ms(mm, ss, red[w][threadIdx.x].x, red[w][threadIdx.x].y);
    region[((int64_t)h * nkc + kc) * R + threadIdx.x] = make_float2(mm, ss);
  }
}

// Work item = (sequence, KV head, chunk of kSmallChunk keys). The LSE is supplied (lse), or merged
// from the chunk partials that small_lse_pass left at ws + T.off[i].
template <int LAYOUT>
__global__ __launch_bounds__(kThreads) void small_score_keys(const uint16_t* __restrict__ q, const void* __restrict__ k,
                                                             const int32_t* __restrict__ table, int max_blocks,
                                                             const float* __restrict__ lse,
                                                             const float2* __restrict__ ws,
                                                             const float* __restrict__ bias,
                                                             const int32_t* __restrict__ rpos,
                                                             float* __restrict__ out, int H, int R, int64_t n_max,
                                                             float scale, int pw, int dead, SeqTable T) {
  __shared__ __attribute__((aligned(16))) SmallLds S;
  __shared__ float sacc[kSmallChunk];
  __shared__ float nbs[16];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int ko = T.kofs[i];
  const int nch = (n + kSmallChunk - 1) / kSmallChunk;
  const int local = t - T.start[i];
  const int h = local / nch;
  const int kbeg = (local - h * nch) * kSmallChunk, kend = min(n, kbeg + kSmallChunk);
  const int64_t unit = (int64_t)s * H + h;
  const float2* parts = lse ? nullptr : ws + T.off[i] + (int64_t)h * nch * R;
  const float pwf = (float)pw;

  few::row_terms(lse, parts, nch, unit, R, 0, R, few::lanes_per_row(R), pwf, nbs);
  __syncthreads();  // the row terms' loads have landed before any key-row load is issued
  begin_chunk<LAYOUT>(S, q, k, table, max_blocks, bias, rpos, H, h, R, n_max, s, unit, ko, kbeg, kend);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  bf16x8 bq[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) bq[st] = *reinterpret_cast<const bf16x8*>(&S.qs[mfma::swz(c, 4 * st + g)]);
  const int rp = rpos ? S.pos[c] : INT_MAX;
  const float nb = c < R ? nbs[c] : 0.0f;
  small_steps<LAYOUT>(S, bq, R, kbeg, kend, kLog2e * scale, bias != nullptr, dead, rp, [&](int, int key0, const f32x4& y) {
    // sum over the rows: the 16 lanes c of a lane group hold the 16 rows of the same 4 keys
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = y[e] > -INFINITY ? __builtin_amdgcn_exp2f(__builtin_fmaf(y[e], pwf, nb)) : 0.0f;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off);
      if (c == 0) sacc[key0 + e - kbeg] = v;  // key0 + e < kbeg + kSmallChunk
    }
  });
  __syncthreads();
  for (int j = threadIdx.x; j < kend - kbeg; j += kThreads) out[unit * n_max + kbeg + j] = few::finish(sacc[j], R, pw);
}

// The key chunk of one workgroup (fixed).
int small_chunk() { return kSmallChunk; }

hipError_t launch_small_lse_pass(int layout, const void* q, const void* k, const int32_t* table, int max_blocks,
                                 const float* bias, const int32_t* rpos, float2* ws, bool cache, int H, int R,
                                 int64_t n_max, float scale, int dead, const SeqTable& T, hipStream_t st) {
  if (R > 16) return hipErrorInvalidValue;
  const auto* qq = static_cast<const uint16_t*>(q);
  dim3 grid(T.total), block(kThreads);
#define KVC_L(L) \
  small_lse_pass<L><<<grid, block, 0, st>>>(qq, k, table, max_blocks, bias, rpos, ws, cache ? 1 : 0, H, R, n_max, \
                                            scale, dead, T)
  if (layout == kPaged) KVC_L(kPaged);
  else if (layout == kSlots) KVC_L(kSlots);
  else KVC_L(kContig);
#undef KVC_L
  return hipGetLastError();
}

hipError_t launch_small_score_keys(int layout, const void* q, const void* k, const int32_t* table, int max_blocks,
                                   const float* lse, const float2* ws, const float* bias, const int32_t* rpos,
                                   float* out, int H, int R, int64_t n_max, float scale, int pw, int dead,
                                   const SeqTable& T, hipStream_t st) {
  if (R > 16) return hipErrorInvalidValue;
  const auto* qq = static_cast<const uint16_t*>(q);
  dim3 grid(T.total), block(kThreads);
#define KVC_S(L)                                                                                                   \
  small_score_keys<L><<<grid, block, 0, st>>>(qq, k, table, max_blocks, lse, ws, bias, rpos, out, H, R, n_max, scale, \
                                              pw, dead, T)
  if (layout == kPaged) KVC_S(kPaged);
  else if (layout == kSlots) KVC_S(kSlots);
  else KVC_S(kContig);
#undef KVC_S
  return hipGetLastError();
}

}  // namespace kvc
