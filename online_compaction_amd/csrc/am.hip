// Attention Matching ("Practical Online KV Cache Compaction for LLM Agents", design-space
// section, the AM equations): after the top-m keys K_C are chosen, an additive bias beta with
//   min_beta || exp(Q K_C^T + beta) 1_m - exp(Q K^T) 1_n ||^2
// and compact values V_C with
//   min_V_C || A_hat(Q; K_C, beta, V_C) - A(Q; K, V) ||_F^2.
// With w = exp(beta) the first is non-negative least squares in w; the second, with
// P_C = diag(1 / (E w)) E diag(w) the compacted attention, is least squares in V_C.
//
// Per unit, with E_ij = exp(c q_i . k_Cj - ME) (ME the largest kept logit) and the target
// A(Q; K, V) = P_full V, P_full_ij = exp(c q_i . k_j - LSE_i) over all n keys:
//   beta: w' <- w' * (E^T z) / (E^T E w') (multiplicative NNLS updates), z_i = exp(LSE_i - Mz);
//   V_C:  V <- V - eta P_C^T (P_C V - Y) from the kept keys' values (Landweber),
//         eta = 1 / max_j sum_i (P_C)_ij.
// E is never stored: every pass that needs it re-forms its tiles from the bf16 rows of Q and of
// the gathered kept keys on the MFMA units (am_bias), which costs less than reading 4 bytes per
// entry back from memory; P_full exists only one 64-key chunk at a time (am_target). P_C and
// P_C^T are written once, as split rows, when beta is fixed. The Landweber steps run as the
// equivalent iteration of the residual on the smaller side of P_C with its Gram matrix (am_gram,
// then one product per step). E and z carry separate factors so that neither underflows in
// float32 (Mz = the largest LSE, lowered to ME + 80 if the kept logits lie far below it). The
// updates are scale-equivariant: with w' = exp(ME - Mz) w they are the updates of w = exp(beta)
// from w = 1 on the unscaled exponentials, so w' starts at exp(ME - Mz) and
// beta = log w' - (ME - Mz).
// The QK^T products use v_mfma_f32_16x16x32_bf16 on the stored bf16 rows; the solver's matrix
// products run on the same instruction with their float32 operands stored split into bf16 high
// and low parts (three products each). Every reduction has a fixed order (partial sums land in
// buffers that one pass adds up in order), so a fit is reproducible bit for bit.
//
// Workspace of sequence i (floats, from T.off[i]; H heads, R rows, m = T.m[i], Rp = R and
// ldm = m rounded up to 64, NR = ceil(R / 64), S1 / S2 the split counts of the two P_C products,
// St that of the target's keys,
// Np the padded rows of the iteration's side (Rp or ldm); every array starts on a 256-byte
// boundary):
//   P [H][R128][ldm] | PT [H][L128][Rp] | Y [St][H][R][128] | ZT [H][128][Rp] | VT [H][128][ldm] |
//   Zp [S1 > 1 ? S1 : 0][H][R][128] | Up [S2 > 1 ? S2 : 0][H][ldm][128] | part [H][NR][ldm] |
//   b [H][ldm] | Mz [H] | eta [H] | ME [H] | ME as an ordered integer key [H] | Mg [H][Np][Np] |
//   X, Sx [H][Np][128] | XT1 [H][128][Np] |
//   KC [H][ldk][128] bf16 (ldk = m rounded up to 256)
// (R128 and L128: R and ldm rounded up to 128; P and PT are held in the blocked split layout.)
// Columns m .. ldm-1 of P_C hold zeros, so tiles never need a column bound on it.
#include <type_traits>

#include "am_cfg.h"
#include "mfma_common.h"

namespace kvc {

using namespace mfma;

namespace {

constexpr int kD = kHeadDim;
constexpr int kRowChunk = 64;  // rows per partial column sum

__host__ __device__ constexpr int64_t pad64(int64_t x) { return (x + 63) & ~int64_t(63); }
__host__ __device__ constexpr int64_t pad128(int64_t x) { return (x + 127) & ~int64_t(127); }
__host__ __device__ constexpr int64_t pad256(int64_t x) { return (x + 255) & ~int64_t(255); }

// E / P_C [H][R][ldm], PT [H][ldm][Rp], ZT [H][128][Rp] and VT [H][128][ldm] (Rp = R rounded up
// to 64): P_C, PT, ZT and VT are held in the split layout below. The value iteration's side
// (am_rows_side) has N rows (R, or m) padded to Np (Rp, or ldm): its Gram matrix Mg [H][Np][Np]
// (split), the iterate X and its running sum Sx [H][Np][128] (float32), and a second buffer XT1
// [H][128][Np] (split) for the iterate's transpose, which alternates with ZT (rows side) or VT
// (keys side) from step to step so that no product rewrites the operand it reads.
struct AmWs {
  float *P, *PT, *Y, *ZT, *VT, *Zp, *Up, *part, *b, *M, *eta, *ME;
  float *Mg, *X, *Sx, *XT1;
  uint16_t* KC;  // the kept keys' rows, gathered: [H][ldk][128] bf16 (ldk = m rounded up to 256), zero rows from m
  uint32_t* mekey;
  int ldm, Rp, N, Np, ldk;
  bool rside;
};
// the iterate's transpose: buffer 0 (ZT or VT) or XT1 (by value, so that the workspace
// description stays in registers)
__device__ __forceinline__ float* am_xt(float* xt1, float* zt, float* vt, bool rside, int sel) {
  return sel ? xt1 : (rside ? zt : vt);
}

// The split layout of a float32 matrix row: each group of 8 consecutive elements keeps its 32
// bytes, as the 8 bfloat16 high parts followed by the 8 bfloat16 low parts (hi = bf16(x),
// lo = bf16(x - hi), so hi + lo carries x to a relative 2^-16). A matrix converts in place, and
// the 16-byte halves load straight into the bf16 MFMA operand tiles of the split products.
__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
  bf16x8 h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 b = (__bf16)x[e];
    h[e] = b;
    l[e] = (__bf16)(x[e] - (float)b);
  }
  hi = __builtin_bit_cast(u32x4, h);
  lo = __builtin_bit_cast(u32x4, l);
}
// group g of a split row (8 elements, 32 bytes) from 8 floats
__device__ __forceinline__ void put_split8(float* row, int g, const float* x) {
  u32x4 hi, lo;
  split8(x, hi, lo);
  u32x4* d = reinterpret_cast<u32x4*>(row + 8 * g);
  d[0] = hi;
  d[1] = lo;
}
// The blocked split layout of P_C and P_C^T, as the tile products (ring_mma) read them: per
// 128-row block and 32-column stage a 16 KB block of 128 rows x 128 bytes (the four 8-column
// groups of the split layout, high half then low half), 16-byte chunk c of row r at position
// c ^ step_sw(r) (the low three bits of r with bits 0 and 1 swapped: the bank-conflict-free
// placement of the products' LDS ring); blocks stage-major within a row block, so a row block
// of a matrix with ncols columns spans 128 ncols floats (rows past the last live row of the last
// block are never written and never reach a kept product).
__device__ __forceinline__ int step_sw(int r) { return ((r & 1) << 1) | ((r >> 1) & 1) | (r & 4); }
__device__ __forceinline__ void blk_put8(float* base, int ncols, int r, int c, const float* x) {
  u32x4 hi, lo;
  split8(x, hi, lo);
  const int row = r & 127, grp = (c & 31) >> 3, sw = step_sw(row);
  uint8_t* blk = reinterpret_cast<uint8_t*>(base) + (((int64_t)(r >> 7) * (ncols >> 5) + (c >> 5)) << 14) + row * 128;
  *reinterpret_cast<u32x4*>(blk + (((2 * grp) ^ sw) << 4)) = hi;
  *reinterpret_cast<u32x4*>(blk + (((2 * grp + 1) ^ sw) << 4)) = lo;
}
// element k of a split row
__device__ __forceinline__ void put_split1(float* row, int k, float x) {
  uint16_t* d = reinterpret_cast<uint16_t*>(row + 8 * (k >> 3));
  const __bf16 b = (__bf16)x;
  d[k & 7] = __builtin_bit_cast(uint16_t, b);
  d[8 + (k & 7)] = __builtin_bit_cast(uint16_t, (__bf16)(x - (float)b));
}

__device__ __forceinline__ AmWs am_ws(float* ws, const SeqTable& T, int i, const AmCfg& C) {
  const int64_t m = T.m[i], H = C.H, R = C.R;
  const int64_t ldm = pad64(m), nr = (R + kRowChunk - 1) / kRowChunk, Rp = pad64(R);
  AmWs w;
  w.ldm = (int)ldm;
  w.Rp = (int)Rp;
  w.rside = am_rows_side((int)R, (int)m);
  w.N = w.rside ? (int)R : (int)m;
  w.Np = w.rside ? (int)Rp : (int)ldm;
  const int64_t Np = w.Np;
  w.P = ws + T.off[i];
  w.PT = w.P + pad64(H * pad128(R) * ldm);
  w.Y = w.PT + pad64(H * pad128(ldm) * Rp);
  w.ZT = w.Y + C.St * pad64(H * R * kD);
  w.VT = w.ZT + pad64(H * kD * Rp);
  w.Zp = w.VT + pad64(H * kD * ldm);
  w.Up = w.Zp + (C.S1 > 1 ? C.S1 : 0) * pad64(H * R * kD);
  w.part = w.Up + (C.S2 > 1 ? C.S2 : 0) * pad64(H * ldm * kD);
  w.b = w.part + pad64(H * nr * ldm);
  w.M = w.b + pad64(H * ldm);
  w.eta = w.M + H;
  w.ME = w.eta + H;
  w.mekey = reinterpret_cast<uint32_t*>(w.ME + H);
  w.Mg = w.M + pad64(4 * H);
  w.X = w.Mg + pad64(H * Np * Np);
  w.Sx = w.X + pad64(H * Np * kD);
  w.XT1 = w.Sx + pad64(H * Np * kD);
  w.ldk = (int)pad256(m);
  w.KC = reinterpret_cast<uint16_t*>(w.XT1 + pad64(H * kD * Np));
  return w;
}

// Unsigned key that orders like the float (for an atomic maximum of signed floats).
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

}  // namespace

// Floats of one sequence's workspace (the layout above).
int64_t am_seq_floats(int H, int R, int n, int m, int S1, int S2, int St) {
  (void)n;
  const int64_t ldm = pad64(m), nr = (R + kRowChunk - 1) / kRowChunk, Rp = pad64(R);
  const int64_t Np = am_rows_side(R, m) ? Rp : ldm;
  const int64_t rk = pad64((int64_t)H * R * kD), xk = pad64((int64_t)H * Np * kD);
  return pad64((int64_t)H * pad128(R) * ldm) + pad64((int64_t)H * pad128(ldm) * Rp) + St * rk +
         pad64((int64_t)H * kD * Rp) +
         pad64((int64_t)H * kD * ldm) + (S1 > 1 ? S1 : 0) * rk +
         (S2 > 1 ? S2 : 0) * pad64((int64_t)H * ldm * kD) + pad64((int64_t)H * nr * ldm) +
         pad64((int64_t)H * ldm) + pad64(4 * (int64_t)H) + pad64((int64_t)H * Np * Np) + 3 * xk + pad64((int64_t)H * pad256(m) * (kD / 2));
}

// Per unit, first: Mz = max_i LSE_i, and the kept-logit maximum reset. Work item = (seq, head).
__global__ __launch_bounds__(64) void am_stats(const float* __restrict__ lse, float* __restrict__ ws, AmCfg C,
                                               SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int s = T.first + i, h = t - T.start[i];
  AmWs W = am_ws(ws, T, i, C);
  const float* lu = lse + ((int64_t)s * C.H + h) * C.R;
  float mx = -INFINITY;
  for (int r = threadIdx.x; r < C.R; r += 64) mx = fmaxf(mx, lu[r]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (threadIdx.x == 0) {
    W.M[h] = mx;
    W.mekey[h] = 0u;  // below every float's key
  }
}

// Per unit, after the kept-logit maximum: ME, and Mz lowered to ME + 80 when the kept keys lie
// far below the largest LSE (so that exp(ME - Mz), the start of w', stays in range).
// Work item = (seq, head).
__global__ __launch_bounds__(64) void am_me(float* __restrict__ ws, AmCfg C, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int h = t - T.start[i];
  AmWs W = am_ws(ws, T, i, C);
  if (threadIdx.x == 0) {
    const float me = key_float(W.mekey[h]);
    W.ME[h] = me;
    W.M[h] = fminf(W.M[h], me + 80.0f);
  }
}

// ------------------------------------------------------------------------------------------------
// Column sums g_j = sum_i part_ij over the 64-row tiles, in tile order, then per kept key:
//   MODE 0: b_j = g_j (E^T z once; or the column sums of P_C, for the step size)
//   MODE 1: w_j <- w_j b_j / g_j, 0 if g_j = 0 (one NNLS step)
// Work item = (seq, head, 256 kept keys).
// ------------------------------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void am_cols_fin(float* __restrict__ w_all, float* __restrict__ ws, AmCfg C,
                                                   SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  AmWs W = am_ws(ws, T, i, C);
  const int ldm = W.ldm;
  const int cb_n = (m + 255) / 256, nr = (C.R + kRowChunk - 1) / kRowChunk;
  const int local = t - T.start[i];
  const int h = local / cb_n;
  const int j = (local - h * cb_n) * 256 + threadIdx.x;
  if (j >= m) return;
  const float* p = W.part + (int64_t)h * nr * ldm + j;
  float g = 0.0f;
  int rc = 0;
  for (; rc + 8 <= nr; rc += 8) {  // eight loads in flight, added in order
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = p[(int64_t)(rc + k) * ldm];
#pragma unroll
    for (int k = 0; k < 8; ++k) g += x[k];
  }
  for (; rc < nr; ++rc) g += p[(int64_t)rc * ldm];
  float* b = W.b + (int64_t)h * ldm + j;
  if constexpr (MODE == 1) {
    float* w = w_all + ((int64_t)s * C.H + h) * C.m_max + j;
    *w = g > 0.0f ? *w * *b / g : 0.0f;
  } else {
    *b = g;
  }
}

// eta = 1 / max_j (column sums of P_C) per unit (0 when every column is empty). Work item = (seq, head).
__global__ __launch_bounds__(256) void am_eta(float* __restrict__ ws, AmCfg C, SeqTable T) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i];
  const int h = t - T.start[i];
  AmWs W = am_ws(ws, T, i, C);
  float mx = 0.0f;
  for (int j = threadIdx.x; j < m; j += 256) mx = fmaxf(mx, W.b[(int64_t)h * W.ldm + j]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float c = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    W.eta[h] = c > 0.0f ? 1.0f / c : 0.0f;
  }
}

// ------------------------------------------------------------------------------------------------
// The kept keys' rows gathered into KC (zero rows from m up to ldk), the operand from which the
// bias updates re-form E. Work item = (seq, head, 64 rows of KC).
// ------------------------------------------------------------------------------------------------
template <int LAYOUT>
__global__ __launch_bounds__(256) void am_gather(const uint16_t* __restrict__ k, const int32_t* __restrict__ table,
                                                 int max_blocks, const int32_t* __restrict__ kept,
                                                 float* __restrict__ ws, int64_t n_max, AmCfg C, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], n = T.n[i], s = T.first + i;
  AmWs W = am_ws(ws, T, i, C);
  const int nb = W.ldk / 64;
  const int local = t - T.start[i];
  const int h = local / nb, blk = local - h * nb;
  const int64_t unit = (int64_t)s * C.H + h;
  const int32_t* map = LAYOUT == kPaged ? table + (int64_t)s * max_blocks
                                        : (LAYOUT == kSlots ? table + unit * n_max : nullptr);
  u32x4* dst = reinterpret_cast<u32x4*>(W.KC + ((int64_t)h * W.ldk + blk * 64) * kD);
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int q = x * 256 + threadIdx.x, j = blk * 64 + (q >> 4), ch = q & 15;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (j < m) {
      const int key = min(max(kept[unit * C.m_max + j], 0), n - 1);
      v = key_row<LAYOUT>(k, map, C.H, h, n_max, unit, T.kofs[i] + key)[ch];
    }
    dst[q] = v;
  }
}

// ------------------------------------------------------------------------------------------------
// Everything the fit needs from E_ij = exp(c q_i . k_Cj - ME), re-formed on the MFMA units from the
// bf16 rows of Q and KC instead of kept in memory, per 64-row tile:
//   MODE 3: the kept logits' maximum ME (one atomic per workgroup)
//   MODE 0: b_j = sum_i E_ij z_i, z_i = exp(LSE_i - Mz)               (column partials)
//   MODE 1: u_i = sum_j E_ij w_j, then the column partials of E^T u      (one NNLS update)
//   MODE 2: u_i as in MODE 1, then P_C = E_ij w_j / u_i written as split rows of P_C and of
//           P_C^T (zeros past R and past m), with the column partials of P_C
// Column partials land one per 64-row tile and kept key, the layout am_cols_fin reads (it adds
// them in order and applies the update).
// Work item = (seq, head, 64-row tile); eight waves, two per SIMD: wave w holds rows
// 32 (w & 1) .. + 31 of the tile (two 16-row fragments of Q in registers) and takes key tiles
// 4 st + (w >> 1) of KC. Each step stages four consecutive 64-key tiles (64 KB, rows swizzled as in
// the score kernels) and their w through double-buffered LDS. Per 16-key slice a B fragment
// serves both row fragments. The row sums meet across the four key quarters in LDS, in order; a
// key's column partial is reduced over the wave's lane groups, then over the two waves of its
// quarter through LDS (even wave first).
// ------------------------------------------------------------------------------------------------
namespace {
constexpr int kBiasThreads = 512;
constexpr int kBiasStep = 256;  // kept keys per step (KC rows are padded to a multiple)
}  // namespace

template <int MODE>
__global__ __launch_bounds__(kBiasThreads) void am_bias(const uint16_t* __restrict__ q,
                                                        const float* __restrict__ w_all,
                                                        const float* __restrict__ lse, float* __restrict__ ws,
                                                        float scale, AmCfg C, SeqTable T) {
  constexpr bool kW = MODE == 1 || MODE == 2;  // the pass needs w
  __shared__ __attribute__((aligned(16))) uint8_t Ks[2][kBiasStep * 256];
  __shared__ __attribute__((aligned(16))) float ws_l[2][kBiasStep];  // w of the step's keys
  __shared__ float rsum[4][64];          // row sums of the four key quarters
  __shared__ float xpart[2][2][kBiasStep];  // column partials per step parity and wave parity
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  const int H = C.H, R = C.R;
  const int rt_n = (R + 63) / 64;
  const int local = t - T.start[i];
  const int h = local / rt_n, rt = local - h * rt_n;
  const int64_t unit = (int64_t)s * H + h;
  AmWs W = am_ws(ws, T, i, C);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int rb = 32 * (wave & 1), kq = wave >> 1;
  const float cl = scale * kLog2e, mb = MODE == 3 ? 0.0f : W.ME[h] * kLog2e;
  const float* wu = w_all + unit * C.m_max;
  const u32x4* kc = reinterpret_cast<const u32x4*>(W.KC + (int64_t)h * W.ldk * kD);
  const int nsteps = W.ldk / kBiasStep;

  bf16x8 qa[2][4];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int row = min(rt * 64 + rb + 16 * rg + c16, R - 1);
    const u32x4* qr = reinterpret_cast<const u32x4*>(q + (unit * R + row) * (int64_t)kD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[rg][ks] = as_bf16x8(qr[4 * ks + g]);
  }

  // Staging of key rows 256 st .. + 255 into buffer buf by LDS-DMA: wave w lands the 1 KB pieces
  // 8 w .. 8 w + 7 (four key rows each), lane L row 4 p + L / 16 of piece p at chunk position
  // L % 16, so it reads chunk (L % 16) ^ (row & 15) of that row (the layout swz reads). The w of
  // the step's keys lands beside them; land() waits for every load of the step and ends with the
  // barrier.
  // (byte offsets from the step's first row; row & 15 repeats every four pieces)
  uint32_t koff[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int row = 4 * (8 * wave + x) + (lane >> 4);
    koff[x] = 16u * (row * 16 + ((lane & 15) ^ (row & 15)));
  }
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t ks_lds = lds_addr(&Ks[0][0]) + (8 * wave_s) * 1024;
  auto issue = [&](int st, int buf) {
    const u32x4* src = kc + (int64_t)st * kBiasStep * 16;
#pragma unroll
    for (int x = 0; x < 8; ++x)
      dma16_s(src, koff[x & 3] + 4096u * (x >> 2), ks_lds + buf * (kBiasStep * 256) + x * 1024);
    if constexpr (kW) {
      // the step's w by LDS-DMA too (waves 0..3, 64 keys each; clamped to the last kept key past
      // m, where E is exactly 0): a register load here would make the compiler wait for every
      // load in flight, the next step's keys included, before this step's arithmetic
      if (wave < 4) dma4(wu + min(st * kBiasStep + 64 * wave + lane, m - 1), &ws_l[buf][64 * wave]);
    }
  };
  auto land = [&](int buf) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  // The kept-logit MFMAs of a step (this wave's 32 rows x its 64-key tile of buffer buf;
  // acc[sub][rg] holds rows rb + 16 rg + 4 g + x, key 256 st + 64 kq + 16 sub + c16, and wv[sub]
  // that key's w). The update passes are software-pipelined: a step's MFMAs run while the
  // previous step's exponentials and sums are formed from registers, so the two waves of a SIMD,
  // which the step barrier keeps in phase, still overlap their MFMAs with vector work.
  auto mma = [&](int buf, f32x4 (&acc)[4][2], float (&wv)[4]) {
    const uint8_t* kb = Ks[buf];
    // the key fragments of k-step ks + 1 are read while those of ks feed the MFMAs
    bf16x8 b[2][4];
    auto frag = [&](int ks, bf16x8 (&f)[4]) {
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
        f[sub] = *reinterpret_cast<const bf16x8*>(&kb[swz(64 * kq + 16 * sub + c16, 4 * ks + g)]);
    };
    frag(0, b[0]);
    if constexpr (kW) {
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) wv[sub] = ws_l[buf][64 * kq + 16 * sub + c16];
    }
    const f32x4 zero = f32x4{0.0f, 0.0f, 0.0f, 0.0f};  // the first k-step starts from 0
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) frag(ks + 1, b[(ks + 1) & 1]);
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        acc[sub][0] = mfma16(qa[0][ks], b[ks & 1][sub], ks ? acc[sub][0] : zero);
        acc[sub][1] = mfma16(qa[1][ks], b[ks & 1][sub], ks ? acc[sub][1] : zero);
      }
    }
  };
  // E = exp(c q.k - ME) of a step's accumulators, 0 past m: a key past m is a zero row of KC, so
  // its logits are exactly 0 and an offset of -inf in place of -ME makes its E exactly 0
  auto expo = [&](int st, const f32x4 (&acc)[4][2], float (&e)[4][2][4]) {
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      const float off = st * kBiasStep + 64 * kq + 16 * sub + c16 < m ? -mb : -INFINITY;
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
#pragma unroll
        for (int x = 0; x < 4; ++x) e[sub][rg][x] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[sub][rg][x], cl, off));
    }
  };
  auto interleave = [] {
    // one MFMA, then three vector instructions, for the 32 MFMAs of a step
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
  };
  // column partial over the lane's 8 rows of each slice (weights rw), reduced over the four lane
  // groups (rows 4g ..): lane group g ends with slice sub = g, i.e. key 64 kq + 16 g + c16 of the
  // step, summed over the wave's 32 rows
  auto colsum = [&](const float (&e)[4][2][4], const float (&rw)[2][4]) {
    float gp[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      float a = 0.0f;
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
#pragma unroll
        for (int x = 0; x < 4; ++x) a = __builtin_fmaf(e[sub][rg][x], rw[rg][x], a);
      gp[sub] = a;
    }
    const bool hi32 = g >= 2;
    const float s0 = hi32 ? gp[0] : gp[2], s1 = hi32 ? gp[1] : gp[3];
    const float r0 = __shfl_xor(s0, 32), r1 = __shfl_xor(s1, 32);
    const float k0 = (hi32 ? gp[2] : gp[0]) + r0, k1 = (hi32 ? gp[3] : gp[1]) + r1;
    const bool odd = g & 1;
    const float rcv = __shfl_xor(odd ? k0 : k1, 16);
    return (odd ? k1 : k0) + rcv;
  };
  float* part = W.part + ((int64_t)h * rt_n + rt) * W.ldm;
  f32x4 acc0[4][2], acc1[4][2];
  float wv0[4], wv1[4];

  if constexpr (MODE == 3) {
    // the largest kept logit c q_i . k_Cj over the tile's rows and the live keys
    float lmax = -INFINITY;
    issue(0, 0);
    land(0);
#pragma unroll 1
    for (int st = 0; st < nsteps; ++st) {
      const bool more = st + 1 < nsteps;
      if (more) issue(st + 1, (st + 1) & 1);
      mma(st & 1, acc0, wv0);
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const bool live = st * kBiasStep + 64 * kq + 16 * sub + c16 < m;
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
          for (int x = 0; x < 4; ++x)
            if (live) lmax = fmaxf(lmax, acc0[sub][rg][x] * scale);
      }
      land((st + 1) & 1);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o));
    if (lane == 0) xpart[0][0][wave] = lmax;
    __syncthreads();
    if (tid == 0) {
      float bm = xpart[0][0][0];
      for (int x = 1; x < kBiasThreads / 64; ++x) bm = fmaxf(bm, xpart[0][0][x]);
      const uint32_t key = float_key(bm);
      if (bm > -INFINITY && key > __atomic_load_n(W.mekey + h, __ATOMIC_RELAXED)) atomicMax(W.mekey + h, key);
    }
    return;
  }

  float rv[2][4];  // the row weights of the lane's rows for the column pass
  if constexpr (kW) {
    // pass A: u_i = sum_j E_ij w_j
    float up[2][4] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    auto post = [&](int st, const f32x4 (&acc)[4][2], const float (&wv)[4]) {
      float e[4][2][4];
      expo(st, acc, e);
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
          for (int x = 0; x < 4; ++x) up[rg][x] = __builtin_fmaf(e[sub][rg][x], wv[sub], up[rg][x]);
    };
    // step st >= 1: loads of st + 1 in flight, MFMAs of st beside the sums of st - 1 (one basic
    // block, so the scheduler can interleave them), then st + 1 staged; step 0 has no sums
    // (the last step stages its own keys again into the free buffer: no branch in the loop body)
    auto step = [&](int st, f32x4 (&cur)[4][2], float (&wc)[4], f32x4 (&prev)[4][2], float (&wp)[4]) {
      issue(min(st + 1, nsteps - 1), (st + 1) & 1);
      mma(st & 1, cur, wc);
      post(st - 1, prev, wp);
      interleave();
      land((st + 1) & 1);
    };
    issue(0, 0);
    land(0);
    issue(min(1, nsteps - 1), 1);
    mma(0, acc0, wv0);
    land(1);
    // two steps per iteration with no branch between them (odd steps in acc1, even in acc0)
    int st = 1;
#pragma unroll 1
    for (; st + 1 < nsteps; st += 2) {
      step(st, acc1, wv1, acc0, wv0);
      step(st + 1, acc0, wv0, acc1, wv1);
    }
    if (st < nsteps) {
      step(st, acc1, wv1, acc0, wv0);
      post(st, acc1, wv1);
    } else {
      post(nsteps - 1, acc0, wv0);
    }
    // reduce over the 16 keys of each lane row (c16), then add the four key quarters in order
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        float v = up[rg][x];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
        up[rg][x] = v;
      }
    if (c16 == 0) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg)
#pragma unroll
        for (int x = 0; x < 4; ++x) rsum[kq][rb + 16 * rg + 4 * g + x] = up[rg][x];
    }
    __syncthreads();
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = rb + 16 * rg + 4 * g + x;
        const float u = ((rsum[0][r] + rsum[1][r]) + rsum[2][r]) + rsum[3][r];
        // MODE 1 weighs the column pass by u; MODE 2 forms P_C = E w / u
        rv[rg][x] = rt * 64 + r < R ? (MODE == 1 ? u : (u > 0.0f ? 1.0f / u : 0.0f)) : 0.0f;
      }
  } else {
    const float* lu = lse + unit * R;
    const float Mz = W.M[h];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int r = rt * 64 + rb + 16 * rg + 4 * g + x;
        rv[rg][x] = r < R ? __builtin_amdgcn_exp2f((lu[r] - Mz) * kLog2e) : 0.0f;
      }
  }

  if constexpr (MODE == 2) {
    // pass C, one step at a time: P_C of the tile's 64 rows x 256 keys, its column partials, then
    // the tile through LDS (in place of the step's keys once every wave has used them; row r at
    // float r * 256 + (key ^ 16 ((r >> 2) & 3)), so the lane groups' rows spread over the banks)
    // and out in the blocked split layout of P_C (8 keys per group) and of P_C^T (8 rows per group)
    float* Pu = W.P + (int64_t)h * pad128(R) * W.ldm;
    float* PTu = W.PT + (int64_t)h * pad128(W.ldm) * W.Rp;
    issue(0, 0);
    land(0);
#pragma unroll 1
    for (int st = 0; st < nsteps; ++st) {
      const int buf = st & 1;
      const bool more = st + 1 < nsteps;
      if (more) issue(st + 1, buf ^ 1);
      mma(buf, acc0, wv0);
      float e[4][2][4];
      expo(st, acc0, e);
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
          for (int x = 0; x < 4; ++x) e[sub][rg][x] = e[sub][rg][x] * wv0[sub] * rv[rg][x];
      const float ones[2][4] = {{1.0f, 1.0f, 1.0f, 1.0f}, {1.0f, 1.0f, 1.0f, 1.0f}};
      const float gsum = colsum(e, ones);
      if (wave & 1) xpart[buf][1][64 * kq + lane] = gsum;
      __syncthreads();  // every wave is done with the step's keys
      if (!(wave & 1)) {
        const int j = st * kBiasStep + 64 * kq + lane;
        if (j < W.ldm) part[j] = gsum + xpart[buf][1][64 * kq + lane];
      }
      float* pl = reinterpret_cast<float*>(Ks[buf]);
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int r = rb + 16 * rg + 4 * g + x, key = 64 * kq + 16 * sub + c16;
            pl[r * kBiasStep + (key ^ (16 * ((r >> 2) & 3)))] = e[sub][rg][x];
          }
      __syncthreads();
      for (int qq = tid; qq < 64 * (kBiasStep / 8); qq += kBiasThreads) {  // rows of P_C
        const int r = qq >> 5, gq = qq & 31;
        const int row = rt * 64 + r, col = st * kBiasStep + 8 * gq;
        if (row < R && col < W.ldm) {
          float x[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) x[k] = pl[r * kBiasStep + ((8 * gq + k) ^ (16 * ((r >> 2) & 3)))];
          blk_put8(Pu, W.ldm, row, st * kBiasStep + 8 * gq, x);
        }
      }
      for (int qq = tid; qq < kBiasStep * 8; qq += kBiasThreads) {  // rows of P_C^T
        const int c = qq >> 3, gq = qq & 7;
        const int key = st * kBiasStep + c;
        if (key < W.ldm) {
          float x[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int r = 8 * gq + k;
            x[k] = pl[r * kBiasStep + (c ^ (16 * ((r >> 2) & 3)))];
          }
          blk_put8(PTu, W.Rp, key, rt * 64 + 8 * gq, x);
        }
      }
      __syncthreads();  // the tile is out before the buffer is staged again
      land(buf ^ 1);
    }
    return;
  }

  // pass B: column partials sum_i E_ij r_i over the tile's 64 rows. A step's partial (lane
  // (g, c16): the wave's 32 rows at key 256 st + 64 kq + 16 g + c16) is formed in the next step;
  // the odd waves leave theirs in LDS, and after that step's barrier the even waves add them
  // (even first) and write the tile's partial.
  auto column = [&](int st, const f32x4 (&acc)[4][2]) {
    float e[4][2][4];
    expo(st, acc, e);
    return colsum(e, rv);
  };
  float gkeep = 0.0f;  // an even wave's own partial of the previous step
  auto flush = [&](int st) {  // the tile's partial of step st (even waves, after the barrier)
    if (!(wave & 1)) {
      const int j = st * kBiasStep + 64 * kq + lane;
      if (j < W.ldm) part[j] = gkeep + xpart[st & 1][1][64 * kq + lane];
    }
  };
  // step st >= 1 (step 0 has no column): the partial of st - 2 leaves first, then the MFMAs of
  // st beside the column of st - 1 in one basic block
  auto stepB = [&](int st, f32x4 (&cur)[4][2], float (&wc)[4], f32x4 (&prev)[4][2]) {
    issue(min(st + 1, nsteps - 1), (st + 1) & 1);
    if (st > 1) flush(st - 2);
    mma(st & 1, cur, wc);
    const float gs = column(st - 1, prev);
    interleave();
    xpart[(st - 1) & 1][wave & 1][64 * kq + lane] = gs;
    gkeep = gs;
    land((st + 1) & 1);
  };
  issue(0, 0);
  land(0);
  issue(min(1, nsteps - 1), 1);
  mma(0, acc0, wv0);
  land(1);
  int st = 1;
#pragma unroll 1
  for (; st + 1 < nsteps; st += 2) {
    stepB(st, acc1, wv1, acc0);
    stepB(st + 1, acc0, wv0, acc1);
  }
  if (st < nsteps) stepB(st, acc1, wv1, acc0);
  if (nsteps > 1) flush(nsteps - 2);
  {
    const float gs = (nsteps & 1) ? column(nsteps - 1, acc0) : column(nsteps - 1, acc1);
    xpart[(nsteps - 1) & 1][wave & 1][64 * kq + lane] = gs;
    gkeep = gs;
    __syncthreads();
    flush(nsteps - 1);
  }
}

// ------------------------------------------------------------------------------------------------
// Target Y = P V with P_ij = exp(c q_i . k_j - LSE_i) over all n keys, without materialising P
// (the weights of one 64-key chunk exist only in registers).
// Work item = (seq, head, 256-row block, key split): the keys are split C.St ways (contiguous
// runs of 64-key chunks) into partial targets Y_t that the first value product adds in order;
// a workgroup re-reads only its share of K and V, and there are C.St times as many of them.
// Eight waves: wave w owns rows 32 w .. + 31 of the block (two 16-row fragments) and all 128
// output columns. Per 64-key chunk, staged through double-buffered LDS (key and value rows alike
// as bf16 rows, chunk c of key row r at c ^ (r & 15), of value row r at c ^ 2 (r & 7)):
//   S^T = K Q^T   per row fragment 16 v_mfma_f32_16x16x32_bf16 (the fragment's query rows stay in
//                 registers as the B operand; a key fragment read serves both row fragments), so
//                 lane (g, c16) holds row c16's logits of keys 16 sub + 4 g + x;
//   P = exp2(S c log2(e) - LSE log2(e)), 0 for keys past n: the lane's eight weights of keys
//                 32 s + {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3} are directly its A operand
//                 of k-step s of the next product, with the contraction taken in that key order;
//   Y += P V      P split as hi + lo (bf16 each; V is bf16 already, so the two products
//                 P_hi V + P_lo V carry P to a relative 2^-16), V's B operand read in the same
//                 key order by ds_read_b64_tr_b16 (a transposing LDS read: within 16 lanes, lane
//                 l's element x comes from the 8 bytes lane 4 x + l / 4 addresses, element l % 4,
//                 so lanes addressing 4 consecutive values of 4 keys receive one value column
//                 each) and used by both row fragments.
// ------------------------------------------------------------------------------------------------
namespace {
constexpr int kTgtThreads = 512;
constexpr int kTgtRows = 256;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16;

// Value rows in LDS: 16-byte chunk c of key row r at position c ^ 2 (r & 7). A transposing read
// (8 bytes per lane; gfx950 serves such reads as two groups of 32 lanes over 64 banks) then has
// each 32-lane group's 8 keys x 2 chunks land on the 16 distinct chunk positions of a 256-byte
// window: free of bank conflicts (with the score kernels' c ^ (r & 15) it took two cycles).
__device__ __forceinline__ int vswz(int row, int chunk) { return row * 256 + ((chunk ^ (2 * (row & 7))) << 4); }
// four consecutive bf16 values of one value column (keys k0 .. k0 + 3) for each lane of a
// 16-lane group: lane j addresses key k0 + j / 4, columns col0 + 4 (j % 4) .. + 3
__device__ __forceinline__ v4i16 tr_read(const uint8_t* rows, int k0, int col0, int j) {
  const int key = k0 + (j >> 2), col = col0 + 4 * (j & 3);
  const uint8_t* p = rows + vswz(key, col >> 3) + 8 * ((col >> 2) & 1);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16)(__attribute__((address_space(3))) const void*)p);
}
}  // namespace

template <int LAYOUT>
__global__ __launch_bounds__(kTgtThreads, 1) void am_target(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const int32_t* __restrict__ table, int max_blocks,
                                                            const int32_t* __restrict__ vtable, int vmax_blocks,
                                                            const float* __restrict__ lse, float* __restrict__ ws,
                                                            int64_t n_max, float scale, AmCfg C, SeqTable T) {
  __shared__ __attribute__((aligned(16))) uint8_t Ks[2][64 * 256];
  __shared__ __attribute__((aligned(16))) uint8_t Vs[2][64 * 256];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i], s = T.first + i;
  const int H = C.H, R = C.R;
  const int rb_n = (R + kTgtRows - 1) / kTgtRows;
  int local = t - T.start[i];
  const int sp = local % C.St;
  local /= C.St;
  const int h = local / rb_n, rb = local - h * rb_n;
  const int64_t unit = (int64_t)s * H + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  AmWs W = am_ws(ws, T, i, C);
  const int32_t* map = LAYOUT == kPaged ? table + (int64_t)s * max_blocks
                                        : (LAYOUT == kSlots ? table + unit * n_max : nullptr);
  const int32_t* vmap = LAYOUT == kPaged ? vtable + (int64_t)s * vmax_blocks
                                         : (LAYOUT == kSlots ? vtable + unit * n_max : nullptr);
  const int kofs = T.kofs[i];
  const int nch_all = (n + 63) / 64, per = (nch_all + C.St - 1) / C.St;
  const int ch0 = sp * per, ch1 = min(nch_all, ch0 + per);

  // query row c16 of each row fragment (B operand of S^T) and its LSE
  bf16x8 qb[2][4];
  float lb[2];
#pragma unroll
  for (int rf = 0; rf < 2; ++rf) {
    const int qrow = min(rb * kTgtRows + 32 * wave + 16 * rf + c16, R - 1);
    const u32x4* qr = reinterpret_cast<const u32x4*>(q + (unit * R + qrow) * (int64_t)kD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[rf][ks] = as_bf16x8(qr[4 * ks + g]);
    lb[rf] = lse[unit * R + qrow] * kLog2e;
  }
  const float cl = scale * kLog2e;

  // chunk staging: thread tid moves 16-byte piece tid & 15 of key and value rows tid >> 4 and
  // 32 + (tid >> 4)
  u32x4 kr[2], vr[2];
  auto load = [&](int c0) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int kk = c0 + x * 32 + (tid >> 4);
      const int pos = kofs + min(kk, n - 1);
      kr[x] = key_row<LAYOUT>(k, map, H, h, n_max, unit, pos)[tid & 15];
      vr[x] = key_row<LAYOUT>(v, vmap, H, h, n_max, unit, pos)[tid & 15];
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int key = x * 32 + (tid >> 4), ch = tid & 15;
      *reinterpret_cast<u32x4*>(&Ks[buf][swz(key, ch)]) = kr[x];
      *reinterpret_cast<u32x4*>(&Vs[buf][vswz(key, ch)]) = vr[x];
    }
  };

  f32x4 acc[2][8];
#pragma unroll
  for (int rf = 0; rf < 2; ++rf)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[rf][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (ch0 < ch1) {
    load(ch0 * 64);
    store(0);
    __syncthreads();
  }
#pragma unroll 1
  for (int ch = ch0; ch < ch1; ++ch) {
    const int buf = (ch - ch0) & 1;
    const bool more = ch + 1 < ch1;
    if (more) load((ch + 1) * 64);
    const uint8_t* kb = Ks[buf];
    const uint8_t* vb = Vs[buf];
    // S^T and the weights: pw[rf][sub][x] is row c16's weight of key 64 ch + 16 sub + 4 g + x
    float pw[2][4][4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      f32x4 sacc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&kb[swz(16 * sub + c16, 4 * ks + g)]);
        sacc[0] = mfma16(ka, qb[0][ks], sacc[0]);
        sacc[1] = mfma16(ka, qb[1][ks], sacc[1]);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const bool live = ch * 64 + 16 * sub + 4 * g + x < n;
#pragma unroll
        for (int rf = 0; rf < 2; ++rf)
          pw[rf][sub][x] = live ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[rf][x], cl, -lb[rf])) : 0.0f;
      }
    }
    // Y += P V over the 64 keys in two k-steps of 32 (keys 32 s + 4 g + x and 32 s + 16 + 4 g + x)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 ph[2], pl[2];
#pragma unroll
      for (int rf = 0; rf < 2; ++rf) {
        const float px[8] = {pw[rf][2 * ks][0],     pw[rf][2 * ks][1],     pw[rf][2 * ks][2],
                             pw[rf][2 * ks][3],     pw[rf][2 * ks + 1][0], pw[rf][2 * ks + 1][1],
                             pw[rf][2 * ks + 1][2], pw[rf][2 * ks + 1][3]};
        split8(px, ph[rf], pl[rf]);
      }
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const v4i16 v0 = tr_read(vb, 32 * ks + 4 * g, 16 * b, c16);
        const v4i16 v1 = tr_read(vb, 32 * ks + 16 + 4 * g, 16 * b, c16);
        const bf16x8 vv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rf = 0; rf < 2; ++rf) {
          acc[rf][b] = mfma16(as_bf16x8(ph[rf]), vv, acc[rf][b]);
          acc[rf][b] = mfma16(as_bf16x8(pl[rf]), vv, acc[rf][b]);
        }
      }
    }
    if (more) store(buf ^ 1);
    __syncthreads();
  }
  float* out = W.Y + sp * pad64((int64_t)H * R * kD) + (int64_t)h * R * kD;
#pragma unroll
  for (int rf = 0; rf < 2; ++rf)
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = rb * kTgtRows + 32 * wave + 16 * rf + 4 * g + e;
        if (r < R) out[(int64_t)r * kD + 16 * b + c16] = acc[rf][b][e];
      }
}

// Row blocks of the target kernel.
int am_target_blocks(int R) { return (R + kTgtRows - 1) / kTgtRows; }

// ------------------------------------------------------------------------------------------------
// The value fit's matrix products (am_gemm, am_gram): one 128 x 128 output tile per workgroup of
// eight waves (wave w: rows 64 (w & 1) .. + 63, columns 32 (w >> 1) .. + 31; four x two 16 x 16
// accumulators). Both operands are read by rows along the contraction: out = A B^T.
// The float32 operands are stored split (x = hi + lo with hi = bf16(x) and lo = bf16(x - hi),
// the layout of put_split8), and a product is taken as hi_a hi_b + hi_a lo_b + lo_a hi_b on
// v_mfma_f32_16x16x32_bf16 with float32 accumulation (the dropped lo_a lo_b and the rounding of
// lo leave a relative error near 2^-16 per product, against 2^-24 for float32 inputs, at a
// third of the float32 MFMA's cycles per product).
// The contraction runs in stages of 32 through a ring of kRing LDS slots filled by LDS-DMA
// kRing stages ahead of the stage whose MFMAs run (a stage's fragments are read into registers
// one stage before its MFMAs): a stage is the 128 rows of the A block, then the 128 rows of the
// B block, 128 bytes per row (the 32 indices' split groups: high half, low half), 16-byte chunk
// c of row r at position c ^ step_sw(r) (the low three bits of r with bits 0 and 1 swapped), so
// every ds_read_b128 of an MFMA operand is free of bank conflicts (gfx950 serves such a read in
// four groups of 16 lanes, group = (lane bit 5, parity of lane bits 2..4), each over 64 banks:
// the 16 rows read at one chunk position must land in 16 distinct 16-byte slots of a 256-byte
// window; measured with the LDS bank-conflict counter). Wave w lands the 1 KB pieces
// 4 w .. 4 w + 3 of the 32 (8 rows each; waves 0-3 the A block, 4-7 the B block), lane L row
// L / 8 of its piece at position L % 8, reading chunk (L % 8) ^ step_sw(row) of that row; rows
// past a block's live ones read its last live row (the caller drops their products). Past the
// last stage the ring is refilled with the last stage again (its fragments are read but not
// used), which keeps four loads per wave per stage and so the fixed wait counts exact.
// ------------------------------------------------------------------------------------------------
namespace {
constexpr int kGTile = 128;
constexpr int kRingThreads = 512;
constexpr int kRing = 4;
constexpr int kRingSlot = 2 * kGTile * 128;  // bytes per stage: both row blocks
__device__ __forceinline__ int sswz(int row, int chunk) { return row * 128 + ((chunk ^ step_sw(row)) << 4); }
// at most N of this wave's loads outstanding (four per stage), then a barrier
template <int N>
__device__ __forceinline__ void ring_wait_barrier() {
  static_assert(kRing == 4, "the wait counts follow the ring depth");
  if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else static_assert(N == 8, "unsupported count");
}

// acc += A B^T over contraction stages st0 .. st1 - 1 of one tile. Xa, Xb: the A and B row
// blocks, each either in the blocked split layout (blk_put8; pitch 0: a stage is 16 KB in the
// ring's order already) or as split rows with a pitch of pa / pb floats (the lane reads chunk
// (L % 8) ^ step_sw(row) of its row; la, lb (at least 1): the live rows, later rows read the last
// live one). sm: the ring (kRing * kRingSlot bytes); when this returns every wave is done with it.
__device__ __forceinline__ void ring_mma(const float* Xa, int la, int pa, const float* Xb, int lb, int pb, int st0,
                                         int st1, f32x4 (&acc)[4][2], uint8_t* sm) {
  if (st0 >= st1) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int wr = wave & 1, wc = wave >> 1;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const float* Xw = wave_s < 4 ? Xa : Xb;  // the wave's block
  const int lw = wave_s < 4 ? la : lb, pw = wave_s < 4 ? pa : pb;
  const int sstep = pw ? 32 : 4096;  // floats per stage
  // this lane's DMA sources: byte offsets from the block's first stage
  uint32_t voff[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int piece = (4 * wave + x) & 15, row = 8 * piece + (lane >> 3);
    voff[x] = pw ? 4u * (uint32_t)(min(row, lw - 1) * pw + 4 * ((lane & 7) ^ step_sw(row)))
                 : 16u * (uint32_t)(64 * piece + lane);
  }
  const uint32_t ring = lds_addr(sm) + 4 * wave_s * 1024;
  auto issue = [&](int stg) {
    const float* src = Xw + (int64_t)sstep * min(stg, st1 - 1);
    const uint32_t slot = ring + ((stg - st0) % kRing) * kRingSlot;
#pragma unroll
    for (int x = 0; x < 4; ++x) dma16_s(src, voff[x], slot + x * 1024);
  };
  // a stage's fragments (A block: four row fragments, B block: two; high and low halves)
  struct Frags {
    bf16x8 ah[4], al[4], bh[2], bl[2];
  };
  auto read = [&](int stg, Frags& f) {
    const uint8_t* slot = sm + ((stg - st0) % kRing) * kRingSlot;
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int rbw = 32 * wc + 16 * y + c16;
      f.bh[y] = *reinterpret_cast<const bf16x8*>(&slot[kGTile * 128 + sswz(rbw, 2 * g)]);
      f.bl[y] = *reinterpret_cast<const bf16x8*>(&slot[kGTile * 128 + sswz(rbw, 2 * g + 1)]);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int ra = 64 * wr + 16 * x + c16;
      f.ah[x] = *reinterpret_cast<const bf16x8*>(&slot[sswz(ra, 2 * g)]);
      f.al[x] = *reinterpret_cast<const bf16x8*>(&slot[sswz(ra, 2 * g + 1)]);
    }
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        acc[x][y] = mfma16(f.ah[x], f.bh[y], acc[x][y]);
        acc[x][y] = mfma16(f.ah[x], f.bl[y], acc[x][y]);
        acc[x][y] = mfma16(f.al[x], f.bh[y], acc[x][y]);
      }
  };
  // Stage s's fragments are read into registers one stage early, so their LDS latency hides
  // behind the MFMAs of stage s - 1: at the top of the iteration for stage s, stage s + 1 has
  // landed (only stages s + 2 and s + 3, eight loads, may be outstanding), and after the barrier
  // every wave holds stage s in registers, so its slot takes stage s + 4.
  Frags f0, f1;
#pragma unroll
  for (int k = 0; k < kRing; ++k) issue(st0 + k);
  ring_wait_barrier<12>();
  read(st0, f0);
  auto iter = [&](int stg, Frags& cur, Frags& nxt) {
    ring_wait_barrier<8>();
    issue(stg + kRing);
    read(stg + 1, nxt);
    mma(cur);
  };
  int stg = st0;
#pragma unroll 1
  for (; stg + 1 < st1; stg += 2) {
    iter(stg, f0, f1);
    iter(stg + 1, f1, f0);
  }
  if (stg < st1) iter(stg, f0, f1);
  vm_wait_barrier<0>();  // the refills past the last stage are in, and every wave is done with the ring
}
}  // namespace

// ------------------------------------------------------------------------------------------------
// The P_C products of the value fit, split over S workgroups along the contraction whose partial
// tiles a second pass (am_split_sum) adds in order:
//   KIND 0: Z = P_C V0 - Y           (rows of P_C, contraction over kept keys)  -> Z, or partials Zp
//           (rows side: also the iterate X = Z and its sum Sx = Z)
//   KIND 1: P_C^T T                  (columns of P_C, contraction over rows; T = Z, or the sum of
//           the iterates when C.xsel = 1)                                      -> or partials Up
//           mode 0: Vc -= eta P_C^T T (the last product of the rows side, or the only step)
//           mode 1: X = Sx = P_C^T Z  (the first iterate of the keys side)
// Work item = (seq, head, output tile, split), split fastest.
// ------------------------------------------------------------------------------------------------
template <int KIND>
__global__ __launch_bounds__(kRingThreads) void am_gemm(float* __restrict__ vc_all, float* __restrict__ ws, AmCfg C,
                                                       SeqTable T) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[kRing * kRingSlot];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  const int R = C.R;
  AmWs W = am_ws(ws, T, i, C);
  const int ldm = W.ldm, Np = W.Np;
  const int S = KIND == 0 ? C.S1 : C.S2;
  const int rows = KIND == 0 ? R : ldm;  // output rows
  const int tiles = (rows + kGTile - 1) / kGTile;
  int local = t - T.start[i];
  const int sp = local % S;
  local /= S;
  const int tile = local % tiles, h = local / tiles;
  const int64_t unit = (int64_t)s * C.H + h;
  // A rows (pitch apitch) and B rows (the 128 columns of the right operand, pitch bpitch)
  const int apitch = KIND == 0 ? ldm : W.Rp;
  const float* A = KIND == 0 ? W.P + (int64_t)h * pad128(R) * ldm : W.PT + (int64_t)h * pad128(ldm) * W.Rp;
  const float* B = KIND == 0 ? W.VT + (int64_t)h * kD * ldm : (C.xsel ? W.XT1 : W.ZT) + (int64_t)h * kD * W.Rp;
  const int nst = KIND == 0 ? ldm / 32 : (R + 31) / 32;
  const int per = (nst + S - 1) / S;
  const int st0 = sp * per, st1 = min(nst, st0 + per);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int wr = wave & 1, wc = wave >> 1;
  const int alim = KIND == 0 ? R : ldm;

  f32x4 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a][0] = acc[a][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  ring_mma(A + (int64_t)tile * kGTile * apitch, alim - tile * kGTile, 0, B, kD, apitch, st0, st1, acc, sm);

  const float eta = W.eta[h];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = tile * kGTile + 64 * wr + 16 * a + 4 * g + e;
        const int col = 32 * wc + 16 * b + c16;
        const float v = acc[a][b][e];
        if constexpr (KIND == 0) {  // Z = P_C V0 - Y, kept as split rows of Z^T (zeros past R)
          const int64_t o = (int64_t)h * R * kD + (int64_t)r * kD + col;
          if (S == 1) {
            if (r < W.Rp) {
              float y = 0.0f;
              if (r < R) {
                y = W.Y[o];
                for (int tp = 1; tp < C.St; ++tp) y += W.Y[tp * pad64((int64_t)C.H * R * kD) + o];
              }
              const float z = r < R ? v - y : 0.0f;
              put_split1(W.ZT + ((int64_t)h * kD + col) * W.Rp, r, z);
              if (W.rside && r < R) {
                const int64_t ox = ((int64_t)h * Np + r) * kD + col;
                W.X[ox] = z;
                W.Sx[ox] = z;
              }
            }
          } else if (r < R) {
            W.Zp[(int64_t)sp * pad64((int64_t)C.H * R * kD) + o] = v;
          }
        } else {
          const int64_t o = (int64_t)r * kD + col;
          if (S == 1) {
            if (r < ldm) {
              if (C.mode == 0) {  // Vc -= eta P_C^T T, with its split rows of Vc^T (zeros past m)
                float x = 0.0f;
                if (r < m) {
                  float* d = vc_all + unit * C.m_max * (int64_t)kD + o;
                  x = *d - eta * v;
                  *d = x;
                }
                put_split1(W.VT + ((int64_t)h * kD + col) * ldm, r, x);
              } else {  // the keys side's first iterate
                const float x = r < m ? v : 0.0f;
                const int64_t ox = ((int64_t)h * Np + r) * kD + col;
                W.X[ox] = x;
                W.Sx[ox] = x;
                put_split1(W.VT + ((int64_t)h * kD + col) * ldm, r, x);
              }
            }
          } else if (r < ldm) {
            W.Up[(int64_t)sp * pad64((int64_t)C.H * ldm * kD) + (int64_t)h * ldm * kD + o] = v;
          }
        }
      }
}

// ------------------------------------------------------------------------------------------------
// One step of the value iteration, X <- X - eta Mg X and Sx += X (the rows of the iteration's
// side), with its epilogue fused: no split of the contraction, so no partial products. The
// product is bound by reading Mg (4 bytes per entry, once per step); its right operand, the
// iterate's transpose (split rows [128][Np]), is shared by all row tiles of a unit and read from
// L2. One 64 x 128 output tile per workgroup of eight waves (wave w: rows 32 (w & 1) .. + 31,
// columns 32 (w >> 1) .. + 31: two x two 16 x 16 accumulators, eight operand reads per stage),
// operands split as in am_gemm (three bf16 products). The contraction runs in stages of 32
// through a ring of kStepRing LDS slots
// filled by LDS-DMA (global_load_lds_dwordx4, three per wave per stage) kStepRing stages ahead
// of the stage whose MFMAs run (deep enough that the bytes in flight cover the memory latency
// at full rate; a stage's fragments are read into registers one stage before its MFMAs): a
// stage is 64 rows of Mg and the 128 rows of the transpose, 128 bytes per row (the 32 indices'
// split groups: high half, low half), 16-byte chunk c of row r at position c ^ step_sw(r) (the
// low three bits of r with bits 0 and 1 swapped), so every ds_read_b128 of an MFMA operand is
// free of bank conflicts (gfx950 serves such a read in four groups of 16 lanes, group = (lane
// bit 5, parity of lane bits 2..4), each over 64 banks: the 16 rows read at one chunk position
// must land in 16 distinct 16-byte slots of a 256-byte window; measured with the LDS
// bank-conflict counter). The DMA lands each wave's 1 KB contiguously, so the source address of
// a lane carries the permutation. Past the last stage the ring is refilled with the last stage
// again (its fragments are read but not used), which keeps three loads per wave per stage and so
// the fixed wait counts exact.
//   mode 0: the new iterate's transpose goes to the other buffer for the next step
//   mode 1 (last step): rows side, Sx's transpose goes there for the last P_C^T product;
//           keys side, Vc -= eta Sx
// The tile leaves through LDS: X and Sx as float32 rows, the transpose as split rows.
// Work item = (seq, head, 64-row tile of the side).
// ------------------------------------------------------------------------------------------------
namespace {
constexpr int kStepRows = 64;
constexpr int kStepThreads = 512;
constexpr int kStepRing = 6;
constexpr int kStepA = kStepRows * 128, kStepB = kGTile * 128, kStepSlot = kStepA + kStepB;
// Mg is stored as the step kernel reads it: per 64-row block and 32-column stage an 8 KB block of
// 64 rows x 128 bytes (the four 8-column groups, high half then low half), 16-byte chunk c of
// row r at position c ^ step_sw(r); a stage of a row block is one contiguous read.
__device__ __forceinline__ void mg_put8(float* mh, int Np, int r, int c, const float* x) {
  u32x4 hi, lo;
  split8(x, hi, lo);
  const int row = r & (kStepRows - 1), grp = (c & 31) >> 3, sw = step_sw(row);
  uint8_t* blk = reinterpret_cast<uint8_t*>(mh) + (((int64_t)(r / kStepRows) * (Np / 32) + (c >> 5)) << 13) + row * 128;
  *reinterpret_cast<u32x4*>(blk + (((2 * grp) ^ sw) << 4)) = hi;
  *reinterpret_cast<u32x4*>(blk + (((2 * grp + 1) ^ sw) << 4)) = lo;
}
// at most N of this wave's loads outstanding (three per stage), then a barrier
template <int N>
__device__ __forceinline__ void step_wait_barrier() {
  static_assert(kStepRing == 6, "the wait counts follow the ring depth");
  if constexpr (N == 15) asm volatile("s_waitcnt vmcnt(15) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else static_assert(N == 12, "unsupported count");
}
}  // namespace

__global__ __launch_bounds__(kStepThreads) void am_step(float* __restrict__ vc_all, float* __restrict__ ws, AmCfg C,
                                                        SeqTable T) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[kStepRing * kStepSlot];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  AmWs W = am_ws(ws, T, i, C);
  const int Np = W.Np;
  const int nb = Np / kStepRows;
  const int local = t - T.start[i];
  const int h = local / nb, blk = local - h * nb;
  const int64_t unit = (int64_t)s * C.H + h;
  const float* A = W.Mg + ((int64_t)h * Np + blk * kStepRows) * Np;  // the row block's stages, 8 KB each
  const float* B = am_xt(W.XT1, W.ZT, W.VT, W.rside, C.xsel) + (int64_t)h * kD * Np;
  const int nst = Np / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int wr = wave & 1, wc = wave >> 1;  // the wave's 32 rows and 32 columns of the tile
  // this lane's DMA sources: the three 1 KB pieces (8 rows x 128 bytes) of a stage that wave w
  // lands are pieces 3 w .. 3 w + 2 of the 24 (8 of A, then 16 of B); lane L lands row L / 8 of
  // its piece at position L % 8. A is stored in that order already (a stage is 8 KB further on);
  // for B the lane reads chunk (L % 8) ^ step_sw(row) of its row (a stage is 32 floats on).
  // The loads are addressed from the stage's start in A or B (scalar) plus per-lane byte offsets
  // fixed for the whole ring, into scalar LDS destinations.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t voff[3];
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    const int piece = 3 * wave + x;
    if (piece < 8) {
      voff[x] = (piece * 64 + lane) * 16;
    } else {
      const int row = 8 * (piece - 8) + (lane >> 3);
      voff[x] = row * Np * 4 + (((lane & 7) ^ step_sw(row)) << 4);
    }
  }
  const uint32_t ring_lds = lds_addr(sm) + 3 * wave_s * 1024;
  auto issue = [&](int stg) {
    const int st = min(stg, nst - 1);
    const uint32_t slot = ring_lds + (stg % kStepRing) * kStepSlot;
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const bool in_a = 3 * wave_s + x < 8;  // (wave-uniform)
      dma16_s(in_a ? A + (int64_t)st * 2048 : B + st * 32, voff[x], slot + x * 1024);
    }
  };
  // the epilogue's operands (this lane's 16 entries of X and of Sx; rows past N are zero) are
  // loaded before the ring starts, so their latency hides behind the product (they are older
  // than every ring load, so the ring's in-order waits cover them)
  // accumulator (a, b) of the wave, element e: tile row 32 wr + 16 a + 4 g + e, column
  // 32 wc + 16 b + c16
  float xo[2][2][4], so[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t ox = ((int64_t)h * Np + blk * kStepRows + 32 * wr + 16 * a + 4 * g + e) * kD + 32 * wc +
                           16 * b + c16;
        xo[a][b][e] = W.X[ox];
        so[a][b][e] = W.Sx[ox];
      }
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a) acc[a][0] = acc[a][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // a stage's fragments: the wave's 32 rows of Mg and its 32 columns of the iterate, high and low
  struct Frags {
    bf16x8 ah[2], al[2], bh[2], bl[2];
  };
  auto read = [&](int stg, Frags& f) {
    const uint8_t* slot = sm + (stg % kStepRing) * kStepSlot;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int ra = 32 * wr + 16 * a + c16;
      f.ah[a] = *reinterpret_cast<const bf16x8*>(&slot[sswz(ra, 2 * g)]);
      f.al[a] = *reinterpret_cast<const bf16x8*>(&slot[sswz(ra, 2 * g + 1)]);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int rbw = 32 * wc + 16 * b + c16;
      f.bh[b] = *reinterpret_cast<const bf16x8*>(&slot[kStepA + sswz(rbw, 2 * g)]);
      f.bl[b] = *reinterpret_cast<const bf16x8*>(&slot[kStepA + sswz(rbw, 2 * g + 1)]);
    }
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        acc[a][b] = mfma16(f.ah[a], f.bh[b], acc[a][b]);
        acc[a][b] = mfma16(f.ah[a], f.bl[b], acc[a][b]);
        acc[a][b] = mfma16(f.al[a], f.bh[b], acc[a][b]);
      }
  };
  // Stage s's fragments are read into registers one stage early, so their LDS latency hides
  // behind the MFMAs of stage s - 1: at the top of the iteration for stage s, stage s + 1 has
  // landed (only stages s + 2 .. s + 5, twelve loads, may be outstanding), and after the barrier
  // every wave holds stage s in registers, so its slot takes stage s + 6.
  Frags f0, f1;
#pragma unroll
  for (int stg = 0; stg < kStepRing; ++stg) issue(stg);
  step_wait_barrier<15>();
  read(0, f0);
  auto iter = [&](int stg, Frags& cur, Frags& nxt) {
    step_wait_barrier<12>();
    issue(stg + kStepRing);
    read(stg + 1, nxt);
    mma(cur);
  };
  int stg = 0;
#pragma unroll 1
  for (; stg + 1 < nst; stg += 2) {
    iter(stg, f0, f1);
    iter(stg + 1, f1, f0);
  }
  if (stg < nst) iter(stg, f0, f1);
  vm_wait_barrier<0>();  // the refills past the last stage are in, and every wave is done with the ring

  // epilogue through LDS: the tile's new iterate in float32 rows of 128 (pitch 129)
  float* tl = reinterpret_cast<float*>(sm);
  static_assert(sizeof(sm) >= sizeof(float) * kStepRows * (kD + 1), "the epilogue tile fits the ring");
  const float eta = W.eta[h];
  const bool to_vc = C.mode == 1 && !W.rside;
  float* vcu = vc_all + unit * C.m_max * (int64_t)kD;
  float vo[2][2][4];  // the last step of the keys side: this lane's entries of Vc (rows clamped below m)
  if (to_vc) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = blk * kStepRows + 32 * wr + 16 * a + 4 * g + e;
          vo[a][b][e] = vcu[(int64_t)min(r, m - 1) * kD + 32 * wc + 16 * b + c16];
        }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rl = 32 * wr + 16 * a + 4 * g + e, r = blk * kStepRows + rl, col = 32 * wc + 16 * b + c16;
        const float xn = xo[a][b][e] - eta * acc[a][b][e];
        const float sum = so[a][b][e] + xn;
        const bool live = r < W.N;
        if (live) {
          const int64_t ox = ((int64_t)h * Np + r) * kD + col;
          W.X[ox] = xn;
          W.Sx[ox] = sum;
          if (to_vc && r < m) vcu[(int64_t)r * kD + col] = vo[a][b][e] - eta * sum;
        }
        tl[rl * (kD + 1) + col] = live ? (C.mode == 1 ? sum : xn) : 0.0f;
      }
  if (to_vc) return;  // uniform across the block
  __syncthreads();
  float* dst = am_xt(W.XT1, W.ZT, W.VT, W.rside, C.xsel ^ 1) + (int64_t)h * kD * Np + blk * kStepRows;
  for (int qq = tid; qq < kD * (kStepRows / 8); qq += kStepThreads) {
    const int d = qq >> 3, gq = qq & 7;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = tl[(8 * gq + e) * (kD + 1) + d];
    put_split8(dst + (int64_t)d * Np, gq, x);
  }
}

// 64-row tiles of a step on an Np-row side.
int64_t am_step_items(int Np) { return Np / kStepRows; }

// Output tiles of the products: KIND 0 over the R rows, KIND 1 over the ldm kept keys, KIND 2
// over the Np rows of the iteration's side.
int am_gemm_tiles(int rows) { return (rows + kGTile - 1) / kGTile; }

// ------------------------------------------------------------------------------------------------
// The Gram matrix of the iteration's side, Mg = X X^T with X = P_C (rows side: Np = Rp rows,
// contraction over the kept keys) or X = P_C^T (keys side: Np = ldm rows, contraction over the
// proxy rows), stored as split rows [Np][Np]. Mg is symmetric: a workgroup forms the 128 x 128
// tile (a, b) with a <= b (ring_mma with row blocks a and b) and writes it and, off the
// diagonal, its transpose, both through LDS (the tile in float32, pitch 129), in the blocked
// layout the step kernel reads (mg_put8). Rows and columns of X past its live rows are zero, so
// are those of Mg. Work item = (seq, head, tile pair), pairs a-major.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kRingThreads) void am_gram(float* __restrict__ ws, AmCfg C, SeqTable T) {
  constexpr int kPitch = kGTile + 1;
  __shared__ __attribute__((aligned(16))) uint8_t sm[kRing * kRingSlot];
  static_assert(sizeof(sm) >= sizeof(float) * kGTile * kPitch, "the epilogue tile fits the ring");
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int R = C.R;
  AmWs W = am_ws(ws, T, i, C);
  const int ldm = W.ldm, Np = W.Np;
  const int nt = (Np + kGTile - 1) / kGTile, pairs = nt * (nt + 1) / 2;
  const int local = t - T.start[i];
  const int h = local / pairs;
  int p = local - h * pairs, a = 0;
  while (p >= nt - a) {
    p -= nt - a;
    ++a;
  }
  const int b = a + p;
  const float* X = W.rside ? W.P + (int64_t)h * pad128(R) * ldm : W.PT + (int64_t)h * pad128(ldm) * W.Rp;
  const int pitch = W.rside ? ldm : W.Rp;
  const int xrows = W.rside ? R : ldm;
  const int nst = W.rside ? ldm / 32 : (R + 31) / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int wr = wave & 1, wc = wave >> 1;
  f32x4 acc[4][2];
#pragma unroll
  for (int x = 0; x < 4; ++x) acc[x][0] = acc[x][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  ring_mma(X + (int64_t)a * kGTile * pitch, xrows - a * kGTile, 0, X + (int64_t)b * kGTile * pitch, xrows - b * kGTile,
           0, 0, nst, acc, sm);

  float* tl = reinterpret_cast<float*>(sm);
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 64 * wr + 16 * x + 4 * g + e, c = 32 * wc + 16 * y + c16;
        const bool live = a * kGTile + r < xrows && b * kGTile + c < xrows;
        tl[r * kPitch + c] = live ? acc[x][y][e] : 0.0f;
      }
  __syncthreads();
  float* Mh = W.Mg + (int64_t)h * Np * Np;
  for (int q = tid; q < kGTile * (kGTile / 8); q += kRingThreads) {
    const int r = q >> 4, gq = q & 15;
    if (a * kGTile + r < Np && b * kGTile + 8 * gq < Np)
      mg_put8(Mh, Np, a * kGTile + r, b * kGTile + 8 * gq, &tl[r * kPitch + 8 * gq]);
  }
  if (a != b) {
    for (int q = tid; q < kGTile * (kGTile / 8); q += kRingThreads) {
      const int c = q >> 4, gq = q & 15;
      if (b * kGTile + c >= Np || a * kGTile + 8 * gq >= Np) continue;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = tl[(8 * gq + e) * kPitch + c];
      mg_put8(Mh, Np, b * kGTile + c, a * kGTile + 8 * gq, x);
    }
  }
}

// Tile pairs of the Gram matrix of an Np-row side.
int64_t am_gram_items(int Np) {
  const int64_t nt = (Np + kGTile - 1) / kGTile;
  return nt * (nt + 1) / 2;
}

// Split sums, in split order, then the product's epilogue (as in am_gemm with one split):
//   KIND 0: Z = sum_s Zp[s] - Y                       work item = (seq, head, 64 rows)
//   KIND 1: mode 0: Vc_j -= eta sum_s Up[s]_j; mode 1: X = Sx = sum_s Up[s]
//                                                     work item = (seq, head, 64 kept keys)
// The block's results (zeros past the live rows) are staged in LDS and leave as split rows of
// the transpose, the form the next product reads; Vc and the iterates are also kept in float32.
template <int KIND>
__global__ __launch_bounds__(256) void am_split_sum(float* __restrict__ vc_all, float* __restrict__ ws, AmCfg C,
                                                    SeqTable T) {
  __shared__ float tile[64][kD + 1];
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  const int R = C.R;
  AmWs W = am_ws(ws, T, i, C);
  const int ldm = W.ldm, Np = W.Np;
  const int nb = KIND == 0 ? (R + 63) / 64 : ldm / 64;
  const int local = t - T.start[i];
  const int h = local / nb, blk = local - h * nb;
  const int lim = KIND == 0 ? R : m;
  const int S = KIND == 0 ? C.S1 : C.S2;
  const int64_t unit = (int64_t)s * C.H + h;
  const int64_t stride = KIND == 0 ? pad64((int64_t)C.H * R * kD) : pad64((int64_t)C.H * ldm * kD);
  const float* src = KIND == 0 ? W.Zp + (int64_t)h * R * kD : W.Up + (int64_t)h * ldm * kD;
  const float eta = W.eta[h];
  for (int x = threadIdx.x; x < 64 * (kD / 4); x += 256) {
    const int row = blk * 64 + (x >> 5), c4 = x & 31;
    float4 val = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (row < lim) {
      const int64_t o = (int64_t)row * kD + 4 * c4;
      float4 a = *reinterpret_cast<const float4*>(src + o);
      for (int sp = 1; sp < S; ++sp) {
        const float4 p = *reinterpret_cast<const float4*>(src + sp * stride + o);
        a.x += p.x;
        a.y += p.y;
        a.z += p.z;
        a.w += p.w;
      }
      const int64_t ox = ((int64_t)h * Np + row) * kD + 4 * c4;
      if constexpr (KIND == 0) {
        float4 y = *reinterpret_cast<const float4*>(W.Y + (int64_t)h * R * kD + o);
        for (int tp = 1; tp < C.St; ++tp) {  // the target's key splits, in order
          const float4 yp = *reinterpret_cast<const float4*>(W.Y + tp * stride + (int64_t)h * R * kD + o);
          y.x += yp.x;
          y.y += yp.y;
          y.z += yp.z;
          y.w += yp.w;
        }
        val = make_float4(a.x - y.x, a.y - y.y, a.z - y.z, a.w - y.w);
        if (W.rside) {
          *reinterpret_cast<float4*>(W.X + ox) = val;
          *reinterpret_cast<float4*>(W.Sx + ox) = val;
        }
      } else {
        if (C.mode == 0) {
          float4* d = reinterpret_cast<float4*>(vc_all + unit * C.m_max * (int64_t)kD + o);
          float4 v = *d;
          v.x -= eta * a.x;
          v.y -= eta * a.y;
          v.z -= eta * a.z;
          v.w -= eta * a.w;
          *d = v;
          val = v;
        } else {
          val = a;
          *reinterpret_cast<float4*>(W.X + ox) = val;
          *reinterpret_cast<float4*>(W.Sx + ox) = val;
        }
      }
    }
    float* tr = &tile[x >> 5][4 * c4];
    tr[0] = val.x;
    tr[1] = val.y;
    tr[2] = val.z;
    tr[3] = val.w;
  }
  __syncthreads();
  const int pitch = KIND == 0 ? W.Rp : ldm;
  float* base = KIND == 0 ? W.ZT : W.VT;
  float* dst = base + (int64_t)h * kD * pitch + blk * 64;
  for (int q = threadIdx.x; q < kD * 8; q += 256) {
    const int d = q >> 3, gq = q & 7;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = tile[8 * gq + e][d];
    put_split8(dst + (int64_t)d * pitch, gq, x);
  }
}

// ------------------------------------------------------------------------------------------------
// Start: w = 1 (w' = exp(ME - Mz)) and Vc = the kept keys' values (float32); finish:
// beta = log w' - (ME - Mz) (-inf for w' = 0).
// Work item = (seq, head, 256 kept entries).
// ------------------------------------------------------------------------------------------------
template <int LAYOUT>
__global__ __launch_bounds__(256) void am_init(const uint16_t* __restrict__ v, const int32_t* __restrict__ table,
                                               int max_blocks, const int32_t* __restrict__ kept, float* __restrict__ w_all,
                                               float* __restrict__ vc_all, const float* __restrict__ ws, int64_t n_max,
                                               AmCfg C, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], n = T.n[i], s = T.first + i;
  const int cb = (m + 255) / 256;
  const int local = t - T.start[i];
  const int h = local / cb;
  const int j = (local - h * cb) * 256 + threadIdx.x;
  AmWs W = am_ws(const_cast<float*>(ws), T, i, C);
  if (j >= W.ldm) return;
  float* vt = W.VT + (int64_t)h * kD * W.ldm;  // split rows of Vc^T: column j of each
  if (j >= m) {  // padding columns of Vc^T are zero
    for (int d = 0; d < kD; ++d) put_split1(vt + (int64_t)d * W.ldm, j, 0.0f);
    return;
  }
  const int64_t unit = (int64_t)s * C.H + h;
  const int32_t* map = LAYOUT == kPaged ? table + (int64_t)s * max_blocks
                                        : (LAYOUT == kSlots ? table + unit * n_max : nullptr);
  w_all[unit * C.m_max + j] = __builtin_amdgcn_exp2f((W.ME[h] - W.M[h]) * kLog2e);  // w = 1 in scaled units
  const int key = min(max(kept[unit * C.m_max + j], 0), n - 1);
  const u32x4* row = key_row<LAYOUT>(v, map, C.H, h, n_max, unit, T.kofs[i] + key);
  float* dst = vc_all + (unit * C.m_max + j) * (int64_t)kD;
#pragma unroll 4
  for (int ch = 0; ch < kD / 8; ++ch) {
    const u32x4 raw = row[ch];
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf16_lo(wd[e]), hi = bf16_hi(wd[e]);
      dst[ch * 8 + 2 * e] = lo;
      dst[ch * 8 + 2 * e + 1] = hi;
      put_split1(vt + (int64_t)(ch * 8 + 2 * e) * W.ldm, j, lo);
      put_split1(vt + (int64_t)(ch * 8 + 2 * e + 1) * W.ldm, j, hi);
    }
  }
}

__global__ __launch_bounds__(256) void am_finish(float* __restrict__ w_all, const float* __restrict__ ws, AmCfg C,
                                                 SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  const int cb = (m + 255) / 256;
  const int local = t - T.start[i];
  const int h = local / cb;
  const int j = (local - h * cb) * 256 + threadIdx.x;
  if (j >= m) return;
  AmWs W = am_ws(const_cast<float*>(ws), T, i, C);
  float* w = w_all + ((int64_t)s * C.H + h) * C.m_max + j;
  *w = *w > 0.0f ? __logf(*w) - (W.ME[h] - W.M[h]) : -INFINITY;
}

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------
#define KVC_AM_LAYOUT(KERNEL, TARGS, ...)                                             \
  do {                                                                                \
    if (layout == kPaged) KERNEL<kPaged TARGS><<<grid, block, 0, st>>>(__VA_ARGS__);  \
    else if (layout == kSlots) KERNEL<kSlots TARGS><<<grid, block, 0, st>>>(__VA_ARGS__); \
    else KERNEL<kContig TARGS><<<grid, block, 0, st>>>(__VA_ARGS__);                  \
  } while (0)
#define KVC_COMMA ,

// Work items per head of each kernel.
int am_row_tiles(int R) { return (R + 63) / 64; }
int am_col_items(int m) { return (m + 255) / 256; }
int64_t am_key_tiles(int m) { return pad64(m) / 64; }
int am_stages_rows(int m) { return (int)(pad64(m) / 32); }
int am_stages_cols(int R) { return (R + 31) / 32; }

hipError_t launch_am_stats(const float* lse, float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  am_stats<<<dim3(T.total), dim3(64), 0, st>>>(lse, ws, C, T);
  return hipGetLastError();
}

hipError_t launch_am_me(float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  am_me<<<dim3(T.total), dim3(64), 0, st>>>(ws, C, T);
  return hipGetLastError();
}

hipError_t launch_am_cols_fin(int mode, float* w, float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  dim3 grid(T.total), block(256);
  if (mode == 1) am_cols_fin<1><<<grid, block, 0, st>>>(w, ws, C, T);
  else am_cols_fin<0><<<grid, block, 0, st>>>(w, ws, C, T);
  return hipGetLastError();
}

hipError_t launch_am_eta(float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  am_eta<<<dim3(T.total), dim3(256), 0, st>>>(ws, C, T);
  return hipGetLastError();
}

hipError_t launch_am_target(int layout, const void* q, const void* k, const void* v, const int32_t* table,
                            int max_blocks, const int32_t* vtable, int vmax_blocks, const float* lse, float* ws,
                            int64_t n_max, float scale, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  dim3 grid(T.total), block(kTgtThreads);
  KVC_AM_LAYOUT(am_target, , qq, kk, vv, table, max_blocks, vtable, vmax_blocks, lse, ws, n_max, scale, C, T);
  return hipGetLastError();
}

hipError_t launch_am_gemm(int kind, float* vc, float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  dim3 grid(T.total), block(kRingThreads);
  if (kind == 0) am_gemm<0><<<grid, block, 0, st>>>(vc, ws, C, T);
  else am_gemm<1><<<grid, block, 0, st>>>(vc, ws, C, T);
  return hipGetLastError();
}

hipError_t launch_am_step(float* vc, float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  am_step<<<dim3(T.total), dim3(kStepThreads), 0, st>>>(vc, ws, C, T);
  return hipGetLastError();
}

hipError_t launch_am_gram(float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  am_gram<<<dim3(T.total), dim3(kRingThreads), 0, st>>>(ws, C, T);
  return hipGetLastError();
}

hipError_t launch_am_split_sum(int kind, float* vc, float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  dim3 grid(T.total), block(256);
  if (kind == 0) am_split_sum<0><<<grid, block, 0, st>>>(vc, ws, C, T);
  else am_split_sum<1><<<grid, block, 0, st>>>(vc, ws, C, T);
  return hipGetLastError();
}

hipError_t launch_am_init(int layout, const void* v, const int32_t* table, int max_blocks, const int32_t* kept,
                          float* w, float* vc, const float* ws, int64_t n_max, const AmCfg& C, const SeqTable& T,
                          hipStream_t st) {
  const auto* vv = static_cast<const uint16_t*>(v);
  dim3 grid(T.total), block(256);
  KVC_AM_LAYOUT(am_init, , vv, table, max_blocks, kept, w, vc, ws, n_max, C, T);
  return hipGetLastError();
}

hipError_t launch_am_gather(int layout, const void* k, const int32_t* table, int max_blocks, const int32_t* kept,
                            float* ws, int64_t n_max, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  const auto* kk = static_cast<const uint16_t*>(k);
  dim3 grid(T.total), block(256);
  KVC_AM_LAYOUT(am_gather, , kk, table, max_blocks, kept, ws, n_max, C, T);
  return hipGetLastError();
}

hipError_t launch_am_bias(int mode, const void* q, const float* w, const float* lse, float* ws, float scale,
                          const AmCfg& C, const SeqTable& T, hipStream_t st) {
  const auto* qq = static_cast<const uint16_t*>(q);
  dim3 grid(T.total), block(256);
  block = dim3(kBiasThreads);
  if (mode == 0) am_bias<0><<<grid, block, 0, st>>>(qq, w, lse, ws, scale, C, T);
  else if (mode == 1) am_bias<1><<<grid, block, 0, st>>>(qq, w, lse, ws, scale, C, T);
  else if (mode == 2) am_bias<2><<<grid, block, 0, st>>>(qq, w, lse, ws, scale, C, T);
  else am_bias<3><<<grid, block, 0, st>>>(qq, w, lse, ws, scale, C, T);
  return hipGetLastError();
}

int64_t am_gather_items(int m) { return pad256(m) / 64; }

hipError_t launch_am_finish(float* w, const float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  am_finish<<<dim3(T.total), dim3(256), 0, st>>>(w, ws, C, T);
  return hipGetLastError();
}

}  // namespace kvc
