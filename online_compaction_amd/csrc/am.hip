// Attention Matching ("Practical Online KV Cache Compaction for LLM Agents", design-space
// section, the AM equations): after the top-m keys K_C are chosen, an additive bias beta with
//   min_beta || exp(Q K_C^T + beta) 1_m - exp(Q K^T) 1_n ||^2
// and compact values V_C with
//   min_V_C || A_hat(Q; K_C, beta, V_C) - A(Q; K, V) ||_F^2.
// With w = exp(beta) the first is non-negative least squares in w; the second, with
// P_C = diag(1 / (E w)) E diag(w) the compacted attention, is least squares in V_C.
//
// Per unit the kernels materialise E_ij = exp(c q_i . k_Cj - ME) (ME the largest kept logit) and
// the target A(Q; K, V) = P_full V, P_full_ij = exp(c q_i . k_j - LSE_i) over all n keys (P_full
// itself only one 64-key chunk at a time, in registers and LDS), then iterate:
//   beta: w' <- w' * (E^T z) / (E^T E w') (multiplicative NNLS updates), z_i = exp(LSE_i - Mz);
//   V_C:  V <- V - eta P_C^T (P_C V - Y) from the kept keys' values (Landweber),
//         eta = 1 / max_j sum_i (P_C)_ij.
// E and z carry separate factors so that neither underflows in float32 (Mz = the largest LSE,
// lowered to ME + 80 if the kept logits lie far below it). The updates are scale-equivariant:
// with w' = exp(ME - Mz) w they are the updates of w = exp(beta) from w = 1 on the unscaled
// exponentials, so w' starts at exp(ME - Mz) and beta = log w' - (ME - Mz). Once beta is fixed,
// E is overwritten in place by P_C and P_C^T is written beside it (PT), so both value products
// read their left operand row by row.
// The QK^T products use v_mfma_f32_16x16x32_bf16 on the stored bf16 rows; the solver's matrix
// products run on the same instruction with their float32 operands stored split into bf16 high
// and low parts (three products each); the vector products are plain VALU. Every
// reduction has a fixed order (split sums land in partial buffers that one pass adds up in
// order), so a fit is reproducible bit for bit.
//
// Workspace of sequence i (floats, from T.off[i]; H heads, R rows, m = T.m[i], n = T.n[i],
// ldm = m rounded up to 64, NR = ceil(R / 64), S1 / S2 the split counts of the two value
// products; every array starts on a 256-byte boundary):
//   E [H][R][ldm] | PT [H][ldm][R] | Y [H][R][128] | Z [H][R][128] | Zp [S1 > 1 ? S1 : 0][H][R][128] |
//   Up [S2 > 1 ? S2 : 0][H][ldm][128] | part [H][NR][ldm] | u [H][R] | b [H][ldm] |
//   Mz [H] | eta [H] | ME [H] | ME as an ordered integer key [H]
// Columns m .. ldm-1 of E hold zeros (logit -inf), so tiles never need a column bound on E.
#include "mfma_common.h"

namespace kvc {

using namespace mfma;

struct AmCfg {
  int H, R, m_max, S1, S2;
};

namespace {

constexpr int kD = kHeadDim;
constexpr int kRowChunk = 64;  // rows per partial column sum

__host__ __device__ constexpr int64_t pad64(int64_t x) { return (x + 63) & ~int64_t(63); }

// E / P_C [H][R][ldm], PT [H][ldm][Rp], ZT [H][128][Rp] and VT [H][128][ldm] (Rp = R rounded up
// to 64): P_C, PT, ZT and VT are held in the split layout below.
struct AmWs {
  float *E, *PT, *Y, *ZT, *VT, *Zp, *Up, *part, *u, *b, *M, *eta, *ME;
  uint32_t* mekey;
  int ldm, Rp;
};

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
  w.E = ws + T.off[i];
  w.PT = w.E + pad64(H * R * ldm);
  w.Y = w.PT + pad64(H * ldm * Rp);
  w.ZT = w.Y + pad64(H * R * kD);
  w.VT = w.ZT + pad64(H * kD * Rp);
  w.Zp = w.VT + pad64(H * kD * ldm);
  w.Up = w.Zp + (C.S1 > 1 ? C.S1 : 0) * pad64(H * R * kD);
  w.part = w.Up + (C.S2 > 1 ? C.S2 : 0) * pad64(H * ldm * kD);
  w.u = w.part + pad64(H * nr * ldm);
  w.b = w.u + pad64(H * R);
  w.M = w.b + pad64(H * ldm);
  w.eta = w.M + H;
  w.ME = w.eta + H;
  w.mekey = reinterpret_cast<uint32_t*>(w.ME + H);
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
int64_t am_seq_floats(int H, int R, int n, int m, int S1, int S2) {
  const int64_t ldm = pad64(m), nr = (R + kRowChunk - 1) / kRowChunk, Rp = pad64(R);
  const int64_t rk = pad64((int64_t)H * R * kD);
  return pad64((int64_t)H * R * ldm) + pad64((int64_t)H * ldm * Rp) + rk + pad64((int64_t)H * kD * Rp) +
         pad64((int64_t)H * kD * ldm) + (S1 > 1 ? S1 : 0) * rk +
         (S2 > 1 ? S2 : 0) * pad64((int64_t)H * ldm * kD) + pad64((int64_t)H * nr * ldm) + pad64((int64_t)H * R) +
         pad64((int64_t)H * ldm) + pad64(4 * (int64_t)H);
}

// ------------------------------------------------------------------------------------------------
// Kept-logit tiles of 64 rows x 64 kept keys into E: the raw logits c q_i . k_Cj, -inf in the
// padding columns; their maximum goes to an atomic per unit, and am_scale turns them into
// exponentials. Work item = (seq, head, row tile, key tile), key tile fastest. Both operands
// come straight from global memory (L2-resident).
// ------------------------------------------------------------------------------------------------
template <int LAYOUT>
__global__ __launch_bounds__(kThreads) void am_exp(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                   const int32_t* __restrict__ table, int max_blocks,
                                                   const int32_t* __restrict__ kept, float* __restrict__ ws,
                                                   int64_t n_max, float scale, AmCfg C, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int n = T.n[i], m = T.m[i];
  const int H = C.H, R = C.R;
  AmWs W = am_ws(ws, T, i, C);
  const int ld = W.ldm;
  const int s = T.first + i;
  const int rt_n = (R + 63) / 64, ct_n = (m + 63) / 64;
  int local = t - T.start[i];
  const int h = local / (rt_n * ct_n);
  local -= h * rt_n * ct_n;
  const int rt = local / ct_n, ct = local - rt * ct_n;
  const int64_t unit = (int64_t)s * H + h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int32_t* map = LAYOUT == kPaged ? table + (int64_t)s * max_blocks
                                        : (LAYOUT == kSlots ? table + unit * n_max : nullptr);

  const int row = rt * 64 + wave * 16 + c16;  // A operand row of this lane
  bf16x8 qa[4];
  const uint16_t* qrow = q + (unit * R + min(row, R - 1)) * (int64_t)kD;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qa[ks] = as_bf16x8(reinterpret_cast<const u32x4*>(qrow)[4 * ks + g]);
  float* out = W.E + ((int64_t)h * R) * ld;
  const int32_t* ku = kept + unit * C.m_max;
  float lmax = -INFINITY;
#pragma unroll 1
  for (int sub = 0; sub < 4; ++sub) {
    const int col = ct * 64 + sub * 16 + c16;  // B operand key of this lane
    const int key = min(max(ku[min(col, m - 1)], 0), n - 1);
    const u32x4* kr = key_row<LAYOUT>(k, map, H, h, n_max, unit, T.kofs[i] + key);
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma16(qa[ks], as_bf16x8(kr[4 * ks + g]), acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int orow = rt * 64 + wave * 16 + 4 * g + e;
      if (orow < R && col < ld) {
        const float l = acc[e] * scale;
        if (col < m) {
          out[(int64_t)orow * ld + col] = l;
          lmax = fmaxf(lmax, l);
        } else {
          out[(int64_t)orow * ld + col] = -INFINITY;
        }
      }
    }
  }
  // one atomic per workgroup at most: the four wave maxima meet in LDS, and the unit's running
  // maximum is read first (it only grows, so a stale read costs at most a redundant atomic)
  __shared__ float wmax[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o));
  if (lane == 0) wmax[wave] = lmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float bm = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const uint32_t key = float_key(bm);
    if (bm > -INFINITY && key > __atomic_load_n(W.mekey + h, __ATOMIC_RELAXED)) atomicMax(W.mekey + h, key);
  }
}

// Per unit, before am_exp: Mz = max_i LSE_i, and the kept-logit maximum reset. Work item = (seq, head).
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

// E <- exp(E - ME), ME the unit's largest kept logit; Mz lowered to ME + 80 when the kept keys
// lie far below the largest LSE (so that exp(ME - Mz), the start of w', stays in range).
// Work item = (seq, head, 4096 elements).
__global__ __launch_bounds__(256) void am_scale(float* __restrict__ ws, AmCfg C, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  AmWs W = am_ws(ws, T, i, C);
  const int64_t per = (int64_t)C.R * W.ldm;
  const int nb = (int)((per + 4095) / 4096);
  const int local = t - T.start[i];
  const int h = local / nb, blk = local - h * nb;
  const float me = key_float(W.mekey[h]);
  if (blk == 0 && threadIdx.x == 0) {
    W.ME[h] = me;
    W.M[h] = fminf(W.M[h], me + 80.0f);
  }
  float* e = W.E + (int64_t)h * per;
  for (int64_t x = (int64_t)blk * 4096 + threadIdx.x; x < min(per, (int64_t)(blk + 1) * 4096); x += 256)
    e[x] = __builtin_amdgcn_exp2f((e[x] - me) * kLog2e);
}

// ------------------------------------------------------------------------------------------------
// u = E w per row (one wave per row). Work item = (seq, head, 4 rows).
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void am_rows_dot(const float* __restrict__ w_all, float* __restrict__ ws, AmCfg C,
                                                   SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  const int R = C.R;
  const int rb = (R + 3) / 4;
  const int local = t - T.start[i];
  const int h = local / rb;
  const int r = (local - h * rb) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= R) return;
  AmWs W = am_ws(ws, T, i, C);
  const float* e = W.E + ((int64_t)h * R + r) * W.ldm;
  const float* w = w_all + ((int64_t)s * C.H + h) * C.m_max;
  float acc = 0.0f;
  for (int j = lane; j < m; j += 64) acc = __builtin_fmaf(e[j], w[j], acc);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) W.u[(int64_t)h * R + r] = acc;
}

// ------------------------------------------------------------------------------------------------
// Column products g_j = sum_i E_ij r_i in two passes: partial sums over chunks of 64 rows (one
// thread per column, rows in order), then the chunks added in order per column. With
//   MODE 0: r_i = exp(LSE_i - M)       -> b_j = g_j                          (E^T z, once)
//   MODE 1: r_i = u_i = (E w)_i        -> w_j <- w_j b_j / g_j, 0 if g_j = 0 (one NNLS step)
//   MODE 2: r_i = 1 / u_i              -> E_ij <- E_ij w_j / u_i in place (E becomes P_C),
//                                         b_j = sum_i (P_C)_ij (column sums, for the step size),
//                                         and P_C^T written to PT
// Partial work item = (seq, head, 256 columns, 64-row chunk); final = (seq, head, 256 columns).
// ------------------------------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void am_cols_part(const float* __restrict__ w_all, const float* __restrict__ lse,
                                                    float* __restrict__ ws, AmCfg C, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  const int R = C.R;
  AmWs W = am_ws(ws, T, i, C);
  const int ldm = W.ldm;
  const int cb_n = (ldm + 255) / 256, nr = (R + kRowChunk - 1) / kRowChunk;
  int local = t - T.start[i];
  const int rc = local % nr;
  local /= nr;
  const int cb = local % cb_n, h = local / cb_n;
  const int j = cb * 256 + threadIdx.x;
  const int64_t unit = (int64_t)s * C.H + h;
  const int r0 = rc * kRowChunk, r1 = min(R, r0 + kRowChunk);
  if constexpr (MODE == 2) {
    // P_C in place of E and P_C^T (row j of PT holds column j), both in the split layout, and
    // the column sums of P_C. The chunk's 64 x 256 block of P_C is staged in LDS (row pitch 257:
    // a column read is conflict-free); after the barrier every float of the block has been read,
    // so the block is rewritten in place, 8 consecutive columns of a row per group, and PT gets
    // 8 consecutive rows of a column per group (zeros for the rows past R up to Rp).
    __shared__ float tile[kRowChunk][257];
    float acc = 0.0f;
    float* E = W.E + (int64_t)h * R * ldm;
    if (j < ldm) {
      const float* u = W.u + (int64_t)h * R;
      const float wj = j < m ? w_all[unit * C.m_max + j] : 0.0f;
      for (int r = r0; r < r1; ++r) {
        const float x = E[(int64_t)r * ldm + j];
        const float pc = u[r] > 0.0f ? x * wj / u[r] : 0.0f;
        tile[r - r0][threadIdx.x] = pc;
        acc += pc;
      }
      W.part[((int64_t)h * nr + rc) * ldm + j] = acc;
    }
    __syncthreads();
    const int cols = min(256, ldm - cb * 256);  // a multiple of 64
    for (int q = threadIdx.x; q < kRowChunk * 32; q += 256) {
      const int rr = q >> 5, gq = q & 31;
      if (r0 + rr < r1 && 8 * gq < cols) put_split8(E + (int64_t)(r0 + rr) * ldm + cb * 256, gq, &tile[rr][8 * gq]);
    }
    const int Rp = W.Rp;
    for (int q = threadIdx.x; q < 256 * (kRowChunk / 8); q += 256) {
      const int c = q >> 3, gq = q & 7;
      if (c >= cols) continue;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = r0 + 8 * gq + e < r1 ? tile[8 * gq + e][c] : 0.0f;
      put_split8(W.PT + ((int64_t)h * ldm + cb * 256 + c) * Rp + r0, gq, x);
    }
  } else {
    if (j >= ldm) return;
    const float* e = W.E + (int64_t)h * R * ldm + j;
    const float* u = W.u + (int64_t)h * R;
    const float* lu = lse + unit * R;
    const float M = W.M[h];
    float acc = 0.0f;
    for (int r = r0; r < r1; ++r) {
      const float x = e[(int64_t)r * ldm];
      if constexpr (MODE == 0) acc = __builtin_fmaf(x, __builtin_amdgcn_exp2f((lu[r] - M) * kLog2e), acc);
      else acc = __builtin_fmaf(x, u[r], acc);
    }
    W.part[((int64_t)h * nr + rc) * ldm + j] = acc;
  }
}

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
  for (int rc = 0; rc < nr; ++rc) g += p[(int64_t)rc * ldm];
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
// Target Y = P V with P_ij = exp(c q_i . k_j - LSE_i) over all n keys, without materialising P
// (the weights of one 64-key chunk exist only in registers and a per-wave LDS tile).
// Work item = (seq, head, 64-row tile), 8 waves: wave w owns rows 16 (w % 4) .. + 15 of the tile
// and output columns 64 (w / 4) .. + 63 (the two halves recompute the same weights, a small
// part of the work). Per 64-key chunk, staged through double-buffered LDS (keys as bf16 rows,
// chunk c of row r at c ^ (r & 15); values transposed, one bf16 row of 64 keys per column):
//   S = Q K^T     16 v_mfma_f32_16x16x32_bf16 (the wave's query rows stay in registers),
//   P = exp2(S c log2(e) - LSE log2(e)), 0 for keys past n, through LDS into the A layout,
//   Y += P V      P split as hi + lo (bf16 each; V is bf16 already, so the two products
//                 P_hi V + P_lo V carry P to a relative 2^-16), 16 v_mfma_f32_16x16x32_bf16.
// ------------------------------------------------------------------------------------------------
namespace {
constexpr int kTgtThreads = 512;
constexpr int kVtPitch = 72;  // bf16 per transposed value row (64 keys + 8 padding)
constexpr int kPPitch = 68;   // per-wave weight tile pitch (float32)

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
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][kD * kVtPitch];
  __shared__ __attribute__((aligned(16))) float Ps[8][16 * kPPitch];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i], s = T.first + i;
  const int H = C.H, R = C.R;
  const int rt_n = (R + 63) / 64;
  const int local = t - T.start[i];
  const int h = local / rt_n, rt = local - h * rt_n;
  const int64_t unit = (int64_t)s * H + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int rw = wave & 3, dh = wave >> 2;
  AmWs W = am_ws(ws, T, i, C);
  const int32_t* map = LAYOUT == kPaged ? table + (int64_t)s * max_blocks
                                        : (LAYOUT == kSlots ? table + unit * n_max : nullptr);
  const int32_t* vmap = LAYOUT == kPaged ? vtable + (int64_t)s * vmax_blocks
                                         : (LAYOUT == kSlots ? vtable + unit * n_max : nullptr);
  const int kofs = T.kofs[i];

  // query rows of this wave (A operand of S), and the LSE of the lane's four output rows
  bf16x8 qa[4];
  {
    const int row = min(rt * 64 + 16 * rw + c16, R - 1);
    const u32x4* qr = reinterpret_cast<const u32x4*>(q + (unit * R + row) * (int64_t)kD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[ks] = as_bf16x8(qr[4 * ks + g]);
  }
  float lb[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) lb[e] = lse[unit * R + min(rt * 64 + 16 * rw + 4 * g + e, R - 1)] * kLog2e;
  const float cl = scale * kLog2e;

  // chunk staging: thread tid moves 16-byte piece tid & 15 of key rows tid >> 4 and 32 + (tid >> 4)
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
      const uint32_t wd[4] = {vr[x].x, vr[x].y, vr[x].z, vr[x].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // values d = 8 ch + 2 e, 8 ch + 2 e + 1 of this key
        Vt[buf][(8 * ch + 2 * e) * kVtPitch + key] = (uint16_t)(wd[e] & 0xffffu);
        Vt[buf][(8 * ch + 2 * e + 1) * kVtPitch + key] = (uint16_t)(wd[e] >> 16);
      }
    }
  };

  f32x4 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float* pw = Ps[wave];
  const int nch = (n + 63) / 64;
  load(0);
  store(0);
  __syncthreads();
#pragma unroll 1
  for (int ch = 0; ch < nch; ++ch) {
    const int buf = ch & 1;
    const bool more = ch + 1 < nch;
    if (more) load((ch + 1) * 64);
    const uint8_t* kb = Ks[buf];
    // S and the weights of 16 rows x 64 keys; lane (g, c16) holds rows 4g + e of key 16 sub + c16
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      f32x4 sacc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sacc = mfma16(qa[ks], *reinterpret_cast<const bf16x8*>(&kb[swz(16 * sub + c16, 4 * ks + g)]), sacc);
      const bool live = ch * 64 + 16 * sub + c16 < n;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pw[(4 * g + e) * kPPitch + 16 * sub + c16] =
            live ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], cl, -lb[e])) : 0.0f;
    }
    // Y += P V over the 64 keys in two steps of 32: lane group g takes keys 32 ks + 8 g .. + 7
    const uint16_t* vb = Vt[buf];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const float4* pr = reinterpret_cast<const float4*>(&pw[c16 * kPPitch + 32 * ks + 8 * g]);
      const float4 p0 = pr[0], p1 = pr[1];
      const float px[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      u32x4 ph, pl;
      split8(px, ph, pl);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bf16x8 vb8 = *reinterpret_cast<const bf16x8*>(&vb[(64 * dh + 16 * b + c16) * kVtPitch + 32 * ks + 8 * g]);
        acc[b] = mfma16(as_bf16x8(ph), vb8, acc[b]);
        acc[b] = mfma16(as_bf16x8(pl), vb8, acc[b]);
      }
    }
    if (more) store(buf ^ 1);
    __syncthreads();
  }
  float* out = W.Y + (int64_t)h * R * kD;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rt * 64 + 16 * rw + 4 * g + e;
      if (r < R) out[(int64_t)r * kD + 64 * dh + 16 * b + c16] = acc[b][e];
    }
}

// ------------------------------------------------------------------------------------------------
// The two products of a Landweber step, one 128 x 128 output tile per workgroup (four waves in a
// 2 x 2 grid, each 64 x 64: sixteen 16 x 16 accumulators), the contraction in stages of 32
// through double-buffered LDS with the next stage's global loads in flight during the current
// stage's MFMAs, and split over S workgroups whose partial tiles a second pass adds in order:
//   KIND 0: Z = P_C Vc - Y          (rows of P_C, contraction over kept keys)  -> Z, or partials Zp
//   KIND 1: Vc -= eta P_C^T Z        (columns of P_C, contraction over rows)    -> Vc, or partials Up
// The float32 operands are stored split (x = hi + lo with hi = bf16(x) and lo = bf16(x - hi),
// the layout of put_split8), and a product is taken as hi_a hi_b + hi_a lo_b + lo_a hi_b on
// v_mfma_f32_16x16x32_bf16 with float32 accumulation (the dropped lo_a lo_b and the rounding of
// lo leave a relative error near 2^-16 per product, against 2^-24 for float32 inputs, at a
// third of the float32 MFMA's cycles per product).
// LDS holds, per operand and half, 128 rows of 32 contraction indices (bf16, 64 bytes per row);
// 16-byte chunk c of row r sits at chunk position c ^ ((r >> 1) & 3), so each MFMA operand read
// (chunk g of 16 consecutive rows) is free of bank conflicts. Lane group g of an MFMA supplies
// contraction indices 8g .. 8g + 7 on both operands.
// Work item = (seq, head, output tile, split), split fastest.
// ------------------------------------------------------------------------------------------------
namespace {
constexpr int kGTile = 128;

__device__ __forceinline__ int gswz(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 1) & 3)) << 4); }
}  // namespace

template <int KIND>
__global__ __launch_bounds__(256, 2) void am_gemm(float* __restrict__ vc_all, float* __restrict__ ws, AmCfg C,
                                                  SeqTable T) {
  __shared__ __attribute__((aligned(16))) uint8_t Ah[2][kGTile * 64], Al[2][kGTile * 64];
  __shared__ __attribute__((aligned(16))) uint8_t Bh[2][kGTile * 64], Bl[2][kGTile * 64];
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  const int R = C.R;
  AmWs W = am_ws(ws, T, i, C);
  const int ldm = W.ldm;
  const int S = KIND == 0 ? C.S1 : C.S2;
  const int rows = KIND == 0 ? R : ldm;  // output rows
  const int tiles = (rows + kGTile - 1) / kGTile;
  int local = t - T.start[i];
  const int sp = local % S;
  local /= S;
  const int tile = local % tiles, h = local / tiles;
  const int64_t unit = (int64_t)s * C.H + h;
  const float* PC = W.E + (int64_t)h * R * ldm;           // split rows of P_C
  const float* PTh = W.PT + (int64_t)h * ldm * W.Rp;      // split rows of P_C^T
  const float* VTh = W.VT + (int64_t)h * kD * ldm;        // split rows of Vc^T
  const float* ZTh = W.ZT + (int64_t)h * kD * W.Rp;       // split rows of Z^T
  const int nst = KIND == 0 ? ldm / 32 : (R + 31) / 32;
  const int per = (nst + S - 1) / S;
  const int st0 = sp * per, st1 = min(nst, st0 + per);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int wr = wave >> 1, wc = wave & 1;

  // staging: A row ar of the tile, contraction indices 16 ak .. + 15; B column bd, indices
  // 16 bk .. + 15 (chunks 2 ak, 2 ak + 1 and 2 bk, 2 bk + 1). Every operand is stored split, so
  // a thread's 16 indices are 64 contiguous bytes: high parts of the first 8, their low parts,
  // then the same for the next 8, copied to the high and low LDS tiles unchanged. The
  // contraction never leaves the stored rows (ldm and Rp are multiples of 64).
  const int ar = tid >> 1, ak = tid & 1;
  const int bd = tid & 127, bk = tid >> 7;
  const int arow = tile * kGTile + ar;                    // A row: output row of the tile
  const bool alive = arow < (KIND == 0 ? R : ldm);
  const u32x4* asrc = reinterpret_cast<const u32x4*>(
      KIND == 0 ? PC + (int64_t)min(arow, R - 1) * ldm + 16 * ak : PTh + (int64_t)min(arow, ldm - 1) * W.Rp + 16 * ak);
  const u32x4* bsrc = reinterpret_cast<const u32x4*>(KIND == 0 ? VTh + (int64_t)bd * ldm + 16 * bk
                                                               : ZTh + (int64_t)bd * W.Rp + 16 * bk);
  u32x4 ra[4], rb[4];
  auto load = [&](int stg) {
    const int o = stg * 8;  // 32 indices = 8 u32x4 per row
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ra[c] = asrc[o + c];
      rb[c] = bsrc[o + c];
    }
    if (!alive) {
#pragma unroll
      for (int c = 0; c < 4; ++c) ra[c] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      *reinterpret_cast<u32x4*>(&Ah[buf][gswz(ar, 2 * ak + c)]) = ra[2 * c];
      *reinterpret_cast<u32x4*>(&Al[buf][gswz(ar, 2 * ak + c)]) = ra[2 * c + 1];
      *reinterpret_cast<u32x4*>(&Bh[buf][gswz(bd, 2 * bk + c)]) = rb[2 * c];
      *reinterpret_cast<u32x4*>(&Bl[buf][gswz(bd, 2 * bk + c)]) = rb[2 * c + 1];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (st0 < st1) {
    load(st0);
    store(0);
    __syncthreads();
#pragma unroll 1
    for (int stg = st0; stg < st1; ++stg) {
      const int buf = (stg - st0) & 1;
      const bool more = stg + 1 < st1;
      if (more) load(stg + 1);
      bf16x8 bh[4], bl[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int o = gswz(64 * wc + 16 * b + c16, g);
        bh[b] = *reinterpret_cast<const bf16x8*>(&Bh[buf][o]);
        bl[b] = *reinterpret_cast<const bf16x8*>(&Bl[buf][o]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int o = gswz(64 * wr + 16 * a + c16, g);
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&Ah[buf][o]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Al[buf][o]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          acc[a][b] = mfma16(ah, bh[b], acc[a][b]);
          acc[a][b] = mfma16(ah, bl[b], acc[a][b]);
          acc[a][b] = mfma16(al, bh[b], acc[a][b]);
        }
      }
      if (more) store(buf ^ 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = tile * kGTile + 64 * wr + 16 * a + 4 * g + e;
        const int col = 64 * wc + 16 * b + c16;
        if constexpr (KIND == 0) {  // Z = P_C Vc - Y, kept as split rows of Z^T (zeros past R)
          const int64_t o = (int64_t)h * R * kD + (int64_t)r * kD + col;
          if (S == 1) {
            if (r < W.Rp) put_split1(W.ZT + ((int64_t)h * kD + col) * W.Rp, r, r < R ? acc[a][b][e] - W.Y[o] : 0.0f);
          } else if (r < R) {
            W.Zp[(int64_t)sp * pad64((int64_t)C.H * R * kD) + o] = acc[a][b][e];
          }
        } else {  // Vc -= eta P_C^T Z, with its split rows of Vc^T (zeros past m)
          const int64_t o = (int64_t)r * kD + col;
          if (S == 1) {
            if (r < ldm) {
              float v = 0.0f;
              if (r < m) {
                float* d = vc_all + unit * C.m_max * (int64_t)kD + o;
                v = *d - W.eta[h] * acc[a][b][e];
                *d = v;
              }
              put_split1(W.VT + ((int64_t)h * kD + col) * ldm, r, v);
            }
          } else if (r < ldm) {
            W.Up[(int64_t)sp * pad64((int64_t)C.H * ldm * kD) + (int64_t)h * ldm * kD + o] = acc[a][b][e];
          }
        }
      }
}

// Output tiles of the Landweber products: KIND 0 over the R rows, KIND 1 over the ldm kept keys.
int am_gemm_tiles(int rows) { return (rows + kGTile - 1) / kGTile; }

// Split sums, in split order: Z = sum_s Zp[s] - Y (KIND 0, work item = (seq, head, 64 rows)) and
// Vc_j -= eta sum_s Up[s]_j (KIND 1, work item = (seq, head, 64 kept keys)). The block's results
// (zeros past R, or past m) are staged in LDS and leave as split rows of Z^T or Vc^T, the form
// the next product reads; Vc itself is also kept in float32.
template <int KIND>
__global__ __launch_bounds__(256) void am_split_sum(float* __restrict__ vc_all, float* __restrict__ ws, AmCfg C,
                                                    SeqTable T) {
  __shared__ float tile[64][kD + 1];
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  const int R = C.R;
  AmWs W = am_ws(ws, T, i, C);
  const int ldm = W.ldm;
  const int nb = KIND == 0 ? (R + 63) / 64 : ldm / 64;
  const int local = t - T.start[i];
  const int h = local / nb, blk = local - h * nb;
  const int lim = KIND == 0 ? R : m;
  const int S = KIND == 0 ? C.S1 : C.S2;
  const int64_t unit = (int64_t)s * C.H + h;
  const int64_t stride = KIND == 0 ? pad64((int64_t)C.H * R * kD) : pad64((int64_t)C.H * ldm * kD);
  const float* src = (KIND == 0 ? W.Zp + (int64_t)h * R * kD : W.Up + (int64_t)h * ldm * kD);
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
      if constexpr (KIND == 0) {
        const float4 y = *reinterpret_cast<const float4*>(W.Y + (int64_t)h * R * kD + o);
        val = make_float4(a.x - y.x, a.y - y.y, a.z - y.z, a.w - y.w);
      } else {
        const float f = W.eta[h];
        float4* d = reinterpret_cast<float4*>(vc_all + unit * C.m_max * (int64_t)kD + o);
        float4 v = *d;
        v.x -= f * a.x;
        v.y -= f * a.y;
        v.z -= f * a.z;
        v.w -= f * a.w;
        *d = v;
        val = v;
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
  float* dst = (KIND == 0 ? W.ZT : W.VT) + (int64_t)h * kD * pitch + blk * 64;
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
int64_t am_exp_items(int R, int cols) { return (int64_t)((R + 63) / 64) * ((cols + 63) / 64); }
int64_t am_scale_items(int R, int m) { return ((int64_t)R * pad64(m) + 4095) / 4096; }
int am_row_tiles(int R) { return (R + 63) / 64; }
int am_dot_row_items(int R) { return (R + 3) / 4; }
int am_col_items(int m) { return (m + 255) / 256; }
int64_t am_col_part_items(int R, int m) { return (int64_t)((pad64(m) + 255) / 256) * ((R + kRowChunk - 1) / kRowChunk); }
int64_t am_key_tiles(int m) { return pad64(m) / 64; }
int am_stages_rows(int m) { return (int)(pad64(m) / 32); }
int am_stages_cols(int R) { return (R + 31) / 32; }

hipError_t launch_am_exp(int layout, const void* q, const void* k, const int32_t* table, int max_blocks,
                         const int32_t* kept, float* ws, int64_t n_max, float scale, const AmCfg& C, const SeqTable& T,
                         hipStream_t st) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  dim3 grid(T.total), block(kThreads);
  KVC_AM_LAYOUT(am_exp, , qq, kk, table, max_blocks, kept, ws, n_max, scale, C, T);
  return hipGetLastError();
}

hipError_t launch_am_stats(const float* lse, float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  am_stats<<<dim3(T.total), dim3(64), 0, st>>>(lse, ws, C, T);
  return hipGetLastError();
}

hipError_t launch_am_scale(float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  am_scale<<<dim3(T.total), dim3(256), 0, st>>>(ws, C, T);
  return hipGetLastError();
}

hipError_t launch_am_rows_dot(const float* w, float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  am_rows_dot<<<dim3(T.total), dim3(256), 0, st>>>(w, ws, C, T);
  return hipGetLastError();
}

hipError_t launch_am_cols_part(int mode, const float* w, const float* lse, float* ws, const AmCfg& C,
                               const SeqTable& T, hipStream_t st) {
  dim3 grid(T.total), block(256);
  if (mode == 0) am_cols_part<0><<<grid, block, 0, st>>>(w, lse, ws, C, T);
  else if (mode == 1) am_cols_part<1><<<grid, block, 0, st>>>(w, lse, ws, C, T);
  else am_cols_part<2><<<grid, block, 0, st>>>(w, lse, ws, C, T);
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
  dim3 grid(T.total), block(256);
  if (kind == 0) am_gemm<0><<<grid, block, 0, st>>>(vc, ws, C, T);
  else am_gemm<1><<<grid, block, 0, st>>>(vc, ws, C, T);
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

hipError_t launch_am_finish(float* w, const float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st) {
  am_finish<<<dim3(T.total), dim3(256), 0, st>>>(w, ws, C, T);
  return hipGetLastError();
}

}  // namespace kvc
