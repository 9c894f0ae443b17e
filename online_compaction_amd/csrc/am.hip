// Attention Matching ("Practical Online KV Cache Compaction for LLM Agents", design-space
// section, the AM equations): after the top-m keys K_C are chosen, an additive bias beta with
//   min_beta || exp(Q K_C^T + beta) 1_m - exp(Q K^T) 1_n ||^2
// and compact values V_C with
//   min_V_C || A_hat(Q; K_C, beta, V_C) - A(Q; K, V) ||_F^2.
// With w = exp(beta) the first is non-negative least squares in w; the second, with
// P = diag(1 / (E w)) E diag(w) the compacted attention, is least squares in V_C.
//
// Per unit the kernels materialise E_ij = exp(c q_i . k_Cj - ME) (ME the largest kept logit) and,
// for the target A(Q; K, V) = P_full V, P_full_ij = exp(c q_i . k_j - LSE_i) over all n keys, then
// iterate:
//   beta: w' <- w' * (E^T z) / (E^T E w') (multiplicative NNLS updates), z_i = exp(LSE_i - Mz);
//   V_C:  V <- V - eta P^T (P V - Y) from the kept keys' values (Landweber), eta = 1 / max_j sum_i P_ij.
// E and z carry separate factors so that neither underflows in float32 (Mz = the largest LSE,
// lowered to ME + 80 if the kept logits lie far below it). The updates are scale-equivariant:
// with w' = exp(ME - Mz) w they are the updates of w = exp(beta) from w = 1 on the unscaled
// exponentials, so w' starts at exp(ME - Mz) and beta = log w' - (ME - Mz).
// The QK^T products use v_mfma_f32_16x16x32_bf16 on the stored bf16 rows; the solver products
// use v_mfma_f32_16x16x4_f32 (float32 throughout); the vector products are plain VALU.
//
// Workspace of sequence i (floats, from T.off[i]; H heads, R rows, m = T.m[i], n = T.n[i]):
//   E [H][R][m] | P [H][R][n] | Y [H][R][128] | Tm [H][R][128] | u [H][R] | b [H][m] |
//   Mz [H] | eta [H] | ME [H] | ME as an ordered integer key [H]
#include "mfma_common.h"

namespace kvc {

using namespace mfma;

namespace {

constexpr int kD = kHeadDim;

struct AmWs {
  float *E, *P, *Y, *Tm, *u, *b, *M, *eta, *ME;
  uint32_t* mekey;
};

__device__ __forceinline__ AmWs am_ws(float* ws, const SeqTable& T, int i, int H, int R) {
  const int64_t m = T.m[i], n = T.n[i];
  AmWs w;
  w.E = ws + T.off[i];
  w.P = w.E + (int64_t)H * R * m;
  w.Y = w.P + (int64_t)H * R * n;
  w.Tm = w.Y + (int64_t)H * R * kD;
  w.u = w.Tm + (int64_t)H * R * kD;
  w.b = w.u + (int64_t)H * R;
  w.M = w.b + (int64_t)H * m;
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

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// Logit tiles of 64 rows x 64 keys: into E the raw kept logits c q_i . k_Cj (ALL = false; their
// maximum goes to an atomic per unit, and am_scale turns them into exponentials), into P the
// weights exp(c q_i . k_j - LSE_i) over every key (ALL = true). Work item = (seq, head, row tile,
// key tile), key tile fastest. Both operands come straight from global memory (L2-resident).
// ------------------------------------------------------------------------------------------------
template <int LAYOUT, bool ALL>
__global__ __launch_bounds__(kThreads) void am_exp(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                   const int32_t* __restrict__ table, int max_blocks,
                                                   const int32_t* __restrict__ kept, int m_max,
                                                   const float* __restrict__ lse, float* __restrict__ ws, int H,
                                                   int R, int64_t n_max, float scale, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int n = T.n[i], m = T.m[i];
  const int cols = ALL ? n : m;
  const int s = T.first + i;
  const int rt_n = (R + 63) / 64, ct_n = (cols + 63) / 64;
  int local = t - T.start[i];
  const int h = local / (rt_n * ct_n);
  local -= h * rt_n * ct_n;
  const int rt = local / ct_n, ct = local - rt * ct_n;
  const int64_t unit = (int64_t)s * H + h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  AmWs W = am_ws(ws, T, i, H, R);
  const float* lu = lse + unit * R;
  const int32_t* map = LAYOUT == kPaged ? table + (int64_t)s * max_blocks
                                        : (LAYOUT == kSlots ? table + unit * n_max : nullptr);

  const int row = rt * 64 + wave * 16 + c16;  // A operand row of this lane
  bf16x8 qa[4];
  const uint16_t* qrow = q + (unit * R + min(row, R - 1)) * (int64_t)kD;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qa[ks] = as_bf16x8(reinterpret_cast<const u32x4*>(qrow)[4 * ks + g]);
  float* out = (ALL ? W.P : W.E) + ((int64_t)h * R) * cols;
  const int32_t* ku = kept + unit * m_max;
  float lmax = -INFINITY;
#pragma unroll 1
  for (int sub = 0; sub < 4; ++sub) {
    const int col = ct * 64 + sub * 16 + c16;  // B operand key of this lane
    const int key = ALL ? min(col, n - 1) : min(max(ku[min(col, m - 1)], 0), n - 1);
    const u32x4* kr = key_row<LAYOUT>(k, map, H, h, n_max, unit, T.kofs[i] + key);
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma16(qa[ks], as_bf16x8(kr[4 * ks + g]), acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int orow = rt * 64 + wave * 16 + 4 * g + e;
      if (orow < R && col < cols) {
        const float l = acc[e] * scale;
        if constexpr (ALL) {
          out[(int64_t)orow * cols + col] = __builtin_amdgcn_exp2f((l - lu[orow]) * kLog2e);
        } else {
          out[(int64_t)orow * cols + col] = l;
          lmax = fmaxf(lmax, l);
        }
      }
    }
  }
  if constexpr (!ALL) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o));
    if (lane == 0 && lmax > -INFINITY) atomicMax(W.mekey + h, float_key(lmax));
  }
}

// Per unit, before am_exp: Mz = max_i LSE_i, and the kept-logit maximum reset. Work item = (seq, head).
__global__ __launch_bounds__(64) void am_stats(const float* __restrict__ lse, float* __restrict__ ws, int H, int R,
                                               SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int s = T.first + i, h = t - T.start[i];
  AmWs W = am_ws(ws, T, i, H, R);
  const float* lu = lse + ((int64_t)s * H + h) * R;
  float mx = -INFINITY;
  for (int r = threadIdx.x; r < R; r += 64) mx = fmaxf(mx, lu[r]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (threadIdx.x == 0) {
    W.M[h] = mx;
    W.mekey[h] = 0u;  // below every float's key
  }
}

// E <- exp(E - ME), ME the unit's largest kept logit; Mz lowered to ME + 80 when the kept keys
// lie far below the largest LSE (so that exp(ME - Mz), the start of w', stays in range).
// Work item = (seq, head, 256 x 16 elements).
__global__ __launch_bounds__(256) void am_scale(float* __restrict__ ws, int H, int R, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i];
  const int64_t per = (int64_t)R * m;
  const int nb = (int)((per + 4095) / 4096);
  const int local = t - T.start[i];
  const int h = local / nb, blk = local - h * nb;
  AmWs W = am_ws(ws, T, i, H, R);
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
__global__ __launch_bounds__(256) void am_rows_dot(const float* __restrict__ w_all, float* __restrict__ ws, int H,
                                                   int R, int m_max, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  const int rb = (R + 3) / 4;
  const int local = t - T.start[i];
  const int h = local / rb;
  const int r = (local - h * rb) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= R) return;
  AmWs W = am_ws(ws, T, i, H, R);
  const float* e = W.E + ((int64_t)h * R + r) * m;
  const float* w = w_all + ((int64_t)s * H + h) * m_max;
  float acc = 0.0f;
  for (int j = lane; j < m; j += 64) acc = __builtin_fmaf(e[j], w[j], acc);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) W.u[(int64_t)h * R + r] = acc;
}

// ------------------------------------------------------------------------------------------------
// Column products g_j = sum_i E_ij r_i (one thread per column, rows in order), with
//   MODE 0: r_i = exp(LSE_i - M)       -> b_j = g_j                      (E^T z, once)
//   MODE 1: r_i = u_i = (E w)_i        -> w_j <- w_j b_j / g_j, 0 if g_j = 0  (one NNLS step)
//   MODE 2: r_i = 1 / u_i              -> b_j = w_j g_j (column sums of P, for the step size)
// Work item = (seq, head, 256 columns).
// ------------------------------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void am_cols_dot(float* __restrict__ w_all, const float* __restrict__ lse,
                                                   float* __restrict__ ws, int H, int R, int m_max, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  const int cb = (m + 255) / 256;
  const int local = t - T.start[i];
  const int h = local / cb;
  const int j = (local - h * cb) * 256 + threadIdx.x;
  if (j >= m) return;
  const int64_t unit = (int64_t)s * H + h;
  AmWs W = am_ws(ws, T, i, H, R);
  const float* e = W.E + (int64_t)h * R * m + j;
  const float* u = W.u + (int64_t)h * R;
  const float* lu = lse + unit * R;
  const float M = W.M[h];
  float acc = 0.0f;
  for (int r = 0; r < R; ++r) {
    float rv;
    if constexpr (MODE == 0) rv = __builtin_amdgcn_exp2f((lu[r] - M) * kLog2e);
    else if constexpr (MODE == 1) rv = u[r];
    else rv = u[r] > 0.0f ? 1.0f / u[r] : 0.0f;
    acc = __builtin_fmaf(e[(int64_t)r * m], rv, acc);
  }
  float* w = w_all + unit * m_max;
  if constexpr (MODE == 0) W.b[(int64_t)h * m + j] = acc;
  else if constexpr (MODE == 1) w[j] = acc > 0.0f ? w[j] * W.b[(int64_t)h * m + j] / acc : 0.0f;
  else W.b[(int64_t)h * m + j] = w[j] * acc;
}

// eta = 1 / max_j (column sums of P) per unit (0 when every column is empty). Work item = (seq, head).
__global__ __launch_bounds__(256) void am_eta(float* __restrict__ ws, int H, int R, SeqTable T) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i];
  const int h = t - T.start[i];
  AmWs W = am_ws(ws, T, i, H, R);
  float mx = 0.0f;
  for (int j = threadIdx.x; j < m; j += 256) mx = fmaxf(mx, W.b[(int64_t)h * m + j]);
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
// Row products out_i = sum_j A_ij B_j (128-wide rows), float32 MFMA, 64 rows x 128 per workgroup:
//   SRC 0: A = P (all n keys), B_j = V row of key j (bf16, through the view) -> Y
//   SRC 1: A = E (kept keys),  B_j = w_j * Vc_j (float32)                   -> Tm
// Work item = (seq, head, 64-row tile). LDS stages 16 columns of A and B at a time.
// ------------------------------------------------------------------------------------------------
template <int LAYOUT, int SRC>
__global__ __launch_bounds__(256) void am_rows_mm(const uint16_t* __restrict__ v, const int32_t* __restrict__ table,
                                                  int max_blocks, const float* __restrict__ w_all,
                                                  const float* __restrict__ vc_all, float* __restrict__ ws, int H,
                                                  int R, int64_t n_max, int m_max, SeqTable T) {
  __shared__ float As[64][17];
  __shared__ float Bs[16][kD];
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int n = T.n[i], m = T.m[i], s = T.first + i;
  const int cols = SRC == 0 ? n : m;
  const int rt_n = (R + 63) / 64;
  const int local = t - T.start[i];
  const int h = local / rt_n, rt = local - h * rt_n;
  const int64_t unit = (int64_t)s * H + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  AmWs W = am_ws(ws, T, i, H, R);
  const float* A = (SRC == 0 ? W.P : W.E) + (int64_t)h * R * cols;
  const int32_t* map = LAYOUT == kPaged ? table + (int64_t)s * max_blocks
                                        : (LAYOUT == kSlots ? table + unit * n_max : nullptr);
  const float* w = w_all + unit * m_max;
  const float* vc = vc_all + unit * m_max * (int64_t)kD;

  f32x4 acc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 1
  for (int c0 = 0; c0 < cols; c0 += 16) {
    // stage A[64 rows][16 cols] and B[16 cols][128]
    for (int x = tid; x < 64 * 16; x += 256) {
      const int rr = x >> 4, cc = x & 15;
      const int r = rt * 64 + rr, c = c0 + cc;
      As[rr][cc] = (r < R && c < cols) ? A[(int64_t)r * cols + c] : 0.0f;
    }
    for (int x = tid; x < 16 * (kD / 8); x += 256) {
      const int cc = x / (kD / 8), ch = x % (kD / 8);  // 8 elements per item
      const int c = c0 + cc;
      float vals[8];
      if (c < cols) {
        if constexpr (SRC == 0) {
          const u32x4 raw = key_row<LAYOUT>(v, map, H, h, n_max, unit, T.kofs[i] + c)[ch];
          const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vals[2 * e] = bf16_lo(wd[e]);
            vals[2 * e + 1] = bf16_hi(wd[e]);
          }
        } else {
          const float wj = w[c];
#pragma unroll
          for (int e = 0; e < 8; ++e) vals[e] = wj * vc[(int64_t)c * kD + ch * 8 + e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) Bs[cc][ch * 8 + e] = vals[e];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const float a = As[wave * 16 + c16][kk * 4 + g];
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[b] = mfma_f32(a, Bs[kk * 4 + g][b * 16 + c16], acc[b]);
    }
    __syncthreads();
  }
  float* out = (SRC == 0 ? W.Y : W.Tm) + (int64_t)h * R * kD;
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rt * 64 + wave * 16 + 4 * g + e;
      if (r < R) out[(int64_t)r * kD + b * 16 + c16] = acc[b][e];
    }
}

// ------------------------------------------------------------------------------------------------
// One Landweber step for 64 kept keys: with Z_i = Tm_i / u_i - Y_i (the residual of P Vc),
// U_j = sum_i (E_ij / u_i) Z_i, then Vc_j -= eta w_j U_j (P^T = diag(w) E^T diag(1/u)).
// float32 MFMA on LDS-staged E^T and Z. Work item = (seq, head, 64-key tile).
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void am_cols_mm(const float* __restrict__ w_all, float* __restrict__ vc_all,
                                                  float* __restrict__ ws, int H, int R, int m_max, SeqTable T) {
  __shared__ float Ats[64][17];
  __shared__ float Zs[16][kD];
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  const int kt_n = (m + 63) / 64;
  const int local = t - T.start[i];
  const int h = local / kt_n, kt = local - h * kt_n;
  const int64_t unit = (int64_t)s * H + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
  AmWs W = am_ws(ws, T, i, H, R);
  const float* E = W.E + (int64_t)h * R * m;
  const float* Y = W.Y + (int64_t)h * R * kD;
  const float* Tm = W.Tm + (int64_t)h * R * kD;
  const float* u = W.u + (int64_t)h * R;

  f32x4 acc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 1
  for (int r0 = 0; r0 < R; r0 += 16) {
    for (int x = tid; x < 16 * 64; x += 256) {  // E[16 rows][64 keys] / u_row -> transposed
      const int rr = x >> 6, jj = x & 63;
      const int r = r0 + rr, j = kt * 64 + jj;
      Ats[jj][rr] = (r < R && j < m && u[r] > 0.0f) ? E[(int64_t)r * m + j] / u[r] : 0.0f;
    }
    for (int x = tid; x < 16 * kD; x += 256) {
      const int rr = x / kD, dd = x % kD;
      const int r = r0 + rr;
      float z = 0.0f;
      if (r < R) {
        const float ur = u[r];
        z = ur > 0.0f ? Tm[(int64_t)r * kD + dd] / ur - Y[(int64_t)r * kD + dd] : 0.0f;
      }
      Zs[rr][dd] = z;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const float a = Ats[wave * 16 + c16][kk * 4 + g];
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[b] = mfma_f32(a, Zs[kk * 4 + g][b * 16 + c16], acc[b]);
    }
    __syncthreads();
  }
  const float eta = W.eta[h];
  const float* w = w_all + unit * m_max;
  float* vc = vc_all + unit * m_max * (int64_t)kD;
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = kt * 64 + wave * 16 + 4 * g + e;
      if (j < m) vc[(int64_t)j * kD + b * 16 + c16] -= eta * w[j] * acc[b][e];
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
                                               float* __restrict__ vc_all, const float* __restrict__ ws, int H, int R,
                                               int64_t n_max, int m_max, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], n = T.n[i], s = T.first + i;
  const int cb = (m + 255) / 256;
  const int local = t - T.start[i];
  const int h = local / cb;
  const int j = (local - h * cb) * 256 + threadIdx.x;
  if (j >= m) return;
  const int64_t unit = (int64_t)s * H + h;
  const int32_t* map = LAYOUT == kPaged ? table + (int64_t)s * max_blocks
                                        : (LAYOUT == kSlots ? table + unit * n_max : nullptr);
  AmWs W = am_ws(const_cast<float*>(ws), T, i, H, R);
  w_all[unit * m_max + j] = __builtin_amdgcn_exp2f((W.ME[h] - W.M[h]) * kLog2e);  // w = 1 in scaled units
  const int key = min(max(kept[unit * m_max + j], 0), n - 1);
  const u32x4* row = key_row<LAYOUT>(v, map, H, h, n_max, unit, T.kofs[i] + key);
  float* dst = vc_all + (unit * m_max + j) * (int64_t)kD;
#pragma unroll 4
  for (int ch = 0; ch < kD / 8; ++ch) {
    const u32x4 raw = row[ch];
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dst[ch * 8 + 2 * e] = bf16_lo(wd[e]);
      dst[ch * 8 + 2 * e + 1] = bf16_hi(wd[e]);
    }
  }
}

__global__ __launch_bounds__(256) void am_finish(float* __restrict__ w_all, const float* __restrict__ ws, int H,
                                                 int R, int m_max, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int m = T.m[i], s = T.first + i;
  const int cb = (m + 255) / 256;
  const int local = t - T.start[i];
  const int h = local / cb;
  const int j = (local - h * cb) * 256 + threadIdx.x;
  if (j >= m) return;
  AmWs W = am_ws(const_cast<float*>(ws), T, i, H, R);
  float* w = w_all + ((int64_t)s * H + h) * m_max + j;
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

int am_exp_items(int R, int cols) { return ((R + 63) / 64) * ((cols + 63) / 64); }
int am_scale_items(int R, int m) { return (int)(((int64_t)R * m + 4095) / 4096); }
int am_row_items(int R) { return (R + 63) / 64; }
int am_dot_row_items(int R) { return (R + 3) / 4; }
int am_col_items(int m) { return (m + 255) / 256; }
int am_key_tiles(int m) { return (m + 63) / 64; }

hipError_t launch_am_exp(int layout, bool all, const void* q, const void* k, const int32_t* table, int max_blocks,
                         const int32_t* kept, int m_max, const float* lse, float* ws, int H, int R, int64_t n_max,
                         float scale, const SeqTable& T, hipStream_t st) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  dim3 grid(T.total), block(kThreads);
  if (all) KVC_AM_LAYOUT(am_exp, KVC_COMMA true, qq, kk, table, max_blocks, kept, m_max, lse, ws, H, R, n_max, scale, T);
  else KVC_AM_LAYOUT(am_exp, KVC_COMMA false, qq, kk, table, max_blocks, kept, m_max, lse, ws, H, R, n_max, scale, T);
  return hipGetLastError();
}

hipError_t launch_am_stats(const float* lse, float* ws, int H, int R, const SeqTable& T, hipStream_t st) {
  am_stats<<<dim3(T.total), dim3(64), 0, st>>>(lse, ws, H, R, T);
  return hipGetLastError();
}

hipError_t launch_am_scale(float* ws, int H, int R, const SeqTable& T, hipStream_t st) {
  am_scale<<<dim3(T.total), dim3(256), 0, st>>>(ws, H, R, T);
  return hipGetLastError();
}

hipError_t launch_am_rows_dot(const float* w, float* ws, int H, int R, int m_max, const SeqTable& T, hipStream_t st) {
  am_rows_dot<<<dim3(T.total), dim3(256), 0, st>>>(w, ws, H, R, m_max, T);
  return hipGetLastError();
}

hipError_t launch_am_cols_dot(int mode, float* w, const float* lse, float* ws, int H, int R, int m_max,
                              const SeqTable& T, hipStream_t st) {
  dim3 grid(T.total), block(256);
  if (mode == 0) am_cols_dot<0><<<grid, block, 0, st>>>(w, lse, ws, H, R, m_max, T);
  else if (mode == 1) am_cols_dot<1><<<grid, block, 0, st>>>(w, lse, ws, H, R, m_max, T);
  else am_cols_dot<2><<<grid, block, 0, st>>>(w, lse, ws, H, R, m_max, T);
  return hipGetLastError();
}

hipError_t launch_am_eta(float* ws, int H, int R, const SeqTable& T, hipStream_t st) {
  am_eta<<<dim3(T.total), dim3(256), 0, st>>>(ws, H, R, T);
  return hipGetLastError();
}

hipError_t launch_am_rows_mm(int layout, int src, const void* v, const int32_t* table, int max_blocks, const float* w,
                             const float* vc, float* ws, int H, int R, int64_t n_max, int m_max, const SeqTable& T,
                             hipStream_t st) {
  const auto* vv = static_cast<const uint16_t*>(v);
  dim3 grid(T.total), block(256);
  if (src == 0)
    KVC_AM_LAYOUT(am_rows_mm, KVC_COMMA 0, vv, table, max_blocks, w, vc, ws, H, R, n_max, m_max, T);
  else
    am_rows_mm<kContig, 1><<<grid, block, 0, st>>>(vv, table, max_blocks, w, vc, ws, H, R, n_max, m_max, T);
  return hipGetLastError();
}

hipError_t launch_am_cols_mm(const float* w, float* vc, float* ws, int H, int R, int m_max, const SeqTable& T,
                             hipStream_t st) {
  am_cols_mm<<<dim3(T.total), dim3(256), 0, st>>>(w, vc, ws, H, R, m_max, T);
  return hipGetLastError();
}

hipError_t launch_am_init(int layout, const void* v, const int32_t* table, int max_blocks, const int32_t* kept,
                          float* w, float* vc, const float* ws, int H, int R, int64_t n_max, int m_max,
                          const SeqTable& T, hipStream_t st) {
  const auto* vv = static_cast<const uint16_t*>(v);
  dim3 grid(T.total), block(256);
  KVC_AM_LAYOUT(am_init, , vv, table, max_blocks, kept, w, vc, ws, H, R, n_max, m_max, T);
  return hipGetLastError();
}

hipError_t launch_am_finish(float* w, const float* ws, int H, int R, int m_max, const SeqTable& T, hipStream_t st) {
  am_finish<<<dim3(T.total), dim3(256), 0, st>>>(w, ws, H, R, m_max, T);
  return hipGetLastError();
}

}  // namespace kvc
