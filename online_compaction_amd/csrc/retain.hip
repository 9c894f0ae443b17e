// ActKV retention state ("ActKV" analysis page, paragraph on action-critical entries and LRFU):
// per unit, the entries holding the top 90 % of the action tokens' attention are "hit", and
// every entry's LRFU value decays and takes its hit: state = decay * state + hit.
//
// One 1024-thread workgroup per unit. The attention masses are non-negative float32, so their
// bit patterns order like the values. The critical set is the shortest run of entries in
// descending mass order (ties to the lower position) whose integer masses
// u = min(floor(mass * 2^32), 2^40) reach ceil(top_p * U), U the unit's total: integer sums are
// exact in any order, so the membership decision does not depend on the reduction order. Three
// radix passes (11 + 11 + 10 bits) with LDS histograms of counts and integer mass find the bit
// pattern T of the last entry taken and how many entries equal to T are needed; one ordered
// sweep with block prefix counts of the ties updates the state.
#include "block_scan.h"

namespace kvc {

namespace {
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kItems = 4;  // consecutive positions per thread in the ordered sweep
typedef unsigned long long u64;
constexpr u64 kMassCap = 1ull << 40;

// min(floor(mass * 2^32), 2^40) of a non-negative float32 given by its bits (scaling by a power
// of two is exact; truncation is the floor for non-negative values)
__device__ __forceinline__ u64 qmass(uint32_t bits) {
  const float v = __uint_as_float(bits) * 4294967296.0f;
  if (!(v > 0.0f)) return 0ull;
  if (!(v < 1099511627776.0f)) return kMassCap;
  return (u64)v;
}
}  // namespace

// Register-resident variant for n <= 1024 K: thread t holds the mass bits of positions
// t + 1024 k (k < K), read once with all K loads in flight (clamped into the row, so every load
// is in bounds; positions past n hold 0, which carries no mass and never reaches the
// threshold, whose integer mass is positive). The passes run on registers; the state update
// reads and writes the same positions. When the entries equal to T number at most `need` (the
// count the last pass leaves in T's bin), all of them are hits and no ranking is needed;
// otherwise the ties are ranked in position order from per-slice ballot counts.
template <int K>
__global__ __launch_bounds__(kThreads) void lrfu_update_reg(const float* __restrict__ mass, float* __restrict__ state,
                                                            int32_t* __restrict__ counts, int H, int64_t n_max,
                                                            double top_p, float decay, SeqTable T) {
  __shared__ uint32_t hcnt[kBins];
  __shared__ u64 hmass[kBins];
  __shared__ uint32_t wsum[kWaves];
  __shared__ u64 wsum64[kWaves];
  __shared__ uint32_t sel_bin, sel_cnt, sel_eq;
  __shared__ u64 sel_mass;
  __shared__ uint32_t eqcnt[K * kWaves];
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int h = t - T.start[i];
  const int64_t unit = (int64_t)s * H + h;
  const uint32_t* mu = reinterpret_cast<const uint32_t*>(mass + unit * n_max);
  float* su = state + unit * n_max;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // buffer loads: one scalar resource for the row, a 32-bit offset per lane
  const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(mu), (short)0,
                                                                       n * 4, 0x00020000);
  uint32_t u[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = tid + k * kThreads;
    const uint32_t x = __builtin_amdgcn_raw_buffer_load_b32(row, min(j, n - 1) * 4, 0, 0);
    u[k] = j < n ? x : 0u;
  }
  u64 part = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) part += qmass(u[k]);
#pragma unroll
  for (int k = 0; k < K; ++k) asm volatile("" : "+v"(u[k]));
  u64 total;
  (void)block_excl_scan<kWaves>(part, total, wsum64);
  const u64 target = total == 0 ? 0ull : (u64)ceil(top_p * (double)total);

  uint32_t thr = 0xffffffffu;  // no entry compares above it
  uint32_t need = 0, above = 0, ties = 0;
  if (target > 0) {
    uint32_t prefix = 0, pmask = 0;
    u64 want = target;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t dmask = pass < 2 ? 0x7ffu : 0x3ffu;
      for (int b = tid; b < kBins; b += kThreads) {
        hcnt[b] = 0u;
        hmass[b] = 0ull;
      }
      __syncthreads();
      // opaque to the optimiser, so that the integer masses are formed per pass instead of being
      // hoisted out of the pass loop (K 64-bit values would not fit the register budget)
#pragma unroll
      for (int k = 0; k < K; ++k) asm volatile("" : "+v"(u[k]));
#pragma unroll
      for (int k = 0; k < K; ++k)
        if ((u[k] & pmask) == prefix && u[k] != 0u) {
          const uint32_t b = (u[k] >> shift) & dmask;
          atomicAdd(&hcnt[b], 1u);
          atomicAdd(&hmass[b], qmass(u[k]));
        }
      __syncthreads();
      const int b0 = 2 * (kThreads - 1 - tid);
      const u64 m0 = hmass[b0], m1 = hmass[b0 + 1];
      const uint32_t c0 = hcnt[b0], c1 = hcnt[b0 + 1];
      u64 mtot;
      uint32_t ctot;
      const u64 above_m = block_excl_scan<kWaves>(m0 + m1, mtot, wsum64);
      const uint32_t above_c = block_excl_scan<kWaves>(c0 + c1, ctot, wsum);
      const u64 ge1 = above_m + m1, ge0 = ge1 + m0;
      if (tid == 0) {
        sel_bin = 0u;
        sel_cnt = 0u;
        sel_mass = 0ull;
        sel_eq = 0u;
      }
      __syncthreads();
      if (above_m < want && ge1 >= want) {
        sel_bin = (uint32_t)(b0 + 1);
        sel_mass = above_m;
        sel_cnt = above_c;
        sel_eq = c1;
      } else if (ge1 < want && ge0 >= want) {
        sel_bin = (uint32_t)b0;
        sel_mass = ge1;
        sel_cnt = above_c + c1;
        sel_eq = c0;
      }
      __syncthreads();
      want -= sel_mass;
      above += sel_cnt;
      ties = sel_eq;  // after the last pass: the entries whose bits equal T
      prefix |= sel_bin << shift;
      pmask |= dmask << shift;
      __syncthreads();
    }
    thr = prefix;
    const u64 uq = qmass(thr);
    need = uq > 0 ? (uint32_t)((want + uq - 1) / uq) : 0u;
  }

  const bool ranked = target > 0 && ties > need;  // uniform
#pragma unroll
  for (int k = 0; k < K; ++k) asm volatile("" : "+v"(u[k]));
  if (ranked) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const uint64_t be = __ballot(u[k] == thr);
      if (lane == 0) eqcnt[k * kWaves + wave] = (uint32_t)__popcll(be);
    }
    __syncthreads();
    uint32_t tot;
    const uint32_t c = tid < K * kWaves ? eqcnt[tid] : 0u;
    const uint32_t ex = block_excl_scan<kWaves>(c, tot, wsum);  // ties before each slice
    if (tid < K * kWaves) eqcnt[tid] = ex;
    __syncthreads();
  }
  // the state update, in groups of 12 positions per thread (loads of a group in flight together);
  // its indices come from an opaque copy of the thread index, so that the clamped offsets of the
  // first loads are not kept alive until here
  int tix = tid;
  asm volatile("" : "+v"(tix));
  constexpr int kGroup = 12;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += kGroup) {
    float st[kGroup];
#pragma unroll
    for (int e = 0; e < kGroup; ++e)
      if (k0 + e < K) st[e] = su[min(tix + (k0 + e) * kThreads, n - 1)];
#pragma unroll
    for (int e = 0; e < kGroup; ++e) {
      const int k = k0 + e;
      if (k >= K) break;
      const int j = tix + k * kThreads;
      bool hit = target > 0 && u[k] > thr;
      if (target > 0 && u[k] == thr) {
        if (!ranked) {
          hit = true;
        } else {
          const uint64_t be = __ballot(true);  // lanes of this wave whose entry ties (inside the branch)
          const uint32_t lb = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(be >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(be), 0u));
          hit = eqcnt[k * kWaves + wave] + lb < need;
        }
      }
      if (j < n) su[j] = __builtin_fmaf(decay, st[e], hit ? 1.0f : 0.0f);
    }
  }
  if (tid == 0 && counts) counts[unit] = (int32_t)(above + need);
}

// Work item = (sequence, KV head). mass, state: [S][H][n_max] (segment-relative); counts: [S][H].
__global__ __launch_bounds__(kThreads) void lrfu_update(const float* __restrict__ mass, float* __restrict__ state,
                                                        int32_t* __restrict__ counts, int H, int64_t n_max,
                                                        double top_p, float decay, SeqTable T) {
  __shared__ uint32_t hcnt[kBins];
  __shared__ u64 hmass[kBins];
  __shared__ uint32_t wsum[kWaves];
  __shared__ u64 wsum64[kWaves];
  __shared__ uint32_t sel_bin, sel_cnt;
  __shared__ u64 sel_mass;
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int h = t - T.start[i];
  const int64_t unit = (int64_t)s * H + h;
  const uint32_t* mu = reinterpret_cast<const uint32_t*>(mass + unit * n_max);
  float* su = state + unit * n_max;
  const int tid = threadIdx.x;

  u64 part = 0;
  for (int j = tid; j < n; j += kThreads) part += qmass(mu[j]);
  u64 total;
  (void)block_excl_scan<kWaves>(part, total, wsum64);
  const u64 target = total == 0 ? 0ull : (u64)ceil(top_p * (double)total);

  uint32_t thr = 0xffffffffu;  // no entry compares above it
  uint32_t need = 0, above = 0;
  if (target > 0) {
    uint32_t prefix = 0, pmask = 0;
    u64 want = target;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t dmask = pass < 2 ? 0x7ffu : 0x3ffu;
      for (int b = tid; b < kBins; b += kThreads) {
        hcnt[b] = 0u;
        hmass[b] = 0ull;
      }
      __syncthreads();
      for (int j = tid; j < n; j += kThreads) {
        const uint32_t u = mu[j];
        if ((u & pmask) == prefix) {
          const uint32_t b = (u >> shift) & dmask;
          atomicAdd(&hcnt[b], 1u);
          atomicAdd(&hmass[b], qmass(u));
        }
      }
      __syncthreads();
      // thread tid owns bins 2(1023 - tid) + {0, 1}: thread-order scans give the candidates'
      // mass and count in the bins above them
      const int b0 = 2 * (kThreads - 1 - tid);
      const u64 m0 = hmass[b0], m1 = hmass[b0 + 1];
      const uint32_t c0 = hcnt[b0], c1 = hcnt[b0 + 1];
      u64 mtot;
      uint32_t ctot;
      const u64 above_m = block_excl_scan<kWaves>(m0 + m1, mtot, wsum64);
      const uint32_t above_c = block_excl_scan<kWaves>(c0 + c1, ctot, wsum);
      const u64 ge1 = above_m + m1, ge0 = ge1 + m0;
      if (tid == 0) {
        sel_bin = 0u;
        sel_cnt = 0u;
        sel_mass = 0ull;
      }
      __syncthreads();
      // the bin where the running mass (from the top) first reaches `want`: unique
      if (above_m < want && ge1 >= want) {
        sel_bin = (uint32_t)(b0 + 1);
        sel_mass = above_m;
        sel_cnt = above_c;
      } else if (ge1 < want && ge0 >= want) {
        sel_bin = (uint32_t)b0;
        sel_mass = ge1;
        sel_cnt = above_c + c1;
      }
      __syncthreads();
      want -= sel_mass;
      above += sel_cnt;
      prefix |= sel_bin << shift;
      pmask |= dmask << shift;
      __syncthreads();
    }
    thr = prefix;
    const u64 uq = qmass(thr);  // > 0: the last bin holds the remaining want > 0
    need = uq > 0 ? (uint32_t)((want + uq - 1) / uq) : 0u;
  }

  uint32_t eq_seen = 0;
#pragma unroll 1
  for (int c0 = 0; c0 < n; c0 += kThreads * kItems) {
    const int j0 = c0 + tid * kItems;
    bool gt[kItems], eq[kItems];
    uint32_t eqc = 0;
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      const bool valid = j0 + e < n;
      const uint32_t u = valid ? mu[j0 + e] : 0u;
      gt[e] = valid && target > 0 && u > thr;
      eq[e] = valid && target > 0 && u == thr;
      eqc += eq[e];
    }
    uint32_t eq_tot;
    uint32_t rank = eq_seen + block_excl_scan<kWaves>(eqc, eq_tot, wsum);
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      const bool hit = gt[e] || (eq[e] && rank < need);
      rank += eq[e];
      if (j0 + e < n) su[j0 + e] = __builtin_fmaf(decay, su[j0 + e], hit ? 1.0f : 0.0f);
    }
    eq_seen += eq_tot;
  }
  if (tid == 0 && counts) counts[unit] = (int32_t)(above + need);
}

hipError_t launch_lrfu_update(const float* mass, float* state, int32_t* counts, int H, int64_t n_max, double top_p,
                              float decay, const SeqTable& T, hipStream_t st) {
  int nl = 0;
  for (int i = 0; i < T.count; ++i) nl = nl > T.n[i] ? nl : T.n[i];
  const dim3 grid(T.total), block(kThreads);
  if (nl <= 8 * kThreads) lrfu_update_reg<8><<<grid, block, 0, st>>>(mass, state, counts, H, n_max, top_p, decay, T);
  else if (nl <= 16 * kThreads)
    lrfu_update_reg<16><<<grid, block, 0, st>>>(mass, state, counts, H, n_max, top_p, decay, T);
  else if (nl <= 36 * kThreads)
    lrfu_update_reg<36><<<grid, block, 0, st>>>(mass, state, counts, H, n_max, top_p, decay, T);
  else lrfu_update<<<grid, block, 0, st>>>(mass, state, counts, H, n_max, top_p, decay, T);
  return hipGetLastError();
}

}  // namespace kvc
