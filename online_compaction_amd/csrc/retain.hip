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
  lrfu_update<<<dim3(T.total), dim3(kThreads), 0, st>>>(mass, state, counts, H, n_max, top_p, decay, T);
  return hipGetLastError();
}

}  // namespace kvc
