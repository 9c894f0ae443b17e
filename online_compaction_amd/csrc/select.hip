// Top-m selection per unit ("Practical Online KV Cache Compaction for LLM Agents", design-space
// section: keep the m highest-scoring positions), ties to the lower position, output ascending.
//
// One 1024-thread workgroup per unit. Scores are non-negative float32 with the sign bit clear,
// so their 31 low bits order like the values as unsigned integers. Three radix passes over bits
// 30..19, 18..8 and 7..0 (LDS histograms of 4096, 2048 and 256 bins; the first pass takes 12
// bits because the scores of one unit crowd into a few binades, and narrower bins there mean
// fewer lanes of one atomic instruction on the same counter) narrow the candidates to the exact bit
// pattern T of the m-th largest score and the number `need` of positions equal to T that must be
// kept. An ordered sweep then keeps every position above T and the first `need` positions equal
// to T, in index order: the output slot of a kept position is (positions above T before it) +
// min(positions equal to T before it, need).
//
// Two kernels with the same result:
//   select_topm_reg<K>  n <= 1024 K: thread t holds positions t + 1024 k (k < K) in registers,
//                       read once with all K loads in flight; the histogram passes and the sweep
//                       run on registers. The sweep counts (above, equal) per 64-position wave
//                       slice with ballots, scans the 16 K slice counts once, lets one lane
//                       place the kept positions of each slice, and writes the row out of LDS.
//   select_topm         any n: the same passes over global memory, 8 loads in flight per thread.
#include <algorithm>

#include "block_scan.h"

namespace kvc {

namespace {
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBins = 4096;
constexpr int kStageMax = 16384;  // longest output row staged in LDS (dynamic LDS, 64 KiB)
constexpr int kItems = 4;   // consecutive positions per thread in the global ordered sweep
constexpr int kBatch = 8;   // global loads in flight per thread in a histogram pass

// Digit of radix pass P: bits [shift, shift + bits) of the 31-bit pattern.
template <int P>
struct Pass {
  static constexpr int kShift = P == 0 ? 19 : (P == 1 ? 8 : 0);
  static constexpr int kBits = P == 0 ? 12 : (P == 1 ? 11 : 8);
  static constexpr int kBins = 1 << kBits;
  static constexpr uint32_t kMask = (1u << kBits) - 1u;
  static constexpr int kPerThread = kBins > kThreads ? kBins / kThreads : 1;  // bins a thread scans
};

// Bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// One radix pass. `feed(f)` calls f(value) for every position of the unit; values whose higher
// digits differ from `prefix` are not counted. On return `prefix` holds the digit of the
// `want`-th largest candidate and `want` is lowered by the candidates in higher bins. Thread tid
// owns the kPerThread bins just below bin B - kPerThread tid, so the thread-order scan of their
// sums counts the candidates above them. Contains barriers.
template <int P, typename Feed>
__device__ __forceinline__ void radix_pass(uint32_t* hist, uint32_t* wsum, uint32_t* sel, uint32_t& prefix,
                                           uint32_t& pmask, uint32_t& want, Feed&& feed) {
  using D = Pass<P>;
  const int tid = threadIdx.x;
  for (int b = tid; b < D::kBins; b += kThreads) hist[b] = 0u;
  __syncthreads();
  const uint32_t pf = prefix, pm = pmask;
  feed([&](uint32_t u) {
    if ((u & pm) == pf) atomicAdd(&hist[(u >> D::kShift) & D::kMask], 1u);
  });
  __syncthreads();
  const int top = D::kBins - D::kPerThread * tid;  // bins [top - kPerThread, top) belong to this thread
  uint32_t hb[D::kPerThread], hsum = 0;
#pragma unroll
  for (int q = 0; q < D::kPerThread; ++q) {
    const int b = top - 1 - q;
    hb[q] = b >= 0 ? hist[b] : 0u;
    hsum += hb[q];
  }
  uint32_t tot;
  uint32_t run = block_excl_scan<kWaves>(hsum, tot, wsum);  // candidates in bins >= top
  if (tid == 0) {
    sel[0] = 0u;
    sel[1] = 0u;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < D::kPerThread; ++q) {
    if (run < want && run + hb[q] >= want) {
      sel[0] = (uint32_t)(top - 1 - q);
      sel[1] = run;
    }
    run += hb[q];
  }
  __syncthreads();
  prefix |= sel[0] << D::kShift;
  pmask |= D::kMask << D::kShift;
  want -= sel[1];
  __syncthreads();
}

}  // namespace

// Work item = (sequence, KV head); n <= 1024 K for every sequence of the launch.
// Two workgroups per CU where the registers allow (K <= 36: 8 waves per SIMD); the output
// staging buffer is dynamic LDS of stage_cap ints (0: kept positions are stored directly).
template <int K>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(K <= 36 ? 8 : 4, 8))) void
select_topm_reg(const float* __restrict__ scores, int32_t* __restrict__ kept, int H, int64_t n_max, int m_max,
                int stage_cap, SeqTable T) {
  __shared__ uint32_t hist[kMaxBins];
  __shared__ uint32_t wsum[kWaves];
  __shared__ uint64_t wsum64[kWaves];
  __shared__ uint32_t sel[2];
  __shared__ uint64_t cnt[K * kWaves];  // per (k, wave) slice: above-T count | equal-T count << 32
  extern __shared__ int32_t outbuf[];
  static_assert(K * kWaves <= kThreads, "one slice count per thread in the sweep's scan");
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int n = T.n[i], m = T.m[i];
  const int s = T.first + i;
  const int h = t - T.start[i];
  const int64_t unit = (int64_t)s * H + h;
  const uint32_t* su = reinterpret_cast<const uint32_t*>(scores + unit * n_max);
  int32_t* ku = kept + unit * m_max;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (m == 0) return;
  if (m == n) {
    for (int j = tid; j < n; j += kThreads) ku[j] = j;
    return;
  }

  // Held as bits + 1 (order-preserving; a finite non-negative float's pattern is below
  // 0x7f800001, so bit 31 stays clear), with 0 for positions past n. Those all fall in the
  // lowest bin of every pass they reach, below every real position, and m < n real positions
  // are always found above them; they are never above or equal to the threshold, so no
  // per-position bound check survives the loads. Buffer loads (one scalar resource for the
  // row, a 32-bit offset per lane) keep the K addresses out of 64-bit register pairs; the
  // offsets are clamped into the row, so every load is in bounds and unconditional, and all K
  // are in flight at once.
  const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(su), (short)0,
                                                                       n * 4, 0x00020000);
  uint32_t u[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = tid + k * kThreads;
    const uint32_t x = __builtin_amdgcn_raw_buffer_load_b32(row, min(j, n - 1) * 4, 0, 0);
    u[k] = j < n ? x + 1u : 0u;
  }

  uint32_t prefix = 0, pmask = 0, want = (uint32_t)m;
  auto feed = [&](auto&& f) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      f(u[k]);
      __builtin_amdgcn_sched_barrier(0);  // one position at a time: no precomputed addresses
    }
  };
  radix_pass<0>(hist, wsum, sel, prefix, pmask, want, feed);
  radix_pass<1>(hist, wsum, sel, prefix, pmask, want, feed);
  radix_pass<2>(hist, wsum, sel, prefix, pmask, want, feed);
  const uint32_t thr = prefix;  // bit pattern + 1 of the m-th largest score (>= 1)
  const uint32_t need = want;   // positions equal to thr that are kept (lowest first)

  // Slice (k, w) = positions 1024 k + 64 w + lane, in position order (k, w). Lane k of wave w
  // keeps that slice's above-T / equal-T lane masks (K <= 48 < 64 lanes).
  uint32_t g_lo = 0, g_hi = 0, e_lo = 0, e_hi = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const uint64_t bg = __ballot(u[k] > thr), be = __ballot(u[k] == thr);
    const bool mine = lane == k;
    g_lo = mine ? static_cast<uint32_t>(bg) : g_lo;
    g_hi = mine ? static_cast<uint32_t>(bg >> 32) : g_hi;
    e_lo = mine ? static_cast<uint32_t>(be) : e_lo;
    e_hi = mine ? static_cast<uint32_t>(be >> 32) : e_hi;
  }
  if (lane < K)
    cnt[lane * kWaves + wave] = (uint64_t)(__popc(g_lo) + __popc(g_hi)) |
                                ((uint64_t)(__popc(e_lo) + __popc(e_hi)) << 32);
  __syncthreads();
  uint64_t tot;
  const uint64_t c = tid < K * kWaves ? cnt[tid] : 0ull;
  const uint64_t ex = block_excl_scan<kWaves>(c, tot, wsum64);  // kept slots before each slice
  if (tid < K * kWaves) cnt[tid] = ex;
  __syncthreads();
  // Lane k of wave w places the kept positions of slice (k, w), walking its mask bits in
  // position order with running counts (a lane's work is the number of positions of its slice
  // at or above the threshold). Kept positions go to an LDS copy of the output row when it fits
  // (one coalesced write-out afterwards instead of sparse stores).
  const bool staged = m <= stage_cap;
  if (lane < K) {
    const uint64_t base = cnt[lane * kWaves + wave];
    const uint32_t bg0 = static_cast<uint32_t>(base), be0 = static_cast<uint32_t>(base >> 32);
    const uint64_t G = ((uint64_t)g_hi << 32) | g_lo, E = ((uint64_t)e_hi << 32) | e_lo;
    const int j0 = lane * kThreads + wave * 64;  // position of bit 0 of the slice
    uint64_t rest = G | E;
    uint32_t gc = 0, ec = 0;
    while (rest) {
      const int p = __builtin_ctzll(rest);
      rest &= rest - 1;
      uint32_t pos = 0xffffffffu;
      if ((G >> p) & 1u) {
        pos = bg0 + gc + min(be0 + ec, need);
        ++gc;
      } else {
        const uint32_t er = be0 + ec;
        ++ec;
        if (er < need) pos = bg0 + gc + er;
      }
      if (pos < (uint32_t)m) {  // never past the row, whatever the scores hold
        if (staged) outbuf[pos] = j0 + p;
        else ku[pos] = j0 + p;
      }
    }
  }
  if (staged) {
    __syncthreads();
    for (int r = tid; r < m; r += kThreads) ku[r] = outbuf[r];
  }
}

// Work item = (sequence, KV head); any n.
__global__ __launch_bounds__(kThreads) void select_topm(const float* __restrict__ scores, int32_t* __restrict__ kept,
                                                        int H, int64_t n_max, int m_max, SeqTable T) {
  __shared__ uint32_t hist[kMaxBins];
  __shared__ uint32_t wsum[kWaves];
  __shared__ uint32_t sel[2];
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int n = T.n[i], m = T.m[i];
  const int s = T.first + i;
  const int h = t - T.start[i];
  const int64_t unit = (int64_t)s * H + h;
  const uint32_t* su = reinterpret_cast<const uint32_t*>(scores + unit * n_max);
  int32_t* ku = kept + unit * m_max;
  const int tid = threadIdx.x;

  if (m == 0) return;
  if (m == n) {
    for (int j = tid; j < n; j += kThreads) ku[j] = j;
    return;
  }

  uint32_t prefix = 0, pmask = 0, want = (uint32_t)m;
  auto feed = [&](auto&& f) {
#pragma unroll 1
    for (int j0 = tid; j0 < n; j0 += kThreads * kBatch) {
      uint32_t u[kBatch];
#pragma unroll
      for (int e = 0; e < kBatch; ++e) u[e] = su[min(j0 + e * kThreads, n - 1)];  // clamped, so the loads issue together
#pragma unroll
      for (int e = 0; e < kBatch; ++e)
        if (j0 + e * kThreads < n) f(u[e]);
    }
  };
  radix_pass<0>(hist, wsum, sel, prefix, pmask, want, feed);
  radix_pass<1>(hist, wsum, sel, prefix, pmask, want, feed);
  radix_pass<2>(hist, wsum, sel, prefix, pmask, want, feed);
  const uint32_t thr = prefix;  // bit pattern of the m-th largest score
  const uint32_t need = want;   // positions equal to thr that are kept (lowest first)

  uint32_t base = 0, eq_seen = 0;
#pragma unroll 1
  for (int c0 = 0; c0 < n; c0 += kThreads * kItems) {
    const int j0 = c0 + tid * kItems;
    uint32_t u[kItems];
    bool gt[kItems], eq[kItems];
    uint32_t eqc = 0;
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      const bool valid = j0 + e < n;
      u[e] = valid ? su[j0 + e] : 0u;
      gt[e] = valid && u[e] > thr;
      eq[e] = valid && u[e] == thr;
      eqc += eq[e];
    }
    uint32_t eq_tot;
    uint32_t rank = eq_seen + block_excl_scan<kWaves>(eqc, eq_tot, wsum);
    bool take[kItems];
    uint32_t tc = 0;
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      take[e] = gt[e] || (eq[e] && rank < need);
      rank += eq[e];
      tc += take[e];
    }
    uint32_t tk_tot;
    uint32_t pos = base + block_excl_scan<kWaves>(tc, tk_tot, wsum);
#pragma unroll
    for (int e = 0; e < kItems; ++e)
      if (take[e]) {
        if (pos < (uint32_t)m) ku[pos] = j0 + e;  // never past the row, whatever the scores hold
        ++pos;
      }
    base += tk_tot;
    eq_seen += eq_tot;
  }
}

// Positions per thread the register kernel is instantiated for; longer sequences take the
// global kernel.
int select_reg_items(int n_max_launch) {
  for (int k : {8, 16, 24, 36, 48})
    if (n_max_launch <= k * kThreads) return k;
  return 0;
}

hipError_t launch_select(const float* scores, int32_t* kept, int H, int64_t n_max, int m_max, const SeqTable& T,
                         hipStream_t st) {
  int nl = 0, ml = 0;
  for (int i = 0; i < T.count; ++i) {
    nl = std::max(nl, (int)T.n[i]);
    ml = std::max(ml, (int)T.m[i]);
  }
  const int cap = ml <= kStageMax ? ml : 0;
  const size_t lds = (size_t)cap * sizeof(int32_t);
  const dim3 grid(T.total), block(kThreads);
  switch (select_reg_items(nl)) {
    case 8: select_topm_reg<8><<<grid, block, lds, st>>>(scores, kept, H, n_max, m_max, cap, T); break;
    case 16: select_topm_reg<16><<<grid, block, lds, st>>>(scores, kept, H, n_max, m_max, cap, T); break;
    case 24: select_topm_reg<24><<<grid, block, lds, st>>>(scores, kept, H, n_max, m_max, cap, T); break;
    case 36: select_topm_reg<36><<<grid, block, lds, st>>>(scores, kept, H, n_max, m_max, cap, T); break;
    case 48: select_topm_reg<48><<<grid, block, lds, st>>>(scores, kept, H, n_max, m_max, cap, T); break;
    default: select_topm<<<grid, block, 0, st>>>(scores, kept, H, n_max, m_max, T); break;
  }
  return hipGetLastError();
}

}  // namespace kvc
