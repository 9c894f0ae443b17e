// Top-m selection per unit ("Practical Online KV Cache Compaction for LLM Agents", design-space
// section: keep the m highest-scoring positions), ties to the lower position, output ascending.
//
// One 1024-thread workgroup per unit. Scores are non-negative float32, so their bit patterns
// order like the values as unsigned integers. Three radix passes (11 + 11 + 10 bits, LDS
// histograms) narrow the candidates to the exact bit pattern T of the m-th largest score and
// the number `need` of positions equal to T that must be kept. One ordered sweep then keeps
// every position above T and the first `need` positions equal to T, compacting them in index
// order with block-wide prefix sums.
#include "block_scan.h"

namespace kvc {

namespace {
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kItems = 4;  // consecutive positions per thread in the ordered sweep

}  // namespace

// Work item = (sequence, KV head).
__global__ __launch_bounds__(kThreads) void select_topm(const float* __restrict__ scores, int32_t* __restrict__ kept,
                                                        int H, int64_t n_max, int m_max, SeqTable T) {
  __shared__ uint32_t hist[kBins];
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
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass < 2 ? 0x7ffu : 0x3ffu;
    for (int b = tid; b < kBins; b += kThreads) hist[b] = 0u;
    __syncthreads();
    for (int j = tid; j < n; j += kThreads) {
      const uint32_t u = su[j];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread tid owns bins 2(1023 - tid) and 2(1023 - tid) + 1, so the thread-order inclusive
    // scan of their sums is the count of candidates at or above bin 2(1023 - tid)
    const int b0 = 2 * (kThreads - 1 - tid);
    const uint32_t h0 = hist[b0], h1 = hist[b0 + 1];
    uint32_t tot;
    const uint32_t above = block_excl_scan<kWaves>(h0 + h1, tot, wsum);  // candidates in bins >= b0 + 2
    const uint32_t ge1 = above + h1;                               // ... in bins >= b0 + 1
    const uint32_t ge0 = ge1 + h0;                                 // ... in bins >= b0
    if (tid == 0) {
      sel[0] = 0u;
      sel[1] = 0u;
    }
    __syncthreads();
    if (ge1 >= want && above < want) {
      sel[0] = (uint32_t)(b0 + 1);
      sel[1] = above;
    } else if (ge0 >= want && ge1 < want) {
      sel[0] = (uint32_t)b0;
      sel[1] = ge1;
    }
    __syncthreads();
    const uint32_t d = sel[0];
    want -= sel[1];
    prefix |= d << shift;
    pmask |= dmask << shift;
    __syncthreads();
  }
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

hipError_t launch_select(const float* scores, int32_t* kept, int H, int64_t n_max, int m_max, const SeqTable& T,
                         hipStream_t st) {
  select_topm<<<dim3(T.total), dim3(kThreads), 0, st>>>(scores, kept, H, n_max, m_max, T);
  return hipGetLastError();
}

}  // namespace kvc
