// Compaction of the kept K/V rows.
//
// Contiguous ("Practical Online KV Cache Compaction for LLM Agents", design-space section: keep
// the original keys and values of the top-m positions): an order-preserving gather of 256- or
// 512-byte rows into [S][H][m_max][d], 16 bytes per lane.
//
// Paged in place (ActKV page, paged-memory paragraph: conflict-free slot plan over the tail
// logical blocks, one parallel copy, emptied blocks returned). For a sequence with n keys and
// budget m, N = ceil(n/B), X = ceil(m/B), window W = [(N-X)B, (N-X)B + m). For one head let
// `a` = kept positions below W and `w` = kept positions inside W (found by binary search in the
// ascending kept list). Pair p < m - w is:
//   source p  = kept[p]        if p < a, else kept[p + w]        (kept positions outside W)
//   hole p    = W.start + p + c, c = #{t < w : kept[a+t] - W.start - t <= p}
// (kept[a+t] - W.start - t counts the holes in front of the t-th kept position inside W and is
// non-decreasing in t, so c is found by binary search too). No pair needs a global scan, and
// sources are kept positions while holes are not, so all pairs can be copied at once. The
// block-table update runs as a separate launch after every copy of the sequence.
#include "kvc_internal.h"

namespace kvc {

namespace {
constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 64;  // contiguous rows (or paged pairs) per workgroup

__device__ __forceinline__ int lower_bound_i32(const int32_t* __restrict__ a, int len, int key) {
  int lo = 0, hi = len;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo;
}
}  // namespace

// Work item = (sequence, KV head, row tile of 64 bf16 or 32 float32 rows). CH = 16-byte chunks
// per row; every lane moves 4 chunks of K and 4 of V, all loads issued before the stores.
template <int CH>
__global__ __launch_bounds__(kThreads) void compact_contig(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                                           const int32_t* __restrict__ kept, u32x4* __restrict__ ko,
                                                           u32x4* __restrict__ vo, int H, int64_t n_max, int m_max,
                                                           SeqTable T) {
  constexpr int kRowsPerIter = kThreads / CH;
  constexpr int kIters = 4;
  constexpr int kRows = kRowsPerIter * kIters;  // 64 bf16 rows or 32 float32 rows
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int m = T.m[i], n = T.n[i], kofs = T.kofs[i];
  const int s = T.first + i;
  const int tiles = (m + kRows - 1) / kRows;
  const int local = t - T.start[i];
  const int h = local / tiles;
  const int r0 = (local - h * tiles) * kRows;
  const int64_t unit = (int64_t)s * H + h;
  const int c = threadIdx.x % CH;
  const int rr = threadIdx.x / CH;
  // Every load is unconditional (indices clamped into the row, addresses into the unit), so
  // the kept indices, then all K and V chunks, are in flight together; rows past m are not
  // stored and a kept index outside [0, n) is not followed (it comes from select; such a row
  // is written as zeros).
  int j[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) j[it] = kept[unit * m_max + min(r0 + it * kRowsPerIter + rr, m - 1)];
  u32x4 kx[kIters], vx[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int jj = (unsigned)j[it] < (unsigned)n ? j[it] : 0;
    kx[it] = k[(unit * n_max + kofs + jj) * CH + c];
    vx[it] = v[(unit * n_max + kofs + jj) * CH + c];
  }
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int r = r0 + it * kRowsPerIter + rr;
    if (r < m) {
      const bool ok = (unsigned)j[it] < (unsigned)n;
      ko[(unit * m_max + r) * CH + c] = ok ? kx[it] : u32x4{0u, 0u, 0u, 0u};
      vo[(unit * m_max + r) * CH + c] = ok ? vx[it] : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Work item = (sequence, KV head, 64-pair tile); ceil(m/64) tiles per head bound the pairs.
template <int CH>
__global__ __launch_bounds__(kThreads) void paged_copy(u32x4* __restrict__ kp, u32x4* __restrict__ vp,
                                                       const int32_t* __restrict__ table, int max_blocks,
                                                       const int32_t* __restrict__ kept, int H, int m_max, int B,
                                                       SeqTable T) {
  __shared__ int64_t src_row[kRowsPerBlock], dst_row[kRowsPerBlock];
  __shared__ int s_a, s_w;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i], m = T.m[i];
  const int s = T.first + i;
  const int tiles = (m + kRowsPerBlock - 1) / kRowsPerBlock;
  const int local = t - T.start[i];
  const int h = local / tiles;
  const int p0 = (local - h * tiles) * kRowsPerBlock;
  const int64_t unit = (int64_t)s * H + h;
  const int32_t* ku = kept + unit * m_max;
  const int32_t* trow = table + (int64_t)s * max_blocks;
  const int N = (n + B - 1) / B, X = (m + B - 1) / B;
  const int start = (N - X) * B;  // window start, relative to the segment
  const int ko = T.kofs[i];       // the segment's first cache position (a multiple of B)

  if (threadIdx.x == 0) {
    const int a = lower_bound_i32(ku, m, start);
    const int e = lower_bound_i32(ku, m, start + m);
    s_a = a;
    s_w = e - a;
  }
  __syncthreads();
  const int a = s_a, w = s_w;
  const int npairs = m - w;
  if (p0 >= npairs) return;
  if (threadIdx.x < kRowsPerBlock) {
    const int p = p0 + threadIdx.x;
    if (p < npairs) {
      const int src = p < a ? ku[p] : ku[p + w];
      int lo = 0, hi = w;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (ku[a + mid] - start - mid <= p) lo = mid + 1; else hi = mid;
      }
      const int dst = start + p + lo;
      const bool ok = (unsigned)src < (unsigned)n && dst < N * B;  // holds for any strictly ascending kept
      const int ps = ko + src, pd = ko + dst;                       // cache positions
      const int32_t bs = ok ? trow[ps / B] : -1, bd = ok ? trow[pd / B] : -1;
      src_row[threadIdx.x] = (bs >= 0 && bd >= 0) ? ((int64_t)bs * B + ps % B) * H + h : -1;
      dst_row[threadIdx.x] = (bs >= 0 && bd >= 0) ? ((int64_t)bd * B + pd % B) * H + h : -1;
    } else {
      src_row[threadIdx.x] = -1;
      dst_row[threadIdx.x] = -1;
    }
  }
  __syncthreads();
  const int np = min(kRowsPerBlock, npairs - p0);
  constexpr int kRowsPerIter = kThreads / CH;
  constexpr int kIters = kRowsPerBlock / kRowsPerIter;
  const int c = threadIdx.x % CH;
  // Sources are kept positions and destinations are holes, so no row of the launch is both
  // read and written: all of the tile's loads go first (unconditional; an unused slot reads
  // pool row 0), then the stores.
  u32x4 kx[kIters], vx[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int r = threadIdx.x / CH + it * kRowsPerIter;
    const int64_t sr = r < np ? src_row[r] : -1;
    const int64_t row = sr < 0 ? 0 : sr;
    kx[it] = kp[row * CH + c];
    vx[it] = vp[row * CH + c];
  }
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int r = threadIdx.x / CH + it * kRowsPerIter;
    if (r < np && src_row[r] >= 0) {
      kp[dst_row[r] * CH + c] = kx[it];
      vp[dst_row[r] * CH + c] = vx[it];
    }
  }
}

// One workgroup per sequence, with b = segment start block, F = N - X freed blocks and NT blocks
// in use: freed = old[b, b+F); table[b, NT-F) = old[b+F, NT); table[NT-F, NT) = -1.
__global__ __launch_bounds__(1024) void table_update(int32_t* __restrict__ table, int max_blocks,
                                                     int32_t* __restrict__ freed, int B, SeqTable T) {
  const int i = blockIdx.x;
  const int s = T.first + i;
  const int n = T.n[i], m = T.m[i];
  const int N = (n + B - 1) / B, X = (m + B - 1) / B, F = N - X;
  const int b = T.kofs[i] / B;
  const int NT = (T.clen[i] + B - 1) / B;
  int32_t* tr = table + (int64_t)s * max_blocks;
  int32_t* fr = freed + (int64_t)s * max_blocks;
  for (int j = threadIdx.x; j < F; j += blockDim.x) fr[j] = tr[b + j];
  __syncthreads();
  // shift [b+F, NT) left by F one block-wide slice at a time: a slice reads
  // [b + c0 + F, b + c0 + F + 1024), which no earlier slice has written (they wrote [b, b + c0))
  const int len = NT - b - F;
  for (int c0 = 0; c0 < len; c0 += blockDim.x) {
    const int j = c0 + threadIdx.x;
    const int32_t val = j < len ? tr[b + j + F] : 0;
    __syncthreads();
    if (j < len) tr[b + j] = val;
    __syncthreads();
  }
  for (int j = NT - F + threadIdx.x; j < NT; j += blockDim.x) tr[j] = -1;
}

// ------------------------------------------------------------------------------------------------
// Per-entry float32 side array (e.g. LRFU state) carried through a compaction: new position p of
// a unit receives the entry of old position old(p): kept[p] for contiguous compaction (B = 0);
// for the paged slot plan, window slot start + p keeps its own entry when kept, else holds the
// source paired with that hole (the i-th hole gets the i-th kept position outside the window).
// Work item = (sequence, KV head, 256 new positions). src [S][H][n_max] (read at the segment's
// first position + old), dst [S][H][m_max].
// ------------------------------------------------------------------------------------------------
constexpr int kSideTile = 256;

__global__ __launch_bounds__(kSideTile) void compact_side(const float* __restrict__ src, float* __restrict__ dst,
                                                          const int32_t* __restrict__ kept, int H, int64_t n_max,
                                                          int m_max, int B, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int n = T.n[i], m = T.m[i];
  const int s = T.first + i;
  const int tiles = (m + kSideTile - 1) / kSideTile;
  const int local = t - T.start[i];
  const int h = local / tiles;
  const int p = (local - h * tiles) * kSideTile + threadIdx.x;
  if (p >= m) return;
  const int64_t unit = (int64_t)s * H + h;
  const int32_t* ku = kept + unit * m_max;
  int old;
  if (B == 0) {
    old = ku[p];
  } else {
    const int start = ((n + B - 1) / B - (m + B - 1) / B) * B;
    const int w = start + p;
    const int lo = lower_bound_i32(ku, m, w);
    if (lo < m && ku[lo] == w) {
      old = w;
    } else {
      const int a = lower_bound_i32(ku, m, start);      // kept before the window
      const int e = lower_bound_i32(ku, m, start + m);  // first kept past the window
      const int hole = (w - start) - (lo - a);          // rank of w among the holes
      const int q = hole < a ? hole : e + (hole - a);
      old = (unsigned)q < (unsigned)m ? ku[q] : -1;
    }
  }
  if ((unsigned)old >= (unsigned)n) return;  // only for a kept list that breaks the contract
  dst[unit * m_max + p] = src[unit * n_max + T.kofs[i] + old];
}

int side_tiles(int m) { return (m + kSideTile - 1) / kSideTile; }

hipError_t launch_compact_side(const float* src, float* dst, const int32_t* kept, int H, int64_t n_max, int m_max,
                               int B, const SeqTable& T, hipStream_t st) {
  compact_side<<<dim3(T.total), dim3(kSideTile), 0, st>>>(src, dst, kept, H, n_max, m_max, B, T);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Layout-preserving eviction ("IntentKV" page, layout-preserving eviction): the slot-map entry of
// every scored position that is not kept is redirected to the dead slot; nothing moves.
// Work item = (sequence, KV head, 256 positions). slot_map [S][H][n_max], positions taken from
// the segment start.
// ------------------------------------------------------------------------------------------------
constexpr int kRedirectTile = 256;

__global__ __launch_bounds__(kRedirectTile) void evict_redirect(int32_t* __restrict__ slot_map,
                                                                const int32_t* __restrict__ kept, int H,
                                                                int64_t n_max, int m_max, int dead, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int n = T.n[i], m = T.m[i];
  const int s = T.first + i;
  const int tiles = (n + kRedirectTile - 1) / kRedirectTile;
  const int local = t - T.start[i];
  const int h = local / tiles;
  const int p = (local - h * tiles) * kRedirectTile + threadIdx.x;
  if (p >= n) return;
  const int64_t unit = (int64_t)s * H + h;
  const int32_t* ku = kept + unit * m_max;
  const int lo = lower_bound_i32(ku, m, p);
  if (lo < m && ku[lo] == p) return;
  slot_map[unit * n_max + T.kofs[i] + p] = dead;
}

int redirect_tiles(int n) { return (n + kRedirectTile - 1) / kRedirectTile; }

hipError_t launch_evict_redirect(int32_t* slot_map, const int32_t* kept, int H, int64_t n_max, int m_max, int dead,
                                 const SeqTable& T, hipStream_t st) {
  evict_redirect<<<dim3(T.total), dim3(kRedirectTile), 0, st>>>(slot_map, kept, H, n_max, m_max, dead, T);
  return hipGetLastError();
}

int contig_tiles(int m, bool f32) {
  const int rows = f32 ? 32 : 64;
  return (m + rows - 1) / rows;
}
int paged_tiles(int m) { return (m + kRowsPerBlock - 1) / kRowsPerBlock; }

hipError_t launch_compact_contig(bool f32, const void* k, const void* v, const int32_t* kept, void* ko, void* vo, int H,
                                 int64_t n_max, int m_max, const SeqTable& T, hipStream_t st) {
  dim3 grid(T.total), block(kThreads);
  if (f32)
    compact_contig<32><<<grid, block, 0, st>>>(static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), kept,
                                              static_cast<u32x4*>(ko), static_cast<u32x4*>(vo), H, n_max, m_max, T);
  else
    compact_contig<16><<<grid, block, 0, st>>>(static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), kept,
                                              static_cast<u32x4*>(ko), static_cast<u32x4*>(vo), H, n_max, m_max, T);
  return hipGetLastError();
}

hipError_t launch_paged_copy(bool f32, void* kp, void* vp, const int32_t* table, int max_blocks, const int32_t* kept,
                             int H, int m_max, int B, const SeqTable& T, hipStream_t st) {
  dim3 grid(T.total), block(kThreads);
  if (f32)
    paged_copy<32><<<grid, block, 0, st>>>(static_cast<u32x4*>(kp), static_cast<u32x4*>(vp), table, max_blocks, kept,
                                          H, m_max, B, T);
  else
    paged_copy<16><<<grid, block, 0, st>>>(static_cast<u32x4*>(kp), static_cast<u32x4*>(vp), table, max_blocks, kept,
                                          H, m_max, B, T);
  return hipGetLastError();
}

hipError_t launch_table_update(int32_t* table, int max_blocks, int32_t* freed, int B, const SeqTable& T,
                               hipStream_t st) {
  table_update<<<dim3(T.count), dim3(1024), 0, st>>>(table, max_blocks, freed, B, T);
  return hipGetLastError();
}

}  // namespace kvc
