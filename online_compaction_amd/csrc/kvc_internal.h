// Internal definitions shared by the libkvc kernels and the host entry points (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvc.h"

namespace kvc {

constexpr int kHeadDim = 128;
constexpr int kChunkSeqs = 128;     // sequences described per launch (kernel-argument table)
// How keys are addressed: contiguous [S][H][n_max][d]; paged pool through a per-sequence block
// table; slot pool [slots][H][d] through a per-(sequence, head) slot map with a dead slot.
enum : int { kContig = 0, kPaged = 1, kSlots = 2 };

// longest key chunk one LSE-pass workgroup may cover (the host picks 4096, 2048, 1024 or 512)
constexpr int kLseMaxChunk = 4096;
// VALU scoring: longest key chunk of one workgroup, and the most proxy rows whose logits are cached
// (R floats per key, written by the LSE pass and read by the score pass instead of the key rows)
constexpr int kValuMaxChunk = 1024;
constexpr int kValuMaxCacheRows = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Squared weights are accumulated as exp2(2*log2(alpha) + kSqOffset) so that alpha down to
// 2^-113 survives float32's normal range; the offset is removed after the square root.
constexpr float kSqOffset = 100.0f;
constexpr float kSqUnscale = 8.8817841970012523e-16f;  // 2^-50
// Attention mass (plain weights) uses the same offset: exp2(log2(alpha) + kSqOffset), unscaled by 2^-100.
constexpr float kMassUnscale = 7.8886090522101181e-31f;  // 2^-100

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Per-launch description of up to kChunkSeqs sequences, passed by value as a kernel argument
// (so a launch never needs a host-to-device copy). `start[i]` is the first work item of
// sequence i; work items of one sequence are contiguous.
struct SeqTable {
  int32_t count;                  // sequences in this launch
  int32_t first;                  // global index of sequence 0 of this launch
  int32_t total;                  // work items in this launch (grid size)
  int32_t pad;
  int32_t start[kChunkSeqs + 1];
  int32_t n[kChunkSeqs];          // keys scored (segment length)
  int32_t m[kChunkSeqs];          // kept positions
  int32_t kofs[kChunkSeqs];       // cache position of the segment's first key
  int32_t clen[kChunkSeqs];       // total cache length (paged compaction)
  int64_t off[kChunkSeqs];        // kernel-specific per-sequence offset (workspace slots)
};
static_assert(sizeof(SeqTable) <= 3800, "SeqTable must fit the kernel-argument segment");

// Workspace region of one sequence for the few-row LSE pass, in float2 units (16-byte
// multiples): the chunk partials [H][nkc][R] (float2 (max, sum)), nkc = ceil(n/kchunk), then,
// when the logits are cached, [H][R][nkc * kchunk] float32 logits (whole chunks, so the pass stores
// every lane's logit without a bounds test).
__host__ __device__ inline int64_t valu_partials_float2(int H, int R, int n, int kchunk) {
  const int64_t p = (int64_t)H * ((n + kchunk - 1) / kchunk) * R;
  return (p + 1) & ~(int64_t)1;
}
__host__ __device__ inline int64_t valu_region_float2(int H, int R, int n, int kchunk, bool cache) {
  const int64_t npad = (int64_t)((n + kchunk - 1) / kchunk) * kchunk;
  const int64_t lg = cache ? (((int64_t)H * R * npad + 3) & ~(int64_t)3) / 2 : 0;
  return valu_partials_float2(H, R, n, kchunk) + lg;
}

// Order in which the MFMA kernels take a unit's proxy rows when the rows are causal. A unit's
// R = G * q rows are stored head-major (row g * q + i is query i of query head g); with causal
// rows the kernels group them query-major instead (work row rho is row (rho mod G) * q + rho / G),
// so that the rows a wave holds together share query positions and more of its key stages are
// wholly visible or wholly hidden. g = 1 keeps the stored order. rho / G is one multiply-high by
// magic = ceil(2^32 / g), exact for rho * g < 2^32 (the host uses it for g <= 256 only).
struct RowOrder {
  int32_t g, q;
  uint32_t magic;
};
__device__ __forceinline__ int row_of(const RowOrder& o, int rho) {
  if (o.g == 1) return rho;
  const int i = (int)__umulhi((uint32_t)rho, o.magic);
  return (rho - i * o.g) * o.q + i;
}

// Map a dispatch-ordered block index to a logical work index so that logically consecutive
// work items run on the same XCD (blocks are dispatched round-robin over the 8 XCDs, each with
// its own L2): neighbours then share the operands they re-read.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int q = nb >> 3, r = nb & 7;
  const int x = b & 7, i = b >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// Wave-uniform search: the sequence whose work range holds item t.
__device__ __forceinline__ int find_seq(const SeqTable& T, int t) {
  int lo = 0, hi = T.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (T.start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace kvc
