// Block-wide exclusive prefix sum in thread order, for the one-workgroup-per-unit kernels
// (select.hip, retain.hip). Threads = 64 * WAVES; wsum is LDS scratch of WAVES elements.
#pragma once

#include "kvc_internal.h"

namespace kvc {

// Returns the sum of v over the threads before this one; `total` gets the block sum. Contains
// barriers: every thread of the block must call it.
template <int WAVES, typename T>
__device__ __forceinline__ T block_excl_scan(T v, T& total, T* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    T w = lane < WAVES ? wsum[lane] : T(0);
#pragma unroll
    for (int off = 1; off < WAVES; off <<= 1) {
      const T y = __shfl_up(w, off);
      if (lane >= off) w += y;
    }
    if (lane < WAVES) wsum[lane] = w;
  }
  __syncthreads();
  const T before = wave > 0 ? wsum[wave - 1] : T(0);
  total = wsum[WAVES - 1];
  __syncthreads();
  return before + x - v;
}

}  // namespace kvc
