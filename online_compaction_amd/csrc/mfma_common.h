// Shared pieces of the MFMA kernels for gfx950 (score_mfma.hip, lse_mfma.hip, am.hip).
//
// The d = 128 contraction is 4 k-steps of v_mfma_f32_16x16x32_bf16. Within a k-step, lane
// group g = lane / 16 supplies d-chunk 4*kstep + g (8 bf16 = 16 bytes) of its row, the same
// d permutation on both operands. LDS rows are 256 bytes; 16-byte chunk c of row r is stored
// at chunk position c ^ (r & 15) so the 16 rows read by one MFMA operand hit distinct banks.
#pragma once

#include <type_traits>

#include "kvc_internal.h"

namespace kvc {
namespace mfma {

constexpr int kThreads = 256;           // 4 waves per workgroup
constexpr int kStage = 64;              // rows / keys per LDS stage

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Pointer to the 256-byte stored row of key position `pos` of unit (s, h). `map` is the
// sequence's block table (kPaged) or the unit's slot-map row (kSlots); unused when contiguous.
template <int LAYOUT>
__device__ __forceinline__ const u32x4* key_row(const uint16_t* __restrict__ k, const int32_t* __restrict__ map,
                                                int H, int h, int64_t n_max, int64_t unit, int pos) {
  if constexpr (LAYOUT == kPaged) {
    const int64_t blk = map[pos >> 4];
    return reinterpret_cast<const u32x4*>(k + ((blk * 16 + (pos & 15)) * H + h) * kHeadDim);
  } else if constexpr (LAYOUT == kSlots) {
    return reinterpret_cast<const u32x4*>(k + ((int64_t)map[pos] * H + h) * kHeadDim);
  } else {
    return reinterpret_cast<const u32x4*>(k + (unit * n_max + pos) * kHeadDim);
  }
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

typedef __attribute__((address_space(3))) void* lds_ptr;

// LDS-DMA loads (global_load_lds_dwordx4 / _dword): every active lane reads its own global
// address and the wave's data lands contiguously at the LDS byte address in M0 plus 16 * lane
// (or 4 * lane); the destination must be wave-uniform. Issued as inline assembly so that the
// compiler does not guard later LDS reads with waits for every load in flight: a stage
// pipeline waits for exactly the loads it needs (vm_wait_barrier), and any wait the
// compiler places for its own loads can only be stricter than necessary.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)p));
}
// M0 is declared clobbered; no other instruction of these kernels reads M0 (gfx9 LDS accesses do
// not use it), which the device-assembly test checks.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const u32x4* src, const void* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(dst));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const float* src, const void* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(dst));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}
// The same loads addressed by a wave-uniform base in SGPRs plus a 32-bit per-lane byte offset,
// with the LDS destination already wave-uniform: no per-lane 64-bit address arithmetic and no
// read of the destination from a vector register.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_dst)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_s(const void* sbase, uint32_t voff, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_dst)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N of this wave's vector-memory loads are outstanding (the LDS-DMA loads
// count there), then a workgroup barrier. No fence: __syncthreads() would also wait for the
// loads meant to stay in flight.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 5) asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else static_assert(N == 0, "unsupported count");
}

// Minimum and maximum of an int over the 64 lanes of the wave (the result is wave-uniform).
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return __builtin_amdgcn_readfirstlane(v);
}

}  // namespace mfma
}  // namespace kvc
