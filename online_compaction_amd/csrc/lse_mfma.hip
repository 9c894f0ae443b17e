// Per-proxy-row log-sum-exp on MFMA (bf16 operands, float32 accumulate) for gfx950.
//
// LSE_r = ln sum_j exp(l_rj) over the same keys the score pass weighs (ActKV page, paged-memory
// paragraph: the weights are recovered from the LSE; an engine gets it from its attention
// kernel, here it is also computed). Mirror image of score_mfma: lse_partials_mfma reduces over
// KEYS for every proxy row; the WG keeps 512 proxy rows in registers (MFMA B operand) and
// streams 64-key stages of K through LDS (A operand) by LDS-DMA, two stages in flight; online
// sum in the log2 domain against a lazily moved reference exponent; one (reference, sum)
// partial per row and key chunk goes to the workspace, and lse_combine merges the chunks.
#include <type_traits>

#include "mfma_common.h"

namespace kvc {

using namespace mfma;

namespace {

constexpr int kSub = 8;                 // 16-wide subtiles per wave held in registers
constexpr int kPerWave = 16 * kSub;     // 128 rows per wave
constexpr int kPerBlock = 4 * kPerWave; // 512 per workgroup
constexpr int kLseBufs = 3;             // LDS stage buffers (two loads in flight)

}  // namespace

// 16-key tiles per unrolled step of the cheap form: all four (fewer branches and loop instructions
// per stage) where the registers allow it, outside the slot map and, with a bias, only for paged
// keys without the causal mask
template <int LAYOUT, bool BIAS, bool CAUSAL>
constexpr int lse_lazy_unroll() {
  return (LAYOUT != kSlots && (!BIAS || (LAYOUT == kPaged && !CAUSAL))) ? kStage / 16 : 1;
}

// whether full stages are loaded from scalar bases (without the causal mask, outside the slot map)
template <int LAYOUT, bool BIAS, bool CAUSAL>
constexpr bool lse_scalar_dma() {
  return !CAUSAL && LAYOUT != kSlots;
}
// whether the stages that need no per-key term run in a loop of their own (as above, and without
// a bias, which every stage adds)
template <int LAYOUT, bool BIAS, bool CAUSAL>
constexpr bool lse_plain_loop() {
  return !BIAS && lse_scalar_dma<LAYOUT, BIAS, CAUSAL>();
}

// ------------------------------------------------------------------------------------------------
// Per proxy row, partial (reference, sum) of 2^(log2e * l_rj) over one key chunk, with the
// reference exponent moved only when a tile's sum would leave the float range (see below).
// Work item = (sequence, KV head, key chunk kc, 512-row block rb), rb fastest so the blocks
// sharing a key chunk run together on one XCD.
// partials: float2 [T.off[i] + (h * nkc + kc) * R + row]
// ------------------------------------------------------------------------------------------------
// CAUSAL: proxy row r sees only the keys at positions j <= rpos[unit][r]; per stage, a wave whose
// rows see none of the stage's keys skips it, one whose rows see all of them runs the plain
// stage, and otherwise the logits are masked element by element.
template <int LAYOUT, bool BIAS, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void lse_partials_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const int32_t* __restrict__ table,
    int max_blocks, const float* __restrict__ bias, const int32_t* __restrict__ rpos, float2* __restrict__ partials,
    int H, int R, int64_t n_max, float scale, int kchunk, int dead, RowOrder ord, SeqTable T) {
  __shared__ __attribute__((aligned(16))) uint8_t ks_[kLseBufs][kStage * 256];
  __shared__ __attribute__((aligned(16))) float kts[BIAS ? kLseBufs : 1][kStage];
  // causal: the positions of the workgroup's rows (read only by the stages that mask, so they
  // cost no registers across the sweep)
  __shared__ int32_t pls[CAUSAL ? kPerBlock : 1];
  // the chunk's block-table entries (paged) or slots (slot map)
  __shared__ __attribute__((aligned(16)))
  int32_t idx[LAYOUT == kPaged ? kLseMaxChunk / 16 + 1 : (LAYOUT == kSlots ? kLseMaxChunk : 1)];

  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int ko = T.kofs[i];
  const int nkc = (n + kchunk - 1) / kchunk;
  const int nrb = (R + kPerBlock - 1) / kPerBlock;
  int local = t - T.start[i];
  const int h = local / (nkc * nrb);
  local -= h * nkc * nrb;
  const int kc = local / nrb;
  const int rb = local - kc * nrb;
  const int64_t unit = (int64_t)s * H + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;

  const int kbeg = kc * kchunk;
  const int kend = min(n, kbeg + kchunk);
  int nst = (kend - kbeg + kStage - 1) / kStage;
  const float c2 = kLog2e * scale;

  // paged: the chunk's block-table entries (at most kchunk / 16 + 1 <= kLseMaxChunk / 16 + 1,
  // the host never picks a longer chunk); slot map: the chunk's slots (at most kLseMaxChunk).
  // Read once, so the streamed loads (and the dead-slot mask) depend on LDS only.
  const int blk0 = (ko + kbeg) >> 4;
  if constexpr (LAYOUT == kPaged) {
    const int32_t* trow = table + (int64_t)s * max_blocks;
    const int nb = ((ko + kend - 1) >> 4) - blk0 + 1;
    for (int b = tid; b < nb; b += kThreads) idx[b] = trow[blk0 + b];
  } else if constexpr (LAYOUT == kSlots) {
    const int32_t* srow = table + unit * n_max + ko;  // the unit's slot-map row, segment start
    for (int j = tid; j < kend - kbeg; j += kThreads) idx[j] = srow[kbeg + j];
  }
  if constexpr (LAYOUT != kContig) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing of this loop stays pending below
    __syncthreads();
  }
  auto key_ptr = [&](int key) -> const u32x4* {
    const int pos = ko + key;
    if constexpr (LAYOUT == kPaged) {
      const int64_t blk = idx[(pos >> 4) - blk0];
      return reinterpret_cast<const u32x4*>(k + ((blk * 16 + (pos & 15)) * H + h) * kHeadDim);
    } else if constexpr (LAYOUT == kSlots) {
      return reinterpret_cast<const u32x4*>(k + ((int64_t)idx[key - kbeg] * H + h) * kHeadDim);
    } else {
      return reinterpret_cast<const u32x4*>(k + (unit * n_max + pos) * kHeadDim);
    }
  };

  // proxy rows of this wave, held for the whole key sweep
  const uint16_t* qu = q + unit * (int64_t)R * kHeadDim;
  const int row0 = rb * kPerBlock + wave * kPerWave;
  bf16x8 qb[kSub][4];
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    const int r = row0 + sub * 16 + c16;
    if (r < R) {
      const int rr = CAUSAL ? row_of(ord, r) : r;  // stored row (causal rows are taken query-major)
      const u32x4* p = reinterpret_cast<const u32x4*>(qu + (int64_t)rr * kHeadDim);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qb[sub][kk] = as_bf16x8(p[4 * kk + g]);
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qb[sub][kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }
  // causal: the wave's row positions go to LDS, with their range over the wave in registers
  // (rows past R repeat the last row)
  int wpmin = 0, wpmax = 0;
  if constexpr (CAUSAL) {
    int lo = INT32_MAX, hi = INT32_MIN;
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
      const int p = rpos[unit * (int64_t)R + row_of(ord, min(row0 + sub * 16 + c16, R - 1))];
      if (g == 0) pls[wave * kPerWave + sub * 16 + c16] = p;
      lo = min(lo, p);
      hi = max(hi, p);
    }
    wpmin = wave_min(lo);
    wpmax = wave_max(hi);
    // the workgroup stops after the last stage that any of its rows sees (no loads past it)
    __shared__ int wgmax[4];
    if (lane == 0) wgmax[wave] = wpmax;
    __syncthreads();
    const int last = max(max(wgmax[0], wgmax[1]), max(wgmax[2], wgmax[3]));
    nst = last < kbeg ? 0 : min(nst, (last - kbeg) / kStage + 1);
  }

  // A stage (64 keys) goes global -> LDS without passing through registers: each wave issues 4
  // 16-byte-per-lane LDS-DMA loads (4 key rows each, the lane's chunk chosen so the rows land
  // XOR-swizzled) plus, with a bias, one 4-byte load of its 16 keys' bias. Keys past the chunk
  // load the chunk's last row (finite bytes, masked in the epilogue).
  // paged, a full stage: lane row j's key is 64 st further on, so its block-table slot moves by 4
  // per stage and its place inside the block (and so its byte offset koff[j] past the block's
  // start, below) stays
  int slot0[4];
  if constexpr (LAYOUT == kPaged) {
#pragma unroll
    for (int j = 0; j < 4; ++j) slot0[j] = ((ko + kbeg + (wave * 4 + j) * 4 + (lane >> 4)) >> 4) - blk0;
  }
  // A full stage of a contiguous cache, or of a paged one whose segment starts 4-aligned (each
  // load's four rows then lie in one block), is addressed from scalar bases (the stage's first
  // key row, or the block's start) plus per-lane byte offsets that are the same for every stage,
  // and its LDS destinations are scalar: its loads cost no vector instructions beyond reading the
  // four block numbers.
  constexpr bool kSdma = lse_scalar_dma<LAYOUT, BIAS, CAUSAL>();
  const bool sdma = kSdma && (LAYOUT != kPaged || (ko & 3) == 0);
  const bool blk16 = (ko & 15) == 0;  // paged: a full stage's 64 rows are four whole blocks
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t ks_lds = lds_addr(&ks_[0][0]) + wave_s * 4 * 1024;
  const uint32_t kts_lds = lds_addr(&kts[0][0]) + wave_s * 16 * 4;
  uint32_t koff[4];
  int sl0[4];  // paged: the block-table slot of load j's rows at stage 0 (the same for all its lanes)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (wave * 4 + j) * 4 + (lane >> 4), chunk = (lane & 15) ^ (row & 15);
    if constexpr (LAYOUT == kPaged) {
      koff[j] = (((ko + kbeg + row) & 15) * H + h) * 256 + chunk * 16;
      sl0[j] = ((ko + kbeg + (wave_s * 4 + j) * 4) >> 4) - blk0;
    } else {
      koff[j] = row * 256 + chunk * 16;
      sl0[j] = 0;
    }
  }
  auto issue = [&](int st) {
    const int k0 = kbeg + st * kStage;
    const int b = st % kLseBufs;
    if (kSdma && sdma && k0 + kStage <= kend) {
      if constexpr (LAYOUT == kPaged) {
        if (blk16) {  // the wave's 16 rows are one block
          const int64_t blk = __builtin_amdgcn_readfirstlane(idx[sl0[0] + 4 * st]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            dma16_s(k + blk * (16 * H * kHeadDim), koff[j], ks_lds + b * (kStage * 256) + j * 1024);
        } else {
          int e[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) e[j] = idx[sl0[j] + 4 * st];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int64_t blk = __builtin_amdgcn_readfirstlane(e[j]);
            dma16_s(k + blk * (16 * H * kHeadDim), koff[j], ks_lds + b * (kStage * 256) + j * 1024);
          }
        }
      } else {
        const uint16_t* base = k + (unit * n_max + ko + k0) * kHeadDim;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16_s(base, koff[j], ks_lds + b * (kStage * 256) + j * 1024);
      }
      if constexpr (BIAS) {
        if (lane < 16) dma4_s(bias + (int64_t)s * n_max + k0, (wave * 16 + lane) * 4, kts_lds + b * (kStage * 4));
      }
      return;
    }
    // the four sources first (their table entries are LDS reads that then complete together),
    // then the four loads
    const u32x4* src[4];
    if (LAYOUT == kPaged && k0 + kStage <= kend) {
      const u32x4* pool = reinterpret_cast<const u32x4*>(k);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        src[j] = pool + (int64_t)idx[slot0[j] + 4 * st] * (16 * H * (kHeadDim / 8)) + (koff[j] >> 4);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = (wave * 4 + j) * 4 + (lane >> 4);
        const int key = min(k0 + row, kend - 1);
        src[j] = key_ptr(key) + ((lane & 15) ^ (row & 15));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(src[j], &ks_[b][(wave * 4 + j) * 1024]);
    if constexpr (BIAS) {
      if (lane < 16) dma4(bias + (int64_t)s * n_max + min(k0 + wave * 16 + lane, kend - 1), &kts[b][wave * 16]);
    }
  };

  // Per row: a reference exponent mref (a logit in log2 units seen earlier in the chunk, or -1e30
  // before the first) and the running sum of 2^(x - mref). A stage first runs the cheap form (one
  // FMA, one exp2 and one add per logit against the current mref) into stage sums; if any lane's
  // stage sum leaves [0, 2^64] (a logit rose more than about 60 above its mref) the whole wave
  // discards them and redoes the stage exactly, moving mref to every new maximum. The wave's
  // first stage starts mref at one of the lane's own logits of that stage (below), or takes the
  // exact form directly. Terms never exceed 2^64 and the largest one seen is about 1 or more, so
  // the dominant terms neither overflow nor underflow.
  float mref[kSub], ssum[kSub];
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    mref[sub] = -1.0e30f;
    ssum[sub] = 0.0f;
  }
  constexpr float kLazyLimit = 18446744073709551616.0f;  // 2^64

  // logits of tile kt for the subtiles s0 .. s0 + NS - 1
  auto tile_acc = [&](int buf, int kt, int s0, auto& acc) {
    constexpr int NS = std::extent<std::remove_reference_t<decltype(acc)>>::value;
    const int row = kt * 16 + c16;
    bf16x8 a[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) a[kk] = *reinterpret_cast<const bf16x8*>(&ks_[buf][swz(row, 4 * kk + g)]);
#pragma unroll
    for (int sub = 0; sub < NS; ++sub) acc[sub] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int sub = 0; sub < NS; ++sub) acc[sub] = mfma16(a[kk], qb[s0 + sub][kk], acc[sub]);
  };
  // per-key term of the lane's 4 keys in tile kt (log2 units): the bias, -inf past the chunk
  // and for keys in the dead slot
  auto key_term = [&](int buf, int k0, int kt) {
    f32x4 t4 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (BIAS) {
      t4 = *reinterpret_cast<const f32x4*>(&kts[buf][kt * 16 + 4 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j) t4[j] *= kLog2e;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + kt * 16 + 4 * g + j;
      if (key >= kend) t4[j] = -INFINITY;
      if constexpr (LAYOUT == kSlots)
        if (key < kend && idx[key - kbeg] == dead) t4[j] = -INFINITY;
    }
    return t4;
  };
  auto row_pos = [&](int sub) -> int { return pls[wave * kPerWave + sub * 16 + c16]; };
  // The wave's first stage has no reference yet. In a stage without per-key terms whose cheap
  // form is unrolled, each lane takes the largest of its own first four logits of the stage per
  // row as its reference and runs the cheap form with the usual check; otherwise the first stage
  // runs the exact form at once.
  bool fresh = true;
  auto stage = [&](int buf, int k0, auto masked, auto causal, auto seeded) {
    constexpr bool MASK = decltype(masked)::value;
    constexpr bool CM = decltype(causal)::value;  // mask element by element (rows near the keys)
    // a masked tile is formed in halves, so that the row positions fit beside the accumulators
    constexpr int NH = CM ? 2 : 1, NS = kSub / NH;
    constexpr bool kSeed = decltype(seeded)::value;  // (the wave's first stage, unmasked, unrolled)
    const bool exact = fresh && !kSeed;
    fresh = false;
    if constexpr (kSeed) {  // the references from the stage's first tile (its MFMAs formed once more below)
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) {
        f32x4 acc[1];
        tile_acc(buf, 0, sub, acc);
        mref[sub] = fmaxf(fmaxf(acc[0][0], acc[0][1]), fmaxf(acc[0][2], acc[0][3])) * c2;
      }
    }
    if (!exact) {
      float sst[kSub];
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) sst[sub] = 0.0f;
#pragma unroll lse_lazy_unroll<LAYOUT, BIAS, CAUSAL>()
      for (int kt = 0; kt < kStage / 16; ++kt) {
        f32x4 kt4 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (MASK) kt4 = key_term(buf, k0, kt);
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          f32x4 acc[NS];
          tile_acc(buf, kt, hh * NS, acc);
#pragma unroll
          for (int s2 = 0; s2 < NS; ++s2) {
            const int sub = hh * NS + s2;
            // (CM) how far past the lane's first key of the tile the row still sees
            const int lim = CM ? row_pos(sub) - (k0 + kt * 16 + 4 * g) : 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float x = MASK ? __builtin_fmaf(acc[s2][j], c2, kt4[j]) - mref[sub]
                             : __builtin_fmaf(acc[s2][j], c2, -mref[sub]);
              if constexpr (CM) x = j > lim ? -INFINITY : x;
              const float e = __builtin_amdgcn_exp2f(x);
              // unrolled, the first term is the stage sum's start (e >= +0, so 0 + e == e)
              if constexpr (lse_lazy_unroll<LAYOUT, BIAS, CAUSAL>() == kStage / 16)
                sst[sub] = (kt == 0 && j == 0) ? e : sst[sub] + e;
              else
                sst[sub] += e;
            }
          }
        }
      }
      // the stage sums are +0 or positive (or inf / NaN after an overflow), so their bit patterns
      // order like their values and every non-finite one lies above the limit's
      uint32_t mx = __float_as_uint(sst[0]);
#pragma unroll
      for (int sub = 1; sub < kSub; ++sub) mx = max(mx, __float_as_uint(sst[sub]));
      if (__builtin_amdgcn_ballot_w64(mx > __float_as_uint(kLazyLimit)) == 0) {
#pragma unroll
        for (int sub = 0; sub < kSub; ++sub) ssum[sub] += sst[sub];
        return;
      }
    }
    // the first stage, or (rare, wave-uniform) an exact redo: the reference moves to every new
    // maximum
#pragma unroll 1
    for (int kt = 0; kt < kStage / 16; ++kt) {
      const f32x4 kt4 = key_term(buf, k0, kt);
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
      f32x4 acc[NS];
      tile_acc(buf, kt, hh * NS, acc);
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        const int sub = hh * NS + s2;
        const int lim = CM ? row_pos(sub) - (k0 + kt * 16 + 4 * g) : 0;
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = __builtin_fmaf(acc[s2][j], c2, kt4[j]);
          if constexpr (CM) x[j] = j > lim ? -INFINITY : x[j];
        }
        const float m4 = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        if (m4 > mref[sub]) {
          ssum[sub] *= __builtin_amdgcn_exp2f(mref[sub] - m4);
          mref[sub] = m4;
        }
        const float mr = mref[sub];
        ssum[sub] += (__builtin_amdgcn_exp2f(x[0] - mr) + __builtin_amdgcn_exp2f(x[1] - mr)) +
                     (__builtin_amdgcn_exp2f(x[2] - mr) + __builtin_amdgcn_exp2f(x[3] - mr));
      }
      }
    }
  };

  // kLseBufs - 1 stages in flight. At stage st a wave waits for its own loads of st (those of the
  // later stages already issued may stay outstanding), the barrier then makes every wave's loads
  // visible and guarantees that nobody still reads the buffer the next issue overwrites.
  constexpr int kLoadsPerStage = BIAS ? 5 : 4;  // (the causal positions are in registers)
  static_assert(kLseBufs == 3, "the wait counts below assume two stages in flight");
  // the stationary rows have landed before any stage load is issued, so inside the loop the
  // compiler has no register load left to wait for (its own waits would be vmcnt(0)); the
  // first barrier below also publishes the causal positions
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (nst > 0) issue(0);  // (causal rows may leave a workgroup nothing to do)
  if (nst > 1) issue(1);
  // the stages that need no per-key term run in a loop of their own (one code path, so the sums
  // stay in place from one stage to the next); the masked last stage, and every stage of the
  // other variants, follow in the general loop
  const int nplain = lse_plain_loop<LAYOUT, BIAS, CAUSAL>() ? (kend - kbeg) / kStage : 0;
  auto plain_step = [&](int st, auto seeded) {
    if (st + 1 < nst) {
      vm_wait_barrier<kLoadsPerStage>();
    } else {
      vm_wait_barrier<0>();
    }
    if (st + 2 < nst) issue(st + 2);
    stage(st % kLseBufs, kbeg + st * kStage, std::false_type{}, std::false_type{}, seeded);
  };
  int st0 = 0;
  if constexpr (lse_lazy_unroll<LAYOUT, BIAS, CAUSAL>() == kStage / 16) {
    if (nplain > 0) {  // the wave's first stage, seeded (every wave starts at the chunk's first key)
      plain_step(0, std::true_type{});
      st0 = 1;
    }
  }
  for (int st = st0; st < nplain; ++st) plain_step(st, std::false_type{});
  for (int st = nplain; st < nst; ++st) {
    if (st + 1 < nst) {
      vm_wait_barrier<kLoadsPerStage>();
    } else {
      vm_wait_barrier<0>();
    }
    if (st + 2 < nst) issue(st + 2);
    const int k0 = kbeg + st * kStage;
    if constexpr (CAUSAL) {
      if (wpmax < k0) continue;  // no row of the wave sees a key of this stage
      if (wpmin < k0 + kStage - 1) {
        stage(st % kLseBufs, k0, std::true_type{}, std::true_type{}, std::false_type{});
        continue;
      }
    }
    // the bias, dead slots and the keys past the chunk enter through the per-key term; other
    // stages skip it
    if (BIAS || LAYOUT == kSlots || k0 + kStage > kend) {
      stage(st % kLseBufs, k0, std::true_type{}, std::false_type{}, std::false_type{});
    } else {
      stage(st % kLseBufs, k0, std::false_type{}, std::false_type{}, std::false_type{});
    }
  }

  const int64_t pbase = T.off[i] + ((int64_t)h * nkc + kc) * R;
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    float m1 = mref[sub], s1 = ssum[sub];
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float m2 = __shfl_xor(m1, off), s2 = __shfl_xor(s1, off);
      const float mm = fmaxf(m1, m2);
      s1 = s1 * __builtin_amdgcn_exp2f(m1 - mm) + s2 * __builtin_amdgcn_exp2f(m2 - mm);
      m1 = mm;
    }
    const int r = row0 + sub * 16 + c16;
    if (g == 0 && r < R) partials[pbase + (CAUSAL ? row_of(ord, r) : r)] = make_float2(m1, s1);
  }
}

// ------------------------------------------------------------------------------------------------
// Combine the per-chunk partials of every proxy row into its natural-log LSE.
// Work item = (sequence, KV head, 64-row block): four lanes per row each merge every fourth
// chunk's (reference, sum) online, then the four merge by two exchanges.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lse_combine(const float2* __restrict__ partials, float* __restrict__ lse_out,
                                                   int H, int R, int kchunk, SeqTable T) {
  const int t = blockIdx.x;
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int nkc = (n + kchunk - 1) / kchunk;
  const int nrb = (R + 63) / 64;
  const int local = t - T.start[i];
  const int h = local / nrb;
  const int r = (local - h * nrb) * 64 + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  // (mm, sum): sum of 2^(x - mm) over the merged chunks with live keys; mm = -inf before any
  float mm = -INFINITY, sum = 0.0f;
  if (r < R) {
    const float2* p = partials + T.off[i] + (int64_t)h * nkc * R + r;
    auto merge = [&](float2 v) {
      if (!(v.y > 0.0f)) return;  // a chunk without live keys adds nothing
      if (v.x > mm) {
        sum = sum * __builtin_amdgcn_exp2f(mm - v.x) + v.y;
        mm = v.x;
      } else {
        sum += v.y * __builtin_amdgcn_exp2f(v.x - mm);
      }
    };
    int c = part;
    for (; c + 12 < nkc; c += 16) {  // four loads in flight per lane
      const float2 v0 = p[(int64_t)c * R], v1 = p[(int64_t)(c + 4) * R];
      const float2 v2 = p[(int64_t)(c + 8) * R], v3 = p[(int64_t)(c + 12) * R];
      merge(v0);
      merge(v1);
      merge(v2);
      merge(v3);
    }
    for (; c < nkc; c += 4) merge(p[(int64_t)c * R]);
  }
#pragma unroll
  for (int off = 1; off <= 2; off <<= 1) {
    const float m2 = __shfl_xor(mm, off), s2 = __shfl_xor(sum, off);
    const float mx = fmaxf(mm, m2);
    if (mx > -INFINITY) sum = (sum > 0.0f ? sum * __builtin_amdgcn_exp2f(mm - mx) : 0.0f) +
                              (s2 > 0.0f ? s2 * __builtin_amdgcn_exp2f(m2 - mx) : 0.0f);
    mm = mx;
  }
  if (part == 0 && r < R)
    lse_out[((int64_t)s * H + h) * R + r] = sum > 0.0f ? (mm + __builtin_log2f(sum)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------
int lse_mfma_row_blocks(int R) { return (R + kPerBlock - 1) / kPerBlock; }

hipError_t launch_lse_partials_mfma(int layout, bool has_bias, const void* q, const void* k, const int32_t* table,
                                    int max_blocks, const float* bias, const int32_t* rpos, float2* partials, int H,
                                    int R, int64_t n_max, float scale, int kchunk, int dead, const RowOrder& ord,
                                    const SeqTable& T, hipStream_t st) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  dim3 grid(T.total), block(kThreads);
#define KVC_LSE_LAUNCH(L, B, C)                                                                                  \
  lse_partials_mfma<L, B, C><<<grid, block, 0, st>>>(qq, kk, table, max_blocks, bias, rpos, partials, H, R, n_max, \
                                                     scale, kchunk, dead, ord, T)
#define KVC_LSE_LAUNCH_C(L, B)            \
  do {                                   \
    if (rpos) KVC_LSE_LAUNCH(L, B, true);  \
    else KVC_LSE_LAUNCH(L, B, false);      \
  } while (0)
  if (layout == kPaged) {
    if (has_bias) KVC_LSE_LAUNCH_C(kPaged, true); else KVC_LSE_LAUNCH_C(kPaged, false);
  } else if (layout == kSlots) {
    if (has_bias) KVC_LSE_LAUNCH_C(kSlots, true); else KVC_LSE_LAUNCH_C(kSlots, false);
  } else {
    if (has_bias) KVC_LSE_LAUNCH_C(kContig, true); else KVC_LSE_LAUNCH_C(kContig, false);
  }
#undef KVC_LSE_LAUNCH_C
#undef KVC_LSE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_lse_combine(const float2* partials, float* lse_out, int H, int R, int kchunk, const SeqTable& T,
                              hipStream_t st) {
  lse_combine<<<dim3(T.total), dim3(256), 0, st>>>(partials, lse_out, H, R, kchunk, T);
  return hipGetLastError();
}

}  // namespace kvc
