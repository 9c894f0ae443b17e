// Token Eviction scoring on MFMA (bf16 operands, float32 accumulate) for gfx950: the score pass.
//
// Score of key j of one unit ("Practical Online KV Cache Compaction for LLM Agents", design-space
// section, TE score equation): s_j = sqrt((1/R) sum_r alpha_rj^2) with
// alpha_rj = exp(l_rj - LSE_r) (ActKV page, paged-memory paragraph: weights recovered from the
// LSE without gathering or materialising the attention matrix).
//
// score_mfma reduces over ROWS for every key: the WG keeps 512 keys in registers (MFMA B
// operand) and streams 64-row stages of Q and of the per-row LSE into LDS by LDS-DMA, two stages
// in flight (A operand);
// each lane accumulates exp2(2 log2(alpha) + 100) for its key, and the 4 lane groups that share
// a key are summed with two cross-lane exchanges. The LSE it needs comes from the caller or from
// the mirror-image pass in lse_mfma.hip.
#include "mfma_common.h"

namespace kvc {

using namespace mfma;

namespace {

#ifndef KVC_SCORE_OCC
#define KVC_SCORE_OCC 2
#endif
constexpr int kBufs = 3;  // LDS stage buffers (two loads in flight)

// 16-row tiles per unrolled step of a stage: all four (their LDS offsets become immediates), but
// one at a time where the registers would not hold them (nine key subtiles per wave, or the
// biased causal slot-map variant)
template <int LAYOUT, bool BIAS, bool CAUSAL, int KSUB>
constexpr int score_rt_unroll() {
  return (KSUB == 9 || (CAUSAL && BIAS && LAYOUT == kSlots)) ? 1 : kStage / 16;
}
// whether full stages of rows are loaded from a scalar base, run in a loop of their own and form
// their rows' exponent offsets once per wave (stored row order, and registers to spare: not with
// nine biased key subtiles per wave)
template <bool BIAS, bool CAUSAL, int KSUB>
constexpr bool score_scalar_dma() {
  return !CAUSAL && !(BIAS && KSUB == 9);
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// Scores. Work item = (sequence, KV head, key tile of 64 * KSUB keys): each of the 4 waves holds
// KSUB 16-key subtiles (8 by default; 4 or 9 when that fills the GPU's resident workgroups better,
// chosen by the host).
// lse: natural-log LSE per proxy row, [S][H*G][q] == [unit][R].
// pw = 2: s_j = sqrt((1/R) sum_r alpha_rj^2) (the TE score); pw = 1: (1/R) sum_r alpha_rj, the
// mean attention weight the proxy rows give key j (the per-entry action-attention tally of ActKV).
// ------------------------------------------------------------------------------------------------
// CAUSAL: proxy row r sees only the keys at positions j <= rpos[unit][r] (segment-relative);
// the stage's row positions arrive with its rows, and per stage and wave the 128 keys are either
// all visible to the stage's 64 rows (the plain epilogue), all hidden (the stage is skipped), or
// masked element by element.
template <int LAYOUT, bool BIAS, bool CAUSAL, int KSUB>
__global__ __launch_bounds__(kThreads, KVC_SCORE_OCC) void score_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const int32_t* __restrict__ table,
    int max_blocks, const float* __restrict__ lse, const float* __restrict__ bias, const int32_t* __restrict__ rpos,
    float* __restrict__ scores, int H, int R, int64_t n_max, float scale, int pw, int dead, RowOrder ord, SeqTable T) {
  constexpr int kScoreSub = KSUB;               // key subtiles per wave
  constexpr int kScoreKeys = 4 * 16 * kScoreSub;  // keys per workgroup
  __shared__ __attribute__((aligned(16))) uint8_t qs[kBufs][kStage * 256];
  __shared__ __attribute__((aligned(16))) float lss[kBufs][kStage];
  __shared__ __attribute__((aligned(16))) int32_t pss[CAUSAL ? kBufs : 1][kStage];
  // a plain stage's exponent offsets, one row per lane, each wave its own copy
  __shared__ __attribute__((aligned(16))) float nbw[4][kStage];

  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int i = find_seq(T, t);
  const int n = T.n[i];
  const int s = T.first + i;
  const int ko = T.kofs[i];
  const int tiles = (n + kScoreKeys - 1) / kScoreKeys;
  const int local = t - T.start[i];
  const int h = local / tiles;
  const int kt = local - h * tiles;
  const int64_t unit = (int64_t)s * H + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // block-table row of the sequence, or slot-map row of the unit ([S][H][n_max])
  const int32_t* map = LAYOUT == kPaged ? table + (int64_t)s * max_blocks
                                        : (LAYOUT == kSlots ? table + unit * n_max : nullptr);

  // pw = 2: squared weights (the score); pw = 1: the weights themselves (attention mass)
  const float pl2 = (float)pw * kLog2e;
  // keys of this wave, held for the whole row sweep
  bf16x8 kb[kScoreSub][4];
  float bb[kScoreSub];
  uint32_t deadmask = 0;  // slot map: subtiles whose key sits in the dead slot (scored 0)
  const int key0 = kt * kScoreKeys + wave * (16 * kScoreSub);
#pragma unroll
  for (int sub = 0; sub < kScoreSub; ++sub) {
    const int key = key0 + sub * 16 + c16;
    bool live = key < n;
    if constexpr (LAYOUT == kSlots)
      if (live && map[ko + key] == dead) {
        live = false;
        deadmask |= 1u << sub;
      }
    if (live) {
      const u32x4* p = key_row<LAYOUT>(k, map, H, h, n_max, unit, ko + key);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[sub][ks] = as_bf16x8(p[4 * ks + g]);
      if constexpr (BIAS) bb[sub] = pl2 * bias[(int64_t)s * n_max + key];
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[sub][ks] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      if constexpr (BIAS) bb[sub] = 0.0f;
    }
  }

  const uint16_t* qu = q + unit * (int64_t)R * kHeadDim;
  const float* lu = lse + unit * (int64_t)R;
  const float a2 = pl2 * scale;
  const int nst = (R + kStage - 1) / kStage;

  // A stage (64 proxy rows) goes global -> LDS without passing through registers: each wave
  // issues 4 16-byte-per-lane LDS-DMA loads (4 rows each, the lane's chunk chosen so the rows
  // land XOR-swizzled) and one 4-byte load of its 16 rows' LSE. Rows past R load row R - 1
  // (finite bytes, masked in the epilogue). A full stage of rows in stored order is addressed
  // from the stage's first row (a scalar base) plus per-lane offsets that are the same for every
  // stage, and its LDS destinations are scalar too, so its loads cost no vector instructions.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t qs_lds = lds_addr(&qs[0][0]) + wave_s * 4 * 1024, ls_lds = lds_addr(&lss[0][0]) + wave_s * 16 * 4;
  uint32_t qoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (wave * 4 + j) * 4 + (lane >> 4);
    qoff[j] = row * 256 + (((lane & 15) ^ (row & 15)) << 4);
  }
  const uint32_t loff = (wave * 16 + lane) * 4;
  auto issue = [&](int st) {
    const int r0 = st * kStage;
    const int b = st % kBufs;
    if (score_scalar_dma<BIAS, CAUSAL, KSUB>() && r0 + kStage <= R) {
      const uint16_t* qb0 = qu + (int64_t)r0 * kHeadDim;
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16_s(qb0, qoff[j], qs_lds + b * (kStage * 256) + j * 1024);
      if (lane < 16) dma4_s(lu + r0, loff, ls_lds + b * (kStage * 4));
      return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = (wave * 4 + j) * 4 + (lane >> 4);
      int r = min(r0 + row, R - 1);
      if constexpr (CAUSAL) r = row_of(ord, r);
      dma16(reinterpret_cast<const u32x4*>(qu + (int64_t)r * kHeadDim) + ((lane & 15) ^ (row & 15)),
            &qs[b][(wave * 4 + j) * 1024]);
    }
    if constexpr (CAUSAL) {
      if (lane < 16) {
        const int r = row_of(ord, min(r0 + wave * 16 + lane, R - 1));
        dma4(lu + r, &lss[b][wave * 16]);
        dma4(reinterpret_cast<const float*>(rpos + unit * (int64_t)R + r), &pss[b][wave * 16]);
      }
    } else {
      if (lane < 16) dma4(lu + min(r0 + wave * 16 + lane, R - 1), &lss[b][wave * 16]);
    }
  };

  float ssum[kScoreSub];
#pragma unroll
  for (int sub = 0; sub < kScoreSub; ++sub) ssum[sub] = 0.0f;

  auto stage = [&](int buf, int r0, auto masked, auto causal) {
    constexpr bool MASK = decltype(masked)::value;
    constexpr bool CM = decltype(causal)::value;  // mask element by element (rows near the keys)
    constexpr bool PLAIN = !MASK && !CM && score_scalar_dma<BIAS, CAUSAL, KSUB>();
    if constexpr (PLAIN) {
      // lane l forms row l's offset once for the wave (LDS accesses of one wave complete in order,
      // so its own reads below see the write)
      nbw[wave][lane] = __builtin_fmaf(lss[buf][lane], -pl2, kSqOffset);
    }
#pragma unroll score_rt_unroll<LAYOUT, BIAS, CAUSAL, KSUB>()
    for (int rt = 0; rt < kStage / 16; ++rt) {
      const int row = rt * 16 + c16;
      bf16x8 a[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) a[ks] = *reinterpret_cast<const bf16x8*>(&qs[buf][swz(row, 4 * ks + g)]);
      f32x4 nb4 = *reinterpret_cast<const f32x4*>(PLAIN ? &nbw[wave][rt * 16 + 4 * g] : &lss[buf][rt * 16 + 4 * g]);
      int32_t p4[4] = {0, 0, 0, 0};
      if constexpr (CM) {
        const int4 pv = *reinterpret_cast<const int4*>(&pss[buf][rt * 16 + 4 * g]);
        p4[0] = pv.x;
        p4[1] = pv.y;
        p4[2] = pv.z;
        p4[3] = pv.w;
      }
      if constexpr (!PLAIN) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          nb4[e] = __builtin_fmaf(nb4[e], -pl2, kSqOffset);
          if constexpr (MASK)
            if (r0 + rt * 16 + 4 * g + e >= R) nb4[e] = -INFINITY;
        }
      }
      f32x4 acc[kScoreSub];
#pragma unroll
      for (int sub = 0; sub < kScoreSub; ++sub) acc[sub] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int sub = 0; sub < kScoreSub; ++sub) acc[sub] = mfma16(a[ks], kb[sub][ks], acc[sub]);
#pragma unroll
      for (int sub = 0; sub < kScoreSub; ++sub) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = __builtin_fmaf(acc[sub][e], a2, nb4[e]);
          if constexpr (BIAS) x += bb[sub];
          if constexpr (CM) x = key0 + sub * 16 + c16 > p4[e] ? -INFINITY : x;
          ssum[sub] += __builtin_amdgcn_exp2f(x);
        }
      }
    }
  };

  // kBufs - 1 stages in flight, as in the LSE pass: at stage st a wave waits for its own loads
  // of st, the barrier publishes every wave's loads and frees the buffer the next issue refills.
  // The stationary keys have landed before the first issue, so the compiler has no register load
  // left to wait for inside the loop.
  static_assert(kBufs == 3, "the wait counts below assume two stages in flight");
  constexpr int kLoadsPerStage = CAUSAL ? 6 : 5;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  issue(0);
  if (nst > 1) issue(1);
  // Without the causal mask the stages whose rows are all live run in a loop of their own (one
  // code path, so the row sums stay in place from one stage to the next); the masked last stage
  // and every causal stage follow in the general loop (all stages, with nine biased key
  // subtiles per wave, whose registers would not hold the second copy).
  const int nfull = score_scalar_dma<BIAS, CAUSAL, KSUB>() ? R / kStage : 0;
  for (int st = 0; st < nfull; ++st) {
    if (st + 1 < nst) {
      vm_wait_barrier<kLoadsPerStage>();
    } else {
      vm_wait_barrier<0>();
    }
    if (st + 2 < nst) issue(st + 2);
    stage(st % kBufs, st * kStage, std::false_type{}, std::false_type{});
  }
  for (int st = nfull; st < nst; ++st) {
    if (st + 1 < nst) {
      vm_wait_barrier<kLoadsPerStage>();
    } else {
      vm_wait_barrier<0>();
    }
    if (st + 2 < nst) issue(st + 2);
    const int r0 = st * kStage;
    const int buf = st % kBufs;
    int vis = 0;  // 0: every key of the wave visible to every row of the stage; 1: mixed; 2: none
    if constexpr (CAUSAL) {
      const int pr = pss[buf][lane];
      const int pmin = wave_min(pr), pmax = wave_max(pr);
      vis = pmax < key0 ? 2 : (pmin >= key0 + 16 * kScoreSub - 1 ? 0 : 1);
    }
    if (vis == 2) continue;
    if (vis == 1) {
      if constexpr (CAUSAL) stage(buf, r0, std::true_type{}, std::true_type{});
    } else if (r0 + kStage > R) {
      stage(buf, r0, std::true_type{}, std::false_type{});
    } else {
      stage(buf, r0, std::false_type{}, std::false_type{});
    }
  }

  const float invR = 1.0f / (float)R;
#pragma unroll
  for (int sub = 0; sub < kScoreSub; ++sub) {
    float v = ssum[sub];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    const int key = key0 + sub * 16 + c16;
    if (g == 0 && key < n)
      scores[unit * n_max + key] = (deadmask >> sub) & 1u ? 0.0f
                                   : pw == 2 ? __builtin_sqrtf(v * invR) * kSqUnscale : v * invR * kMassUnscale;
  }
}

// ------------------------------------------------------------------------------------------------
// launcher
// ------------------------------------------------------------------------------------------------
int score_mfma_tiles(int n, int ksub) { return (n + 64 * ksub - 1) / (64 * ksub); }

bool score_mfma_ksub_ok(int ksub, int layout, bool has_bias, bool causal) {
  if (ksub == 4 || ksub == 8) return true;
  return ksub == 9 && !causal && !(layout == kSlots && has_bias);
}

namespace {

// Everything a score launch passes through to the kernel, bundled for the dispatch below.
struct ScoreArgs {
  const uint16_t* q;
  const uint16_t* k;
  const int32_t* table;
  int max_blocks;
  const float* lse;
  const float* bias;
  const int32_t* rpos;
  float* scores;
  int H, R;
  int64_t n_max;
  float scale;
  int pw, dead;
  RowOrder ord;
};

template <int L, bool B, bool C, int KS>
void launch_ks(dim3 grid, hipStream_t st, const ScoreArgs& a, const SeqTable& T) {
  score_mfma<L, B, C, KS><<<grid, dim3(kThreads), 0, st>>>(a.q, a.k, a.table, a.max_blocks, a.lse, a.bias, a.rpos,
                                                            a.scores, a.H, a.R, a.n_max, a.scale, a.pw, a.dead, a.ord,
                                                            T);
}

template <int L, bool B, bool C>
void launch_c(int ksub, dim3 grid, hipStream_t st, const ScoreArgs& a, const SeqTable& T) {
  if (ksub == 4) {
    launch_ks<L, B, C, 4>(grid, st, a, T);
  } else if (ksub == 9) {
    if constexpr (!C && !(L == kSlots && B)) launch_ks<L, B, C, 9>(grid, st, a, T);
  } else {
    launch_ks<L, B, C, 8>(grid, st, a, T);
  }
}

template <int L>
void launch_l(bool has_bias, int ksub, dim3 grid, hipStream_t st, const ScoreArgs& a, const SeqTable& T) {
  if (has_bias) {
    if (a.rpos) launch_c<L, true, true>(ksub, grid, st, a, T);
    else launch_c<L, true, false>(ksub, grid, st, a, T);
  } else {
    if (a.rpos) launch_c<L, false, true>(ksub, grid, st, a, T);
    else launch_c<L, false, false>(ksub, grid, st, a, T);
  }
}

}  // namespace

hipError_t launch_score_mfma(int layout, bool has_bias, int ksub, const void* q, const void* k, const int32_t* table,
                             int max_blocks, const float* lse, const float* bias, const int32_t* rpos, float* scores,
                             int H, int R, int64_t n_max, float scale, int pw, int dead, const RowOrder& ord,
                             const SeqTable& T, hipStream_t st) {
  // 9 subtiles per wave fit the registers only without the causal mask and outside the biased
  // slot-map variant (score_mfma_ksub_ok); the host asks for them only there
  if (!score_mfma_ksub_ok(ksub, layout, has_bias, rpos != nullptr)) return hipErrorInvalidValue;
  const ScoreArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), table, max_blocks, lse, bias,
                    rpos, scores, H, R, n_max, scale, pw, dead, ord};
  const dim3 grid(T.total);
  if (layout == kPaged) launch_l<kPaged>(has_bias, ksub, grid, st, a, T);
  else if (layout == kSlots) launch_l<kSlots>(has_bias, ksub, grid, st, a, T);
  else launch_l<kContig>(has_bias, ksub, grid, st, a, T);
  return hipGetLastError();
}

}  // namespace kvc
