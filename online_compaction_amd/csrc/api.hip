// Host side of libkvc: argument validation, workspace sizing, work tables and kernel dispatch.
// Declarations and the contract of every entry point are in include/kvc.h.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "am_cfg.h"
#include "kvc_internal.h"

namespace kvc {
// kernel launchers (score_mfma.hip, lse_mfma.hip, score_valu.hip, select.hip, retain.hip, compact.hip, am.hip)
int score_mfma_tiles(int n, int ksub);
bool score_mfma_ksub_ok(int ksub, int layout, bool has_bias, bool causal);
int lse_mfma_row_blocks(int R);
int valu_row_block(int R);
int valu_min_chunk_f32(int R);
int small_chunk();
int valu_cached_tiles(int n);
int contig_tiles(int m, bool f32);
int paged_tiles(int m);
hipError_t launch_score_mfma(int layout, bool has_bias, int ksub, const void* q, const void* k, const int32_t* table,
                             int max_blocks, const float* lse, const float* bias, const int32_t* rpos, float* scores,
                             int H, int R, int64_t n_max, float scale, int pw, int dead, const RowOrder& ord,
                             const SeqTable& T, hipStream_t st);
hipError_t launch_lse_partials_mfma(int layout, bool has_bias, const void* q, const void* k, const int32_t* table,
                                    int max_blocks, const float* bias, const int32_t* rpos, float2* partials, int H,
                                    int R, int64_t n_max, float scale, int kchunk, int dead, const RowOrder& ord,
                                    const SeqTable& T, hipStream_t st);
hipError_t launch_lse_combine(const float2* partials, float* lse_out, int H, int R, int kchunk, const SeqTable& T,
                              hipStream_t st);
// few proxy rows: float32 on the vector ALU (score_valu.hip), bf16 on MFMA (score_small.hip)
hipError_t launch_valu_lse_pass(int layout, const void* q, const void* k, const int32_t* table, int max_blocks,
                                const float* bias, const int32_t* rpos, float2* ws, bool cache, int H, int R,
                                int64_t n_max, float scale, int kchunk, int dead, const SeqTable& T, hipStream_t st);
hipError_t launch_valu_score_keys(int layout, const void* q, const void* k, const int32_t* table, int max_blocks,
                                  const float* lse, const float2* ws, const float* bias, const int32_t* rpos,
                                  float* out, int H, int R, int64_t n_max, float scale, int pw, int lse_kchunk,
                                  int chunk, int dead, const SeqTable& T, hipStream_t st);
hipError_t launch_small_lse_pass(int layout, const void* q, const void* k, const int32_t* table, int max_blocks,
                                 const float* bias, const int32_t* rpos, float2* ws, bool cache, int H, int R,
                                 int64_t n_max, float scale, int dead, const SeqTable& T, hipStream_t st);
hipError_t launch_small_score_keys(int layout, const void* q, const void* k, const int32_t* table, int max_blocks,
                                   const float* lse, const float2* ws, const float* bias, const int32_t* rpos,
                                   float* out, int H, int R, int64_t n_max, float scale, int pw, int dead,
                                   const SeqTable& T, hipStream_t st);
hipError_t launch_valu_score_cached(const float2* ws, float* out, int H, int R, int64_t n_max, int kchunk, int pw,
                                    const SeqTable& T, hipStream_t st);
hipError_t launch_evict_redirect(int32_t* slot_map, const int32_t* kept, int H, int64_t n_max, int m_max, int dead,
                                 const SeqTable& T, hipStream_t st);
int redirect_tiles(int n);
int64_t am_seq_floats(int H, int R, int n, int m, int S1, int S2, int St);
int am_target_blocks(int R);
int am_row_tiles(int R);
int am_col_items(int m);
int64_t am_key_tiles(int m);
int am_gemm_tiles(int rows);
int am_stages_rows(int m);
int am_stages_cols(int R);
hipError_t launch_am_stats(const float* lse, float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st);
hipError_t launch_am_me(float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st);
hipError_t launch_am_cols_fin(int mode, float* w, float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st);
hipError_t launch_am_eta(float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st);
hipError_t launch_am_target(int layout, const void* q, const void* k, const void* v, const int32_t* table,
                            int max_blocks, const int32_t* vtable, int vmax_blocks, const float* lse, float* ws,
                            int64_t n_max, float scale, const AmCfg& C, const SeqTable& T, hipStream_t st);
hipError_t launch_am_gemm(int kind, float* vc, float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st);
hipError_t launch_am_gram(float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st);
hipError_t launch_am_step(float* vc, float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st);
int64_t am_step_items(int Np);
hipError_t launch_am_gather(int layout, const void* k, const int32_t* table, int max_blocks, const int32_t* kept,
                            float* ws, int64_t n_max, const AmCfg& C, const SeqTable& T, hipStream_t st);
hipError_t launch_am_bias(int mode, const void* q, const float* w, const float* lse, float* ws, float scale,
                          const AmCfg& C, const SeqTable& T, hipStream_t st);
int64_t am_gather_items(int m);
int64_t am_gram_items(int Np);
hipError_t launch_am_split_sum(int kind, float* vc, float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st);
hipError_t launch_am_init(int layout, const void* v, const int32_t* table, int max_blocks, const int32_t* kept,
                          float* w, float* vc, const float* ws, int64_t n_max, const AmCfg& C, const SeqTable& T,
                          hipStream_t st);
hipError_t launch_am_finish(float* w, const float* ws, const AmCfg& C, const SeqTable& T, hipStream_t st);
hipError_t launch_select(const float* scores, int32_t* kept, int H, int64_t n_max, int m_max, const SeqTable& T,
                         hipStream_t st);
hipError_t launch_lrfu_update(const float* mass, float* state, int32_t* counts, int H, int64_t n_max, double top_p,
                              float decay, const SeqTable& T, hipStream_t st);
int side_tiles(int m);
hipError_t launch_compact_side(const float* src, float* dst, const int32_t* kept, int H, int64_t n_max, int m_max,
                               int B, const SeqTable& T, hipStream_t st);
hipError_t launch_compact_contig(bool f32, const void* k, const void* v, const int32_t* kept, void* ko, void* vo, int H,
                                 int64_t n_max, int m_max, const SeqTable& T, hipStream_t st);
hipError_t launch_paged_copy(bool f32, void* kp, void* vp, const int32_t* table, int max_blocks, const int32_t* kept,
                             int H, int m_max, int B, const SeqTable& T, hipStream_t st);
hipError_t launch_table_update(int32_t* table, int max_blocks, int32_t* freed, int B, const SeqTable& T,
                               hipStream_t st);
}  // namespace kvc

using namespace kvc;

namespace {

thread_local std::string g_err;

constexpr int kVersion = 300;          // 0.3.0: causal proxy rows (kvc_shape.row_pos)
constexpr int kBlockSize = 16;         // the one page size this build supports
constexpr int kMfmaMinRows = 16;       // bf16 units with fewer proxy rows use the VALU path
constexpr int kLseStage = 64;          // keys per stage of the MFMA LSE pass
constexpr int64_t kCUs = 256;          // compute units of the MI355X
constexpr int64_t kLseSlots = 2 * kCUs; // LSE workgroups resident at once (two per CU)
constexpr int kLseChunkOverhead = 256; // per-workgroup start-up cost, in keys
constexpr int64_t kMaxRows = 1 << 24;  // proxy rows per unit
constexpr int kMaxLen = 1 << 28;       // keys per sequence
constexpr size_t kAlign = 256;

kvc_status fail(kvc_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kvc_status fail(kvc_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

kvc_status ok() {
  g_err.clear();
  return KVC_OK;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int seq_start(const kvc_shape* sh, int s) { return sh->seq_starts ? sh->seq_starts[s] : 0; }

kvc_status check_shape(const kvc_shape* sh) {
  if (!sh) return fail(KVC_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (sh->num_seqs < 1 || sh->num_kv_heads < 1 || sh->group < 1 || sh->num_queries < 1)
    return fail(KVC_ERR_INVALID_ARGUMENT, "num_seqs, num_kv_heads, group and num_queries must be >= 1");
  if (sh->head_dim != kHeadDim)
    return fail(KVC_ERR_UNSUPPORTED, "head_dim %d: this build supports %d only", sh->head_dim, kHeadDim);
  if ((int64_t)sh->group * sh->num_queries > kMaxRows)
    return fail(KVC_ERR_UNSUPPORTED, "group * num_queries exceeds %lld proxy rows", (long long)kMaxRows);
  if (!sh->seq_lens) return fail(KVC_ERR_INVALID_ARGUMENT, "seq_lens is NULL");
  if (sh->n_max < 1 || sh->n_max > kMaxLen) return fail(KVC_ERR_INVALID_ARGUMENT, "n_max %d out of range", sh->n_max);
  for (int s = 0; s < sh->num_seqs; ++s) {
    const int n = sh->seq_lens[s];
    if (n < 1 || n > sh->n_max)
      return fail(KVC_ERR_INVALID_ARGUMENT, "seq_lens[%d] = %d outside [1, n_max = %d]", s, n, sh->n_max);
    const int a = seq_start(sh, s);
    if (a < 0 || (int64_t)a + n > kMaxLen)
      return fail(KVC_ERR_INVALID_ARGUMENT, "seq_starts[%d] = %d out of range", s, a);
  }
  return KVC_OK;
}

// Contiguous K/V rows of a segment must lie inside the n_max-row stride.
kvc_status check_contig_extent(const kvc_shape* sh, const char* what) {
  for (int s = 0; s < sh->num_seqs; ++s) {
    const int64_t end = (int64_t)seq_start(sh, s) + sh->seq_lens[s];
    if (end > sh->n_max)
      return fail(KVC_ERR_INVALID_ARGUMENT, "%s: sequence %d ends at cache row %lld > n_max %d", what, s,
                  (long long)end, sh->n_max);
  }
  return KVC_OK;
}

kvc_status check_dtype(kvc_dtype dt) {
  if (dt != KVC_F32 && dt != KVC_BF16) return fail(KVC_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dt);
  return KVC_OK;
}

kvc_status check_paging(const kvc_shape* sh, int32_t block_size, const int32_t* table, int32_t max_blocks,
                        const char* what) {
  if (block_size != kBlockSize)
    return fail(KVC_ERR_UNSUPPORTED, "%s: block_size %d: this build supports %d", what, block_size, kBlockSize);
  if (!table) return fail(KVC_ERR_INVALID_ARGUMENT, "%s: block_table is NULL", what);
  if (max_blocks < 1) return fail(KVC_ERR_INVALID_ARGUMENT, "%s: max_blocks must be >= 1", what);
  for (int s = 0; s < sh->num_seqs; ++s) {
    const int a = seq_start(sh, s);
    if (a % block_size)
      return fail(KVC_ERR_INVALID_ARGUMENT, "%s: seq_starts[%d] = %d is not a multiple of the block size", what, s,
                  a);
    const int64_t nb = ((int64_t)a + sh->seq_lens[s] + block_size - 1) / block_size;
    if (nb > max_blocks)
      return fail(KVC_ERR_INVALID_ARGUMENT, "%s: sequence %d needs %lld blocks > max_blocks %d", what, s,
                  (long long)nb, max_blocks);
  }
  return KVC_OK;
}

kvc_status check_view(const kvc_shape* sh, const kvc_kv_view* kv) {
  if (!kv) return fail(KVC_ERR_INVALID_ARGUMENT, "key view is NULL");
  if (!kv->data) return fail(KVC_ERR_INVALID_ARGUMENT, "key data is NULL");
  if (kvc_status st = check_dtype(kv->dtype)) return st;
  if (kv->slot_map) {
    if (kv->dead_slot < -1) return fail(KVC_ERR_INVALID_ARGUMENT, "dead_slot = %d < -1", kv->dead_slot);
    return check_contig_extent(sh, "slot map");
  }
  if (kv->block_size == 0) return check_contig_extent(sh, "keys");
  return check_paging(sh, kv->block_size, kv->block_table, kv->max_blocks, "keys");
}

// Kernel-side addressing of a validated view, and the index table it reads.
int layout_of(const kvc_kv_view* kv) { return kv->slot_map ? kSlots : (kv->block_size ? kPaged : kContig); }
const int32_t* index_of(const kvc_kv_view* kv) { return kv->slot_map ? kv->slot_map : kv->block_table; }

bool use_mfma(const kvc_shape* sh, const kvc_kv_view* kv) {
  return kv->dtype == KVC_BF16 && sh->group * sh->num_queries >= kMfmaMinRows;
}

// Key-chunk length of the MFMA LSE pass. kLseSlots workgroups (256 CUs, two resident each) run at
// once and a workgroup takes time in proportion to its keys plus kLseChunkOverhead (the rows it
// loads before its first key). With many workgroups the longest chunk is best (fewer partials,
// less overhead, and the last partial round costs little). With few, the chunk splits the longest
// sequence into equal parts (a multiple of the 64-key stage, at least 512 keys), choosing the
// split that minimises rounds x (chunk + overhead); ties go to the longer chunk. (The partials,
// and so the workspace, depend on the chunk: sizes come from the same shape, row_pos included.)
int64_t lse_workgroups(const kvc_shape* sh, int64_t rb, int kc) {
  int64_t wg = 0;
  for (int s = 0; s < sh->num_seqs; ++s) wg += (int64_t)sh->num_kv_heads * rb * ((sh->seq_lens[s] + kc - 1) / kc);
  return wg;
}

int mfma_kchunk(const kvc_shape* sh) {
  const int R = sh->group * sh->num_queries;
  const int64_t rb = lse_mfma_row_blocks(R);
  if (lse_workgroups(sh, rb, kLseMaxChunk) >= 8 * kLseSlots) return kLseMaxChunk;
  // causal rows: workgroups whose rows see few of their keys end early, so the shortest chunk
  // lets the others spread over the freed slots
  if (sh->row_pos) return 512;
  int longest = 0;
  for (int s = 0; s < sh->num_seqs; ++s) longest = std::max(longest, sh->seq_lens[s]);
  int best = kLseMaxChunk;
  int64_t best_cost = INT64_MAX;
  for (int parts = 1;; ++parts) {
    const int per = (longest + parts - 1) / parts;
    const int kc = (per + kLseStage - 1) / kLseStage * kLseStage;
    if (kc > kLseMaxChunk) continue;
    if (kc < 512) break;
    const int64_t rounds = (lse_workgroups(sh, rb, kc) + kLseSlots - 1) / kLseSlots;
    const int64_t cost = rounds * (std::min(kc, longest) + kLseChunkOverhead);
    if (cost < best_cost) {
      best_cost = cost;
      best = kc;
    }
  }
  return best;
}

// Keys per workgroup of a few-row pass. bf16 (MFMA): the kernels' fixed chunk. float32: a power
// of two, at least the kernels' shortest chunk (whole rounds of their key-row prefetch ring) and
// at most kValuMaxChunk; the longest that still gives every CU four workgroups (`per` = workgroups
// per key chunk: the row blocks of the LSE pass, 1 for the score pass), else the shortest.
int valu_chunk(const kvc_shape* sh, const kvc_kv_view* kv, int per) {
  if (kv->dtype != KVC_F32) return small_chunk();
  const int lo = valu_min_chunk_f32(sh->group * sh->num_queries);
  for (int c = kValuMaxChunk; c > lo; c >>= 1) {
    int64_t wg = 0;
    for (int s = 0; s < sh->num_seqs; ++s) wg += (int64_t)sh->num_kv_heads * per * ((sh->seq_lens[s] + c - 1) / c);
    if (wg >= 4 * kCUs) return c;
  }
  return lo;
}

// Row blocks of the few-row LSE pass: float32 takes the rows in blocks (of valu_row_block), the
// bf16 MFMA pass all of them (fewer than 16) at once.
int valu_row_blocks(const kvc_shape* sh, const kvc_kv_view* kv) {
  const int R = sh->group * sh->num_queries;
  if (kv->dtype != KVC_F32) return 1;
  const int rb = valu_row_block(R);
  return (R + rb - 1) / rb;
}

int lse_kchunk(const kvc_shape* sh, const kvc_kv_view* kv) {
  return use_mfma(sh, kv) ? mfma_kchunk(sh) : valu_chunk(sh, kv, valu_row_blocks(sh, kv));
}

// A VALU score call that computes its LSE keeps the logits of its LSE pass when there are few rows.
bool valu_cache(const kvc_shape* sh, const kvc_kv_view* kv) {
  return !use_mfma(sh, kv) && sh->group * sh->num_queries <= kValuMaxCacheRows;
}

// float2 slots of sequence s in the LSE pass's workspace region: the chunk partials (MFMA), or the
// VALU region (partials, then the cached logits when `for_score` and the rows are few).
int64_t lse_region_slots(const kvc_shape* sh, const kvc_kv_view* kv, int s, int kchunk, bool for_score) {
  const int R = sh->group * sh->num_queries;
  if (use_mfma(sh, kv)) return (int64_t)sh->num_kv_heads * ((sh->seq_lens[s] + kchunk - 1) / kchunk) * R;
  return valu_region_float2(sh->num_kv_heads, R, sh->seq_lens[s], kchunk, for_score && valu_cache(sh, kv));
}

size_t lse_region_bytes(const kvc_shape* sh, const kvc_kv_view* kv, bool for_score) {
  const int kc = lse_kchunk(sh, kv);
  int64_t slots = 0;
  for (int s = 0; s < sh->num_seqs; ++s) slots += lse_region_slots(sh, kv, s, kc, for_score);
  return align_up((size_t)slots * sizeof(float2));
}

size_t lse_bytes(const kvc_shape* sh) {
  return align_up((size_t)sh->num_seqs * sh->num_kv_heads * sh->group * sh->num_queries * sizeof(float));
}

// Run `body(T)` for consecutive slices of at most kChunkSeqs sequences; `items(s)` is the number
// of work items (workgroups) of sequence s and `offset(s)` a kernel-specific per-sequence value.
// Every entry point checks its launches' item counts with check_items before the first launch, so
// the count test here never fires on a validated call.
template <class Items, class Offset, class Body>
hipError_t for_each_chunk(const kvc_shape* sh, const int32_t* m, Items&& items, Offset&& offset, Body&& body,
                          const int32_t* cache_lens = nullptr) {
  for (int s0 = 0; s0 < sh->num_seqs; s0 += kChunkSeqs) {
    SeqTable T{};
    T.count = std::min(kChunkSeqs, sh->num_seqs - s0);
    T.first = s0;
    int64_t total = 0;
    for (int i = 0; i < T.count; ++i) {
      const int s = s0 + i;
      T.start[i] = (int32_t)total;
      T.n[i] = sh->seq_lens[s];
      T.m[i] = m ? m[s] : 0;
      T.kofs[i] = seq_start(sh, s);
      T.clen[i] = cache_lens ? cache_lens[s] : T.kofs[i] + T.n[i];
      T.off[i] = offset(s);
      total += (int64_t)items(s);
      if (total > INT32_MAX) return hipErrorInvalidConfiguration;
    }
    T.start[T.count] = (int32_t)total;
    T.total = (int32_t)total;
    if (total > 0) {
      const hipError_t e = body(T);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// Validation of one launch family: the work items of every slice of kChunkSeqs sequences, summed
// in 64 bits, must fit the int32 grid and work-item indices.
template <class Items>
kvc_status check_items(const kvc_shape* sh, Items&& items, const char* what) {
  for (int s0 = 0; s0 < sh->num_seqs; s0 += kChunkSeqs) {
    int64_t total = 0;
    for (int s = s0; s < std::min(sh->num_seqs, s0 + kChunkSeqs); ++s) {
      const int64_t it = (int64_t)items(s);
      if (it < 0 || it > INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "%s: sequence %d needs %lld work items", what, s,
                                                (long long)it);
      total += it;
    }
    if (total > INT32_MAX)
      return fail(KVC_ERR_UNSUPPORTED, "%s: %lld work items in one launch of sequences %d.. exceed 2^31 - 1", what,
                  (long long)total, s0);
  }
  return KVC_OK;
}

auto no_offset = [](int) -> int64_t { return 0; };

kvc_status hip_fail(hipError_t e, const char* what) {
  return fail(KVC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Key subtiles per wave of the MFMA score kernel (4, 8 or 9; 64 x that many keys per workgroup).
// A workgroup streams every proxy row past its keys, so its time grows with its keys plus about
// one subtile's worth of per-row work; a CU runs its share of the workgroups one after another
// in effect, and one alone on a CU (nothing to interleave with) still takes about 0.7 of two.
// 8 unless 4 (three resident per CU) or 9 (fewer, longer workgroups: fills the 512 resident
// slots when 512-key tiles overshoot them slightly) is estimated at least 5 % faster.
int score_ksub(const kvc_shape* sh, int layout, bool bias) {
  auto cost = [&](int ks) -> double {
    int64_t wg = 0;
    for (int s = 0; s < sh->num_seqs; ++s) wg += (int64_t)sh->num_kv_heads * score_mfma_tiles(sh->seq_lens[s], ks);
    const int64_t per_cu = (wg + kCUs - 1) / kCUs;
    return (per_cu >= 2 ? (double)per_cu : 1.4) * (ks + 1);
  };
  const double base = cost(8);
  int best = 8;
  double best_cost = 0.95 * base;
  for (int ks : {9, 4}) {
    if (!score_mfma_ksub_ok(ks, layout, bias, sh->row_pos != nullptr)) continue;
    const double c = cost(ks);
    if (c < best_cost) {
      best_cost = c;
      best = ks;
    }
  }
  return best;
}

// The order the MFMA kernels take the proxy rows in: query-major (the G query heads' rows of one
// query position together) with causal rows, when 1 < G <= 256 (the multiply-high division is
// exact there); the stored order otherwise.
RowOrder row_order(const kvc_shape* sh) {
  const int G = sh->group;
  if (!sh->row_pos || G <= 1 || G > 256) return RowOrder{1, sh->num_queries, 0u};
  const uint32_t magic = (uint32_t)(((uint64_t)1 << 32) / (uint64_t)G + 1);
  return RowOrder{G, sh->num_queries, magic};
}

// Work items of the LSE pass per sequence: the partial kernel's (key chunk x row block) workgroups
// and the combine kernel's 64-row items.
int64_t lse_partial_items(const kvc_shape* sh, const kvc_kv_view* kv, int s) {
  const int R = sh->group * sh->num_queries;
  const int kc = lse_kchunk(sh, kv);
  const int64_t rb = use_mfma(sh, kv) ? lse_mfma_row_blocks(R) : valu_row_blocks(sh, kv);
  return (int64_t)sh->num_kv_heads * rb * ((sh->seq_lens[s] + kc - 1) / kc);
}

int64_t lse_combine_items(const kvc_shape* sh) {
  return (int64_t)sh->num_kv_heads * ((sh->group * sh->num_queries + 63) / 64);
}

kvc_status check_lse_work(const kvc_shape* sh, const kvc_kv_view* kv) {
  if (kvc_status st = check_items(sh, [&](int s) { return lse_partial_items(sh, kv, s); }, "lse partial kernel"))
    return st;
  return check_items(sh, [&](int) { return lse_combine_items(sh); }, "lse combine kernel");
}

// Per-sequence offsets (float2 units) of the LSE pass's regions in the workspace.
std::vector<int64_t> lse_region_offsets(const kvc_shape* sh, const kvc_kv_view* kv, bool for_score) {
  const int kc = lse_kchunk(sh, kv);
  std::vector<int64_t> off(sh->num_seqs);
  int64_t acc = 0;
  for (int s = 0; s < sh->num_seqs; ++s) {
    off[s] = acc;
    acc += lse_region_slots(sh, kv, s, kc, for_score);
  }
  return off;
}

// The LSE pass: per-chunk partials (and, for a VALU score call with few rows, the cached logits)
// into the workspace regions at ws_partials. Unless `for_score` is a VALU call (whose score kernel
// merges the partials itself), the partials are then combined into lse_out. The work was checked
// by check_lse_work.
kvc_status run_lse(const kvc_shape* sh, const void* q, const kvc_kv_view* kv, const float* bias, float* lse_out,
                   void* ws_partials, hipStream_t st, bool for_score = false) {
  const int H = sh->num_kv_heads;
  const int R = sh->group * sh->num_queries;
  const bool mf = use_mfma(sh, kv);
  const int layout = layout_of(kv);
  const int32_t* index = index_of(kv);
  const bool has_bias = bias != nullptr;
  const int kc = lse_kchunk(sh, kv);
  const std::vector<int64_t> off = lse_region_offsets(sh, kv, for_score);
  auto* parts = static_cast<float2*>(ws_partials);
  auto offset = [&](int s) -> int64_t { return off[s]; };
  hipError_t e = for_each_chunk(
      sh, nullptr, [&](int s) { return lse_partial_items(sh, kv, s); }, offset,
      [&](const SeqTable& T) {
        if (mf)
          return launch_lse_partials_mfma(layout, has_bias, q, kv->data, index, kv->max_blocks, bias, sh->row_pos,
                                          parts, H, R, sh->n_max, sh->scale, kc, kv->dead_slot, row_order(sh), T,
                                          st);
        const bool cache = for_score && valu_cache(sh, kv);
        if (kv->dtype == KVC_F32)
          return launch_valu_lse_pass(layout, q, kv->data, index, kv->max_blocks, bias, sh->row_pos, parts, cache, H, R,
                                      sh->n_max, sh->scale, kc, kv->dead_slot, T, st);
        return launch_small_lse_pass(layout, q, kv->data, index, kv->max_blocks, bias, sh->row_pos, parts, cache, H, R,
                                     sh->n_max, sh->scale, kv->dead_slot, T, st);
      });
  if (e != hipSuccess) return hip_fail(e, "lse partial kernel");
  if (for_score && !mf) return KVC_OK;
  e = for_each_chunk(
      sh, nullptr, [&](int) { return lse_combine_items(sh); }, offset,
      [&](const SeqTable& T) { return launch_lse_combine(parts, lse_out, H, R, kc, T, st); });
  if (e != hipSuccess) return hip_fail(e, "lse combine kernel");
  return KVC_OK;
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// Static scratch of kvc_score_noalloc: the LSE partials and the LSE of a score call that computes
// its own LSE, in a device array of fixed size instead of a caller-provided workspace. Each GPU
// holds its own copy for the life of the process. Host code never passes `scratch` itself to a
// kernel (on the host it only names the variable): its device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept in g_scratch_ptr.
// ------------------------------------------------------------------------------------------------
static constexpr size_t kScratchBytes = KVC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this process's scratch on the device that runs `stream`.
kvc_status scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "device of the stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(KVC_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) return hip_fail(e2, "hipSetDevice");
    }
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(KVC_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVC_OK;
}

}  // namespace

extern "C" {

const char* kvc_status_string(kvc_status st) {
  switch (st) {
    case KVC_OK: return "ok";
    case KVC_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KVC_ERR_UNSUPPORTED: return "unsupported";
    case KVC_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KVC_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* kvc_last_error(void) { return g_err.c_str(); }

int kvc_version(void) { return kVersion; }

size_t kvc_lse_workspace_size(const kvc_shape* sh, const kvc_kv_view* k) {
  if (check_shape(sh) != KVC_OK || check_view(sh, k) != KVC_OK) return 0;
  return lse_region_bytes(sh, k, false);
}

kvc_status kvc_lse(const kvc_shape* sh, const void* q, const kvc_kv_view* k, const float* bias, float* lse_out,
                   void* ws, size_t ws_bytes, void* stream) {
  if (kvc_status st = check_shape(sh)) return st;
  if (kvc_status st = check_view(sh, k)) return st;
  if (!q || !lse_out) return fail(KVC_ERR_INVALID_ARGUMENT, "q and lse_out must be non-NULL");
  if (!isfinite(sh->scale)) return fail(KVC_ERR_INVALID_ARGUMENT, "scale must be finite");
  const size_t need = lse_region_bytes(sh, k, false);
  if (!ws || ws_bytes < need)
    return fail(KVC_ERR_WORKSPACE_TOO_SMALL, "lse needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
  if (kvc_status st = check_lse_work(sh, k)) return st;
  if (kvc_status st = run_lse(sh, q, k, bias, lse_out, ws, static_cast<hipStream_t>(stream))) return st;
  return ok();
}

size_t kvc_score_workspace_size(const kvc_shape* sh, const kvc_kv_view* k, int lse_supplied) {
  if (check_shape(sh) != KVC_OK || check_view(sh, k) != KVC_OK) return 0;
  if (lse_supplied) return 0;
  return lse_region_bytes(sh, k, true) + lse_bytes(sh);
}

// Per-key reduction over the proxy rows of alpha^pw: pw = 2 gives the TE score (after the square
// root), pw = 1 the attention mass.
static kvc_status run_score(const kvc_shape* sh, const void* q, const kvc_kv_view* k, const float* lse,
                            const float* bias, float* out, void* ws, size_t ws_bytes, void* stream, int pw,
                            const char* what) {
  if (kvc_status st = check_shape(sh)) return st;
  if (kvc_status st = check_view(sh, k)) return st;
  if (!q || !out) return fail(KVC_ERR_INVALID_ARGUMENT, "q and %s must be non-NULL", what);
  if (!isfinite(sh->scale)) return fail(KVC_ERR_INVALID_ARGUMENT, "scale must be finite");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int R = sh->group * sh->num_queries;
  const bool mf = use_mfma(sh, k);
  const int layout = layout_of(k);
  const int32_t* index = index_of(k);
  const int H = sh->num_kv_heads;
  const bool f32 = k->dtype == KVC_F32;
  // MFMA: LSE pass + combine (when not supplied), then the score kernel over key tiles. VALU: the
  // LSE pass (logits cached when the rows are few), then the score kernel -- from the cached
  // logits, or from the keys again -- merging the partials itself.
  const bool cached = !lse && valu_cache(sh, k);
  const int ksub = mf ? score_ksub(sh, layout, bias != nullptr) : 0;
  const int vchunk = mf ? 0 : valu_chunk(sh, k, 1);
  auto items = [&](int s) -> int64_t {
    const int n = sh->seq_lens[s];
    return (int64_t)H * (mf ? score_mfma_tiles(n, ksub) : cached ? valu_cached_tiles(n) : (n + vchunk - 1) / vchunk);
  };
  if (kvc_status s2 = check_items(sh, items, "score kernel")) return s2;
  const float* lse_rows = lse;
  const size_t rb_bytes = lse ? 0 : lse_region_bytes(sh, k, true);
  if (!lse) {
    const size_t need = rb_bytes + lse_bytes(sh);
    if (!ws || ws_bytes < need)
      return fail(KVC_ERR_WORKSPACE_TOO_SMALL, "%s needs %zu workspace bytes, got %zu", what, need, ws ? ws_bytes : 0);
    if (kvc_status s2 = check_lse_work(sh, k)) return s2;
    float* lse_ws = reinterpret_cast<float*>(static_cast<char*>(ws) + rb_bytes);
    if (kvc_status s2 = run_lse(sh, q, k, bias, lse_ws, ws, st, true)) return s2;
    lse_rows = mf ? lse_ws : nullptr;  // VALU: merged from the partials by the score kernel
  }
  const float2* regions = static_cast<const float2*>(ws);
  const std::vector<int64_t> off = (!lse && !mf) ? lse_region_offsets(sh, k, true) : std::vector<int64_t>();
  auto offset = [&](int s) -> int64_t { return off.empty() ? 0 : off[s]; };
  const int lkc = (!lse && !mf) ? lse_kchunk(sh, k) : 0;
  const hipError_t e = for_each_chunk(
      sh, nullptr, items, offset, [&](const SeqTable& T) {
        if (mf)
          return launch_score_mfma(layout, bias != nullptr, ksub, q, k->data, index, k->max_blocks, lse_rows, bias,
                                   sh->row_pos, out, H, R, sh->n_max, sh->scale, pw, k->dead_slot, row_order(sh), T,
                                   st);
        if (cached) return launch_valu_score_cached(regions, out, H, R, sh->n_max, lkc, pw, T, st);
        if (f32)
          return launch_valu_score_keys(layout, q, k->data, index, k->max_blocks, lse_rows, regions, bias, sh->row_pos,
                                        out, H, R, sh->n_max, sh->scale, pw, lkc, vchunk, k->dead_slot, T, st);
        return launch_small_score_keys(layout, q, k->data, index, k->max_blocks, lse_rows, regions, bias, sh->row_pos,
                                       out, H, R, sh->n_max, sh->scale, pw, k->dead_slot, T, st);
      });
  if (e != hipSuccess) return hip_fail(e, "score kernel");
  return ok();
}

kvc_status kvc_score(const kvc_shape* sh, const void* q, const kvc_kv_view* k, const float* lse, const float* bias,
                     float* scores, void* ws, size_t ws_bytes, void* stream) {
  return run_score(sh, q, k, lse, bias, scores, ws, ws_bytes, stream, 2, "scores");
}

kvc_status kvc_score_noalloc(const kvc_shape* sh, const void* q, const kvc_kv_view* k, const float* lse,
                             const float* bias, float* scores, void* stream) {
  if (kvc_status st = check_shape(sh)) return st;
  if (kvc_status st = check_view(sh, k)) return st;
  if (lse) return run_score(sh, q, k, lse, bias, scores, nullptr, 0, stream, 2, "scores");
  const size_t need = lse_region_bytes(sh, k, true) + lse_bytes(sh);
  if (need > kScratchBytes)
    return fail(KVC_ERR_UNSUPPORTED,
                "kvc_score_noalloc: computing the LSE of this shape needs %zu bytes of scratch; the static scratch "
                "holds %zu (supply the LSE, or call kvc_score with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  if (kvc_status st = scratch_for_stream(static_cast<hipStream_t>(stream), &ws)) return st;
  return run_score(sh, q, k, lse, bias, scores, ws, kScratchBytes, stream, 2, "scores");
}

kvc_status kvc_attention_mass(const kvc_shape* sh, const void* q, const kvc_kv_view* k, const float* lse,
                              const float* bias, float* mass, void* ws, size_t ws_bytes, void* stream) {
  return run_score(sh, q, k, lse, bias, mass, ws, ws_bytes, stream, 1, "mass");
}

static kvc_status check_budgets(const kvc_shape* sh, const int32_t* m, int32_t m_max) {
  if (!m) return fail(KVC_ERR_INVALID_ARGUMENT, "m is NULL");
  int mm = 0;
  for (int s = 0; s < sh->num_seqs; ++s) {
    if (m[s] < 0 || m[s] > sh->seq_lens[s])
      return fail(KVC_ERR_INVALID_ARGUMENT, "m[%d] = %d outside [0, n = %d]", s, m[s], sh->seq_lens[s]);
    mm = std::max(mm, m[s]);
  }
  if (m_max < mm || m_max < 1)
    return fail(KVC_ERR_INVALID_ARGUMENT, "m_max %d must be >= 1 and >= max m (%d)", m_max, mm);
  return KVC_OK;
}

kvc_status kvc_select_topm(const kvc_shape* sh, const float* scores, const int32_t* m, int32_t m_max, int32_t* kept,
                           void* stream) {
  if (kvc_status st = check_shape(sh)) return st;
  if (kvc_status st = check_budgets(sh, m, m_max)) return st;
  if (!scores || !kept) return fail(KVC_ERR_INVALID_ARGUMENT, "scores and kept must be non-NULL");
  auto items = [&](int) -> int64_t { return sh->num_kv_heads; };
  if (kvc_status st = check_items(sh, items, "select kernel")) return st;
  const hipError_t err = for_each_chunk(
      sh, m, items, no_offset, [&](const SeqTable& T) {
        return launch_select(scores, kept, sh->num_kv_heads, sh->n_max, m_max, T, static_cast<hipStream_t>(stream));
      });
  if (err != hipSuccess) return hip_fail(err, "select kernel");
  return ok();
}

kvc_status kvc_lrfu_update(const kvc_shape* sh, const float* mass, double top_p, float decay, float* state,
                           int32_t* counts, void* stream) {
  if (kvc_status st = check_shape(sh)) return st;
  if (!mass || !state) return fail(KVC_ERR_INVALID_ARGUMENT, "mass and state must be non-NULL");
  if (!(top_p > 0.0 && top_p <= 1.0)) return fail(KVC_ERR_INVALID_ARGUMENT, "top_p = %g outside (0, 1]", top_p);
  if (!(decay >= 0.0f && decay <= 1.0f)) return fail(KVC_ERR_INVALID_ARGUMENT, "decay = %g outside [0, 1]", decay);
  auto items = [&](int) -> int64_t { return sh->num_kv_heads; };
  if (kvc_status st = check_items(sh, items, "lrfu kernel")) return st;
  const hipError_t err = for_each_chunk(
      sh, nullptr, items, no_offset, [&](const SeqTable& T) {
        return launch_lrfu_update(mass, state, counts, sh->num_kv_heads, sh->n_max, top_p, decay, T,
                                  static_cast<hipStream_t>(stream));
      });
  if (err != hipSuccess) return hip_fail(err, "lrfu kernel");
  return ok();
}

kvc_status kvc_compact_side(const kvc_shape* sh, int32_t block_size, const int32_t* kept, const int32_t* m,
                            int32_t m_max, const float* src, float* dst, void* stream) {
  if (kvc_status st = check_shape(sh)) return st;
  if (kvc_status st = check_budgets(sh, m, m_max)) return st;
  if (kvc_status st = check_contig_extent(sh, "compact_side")) return st;
  if (block_size < 0) return fail(KVC_ERR_INVALID_ARGUMENT, "block_size = %d < 0", block_size);
  if (!kept || !src || !dst) return fail(KVC_ERR_INVALID_ARGUMENT, "kept, src and dst must be non-NULL");
  if (static_cast<const void*>(src) == static_cast<const void*>(dst))
    return fail(KVC_ERR_INVALID_ARGUMENT, "src and dst must be distinct buffers");
  auto items = [&](int s) -> int64_t { return (int64_t)sh->num_kv_heads * side_tiles(m[s]); };
  if (kvc_status st = check_items(sh, items, "side-array compaction kernel")) return st;
  const hipError_t err = for_each_chunk(
      sh, m, items, no_offset, [&](const SeqTable& T) {
        return launch_compact_side(src, dst, kept, sh->num_kv_heads, sh->n_max, m_max, block_size, T,
                                   static_cast<hipStream_t>(stream));
      });
  if (err != hipSuccess) return hip_fail(err, "side-array compaction kernel");
  return ok();
}

kvc_status kvc_evict_redirect(const kvc_shape* sh, const int32_t* kept, const int32_t* m, int32_t m_max,
                              int32_t* slot_map, int32_t dead_slot, void* stream) {
  if (kvc_status st = check_shape(sh)) return st;
  if (kvc_status st = check_budgets(sh, m, m_max)) return st;
  if (kvc_status st = check_contig_extent(sh, "slot map")) return st;
  if (!kept || !slot_map) return fail(KVC_ERR_INVALID_ARGUMENT, "kept and slot_map must be non-NULL");
  if (dead_slot < 0) return fail(KVC_ERR_INVALID_ARGUMENT, "dead_slot = %d < 0", dead_slot);
  auto items = [&](int s) -> int64_t { return (int64_t)sh->num_kv_heads * redirect_tiles(sh->seq_lens[s]); };
  if (kvc_status st = check_items(sh, items, "redirect kernel")) return st;
  const hipError_t err = for_each_chunk(
      sh, m, items, no_offset,
      [&](const SeqTable& T) {
        return launch_evict_redirect(slot_map, kept, sh->num_kv_heads, sh->n_max, m_max, dead_slot, T,
                                     static_cast<hipStream_t>(stream));
      });
  if (err != hipSuccess) return hip_fail(err, "redirect kernel");
  return ok();
}

// ------------------------------------------------------------------------------------------------
// Attention Matching
// ------------------------------------------------------------------------------------------------
// Split counts of the two P_C products (at most 8 splits, at least 4 stages of 32 per split). A function of the shape alone, so that the workspace size and the fit agree.
static int am_side_rows_padded(int R, int m) { return am_rows_side(R, m) ? (R + 63) / 64 * 64 : (m + 63) / 64 * 64; }

static void am_splits(const kvc_shape* sh, const int32_t* m, int* S1, int* S2, int* St) {
  const int H = sh->num_kv_heads, R = sh->group * sh->num_queries;
  int64_t t1 = 0, t2 = 0, out1 = 0, out2 = 0;
  int st1 = INT32_MAX, st2 = am_stages_cols(R);
  for (int s = 0; s < sh->num_seqs; ++s) {
    if (m[s] == 0) continue;
    const int ldm = (m[s] + 63) / 64 * 64;
    t1 += (int64_t)H * am_gemm_tiles(R);
    t2 += (int64_t)H * am_gemm_tiles(ldm);
    out1 += (int64_t)H * R * 128;
    out2 += (int64_t)H * ldm * 128;
    st1 = std::min(st1, am_stages_rows(m[s]));
  }
  // The split count that minimises rounds of workgroups (one per CU) x stages per split, plus
  // the round trip of the partial products through memory: each split writes the whole output
  // once and the split sum reads it back (8 bytes per output element), priced against a round
  // of stages, in which the 256 resident workgroups read 16 KB of the left operand each.
  // Fewer splits on a tie.
  auto pick = [](int64_t tiles, int stages, int64_t out) {
    if (tiles == 0) return 1;
    const double part = 8.0 * (double)out / (256.0 * 16384.0);
    int best = 1;
    double best_cost = 1e300;
    for (int sp = 1; sp <= 8 && sp <= std::max(1, stages / 4); ++sp) {
      const int64_t rounds = (tiles * sp + 255) / 256, per = (stages + sp - 1) / sp;
      const double cost = (double)(rounds * per) + (sp > 1 ? sp * part : 0.0);
      if (cost < best_cost) {
        best_cost = cost;
        best = sp;
      }
    }
    return best;
  };
  *S1 = pick(t1, st1, out1);
  *S2 = pick(t2, st2, out2);
  // the target's key splits: enough workgroups for every CU (one each), at least four 64-key
  // chunks per split
  int64_t tt = 0;
  int chunks = INT32_MAX;
  for (int s = 0; s < sh->num_seqs; ++s) {
    if (m[s] == 0) continue;
    tt += (int64_t)H * am_target_blocks(R);
    chunks = std::min(chunks, (sh->seq_lens[s] + 63) / 64);
  }
  int sp = 1;
  while (sp < 8 && tt * sp < 256 && chunks / (2 * sp) >= 4) sp *= 2;
  *St = sp;
}

static size_t am_bytes(const kvc_shape* sh, const int32_t* m) {
  int S1, S2, St;
  am_splits(sh, m, &S1, &S2, &St);
  const int H = sh->num_kv_heads, R = sh->group * sh->num_queries;
  int64_t f = 0;
  for (int s = 0; s < sh->num_seqs; ++s) f += am_seq_floats(H, R, sh->seq_lens[s], m[s], S1, S2, St);
  return ((size_t)f * sizeof(float) + 255) & ~size_t(255);
}

static kvc_status check_am(const kvc_shape* sh, const kvc_kv_view* k, const kvc_kv_view* v) {
  if (kvc_status st = check_view(sh, k)) return st;
  if (kvc_status st = check_view(sh, v)) return st;
  if (k->slot_map || v->slot_map) return fail(KVC_ERR_UNSUPPORTED, "attention matching: slot-map views");
  if (sh->row_pos) return fail(KVC_ERR_UNSUPPORTED, "attention matching: causal proxy rows (row_pos)");
  if (k->dtype != KVC_BF16 || v->dtype != KVC_BF16) return fail(KVC_ERR_UNSUPPORTED, "attention matching: bf16 only");
  if (!use_mfma(sh, k))
    return fail(KVC_ERR_UNSUPPORTED, "attention matching needs G * q >= %d proxy rows", kMfmaMinRows);
  if (k->block_size != v->block_size) return fail(KVC_ERR_INVALID_ARGUMENT, "K and V views differ in layout");
  return KVC_OK;
}

size_t kvc_am_workspace_size(const kvc_shape* sh, const kvc_kv_view* k, const kvc_kv_view* v, const int32_t* m,
                             int lse_supplied) {
  if (check_shape(sh) != KVC_OK || check_am(sh, k, v) != KVC_OK || !m) return 0;
  for (int s = 0; s < sh->num_seqs; ++s)
    if (m[s] < 0 || m[s] > sh->seq_lens[s]) return 0;
  const size_t lse_part = lse_supplied ? 0 : lse_region_bytes(sh, k, false) + lse_bytes(sh);
  return lse_part + am_bytes(sh, m);
}

kvc_status kvc_am_fit(const kvc_shape* sh, const void* q, const kvc_kv_view* k, const kvc_kv_view* v,
                      const float* lse, const int32_t* kept, const int32_t* m, int32_t m_max, int32_t iters_beta,
                      int32_t iters_v, float* beta, float* v_c, void* ws, size_t ws_bytes, void* stream) {
  if (kvc_status st = check_shape(sh)) return st;
  if (kvc_status st = check_am(sh, k, v)) return st;
  if (kvc_status st = check_budgets(sh, m, m_max)) return st;
  if (!q || !kept || !beta || !v_c) return fail(KVC_ERR_INVALID_ARGUMENT, "q, kept, beta and v_c must be non-NULL");
  if (!isfinite(sh->scale)) return fail(KVC_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (iters_beta < 0 || iters_beta > 100000 || iters_v < 0 || iters_v > 100000)
    return fail(KVC_ERR_INVALID_ARGUMENT, "iteration counts must lie in [0, 100000]");
  const size_t lse_part = lse ? 0 : lse_region_bytes(sh, k, false) + lse_bytes(sh);
  const size_t need = lse_part + am_bytes(sh, m);
  if (!ws || ws_bytes < need)
    return fail(KVC_ERR_WORKSPACE_TOO_SMALL, "attention matching needs %zu workspace bytes, got %zu", need,
                ws ? ws_bytes : 0);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int H = sh->num_kv_heads, R = sh->group * sh->num_queries;
  AmCfg C{H, R, m_max, 1, 1, 1, 0, 0};
  am_splits(sh, m, &C.S1, &C.S2, &C.St);
  // work items per sequence of every launch family; a sequence with m = 0 has nothing to fit and
  // gets no work items
  auto per = [&](auto&& f) { return [&, f](int s) -> int64_t { return m[s] ? (int64_t)H * f(s) : 0; }; };
  auto units = per([](int) -> int64_t { return 1; });
  auto cols = per([&](int s) -> int64_t { return am_col_items(m[s]); });
  auto rtiles = per([&](int) -> int64_t { return am_row_tiles(R); });
  auto tblocks = per([&](int) -> int64_t { return (int64_t)am_target_blocks(R) * C.St; });
  auto ktiles = per([&](int s) { return am_key_tiles(m[s]); });
  auto gemm0 = per([&](int) -> int64_t { return (int64_t)am_gemm_tiles(R) * C.S1; });
  auto gemm1 = per([&](int s) -> int64_t { return (int64_t)am_gemm_tiles((m[s] + 63) / 64 * 64) * C.S2; });
  // the value iteration (am_rows_side): Gram tile pairs, step tiles and their split sums, and the
  // launches that only one side's sequences take part in
  auto side = [&](int s) { return am_rows_side(R, m[s]); };
  auto gram = per([&](int s) { return am_gram_items(am_side_rows_padded(R, m[s])); });
  auto gathers = per([&](int s) { return am_gather_items(m[s]); });
  auto steps = per([&](int s) { return am_step_items(am_side_rows_padded(R, m[s])); });
  auto ktile_items = [&](int s) -> int64_t { return (int64_t)am_gemm_tiles((m[s] + 63) / 64 * 64) * C.S2; };
  auto gemm1_rows = per([&](int s) -> int64_t { return side(s) ? ktile_items(s) : 0; });
  auto gemm1_keys = per([&](int s) -> int64_t { return side(s) ? 0 : ktile_items(s); });
  auto ktiles_rows = per([&](int s) -> int64_t { return side(s) ? am_key_tiles(m[s]) : 0; });
  auto ktiles_keys = per([&](int s) -> int64_t { return side(s) ? 0 : am_key_tiles(m[s]); });
  {
    const char* what = "attention matching kernel";
    kvc_status e = KVC_OK;
    if (!e) e = check_items(sh, units, what);
    if (!e) e = check_items(sh, cols, what);
    if (!e) e = check_items(sh, rtiles, what);
    if (!e) e = check_items(sh, tblocks, what);
    if (!e) e = check_items(sh, ktiles, what);
    if (!e) e = check_items(sh, gemm0, what);
    if (!e) e = check_items(sh, gemm1, what);
    if (!e) e = check_items(sh, gram, what);
    if (!e) e = check_items(sh, gathers, what);
    if (!e) e = check_items(sh, steps, what);
    if (!e && !lse) e = check_lse_work(sh, k);
    if (e) return e;
  }
  const float* lse_rows = lse;
  if (!lse) {
    float* lse_ws = reinterpret_cast<float*>(static_cast<char*>(ws) + lse_region_bytes(sh, k, false));
    if (kvc_status s2 = run_lse(sh, q, k, nullptr, lse_ws, ws, st)) return s2;
    lse_rows = lse_ws;
  }
  float* amws = reinterpret_cast<float*>(static_cast<char*>(ws) + lse_part);
  std::vector<int64_t> off(sh->num_seqs);
  int64_t acc = 0;
  for (int s = 0; s < sh->num_seqs; ++s) {
    off[s] = acc;
    acc += am_seq_floats(H, R, sh->seq_lens[s], m[s], C.S1, C.S2, C.St);
  }
  auto offset = [&](int s) -> int64_t { return off[s]; };
  const int layout = layout_of(k);
  const int64_t nm = sh->n_max;
  auto run = [&](auto&& items, auto&& body) -> hipError_t { return for_each_chunk(sh, m, items, offset, body); };
#define KVC_AM_STEP(ITEMS, CALL)                                              \
  do {                                                                        \
    const hipError_t e_ = run(ITEMS, [&](const SeqTable& T) { return CALL; }); \
    if (e_ != hipSuccess) return hip_fail(e_, "attention matching kernel");      \
  } while (0)
  KVC_AM_STEP(units, launch_am_stats(lse_rows, amws, C, T, st));
  KVC_AM_STEP(gathers,
              launch_am_gather(layout, k->data, k->block_table, k->max_blocks, kept, amws, nm, C, T, st));
  KVC_AM_STEP(rtiles, launch_am_bias(3, q, beta, lse_rows, amws, sh->scale, C, T, st));  // ME
  KVC_AM_STEP(units, launch_am_me(amws, C, T, st));
  KVC_AM_STEP(rtiles, launch_am_bias(0, q, beta, lse_rows, amws, sh->scale, C, T, st));  // E^T z
  KVC_AM_STEP(cols, launch_am_cols_fin(0, beta, amws, C, T, st));
  KVC_AM_STEP(cols, launch_am_init(layout, v->data, v->block_table, v->max_blocks, kept, beta, v_c, amws, nm, C, T,
                                   st));
  for (int it = 0; it < iters_beta; ++it) {
    KVC_AM_STEP(rtiles, launch_am_bias(1, q, beta, lse_rows, amws, sh->scale, C, T, st));
    KVC_AM_STEP(cols, launch_am_cols_fin(1, beta, amws, C, T, st));
  }
  KVC_AM_STEP(rtiles, launch_am_bias(2, q, beta, lse_rows, amws, sh->scale, C, T, st));  // P_C, P_C^T
  KVC_AM_STEP(cols, launch_am_cols_fin(0, beta, amws, C, T, st));                       // column sums
  KVC_AM_STEP(units, launch_am_eta(amws, C, T, st));
  // Values: k = iters_v Landweber steps V <- V - eta P_C^T (P_C V - Y), run as the iteration of
  // the residual on the smaller side of P_C (exact rewriting of the same steps): with
  // Z_0 = P_C V_0 - Y,
  //   rows side:  Z_{t+1} = Z_t - eta (P_C P_C^T) Z_t,          V_k = V_0 - eta P_C^T sum_{t<k} Z_t
  //   keys side:  r_0 = P_C^T Z_0, r_{t+1} = r_t - eta (P_C^T P_C) r_t,   V_k = V_0 - eta sum_{t<k} r_t
  // (one step, k = 1, is the direct product for both).
  if (iters_v > 0) {
    KVC_AM_STEP(tblocks, launch_am_target(layout, q, k->data, v->data, k->block_table, k->max_blocks, v->block_table,
                                         v->max_blocks, lse_rows, amws, nm, sh->scale, C, T, st));
    C.mode = 0;
    C.xsel = 0;
    KVC_AM_STEP(gemm0, launch_am_gemm(0, v_c, amws, C, T, st));
    if (C.S1 > 1) KVC_AM_STEP(rtiles, launch_am_split_sum(0, v_c, amws, C, T, st));
    if (iters_v == 1) {
      KVC_AM_STEP(gemm1, launch_am_gemm(1, v_c, amws, C, T, st));
      if (C.S2 > 1) KVC_AM_STEP(ktiles, launch_am_split_sum(1, v_c, amws, C, T, st));
    } else {
      C.mode = 1;  // keys side: the first iterate r_0
      KVC_AM_STEP(gemm1_keys, launch_am_gemm(1, v_c, amws, C, T, st));
      if (C.S2 > 1) KVC_AM_STEP(ktiles_keys, launch_am_split_sum(1, v_c, amws, C, T, st));
      KVC_AM_STEP(gram, launch_am_gram(amws, C, T, st));
      for (int it = 1; it < iters_v; ++it) {
        C.xsel = (it - 1) & 1;
        C.mode = it == iters_v - 1;
        KVC_AM_STEP(steps, launch_am_step(v_c, amws, C, T, st));
      }
      C.mode = 0;  // rows side: V_k = V_0 - eta P_C^T (sum of the iterates), read from where the last step put it
      C.xsel = (iters_v - 1) & 1;
      KVC_AM_STEP(gemm1_rows, launch_am_gemm(1, v_c, amws, C, T, st));
      if (C.S2 > 1) KVC_AM_STEP(ktiles_rows, launch_am_split_sum(1, v_c, amws, C, T, st));
    }
  }
  KVC_AM_STEP(cols, launch_am_finish(beta, amws, C, T, st));
#undef KVC_AM_STEP
  return ok();
}

kvc_status kvc_compact_contig(const kvc_shape* sh, kvc_dtype dtype, const void* k, const void* v, const int32_t* kept,
                              const int32_t* m, int32_t m_max, void* k_out, void* v_out, void* stream) {
  if (kvc_status st = check_shape(sh)) return st;
  if (kvc_status st = check_dtype(dtype)) return st;
  if (kvc_status st = check_budgets(sh, m, m_max)) return st;
  if (kvc_status st = check_contig_extent(sh, "compact_contig")) return st;
  if (!k || !v || !kept || !k_out || !v_out)
    return fail(KVC_ERR_INVALID_ARGUMENT, "k, v, kept, k_out and v_out must be non-NULL");
  auto items = [&](int s) -> int64_t { return (int64_t)sh->num_kv_heads * contig_tiles(m[s], dtype == KVC_F32); };
  if (kvc_status st = check_items(sh, items, "contiguous compaction kernel")) return st;
  const hipError_t err = for_each_chunk(
      sh, m, items, no_offset, [&](const SeqTable& T) {
        return launch_compact_contig(dtype == KVC_F32, k, v, kept, k_out, v_out, sh->num_kv_heads, sh->n_max, m_max,
                                     T, static_cast<hipStream_t>(stream));
      });
  if (err != hipSuccess) return hip_fail(err, "contiguous compaction kernel");
  return ok();
}

kvc_status kvc_compact_paged(const kvc_shape* sh, kvc_dtype dtype, void* k_pool, void* v_pool, int32_t block_size,
                             int32_t* block_table, int32_t max_blocks, const int32_t* kept, const int32_t* m,
                             int32_t m_max, const int32_t* cache_lens, int32_t* freed_blocks, int32_t* freed_counts,
                             void* stream) {
  if (kvc_status st = check_shape(sh)) return st;
  if (kvc_status st = check_dtype(dtype)) return st;
  if (kvc_status st = check_budgets(sh, m, m_max)) return st;
  if (kvc_status st = check_paging(sh, block_size, block_table, max_blocks, "pool")) return st;
  if (cache_lens) {
    for (int s = 0; s < sh->num_seqs; ++s) {
      const int a = seq_start(sh, s), n = sh->seq_lens[s], L = cache_lens[s];
      if (L < a + n || L > kMaxLen || ((int64_t)L + block_size - 1) / block_size > max_blocks)
        return fail(KVC_ERR_INVALID_ARGUMENT, "cache_lens[%d] = %d inconsistent with segment [%d, %d)", s, L, a,
                    a + n);
      if (a + n < L && (n % block_size || m[s] % block_size))
        return fail(KVC_ERR_INVALID_ARGUMENT,
                    "sequence %d: a segment followed by more tokens needs n (%d) and m (%d) to be multiples of %d",
                    s, n, m[s], block_size);
    }
  }
  if (!k_pool || !v_pool || !kept || !freed_blocks || !freed_counts)
    return fail(KVC_ERR_INVALID_ARGUMENT, "k_pool, v_pool, kept, freed_blocks and freed_counts must be non-NULL");
  if (k_pool == v_pool) return fail(KVC_ERR_INVALID_ARGUMENT, "k_pool and v_pool must be distinct");
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto items = [&](int s) -> int64_t { return (int64_t)sh->num_kv_heads * paged_tiles(m[s]); };
  if (kvc_status s2 = check_items(sh, items, "paged copy kernel")) return s2;
  hipError_t err = for_each_chunk(
      sh, m, items, no_offset, [&](const SeqTable& T) {
        return launch_paged_copy(dtype == KVC_F32, k_pool, v_pool, block_table, max_blocks, kept, sh->num_kv_heads,
                                 m_max, block_size, T, st);
      });
  if (err != hipSuccess) return hip_fail(err, "paged copy kernel");
  err = for_each_chunk(
      sh, m, [](int) { return 1; }, no_offset,
      [&](const SeqTable& T) { return launch_table_update(block_table, max_blocks, freed_blocks, block_size, T, st); },
      cache_lens);
  if (err != hipSuccess) return hip_fail(err, "block table kernel");
  for (int s = 0; s < sh->num_seqs; ++s)
    freed_counts[s] = (sh->seq_lens[s] + block_size - 1) / block_size - (m[s] + block_size - 1) / block_size;
  return ok();
}

}  // extern "C"
