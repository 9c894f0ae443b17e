/*
 * kvc.h -- C ABI of libkvc: proxy-query Token Eviction on AMD Instinct MI355X (gfx950).
 *
 * The library scores every cached key of every KV head with the proxy queries that attend to
 * it, keeps the top-m positions and compacts the kept K/V, either into a contiguous buffer or
 * in place inside a paged pool. Sources (titles as they appear on the pages):
 *   [TE]  "Practical Online KV Cache Compaction for LLM Agents: An Empirical Study", design-space
 *         section, Token Eviction score equation: s_j = ((1/q) sum_i alpha_ij^2)^(1/2), then keep
 *         the top-m positions with their original keys and values.
 *   [ACT] ActKV analysis page (zhichai.net), paragraph on paged memory management: attention is
 *         recovered block by block as exp(logit - LSE), the LSE being a byproduct of paged
 *         attention; eviction holes are closed by a conflict-free slot plan (tail X logical blocks
 *         are the target region, kept entries outside it are paired one-to-one with holes inside
 *         it, all pairs are copied in one parallel pass) and the emptied blocks are returned.
 *         Paragraph on the eviction policy: action-critical entries (the top 90 % of the action
 *         tokens' attention) feed an LRFU ranking with decay lambda = 0.5.
 *   [IKV] "IntentKV: Cross-Turn Intent-Aware KV Cache Pruning for Agent Inference" (gist.science),
 *         layout-preserving eviction: evicted positions are redirected to a sentinel dead slot.
 *
 * Conventions shared by every entry point
 *   unit        one (sequence s, KV head h). A "sequence" may also be one layer of a trajectory or
 *               one serving session; units never interact.
 *   R = G * q   proxy rows of a unit: the q queries of each of the G query heads h*G .. h*G+G-1
 *               that share KV head h, stacked head-major. The mean in the score runs over all R.
 *   logit       l_rj = scale * (q_r . k_j) + bias_j  (bias optional, 0 when NULL).
 *   LSE         natural log: LSE_r = ln sum_{j<n_s} exp(l_rj).
 *   score       s_j = sqrt((1/R) sum_r exp(2 (l_rj - LSE_r)))  in [0, 1] when the LSE is exact.
 *   ties        equal scores (equal float32 bit patterns) are ordered by lower position first.
 *
 * Memory: every pointer marked "device" is HIP device memory; "host" arrays are read (or, for
 * freed_counts, written) synchronously during the call. The library never allocates or frees
 * memory, keeps no pointer after returning, holds no state between calls and never
 * synchronises the stream: device work is enqueued on `stream` (a hipStream_t, NULL = the
 * default stream) and runs asynchronously. All functions are thread-safe. One exception:
 * kvc_score_noalloc keeps its scratch in a static device array per GPU (below), whose address
 * the library looks up once per device and keeps; calls of it that overlap on one GPU race.
 *
 * Errors: arguments are validated before anything is enqueued; on an error nothing is launched
 * and no output is touched. Inputs must be finite (unchecked). kvc_last_error() returns a
 * thread-local description of the last failure.
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARGUMENT = 1,   /* a pointer, size or layout is inconsistent            */
  KVC_ERR_UNSUPPORTED = 2,        /* a valid request this build does not implement        */
  KVC_ERR_WORKSPACE_TOO_SMALL = 3,/* ws_bytes < the matching *_workspace_size()           */
  KVC_ERR_HIP = 4                 /* a kernel launch failed; see kvc_last_error()         */
} kvc_status;

typedef enum { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;

/* Problem shape (host memory).
 * The n_s scored keys of sequence s are the cache positions [start_s, start_s + n_s), where
 * start_s = seq_starts[s] (0 when seq_starts is NULL). A nonzero start scores, selects and
 * compacts one segment of a longer cache -- e.g. one agent turn, with proxy queries taken from the
 * turns that followed it ("Practical Online KV Cache Compaction for LLM Agents", delayed
 * future-turn queries). Per-key arrays (bias, scores, kept) are indexed relative to the segment. */
typedef struct {
  int32_t num_seqs;          /* S >= 1                                                         */
  int32_t num_kv_heads;      /* H >= 1                                                         */
  int32_t group;             /* G >= 1 query heads per KV head                                 */
  int32_t num_queries;       /* q >= 1 proxy queries per query head                            */
  int32_t head_dim;          /* d; this build supports 128 only (else KVC_ERR_UNSUPPORTED)     */
  int32_t n_max;             /* token stride of contiguous K/V, bias and scores;
                                start_s + n_s <= n_max for contiguous K/V, n_s <= n_max always */
  const int32_t* seq_lens;   /* host [S]: n_s >= 1 keys scored in sequence s                   */
  float scale;               /* logit scale c (1/sqrt(d) in the usual attention)               */
  const int32_t* seq_starts; /* host [S]: start_s >= 0, or NULL for all zero; paged caches
                                need start_s to be a multiple of the block size               */
  const int32_t* row_pos;    /* device [S][H*G][q] int32, or NULL: a causal mask on the proxy
                                rows. Row r of unit (s, h) then sees only the keys j <= row_pos
                                (j counted from the segment start, like the per-key arrays):
                                its softmax, LSE and weights run over those keys alone, a row
                                with row_pos < 0 sees none (LSE -inf, weights 0), and the mean
                                over rows still divides by all R = G * q rows. This is how the
                                in-trajectory action tokens of "ActKV" weigh the cache: each
                                attends only to what preceded it. Read by kvc_lse, kvc_score and
                                kvc_attention_mass; kvc_am_fit rejects it                    */
} kvc_shape;

/* How keys are addressed. Contiguous: data is [S][H][n_max][d]. Paged (vLLM-style pool):
 * data is [num_blocks][block_size][H][d] and cache position p of sequence s lives in physical
 * block block_table[s * max_blocks + p / block_size], slot p % block_size. Slot map
 * (layout-preserving eviction, [IKV]): data is a slot pool [num_slots][H][d] -- a paged pool is
 * one, with slot = block * B + offset -- and position p of unit (s, h) lives in slot
 * slot_map[(s * H + h) * n_max + p], row head h. A position whose slot is dead_slot has been
 * evicted without moving anything: it takes no part in any softmax (its logit is -inf, the
 * reading of the page's sentinel key as a logit mask) and its score or mass is 0. The dead
 * slot's row must hold finite values (e.g. the page's constants); a unit with no live key
 * gets LSE -inf. */
typedef struct {
  const void* data;            /* device                                                  */
  kvc_dtype dtype;             /* element type of K (and of the queries)                  */
  int32_t block_size;          /* 0 = contiguous; else B (this build: 16); ignored with a slot map */
  const int32_t* block_table;  /* device [S][max_blocks] (paged only, else NULL)          */
  int32_t max_blocks;          /* row stride of block_table; ceil((start_s + n_s) / B) <= max_blocks */
  const int32_t* slot_map;     /* device [S][H][n_max] int32 slots, or NULL (then block_size decides);
                                  start_s + n_s <= n_max                                   */
  int32_t dead_slot;           /* with slot_map: the sentinel dead slot, or -1 for none   */
} kvc_kv_view;

/* ---------------------------------------------------------------------------------------------
 * kvc_lse -- per proxy row, the log-sum-exp of its logits over the n_s keys ([ACT] LSE; the
 * normaliser of alpha in [TE]). This is what paged attention produces as a byproduct; callers
 * that have it skip this call.
 *   q       device [S][H*G][q][d], dtype of K
 *   k       key view
 *   bias    device [S][n_max] float32 additive logit bias (segment-relative), or NULL
 *   lse_out device out [S][H*G][q] float32, natural log
 *   ws      device workspace of at least kvc_lse_workspace_size(shape, k) bytes (any alignment
 *           of 256 bytes or more); its contents are scratch
 * Result is deterministic (fixed reduction order) and within ~1e-6 relative of the exact LSE.
 * ------------------------------------------------------------------------------------------- */
size_t kvc_lse_workspace_size(const kvc_shape* shape, const kvc_kv_view* k);
kvc_status kvc_lse(const kvc_shape* shape, const void* q, const kvc_kv_view* k, const float* bias,
                   float* lse_out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * kvc_score -- Token Eviction score of every key ([TE] score equation, alpha recovered from the
 * LSE as in [ACT]). The attention matrix is never materialised.
 *   lse     device [S][H*G][q] float32 natural-log LSE per proxy row, or NULL to compute it
 *           (then ws must hold kvc_score_workspace_size(shape, k, 0) bytes). A supplied LSE is
 *           used as given, e.g. one covering more keys makes the weights sum to less than 1.
 *           It must not lie more than ~5 below the exact value (the weights' squares are
 *           accumulated with a 2^100 offset and would overflow float32).
 *   scores  device out [S][H][n_max] float32, segment-relative; entries j >= n_s not written.
 * Accuracy: within 1e-3 relative of the float64 definition for every score >= 1e-30
 * (squared weights below 2^-226 are flushed to zero). Deterministic.
 * ------------------------------------------------------------------------------------------- */
size_t kvc_score_workspace_size(const kvc_shape* shape, const kvc_kv_view* k, int lse_supplied);
kvc_status kvc_score(const kvc_shape* shape, const void* q, const kvc_kv_view* k, const float* lse,
                     const float* bias, float* scores, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * kvc_score_noalloc -- kvc_score without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, results (bit for bit) and errors as kvc_score, minus ws / ws_bytes.
 * When it computes the LSE (lse == NULL) its scratch -- what kvc_score_workspace_size(shape, k, 0)
 * counts -- lives in a static device array of KVC_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on every GPU it runs on until the process ends; a larger shape is rejected with
 * KVC_ERR_UNSUPPORTED before anything is enqueued (supply the LSE, or call kvc_score with a
 * workspace). The call allocates, frees and clears no memory; nothing in the scratch needs to start
 * at zero (every byte read is first written by the same call). Every call on one GPU shares that
 * GPU's array: calls whose device work overlaps on one GPU (other streams, other threads) race,
 * so callers serialise them, e.g. on one stream. The first call on a device looks the array's
 * address up (hipGetSymbolAddress) and keeps it for the process; the device is the stream's.
 * ------------------------------------------------------------------------------------------- */
#define KVC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kvc_status kvc_score_noalloc(const kvc_shape* shape, const void* q, const kvc_kv_view* k, const float* lse,
                             const float* bias, float* scores, void* stream);

/* ---------------------------------------------------------------------------------------------
 * kvc_attention_mass -- mean attention weight of every key over the proxy rows,
 * mass_j = (1/R) sum_r exp(l_rj - LSE_r). This is the per-entry tally of the attention that the
 * action tokens pay an entry, which ActKV's retention policy thresholds ([ACT], paragraph on
 * action-critical entries). Same arguments, workspace, LSE rules and determinism as kvc_score;
 * mass sums to 1 over the n_s keys when the LSE is computed (or exact).
 *   mass    device out [S][H][n_max] float32, segment-relative; entries j >= n_s not written.
 * Accuracy: within 1e-3 relative of the float64 definition for every mass >= 1e-30 (weights
 * below 2^-126 relative to the 2^100 offset are flushed to zero).
 * ------------------------------------------------------------------------------------------- */
kvc_status kvc_attention_mass(const kvc_shape* shape, const void* q, const kvc_kv_view* k, const float* lse,
                              const float* bias, float* mass, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * kvc_select_topm -- per unit, the m_s positions with the largest scores, ties to the lower
 * position, written in ascending position order ([TE] top-m).
 *   scores  device [S][H][n_max] float32, non-negative (sign bit clear, so +0.0 and not -0.0)
 *           and finite
 *   m       host [S]: 0 <= m_s <= n_s
 *   m_max   row stride of kept, >= max m_s
 *   kept    device out [S][H][m_max] int32; entries r >= m_s are not written
 * Exact: the same float32 scores always give the same kept set.
 * ------------------------------------------------------------------------------------------- */
kvc_status kvc_select_topm(const kvc_shape* shape, const float* scores, const int32_t* m, int32_t m_max,
                           int32_t* kept, void* stream);

/* ---------------------------------------------------------------------------------------------
 * kvc_compact_contig -- order-preserving gather of the kept rows ([TE] keep the original K, V):
 * k_out[s][h][r] = k[s][h][start_s + kept[s][h][r]] for r < m_s, and the same for V, bit for bit.
 * For a segment (start_s > 0) this is the compacted segment; the caller splices it between the
 * untouched prefix and suffix.
 *   k, v          device [S][H][n_max][d] of dtype
 *   kept          device [S][H][m_max] int32, strictly ascending, < n_s (as from select)
 *   k_out, v_out  device out [S][H][m_max][d]; rows r >= m_s are not written
 * ------------------------------------------------------------------------------------------- */
kvc_status kvc_compact_contig(const kvc_shape* shape, kvc_dtype dtype, const void* k, const void* v,
                              const int32_t* kept, const int32_t* m, int32_t m_max, void* k_out,
                              void* v_out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * kvc_compact_paged -- in-place conflict-free compaction of a paged pool ([ACT] slot plan).
 * Per sequence, with a = start_s (a multiple of B), n = n_s, L = cache_lens[s] (the sequence's
 * total length; a + n when cache_lens is NULL): N = ceil(n/B), X = ceil(m_s/B), F = N - X,
 * window W = [a + F*B, a + F*B + m_s). Per head: sources = kept positions outside W, holes =
 * positions of W not kept (both ascending, all relative positions offset by a); the i-th
 * source's K and V rows are copied to the i-th hole, all pairs in one parallel pass (a source is
 * never a hole, so no slot is both read and written). Kept positions inside W stay where they
 * are, so the compacted order is not the original order. Afterwards, with b = a/B and
 * NT = ceil(L/B) table entries in use:
 *   freed_blocks[s][0..F)      = old block_table[s][b..b+F) (logical order); rest untouched
 *   block_table[s][b..NT-F)    = old block_table[s][b+F..NT)  (the window, then any later blocks)
 *   block_table[s][NT-F..NT)   = -1; entries outside [b, NT) untouched
 *   freed_counts[s] (host, written during the call) = F = ceil(n/B) - ceil(m_s/B)
 * The sequence's new length is a + m_s if the segment ends it (a + n = L), else L - F*B.
 * Positions after the segment keep their bytes and only
 * change block-table entries, which is why a segment followed by more tokens (a + n < L) must
 * have n and m_s multiples of B (otherwise the window's last block would hold a hole).
 * Source slots keep their bytes (copy, not move).
 *   k_pool, v_pool  device [num_blocks][B][H][d] of dtype, modified in place (distinct buffers)
 *   block_table     device in/out [S][max_blocks] int32 (valid, distinct ids for p < L)
 *   kept            device [S][H][m_max] int32, strictly ascending, < n_s (segment-relative)
 *   m               host [S]
 *   cache_lens      host [S] total length L >= start_s + n_s of each sequence, or NULL
 * ------------------------------------------------------------------------------------------- */
kvc_status kvc_compact_paged(const kvc_shape* shape, kvc_dtype dtype, void* k_pool, void* v_pool,
                             int32_t block_size, int32_t* block_table, int32_t max_blocks,
                             const int32_t* kept, const int32_t* m, int32_t m_max,
                             const int32_t* cache_lens, int32_t* freed_blocks, int32_t* freed_counts,
                             void* stream);

/* ---------------------------------------------------------------------------------------------
 * kvc_evict_redirect -- layout-preserving eviction ([IKV], IntentKV page, layout-preserving
 * eviction: an evicted position's slot-map entry is redirected to a reserved sentinel dead slot
 * instead of compacting). For every unit and every scored position j < n_s that is not in
 * kept[s][h][0..m_s):  slot_map[(s * H + h) * n_max + start_s + j] = dead_slot. Kept positions,
 * positions outside the segment and every K/V row stay where they are, so prefix identity and
 * RoPE phases are preserved; scoring through the map (kvc_kv_view.slot_map) then masks them.
 *   kept       device [S][H][m_max] int32, strictly ascending, < n_s (as from select)
 *   m          host [S]; m_max >= max m_s
 *   slot_map   device in/out [S][H][n_max] int32
 *   dead_slot  >= 0
 * ------------------------------------------------------------------------------------------- */
kvc_status kvc_evict_redirect(const kvc_shape* shape, const int32_t* kept, const int32_t* m, int32_t m_max,
                              int32_t* slot_map, int32_t dead_slot, void* stream);

/* ---------------------------------------------------------------------------------------------
 * kvc_am_fit -- Attention Matching on top of a Token Eviction selection ([TE], design-space
 * section, the AM equations): for the kept keys K_C of every unit, an additive logit bias beta
 * with  min || exp(Q K_C^T + beta) 1_m - exp(Q K^T) 1_n ||^2  and compact values V_C with
 * min || softmax(Q K_C^T + beta) V_C - softmax(Q K^T) V ||_F^2  (logits carry `scale`, no bias).
 * The pages name no optimiser; this library uses, with w = exp(beta):
 *   beta: iters_beta multiplicative non-negative least-squares updates
 *         w <- w * (E^T z) / (E^T E w) from w = 1 (beta = 0, plain eviction), where
 *         E_ij = exp(l_ij) over the kept keys and z_i = exp(LSE_i); internally both carry
 *         their own constant factor (E its largest kept logit, z its largest LSE, moved to within
 *         80 of the former) so float32 holds them -- the updates are scale-equivariant, so the
 *         iterates are unchanged; w_j = 0 gives beta_j = -inf;
 *   V_C:  iters_v Landweber steps V <- V - eta P^T (P V - Y) from the kept keys' stored values,
 *         P = the compacted attention softmax(Q K_C^T + beta), Y = softmax(Q K^T) V, and
 *         eta = 1 / max_j sum_i P_ij (stable: eta ||P||_2^2 <= 1).
 * Arithmetic on the GPU: the QK^T products on bf16 MFMA with float32 accumulation; every other
 * quantity float32, with the two matrix products of the value fit (and P V of the target) taken as
 * bf16 MFMA products of float32 operands split into two bf16 halves each (hi = bf16(x),
 * lo = bf16(x - hi); hi hi + hi lo + lo hi, relative error near 2^-16 per product).
 *   q          device [S][H*G][q][d] bf16;  G * q >= 16 (else KVC_ERR_UNSUPPORTED)
 *   k, v       key and value views, bf16, both contiguous or both paged (no slot maps)
 *   lse        device [S][H*G][q] LSE over the n_s keys, or NULL to compute it (in ws)
 *   kept       device [S][H][m_max] int32, strictly ascending, < n_s (as from select)
 *   m, m_max   host budgets [S] and the row stride of kept / beta / v_c
 *   beta       device out [S][H][m_max] float32 (natural-log bias per kept key)
 *   v_c        device out [S][H][m_max][d] float32
 *   ws         device workspace of kvc_am_workspace_size(shape, k, v, m, lse != NULL) bytes:
 *              at most about 4 * H * (R * (2 m_s + 10 d) + 9 m_s d) bytes per sequence (the kept
 *              exponentials and their transpose are materialised, plus up to 8 split partial
 *              sums of each value product; the attention over all n_s keys is not stored)
 * ------------------------------------------------------------------------------------------- */
size_t kvc_am_workspace_size(const kvc_shape* shape, const kvc_kv_view* k, const kvc_kv_view* v, const int32_t* m,
                             int lse_supplied);
kvc_status kvc_am_fit(const kvc_shape* shape, const void* q, const kvc_kv_view* k, const kvc_kv_view* v,
                      const float* lse, const int32_t* kept, const int32_t* m, int32_t m_max, int32_t iters_beta,
                      int32_t iters_v, float* beta, float* v_c, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * kvc_lrfu_update -- one step of ActKV's retention state ([ACT], paragraph on action-critical
 * entries: the attention of all action tokens on each entry is tallied, entries within the top
 * 90 % are action-critical, and LRFU -- with "hit by action attention" as its hit signal and a
 * decay of lambda = 0.5 -- ranks the entries). Per unit:
 *   critical set  the shortest run of entries in descending mass order (ties to the lower
 *                 position) whose integer masses u_j = min(floor(mass_j * 2^32), 2^40) add up to
 *                 at least ceil(top_p * U), U = sum_j u_j computed exactly (empty when U = 0);
 *   state_j       = fmaf(decay, state_j, critical ? 1 : 0) for every j < n_s.
 * Exact: the same float32 masses always give the same critical set, whatever the summation order.
 *   mass    device [S][H][n_max] float32, non-negative (e.g. from kvc_attention_mass),
 *           segment-relative
 *   top_p   in (0, 1] (0.9 for ActKV); decay in [0, 1] (2^-lambda per step; 2^-0.5 for ActKV)
 *   state   device in/out [S][H][n_max] float32, segment-relative; entries j >= n_s untouched
 *   counts  device out [S][H] int32, the size of each unit's critical set, or NULL
 * Retention then keeps the m_s entries with the largest state: kvc_select_topm(state), the
 * compaction of K/V, and kvc_compact_side to carry the state along.
 * ------------------------------------------------------------------------------------------- */
kvc_status kvc_lrfu_update(const kvc_shape* shape, const float* mass, double top_p, float decay, float* state,
                           int32_t* counts, void* stream);

/* ---------------------------------------------------------------------------------------------
 * kvc_compact_side -- carries a per-entry float32 side array (such as the LRFU state) through a
 * compaction, so that it stays aligned with the compacted K/V:
 *   dst[s][h][p] = src[s][h][start_s + old(p)] for p < m_s,
 * where old(p) = kept[p] for contiguous compaction (block_size = 0) and, for the paged slot plan
 * of kvc_compact_paged with block size B (block_size = B), the position whose K/V occupies window
 * slot p afterwards: a kept position inside the window stays, a hole receives its paired source.
 *   kept    device [S][H][m_max] int32, strictly ascending, < n_s (as from select)
 *   m       host [S]; m_max >= max m_s
 *   src     device [S][H][n_max] float32; dst device out [S][H][m_max] float32 (distinct from src;
 *           rows p >= m_s not written)
 * ------------------------------------------------------------------------------------------- */
kvc_status kvc_compact_side(const kvc_shape* shape, int32_t block_size, const int32_t* kept, const int32_t* m,
                            int32_t m_max, const float* src, float* dst, void* stream);

/* Static text for a status code; never NULL. */
const char* kvc_status_string(kvc_status status);
/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* kvc_last_error(void);
/* Library version as an integer (major * 10000 + minor * 100 + patch). */
int kvc_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H_ */
