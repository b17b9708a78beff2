/*
 * hs_attn.h - C ABI of the MI355X (gfx950) query-guided block-sparse decode
 * attention library `libhs_attn.so`.
 *
 * The library computes one decode step of hierarchical sparse attention in
 * three stages, each an entry point below:
 *
 *   hs_build_summaries  per-block key summaries (mean-pooled keys, or the
 *                       per-dimension key min/max "bounding box")
 *   hs_select_blocks    score every block against the current query, keep a
 *                       top-k (one or two levels) and always add the blocks of
 *                       the local window
 *   hs_sparse_decode    exact softmax attention over the selected blocks only,
 *                       read in place from a paged KV cache
 *
 * hs_select_decode runs the last two stages for one layer in a single launch
 * (same results as hs_select_blocks followed by hs_sparse_decode), and
 * hs_decode_step all three as one decode step: the refresh of the trailing
 * summary blocks, the selection and the attention.
 *
 * Sources (web pages; cited by title and section):
 *   [QSA]     "8x256K long-context sparse attention: porting HiSparse to QSA"
 *             (xxmr.cn), sections 2.2 (three-level coarse/fine/window
 *             selection), 2.3 (sparsify on block boundaries), 3.1 (C config
 *             struct instead of a Python dict), 3.2 (selection on the GPU),
 *             3.3 (attention loop over a compact index list), 5.1 (fp32
 *             block scores).
 *   [HiSp]    untitled HiSparse project write-up (trdm.cn), sections 3.1
 *             (per-block table resident in HBM), 3.2 (64-token block slots),
 *             3.3 (decode loop: force the window, then top-K), 4.1
 *             (write/read-top-k wrapper).
 *   [SGL]     "SGLang hierarchical sparse attention: analysis and practice"
 *             (intelliparadigm.com), sections 2.2 (representation phase,
 *             query-guided decode phase, logical->physical page table) and
 *             3.1.2 (Quest: per-block key bounding boxes).
 *   [SparDA]  SparDA article (2kiu.com), sections 2.3 (64-token blocks),
 *             3.1 (mean-pooled block representatives), 3.3 (the kernel walks
 *             only the selected pages), 3.4 (one selection shared by all
 *             later layers and reused while decoding).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers on the current HIP device; the
 *     caller allocates and owns every buffer. The library allocates nothing,
 *     keeps no host state between calls and is reentrant: two calls may run
 *     at the same time if they do not share output or workspace buffers
 *     (hs_select_decode and hs_decode_step then report an expired wait in
 *     their status word if the other call kept part of their launch from
 *     running; see there).
 *   - Struct arguments are read only during the call.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t, passed as
 *     void*; NULL = the default stream). Outputs are valid once the stream
 *     reaches that point.
 *   - Every argument is validated on the host BEFORE any HIP call; an invalid
 *     call returns an error code and enqueues nothing. A failed kernel launch
 *     returns HS_ERR_HIP. No C++ exception crosses this boundary.
 *   - Device-side values that the host cannot see (seq_lens, page-table
 *     entries, block ids, counts) are range-checked in the kernels: a sequence
 *     length is clamped to [0, max_seq_len]; a page-table entry outside
 *     [0, num_phys_pages) is never dereferenced: the attention, the token
 *     selection and the summaries leave its tokens out (a summary row of a
 *     block with such tokens is then unspecified, as is a mean over none);
 *     a block id outside [0, ceil(T_b / block_size)) is skipped; a count is
 *     clamped to [0, max_selected]. No such value can make a kernel read or
 *     write out of bounds.
 *   - Indexing: B = batch, Hkv = num_kv_heads, Hq = num_q_heads,
 *     G = Hq / Hkv (query head h uses KV head h / G), d = head_dim,
 *     P = page_size, S = block size of a summary level, T_b = seq_lens[b].
 *     A "unit" is one (b, kv-head) pair; units are independent.
 */
#ifndef HS_ATTN_H
#define HS_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HS_ATTN_VERSION 4

/* Most dynamic LDS that hs_select_tokens uses above its register path (a
 * bitmap of max_seq_len bits and the staged id list); with the kernel's own
 * static LDS it stays within one gfx950 workgroup's 160 KiB. */
#define HS_TOKEN_LDS_BYTES (120 << 10)

/* Value of the status word of a fused-step workspace (hs_step_status) after
 * a call in which a workgroup's bounded wait for another expired. */
#define HS_STEP_WAIT_EXPIRED 1

typedef enum {
  HS_OK = 0,
  HS_ERR_INVALID_ARG = 1, /* null pointer, bad shape, inconsistent sizes     */
  HS_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, group size, dtype */
  HS_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required       */
  HS_ERR_HIP = 4          /* a HIP launch failed                              */
} hs_status;

typedef enum { HS_F32 = 0, HS_BF16 = 1 } hs_dtype;

typedef enum {
  HS_SUMMARY_MEAN = 0,   /* mean-pooled keys [SparDA 3.1], [QSA 2.2]          */
  HS_SUMMARY_MINMAX = 1  /* per-dimension key min and max [SGL 3.1.2]          */
} hs_summary_kind;

/* Paged KV cache of ONE layer ([SGL 2.2]: logical block -> physical page
 * through a page table; [HiSp 3.2]: fixed-size token slots, contiguous inside
 * a slot).
 *   k_pool, v_pool : dtype[num_phys_pages][num_kv_heads][page_size][head_dim]
 *                    token t of sequence b, KV head g lives in physical page
 *                    page_table[b][t / P] at row (g, t % P).
 *   page_table     : int32[batch][max_pages], logical page -> physical page.
 *   seq_lens       : int32[batch], T_b, on the device.
 *   max_seq_len    : host-side upper bound of every T_b (sizes the grids);
 *                    must be <= max_pages * page_size.
 * Supported: head_dim in {64, 128}; dtype HS_F32 or HS_BF16. */
typedef struct {
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages;
  int32_t num_phys_pages;
  int32_t max_seq_len;
  int32_t dtype; /* hs_dtype */
} hs_kv_cache;

/* One level of block summaries, caller-allocated ([HiSp 3.1]: a small per-
 * block table resident in HBM; [SGL 2.2]: key statistics kept on the GPU).
 *   kind MEAN   : float32[batch][num_kv_heads][max_blocks][head_dim]
 *                 row beta = mean of k_t over the valid tokens of block beta
 *                 (fp32; [SparDA 3.1] mean pooling).
 *   kind MINMAX : dtype[batch][num_kv_heads][max_blocks][2][head_dim]
 *                 [..][0][i] = min_t k_t,i and [..][1][i] = max_t k_t,i over
 *                 the valid tokens of block beta, in the KV dtype (exact).
 *   block_size  : S (tokens per block), >= 1.
 *   max_blocks  : rows per unit, >= ceil(max_seq_len / S) and <= 32768.
 * Rows at or beyond ceil(T_b / S) are left untouched by the build and never
 * read by the selection. */
typedef struct {
  void* data;
  int32_t kind;       /* hs_summary_kind */
  int32_t block_size;
  int32_t max_blocks;
} hs_summaries;

/* Selection parameters ([QSA 3.1]: a plain C struct instead of a per-request
 * dictionary).
 *   num_q_heads   : Hq; G = Hq / Hkv in {1, 2, 4, 8}. The block score of a
 *                   unit is the SUM of the scores of its G query heads.
 *   top_k         : k of the fine level ([QSA 2.2], [HiSp 3.3]); 0 = none.
 *   window_tokens : W. Blocks holding any of tokens [T_b - W, T_b) are always
 *                   selected ([QSA 2.2] window level, [HiSp 3.3] step one).
 *   top_k_coarse  : 0 = single level. Otherwise the two-level scheme of
 *                   [QSA 2.2]: top_k_coarse blocks of the `coarse` table, then
 *                   top_k fine blocks among the fine blocks inside them.
 *   max_selected  : row capacity of block_ids. Must be >= the largest possible
 *                   count: min(max_blocks, min(K, max_blocks) + ceil(W / S)
 *                   + 1 + forced_cap), K = top_k, or with a ratio the k of
 *                   max_blocks blocks.
 *   top_k_ratio   : 0 = use top_k. In (0, 1]: the fine level keeps
 *                   k_b = max(1, int(nb_b * top_k_ratio)) blocks of unit b,
 *                   nb_b = ceil(T_b / S), computed on the device per unit
 *                   ([SparDA 3.2] fixed-ratio top-k and its length-dependent
 *                   ratio; [SparDA 3.4] k = max(1, int(n * ratio))).
 *   forced_ids    : NULL, or int32[batch][Hkv][forced_cap] block ids unioned
 *                   into every unit's selection ([SparDA 3.4] the reserve set
 *                   of 1-2 % random blocks kept besides the scored top-k; the
 *                   caller draws them). Entries outside [0, nb_b) (e.g. -1
 *                   padding) are ignored; duplicates count once. */
typedef struct {
  int32_t num_q_heads;
  int32_t top_k;
  int32_t window_tokens;
  int32_t top_k_coarse;
  int32_t max_selected;
  float top_k_ratio;
  const int32_t* forced_ids;
  int32_t forced_cap;
} hs_select_params;

/* Workspace sizes (bytes) for hs_select_blocks / hs_sparse_decode. Pure host
 * functions: they validate like the matching entry point and write *bytes.
 * `coarse` may be NULL for single-level selection. */
hs_status hs_select_workspace_size(const hs_select_params* p,
                                   const hs_kv_cache* kv,
                                   const hs_summaries* fine,
                                   const hs_summaries* coarse, size_t* bytes);
hs_status hs_decode_workspace_size(const hs_kv_cache* kv, int32_t num_q_heads,
                                   int32_t block_size, int32_t max_selected,
                                   size_t* bytes);

/* Stage 1 - block summaries ([SGL 2.2] representation phase; [SGL 3.1.2]
 * bounding boxes; [SparDA 3.1] / [QSA 2.2] mean pooling).
 * Rebuilds, for every unit (b, g), rows beta in [block_begin, ceil(T_b / S))
 * of `out` from the keys of k_pool. block_begin = 0 builds everything (after
 * prefill); block_begin = ceil(T_b / S) - 1 refreshes only the last, growing
 * block after a decode-time append. A partial last block is summarised over
 * its valid tokens only. Only k_pool of `kv` is read (v_pool may be NULL). */
hs_status hs_build_summaries(const hs_kv_cache* kv, int32_t block_begin,
                             const hs_summaries* out, void* stream);

/* Decode-time append ([SGL 2.2] each decode step writes the new token's K/V
 * into the paged cache through the page table; [HiSp 3.1] the per-block
 * table is then updated: refresh the growing block with hs_build_summaries
 * or hs_decode_step, block_begin = ceil(T_b / S) - 1 with the new T_b).
 * For every sequence b, t = seq_lens[b] is read on the device; if
 * 0 <= t < kv->max_seq_len and page_table[b][t / P] is a valid page id, the
 * rows k_new[b][g][:] and v_new[b][g][:] of every KV head g are written to
 * slot t % P of that page of k_pool and v_pool, and seq_lens[b] becomes
 * t + 1. A sequence at capacity (or with an invalid page id) is left
 * unchanged: nothing is written and its length is not advanced, which the
 * caller can see by reading seq_lens.
 *   k_new, v_new : dtype[batch][Hkv][head_dim], 16-byte aligned.
 *   seq_lens     : must be kv->seq_lens (the one array that is advanced).
 * Requires both pools. Later calls on the same stream see the new rows and
 * lengths. */
hs_status hs_append_kv(const hs_kv_cache* kv, const void* k_new, const void* v_new,
                       int32_t* seq_lens, void* stream);

/* Token-level second stage inside the selected blocks ([SparDA 2.3]: after
 * the block selection, a finer pass keeps single tokens inside the chosen
 * blocks, for very high compression). For every unit, the candidates are the
 * tokens t < T_b of its selected blocks (block_ids / num_selected as written
 * by hs_select_blocks with block size `block_size`: ascending and distinct;
 * for other lists the output is in list order and ties are broken by list
 * position, but every access stays in bounds). Token score, fp32,
 * unscaled: sum over the unit's G query heads of q_j . k_t (the block score
 * of a one-token block). Kept, ascending, without duplicates: the first
 * min(top_k_tokens, #candidates) candidates by (score descending, token
 * ascending), plus every token of the window [T_b - window_tokens, T_b).
 *   token_ids  : int32[batch][Hkv][max_tokens] (entries past the count left
 *                untouched); num_tokens : int32[batch][Hkv].
 *   max_tokens : >= min(max_selected * block_size, top_k_tokens) +
 *                min(window_tokens, max_seq_len).
 * Attention over the kept tokens is hs_sparse_decode with block_size 1 and
 * token_ids / num_tokens / max_tokens as its ids.
 * workspace: at least hs_select_tokens_workspace_size() bytes, 16-byte
 *   aligned and ZERO-FILLED before its first use; every call leaves its
 *   counters at zero. Requires k_pool. One launch on the stream. Up to 8192
 *   candidate slots (max_selected * block_size) and 512 selected blocks the
 *   selection keeps its state in registers and needs no per-sequence LDS.
 *   Above that it marks
 *   kept tokens in an LDS bitmap of max_seq_len bits next to the staged id
 *   list (max_tokens + 64 entries); HS_ERR_UNSUPPORTED when those would
 *   exceed HS_TOKEN_LDS_BYTES. */
hs_status hs_select_tokens_workspace_size(const hs_kv_cache* kv, int32_t num_q_heads,
                                          int32_t block_size, int32_t max_selected,
                                          int32_t top_k_tokens, int32_t window_tokens,
                                          int32_t max_tokens, size_t* bytes);
hs_status hs_select_tokens(const hs_kv_cache* kv, const void* q, int32_t num_q_heads,
                           int32_t block_size, const int32_t* block_ids,
                           const int32_t* num_selected, int32_t max_selected,
                           int32_t top_k_tokens, int32_t window_tokens, int32_t* token_ids,
                           int32_t* num_tokens, int32_t max_tokens, void* workspace,
                           size_t workspace_bytes, void* stream);

/* LRU cache of selected blocks and the step difference ([SGL 3.2] sparse
 * diff kernel: consecutive steps select largely the same blocks; a cache pool
 * a few times the top-k is kept least-recently-used; each step takes the
 * difference from the previous selection, finds the cached blocks, loads the
 * misses and updates the cache index). With the whole cache in HBM this is
 * the index alone: which block each slot holds, and which selected blocks a
 * host tier would have to load.
 * Per unit, `capacity` slots hold a block id (-1 = empty) and the step at
 * which that block was last selected (-1 for empty slots); the caller starts
 * from all -1 (e.g. a 0xFF fill) and passes increasing steps.
 * One call = one step `step` for every unit, with this step's selection
 * (block_ids / num_selected as written by hs_select_blocks, ids ascending):
 *   - a selected block found in a slot is a hit; its stamp becomes `step`;
 *   - the misses, in ascending block order, take the slots not hit at this
 *     step in order of (stamp ascending, slot index ascending): empty slots
 *     first, then the least recently used; they get stamp `step`;
 *   slot_of     : int32[units][max_selected], the slot of each selected block;
 *   miss_blocks : int32[units][max_selected], the missed blocks, ascending
 *                 (the loads of a host tier); entries past the misses are
 *                 left untouched;
 *   stats       : int32[units][3] = hits, misses, |S_t minus S_(t-1)| (the
 *                 selected blocks whose slot did not carry stamp step - 1;
 *                 the set difference from the previous call's selection when
 *                 capacity >= 2 * max_selected, as with the pages' 2-4 x
 *                 top-k pool).
 * Requires max_selected <= capacity <= 1024, max_selected <= 2048, units in
 * [1, 65535], 0 <= step < INT32_MAX. Calls that share a cache must not
 * overlap. */
typedef struct {
  int32_t* slot_block;  /* [units][capacity] */
  int32_t* slot_stamp;  /* [units][capacity] */
  int32_t capacity;
} hs_block_cache;

hs_status hs_block_cache_update(const hs_block_cache* cache, int32_t units, int32_t step,
                                const int32_t* block_ids, const int32_t* num_selected,
                                int32_t max_selected, int32_t* slot_of, int32_t* miss_blocks,
                                int32_t* stats, void* stream);

/* Stage 2 - query-guided block selection ([SGL 2.2] decode phase step a;
 * [QSA 2.2] three-level scheme; [QSA 3.2] selection on the GPU; [QSA 5.1]
 * fp32 scores).
 *   q            : dtype[batch][Hq][head_dim], same dtype as the cache.
 *   fine         : summaries of the fine level (block size S).
 *   coarse       : NULL, or the coarse level (MEAN or MINMAX, block size C,
 *                  C % S == 0) when p->top_k_coarse > 0.
 * Score of block beta for unit (b, g), accumulated in fp32, unscaled:
 *   MEAN   : s = sum_{j<G} q_j . mu_beta
 *   MINMAX : s = sum_{j<G} sum_i max(q_j,i * m_beta,i, q_j,i * M_beta,i)
 *            (the largest value q_j . k can take inside the box).
 * Top-k orders candidates by score descending, then block index ascending,
 * and keeps the first min(k, #candidates). Two-level: the candidates of the
 * fine level are the fine blocks inside the top_k_coarse coarse blocks.
 * Output per unit: the union of the top-k and the window blocks, sorted
 * ascending, without duplicates:
 *   block_ids    : int32[batch][Hkv][max_selected] (entries past the count
 *                  are left untouched)
 *   num_selected : int32[batch][Hkv]
 * Only shapes and seq_lens of `kv` are used (pools may be NULL).
 * workspace: device buffer of at least hs_select_workspace_size() bytes,
 *   16-byte aligned and ZERO-FILLED before its first use. It starts with
 *   per-unit arrival counters (the last workgroup of a unit to finish scoring
 *   runs that unit's top-k); every call returns them to zero, so a workspace
 *   can be reused by later calls on the same stream but must not be shared by
 *   calls that may run at the same time. */
hs_status hs_select_blocks(const hs_select_params* p, const hs_kv_cache* kv,
                           const void* q, const hs_summaries* fine,
                           const hs_summaries* coarse, int32_t* block_ids,
                           int32_t* num_selected, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Stage 3 - sparse paged decode attention ([QSA 3.3] loop over a compact
 * index list of selected blocks; [SparDA 3.3] only the selected pages are
 * read; [QSA 2.3] no gather into a compact copy).
 * For query head h of unit (b, g = h / G), with A the tokens t < T_b of the
 * blocks block_ids[b][g][0 .. num_selected[b][g]):
 *   out[b][h] = sum_{t in A} exp(l_t - m) v_t / sum_{t in A} exp(l_t - m),
 *   l_t = scale * q_h . k_t,  m = max_{t in A} l_t,
 * fp32 softmax and accumulation. If A is empty, out[b][h] = 0.
 *   q            : dtype[batch][Hq][head_dim]
 *   scale        : logit scale; 0 means 1 / sqrt(head_dim)
 *   block_size   : S of the ids (any S >= 1; need not equal page_size).
 *                  S = 1: the ids are single tokens (e.g. the token_ids of
 *                  hs_select_tokens), each looked up through the page table.
 *   out          : float32[batch][Hq][head_dim]
 * The same block_ids may be passed to the decode of every layer (shared
 * selection, [SparDA 3.4]); they are only read. Ids outside
 * [0, ceil(T_b / S)) are skipped. Ids of one unit must be distinct
 * (hs_select_blocks guarantees it); an id listed twice is attended twice.
 * A unit's list is cut into n split tasks (n = ceil(256 / units), or
 * ceil(512 / units) when max_selected * S >= 2048 * ceil(256 / units); then
 * at most max_selected and 128), each holding ceil(max_selected / n) entries
 * in LDS, 4 bytes each (8 for S = 1 on a bf16 cache), at most 96 KiB:
 * larger lists return HS_ERR_INVALID_ARG (here and from
 * hs_decode_workspace_size).
 * workspace: device buffer of at least hs_decode_workspace_size() bytes,
 *   16-byte aligned and ZERO-FILLED before its first use. It starts with
 *   per-unit arrival counters (the last split of a unit to finish merges the
 *   unit's partial results); every call returns them to zero, so a workspace
 *   can be reused by later calls on the same stream but must not be shared by
 *   calls that may run at the same time. */
hs_status hs_sparse_decode(const hs_kv_cache* kv, const void* q,
                           int32_t num_q_heads, float scale,
                           int32_t block_size, const int32_t* block_ids,
                           const int32_t* num_selected, int32_t max_selected,
                           float* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Stages 2 and 3 of one layer in one launch: the selection of
 * hs_select_blocks and the attention of hs_sparse_decode over the ids it
 * selects ([QSA 3.2] selection on the GPU, then [QSA 3.3] the attention loop
 * over the compact index list; [SGL 2.2] decode phase, steps a and b).
 * Arguments mean what they mean for those two calls; the decode uses
 * fine->block_size and p->max_selected. block_ids and num_selected are
 * written as by hs_select_blocks, out as by hs_sparse_decode, and the results
 * are bitwise identical to the two calls on the same inputs. A two-level
 * selection launches its coarse level first, then one fused launch; id lists
 * too long for the fused kernel's LDS, and a fine block size of 1, run as the
 * separate launches instead (same results).
 * Inside the launch, a unit's attention starts as soon as that unit's
 * selection is done, while other units are still being scored.
 * The launch is a persistent grid sized to what the GPU holds at once, and a
 * unit's attention tasks wait for that unit's scoring tasks, which run on
 * other workgroups of the grid. Those waits end when the whole grid is
 * resident, as it is when the call has the GPU to itself. When another
 * kernel (or another fused call) holds part of the GPU at the same time, a
 * scoring task can be held back until then; every wait is therefore bounded
 * by wall-clock time (a quarter of a second). If one expires, the call's
 * outputs are not valid and the workspace's status word is set to
 * HS_STEP_WAIT_EXPIRED (read it with hs_step_status): callers that run other
 * kernels concurrently with this one should check it, or use
 * hs_select_blocks and hs_sparse_decode, which never wait. A workspace that
 * was not zero-filled, or that overlapping calls share, also sets it.
 * workspace: device buffer of at least hs_select_decode_workspace_size()
 *   bytes, 16-byte aligned and ZERO-FILLED before its first use; it holds a
 *   256-byte control line (status word at byte 0), then the workspace of the
 *   selection (from byte 256; the last selection level's per-unit arrival
 *   counters first, one int32 per 256 bytes), then that of the attention.
 *   Every call returns its counters to zero, so it can be reused by later
 *   calls on the same stream but must not be shared by calls that may run at
 *   the same time. The status word is only ever set, never cleared, by the
 *   library. */
hs_status hs_select_decode_workspace_size(const hs_select_params* p,
                                          const hs_kv_cache* kv,
                                          const hs_summaries* fine,
                                          const hs_summaries* coarse,
                                          size_t* bytes);
hs_status hs_select_decode(const hs_select_params* p, const hs_kv_cache* kv,
                           const void* q, const hs_summaries* fine,
                           const hs_summaries* coarse, float scale,
                           int32_t* block_ids, int32_t* num_selected,
                           float* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* One decode step of one layer ([SGL 2.2] decode phase after a token is
 * appended; [HiSp 3.1] the per-block table is updated as the cache is
 * written; [QSA 3.2], [QSA 3.3]): the summary blocks
 * [refresh_begin, ceil(T_b / S)) of `fine` (and, with two levels, the
 * coarse blocks from refresh_begin * S / C on) are rebuilt from the K cache
 * as hs_build_summaries would, then the selection and the attention of
 * hs_select_decode run on the refreshed tables. Results (the tables, ids,
 * counts and outputs) are bitwise identical to hs_build_summaries on each
 * table followed by hs_select_decode.
 *   refresh_begin : >= 0; ceil(T_b / S) - 1 refreshes only the growing last
 *                   block; a value at or past every unit's block count
 *                   refreshes nothing. Negative values are rejected.
 * Requires kv->k_pool. The workspace is that of hs_select_decode
 * (hs_select_decode_workspace_size), with the same rules. */
hs_status hs_decode_step(const hs_select_params* p, const hs_kv_cache* kv,
                         const void* q, const hs_summaries* fine,
                         const hs_summaries* coarse, int32_t refresh_begin,
                         float scale, int32_t* block_ids,
                         int32_t* num_selected, float* out, void* workspace,
                         size_t workspace_bytes, void* stream);

/* hs_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Arguments, results and their bitwise
 * equality with hs_build_summaries + hs_select_decode are those of
 * hs_decode_step. The workspace is a device array of the library,
 * HS_NOALLOC_SCRATCH_BYTES long, that each GPU the library runs on holds
 * until the process ends; its device address is looked up on the first call
 * on each device (HIP's symbol lookup, no allocation). Each call first
 * zeroes the array's control line and arrival counters with a small kernel
 * on `stream`, then runs the step. Calls on one GPU share the array: calls
 * that overlap on one GPU (several streams, or threads) race and give wrong
 * results. The status word of an expired wait (see hs_decode_step) is not
 * readable for this variant; use it when the call has the GPU to itself.
 * Returns HS_ERR_WORKSPACE, before any HIP call, when the step's workspace
 * (hs_select_decode_workspace_size) would exceed HS_NOALLOC_SCRATCH_BYTES.
 * Calls no hipMalloc, hipFree or other allocating routine. */
#define HS_NOALLOC_SCRATCH_BYTES (16 << 20)
hs_status hs_decode_step_noalloc(const hs_select_params* p, const hs_kv_cache* kv,
                                 const void* q, const hs_summaries* fine,
                                 const hs_summaries* coarse, int32_t refresh_begin, float scale,
                                 int32_t* block_ids, int32_t* num_selected, float* out,
                                 void* stream);

/* Reads the status word of a workspace of hs_select_decode / hs_decode_step
 * into *status (0, or HS_STEP_WAIT_EXPIRED once a call on the workspace had
 * an expired wait; it stays set until the caller zero-fills the workspace
 * again). Waits for `stream` to reach this point (a device-to-host copy of
 * 4 bytes on it, then a stream synchronisation), so it is meant for checks
 * and tests rather than for every step. workspace_bytes must be >= 4. */
hs_status hs_step_status(const void* workspace, size_t workspace_bytes, int32_t* status,
                         void* stream);

/* Static, NUL-terminated name of a status code. */
const char* hs_status_string(hs_status s);

/* HS_ATTN_VERSION of the built library. */
int32_t hs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HS_ATTN_H */
