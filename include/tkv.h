/*
 * tkv.h -- C ABI of the tiered KV-cache sparse decode library (gfx950).
 *
 * The method (FreeToken PR #499, "feat(kvcache): host-RAM KV tier for
 * sparse-attention models", sections "What", "Why this works for sparse
 * attention" and "Design"): the full KV cache lives in a pinned host mirror
 * (the backing store); the GPU pool is an LRU cache of physical slots over
 * the logical page space.  Each attention step first runs the indexer (top-k
 * page selection over a compressed key slab kept on the GPU), compacts the
 * selection (cap max_sel_pages = 2*block_topk + 8, with a drop counter),
 * makes the selected pages resident with a device-side LRU, copies the missed
 * pages host->device in one fused copy that moves K+V (codes and scales) of a
 * page for every layer, translates logical page ids to slots, and runs sparse
 * paged attention over the selected pages only.  Every store of new K/V is
 * quantised and written through to the mirror, so eviction is a pure rebind.
 *
 * Conventions
 *  - All device pointers are caller-owned device memory.  The library
 *    allocates no device memory, except for a staging buffer that
 *    tkv_prefix_save and tkv_prefix_restore allocate and free within the
 *    call.  The pinned host mirror is owned by the ctx.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    calls except tkv_create/tkv_attach_device/tkv_read_counters/
 *    tkv_debug_read_state and the cold-prefix calls (tkv_prefix_save/
 *    tkv_prefix_restore: host-side copies, a staging buffer) are
 *    asynchronous, launch a fixed number of kernels whose shapes depend only
 *    on the arguments' sizes, never synchronise and never allocate, so they
 *    can be captured in a HIP graph (tkv_decode_layer_split: see its
 *    ordering notes).
 *  - Return value: TKV_OK (0) or a negative TKV_E_* code; tkv_last_error()
 *    returns a thread-local message naming the offending argument or knob.
 *  - bf16 row buffers (queries, attention outputs, new keys and values) are
 *    read and written in 16-byte vectors and must be 16-byte aligned
 *    (TKV_E_INVALID_ARG otherwise, before anything is launched).
 *  - Anomalies found on the device (page id out of range, a selection that
 *    does not fit the pool, a store to a non-resident page) set bits of a
 *    sticky error word returned by tkv_read_counters.  Pages cut by the
 *    selection cap are not errors: they are counted in `drops`.
 *  - One ctx is used from one stream at a time; calls on one ctx that
 *    overlap on different streams race.  (tkv_decode_layer_split and
 *    tkv_decode_layer_prefetch also use the `copy_stream` they are given,
 *    ordered by events the ctx owns.)
 *
 * Page row layout (identical in a pool slot and a mirror row; one row holds
 * one logical page for ALL layers): for layer l at l*layer_bytes,
 *   fp8  : K codes u8[Hkv][page][d] | V codes u8[Hkv][d][page] |
 *          K scales f32[page] | V scales f32[page]
 *          (V transposed: one head-dim row of a page is contiguous, the
 *          operand order of the P.V matrix product)
 *   bf16 : K bf16[Hkv][page][d] | V bf16[Hkv][page][d]
 * fp8 is OCP E4M3FN; one fp32 scale per token per tensor over all Hkv*d
 * values: scale = amax/448 (1 if amax == 0), code = e4m3(x / scale), round
 * to nearest even, saturating.
 *
 * Slab: bf16 [L][num_logical_pages][Hkv][d], the mean of each page's written
 * keys rounded once to bf16.
 */
#ifndef TKV_H
#define TKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TKV_OK 0
#define TKV_E_INVALID_ARG (-1)
#define TKV_E_UNSUPPORTED_FORMAT (-2)
#define TKV_E_CAPACITY (-3)
#define TKV_E_OOM (-4)
#define TKV_E_HIP (-5)
#define TKV_E_STATE (-6)

/* kv_format */
#define TKV_KV_BF16 0
#define TKV_KV_FP8_E4M3_PER_TOKEN 1
#define TKV_KV_NVFP4_BLOCK 2 /* recognised and refused: per-block scales the mirror cannot hold */

/* device error word bits */
#define TKV_ERR_PAGE_RANGE 1   /* a needed/selected page id outside [-1, num_logical_pages) */
#define TKV_ERR_CAPACITY 2     /* an ensure needed more distinct pages than slots: call ignored */
#define TKV_ERR_NOT_RESIDENT 4 /* store to a page with no slot: mirror and slab written, pool not */
#define TKV_ERR_BAD_MISS 8     /* fetch list entry outside the pool or the page space: skipped */
#define TKV_ERR_RUN_LEN 16     /* a write run spans more pages than its call's max_run_len allows:
                                  the pages past that reach were not made resident / not written */

typedef struct tkv_config {
  int32_t num_layers;
  int32_t num_q_heads;
  int32_t num_kv_heads;     /* num_q_heads / num_kv_heads must be 8; head_dim 128 */
  int32_t head_dim;
  int32_t page_size;        /* 16 or 64 tokens */
  int32_t kv_format;        /* TKV_KV_* */
  int64_t num_logical_pages;/* mirror rows (cf. --kv-host-pages + --num-pages) */
  int32_t num_slots;        /* GPU pool slots (cf. --num-pages), 1 .. 524288 */
  int32_t max_batch;        /* requests per call */
  int32_t max_rows;         /* query rows per call (decode: requests; prefill: chunk tokens) */
  int32_t max_topk;         /* pages selected per row */
  int32_t max_pages_per_req;/* block-table width */
  int32_t max_width;        /* entries of one ensure call (>= max_batch*max_sel_pages and write-ensures) */
} tkv_config;

typedef struct tkv_sizes {
  size_t pool_bytes;      /* num_slots * row_bytes */
  size_t slab_bytes;      /* bf16 slab */
  size_t state_bytes;     /* residency state, counters and the slab's fp64 running key sums */
  size_t workspace_bytes; /* per-call scratch for the largest call the config allows */
  size_t mirror_bytes;    /* pinned host mirror (allocated by tkv_create) */
  size_t row_bytes;       /* bytes of one page row (all layers) */
  size_t layer_bytes;     /* bytes of one layer of a row */
} tkv_sizes;

typedef struct tkv_device_buffers {
  void* pool;      /* >= pool_bytes, 256-byte aligned */
  void* slab;      /* >= slab_bytes */
  void* state;     /* >= state_bytes */
  void* workspace; /* >= workspace_bytes */
} tkv_device_buffers;

typedef struct tkv_counters {
  int64_t ensure_calls, hits, misses, fresh_allocs, evictions, drops, bytes_fetched, bytes_mirrored;
  int64_t clock;
  int32_t error_word;
  int32_t reserved;
} tkv_counters;

typedef struct tkv_ctx tkv_ctx;

/* Sizes of every buffer the config needs.  TKV_E_UNSUPPORTED_FORMAT for a
 * kv_format whose scales the mirror cannot hold (the message names
 * kv_format); TKV_E_INVALID_ARG for shapes the kernels do not support. */
int tkv_required_bytes(const tkv_config* cfg, tkv_sizes* out);

/* Validates the config and allocates the pinned, device-mapped host mirror
 * (zero-filled).  *out is owned by the caller until tkv_destroy. */
int tkv_create(const tkv_config* cfg, tkv_ctx** out);

/* Binds caller-allocated device buffers and initialises them on `stream`
 * (empty pool, zero slab, zero counters).  Synchronises `stream`. */
int tkv_attach_device(tkv_ctx* ctx, const tkv_device_buffers* bufs, void* stream);

/* FreeToken PR #525 commit summary (set_select_width takes max_bs): the
 * width is chosen so that a full batch's compacted selection always has
 * enough slots.  Sets the compaction width C = max_sel_pages (0 ->
 * 2*block_topk + 8, PR #499 "Design").  TKV_E_CAPACITY if max_bs*C >
 * num_slots or > max_width; the width is then left as it was. */
int tkv_set_select_width(tkv_ctx* ctx, int32_t max_bs, int32_t block_topk, int32_t max_sel_pages);

/* The compaction width C the last successful tkv_set_select_width set: the
 * row length of `needed` (int32 [B][C]) and the ensure width per request of
 * the fused decode calls (B*C entries of out_slots and miss).  Callers size
 * those buffers from this value.  0 before any width is set or for a NULL
 * ctx. */
int32_t tkv_select_width(const tkv_ctx* ctx);

/* Empties the pool (every page non-resident, clock 0) and zeroes the
 * counters and error word.  Slab and mirror contents are kept. */
int tkv_reset_residency(tkv_ctx* ctx, void* stream);

/* Indexer + compact_selected_pages (PR #499 "Why this works for sparse
 * attention", "Design").  Rows of request b are row_start[b] ..
 * row_start[b+1]-1 (device int32[B+1]).  For each row: qg[g] = bf16(sum of
 * the group's bf16 query heads), score of local page i = sum_g qg[g] .
 * slab[layer][block_table[b][i]][g] + page_bias[logical] (fp32), top-k by
 * score with ties to the lower page index, written ascending to
 * sel_local[row][0..topk) and padded with -1.  A row with row_pos != NULL
 * sees page i only if page_size*i <= row_pos[row].  Per request: union of
 * its rows' selections, ascending, unique, the first C logical ids written
 * to needed[b][0..C) (-1 padded), the rest counted as drops.
 *   q          bf16 [rows][Hq][d]           row_pos   int32 [rows] or NULL
 *   block_table int32 [B][max_pages]        n_pages   int32 [B]
 *   page_bias  f32 [num_logical_pages] or NULL
 *   sel_local  int32 [rows][topk] (out)     needed    int32 [B][C] (out) */
int tkv_select_pages(tkv_ctx* ctx, int32_t layer, const uint16_t* q, int32_t rows,
                     const int32_t* row_start, const int32_t* row_pos,
                     const int32_t* block_table, int32_t max_pages, const int32_t* n_pages,
                     int32_t B, const float* page_bias, int32_t topk, int32_t* sel_local,
                     int32_t* needed, void* stream);

/* Device-side LRU (PR #499 "What", "Design": fixed-shape, graph-safe, the
 * pool is an LRU cache over logical pages, eviction is a rebind).  One clock
 * tick per call; hits are restamped; misses in first-occurrence order take
 * the slots not hit by this call in ascending (stamp, slot) order.  A miss
 * whose first occurrence has no_fetch[j] != 0 is bound without a fetch.
 *   needed    int32 [width] logical ids, -1 = padding
 *   no_fetch  uint8 [width] or NULL
 *   out_slots int32 [width] (out): slot of needed[j] after the call, or -1
 *   miss      int32 [width][2] (out): (slot, page) rows to fetch
 *   miss_count int32 [1] (out)
 * A call needing more distinct pages than slots changes nothing and sets
 * TKV_ERR_CAPACITY. */
int tkv_lru_ensure(tkv_ctx* ctx, const int32_t* needed, int32_t width, const uint8_t* no_fetch,
                   int32_t* out_slots, int32_t* miss, int32_t* miss_count, void* stream);

/* Fused host->device page copy (PR #499 "Design": one launch copies K+V of
 * a page across all layers; PR #525 commit summary: with the scale banks):
 * pool row miss[i][0] := mirror row miss[i][1] for i < *miss_count, all
 * layers, codes and scales.  `width` bounds *miss_count (fixed launch shape).
 * The miss list is one an ensure of this ctx wrote (tkv_lru_ensure): that
 * ensure completed the mirror rows of its misses from any block a split
 * store still held in its staging copy, so the fetch does not wait for a
 * split store's mirror copy. */
int tkv_fetch_pages(tkv_ctx* ctx, const int32_t* miss, const int32_t* miss_count, int32_t width,
                    void* stream);

/* The copy of tkv_fetch_pages in two parts, the parts tkv_decode_layer_split
 * issues.  tkv_fetch_pages_layer copies, for every miss, only layer
 * `layer`'s slice of the row (its K and V codes and scales) and keeps a copy
 * of the miss list and count in the ctx; it adds the whole rows to
 * bytes_fetched.  tkv_fetch_pages_rest copies the rest of the rows of the
 * list the last tkv_fetch_pages_layer kept, for the same `layer`; it must
 * follow that call in stream order (or by an event) and come before the next
 * one.  Both parts together write exactly what tkv_fetch_pages writes.
 * width <= max_width; miss, miss_count as for tkv_fetch_pages. */
int tkv_fetch_pages_layer(tkv_ctx* ctx, const int32_t* miss, const int32_t* miss_count, int32_t width,
                          int32_t layer, void* stream);
int tkv_fetch_pages_rest(tkv_ctx* ctx, int32_t width, int32_t layer, void* stream);

/* Sparse paged attention over the selected pages (PR #499 "Design": after
 * ensure the block table is translated logical->physical; the page ids are
 * translated here through the LRU's page->slot map).  For row r of request b
 * and query head h (KV head h/8): softmax over the tokens 64*i+j of the
 * selected resident pages i with position < ctx_len[b] (and <= row_pos[r]
 * when row_pos != NULL) of (q_h . k)/sqrt(d), times v; k and v dequantised.
 * Empty selection -> zeros.  out bf16 [rows][Hq][d], round to nearest even.
 * Rows of request b are row_start[b] .. row_start[b+1]-1 (device int32[B+1]);
 * block_table int32 [B][max_pages]; ctx_len int32 [B]; sel_local as
 * written by tkv_select_pages.  With rows > max_batch (prefill chunks) topk
 * must be <= 64. */
int tkv_sparse_paged_attn(tkv_ctx* ctx, int32_t layer, const uint16_t* q, int32_t rows,
                          const int32_t* row_start, const int32_t* row_pos,
                          const int32_t* ctx_len, int32_t B, const int32_t* sel_local,
                          const int32_t* block_table, int32_t max_pages, int32_t topk,
                          uint16_t* out, void* stream);

/* Sparse paged attention with the host tail read in place (vLLM RFC #33980,
 * discussion: KV beyond the HBM tier is host memory that the attention
 * kernel loads over the interconnect, with no staging copy).  Arguments and
 * results as tkv_sparse_paged_attn; a selected page that is not resident is
 * read from its mirror row (this layer's block only: K and V codes and
 * scales, 66,048 bytes at 4 KV heads x d 128 x 64-token fp8 pages) instead of
 * being skipped.  Nothing is fetched, no slot is bound, the LRU state and the
 * counters do not move, so a step built from tkv_select_pages and this call
 * leaves the pool as it was.  Mirror rows of pages never written read as
 * zeros. */
int tkv_sparse_paged_attn_host_tail(tkv_ctx* ctx, int32_t layer, const uint16_t* q, int32_t rows,
                                    const int32_t* row_start, const int32_t* row_pos, const int32_t* ctx_len,
                                    int32_t B, const int32_t* sel_local, const int32_t* block_table,
                                    int32_t max_pages, int32_t topk, uint16_t* out, void* stream);

/* One decode step of one layer for B requests with one query row each:
 * select + compact + ensure in one launch, then fetch, then attention.
 * Same semantics as tkv_select_pages -> tkv_lru_ensure(needed, B*C) ->
 * tkv_fetch_pages -> tkv_sparse_paged_attn.  out_slots int32 [B*C],
 * miss int32 [B*C][2], miss_count int32 [1].  With topk <= C and the
 * matrix-core decode attention (fp8, 64-token pages, B*Hkv < 256) the fetch
 * runs inside the attention launch: the pages it brings in are read for
 * this layer from their mirror rows, and the pool and mirror end the call
 * as after the separate fetch. */
int tkv_decode_layer(tkv_ctx* ctx, int32_t layer, const uint16_t* q, int32_t B,
                     const int32_t* block_table, int32_t max_pages, const int32_t* n_pages,
                     const int32_t* ctx_len, const float* page_bias, int32_t topk,
                     int32_t* sel_local, int32_t* needed, int32_t* out_slots, int32_t* miss,
                     int32_t* miss_count, uint16_t* out, void* stream);

/* tkv_decode_layer with the fused row copy (FreeToken PR #499, "Design":
 * one copy per miss carries the page for every layer) issued in two parts:
 * on `stream`, for every miss, the slices of `layer` (what this layer's
 * attention reads) and of the next layer ((layer+1) mod num_layers); then on
 * `copy_stream` the rest of the rows, overlapping this layer's attention and
 * the next call's selection and ensure.  A call for the layer after the
 * previous call's, with num_slots >= W_prev + 2*W (W = B * the compaction
 * width), chains: no slot the previous call filled can be rebound by this
 * call's ensure, so this call's slice copy waits only for the rest copy of
 * the call two back, and its attention for nothing on `copy_stream`.  Any
 * other call waits for every earlier copy; so does every other call of this
 * library that touches the pool or the state (select_pages and lru_ensure
 * end a chain).
 * Results (sel, needed, slots, misses, attention, LRU state, counters) and,
 * once the copy stream is done, pool contents are those of tkv_decode_layer.
 * Ordering the caller owns: work of its own that reads the pool, and the
 * end of a graph capture, must first wait for `copy_stream` (one wait at
 * the end of a step suffices).  Inside a capture the first call does not
 * wait for copies issued outside it: order graph replays after eager work,
 * as for any capture.  `copy_stream` may equal `stream` (the parts then run
 * in order on it).  One layer (num_layers == 1): same as tkv_decode_layer.
 * Calls on one ctx must not overlap. */
int tkv_decode_layer_split(tkv_ctx* ctx, int32_t layer, const uint16_t* q, int32_t B,
                           const int32_t* block_table, int32_t max_pages, const int32_t* n_pages,
                           const int32_t* ctx_len, const float* page_bias, int32_t topk,
                           int32_t* sel_local, int32_t* needed, int32_t* out_slots, int32_t* miss,
                           int32_t* miss_count, uint16_t* out, void* stream, void* copy_stream);

/* tkv_decode_layer preceded by a preload of a predicted page list (vLLM RFC
 * #33980, "Topk KV preload": an earlier top-k index, e.g. the next layer's
 * needed list from the previous step, is loaded ahead; after the real
 * selection only the pages it missed are loaded).  pred: int32 [pred_width]
 * logical page ids, -1 ignored, pred_width <= min(max_width, num_slots);
 * device memory, read on `stream` before anything else of this call.  The
 * preload is an LRU ensure of pred on `stream`; the copy of its misses runs
 * on `copy_stream` (a different stream; NULL or `stream` itself = serial),
 * overlapped with this layer's selection and ensure; this layer's fetch and
 * attention wait for that copy, since this layer's ensure may rebind a slot
 * the copy still writes.  Results (sel, needed, slots, misses, attention,
 * LRU state) are those of an ensure+fetch of pred followed by
 * tkv_decode_layer.  Uses one preload workspace per ctx: calls on one ctx
 * must not overlap. */
int tkv_decode_layer_prefetch(tkv_ctx* ctx, int32_t layer, const uint16_t* q, int32_t B,
                              const int32_t* block_table, int32_t max_pages, const int32_t* n_pages,
                              const int32_t* ctx_len, const float* page_bias, int32_t topk, int32_t* sel_local,
                              int32_t* needed, int32_t* out_slots, int32_t* miss, int32_t* miss_count,
                              uint16_t* out, const int32_t* pred, int32_t pred_width, void* stream,
                              void* copy_stream);

/* ensure_write_pages (PR #499 "Design": one fixed-shape launch of stride
 * samples at page steps and a last sample at each run's end): run r writes tokens
 * run_start[r] .. run_start[r]+run_len[r]-1 of request run_req[r].  Every
 * page the runs touch is made resident (one ensure call); a page whose
 * first position is >= old_len[req] has no content yet and is bound without
 * a fetch; other missed pages are fetched.  run_len[r] <= max_run_len. */
int tkv_ensure_write_pages(tkv_ctx* ctx, int32_t n_runs, const int32_t* run_req,
                           const int32_t* run_start, const int32_t* run_len, int32_t max_run_len,
                           const int32_t* block_table, int32_t max_pages, const int32_t* old_len,
                           void* stream);

/* store_kv with the write-through mirror (PR #499 "Design"; PR #525 commit
 * summary, mirror_store_quant: the mirror takes the codes and scales read
 * after quantisation).  k, v bf16 [n_tok][Hkv][d]: the tokens of run r are
 * at rows run_tok_off[r] ..; they are quantised (fp8) or copied (bf16) into
 * the page's slot and its mirror row; a write that begins a page zero-fills
 * the page's later positions; the slab entry of each touched page becomes
 * the mean of all its written keys.  Runs of one call must not share pages.
 * Pages must be resident (tkv_ensure_write_pages). */
int tkv_store_kv_mirror(tkv_ctx* ctx, int32_t layer, const uint16_t* k, const uint16_t* v,
                        int32_t n_runs, const int32_t* run_req, const int32_t* run_start,
                        const int32_t* run_len, const int32_t* run_tok_off, int32_t max_run_len,
                        const int32_t* block_table, int32_t max_pages, void* stream);

/* tkv_store_kv_mirror with its mirror writes moved off `stream` (FreeToken
 * PR #499, "Design": the write-through mirror; here the writes of a run's
 * whole pages leave after the pool's).  On `stream` the new K/V are
 * quantised into the pool slots and the slab, and the layer's block of each
 * page the write begins (the block is then defined in full: written
 * positions and the zero-filled tail) is built in a staging copy in the
 * workspace; a copy kernel on `copy_stream` then moves those blocks to the
 * mirror rows.  Writes that continue a page go to the mirror directly, on
 * `stream`.  Once `copy_stream` reaches the end of the copy, pool, slab and
 * mirror hold what tkv_store_kv_mirror writes.
 * When `stream` is not being captured, the copy is enqueued later: by the
 * next attention call on the ctx (tkv_sparse_paged_attn, a decode layer),
 * ordered after that call's position on `stream` so that it runs beside the
 * attention, or by any earlier call that needs the mirror, or by
 * tkv_mirror_flush.  Calls that read or write the mirror wait for it
 * (stores, write-ensures, prefix calls, host-tail attention, tkv_read_
 * counters and the debug readbacks); ensures meanwhile copy the staged
 * block of any page they make a fetch of into its mirror row first, so
 * fetches and the copies of decode layers need no wait; tkv_select_pages,
 * tkv_lru_ensure and attention over the pool run beside the copy.  A caller
 * that reads the mirror itself first calls tkv_mirror_flush and waits for
 * `stream`.  The staging holds one run of max_rows tokens (max_rows/
 * page_size + 1 blocks); blocks past it are written directly.  `copy_stream`
 * NULL or equal to `stream`: the same as tkv_store_kv_mirror.  Calls on one
 * ctx must not overlap. */
int tkv_store_kv_mirror_split(tkv_ctx* ctx, int32_t layer, const uint16_t* k, const uint16_t* v,
                              int32_t n_runs, const int32_t* run_req, const int32_t* run_start,
                              const int32_t* run_len, const int32_t* run_tok_off, int32_t max_run_len,
                              const int32_t* block_table, int32_t max_pages, void* stream, void* copy_stream);

/* Enqueues the mirror copy a split store deferred (if any) and orders
 * `stream` after it (the write-through mirror of FreeToken PR #499,
 * "Design", complete from `stream`'s point of view).  Fails with
 * TKV_E_STATE when the deferred copy's store stream is being captured. */
int tkv_mirror_flush(tkv_ctx* ctx, void* stream);

/* Cold-prefix records (FreeToken PR #525, "What the patch does", items
 * 2-4: a prefix leaving the tier is copied out because logical ids get
 * reused; on a later hit it comes back host to host into the mirror and the
 * LRU's fetch on selection covers residency).  A record is one page's
 * mirror row (row_bytes) followed by its indexer slab entries for every
 * layer: bf16 values [L][Hkv*d], then fp64 key sums [L][Hkv*d] (what a
 * partly written page's later tokens add to); tkv_prefix_record_bytes
 * gives its size (row_bytes + L*Hkv*d*10). */
int64_t tkv_prefix_record_bytes(const tkv_ctx* ctx);

/* Copies the records of `n` logical pages (pages: host int32 [n], each in
 * [0, num_logical_pages)) into `records` (host memory, n records).  Rows
 * are copied host to host from the pinned mirror (which holds every
 * written byte); the slab entries come from the GPU in 128-page slices
 * through a staging buffer this call allocates and frees.  Synchronises
 * `stream` first (stores queued before it have landed) and before
 * returning.  The tier's state does not change. */
int tkv_prefix_save(tkv_ctx* ctx, const int32_t* pages, int32_t n, void* records, void* stream);

/* Rehydration: writes `n` records into the mirror rows and slab entries of
 * `pages` (host int32 [n], distinct, each in [0, num_logical_pages); they
 * may differ from the ids the records were saved from), and unbinds any of
 * these ids that is resident in the pool (its slot holds the id's previous
 * content; the slot keeps its recency and is reused in LRU order).
 * Nothing is fetched: a later ensure brings a page in when it is needed.
 * Synchronises `stream` first (no queued copy still reads these rows) and
 * before returning; allocates and frees a staging buffer. */
int tkv_prefix_restore(tkv_ctx* ctx, const int32_t* pages, int32_t n, const void* records, void* stream);

/* tkv_prefix_restore for callers that cannot allocate memory during the
 * call (serving loops and harnesses that forbid hipMalloc/hipFree): same
 * arguments, results and synchronisation; the slab entries pass through a
 * fixed 2 MiB device array the library holds on each GPU until the process
 * ends (its address is taken once per device in tkv_attach_device), in
 * passes of as many pages as fit (34 at 12 layers x 4 KV heads x d 128), and
 * the mirror rows are copied in the calling thread.  TKV_E_CAPACITY when one
 * page's slab entries (num_layers*num_kv_heads*head_dim*10 bytes) do not
 * fit.  All ctxs on one GPU share the array; calls are serialised within a
 * process, and each pass overwrites what the previous one staged. */
int tkv_prefix_restore_noalloc(tkv_ctx* ctx, const int32_t* pages, int32_t n, const void* records, void* stream);

/* Copies the counters to the host.  Synchronises `stream`. */
int tkv_read_counters(tkv_ctx* ctx, tkv_counters* out, void* stream);

/* Test hooks.  Copy the LRU state to host arrays (page_to_slot
 * [num_logical_pages], slot_to_page [num_slots], stamp [num_slots]);
 * synchronises `stream`. */
int tkv_debug_read_state(tkv_ctx* ctx, int32_t* page_to_slot, int32_t* slot_to_page,
                         int64_t* stamp, int64_t* clock, void* stream);
/* Chooses the attention kernel of later calls: TKV_ATTN_AUTO (the matrix-core
 * kernel where it applies: fp8, 64-token pages, d = 128, 8 query heads per
 * KV head; else the vector kernel), TKV_ATTN_VECTOR, or TKV_ATTN_MATRIX
 * (TKV_E_UNSUPPORTED_FORMAT when the shapes do not fit it).  Both compute the
 * same softmax; tests compare them. */
enum { TKV_ATTN_AUTO = 0, TKV_ATTN_VECTOR = 1, TKV_ATTN_MATRIX = 2 };
int tkv_debug_set_attn_kernel(tkv_ctx* ctx, int32_t kernel);
/* Pages per range of the multi-pass attention over many rows (prefill
 * chunks on the matrix-core kernel): one launch per range of `pages` local
 * page ids, the softmax state carried between launches; 0 = a single pass
 * (the default: the passes cut the bytes past the L2s 3.6x at 192 pages but
 * the kernel is bound by instruction issue, not by those bytes).  Both give
 * the same bits; tests compare them. */
int tkv_debug_set_attn_range(tkv_ctx* ctx, int32_t pages);
/* fp32 -> e4m3 codes with the store's encoder; device pointers. */
int tkv_debug_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream);
/* e4m3 codes -> fp32 with the attention kernel's decoder; device pointers. */
int tkv_debug_e4m3_decode(const uint8_t* in, float* out, int64_t n, void* stream);

/* Host pointer to the pinned mirror (read-only view for tests). */
const void* tkv_mirror_host_ptr(const tkv_ctx* ctx);

/* Frees the mirror and the ctx.  Device buffers stay with the caller.  The
 * caller first synchronises the streams it passed to this ctx's calls:
 * kernels still running may read or write the mirror (a plain store writes
 * it directly).  The ctx's own copies (rest-of-rows copies, a launched
 * mirror copy) are waited for here; a split store's copy not yet launched
 * is dropped with the mirror. */
void tkv_destroy(tkv_ctx* ctx);

const char* tkv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TKV_H */
