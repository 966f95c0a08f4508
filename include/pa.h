/*
 * pa.h - paged KV cache and single-token decode attention for AMD MI355X (gfx950).
 *
 * C ABI of libpa.so.  Plain pointers and sizes only.
 *
 * Sources this interface follows (one page each):
 *   [KVP] "Insights into LLM Serving Systems: KV-Cache Memory Allocation
 *         Patterns", section 4, Observations 1 and 2.
 *   [PAS] "Efficient Memory Management for Large Language Model Serving with
 *         PagedAttention" (summary page), Summary and Key points.
 *   [ROC] "Running Out of Cache" (serving plate XXIII.3): paging paragraph,
 *         block-size paragraph, Workshop, "Fragmentation is lost users", Terms.
 *   [VAC] "Leveraging Low-Level CUDA APIs for vAttention's Dynamic Memory",
 *         section 5.2.3 (request-level KV-cache indexing).
 *
 * ---------------------------------------------------------------------------
 * Cache layout (device memory owned by the caller)
 * ---------------------------------------------------------------------------
 * One device array, element type kv_dtype, holds the K and V caches of all
 * layers.  Each layer is an array of (block, KV head) regions; a region holds
 * block_size / sub tile pairs of sub = min(block_size, 16) token rows each:
 * the K tile of those rows, then their V tile.  VE = 16 / sizeof(element)
 * (8 for bf16, 4 for fp32):
 *
 *   cache: [num_layers][units][num_kv_heads][block_size/sub][2][tile]  (2: K, then V)
 *   K tile [head_dim/VE][sub][VE]
 *   V tile [head_dim][sub]
 *
 * The K tile keeps each token row in 16-byte chunks (chunk-major); the V tile
 * is dimension-major.  Both make the decode kernel's matrix-core operand
 * loads contiguous wave accesses, and the K and V of 16 consecutive tokens of
 * a head are one contiguous run for the decode to read (8 KiB for bf16,
 * head_dim 128), with blocks of 32 tokens as with blocks of 16.
 *
 * PA_PAGED: units = num_blocks.  Block b holds, for every KV head,
 * block_size consecutive tokens; a sequence's blocks need not be adjacent and
 * its block table maps logical block j (tokens j*BS .. j*BS+BS-1) to a
 * physical block ([ROC] paging paragraph and Terms; [PAS] Summary).  One block
 * id names the same block in every layer, in K and in V.
 * PA_CONTIGUOUS: units = max_seqs * max_seq_len / block_size.  Request r owns
 * the max_seq_len / block_size consecutive blocks starting at block
 * r * max_seq_len / block_size, i.e. the sub-tensor at offset r x (max K-cache
 * size of one request) of each layer's tensor ([VAC] 5.2.3); the library
 * hands out r.
 *
 * A "slot" names one token row: slot = u*block_size + o, u the block, o the
 * row in it (contiguous: slot = reqId*max_seq_len + position).  Element
 * (slot, head h, dim e) of layer l is, with r = o % sub and pair =
 * ((l*units + u)*num_kv_heads + h) * 2 * head_dim * block_size
 * + (o / sub) * 2 * head_dim * sub (in elements from the array's start):
 *   K: pair + ((e / VE) * sub + r) * VE + e % VE
 *   V: pair + head_dim * sub + e * sub + r
 *
 * ---------------------------------------------------------------------------
 * Conventions
 * ---------------------------------------------------------------------------
 * Ownership: the caller owns all device memory (cache, q, out, tables, slots,
 *   workspace) and keeps it alive while the pool uses it.  The library owns
 *   only the opaque host-side pa_pool and frees it in pa_destroy_pool.  No
 *   function allocates device memory, except that a demand-paged pool
 *   (pa_create_pool_vmm) maps its own cache pages in pa_reserve.
 * Errors: every call returns a pa_status; PA_OK is 0, errors are negative.
 *   Nothing throws across the ABI.  On error no state changes (pa_reserve is
 *   all-or-nothing) and pa_last_error() gives a message for the calling thread.
 * Validation: host-visible arguments are checked on the host.  Device arrays
 *   (tables, lengths, slots, pairs) are trusted: their entries must be in
 *   range; out-of-range entries give undefined results.  pa_check_decode_args,
 *   pa_check_slots, pa_check_block_pairs and pa_check_shared_args check host
 *   copies of them.
 * Threads and streams: a pool is not thread-safe.  Device calls only enqueue
 *   work on the given stream (hipStream_t passed as void*, NULL = the default
 *   stream) and never synchronise; the caller orders them.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,   /* bad argument; nothing changed */
  PA_ERR_NO_BLOCKS = -2,     /* not enough free blocks: pre-empt a request and retry */
  PA_ERR_NO_REQ_ID = -3,     /* all max_seqs request ids are live */
  PA_ERR_UNKNOWN_SEQ = -4,   /* request id is not live */
  PA_ERR_WORKSPACE = -5,     /* decode workspace missing or too small */
  PA_ERR_HIP = -6,           /* a HIP call failed (launch error) */
  PA_ERR_UNSUPPORTED = -7,   /* valid request this build has no kernel for */
  PA_ERR_NO_MEMORY = -8      /* the library's host-side state could not be allocated */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

typedef enum pa_layout { PA_PAGED = 0, PA_CONTIGUOUS = 1 } pa_layout;

typedef struct pa_pool_desc {
  int32_t num_layers;    /* >= 1 */
  int32_t num_blocks;    /* paged: physical blocks (>= 1); contiguous: ignored */
  int32_t block_size;    /* tokens per block: 8, 16 (the pages' default) or 32 */
  int32_t num_kv_heads;  /* >= 1 */
  int32_t head_dim;      /* 64 or 128 */
  pa_dtype kv_dtype;     /* element type of the cache (K and V) */
  pa_layout layout;
  int32_t max_seqs;      /* live requests at once; reqIds are 0 .. max_seqs-1 */
  int32_t max_seq_len;   /* S: most tokens per request; contiguous: multiple of block_size */
} pa_pool_desc;

typedef struct pa_stats {
  int64_t free_blocks;      /* paged: blocks on the free list */
  int64_t used_blocks;      /* paged: blocks held by at least one request */
  int64_t tokens;           /* token rows physically held (a shared row counts once) */
  int64_t logical_tokens;   /* sum of resident requests' lengths */
  int64_t reserved_tokens;  /* paged: used_blocks*block_size; contiguous: live*S */
  int64_t live_seqs;        /* resident requests (swapped-out ones not counted) */
  int64_t cow_copies;       /* copy-on-write copies made since creation */
  int64_t shared_blocks;    /* blocks currently held by more than one request */
  double utilisation;       /* tokens / reserved_tokens: share of reserved cache
                               holding real tokens ([ROC] readouts, [PAS] Key points) */
  int64_t swapped_seqs;     /* requests swapped out (pa_swap_out) */
  int64_t swapped_tokens;   /* sum of their lengths */
} pa_stats;

typedef struct pa_pool pa_pool; /* opaque, host memory */

/* Bytes of the cache array (K and V of every layer) described by desc, or 0
 * if desc is invalid. */
size_t pa_cache_bytes(const pa_pool_desc* desc);

/* KV bytes one token takes over all layers, K plus V:
 * 2 * num_layers * num_kv_heads * head_dim * sizeof(kv_dtype)  ([KVP]
 * Observation-2 prints 64, 128 and 240 KB for Yi-6B, Llama-3-8B and Yi-34B). */
size_t pa_bytes_per_token(const pa_pool_desc* desc);

/* Create a cache of fixed-size blocks over caller memory ([ROC] paging
 * paragraph).  d_cache: device array of pa_cache_bytes(desc) bytes, 16-byte
 * aligned.  Host-only: touches no device memory.  All blocks start free and
 * are handed out in ascending id order; all request ids start free, 0 first.
 * *out receives the handle. */
pa_status pa_create_pool(const pa_pool_desc* desc, void* d_cache, pa_pool** out);

/* Free the host handle.  The cache is the caller's (a demand-paged pool's is
 * the library's: it is unmapped and freed here, so no queued or running work
 * may still use it). */
pa_status pa_destroy_pool(pa_pool* pool);

/* ---- demand-paged contiguous caches ([VAC] 5.2.1-5.2.3) -------------------
 * The contiguous layout with its cache backed on demand: the library reserves
 * the virtual range of the cache (num_layers x max_seqs x one request's
 * sub-range, request reqId's sub-range at reqId x S, as pa_create_pool lays
 * it out) without physical memory, and pa_reserve maps physical pages into a
 * request's sub-range of every layer before it hands out slots past the pages
 * already there.  A request's sub-range of one layer holds its S /
 * block_size blocks, K and V: S x num_kv_heads x head_dim x elt x 2 bytes.
 * Pages are 2 MiB where that is a multiple of 2 MiB, else the device's
 * allocation granularity (which it must then be a multiple of); each page is
 * its own physical allocation.  physical_bytes caps the memory mapped: a
 * pa_reserve that would pass it fails with PA_ERR_NO_BLOCKS and changes
 * nothing (PA_ERR_HIP from the mapping calls may leave pages mapped but
 * changes no length).  A freed request's pages stay mapped for the next
 * request given its id (ids are reused last-freed first) until pa_vmm_trim.
 * Everything else is the contiguous pool's.  PA_ERR_UNSUPPORTED: the device
 * or the sizes do not allow it. */
typedef struct pa_vmm_stats {
  int64_t page_bytes;    /* physical page (allocation granularity) */
  int64_t mapped_bytes;  /* physical memory mapped, all layers */
  int64_t budget_bytes;  /* physical_bytes rounded down to whole pages */
  int64_t region_bytes;  /* one request's sub-range of one layer (K and V) */
} pa_vmm_stats;

pa_status pa_create_pool_vmm(const pa_pool_desc* desc, size_t physical_bytes, pa_pool** out);

pa_status pa_vmm_info(const pa_pool* pool, pa_vmm_stats* out);

/* Unmap the pages of every request id that is not live; *freed_bytes_out (may
 * be NULL) gets the bytes given back.  No queued or running work may still
 * touch those requests' caches: synchronise the streams that used them
 * first. */
pa_status pa_vmm_trim(pa_pool* pool, int64_t* freed_bytes_out);

/* Replace the order in which free blocks are handed out: block_ids[0] first.
 * block_ids must be a permutation of 0..num_blocks-1 and no block may be in
 * use.  Paged only.  (Seeded placements: results must not depend on it.) */
pa_status pa_set_free_order(pa_pool* pool, const int32_t* block_ids, int32_t n);

/* ---- host block allocator: synchronous, touches no device memory ---------- */

/* Admit a request: *req_id_out gets a free id in [0, max_seqs) ([VAC] 5.2.3:
 * the library allocates reqId).  Its length is 0 and it holds no block. */
pa_status pa_seq_add(pa_pool* pool, int32_t* req_id_out);

/* Share all of parent's blocks with a new request ([PAS] Summary and Key
 * points: sharing within a request for parallel samples or beam search, and
 * across requests).  Each shared block's share count goes up by one; the
 * child's length equals the parent's.  Paged only. */
pa_status pa_seq_fork(pa_pool* pool, int32_t parent, int32_t* child_out);

/* End a request or pre-empt it ([ROC] "Fragmentation is lost users" and the
 * Pre-emption term): each of its blocks loses one share and returns to the
 * free list (in table order, last freed is reused first) when none is left;
 * its id becomes free. */
pa_status pa_seq_free(pa_pool* pool, int32_t req_id);

/* Grow requests by counts[i] tokens each (counts NULL: one token each, the
 * decode step of [KVP] Observation-1).  Allocate-on-fill: a request takes a
 * new block only when its last block is full, so it wastes under one block
 * ([ROC] paging paragraph).  Copy-on-write: if the next position falls inside
 * a last block that is still shared, the request first moves to a fresh copy
 * and drops its share; the last holder writes in place; full shared blocks are
 * never copied ([PAS] Summary, [ROC] "Fragmentation is lost users").
 * Requests are handled in the order given; each may appear once.
 *   slots_out:     receives sum(counts) slots, request by request, position
 *                  order (capacity slots_cap).
 *   cow_pairs_out: receives *n_cow_out pairs {src_block, dst_block}
 *                  (capacity cow_cap pairs; may be NULL if cow_cap is 0).
 *                  Copy them with pa_copy_blocks BEFORE appending any slot
 *                  returned by this call.
 * All-or-nothing: PA_ERR_NO_BLOCKS (caller pre-empts and retries),
 * PA_ERR_INVALID_ARG (cap too small, length beyond max_seq_len, duplicate id)
 * and PA_ERR_UNKNOWN_SEQ change nothing.  Contiguous: slot = reqId*S + pos,
 * no blocks, no copies. */
pa_status pa_reserve(pa_pool* pool, const int32_t* req_ids, int32_t n, const int32_t* counts,
                     int32_t* slots_out, int64_t slots_cap, int32_t* cow_pairs_out,
                     int32_t cow_cap, int32_t* n_cow_out);

/* Read block tables ([ROC] Terms: block table) into tables_out[n][stride],
 * padded with -1, and lengths into lens_out[n] (either may be NULL).
 * PA_ERR_INVALID_ARG if a table has more than stride entries.  Contiguous:
 * tables are all -1 (none exist). */
pa_status pa_get_block_tables(const pa_pool* pool, const int32_t* req_ids, int32_t n,
                              int32_t stride, int32_t* tables_out, int32_t* lens_out);

pa_status pa_get_stats(const pa_pool* pool, pa_stats* out);

/* ---- shared prefixes: one read of a shared block for all its sharers ------
 * Samples of one prompt (pa_seq_fork) point at the same physical blocks
 * ([PAS] Summary and Key points; [ROC] "Fragmentation is lost users"), so
 * their attention over those blocks reads the same K and V.  pa_decode_shared
 * reads each shared block once per group and KV head and attends every
 * member's query heads to it; the rest of each context is decoded as by
 * pa_decode, and the partitions are merged in the same order. */

/* Find the groups among req_ids (in the order given, as the batch will be):
 * runs of at least two consecutive requests whose block tables start with
 * the same blocks for at least partition_tokens tokens.  For each request i,
 * seq_shared_out[i] gets the tokens its group shares, cut to a multiple of
 * partition_tokens and to every member's length (0 outside groups);
 * groups_out[2g] and groups_out[2g+1] get the batch index of group g's first
 * member and its member count (capacity 2n); *n_groups_out the number of
 * groups; *max_members_out and *max_shared_out the largest group and shared
 * prefix (0 if none).  Paged only; partition_tokens as for pa_decode. */
pa_status pa_shared_groups(const pa_pool* pool, const int32_t* req_ids, int32_t n,
                           int32_t partition_tokens, int32_t* seq_shared_out, int32_t* groups_out,
                           int32_t* n_groups_out, int32_t* max_members_out, int32_t* max_shared_out);

/* pa_decode for a batch whose groups pa_shared_groups found (the batch in
 * the order given to it): d_seq_shared (device int32 [num_seqs]) and d_groups
 * (device int32 [num_groups][2]) are its outputs copied to the device, and
 * num_groups, max_members, max_shared its host outputs; partition_tokens must
 * be the one given to it.  The result is pa_decode's with the same
 * partition_tokens up to the order of fp32 sums within the shared partitions.
 * The workspace holds max(2, ceil(max_context / partition_tokens)) partitions:
 * pa_decode_workspace_bytes(pool, num_seqs, num_q_heads,
 * max(max_context, partition_tokens + 1), partition_tokens) bytes.  Paged
 * only; query heads per KV head <= 16. */
pa_status pa_decode_shared(pa_pool* pool, int32_t layer, const void* d_q, pa_dtype q_dtype,
                           int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                           int32_t table_stride, const int32_t* d_context_lens, int32_t num_seqs,
                           int32_t max_context, int32_t partition_tokens, const int32_t* d_seq_shared,
                           const int32_t* d_groups, int32_t num_groups, int32_t max_members,
                           int32_t max_shared, float* d_out, void* d_workspace,
                           size_t workspace_bytes, void* stream);

/* One decode step of a layer for such a batch in one launch (plus the
 * merge): pa_append_kv of each sequence's new token, then pa_decode_shared
 * over contexts that end with it.  d_k, d_v, d_slots as for
 * pa_append_decode; the other arguments as for pa_decode_shared.  The new
 * token of every sequence that appends (slot >= 0) must lie past its shared
 * prefix (seq_shared[s] <= L_s - 1): pa_shared_groups called after the
 * step's pa_reserve gives that, since the reserve makes each writer's last
 * block its own ([PAS] Summary: a shared block is copied before a sharer
 * writes into it); pa_check_shared_args checks it on host copies.  The cache
 * afterwards equals pa_append_kv's, the output pa_decode_shared's after that
 * append, bit for bit. */
pa_status pa_append_decode_shared(pa_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                                  const int32_t* d_slots, const void* d_q, pa_dtype q_dtype,
                                  int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                                  int32_t table_stride, const int32_t* d_context_lens, int32_t num_seqs,
                                  int32_t max_context, int32_t partition_tokens, const int32_t* d_seq_shared,
                                  const int32_t* d_groups, int32_t num_groups, int32_t max_members,
                                  int32_t max_shared, float* d_out, void* d_workspace,
                                  size_t workspace_bytes, void* stream);

/* ---- pre-emption by swapping ([ROC] "Fragmentation is lost users" and the
 * Pre-emption term: when paging runs out, a request's cache is evicted and
 * swapped back in later; [PAS] Summary: the scheduler pre-empts requests) ----
 *
 * A swapped-out request keeps its id and length but holds no blocks: it cannot
 * grow (pa_reserve), fork, or have its table read (PA_ERR_INVALID_ARG) until
 * it is swapped in; pa_seq_free drops it.  Its image, in memory the caller
 * owns, holds every layer's copy of its blocks:
 *     image[layer][j][num_kv_heads][region]
 * for j < ceil(L / block_size) in logical order, each (block, head) region as
 * the pool lays it out (its tile pairs), i.e.
 * num_layers * ceil(L/BS) * 2 * num_kv_heads * head_dim * BS * elt bytes.
 * Whole blocks are copied, rows past L included.  Sharing is not kept: blocks
 * the request shared are copied out in full and come back as its own.
 * Paged only. */

/* Bytes of req_id's image (a resident or swapped-out request). */
pa_status pa_swap_bytes(const pa_pool* pool, int32_t req_id, size_t* bytes_out);

/* Copy resident request req_id's blocks into the image at d_image (capacity
 * image_bytes; pinned host memory from hipHostMalloc, or device memory; 16-byte
 * aligned), then give the blocks back as pa_seq_free does (table order, a
 * block is free once no other request holds it).  Asynchronous on stream: the
 * image is complete when the stream reaches this point, and the released
 * blocks may be handed out again at once, so work that writes them must be
 * ordered after this call (same stream, or an event).  d_image NULL with
 * image_bytes 0: no copy, the contents are dropped (pre-emption by
 * recomputation; no device work, no stream use).  PA_ERR_INVALID_ARG
 * (contiguous pool, swapped-out request, image too small, unaligned, or memory
 * the device cannot address) and PA_ERR_UNKNOWN_SEQ change nothing. */
pa_status pa_swap_out(pa_pool* pool, int32_t req_id, void* d_image, size_t image_bytes,
                      void* stream);

/* Take ceil(L / block_size) fresh blocks for swapped-out request req_id (off
 * the free list, all or nothing: PA_ERR_NO_BLOCKS changes nothing) and copy
 * its image back into them.  Asynchronous on stream; the image must stay
 * unchanged until the stream passes this point.  Afterwards the request is
 * resident with a new block table and the same contents.  d_image NULL with
 * image_bytes 0: no copy; the blocks' rows are undefined until the caller
 * rewrites them (pa_append_kv into the slots of positions 0..L-1, which the
 * new table gives), as after a recomputation. */
pa_status pa_swap_in(pa_pool* pool, int32_t req_id, const void* d_image, size_t image_bytes,
                     void* stream);

/* ---- device calls: enqueue on stream, asynchronous ------------------------ */

/* Copy-on-write copies: for each of the n pairs d_pairs[i] = {src, dst}
 * (device int32[n][2]), block dst takes block src's rows in every layer, K and
 * V.  No dst may be a src of another pair (pa_reserve never makes such pairs).
 * Paged only.  n == 0 is a no-op. */
pa_status pa_copy_blocks(pa_pool* pool, const int32_t* d_pairs, int32_t n, void* stream);

/* KV append ([KVP] Observation-1): for i < n with d_slots[i] >= 0, write token
 * i's rows d_k[i][h][:] and d_v[i][h][:] (device, [n][num_kv_heads][head_dim],
 * kv_dtype, 16-byte aligned) into slot d_slots[i] of layer `layer`, for every
 * KV head.  A bit copy: no rounding.  Negative slots are skipped.  Slots in
 * one call must be distinct. */
pa_status pa_append_kv(pa_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                       const int32_t* d_slots, int32_t n, void* stream);

/* Context partition pa_decode uses for these sizes (partition_tokens 0 =
 * the library's choice), in tokens: a multiple of 16 and of block_size.
 * Returns 0 for invalid arguments. */
int32_t pa_decode_partition_tokens(const pa_pool* pool, int32_t num_seqs, int32_t max_context,
                                   int32_t partition_tokens);

/* Workspace bytes pa_decode needs (0 when one partition covers max_context). */
size_t pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_context, int32_t partition_tokens);

/* Single-token decode attention over the cache ([PAS] Summary, [ROC] paging
 * paragraph and Terms: attention reads K and V through the block table).
 * For each sequence s < num_seqs and query head h (KV head h / G, G =
 * num_q_heads / num_kv_heads):
 *     out[s][h][:] = sum_t w_t V_s[t],  w = softmax_t(scale * <q[s][h], K_s[t]>)
 * over the L_s = d_context_lens[s] tokens of sequence s (L_s = 0 gives zeros).
 *   d_q:            device [num_seqs][num_q_heads][head_dim], q_dtype (must
 *                   equal kv_dtype); 16-byte aligned.
 *   d_block_tables: paged: device int32 [num_seqs][table_stride], entry j the
 *                   physical block of tokens j*BS..; contiguous: ignored.
 *   d_req_ids:      contiguous: device int32 [num_seqs] request ids, or NULL
 *                   for "request id = s"; paged: ignored.
 *   d_context_lens: device int32 [num_seqs], each in [0, max_context].
 *   max_context:    bound on the lengths; sizes the launch.
 *   d_out:          device fp32 [num_seqs][num_q_heads][head_dim].
 *   d_workspace:    device scratch of >= pa_decode_workspace_bytes(...) bytes
 *                   (may be NULL when that is 0): the partitions' partial
 *                   results and, before them in time, the launch's work plan
 *                   (which partitions hold tokens, longest first); written
 *                   and read within the call.
 *   partition_tokens: context tokens per workgroup, 0 = the library's choice,
 *                   else a multiple of 16 and of block_size; contexts longer
 *                   than one partition are split and merged (split-K).
 * Softmax is computed online in fp32 per context partition; partitions are
 * merged in a fixed order, so results depend only on logical positions, never
 * on which physical blocks hold them.  bf16 caches weight V with each softmax
 * weight split into two bf16 parts (relative error below 2^-16 per weight).
 * K and V are read with non-temporal loads while no block of the pool is
 * shared, with cached loads otherwise.  Supported: G <= 16, head_dim 64/128.
 * The workspace serves one call at a time. */
pa_status pa_decode(pa_pool* pool, int32_t layer, const void* d_q, pa_dtype q_dtype,
                    int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                    int32_t table_stride, const int32_t* d_req_ids,
                    const int32_t* d_context_lens, int32_t num_seqs, int32_t max_context,
                    int32_t partition_tokens, float* d_out, void* d_workspace,
                    size_t workspace_bytes, void* stream);

/* One decode step of a layer in one launch: pa_append_kv of each sequence's
 * new token, then pa_decode over contexts that end with it ([KVP]
 * Observation-1: every running request grows by one token per iteration).
 *   d_k, d_v:   device [num_seqs][num_kv_heads][head_dim], kv_dtype, 16-byte
 *               aligned: the new token of sequence s.
 *   d_slots:    device int32 [num_seqs]: slot of sequence s's new token, as
 *               pa_reserve handed it out, i.e. the slot of position L_s - 1;
 *               < 0: sequence s appends nothing (its cache is read as is).
 * The other arguments, the result and the errors are those of pa_decode.  The
 * cache afterwards equals pa_append_kv's; the output equals pa_decode's after
 * that append, bit for bit.  With blocks of 16 or more tokens the launch
 * stores whole 32-byte sectors: it rewrites the 16 token rows around each new
 * token (every other row with the bytes it read from it earlier in the same
 * launch), so nothing else may write those rows while the launch runs. */
pa_status pa_append_decode(pa_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                           const int32_t* d_slots, const void* d_q, pa_dtype q_dtype,
                           int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                           int32_t table_stride, const int32_t* d_req_ids,
                           const int32_t* d_context_lens, int32_t num_seqs, int32_t max_context,
                           int32_t partition_tokens, float* d_out, void* d_workspace,
                           size_t workspace_bytes, void* stream);

/* Work plan of a split decode, made once for a decode iteration and used by
 * every layer's pa_decode_planned / pa_append_decode_planned of that
 * iteration ([KVP] Observation-1: an iteration advances each running request
 * by one token, so all its layers attend the same context lengths; one block
 * table serves every layer).  Arguments as pa_decode's, same meaning.  A
 * launch with these sizes runs from a plan when its contexts are split into
 * partitions and its grid holds at least 2048 workgroups; for such a launch
 * the call enqueues the plan into its place in d_workspace (after the
 * partials) and sets *planned_out (may be NULL) to 1, for any other launch it
 * enqueues nothing and sets 0.  The plan depends only on the values of
 * d_context_lens, num_seqs, num_q_heads, max_context and partition_tokens.
 * Errors: as pa_decode (PA_ERR_WORKSPACE when d_workspace is too small for a
 * launch that uses a plan). */
pa_status pa_decode_plan(pa_pool* pool, const int32_t* d_context_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t max_context, int32_t partition_tokens,
                         void* d_workspace, size_t workspace_bytes, int32_t* planned_out, void* stream);

/* pa_decode and pa_append_decode without their own plan: they read the plan
 * that pa_decode_plan left in d_workspace, for the same context length values,
 * num_seqs, num_q_heads, max_context and partition_tokens (so one plan serves
 * all layers of an iteration; nothing else may write the workspace between
 * the plan and its last use; pa_decode / pa_append_decode with those same
 * arguments write an equivalent plan in its place).  Launches that use no plan run exactly as
 * pa_decode / pa_append_decode.  Arguments, results (bit for bit) and errors
 * are theirs.  A plan made for other values gives wrong outputs (and, with
 * the append, wrong bytes in the rows the append rewrites); its items are
 * range-checked, so the call still reads and writes only memory that a
 * correct call with these arguments may. */
pa_status pa_decode_planned(pa_pool* pool, int32_t layer, const void* d_q, pa_dtype q_dtype,
                            int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                            int32_t table_stride, const int32_t* d_req_ids,
                            const int32_t* d_context_lens, int32_t num_seqs, int32_t max_context,
                            int32_t partition_tokens, float* d_out, void* d_workspace,
                            size_t workspace_bytes, void* stream);
pa_status pa_append_decode_planned(pa_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                                   const int32_t* d_slots, const void* d_q, pa_dtype q_dtype,
                                   int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                                   int32_t table_stride, const int32_t* d_req_ids,
                                   const int32_t* d_context_lens, int32_t num_seqs,
                                   int32_t max_context, int32_t partition_tokens, float* d_out,
                                   void* d_workspace, size_t workspace_bytes, void* stream);

/* pa_append_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace; the split-K partials
 * and the work plan go to a device array the library holds, 64 MiB
 * (PA_NOALLOC_SCRATCH_BYTES) on each GPU it runs on, until the process ends.
 * Calls whose pa_decode_workspace_bytes(...) exceeds that fail with
 * PA_ERR_WORKSPACE before anything is launched.  The call allocates nothing:
 * no hipMalloc, no hipFree; its first call on a device looks up the array's
 * address there.  The array keeps the last call's contents; every byte a call
 * reads from it, the same call wrote first, so nothing needs clearing.  All
 * calls on one GPU share the array: calls that may overlap (other streams,
 * other threads) race and must be ordered by the caller.  Result and cache
 * bytes are pa_append_decode's, bit for bit. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status pa_append_decode_noalloc(pa_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                                   const int32_t* d_slots, const void* d_q, pa_dtype q_dtype,
                                   int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                                   int32_t table_stride, const int32_t* d_req_ids,
                                   const int32_t* d_context_lens, int32_t num_seqs,
                                   int32_t max_context, int32_t partition_tokens, float* d_out,
                                   void* stream);

/* ---- host-side checks of the device arrays (debugging aids) ---------------
 * The device calls trust their device arrays (see Validation above): an entry
 * out of range makes a kernel read or write outside the cache.  These calls
 * take HOST copies of those arrays and check them against the pool, on the
 * CPU; they launch nothing and change nothing.  PA_OK, or PA_ERR_INVALID_ARG
 * with the first offending entry in pa_last_error(). */

/* The arrays of a pa_decode / pa_append_decode call (same meaning, same
 * num_seqs and max_context; host int32):
 *   h_context_lens[s] in [0, max_context], max_context <= max_seq_len;
 *   paged: table_stride >= ceil(max_context / block_size) and entries j <
 *     ceil(L_s / block_size) of row s of h_block_tables are blocks of the
 *     pool ([ROC] Terms: the table maps a sequence's logical blocks to
 *     physical ones);
 *   contiguous: request ids (h_req_ids[s], or s if NULL) in [0, max_seqs),
 *     and for a demand-paged pool the first ceil(L_s / block_size) blocks of
 *     each request mapped;
 *   h_slots (NULL: no append): each slot >= 0 is the slot of position L_s - 1
 *     (L_s >= 1) and no two sequences append to the same slot. */
pa_status pa_check_decode_args(const pa_pool* pool, const int32_t* h_block_tables,
                               int32_t table_stride, const int32_t* h_req_ids,
                               const int32_t* h_context_lens, const int32_t* h_slots,
                               int32_t num_seqs, int32_t max_context);

/* The slots of a pa_append_kv call: each slot >= 0 names a row of the pool
 * (of a mapped page, for a demand-paged pool) and no slot appears twice. */
pa_status pa_check_slots(const pa_pool* pool, const int32_t* h_slots, int32_t n);

/* The pairs of a pa_copy_blocks call: both blocks of every pair belong to the
 * pool and differ, no block is the destination of two pairs, and no
 * destination is also a source ([PAS] Summary: a shared block is copied
 * before a sharer writes into it).  Paged only. */
pa_status pa_check_block_pairs(const pa_pool* pool, const int32_t* h_pairs, int32_t n);

/* The shared prefixes of a pa_decode_shared / pa_append_decode_shared call
 * (host int32 [num_seqs], with the lengths and, for the fused call, the
 * slots): each a multiple of partition_tokens within its context, and no
 * appending sequence's new token inside its shared prefix. */
pa_status pa_check_shared_args(const pa_pool* pool, const int32_t* h_seq_shared,
                               const int32_t* h_context_lens, const int32_t* h_slots, int32_t num_seqs,
                               int32_t partition_tokens);

/* Message of the calling thread's last error ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
