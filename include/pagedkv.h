/*
 * pagedkv.h -- C ABI of libpagedkv.so: paged-KV decode on MI355X (gfx950).
 *
 * The library implements the hot path of paged KV-cache decoding as the
 * reference pages describe it:
 *   - a host-side block manager (refcounts, chained prefix hashes, an LRU
 *     evictable pool, all-or-nothing allocate/append, reverse-order free,
 *     fork and copy-on-write append);
 *   - pa_write_kv: scatter new tokens' K/V into their slots;
 *   - pa_copy_blocks: the copy-on-write block copy;
 *   - pa_swap_out / pa_swap_in: whole blocks of every layer to and from
 *     pinned host memory when a sequence is preempted and resumed;
 *   - pa_decode: attention of one query token per sequence over K/V that
 *     live in fixed-size blocks scattered through HBM, found through the
 *     sequence's block table, with split-KV partitions and a final reduce;
 *     pa_decode_shared reads blocks shared by several sequences once;
 *   - pa_write_decode / pa_write_decode_shared: each sequence's new token
 *     written and the decode over it, in one call;
 *   - pa_prefill: causal attention of prompts' uncached suffixes;
 *   - pa_sched_*: a continuous-batching scheduler over the block manager.
 *
 * Pages cited:
 *   [A130]  "qaqbuyan.com article 130" (vLLM PagedAttention walk-through):
 *           KV-cache and block-size formulas, BlockTable, paged_attention
 *           pseudocode, BlockAllocator, continuous-batching scheduler
 *           (_preempt_request), paged_attention_kernel listing.
 *   [D31]   "day31" (blog.ans20xx.com): toy block allocator, toy COW append
 *           (fork_sequence / ensure_private_last_block / append_with_cow).
 *   [P06]   "P06 · BlockManager: paged KV + prefix cache" (kuanzhou.online
 *           nano-vllm-omni drills): spec overview, operations table,
 *           invariants I1-I5, pitfalls, Examples 1-3, details, data-structure
 *           table, algorithm notes, eviction trace.
 *
 * Conventions for every call:
 *   - Every call returns a pa_status (0 = PA_OK) unless documented otherwise.
 *     On any error nothing is modified and no kernel is launched; a
 *     human-readable detail is available from pa_last_error() on the same
 *     thread.
 *   - The library never allocates device memory and never synchronizes a
 *     stream.  Device buffers are owned by the caller.  `stream` is a
 *     hipStream_t passed as void* (NULL = the null stream); device calls are
 *     asynchronous on it.
 *   - The KV cache of one layer is two arrays (K and V), each laid out
 *     [num_blocks][block_size][num_kv_heads][head_dim] in the element type
 *     `dtype`, densely packed ([A130] paged_attention pseudocode and kernel
 *     listing).  One physical block id names the same block in every layer
 *     ([A130] block-size formula: a block's bytes span all layers).
 *   - Token position `pos` of a sequence lives in flat slot
 *     table[pos / block_size] * block_size + pos % block_size ([P06] spec
 *     overview).
 *   - Block-manager calls on one pa_bm are serialized by an internal mutex.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum pa_status {
  PA_OK = 0,
  PA_ERR_OUT_OF_BLOCKS = 1, /* [P06] OutOfBlocks: nothing free or evictable */
  PA_ERR_INVALID = 2,       /* bad argument, unknown/duplicate sequence id  */
  PA_ERR_UNSUPPORTED = 3,   /* valid but not implemented (dtype, head_dim)  */
  PA_ERR_DEVICE = 4         /* a HIP runtime call failed                    */
};

/* Element types of Q and of the KV cache. */
enum pa_dtype { PA_DTYPE_F32 = 0, PA_DTYPE_F16 = 1, PA_DTYPE_BF16 = 2 };

/* Static name of a status code ("PA_OK", ...). */
const char* pa_status_str(int status);
/* Detail of the last error raised on the calling thread ("" if none). The
 * pointer stays valid until the next library call on this thread. */
const char* pa_last_error(void);

/* ==== host block manager ================================================
 * [P06] data-structure table, operations table and algorithm notes, with
 * [D31] fork and copy-on-write append.  Semantics:
 *   - free list: FIFO, initially 0..num_blocks-1 ([P06] Example 1);
 *   - a full block is identified by h_i = H(h_{i-1}, tokens of block i),
 *     h_{-1} a fixed sentinel; H is a 64-bit splitmix64-based chain and a
 *     hit also verifies the stored parent hash and tokens, so a false hit
 *     needs a 64-bit collision of whole prefixes;
 *   - allocate matches at most (len-1)/block_size leading blocks,
 *     contiguously from block 0, stopping at the first miss;
 *   - free walks the table in reverse; a block reaching ref 0 goes to the
 *     newest end of the evictable pool if it carries a hash, else to the
 *     free list;
 *   - taking a block: free list first, else evict the oldest evictable block
 *     and drop its registration (the hash->block entry only if it points at
 *     that block);
 *   - num_free_blocks = free + evictable.
 */
typedef struct pa_bm pa_bm;

/* Create a manager for `num_blocks` blocks of `block_size` tokens.  Prefix
 * caching on iff enable_prefix_cache != 0 ([P06] details: off means nothing
 * is hashed, every freed block returns to the free list, cached is 0).
 * Returns NULL (with pa_last_error set) if num_blocks <= 0 or
 * block_size <= 0.  Owned by the caller; release with pa_bm_destroy. */
pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t enable_prefix_cache);
void pa_bm_destroy(pa_bm* bm);

/* [P06] operations table, allocate row.  Admit sequence `seq` with prompt
 * tokens[0..n).  Matches cached prefix blocks, checks capacity exactly
 * (new blocks needed <= num_free_blocks - hits that sit in the evictable
 * pool) before any change, revives hits, takes new blocks in logical order,
 * registers the full blocks and records the sequence.  On success writes
 * the ceil(n/block_size) physical ids to table_out[0..] (if table_out is
 * not NULL) and their count to *nblocks_out (if not NULL).
 * Errors: PA_ERR_OUT_OF_BLOCKS (state unchanged); PA_ERR_INVALID if `seq`
 * exists, n < 0, tokens is NULL with n > 0, or table_out is given with
 * cap < ceil(n/block_size).  n == 0 is allowed (empty table). */
int pa_bm_allocate(pa_bm* bm, int64_t seq, const int32_t* tokens, int32_t n,
                   int32_t* table_out, int32_t cap, int32_t* nblocks_out);

/* [P06] operations table, append_slot row, with [D31] copy-on-write.
 * pos = current length.  If pos/block_size == table length, a new block is
 * taken; otherwise, if the last block is shared (ref > 1), a new block is
 * taken, the old one decref'd and replaced in the table, and the pair
 * (old, new) is reported in *cow_src_out and *cow_dst_out (both -1 when no copy
 * is needed) -- the caller must copy that block (pa_copy_blocks) before
 * writing the token.  Then the token is appended; if the block just became
 * full and prefix caching is on it is hashed with the chain tail as parent
 * and registered.  *slot_out receives the token's flat slot.
 * Errors: PA_ERR_OUT_OF_BLOCKS at the take-block step (state unchanged);
 * PA_ERR_INVALID for an unknown seq.  Output pointers may be NULL. */
int pa_bm_append_slot(pa_bm* bm, int64_t seq, int32_t token, int64_t* slot_out,
                      int32_t* cow_src_out, int32_t* cow_dst_out);

/* pa_bm_append_slot for seqs[0..B) with tokens[0..B), in order.  slots_out
 * [B] receives each slot; cow_pairs_out [B][2] receives the copy pairs
 * packed from the front, their count in *n_cow_out.  Stops at the first
 * failing append and returns its status; *n_done_out (if not NULL) is the
 * number of appends completed, which stay done. */
int pa_bm_append_slots(pa_bm* bm, const int64_t* seqs, const int32_t* tokens, int32_t B,
                       int64_t* slots_out, int32_t* cow_pairs_out, int32_t* n_cow_out,
                       int32_t* n_done_out);

/* [D31] fork_sequence: `child` gets a copy of the parent's table, tokens,
 * hash chain and cached count; every block's ref is incremented.  Never
 * needs a block.  PA_ERR_INVALID if parent is unknown or child exists. */
int pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child);

/* pa_bm_fork(parents[i], children[i]) for i in [0, n), in order, under one
 * lock (beam search forks every beam each step).  Stops at the first
 * failing fork and returns its status; *n_done_out (if not NULL) is the
 * number of forks done, which stay done. */
int pa_bm_fork_batch(pa_bm* bm, const int64_t* parents, const int64_t* children, int32_t n,
                     int32_t* n_done_out);

/* pa_bm_free of seqs[0..n) in order, under one lock.  Never fails on ids. */
int pa_bm_free_batch(pa_bm* bm, const int64_t* seqs, int32_t n);

/* [P06] operations table, free row: reverse walk, ref-1, blocks at 0 to the
 * evictable pool (hashed) or free list (not hashed); the sequence's records
 * are dropped.  Never fails; an unknown seq is a no-op returning PA_OK. */
int pa_bm_free(pa_bm* bm, int64_t seq);

/* Preemption ([A130] continuous-batching scheduler, _preempt_request: the
 * victim's KV goes to CPU memory and its blocks are freed).  Copies the
 * table of `seq` (logical order) into table_out[0..cap), *nblocks_out = its
 * length, then frees the blocks exactly as pa_bm_free does; the sequence
 * keeps only its tokens and is "swapped out".  The caller copies those
 * blocks' bytes to host memory (pa_swap_out) before any later write into
 * them -- on the same stream, stream order guarantees that.
 * PA_ERR_INVALID for an unknown seq or a too small table_out (nothing
 * changed).  A swapped-out id cannot be allocated or forked onto;
 * pa_bm_free drops it. */
int pa_bm_swap_out(pa_bm* bm, int64_t seq, int32_t* table_out, int32_t cap, int32_t* nblocks_out);

/* Resume a swapped-out sequence: the [P06] allocate over its saved tokens
 * (the pages show no swap-in; this is the reading used).  Full prefix
 * blocks still registered come back as hits -- their KV never left the
 * GPU -- so only logical blocks first_restore.. need their host copy
 * (pa_swap_in into table[first_restore..]).  *first_restore_out = number of
 * hit blocks = num_cached_tokens / block_size.  All or nothing:
 * PA_ERR_OUT_OF_BLOCKS leaves every state unchanged and the sequence still
 * swapped out.  PA_ERR_INVALID if seq is not swapped out or cap is too
 * small. */
int pa_bm_swap_in(pa_bm* bm, int64_t seq, int32_t* table_out, int32_t cap, int32_t* nblocks_out,
                  int32_t* first_restore_out);

/* 1 if seq is swapped out, 0 if not, -1 if bm is NULL. */
int32_t pa_bm_is_swapped(const pa_bm* bm, int64_t seq);

/* Swapped-out sequences in ascending id order: seqs_out[0..*n_out) and
 * their lengths lens_out[0..*n_out).  With both arrays NULL only *n_out is
 * set.  PA_ERR_INVALID if cap is too small (nothing written). */
int pa_bm_swapped(const pa_bm* bm, int64_t* seqs_out, int32_t* lens_out, int32_t cap,
                  int32_t* n_out);

/* Flat slot of token `pos` (0 <= pos < len) of `seq` ([P06] spec overview).
 * PA_ERR_INVALID for an unknown seq or pos out of range. */
int pa_bm_slot(const pa_bm* bm, int64_t seq, int32_t pos, int64_t* slot_out);
/* The manager's block size and pool size; -1 if bm is NULL. */
int32_t pa_bm_block_size(const pa_bm* bm);
int32_t pa_bm_num_blocks(const pa_bm* bm);
/* Free + evictable block count; -1 if bm is NULL. */
int32_t pa_bm_num_free_blocks(const pa_bm* bm);
/* [P06] details: coarse check ceil(n_tokens/block_size) <= num_free_blocks
 * (ignores prefix hits).  Returns 1 or 0 (0 also for bad arguments). */
int32_t pa_bm_can_allocate(const pa_bm* bm, int32_t n_tokens);
/* Tokens of `seq` served from the prefix cache at allocate (hits * bs). */
int pa_bm_num_cached_tokens(const pa_bm* bm, int64_t seq, int32_t* out);
/* Current length (tokens) of `seq`. */
int pa_bm_seq_len(const pa_bm* bm, int64_t seq, int32_t* out);
/* Copy the block table of `seq` into out[0..cap); *n_out = its length.
 * PA_ERR_INVALID if unknown or cap is too small (nothing written). */
int pa_bm_get_table(const pa_bm* bm, int64_t seq, int32_t* out, int32_t cap, int32_t* n_out);
/* Number of live sequences; -1 if bm is NULL. */
int32_t pa_bm_num_seqs(const pa_bm* bm);
/* Ids of the live sequences in ascending order into out[0..cap); *n_out =
 * their count.  PA_ERR_INVALID if cap is too small (nothing written). */
int pa_bm_seq_ids(const pa_bm* bm, int64_t* out, int32_t cap, int32_t* n_out);

/* Export the decode inputs for seqs[0..B): tables_out is a row-major
 * [B][max_blocks] int32 host array, each row the sequence's table padded
 * with pad_block; context_lens_out [B] gets each length.  PA_ERR_INVALID if
 * a seq is unknown or its table is longer than max_blocks (nothing
 * written).  The caller uploads both arrays to the device. */
int pa_bm_export_batch(const pa_bm* bm, const int64_t* seqs, int32_t B, int32_t* tables_out,
                       int32_t max_blocks, int32_t pad_block, int32_t* context_lens_out);

/* Check [P06] invariants I1-I5 (plus tight tables).  PA_OK, or
 * PA_ERR_INVALID with the violated invariant in pa_last_error(). */
int pa_bm_check_invariants(const pa_bm* bm);
/* Observable state: ref[num_blocks], has_hash[num_blocks] (1 if a hash is
 * registered on the block), the free list front to back in
 * free_order[0..*n_free) and the evictable pool oldest to newest in
 * evict_order[0..*n_evict).  Each array must hold num_blocks entries; any
 * pointer may be NULL to skip that output. */
int pa_bm_dump(const pa_bm* bm, int32_t* ref, int8_t* has_hash, int32_t* free_order,
               int32_t* n_free, int32_t* evict_order, int32_t* n_evict);

/* ==== continuous-batching scheduler (host) =============================== */

/* [A130] continuous-batching section: the step timeline and the scheduler's
 * step (finish, admit first come first served, run, append; when an append
 * finds no block, _preempt_request takes the running request with the most
 * generated tokens).  It drives a pa_bm (which must outlive it and is used
 * for nothing else while the scheduler runs) and only decides; the caller
 * does each step's device work from the plan.
 * Readings where the page stops short:
 *   - the admitting step runs the prompt and yields the first token; each
 *     later step appends the previous token and decodes the next one; a
 *     request whose budget is met leaves at the next step;
 *   - preempted requests resume before new admissions, oldest first;
 *   - appends run in running order over the list as it stood when they
 *     began, skipping requests preempted meanwhile; when one finds no
 *     block, the victim is the request with the most generated tokens
 *     among ALL running requests (ties to the earliest in running order),
 *     whether or not it appended or was admitted in this step, and the
 *     failing request retries until it succeeds or is the victim itself;
 *   - nothing is undone: a victim that already appended keeps its token
 *     (its K/V is written before its blocks are copied out) and is not
 *     decoded in this step; a request whose last token is cached but not
 *     yet decoded joins a later step's decode batch without appending;
 *   - host swap space is a FIFO pool of `host_slots` block records
 *     (pa_swap_out's record layout); a victim that does not fit there is
 *     recomputed: freed and put back at the front of the waiting queue with
 *     every token it produced or appended as its prompt.
 * Device order of a step: swap-in copies (pa_swap_in); prompt K/V writes
 * (and the prompts' attention, pa_prefill); then, for each preemption k in
 * order, the copy-on-write copies (pa_copy_blocks) and K/V writes
 * (pa_write_kv) of the appends made before it that no earlier preemption
 * covered, followed by its swap-out copies (pa_swap_out); then the rest of
 * the copies and writes; then decode of the batch.  A preemption can free
 * blocks that later appends of the same step take again, and a victim's
 * own write must reach its blocks before they are copied out: this order
 * satisfies both. */
typedef struct pa_sched pa_sched;

/* One step's plan, in caller-owned host arrays.  Capacities (checked
 * before the step starts, so a step never stops half done): every id
 * array, writes, slots, batch, prefill_counts, cow_pairs (pairs) and cuts
 * (triples) hold ids_cap >= max_batch entries; swap_in / swap_out hold
 * pairs_cap >= host_slots pairs; prefill_slots holds prefill_cap >=
 * num_blocks * block_size entries.  pa_sched_step fills the n_* counts. */
typedef struct pa_sched_plan {
  int32_t ids_cap, pairs_cap, prefill_cap;
  int64_t* finished;    int32_t n_finished;    /* left at this step */
  int64_t* resumed;     int32_t n_resumed;     /* swapped in */
  int64_t* admitted;    int32_t n_admitted;    /* prompt runs this step */
  int64_t* preempted;   int32_t n_preempted;   /* swapped out or recomputed, in order */
  int64_t* recomputed;  int32_t n_recomputed;  /* the preempted ones sent back to waiting */
  int32_t* swap_in;     int32_t n_swap_in;     /* [n][2] (host record, block) */
  int32_t* swap_out;    int32_t n_swap_out;    /* [n][2] (block, host record) */
  int64_t* prefill_slots; int32_t n_prefill_slots;  /* uncached prompt tokens' slots */
  int32_t* prefill_counts;                     /* [n_admitted] slots per admitted request */
  int64_t* writes;      int64_t* slots;  int32_t n_writes;  /* appends: K/V to write at slots */
  int32_t* cow_pairs;   int32_t n_cow;         /* [n][2] (src, dst) */
  int32_t* cuts;        /* [n_preempted][3]: writes and cow pairs made before
                           preemption k, swap-out pairs through it */
  int64_t* batch;       int32_t n_batch;       /* decode batch, running order */
} pa_sched_plan;

/* NULL on bad arguments (max_batch > 0, host_slots >= 0). */
pa_sched* pa_sched_create(pa_bm* bm, int32_t max_batch, int32_t host_slots);
/* Frees the scheduler only; blocks its requests hold stay in the manager. */
void pa_sched_destroy(pa_sched* s);
/* Queue a request (id unused by the scheduler and the manager, n >= 1
 * prompt tokens, max_new_tokens >= 1). */
int pa_sched_add_request(pa_sched* s, int64_t id, const int32_t* prompt, int32_t n,
                         int32_t max_new_tokens);
/* Run one step's decisions and fill the plan.  PA_ERR_INVALID if the
 * previous step was not committed or the plan is too small. */
int pa_sched_step(pa_sched* s, pa_sched_plan* plan);
/* Tokens produced by the step just planned: exactly one for each request
 * in its decode batch and each one it admitted that is still running (any
 * order).  PA_ERR_INVALID (nothing changed) otherwise. */
int pa_sched_commit(pa_sched* s, const int64_t* ids, const int32_t* tokens, int32_t n);
/* State queries (arrays NULL = count only; PA_ERR_INVALID if too small):
 * running requests in batch order with their generated counts; waiting
 * ids front to back; swapped ids oldest first with their host records
 * (num_records[i] each, concatenated); free host records front to back. */
int pa_sched_running(pa_sched* s, int64_t* ids, int32_t* generated, int32_t cap, int32_t* n_out);
int pa_sched_waiting(pa_sched* s, int64_t* ids, int32_t cap, int32_t* n_out);
int pa_sched_swapped(pa_sched* s, int64_t* ids, int32_t* num_records, int32_t cap,
                     int32_t* records, int32_t records_cap, int32_t* n_out);
int pa_sched_host_free(pa_sched* s, int32_t* records, int32_t cap, int32_t* n_out);

/* ==== device operations (gfx950) ========================================= */

/* Paged KV write.  For t in [0, T): copy the row k_new[t] (num_kv_heads *
 * head_dim elements) into K at flat slot s = slot_mapping[t], i.e.
 * k_cache[s / block_size][s % block_size][:][:], and likewise v_new into V
 * ([A130] KV-cache section: each step appends the new token's K and V;
 * [D31]: it goes into the last, partly filled block).  Bitwise copy.
 * k_new/v_new: device, [T][num_kv_heads][head_dim] in `dtype`.
 * slot_mapping: device int64 [T].  A slot outside
 * [0, num_blocks*block_size) is skipped (e.g. -1 for padding).
 * Precondition: valid slots are unique (otherwise which row lands is
 * unspecified).  T == 0 launches nothing. */
int pa_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                const int64_t* slot_mapping, int32_t T, int32_t num_blocks, int32_t block_size,
                int32_t num_kv_heads, int32_t head_dim, int32_t dtype, void* stream);

/* Copy-on-write block copy ([D31] toy COW append: the new private block
 * receives the old block's KV bytes).  For every layer l < num_layers and
 * every pair p < num_pairs: K_l[dst] = K_l[src] and V_l[dst] = V_l[src],
 * whole blocks of `block_bytes` bytes (= block_size * num_kv_heads *
 * head_dim * element size).  k_caches/v_caches: HOST arrays of num_layers
 * device pointers.  pairs: device int32 [num_pairs][2] = (src, dst).
 * A pair with an id outside [0, num_blocks) is skipped.  Preconditions:
 * destinations are distinct and none is also a source.  block_bytes must be
 * a positive multiple of 16 and every cache pointer 16-byte aligned. */
int pa_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                   int64_t block_bytes, int32_t num_blocks, const int32_t* pairs,
                   int32_t num_pairs, void* stream);

/* Preemption copy to host memory ([A130] continuous-batching scheduler,
 * _preempt_request: each of the victim's blocks is copied to CPU memory).
 * The host buffer is an array of records of R = num_layers * 2 *
 * block_bytes bytes; a record holds one block of every layer, layer l's K
 * at byte (2l) * block_bytes and its V at (2l + 1) * block_bytes.  For
 * list entry i < n with b = blocks[i], record r = host_slots[i] (or r = i
 * when host_slots is NULL) receives K_l[b] and V_l[b] for every layer l.
 *   k_caches/v_caches: HOST arrays of num_layers device pointers (the
 *     per-layer caches, layout above).
 *   blocks: device int32 [n]; host_slots: device int32 [n] or NULL.  An
 *     entry whose block is outside [0, num_blocks) or whose record is
 *     outside the buffer is skipped (its record is left untouched).
 *   host_dst: pinned host memory from hipHostMalloc (torch pin_memory) of
 *     host_bytes bytes (floor(host_bytes / R) records; without host_slots
 *     at least n of them); the GPU writes it directly over the host link.
 * Errors (nothing launched): PA_ERR_INVALID if host_dst is not host memory
 * that HIP maps for the device (checked at both ends of the records), if
 * it holds too few records, or for bad sizes / misalignment (block_bytes a
 * positive multiple of 16; caches and host_dst 16-byte aligned).
 * Asynchronous on `stream`: the records are complete once the stream has
 * passed this call (synchronize before reading them on the host). */
int pa_swap_out(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                int64_t block_bytes, int32_t num_blocks, const int32_t* blocks,
                const int32_t* host_slots, int32_t n, void* host_dst, int64_t host_bytes,
                void* stream);

/* The inverse copy: for list entry i < n with b = blocks[i] and every layer
 * l, K_l[b] and V_l[b] receive the record host_slots[i] (or i) laid out as
 * in pa_swap_out.  To resume a sequence, pass table[first_restore..] from
 * pa_bm_swap_in and the records of those logical blocks.  Same arguments,
 * checks and errors as pa_swap_out; destination blocks must be distinct.
 * The host records must stay unchanged until the stream has passed this
 * call. */
int pa_swap_in(void* const* k_caches, void* const* v_caches, int32_t num_layers,
               int64_t block_bytes, int32_t num_blocks, const int32_t* blocks,
               const int32_t* host_slots, int32_t n, const void* host_src, int64_t host_bytes,
               void* stream);

/* Prefill attention of uncached suffixes ([P06] spec overview and
 * key-question answers: after num_cached_tokens prefix hits only the rest
 * of a prompt needs a forward pass; [A130] system-prompt section: a request
 * reuses the shared prompt's blocks and computes what follows).  Sequence
 * b has total length n = context_lens[b] and suffix rows query_start[b] ..
 * query_start[b+1]-1 of q (q_b rows); row i of it sits at position
 * n - q_b + i and attends causally to tokens 0 .. n - q_b + i through the
 * block table, its own K/V already written (pa_write_kv):
 *   out[row][h] = softmax_t(scale * <q[row][h], K[slot(b,t)][g]>) V,
 *   t <= position, g = h / (num_q_heads / num_kv_heads).
 *   out:  device float32 [num_tokens][num_q_heads][head_dim] (written).
 *   q:    device [num_tokens][num_q_heads][head_dim] in `dtype`.
 *   k_cache, v_cache, block_tables, context_lens: as in pa_decode.
 *   query_start: device int32 [B+1], nondecreasing, query_start[B] <=
 *     num_tokens; max_query_len (host) >= every q_b.
 * float16 / bfloat16 only (matrix-core path), head_dim 64 or 128,
 * block_size 16; PA_ERR_UNSUPPORTED otherwise.  A sequence with q_b > n,
 * q_b > max_query_len, n beyond the table, rows outside [0, num_tokens) or
 * any of its first ceil(n / 16) table entries outside the pool gets NaN in
 * all its rows (when its row range is valid); nothing is read or written
 * out of range.  No workspace. */
int pa_prefill(float* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, int32_t max_blocks_per_seq,
               const int32_t* query_start, const int32_t* context_lens, int32_t B,
               int32_t num_tokens, int32_t max_query_len, int32_t num_q_heads,
               int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
               float scale, int32_t dtype, void* stream);

/* Workspace bytes pa_decode needs for these sizes (0 when one partition
 * covers max_context_len, i.e. partition_tokens == 0 or >= max_context_len). */
size_t pa_decode_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_tokens);

/* Paged decode attention ([A130] paged_attention pseudocode: gather the
 * sequence's blocks through its block table, then scaled dot-product
 * attention; kernel listing: layout, float output, scale).  For each
 * sequence b and query head h, with g = h / (num_q_heads / num_kv_heads)
 * and n = context_lens[b]:
 *   s_t = scale * <q[b][h], K[slot(b,t)][g]>,  t < n
 *   out[b][h] = sum_t softmax(s)_t * V[slot(b,t)][g]
 * computed with float32 accumulation as an online softmax over split-KV
 * partitions of `partition_tokens` tokens, combined by a reduce kernel
 * (or, when one workgroup holds all of a sequence's partitions, by that
 * workgroup).
 *   out:  device float32 [B][num_q_heads][head_dim] (written, never read).
 *   q:    device [B][num_q_heads][head_dim] in `dtype`.
 *   k_cache, v_cache: device, one layer, layout above, in `dtype`.
 *   block_tables: device int32 [B][max_blocks_per_seq], every entry
 *     readable: the kernel may read any entry of a row ahead of need
 *     (indices are clamped into the row), but the values past a sequence's
 *     last block are ignored and need not be valid block ids; may be NULL
 *     when max_blocks_per_seq is 0.
 *   context_lens: device int32 [B].
 *   max_context_len: host-side upper bound of context_lens (sizes the grid;
 *     no device-to-host read is made).
 *   partition_tokens: multiple of block_size, or 0 for one partition.
 *   workspace: device, >= pa_decode_workspace_bytes(...) bytes, 16-byte
 *     aligned (may be NULL when that is 0).  Scratch owned by the caller:
 *     its contents on entry do not matter, and it holds partition results
 *     afterwards; calls that overlap on one workspace race.
 * Supported: dtype F32/F16/BF16, head_dim 64 or 128, block_size 16,
 * num_q_heads a multiple of num_kv_heads with group size 1, 2, 4 or 8.
 * Degenerate and invalid inputs: n == 0 gives a zero output row; a
 * sequence with n < 0, n > max_context_len, more than max_blocks_per_seq
 * blocks, or a table entry outside [0, num_blocks) gets NaN output rows
 * (the kernel reads no out-of-range memory).  B == 0 launches nothing. */
int pa_decode(float* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t max_context_len, int32_t B,
              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int32_t num_blocks, float scale, int32_t partition_tokens, int32_t dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/* pa_write_kv of each sequence's new token, then pa_decode, in one call
 * ("qaqbuyan.com article 130", no-cache decode loop: the step computes the
 * new token's K and V, appends them to the cache, then attends over every
 * cached token including it; "P06 · BlockManager" spec overview: the slot
 * of position pos is table[pos / bs] * bs + pos % bs).  For every sequence b
 * with a valid context_lens[b] = n >= 1, the row of position n - 1 (the new
 * token, whose slot was appended before this call) is written from
 * k_new / v_new to that slot of k_cache / v_cache, and the attention is
 * computed as pa_decode computes it after that write: the same output, bit
 * for bit, and the same cache bytes as pa_write_kv followed by pa_decode.
 * The wave that reads a sequence's last block writes the new row there:
 * on the vector path it takes the row from k_new / v_new into its loaded
 * registers; on the matrix-core path (query groups of 4 and 8, 16-bit K/V)
 * it stores the row first, waits for the store, and reads it back.
 *   k_new, v_new: device [B][num_kv_heads][head_dim] in `dtype`, 16-byte
 *     aligned, read only.
 *   k_cache, v_cache: written at the new tokens' slots only.
 * Other arguments, supported shapes, workspace and errors as pa_decode.  A
 * sequence with n == 0 or an invalid length writes nothing; one whose block
 * for position n - 1 is outside [0, num_blocks) writes nothing (and, as in
 * pa_decode, gets NaN rows).  Precondition, as for pa_write_kv: no two
 * sequences' new tokens share a slot (copy-on-write has been done). */
int pa_write_decode(float* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                    const void* v_new, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t max_context_len, int32_t B,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t num_blocks, float scale, int32_t partition_tokens,
                    int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* pa_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, semantics, supported shapes and
 * errors as pa_decode, except that the split-KV partition results go to a
 * scratch array inside the library: a file-scope device array of
 * pa_decode_noalloc_max_bytes() bytes (64 MiB), one per GPU the library
 * runs on, held until the process ends.  The call itself allocates nothing
 * (no hipMalloc, no hipFree); its first call on a device looks up that
 * device's copy of the array once.  Sizes whose workspace
 * (pa_decode_workspace_bytes) exceeds the scratch size are rejected with
 * PA_ERR_INVALID before anything is launched.  The scratch needs no
 * initialisation.  Every call on one GPU shares that GPU's scratch: calls
 * that overlap on one device (on different streams, or from several
 * threads without ordering) race. */
size_t pa_decode_noalloc_max_bytes(void);
int pa_decode_noalloc(float* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t max_context_len, int32_t B,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, float scale,
                      int32_t partition_tokens, int32_t dtype, void* stream);

/* ---- shared-prefix decode ------------------------------------------------
 * Sequences forked from one parent share the parent's blocks ([D31] fork
 * and copy-on-write) and prefix-cache hits share full blocks ([P06] spec
 * overview), so in a batch several block tables can start with the same
 * physical blocks.  pa_decode reads such a block once per sequence;
 * pa_decode_shared reads the shared leading blocks of a group of sequences
 * once for the whole group, then each member's own blocks.  The output is
 * the attention pa_decode defines (same formula, same float32
 * accumulation; partial results are merged in a different order).
 *
 * A plan is two int32 arrays:
 *   seq_group [B]: the group of sequence b, or -1;
 *   groups [n_groups][PA_SHARED_ROW]: row = {S, m_0, ..., m_15}: S shared
 *     leading blocks (S * block_size tokens), then the batch indices of the
 *     members, -1 in unused slots.  At most PA_SHARED_MAX_MEMBERS /
 *     (num_q_heads / num_kv_heads) slots are used.
 * The shared blocks are cut into ceil(S * block_size / partition_tokens)
 * shared partitions from block 0 (the last may be short).  Sequence b is a
 * member of group g when seq_group[b] == g, b is listed in row g, S >= 1,
 * the shared partitions number at most max_shared_parts, and S is below
 * b's block count (its last block is never shared).  A member's first S
 * blocks are read from the table row of m_0 (which need not be a member
 * itself); its other blocks, cut into partitions from block S on, and every
 * sequence that is not a member, as in pa_decode.  A member whose table
 * differs from row m_0 inside the shared blocks, or a group whose m_0 is
 * outside [0, B), gives NaN output rows for those members (nothing is read
 * out of range). */
#define PA_SHARED_MAX_MEMBERS 16
#define PA_SHARED_ROW (1 + PA_SHARED_MAX_MEMBERS)

/* A plan for pa_decode_shared from the host copies of the batch's tables
 * and lengths.  Candidates are sequences with at least 2 full blocks
 * before their last block.  They are bucketed by first block id and sorted
 * by table row; a bucket is cut greedily into groups of at most
 * PA_SHARED_MAX_MEMBERS / query_group sequences, a sequence joining the
 * open group while (members - 1) x shared blocks does not drop; a group's
 * S is the common leading run of its rows (at least 2 blocks).  Groups are
 * written by S, largest first (the decode's shared pass starts its
 * workgroups in group order, so the longest start first).
 *   tables: host int32 [B][max_blocks]; lens: host int32 [B].
 *   partition_tokens: the value pa_decode_shared will get (> 0, multiple of
 *     block_size); query_group: num_q_heads / num_kv_heads (1, 2, 4, 8).
 *   seq_group_out: host int32 [B].
 *   groups_out: host int32 [B / 2][PA_SHARED_ROW] (unused if B < 2).
 *   *n_groups_out: groups written; *max_parts_out: the most shared
 *     partitions of any group (0 if none);
 *   *max_private_parts_out: the most partitions any sequence has after its
 *     group's shared blocks (a sequence in no group: all of its partitions);
 *   *max_private_blocks_out: likewise in blocks (0 for an empty or invalid
 *     length), the hint pa_decode_shared takes as max_private_blocks.
 * Every group it writes satisfies the membership rule above for all its
 * members. */
int pa_shared_plan(const int32_t* tables, int32_t max_blocks, const int32_t* lens, int32_t B,
                   int32_t block_size, int32_t partition_tokens, int32_t query_group,
                   int32_t* seq_group_out, int32_t* groups_out, int32_t* n_groups_out,
                   int32_t* max_parts_out, int32_t* max_private_parts_out,
                   int32_t* max_private_blocks_out);

/* pa_decode with a shared-prefix plan (above).  Arguments as pa_decode,
 * plus:
 *   seq_group: device int32 [B]; groups: device int32
 *     [n_groups][PA_SHARED_ROW]; both may be NULL when n_groups == 0, which
 *     makes the call exactly pa_decode.
 *   max_shared_parts: host-side bound on every group's shared partitions
 *     (sizes the grid; a group with more has no members).
 *   max_private_parts: host-side bound on the partitions any sequence has
 *     after its group's shared blocks (sizes the private grid; 0 = no
 *     bound, the grid then covers max_context_len).  A sequence with more
 *     gets NaN output rows.
 *   max_private_blocks: host-side hint, the most blocks any sequence reads
 *     outside the shared pass (0 = unknown).  It only picks how the private
 *     pass maps waves (up to 8 blocks: four KV heads per workgroup, one per
 *     wave; otherwise one head per workgroup, its blocks split over the
 *     waves); the results are the same either way, whatever its value.
 * With n_groups > 0: dtype F16 or BF16 (the shared partitions run on the
 * matrix cores with up to 16 query columns: members x query group),
 * partition_tokens > 0, and, when max_shared_parts > 0, a workspace of
 * pa_decode_shared_workspace_bytes(...) bytes (a member's partitions can
 * number one more than the plain split).  Otherwise the workspace is the
 * one pa_decode needs. */
size_t pa_decode_shared_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t head_dim,
                                        int32_t max_context_len, int32_t partition_tokens);
int pa_decode_shared(float* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len, int32_t B,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t num_blocks, float scale,
                     int32_t partition_tokens, int32_t dtype, const int32_t* seq_group,
                     const int32_t* groups, int32_t n_groups, int32_t max_shared_parts,
                     int32_t max_private_parts, int32_t max_private_blocks, void* workspace,
                     size_t workspace_bytes, void* stream);

/* pa_write_kv of each sequence's new token, then pa_decode_shared, in one
 * call: pa_write_decode's write ("qaqbuyan.com article 130", no-cache
 * decode loop: append the new K/V, then attend over every cached token)
 * with a shared-prefix plan's decode ("day31", fork and copy-on-write:
 * forked sequences share the parent's blocks).  Arguments as
 * pa_decode_shared, plus k_new / v_new as in pa_write_decode.  A plan
 * never shares a sequence's last block, so the private pass, which reads
 * it, writes the row of position n - 1 there and reads the new row from
 * k_new / v_new; the shared pass reads only blocks before it.  The result
 * is that of pa_write_kv followed by pa_decode_shared: the same cache
 * bytes, and the same output up to rounding in the last bit (the fused
 * kernels are compiled apart from the others, and the compiler may fuse a
 * multiply and an add differently in each).  One exception: a sequence
 * that gets NaN rows because the private grid does not reach its last
 * block (more private partitions than max_private_parts, as for a plan
 * that does not match the tables) is not written.  Otherwise a sequence is
 * written as pa_write_decode writes it. */
int pa_write_decode_shared(float* out, const void* q, void* k_cache, void* v_cache,
                           const void* k_new, const void* v_new, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, int32_t B, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, float scale, int32_t partition_tokens,
                           int32_t dtype, const int32_t* seq_group, const int32_t* groups,
                           int32_t n_groups, int32_t max_shared_parts, int32_t max_private_parts,
                           int32_t max_private_blocks, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ==== measurement helper (gfx950) ========================================
 * Streaming read of `bytes` bytes of device memory at `buf` (both multiples
 * of 16): `workgroups` workgroups each read one contiguous chunk once, with
 * the nontemporal 16-byte buffer loads the decode kernels use.  Used to
 * measure the HBM read rate actually reachable on the GPU, which the decode
 * bandwidth is reported beside.  Nothing is written except, rarely, a
 * checksum into sink[workgroup] (device, >= workgroups uint32 entries),
 * which exists only so the loads are not optimised away.  workgroups in
 * [1, 2^24]; a chunk must stay under 2 GiB.  bytes == 0 launches nothing. */
int pa_stream_read(const void* buf, uint64_t bytes, int32_t workgroups, uint32_t* sink,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
