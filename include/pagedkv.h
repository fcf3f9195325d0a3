/*
 * pagedkv.h -- C ABI of libpagedkv: a block-paged KV cache and PagedAttention
 * decode for AMD Instinct MI355X (gfx950).
 *
 * Sources.  The method is the one described on these pages:
 *   [P5] "PagedAttention por dentro: bloques, tabla de paginas, eviccion y el
 *        estado del arte del KV cache en 2026" (blog.lo0.es/posts/
 *        pagedattention-deep-dive): sections "El modelo de bloques",
 *        "La tabla de paginas (block table)" with its figure, "El pool de
 *        bloques", "Copy-on-write para sampling paralelo", "El kernel CUDA",
 *        "Eviccion y preemption" ("Estrategia 2: swap"), and under "Lo que
 *        vLLM hace hoy": "Chunked prefill integrado con paged KV", "Prefix
 *        caching cross-session", "Sliding window attention".
 *   [P3] "Como funciona realmente vLLM (y por que lo necesitas)"
 *        (alexanderzelada.com): "Que es el mecanismo de atencion",
 *        "PagedAttention: la paginacion del sistema operativo aplicada a la
 *        GPU" and its box "Que guarda cada entrada de la tabla de bloques".
 *   [P1] "KV cache: la memoria de trabajo que sostiene la inferencia LLM"
 *        (blog.lo0.es): "El mecanismo en si", "El precio", "Trucos para que
 *        el cuaderno sea mas fino" (grouped-query attention).
 *
 * Conventions for every call:
 *   - Calls return pkv_status (0 = PKV_OK) and never throw or abort.
 *   - "device" pointers are HIP device memory owned by the caller; the
 *     library only borrows them for the duration of the enqueued work.
 *     "host" pointers are ordinary host memory, read or written before the
 *     call returns.
 *   - Device work is enqueued asynchronously on `stream` (0 = null stream);
 *     the call returns once the kernels are launched.  Launch failures map
 *     to PKV_ERR_HIP.
 *   - The library never allocates device memory.
 *
 * ---------------------------------------------------------------------------
 * Cache layout (the contract between paged_kv_write, paged_kv_copy_blocks and
 * paged_attention_decode).
 *
 * A physical block holds the K and V of 16 consecutive tokens of one sequence
 * for one layer [P5 "El modelo de bloques"].  k_cache and v_cache are two
 * separate device buffers of num_blocks * num_kv_heads tiles each.  The tile
 * of (block b, kv head h) starts at element (b * num_kv_heads + h) * 16 * D,
 * where D = head_dim, so one block of all heads is one contiguous run of
 * num_kv_heads * 16 * D elements.  Inside a tile, the element of token slot t
 * (0..15) and channel d (0..D-1) sits at
 *
 *   K:  (d / 8) * 128 + t * 8 + (d % 8)
 *       -- channel groups of 8: for each group, 16 tokens x 8 channels
 *   V:  (d / 32) * 512 + (t / 4) * 128 + (d % 16) * 8 + ((d / 16) % 2) * 4 + (t % 4)
 *       -- channel groups of 32: for each, 4 token quads, and inside a quad
 *          16 channel columns, each holding 2 channels x 4 tokens
 *
 * (integer division).  D must be a multiple of 32.  Both orders are chosen
 * so that one wavefront reads a whole tile as 64 lanes x 16 contiguous bytes
 * per load instruction and each lane's bytes are already the operand
 * fragment the gfx950 matrix instructions consume; the element type (fp32 or
 * bf16) does not change the order.
 *
 * FP8 cache (PKV_FP8_E4M3, one byte per element, tile of 16 * D bytes).  The
 * codes of bf16 piece j of lane l (in the tile above: the 8 elements from
 * 512 j + 8 l) form an 8-byte piece.  Pieces 2i and 2i + 1 of all 64 lanes
 * fill bytes [1024 i, 1024 i + 1024), lane l's 16 bytes at 1024 i + 16 l, so
 * one 16-byte load per lane reads 1 KiB in order and expands to two bf16
 * operand pieces; a last piece without a partner (D / 32 odd) is stored as
 * 64 lanes x 8 bytes at 1024 i + 8 l.  With
 *   piece(l, j) = 1024 * (j / 2) + (j paired ? 16 : 8) * l + 8 * (j % 2):
 *
 *   K:  piece(16 * ((d / 8) % 4) + t, d / 32) + (d % 8)
 *   V:  piece(16 * (t / 4) + d % 16, d / 32) + ((d / 16) % 2) * 4 + (t % 4)
 *
 * A byte is an OCP FP8 E4M3 code (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits, subnormals m * 2^-9, no infinity, 0x7F/0xFF = NaN, largest
 * finite 448) standing for its value times the tensor's scale (one scale
 * for K, one for V).  ["KV cache: la memoria de trabajo...", «Trucos para
 * que el cuaderno sea más fino»: an 8-bit cache halves its size and the
 * bytes read per step; "PagedAttention por dentro", «Trampas y mitos
 * comunes»: FP8 is described as safe almost always.  The format and the
 * scaling are this library's reading.]
 *
 * Token position p of sequence s (0-based) lives in physical block
 * block_tables[s * max_blocks_per_seq + p / 16] at slot p % 16
 * [P5 "La tabla de paginas": token 200 is found at table position 200/16 = 12].
 * A flat slot index is block * 16 + slot.
 *
 * Other tensors (row-major):
 *   q, out           [num_seqs][num_q_heads][D]; q in the cache dtype, out fp32
 *   k_new, v_new     [num_tokens][num_kv_heads][D] in the cache dtype
 *   slot_mapping     int64 [num_tokens]
 *   block_tables     int32 [num_seqs][max_blocks_per_seq]
 *   context_lens     int32 [num_seqs]
 * Query head h reads kv head h / (num_q_heads / num_kv_heads): query heads
 * share kv heads in contiguous groups [P1 "Trucos ...", grouped-query
 * attention].
 * ---------------------------------------------------------------------------
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_BLOCK_SIZE 16

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID = 1,     /* bad argument, id out of range, double free, ... */
  PKV_ERR_OOM = 2,         /* not enough free blocks (state left unchanged) */
  PKV_ERR_UNSUPPORTED = 3, /* head_dim / dtype / group size without a kernel */
  PKV_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} pkv_status;

typedef enum pkv_dtype {
  PKV_F32 = 0,
  PKV_BF16 = 1,
  PKV_FP8_E4M3 = 2 /* OCP FP8 E4M3 codes with one scale per tensor (see "FP8 cache") */
} pkv_dtype;

typedef struct pkv_pool pkv_pool;

typedef struct pkv_stats {
  int32_t num_blocks;
  int32_t num_free;       /* refcount 0, on the free list */
  int32_t num_used;       /* refcount >= 1 */
  int32_t num_shared;     /* refcount >= 2 */
  int64_t num_refs;       /* sum of refcounts = table entries pointing into the pool */
  double usage_percent;   /* 100 * num_used / num_blocks */
} pkv_stats;

/* Human-readable name of a status code (static storage). */
const char* pkv_status_string(pkv_status status);

/* ===== Host block pool ======================================================
 * [P5 "El pool de bloques"]: one global pool of fixed-size blocks, sized once
 * when the engine starts; allocation is O(1) and a finished sequence returns
 * its blocks, which another sequence may take at the next step [P5 figure in
 * "La tabla de paginas"].  [P5 "Copy-on-write para sampling paralelo"]:
 * sequences share prefix blocks through their tables, with reference counts;
 * a shared block is copied only when a sequence is about to modify it.
 *
 * The free list is a LIFO stack.  With init_order == NULL the first
 * allocations return 0, 1, 2, ...; otherwise they return init_order[0],
 * init_order[1], ... (init_order must be a permutation of 0..num_blocks-1).
 * A block freed last is handed out first.  The pool is host memory owned by
 * the library; it is not thread-safe (one caller at a time).
 */
/* block_size must be 16 (else PKV_ERR_UNSUPPORTED); num_blocks >= 1. */
pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size,
                           const int32_t* init_order /* host, nullable */,
                           pkv_pool** out_pool /* host */);
void pkv_pool_destroy(pkv_pool* pool);

/* Pop n ids (refcount 1 each) into out_ids[0..n).  All or nothing: fewer
 * than n free blocks -> PKV_ERR_OOM with the pool unchanged.  n >= 0. */
pkv_status kv_block_alloc(pkv_pool* pool, int32_t n, int32_t* out_ids /* host */);

/* Add one reference to each id (a sequence forked, or a prefix reused).
 * Any id out of range or free -> PKV_ERR_INVALID, pool unchanged. */
pkv_status kv_block_share(pkv_pool* pool, int32_t n, const int32_t* ids /* host */);

/* Drop one reference from each id; an id whose count reaches 0 is pushed on
 * the free list (in array order).  Validated first: an id out of range, or
 * more drops of one id than it has references -> PKV_ERR_INVALID, pool
 * unchanged. */
pkv_status kv_block_free(pkv_pool* pool, int32_t n, const int32_t* ids /* host */);

/* Make block `id` private to the caller before a write [P5 copy-on-write].
 * refcount 1: *out_id = id, *needs_copy = 0.  refcount > 1: pops a new id
 * (refcount 1), drops one reference of `id`, *out_id = new id,
 * *needs_copy = 1; the caller must copy id -> new id on the device
 * (paged_kv_copy_blocks) before writing into it.  Free or out-of-range id
 * -> PKV_ERR_INVALID; no free block -> PKV_ERR_OOM (pool unchanged). */
pkv_status kv_block_cow(pkv_pool* pool, int32_t id, int32_t* out_id, int32_t* needs_copy);

/* Current reference count of `id` (0 = free). */
pkv_status kv_block_refcount(const pkv_pool* pool, int32_t id, int32_t* out_refcount);

/* Pool occupancy counters: free, used and shared blocks and the share of
 * the pool in use -- the cache-usage figure a serving engine exports for
 * autoscaling ["vLLM en Kubernetes: la pieza de inferencia LLM que si
 * escala", «Autoscaling: HPA estandar no sirve»: the vLLM metric
 * gpu_cache_usage_perc]. */
pkv_status kv_pool_stats(const pkv_pool* pool, pkv_stats* out_stats);

/* Snapshot of the free list, next id to be allocated first.  Writes
 * min(capacity, num_free) ids and the full count to *out_n. */
pkv_status kv_pool_free_list(const pkv_pool* pool, int32_t capacity, int32_t* out_ids,
                             int32_t* out_n);

/* ===== Prefix caching by block hash ==========================================
 * ["Como funciona realmente vLLM", «Automatic Prefix Caching»: instead of
 * dropping a finished request's blocks, the engine indexes them by a hash of
 * their content, and a new request that starts with the same tokens (a
 * shared system prompt or conversation history) reuses those blocks in
 * VRAM without recomputing them; "PagedAttention por dentro", «Prefix
 * caching cross-session»: blocks are hashed, no radix tree.]  Readings:
 *   - only full blocks are indexed; a block's content is its 16 token ids
 *     together with the chain of indexed blocks holding every earlier token
 *     (a block matches only as part of a matching prefix);
 *   - an indexed block whose last reference is dropped stays indexed on a
 *     second free list, least recently freed first; allocations take blocks
 *     holding nothing first (the LIFO stack), then evict the least recently
 *     freed indexed block, which leaves the index together with every block
 *     indexed below it;
 *   - the hash (FNV-1a over the parent id and tokens) only locates
 *     candidates; a hit is confirmed by comparing parent and tokens, so a
 *     match is exact.
 * The free list seen by kv_pool_free_list / kv_pool_stats is the stack
 * (top first) followed by the indexed free blocks (least recent first). */

/* Turns prefix caching on for this pool (idempotent). */
pkv_status pkv_prefix_cache_enable(pkv_pool* pool);

/* The longest run of indexed blocks holding tokens[0 .. 16 k) (k <= number
 * of full blocks of tokens, k <= max_blocks): their ids go to out_ids[0..k)
 * in order and each gains one reference (an indexed free block leaves the
 * free list).  The caller puts them at the head of the new sequence's
 * table with length 16 k and appends the remaining tokens as usual.
 * tokens: host int32 [num_tokens].  Prefix caching off -> PKV_ERR_INVALID. */
pkv_status pkv_prefix_match(pkv_pool* pool, const int32_t* tokens, int32_t num_tokens,
                            int32_t max_blocks, int32_t* out_ids, int32_t* out_num_blocks);

/* Indexes the full blocks of a sequence whose K/V are written: block i
 * (i < num_tokens / 16) is block_ids[i] and holds tokens[16 i .. 16 i + 16).
 * A block already indexed is left as it is (it must hold exactly that
 * content); a block whose content is already indexed under another id is
 * not indexed again (the chain continues through the indexed one).  The
 * blocks must be live and distinct, else PKV_ERR_INVALID with nothing
 * changed. */
pkv_status pkv_prefix_register(pkv_pool* pool, const int32_t* tokens, int32_t num_tokens,
                               const int32_t* block_ids);

/* Number of indexed blocks, and how many of them are free. */
pkv_status pkv_prefix_stats(const pkv_pool* pool, int32_t* num_cached, int32_t* num_cached_free);

/* ===== Block swap and sliding-window release (host) =========================
 * [P5 "Eviccion y preemption", "Estrategia 2: swap"]: when the pool runs
 * dry, a session can be preempted by moving its blocks to CPU memory over
 * the host link, which frees their device blocks, and brought back when it
 * is scheduled again.  The swap space is a second pkv_pool (its ids index a
 * cache of the same block shape in pinned host memory); a swap moves block
 * references from one pool to the other, and paged_kv_swap_blocks copies the
 * data. */

/* Moves n block references, ids[0..n) held in `from`, to fresh blocks of
 * `to`.  Each distinct id gets one new block (first-seen order), whose
 * refcount in `to` is the number of times the id occurs in ids (so blocks
 * shared inside a group of sequences stay shared); out_ids[i] is the new
 * block of ids[i].  Every occurrence then drops one reference in `from`
 * (a block reaching 0 returns to its free list).  pairs[2k], pairs[2k+1] =
 * (old id, new id) for each distinct id, *num_pairs of them: the copies to
 * enqueue with paged_kv_swap_blocks BEFORE any later write can reuse the
 * freed blocks (same stream).  Swap-out: from = device pool, to = host
 * pool; swap-in: the reverse.  Host arrays: ids, out_ids [n], pairs [2 n].
 * All-or-nothing: an id that is not live in `from` or occurs more often
 * than its refcount, or from == to -> PKV_ERR_INVALID; fewer free blocks in
 * `to` than distinct ids -> PKV_ERR_OOM; nothing is changed then. */
pkv_status kv_block_swap(pkv_pool* from, pkv_pool* to, int32_t n, const int32_t* ids,
                         int32_t* out_ids, int32_t* pairs, int32_t* num_pairs);

/* Sliding-window release [P5 "Sliding window attention": a model that
 * attends only to the last W tokens needs only the blocks of the active
 * window; the engine frees the older ones, so the cache stops growing].
 * For each sequence s, every table entry i < max(0, context_lens[s] -
 * window) / 16 (blocks whose 16 positions all lie before the window start)
 * that is >= 0 drops one reference (the block returns to the free list at
 * 0) and becomes -1; the change goes to table_updates as (s *
 * max_blocks_per_seq + i, -1), for paged_block_table_update.  Entries
 * already -1 are skipped, so repeated calls are harmless.  context_lens[s]
 * is the context length seen by the sequence's earliest query still to
 * run: its length for a decode step, L - n + 1 before a chunk of n new
 * tokens (paged_attention_prefill's first row).  The last block is never
 * released (window >= 1).
 *   tables: host int32 [num_seqs][max_blocks_per_seq], updated in place
 *   context_lens: host int32 [num_seqs]
 *   table_updates: host int32 [update_capacity][2]
 * All-or-nothing: window < 1, a length outside [0, 16 max_blocks_per_seq],
 * an entry >= 0 that is not a live block (or more releases of a block than
 * its references), or too small a capacity -> PKV_ERR_INVALID, nothing
 * changed. */
pkv_status pkv_window_release(pkv_pool* pool, int32_t num_seqs, int32_t max_blocks_per_seq,
                              int32_t* tables, const int32_t* context_lens, int32_t window,
                              int32_t* table_updates, int32_t update_capacity,
                              int32_t* num_updates);

/* ===== Slot planning for appended tokens (host) =============================
 * [P5 "La tabla de paginas"]: when a sequence produces a token at position
 * p (p = tokens already cached), it is written into the last block if that
 * block still has room (p % 16 != 0); otherwise a block is taken from the
 * global pool and appended to the table, and the token goes to its slot 0.
 * [P5 copy-on-write]: if the last block is shared (refcount > 1), it is
 * first replaced by a private copy.
 *
 * For s = 0..num_seqs-1 in order, and for each of its num_new[s] tokens
 * (num_new == NULL means 1 each), with p = context_lens[s]:
 *   p % 16 == 0           -> allocate a block, table[s][p/16] = it
 *   refcount(table[s][p/16]) > 1 -> copy-on-write: table[s][p/16] = new id,
 *                            the pair (old, new) is appended to cow_pairs
 *   slot_mapping[k++] = table[s][p/16] * 16 + p % 16;  context_lens[s] = p + 1
 * Every table entry written is also appended to table_updates as the pair
 * (s * max_blocks_per_seq + p/16, id), for paged_block_table_update.
 *
 *   block_tables   host int32 [num_seqs][max_blocks_per_seq], updated in place
 *   context_lens   host int32 [num_seqs], updated in place
 *   slot_mapping   host int64 [slot_capacity]; receives sum(num_new) slots
 *   table_updates  host int32 [update_capacity][2]
 *   cow_pairs      host int32 [cow_capacity][2]  (src block, dst block)
 * All or nothing: a position beyond max_blocks_per_seq * 16, a negative
 * count, a capacity too small, or a partly filled last block that is not a
 * live block -> PKV_ERR_INVALID (checked for all sequences first); otherwise
 * too few free blocks -> PKV_ERR_OOM; in both cases tables, lengths and pool
 * are left unchanged.  num_seqs * max_blocks_per_seq must be < 2^31. */
pkv_status paged_kv_append_slots(pkv_pool* pool, int32_t num_seqs, int32_t max_blocks_per_seq,
                                 int32_t* block_tables, int32_t* context_lens,
                                 const int32_t* num_new, int64_t* slot_mapping,
                                 int64_t slot_capacity, int32_t* table_updates,
                                 int32_t update_capacity, int32_t* num_updates,
                                 int32_t* cow_pairs, int32_t cow_capacity, int32_t* num_cow);

/* ===== Device calls =========================================================
 * The small index inputs of the cache-update calls below (slot_mapping,
 * table updates, block pairs) may be in device memory or in pinned host
 * memory (hipHostMalloc or any other device-accessible host allocation).  The
 * kernels read them with system-scope loads, which are never served from a
 * stale cached copy, so a caller may refill one pinned buffer for every step
 * once the stream has passed the call that read it (an event recorded
 * after the call and waited on before the refill).  A step then needs no
 * separate upload. */

/* The block tables live in device memory next to the cache, not on the host
 * [P5 "La tabla de paginas": a host-side table would cost a PCIe round trip
 * per decode step].  Applies `updates` (int32 [num_updates][2] of
 * (flat index, block id)) to block_tables (device int32 [table_elems]).
 * Pairs whose index is outside [0, table_elems) are skipped.  Any flat int32
 * device array works: with the context lengths stored right after the
 * tables ([num_seqs][max_blocks] then [num_seqs]), a step's new lengths
 * travel as pairs (num_seqs * max_blocks + s, length) in the same launch. */
pkv_status paged_block_table_update(int32_t* block_tables, int64_t table_elems,
                                    const int32_t* updates, int32_t num_updates,
                                    hipStream_t stream);

/* Store the K and V of new tokens into the cache through a slot mapping
 * [P1 "El mecanismo en si": the cache keeps K and V of every processed token;
 * P5: the new token's K,V go to its slot].  For every i < num_tokens with
 * 0 <= slot_mapping[i] < num_blocks * 16, the row k_new[i][h][:] (and
 * v_new[i][h][:]) becomes token slot (slot % 16) of tile (slot / 16, h),
 * in the layout above.  Negative slots are padding and skipped; slots at or
 * beyond num_blocks * 16 are skipped as well (and reported as
 * PKV_ERR_INVALID when the environment variable PKV_DEBUG=1, which also
 * checks uniqueness; that check synchronizes the stream).  Slots must be
 * unique: two rows for one slot race.  Bytes are copied unchanged.
 * k_new, v_new, k_cache, v_cache: device; slot_mapping: device or pinned host. */
pkv_status paged_kv_write(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                          void* k_cache, void* v_cache, int32_t num_tokens,
                          int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                          pkv_dtype dtype, hipStream_t stream);

/* One launch doing both paged_block_table_update(block_tables, table_elems,
 * updates, num_updates) and paged_kv_write(k_new, ..., dtype) above, with
 * their argument meanings, checks and skipping rules (the two parts touch
 * different memory, so their order inside the launch does not matter).  A
 * decode step appends a token per sequence and may grow a table in the same
 * step [P5 "La tabla de paginas"]; one launch instead of two shortens it. */
pkv_status paged_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                           void* k_cache, void* v_cache, int32_t num_tokens, int32_t num_kv_heads,
                           int32_t head_dim, int32_t num_blocks, pkv_dtype dtype,
                           int32_t* block_tables, int64_t table_elems, const int32_t* updates,
                           int32_t num_updates, hipStream_t stream);

/* Copy whole blocks (all kv heads, all 16 slots, K and V) for copy-on-write
 * [P5 "Copy-on-write para sampling paralelo": only the last affected block
 * is copied].  pairs: int32 [num_pairs][2] = (src block, dst block), device
 * or pinned host memory.
 * Pairs with an id outside [0, num_blocks) are skipped.  Destinations must
 * be distinct and must not be sources of other pairs in the same call.
 * Enqueue before paged_kv_write on the same stream so the copy sees the
 * block as it was before the new tokens arrive.  dtype may be PKV_FP8_E4M3 (byte copy). */
pkv_status paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                                int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                                int32_t num_blocks, pkv_dtype dtype, hipStream_t stream);

/* Copies for a block swap [P5 "Estrategia 2: swap": the blocks of a
 * preempted session go to CPU memory over PCIe and come back when it runs
 * again].  Block pairs[i][0] of the source cache (src_k, src_v, with
 * src_num_blocks blocks) is copied to block pairs[i][1] of the destination
 * cache (dst_k, dst_v, dst_num_blocks blocks): whole blocks, all kv heads
 * and 16 slots, K and V, bytes unchanged.  Both caches have the layout
 * above with the same num_kv_heads, head_dim and dtype; either one may be
 * pinned host memory (hipHostMalloc), which the kernel reads or writes
 * directly across the host link.  Plan the pairs with kv_block_swap.
 *   pairs: int32 [num_pairs][2], device or pinned host memory
 * Pairs with an id out of range are skipped; destination blocks must be
 * distinct (two pairs with one destination race).  The source and
 * destination must be different buffers, else PKV_ERR_INVALID (use
 * paged_kv_copy_blocks inside one cache).  Head_dim not a multiple of 32 ->
 * PKV_ERR_UNSUPPORTED.  A host destination holds the data once the stream
 * has passed the call (synchronize or wait on an event first). */
pkv_status paged_kv_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                                const int32_t* pairs, int32_t num_pairs, int32_t num_kv_heads,
                                int32_t head_dim, int32_t src_num_blocks, int32_t dst_num_blocks,
                                pkv_dtype dtype, hipStream_t stream);

/* Bytes of scratch paged_attention_decode needs for these sizes.  For
 * partition_size > 0 it is 0 when every context fits one partition; for
 * partition_size 0 it covers both the balanced bf16 split (two partial
 * states per wavefront of the current device's grid, plus one 8-byte arrival
 * counter per sequence and kv head) and 512-token fp32 partitions.  Queries the current
 * device (returns 0 if that fails, or for invalid sizes).  The counters
 * carry a tag of the launch that wrote them, so the workspace never needs
 * clearing. */
size_t paged_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_context_len, int32_t partition_size);

/* Decode attention: one query token per sequence attends over its whole
 * context, gathering K and V block by block through its table and never
 * copying them into a contiguous buffer [P3 "PagedAttention ..." ; P5 "El
 * kernel CUDA": block-aligned chunks, each located through the table].  The
 * mathematics is plain attention [P3 "Que es el mecanismo de atencion";
 * P1 "El mecanismo en si"]: for query head h of sequence s, with
 * kvh = h / (num_q_heads / num_kv_heads) and L = context_lens[s],
 *   score_t = scale * sum_d q[s][h][d] * K_t[d],   t = 0..L-1
 *   w_t     = exp(score_t - max score) / sum_j exp(score_j - max score)
 *   out[s][h][:] = sum_t w_t * V_t[:]
 * (L = 0 gives a zero row).  The work is split into pieces whose partial
 * results (running max, sum of weights, unnormalised output) are merged by a
 * log-sum-exp reduction; the result does not depend on the split beyond
 * rounding.  partition_size > 0: every context is cut into partitions of
 * that many tokens.  partition_size == 0 (bf16): balanced split -- all
 * (kv head, sequence, block) tiles form one list and every wavefront of a
 * fixed grid (8 per compute unit) takes an equal contiguous slice of it,
 * across sequence boundaries; a sequence split over several wavefronts is
 * merged by the last of them to finish, inside the same launch; for fp32,
 * 0 means 512-token partitions.  Concurrent calls must not share a
 * workspace.
 *
 *   q, k_cache, v_cache, block_tables, context_lens, workspace: device, read
 *   out: device fp32, written
 *   max_context_len: host-side upper bound of context_lens (sizes the grid)
 *   partition_size: tokens per partition, a multiple of 32; 0 = balanced
 *   (bf16) / 512 (fp32)
 *   workspace_bytes >= paged_attention_workspace_size(...) (may be NULL/0
 *   when that is 0)
 * Errors: num_q_heads % num_kv_heads != 0, non-positive sizes, a
 * partition_size that is not a multiple of 32, a short workspace ->
 * PKV_ERR_INVALID.  head_dim not in {64, 128}, or more than 16 query heads
 * per kv head with bf16 -> PKV_ERR_UNSUPPORTED.  On the device, a sequence
 * whose length exceeds max_context_len or max_blocks_per_seq * 16, or whose
 * table holds an id outside [0, num_blocks), gets NaN in all its output rows
 * instead of reading out of bounds.  Table entries at or beyond
 * ceil(L / 16) are never read. */
pkv_status paged_attention_decode(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len,
                                  float scale, int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, pkv_dtype kv_dtype, float* out,
                                  hipStream_t stream);

/* One decode step in one launch: paged_kv_append for one new token per
 * sequence, then paged_attention_decode_window over the grown contexts
 * ["PagedAttention por dentro", «La tabla de páginas (block table)»: each
 * step stores the new token's K/V in its sequence's last block, taking a
 * new block when that one is full; «El kernel CUDA»: attention then reads
 * the context block by block through the table].  Every sequence s with
 * context_lens_in[s] > 0 gains one token: its K and V are row s of k_new /
 * v_new ([num_seqs][num_kv_heads][head_dim], bf16) and slot_mapping[s] is
 * its slot (from paged_kv_append_slots; read only for those sequences).
 * Attention over the context_lens_in[s] + 1 tokens takes the new token from
 * its rows: a tile that holds the new token's slot is used with those bytes
 * replaced, so nothing the launch computes depends on when its own stores
 * land.  The rows are stored in their slots (as paged_kv_write; a slot
 * outside the pool is skipped), the table updates (flat index, block id)
 * with an index inside [0, num_seqs * max_blocks_per_seq) are applied, and
 * context_lens_out[s] = context_lens_in[s] + 1 (an empty or negative length
 * is copied as it is); the next launch on the stream sees all of them.  context_lens_out must
 * not be context_lens_in (a driver alternates two buffers).  The updates
 * may only change table entries this step does not read: a new block's
 * entry, a copy-on-write replacement of the last block whose copy
 * (paged_kv_copy_blocks) is enqueued before this call, or a sliding-window
 * release (pkv_window_release with the grown lengths).  max_context_len
 * bounds the grown lengths.  bf16 cache and the per-CU balanced split (up to
 * 16384 sequences); workspace as paged_attention_decode with partition_size
 * 0; other dtypes or shapes -> PKV_ERR_UNSUPPORTED.  slot_mapping and
 * updates: device or pinned host memory; other arguments and errors as
 * paged_kv_append and paged_attention_decode_window. */
pkv_status paged_kv_append_decode(const void* q, const void* k_new, const void* v_new,
                                  const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                  int32_t* block_tables, const int32_t* context_lens_in,
                                  int32_t* context_lens_out, const int32_t* updates,
                                  int32_t num_updates, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                  int32_t window, void* workspace, size_t workspace_bytes,
                                  pkv_dtype kv_dtype, float* out, hipStream_t stream);

/* FP8 cache write: like paged_kv_write, but k_new / v_new (bf16 or fp32,
 * src_dtype) are quantised into an FP8 E4M3 cache: y = x * (1 / scale) in
 * float32 (1 / scale rounded to float32 on the host), then the nearest E4M3
 * code, ties to the even mantissa; magnitudes from 448 up clamp to 448, NaN
 * gives 0x7F with the input's sign.  k_cache / v_cache hold uint8 codes in
 * the FP8 tile order above.  Scales must be positive and finite, else
 * PKV_ERR_INVALID; argument placement and other errors as paged_kv_write. */
pkv_status paged_kv_write_fp8(const void* k_new, const void* v_new, pkv_dtype src_dtype,
                              const int64_t* slot_mapping, void* k_cache, void* v_cache,
                              int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int32_t num_blocks, float k_scale, float v_scale,
                              hipStream_t stream);

/* Decode over an FP8 E4M3 cache: paged_attention_decode's result for K, V =
 * code value x k_scale, v_scale (q is bf16 [B][Hq][D], out fp32).  The codes
 * are expanded to bf16 exactly in registers; k_scale folds into the score
 * scale and v_scale into the output.  Balanced split only (partition_size
 * 0 implied): up to 16384 sequences and num_seqs * max_blocks_per_seq *
 * num_kv_heads below 2^31, else PKV_ERR_UNSUPPORTED.  Workspace as paged_attention_workspace_size(...,
 * partition_size 0).  Errors otherwise as paged_attention_decode. */
pkv_status paged_attention_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, float k_scale, float v_scale, void* workspace,
                                      size_t workspace_bytes, float* out, hipStream_t stream);

/* Multi-query attention over the paged cache (chunked prefill): several new
 * query tokens per sequence, mixed with one-token decode rows in the same
 * call, over the same block tables ["PagedAttention por dentro", «Chunked
 * prefill integrado con paged KV»: prefill chunks and decode share one step
 * and one paged cache].  Sequence s's chunk is rows query_start[s] ..
 * query_start[s+1]-1 of q; they are the LAST n_s = query_start[s+1] -
 * query_start[s] of its L = context_lens[s] cached tokens (write their K/V
 * with paged_kv_write / paged_kv_append first).  Chunk row i is position
 * p = L - n_s + i and attends causally to positions lo..p:
 *   out[r][h][:] = sum_{lo<=t<=p} softmax_t(scale * q[r][h] . K_t) V_t,
 * kv head h / (num_q_heads / num_kv_heads), lo = 0, or with a sliding window
 * of `window` > 0 tokens ["Sliding window attention": only the last W
 * tokens are attended] lo = max(0, p - window + 1).  Table entries before
 * the block of the first row's lo are never read.  n_s = 1 is a decode
 * step; n_s = 0 leaves the sequence out.
 *
 *   q: device [T][num_q_heads][head_dim] in the cache dtype, T = query_start[num_seqs]
 *   query_start: device int32 [num_seqs + 1], non-decreasing, query_start[0] = 0
 *   out: device fp32 [T][num_q_heads][head_dim], written for every chunk row
 *   max_query_len: host-side upper bound of n_s (sizes the grid); rows of a
 *     chunk beyond it get NaN
 * bf16 caches (kv_dtype PKV_BF16; FP8: paged_attention_prefill_fp8);
 * head_dim 64 or 128; at most 16 query heads per kv head.  Precision: fp32
 * accumulation; the softmax weights and V enter P.V as f16 (11 significant
 * bits), and a workgroup whose stage holds a V element beyond f16's range
 * (|v| >= 65536, inf, NaN) reruns with bf16 operands, so every value of
 * the cache is handled.
 * Errors: as paged_attention_decode (PKV_ERR_INVALID / PKV_ERR_UNSUPPORTED);
 * on the device a sequence with a bad length, n_s > L, or a table entry
 * outside [0, num_blocks) gets NaN rows instead of out-of-range reads. */
pkv_status paged_attention_prefill(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   const int32_t* query_start, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t num_blocks, int32_t max_blocks_per_seq,
                                   int32_t max_context_len, int32_t max_query_len, float scale,
                                   int32_t window, pkv_dtype kv_dtype, float* out,
                                   hipStream_t stream);

/* Chunked prefill over an FP8 E4M3 cache: paged_attention_prefill's result
 * for K, V = code value x k_scale, v_scale ["KV cache: la memoria de
 * trabajo...", «Trucos para que el cuaderno sea más fino»: the cache is
 * read at half the bytes].  q is bf16, out fp32, as above.  The codes are expanded
 * exactly on their way into LDS (K to bf16, V to f16); k_scale folds into the score scale and
 * v_scale into the output.  Scales must be positive and finite, else
 * PKV_ERR_INVALID; other arguments and errors as paged_attention_prefill. */
pkv_status paged_attention_prefill_fp8(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       const int32_t* query_start, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       int32_t max_query_len, float scale, int32_t window,
                                       float k_scale, float v_scale, float* out,
                                       hipStream_t stream);

/* Decode with a sliding window, for every cache dtype [P5 "Sliding window
 * attention": the model attends only to the last W tokens].  The query of
 * sequence s (position L - 1, L = context_lens[s]) attends to positions
 * max(0, L - window) .. L - 1 only; window 0 means the whole context, and
 * the call is then paged_attention_decode (or, for PKV_FP8_E4M3,
 * paged_attention_decode_fp8 with k_scale, v_scale; the scales are ignored
 * for other dtypes).  Table entries before the block holding position
 * L - window are never read (pkv_window_release may have set them to -1).
 * Arguments, layouts, workspace and errors otherwise as
 * paged_attention_decode; window < 0 -> PKV_ERR_INVALID. */
pkv_status paged_attention_decode_window(const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                         int32_t max_blocks_per_seq, int32_t max_context_len,
                                         float scale, int32_t window, int32_t partition_size,
                                         void* workspace, size_t workspace_bytes,
                                         pkv_dtype kv_dtype, float k_scale, float v_scale,
                                         float* out, hipStream_t stream);

/* Decode that allocates nothing, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The result of
 * paged_attention_decode_window with partition_size 0 (bf16 or FP8 cache;
 * per-CU balanced split, every CU's range in fixed wavefront shares), with
 * its partial states and arrival counters in a static device array of
 * 16 MiB that the library holds on each GPU it runs on until the process
 * ends (resolved on the first call on each device, with that device
 * current).  Needs 4 * C * (2 + s) * g * (D + 2) + 8 * num_seqs *
 * num_kv_heads bytes (each of the two parts rounded up to 256), with
 * C = compute units, g = num_q_heads / num_kv_heads, D = head_dim and s
 * the partial states per CU (at most 20) that do not fit in LDS beside the
 * 4 (num_seqs + 1)-byte tile-count prefix (s = 0 for g = 4 or 8 at D = 128
 * with up to 4096 sequences; about 1 MiB for g = 4, D = 128 on 256 CUs,
 * plus the counters); sizes beyond 16 MiB, num_seqs > 16384 or an fp32
 * cache -> PKV_ERR_UNSUPPORTED.
 * The counters carry a launch tag, so the array never needs clearing.
 * Every call on a GPU uses that GPU's one array: calls that overlap on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller.  Arguments and other errors as paged_attention_decode_window;
 * k_scale, v_scale are ignored for bf16.  Calls no allocating routine. */
pkv_status paged_attention_decode_noalloc(const void* q, const void* k_cache,
                                          const void* v_cache, const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t num_blocks,
                                          int32_t max_blocks_per_seq, int32_t max_context_len,
                                          float scale, int32_t window, pkv_dtype kv_dtype,
                                          float k_scale, float v_scale, float* out,
                                          hipStream_t stream);

/* ===== Measurement ==========================================================
 * While profiling is on, decode calls number 0, every, 2 every, ... since
 * pkv_profile_begin (each paged_attention_decode* call that gets past its
 * argument checks counts) record a pair
 * of HIP events around their main (block-walking) kernel on the caller's
 * stream.  The events are created without the system-scope fence (they only
 * time), and sampling with every > 1 keeps their markers out of most steps
 * of a timed loop.  pkv_profile_end synchronizes on the recorded events and
 * returns how many launches were timed and their total duration in
 * milliseconds.  At most 8192 launches are kept per session (later ones are
 * not timed).  every < 1 -> PKV_ERR_INVALID.  Not thread-safe. */
pkv_status pkv_profile_begin(int32_t every);
pkv_status pkv_profile_end(int32_t* num_launches, double* total_ms);
/* While profiling is on: synchronizes on the launches timed so far and
 * writes the duration of each (milliseconds, in call order) to out_ms
 * [min(capacity, count)], the count to *num_launches; the session stays
 * open.  A fixed-partition call's span covers its reduce kernel too.
 * out_ms: host.  Bad arguments -> PKV_ERR_INVALID. */
pkv_status pkv_profile_durations(float* out_ms, int32_t capacity, int32_t* num_launches);

/* Streaming-read reference: reads `bytes` (rounded down to 16) of device
 * memory `buf` once with 16-byte loads, on `stream`, so the caller can time
 * the achievable HBM read rate next to the decode kernel (8192 one-wave
 * workgroups, each streaming its own contiguous chunk with non-temporal
 * 16-byte loads, as the decode kernel does).  `sink` is device memory of at
 * least 32 KiB that the kernel may write.  Chunks must stay below 2 GiB
 * (bytes < 16 TiB) -> else PKV_ERR_UNSUPPORTED.  The decode path reads the whole cache on every token ["KV cache:
 * la memoria de trabajo ...", "La inferencia es memory-bound"], so this is
 * its ceiling. */
pkv_status pkv_stream_read(const void* buf, size_t bytes, void* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
