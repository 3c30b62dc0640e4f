/*
 * pkv — paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * The C ABI of the library libpkv.so.  Plain pointers and sizes only; no C++ or framework
 * types cross it.  Two groups of calls:
 *
 *  - a host block allocator (pkv_alloc_*, pkv_seq_*): the KV Cache Manager of a paged
 *    inference engine.  It owns the free pool of physical blocks, one block table per
 *    sequence, reference counts for shared blocks, and copy-on-write on append.
 *  - device operations (pkv_reshape_and_cache, pkv_append_and_cache, pkv_copy_blocks,
 *    pkv_update_block_tables, pkv_gather_blocks / pkv_scatter_blocks,
 *    pkv_paged_attention_decode / _cascade / _prefill, pkv_read_probe): HIP kernels,
 *    enqueued asynchronously on the caller's stream; the library never synchronises inside
 *    a call.
 *
 * Passages followed (page title, section):
 *  - "vLLM + PagedAttention：打造高并发LLM推理引擎", the numbered steps under
 *    "它是怎么工作的？": blocks are allocated on demand, each request keeps a page table from
 *    token position to block, the attention kernel gathers K/V through that table, and a
 *    finished request's blocks go back to the pool.
 *  - "PagedAttention 与 vLLM 推理加速", §2.2–§2.4 (fixed-size blocks, block table, only the
 *    last block partly empty) and §3.2 (3) (shared prefix blocks, copy-on-write).
 *  - "LLM Systems 24: Efficient LLM Inference with PagedAttention and vLLM", §2.1.3 (the KV
 *    Cache Manager allocates and frees physical blocks and maps logical to physical blocks)
 *    and §3 Conclusion (reference counts with copy-on-write; running out of blocks leads
 *    the caller to preempt).
 *
 * Layouts (the pages fix only a block's element count; these are this library's choices):
 *  - K pool and V pool: [num_blocks][num_kv_heads][block_size][head_dim], dense row-major,
 *    one pool each, element type given by pkv_dtype.  Token t of a sequence lives in
 *    physical block table[t / block_size] at offset t % block_size.
 *  - slot: block * block_size + offset, int64; -1 means "skip this token".
 *  - block_tables: [num_seqs][max_blocks_per_seq] int32, row-major; entries past a
 *    sequence's last block are -1 and never read.
 *  - q, out: [num_seqs][num_q_heads][head_dim] in the cache's element type.
 *  - Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Errors: every call returns a pkv_status.  Nothing aborts or throws across the ABI.  A
 * failed allocator call leaves the allocator unchanged.  A device call that fails host-side
 * validation enqueues nothing; PKV_ERR_HIP reports a launch error seen after enqueueing.
 *
 * Threading: an allocator handle must not be used by two threads at once.  Device calls
 * hold no global state and may run concurrently on different streams.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misaligned pointer, bad permutation */
  PKV_ERR_OUT_OF_BLOCKS = 2, /* not enough free blocks; nothing was changed */
  PKV_ERR_UNKNOWN_SEQ = 3,   /* a sequence id that the allocator does not hold */
  PKV_ERR_DUPLICATE_SEQ = 4, /* a sequence id that already exists */
  PKV_ERR_UNSUPPORTED = 5,   /* a shape or dtype with no kernel instance */
  PKV_ERR_WORKSPACE = 6,     /* workspace missing or smaller than pkv_decode_workspace_bytes */
  PKV_ERR_HIP = 7            /* the HIP runtime reported an error */
};

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

/* Opaque host-side allocator.  Created and destroyed by the caller. */
typedef struct pkv_alloc pkv_alloc;

/* Human-readable name of a status code (static string). */
const char* pkv_status_str(pkv_status status);

/* Text of the last HIP runtime error that a device call on this thread reported as
 * PKV_ERR_HIP ("" if none).  Valid until the next failing call on the same thread. */
const char* pkv_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t pkv_version(void);

/* ======================================================================================
 * Host block allocator
 * ====================================================================================== */

/* Create an allocator over num_blocks physical blocks of block_size token slots: the pool
 * of fixed-size blocks every request draws from ("PagedAttention 与 vLLM 推理加速", §2.2; "LLM
 * Systems 24: Efficient LLM Inference with PagedAttention and vLLM", §2.1.3: the KV Cache
 * Manager allocates and frees physical blocks).
 * free_order (nullable, host, num_blocks entries): a permutation of 0..num_blocks-1 giving
 * the order in which blocks are first handed out (NULL = 0, 1, 2, ...).  The pool is a
 * stack: blocks freed later are handed out before untouched ones, the most recently freed
 * first.  *out receives the handle.  INVALID_ARG on non-positive sizes, a null out, or a
 * free_order that is not a permutation. */
pkv_status pkv_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                            pkv_alloc** out);

/* Destroy an allocator and its whole state (NULL is ignored); the caller's device pools are
 * untouched (same passages as pkv_alloc_create). */
void pkv_alloc_destroy(pkv_alloc* a);

/* Add sequence seq_id holding num_tokens (>= 0) tokens ("vLLM + PagedAttention：打造高并发LLM
 * 推理引擎", step 1 under "它是怎么工作的？": blocks are taken on demand; "PagedAttention 与 vLLM
 * 推理加速", §2.3: 7 tokens in 4-token blocks take two blocks, the last with one free slot):
 * takes ceil(num_tokens/block_size) blocks, in logical order, and writes the tokens' slots to slots_out (host, num_tokens
 * entries; may be NULL only when num_tokens == 0).
 * DUPLICATE_SEQ if seq_id exists; OUT_OF_BLOCKS if the pool is short. */
pkv_status pkv_seq_add(pkv_alloc* a, int64_t seq_id, int32_t num_tokens, int64_t* slots_out);

/* Prefix caching: requests that begin with the same system prompt share the physical blocks
 * of that prompt ("PagedAttention 与 vLLM 推理加速", §3.2 (3), the three requests that keep
 * one copy of a six-block prompt), here also when they arrive independently.  Adds seq_id
 * with the prompt tokens[0..num_tokens) (host, token ids).  A full block of a prompt is
 * identified by the whole token prefix that ends with it; the sequence shares the cached
 * blocks of its longest run of leading full blocks found in the cache (each gains one
 * reference), takes fresh blocks for the rest in logical order, and registers its fresh full
 * blocks.  slots_out (host, num_tokens): -1 for tokens in shared blocks (their K/V is
 * already in the pools; pkv_reshape_and_cache skips them), otherwise the slot as
 * pkv_seq_add gives it.  *n_cached_out = number of shared tokens (a multiple of
 * block_size).  A cached block stays cached after its last holder ends ("evictable"): it is
 * reused only when no plain free block is left, in the order such blocks were released, a
 * sequence's blocks tail first; evictable blocks count as free in pkv_num_free_blocks.
 * Only prompts given here are cached (tokens added by append/extend carry no ids).
 * DUPLICATE_SEQ / OUT_OF_BLOCKS (nothing changes) / INVALID_ARG as for pkv_seq_add. */
pkv_status pkv_seq_add_tokens(pkv_alloc* a, int64_t seq_id, const int32_t* tokens,
                              int32_t num_tokens, int64_t* slots_out, int32_t* n_cached_out);

/* Create child_id sharing every block of parent_id (each block gains one reference):
 * requests with a common prefix point at one physical copy ("PagedAttention 与 vLLM 推理加速",
 * §3.2 (3); "LLM Systems 24", §3 Conclusion: reference counts with copy-on-write).
 * UNKNOWN_SEQ if the parent is missing; DUPLICATE_SEQ if the child exists. */
pkv_status pkv_seq_fork(pkv_alloc* a, int64_t parent_id, int64_t child_id);

/* Append one token to each of the n sequences seq_ids (host), in order; the ids must be
 * distinct (else INVALID_ARG).  ("vLLM + PagedAttention", steps 1–2 under "它是怎么工作的？": a
 * new block only when the last one is full; "PagedAttention 与 vLLM 推理加速", §2.4: only a
 * sequence's last block is partly filled, and §3.2 (3): a shared block is copied only when a
 * sharer writes to it.)  For each sequence: a length that is a multiple of
 * block_size takes a fresh block; otherwise a last block shared with another sequence is
 * replaced by a fresh block and the pair (old, new) is reported for the caller to copy
 * (copy-on-write) before writing; an unshared last block is written in place.
 * slots_out (host, n int64): the slot of each appended token.
 * cow_pairs_out (host, 2n int32): (src, dst) block pairs, *n_cow_out of them.
 * All-or-nothing: OUT_OF_BLOCKS leaves everything unchanged. */
pkv_status pkv_seq_append(pkv_alloc* a, const int64_t* seq_ids, int32_t n, int64_t* slots_out,
                          int32_t* cow_pairs_out, int32_t* n_cow_out);

/* Append n >= 0 tokens to one sequence (a prefill chunk): the same as n calls of
 * pkv_seq_append with seq_id alone (same passages; the chunk's tokens then attend causally,
 * "PagedAttention 与 vLLM 推理加速", §1).  slots_out (host, n int64): the new tokens' slots in
 * order.  cow_pairs_out (host, 2 int32): at most one (src, dst) copy-on-write pair, for the
 * first token when the last block is shared and partly filled; *n_cow_out = 0 or 1.
 * All-or-nothing: OUT_OF_BLOCKS leaves everything unchanged. */
pkv_status pkv_seq_extend(pkv_alloc* a, int64_t seq_id, int32_t n, int64_t* slots_out,
                          int32_t* cow_pairs_out, int32_t* n_cow_out);

/* End a sequence: each of its blocks loses a reference; blocks with none left return to
 * the pool in logical order (so its last block is the next one handed out).  ("vLLM +
 * PagedAttention", step 4 under "它是怎么工作的？": a finished request's blocks go back to the
 * pool; "LLM Systems 24", §3 Conclusion: a shared block is freed with its last reference.) */
pkv_status pkv_seq_free(pkv_alloc* a, int64_t seq_id);

/* Preemption by swapping ("LLM Systems 24: Efficient LLM Inference with PagedAttention and
 * vLLM", §3 Conclusion: when the pool runs out a request is preempted, its cache swapped out
 * to the host, and restored later).  pkv_seq_swap_out writes the sequence's blocks in
 * logical order to blocks_out (host, capacity max_blocks; INVALID_ARG if too small, nothing
 * changed) and *n_blocks_out, then gives up its references exactly like pkv_seq_free; the
 * caller first copies those blocks out (pkv_gather_blocks on the same stream before the
 * blocks are reused).  The id stays taken (add/fork return DUPLICATE_SEQ) until swap-in.
 * pkv_seq_swap_in takes that many fresh blocks, handed out in logical order, writes them to
 * blocks_out and restores the length; the caller then copies the data back
 * (pkv_scatter_blocks).  The restored sequence owns every block (sharing is not
 * re-established).  OUT_OF_BLOCKS leaves everything unchanged; UNKNOWN_SEQ if the id is not
 * resident (swap-out) or not swapped out (swap-in). */
pkv_status pkv_seq_swap_out(pkv_alloc* a, int64_t seq_id, int32_t max_blocks, int32_t* blocks_out,
                            int32_t* n_blocks_out);
pkv_status pkv_seq_swap_in(pkv_alloc* a, int64_t seq_id, int32_t max_blocks, int32_t* blocks_out,
                           int32_t* n_blocks_out);

/* The page tables ("vLLM + PagedAttention", step 2 under "它是怎么工作的？": each request maps
 * token positions to blocks; "PagedAttention 与 vLLM 推理加速", §2.3; "LLM Systems 24", §2.1.3:
 * the logical-to-physical block mapping).  Copy the block tables of n sequences into tables_out (host, n * max_blocks int32,
 * row-major, padded with -1) and their lengths into lens_out (host, n int32; nullable).
 * INVALID_ARG if a sequence holds more than max_blocks blocks. */
pkv_status pkv_get_block_tables(const pkv_alloc* a, const int64_t* seq_ids, int32_t n,
                                int32_t max_blocks, int32_t* tables_out, int32_t* lens_out);

/* For each of the n sequences seq_ids (host): the number of leading block-table entries
 * whose block is also referenced by another sequence, into out (host, n int32).  Requests
 * that share a system prompt point at the same physical blocks ("PagedAttention 与 vLLM
 * 推理加速", §3.2 (3)); this counts that shared run.  Meant as the cached_blocks hint of
 * pkv_paged_attention_decode.  UNKNOWN_SEQ if an id is missing (out untouched). */
pkv_status pkv_shared_prefix_blocks(const pkv_alloc* a, const int64_t* seq_ids, int32_t n,
                                    int32_t* out);

/* Groups for pkv_paged_attention_cascade (cascade attention: "LLM Systems 24: Efficient LLM
 * Inference with PagedAttention and vLLM", §2.2.1.3, names it among the kernels a runtime
 * picks per batch).  For the batch rows seq_ids[0..n) (host): a group is a maximal run of
 * at least two consecutive rows whose block tables start with the same physical block; it
 * shares the longest run of leading table entries all its members agree on, cut to the
 * full blocks every member's length covers.  Rows in no group (or whose group would share
 * nothing) stand alone with 0 shared blocks.  Writes group_start_out (host, n + 1 int32:
 * group g is rows group_start[g] .. group_start[g+1] - 1), shared_blocks_out (host, n
 * int32, per row) and *n_groups_out.  Order the batch so that sharers are adjacent.
 * UNKNOWN_SEQ if an id is missing (outputs untouched). */
pkv_status pkv_prefix_groups(const pkv_alloc* a, const int64_t* seq_ids, int32_t n,
                             int32_t* group_start_out, int32_t* shared_blocks_out,
                             int32_t* n_groups_out);

/* Length (tokens) of one sequence: its page table covers positions 0 .. length - 1 ("vLLM +
 * PagedAttention", step 2 under "它是怎么工作的？"). */
pkv_status pkv_seq_length(const pkv_alloc* a, int64_t seq_id, int32_t* len_out);

/* Lengths (tokens) of the n sequences seq_ids (host) into lens_out (host, n int32): before
 * pkv_seq_append, the positions the appended tokens will take (each request's page table
 * maps token positions to blocks: "vLLM + PagedAttention", step 2 under "它是怎么工作的？").
 * UNKNOWN_SEQ if an id is not resident (lens_out untouched). */
pkv_status pkv_seq_lengths(const pkv_alloc* a, const int64_t* seq_ids, int32_t n,
                           int32_t* lens_out);

/* Number of blocks a call can take: free ones plus evictable cached ones (-1 for a null
 * handle).  A scheduler checks it before admitting or growing requests, and preempts when
 * it runs out ("LLM Systems 24", §3 Conclusion). */
int32_t pkv_num_free_blocks(const pkv_alloc* a);

/* Number of blocks registered in the prefix cache and not yet evicted, held or evictable
 * (-1 for a null handle) ("PagedAttention 与 vLLM 推理加速", §3.2 (3): one copy of a shared
 * system prompt's blocks). */
int32_t pkv_num_cached_blocks(const pkv_alloc* a);

/* Reference count of a physical block: the number of sequences whose table holds it (-1 if
 * out of range or a null handle) ("LLM Systems 24", §3 Conclusion: reference counts decide
 * copy-on-write and freeing). */
int32_t pkv_block_refcount(const pkv_alloc* a, int32_t block);

/* Memory use of the pool ("PagedAttention 与 vLLM 推理加速", §2.4: only the last block of a
 * sequence wastes slots, under 4% in all; §3.2 (1): utilisation near 96% against ~30% for
 * contiguous reservation).  tokens_stored: sum of all sequence lengths (a shared token
 * counts once per sequence); slots_allocated: block_size times the number of blocks
 * referenced at least once. */
pkv_status pkv_usage(const pkv_alloc* a, int64_t* tokens_stored, int64_t* slots_allocated);

/* ======================================================================================
 * Device operations (all pointers are device pointers unless stated; stream is a
 * hipStream_t, NULL = the null stream).  Pointers must be 16-byte aligned.
 * ====================================================================================== */

/* Cache write ("vLLM + PagedAttention", step 1–2 under "它是怎么工作的？": new tokens go
 * into the blocks their table assigns).  For each token t < num_tokens with
 * s = slot_mapping[t] >= 0: K[s / block_size][h][s % block_size][:] = key[t][h][:] for
 * every KV head h, and the same for V.  key, value: [num_tokens][num_kv_heads][head_dim]
 * contiguous.  Exact bit copy.  Slots must be distinct and < num_blocks * block_size;
 * slots outside [0, num_blocks*block_size) are skipped.  num_tokens == 0 is a no-op. */
pkv_status pkv_reshape_and_cache(const void* key, const void* value, const int64_t* slot_mapping,
                                 void* k_cache, void* v_cache, int32_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t num_blocks, pkv_dtype dtype, void* stream);

/* Copy-on-write block copies ("PagedAttention 与 vLLM 推理加速", §3.2 (3)): for each of the
 * n_pairs pairs (src, dst) in pairs ([n_pairs][2] int32, device), copy the whole block src
 * (every head, every slot) to block dst, in both pools.  Destinations must be distinct and
 * must not be sources.  Pairs with an id outside [0, num_blocks) are skipped. */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t n_pairs,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, pkv_dtype dtype, void* stream);

/* Whole-block moves for swap preemption (see pkv_seq_swap_out).  pkv_gather_blocks copies
 * block blocks[i] of the K and V pools (every KV head and slot, blk = num_kv_heads *
 * block_size * head_dim elements) to k_out + i * blk and v_out + i * blk;
 * pkv_scatter_blocks copies k_in + i * blk and v_in + i * blk back into block blocks[i].
 * blocks: device, n_blocks int32 (ids outside [0, num_blocks) are skipped; scatter
 * destinations must be distinct).  The buffers (16-byte aligned, owned by the caller) are
 * either device memory, then moved to and from the host by asynchronous copies on the same
 * stream, or pinned host memory mapped into the device's address space (hipHostMalloc),
 * passed by its device-side address (hipHostGetDevicePointer): the kernel then reads and
 * writes the host copy directly over the host link, with no staging buffer and no separate
 * copy.  Either way the call is asynchronous on `stream`. */
pkv_status pkv_gather_blocks(const void* k_cache, const void* v_cache, const int32_t* blocks,
                             int32_t n_blocks, void* k_out, void* v_out, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             pkv_dtype dtype, void* stream);
pkv_status pkv_scatter_blocks(const void* k_in, const void* v_in, const int32_t* blocks,
                              int32_t n_blocks, void* k_cache, void* v_cache, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              pkv_dtype dtype, void* stream);

/* Device-side upkeep of block tables and lengths after appends, so that a decode loop
 * uploads only the step's slots instead of whole tables ("vLLM + PagedAttention", step 2
 * under "它是怎么工作的？": each request's page table records where token n lives).  For
 * each i < n with rows[i] in [0, num_rows), positions[i] >= 0 and slot s = slot_mapping[i]
 * in [0, num_blocks * block_size): block_tables[rows[i]][positions[i] / block_size] =
 * s / block_size (if that column is below max_blocks_per_seq) and context_lens[rows[i]] =
 * positions[i] + 1; other entries are skipped.  rows (device, n int32, distinct),
 * positions (device, n int32: the token's position = the row's length before the append),
 * slot_mapping (device, n int64, as returned by pkv_seq_append).  After pkv_seq_append the
 * result equals the tables pkv_get_block_tables returns, copy-on-write included (the new
 * token always lands in the row's last block, whose id the slot carries). */
pkv_status pkv_update_block_tables(int32_t* block_tables, int32_t* context_lens,
                                   const int32_t* rows, const int32_t* positions,
                                   const int64_t* slot_mapping, int32_t n, int32_t num_rows,
                                   int32_t max_blocks_per_seq, int32_t block_size,
                                   int32_t num_blocks, void* stream);

/* The cache write and the table upkeep of one decode step in a single launch: the same
 * result as pkv_update_block_tables(block_tables, context_lens, rows, positions,
 * slot_mapping, n, num_rows, max_blocks_per_seq, block_size, num_blocks) followed by
 * pkv_reshape_and_cache(key, value, slot_mapping, k_cache, v_cache, n, num_kv_heads,
 * head_dim, block_size, num_blocks, dtype) ("vLLM + PagedAttention", steps 1–2 under
 * "它是怎么工作的？": the new token goes into the block its table assigns, and the table
 * records where it lives).
 * slot_mapping (n int64), positions (n int32) and rows (n int32; NULL = token i updates row
 * i) may be device memory or pinned host memory mapped into the device's address space,
 * passed by its device-side address (hipHostGetDevicePointer): a decode loop then uploads
 * nothing.  They are read once per token with system-coherent loads, so the host may rewrite
 * such a buffer for a later call once this call has completed.
 * key, value: device, [n][num_kv_heads][head_dim] contiguous, 16-byte aligned.
 * block_tables, context_lens: device, both NULL for the cache write alone (rows and
 * positions are then not read).  Slots and rows must be distinct.  A token whose slot lies
 * outside [0, num_blocks * block_size) is skipped entirely; a table update whose row,
 * position or column is out of range is skipped (the cache write still happens).
 * n == 0 is a no-op. */
pkv_status pkv_append_and_cache(const void* key, const void* value, const int64_t* slot_mapping,
                                const int32_t* rows, const int32_t* positions, int32_t n,
                                void* k_cache, void* v_cache, int32_t* block_tables,
                                int32_t* context_lens, int32_t num_rows, int32_t max_blocks_per_seq,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, pkv_dtype dtype, void* stream);

/* Bytes of workspace pkv_paged_attention_decode needs for this shape, max_context_len and
 * partition_size (same meanings as for the decode call): num_seqs * num_q_heads * P *
 * (head_dim + 2) floats when contexts are split into P > 1 partitions, else 0. */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                  pkv_dtype dtype, int32_t partition_size);

/* Paged decode attention ("vLLM + PagedAttention", step 3 under "它是怎么工作的？";
 * "PagedAttention 与 vLLM 推理加速", §2.3).  For each sequence b and query head h, with
 * g = h / (num_q_heads / num_kv_heads) and n = context_lens[b]:
 *     out[b][h] = sum_t softmax_t(scale * <q[b][h], K_t>) V_t,   t = 0 .. n-1,
 * where K_t, V_t are read from block block_tables[b][t / block_size] at offset
 * t % block_size, KV head g.  n == 0 gives zeros.  Accumulation in fp32; out is rounded
 * to the cache's element type (round to nearest even).
 *
 * partition_size: 0 = one workgroup per (sequence, head or head group) covering the whole
 * context; > 0 = split each context into partitions of that many tokens (a multiple of 16
 * and of block_size), each reduced to (max, sum, partial output) in the workspace and merged
 * by a second kernel; -1 = automatic: the fewest equal partitions (a multiple of 32 tokens,
 * at least 512) that give the launch about 1024 workgroups (no split when the batch already
 * has that many (sequence, head) rows), decided from the shape and max_context_len only.  All choices compute the
 * same quantity; results differ only in fp32 rounding order.  For a given shape, length set
 * and partition_size the result is bit-for-bit reproducible and does not depend on
 * physical block placement.
 * max_context_len: an upper bound of context_lens (sizes the launch without reading device
 * memory on the host; larger lengths are clamped to it and to
 * max_blocks_per_seq * block_size).  Table entries outside [0, num_blocks) are treated as
 * empty blocks and never dereferenced.  With PKV_DEBUG=1 in the environment the call first
 * waits for the stream, reads context_lens and block_tables back and returns
 * PKV_ERR_INVALID_ARG (message in pkv_last_error, nothing enqueued) if a length lies outside
 * [0, that clamp] or a table entry a length covers lies outside [0, num_blocks).
 * cached_blocks (nullable, device, num_seqs int32): a cache-policy hint.  K/V blocks are
 * streamed with non-temporal loads, which is fastest for data read once; the first
 * cached_blocks[b] table entries of sequence b (for example a prefix shared with other
 * sequences, see pkv_shared_prefix_blocks) are read through the caches instead, so that
 * sequences reading the same blocks at about the same time share them.  The result does not
 * depend on it.
 * workspace / workspace_bytes: device scratch of at least pkv_decode_workspace_bytes(...)
 * bytes, 16-byte aligned (may be NULL when that is 0); its contents need no initialisation
 * and are overwritten.  After a split call it holds the partials, fp32, with P =
 * ceil(max_context_len / partition size): o [num_seqs][num_q_heads][P][head_dim], then m and
 * l [num_seqs][num_q_heads][P] (m in the log2 domain, a reference that need not be the
 * partition's largest score; o / l is the partition's attention); only the partitions a
 * sequence's context reaches are written, and none for a sequence with one partition.
 * Supported: dtype f32, f16, bf16; head_dim 8, 64, 128; block_size 4, 8, 16, 32;
 * num_q_heads a multiple of num_kv_heads.  Grouped-query attention with 16-bit elements,
 * head_dim 64 or 128 and block_size >= 8 runs on matrix cores (MFMA). */
pkv_status pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, const int32_t* cached_blocks,
                                      int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, pkv_dtype dtype, int32_t partition_size,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): pkv_paged_attention_decode with the same
 * arguments and result, minus the workspace.  When contexts are split, the partials go to a
 * scratch array of PKV_DECODE_SCRATCH_BYTES bytes inside the library, one per GPU, reserved
 * when the library's code is loaded onto the device and held until the process ends; its
 * device address is looked up once per device (with that device current) on the first call.
 * The call allocates nothing.  The current device must be the stream's.  A shape whose
 * partials need more than PKV_DECODE_SCRATCH_BYTES (pkv_decode_workspace_bytes says how
 * many) fails with PKV_ERR_WORKSPACE before anything is enqueued.  All calls on one GPU
 * share its array: calls that overlap in time on one GPU (different streams, or several
 * host threads) race and give undefined results; calls on one stream are safe.  Nothing in
 * the array needs clearing between calls (every partial is written before it is read). */
#define PKV_DECODE_SCRATCH_BYTES (64u << 20)
pkv_status pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                              const void* v_cache, const int32_t* block_tables,
                                              const int32_t* context_lens,
                                              const int32_t* cached_blocks, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t block_size,
                                              int32_t num_blocks, int32_t max_blocks_per_seq,
                                              int32_t max_context_len, float scale,
                                              pkv_dtype dtype, int32_t partition_size,
                                              void* stream);

/* Cascade decode: the same result as pkv_paged_attention_decode (plain attention of each
 * sequence's query over its whole context, up to fp32 rounding order), computed with the
 * shared prefix of each group of sequences read once per 16 queries instead of once per
 * sequence.  Cascade attention is named among the kernels a runtime picks per batch ("LLM
 * Systems 24: Efficient LLM Inference with PagedAttention and vLLM", §2.2.1.3); requests
 * sharing a system prompt share its blocks ("PagedAttention 与 vLLM 推理加速", §3.2 (3)).
 * One launch on `stream`: per (KV head, group, tile of 16 (member, query head) columns), a
 * workgroup walks the group's shared blocks once for all its columns (on matrix cores,
 * through the caches), then each member's own blocks for that member's columns only (streamed),
 * and writes the outputs; no partial results leave the workgroup.
 * group_start (device, num_groups + 1 int32, non-decreasing): group g is the rows
 * group_start[g] .. group_start[g+1] - 1; every row must lie in exactly one group
 * (group_start[0] = 0, group_start[num_groups] = num_seqs), and a row outside every group is
 * not written.  shared_blocks (device, num_seqs int32): the group's shared count is its
 * first row's entry, clamped to [0, that row's full blocks]; every member shares that many
 * leading table entries, or its own full blocks if fewer (a member's other entries of
 * shared_blocks are not read).  pkv_prefix_groups's output for the batch rows in order
 * meets all of this; a grouping whose members' tables differ within the shared count gives
 * those members attention over the first row's blocks there.
 * max_group_size: sizes the launch (ceil(max_group_size * query heads per KV head / 16)
 * workgroups per group and KV head); a workgroup also takes every later tile at that stride,
 * so groups larger than the bound are still covered in full.
 * workspace: the kernels need none (pkv_cascade_workspace_bytes returns 0); it may be NULL.
 * partition_size: validated as for pkv_paged_attention_decode; each workgroup walks its
 * columns' whole contexts, so it does not change the work.
 * Other arguments as for pkv_paged_attention_decode (no cache hint: the shared blocks are
 * read through the caches, the rest streamed).
 * Supported: fp16 and bf16, head_dim 64 or 128, block_size 8, 16 or 32; otherwise
 * PKV_ERR_UNSUPPORTED (use pkv_paged_attention_decode).  num_groups == 0 is a no-op. */
size_t pkv_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                   pkv_dtype dtype, int32_t partition_size);
pkv_status pkv_paged_attention_cascade(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, const int32_t* group_start,
                                       const int32_t* shared_blocks, int32_t num_groups,
                                       int32_t max_group_size, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_context_len,
                                       float scale, pkv_dtype dtype, int32_t partition_size,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Paged causal prefill attention (a prompt, or one chunk of it, for several sequences at
 * once).  Each new token attends to every earlier token of its sequence and to itself
 * ("PagedAttention 与 vLLM 推理加速", §1: every new token sees all previous tokens), read
 * through the block table as in decode.  Sequence b's new tokens are the rows
 * query_start[b] .. query_start[b+1] - 1 of q and out ([num_tokens][num_q_heads][head_dim],
 * the cache's element type); their K/V must already be in the cache (reshape_and_cache),
 * so that context_lens[b] counts them: new token j of n_b sits at position
 * context_lens[b] - n_b + j and
 *     out[row][h] = sum_{t <= pos} softmax_t(scale * <q[row][h], K_t>) V_t,
 * KV head h / (num_q_heads / num_kv_heads), fp32 accumulation, rounded to nearest even.
 * query_start (device, num_seqs + 1 int32, non-decreasing, query_start[num_seqs] <=
 * num_tokens): rows outside [0, num_tokens) are neither read nor written.
 * max_query_len: an upper bound of the n_b (sizes the launch); max_context_len as for
 * decode.  A token whose position would be negative (n_b > context_lens[b]) gets zeros.
 * Supported: fp16 and bf16, head_dim 64 or 128, block_size 8, 16 or 32 (matrix cores);
 * other shapes return PKV_ERR_UNSUPPORTED, and so do launches of more than 2^31 - 1
 * workgroups (8 * ceil(num_seqs * num_kv_heads / 8) * (num_q_heads / num_kv_heads) *
 * ceil(max_query_len / 128)) and K/V blocks of 2^32 bytes or more.  Enqueued on stream; no
 * workspace. */
pkv_status pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, const int32_t* query_start,
                                       int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       int32_t num_blocks, int32_t max_blocks_per_seq,
                                       int32_t max_query_len, int32_t max_context_len, float scale,
                                       pkv_dtype dtype, void* stream);

/* ======================================================================================
 * Measurement
 * ====================================================================================== */

/* Read-bandwidth probe.  Decode attention is bound by memory traffic ("LLM Systems 24:
 * Efficient LLM Inference with PagedAttention and vLLM", §2.2.3.6), so its kernels are rated
 * against the read rate this call reaches on the same device.  Reads num_chunks chunks of
 * chunk_bytes bytes of buf (device, 16-byte aligned, at least num_chunks * chunk_bytes
 * bytes): the i-th chunk read is chunk chunk_order[i] (device, num_chunks int32; entries
 * outside [0, num_chunks) are skipped), or chunk i when chunk_order is NULL.  The XOR of
 * every 32-bit word read is XORed into *checksum (device, 4-byte aligned; the caller sets it
 * first, usually to 0), so with a permutation as the order the result is the XOR of the
 * whole buffer.  chunk_bytes: a power of two from 1024 to 2^30, and num_chunks * chunk_bytes
 * at most 2^41, else INVALID_ARG.
 * num_chunks == 0 is a no-op.  Enqueued on stream; nothing is written but *checksum. */
pkv_status pkv_read_probe(const void* buf, const int32_t* chunk_order, int64_t num_chunks,
                          int32_t chunk_bytes, uint32_t* checksum, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
