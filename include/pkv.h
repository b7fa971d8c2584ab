/*
 * pkv.h — C interface of libpkv, a paged KV-cache decode-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (four web pages about the PagedAttention paper,
 * "Efficient Memory Management for Large Language Model Serving with
 * PagedAttention"):
 *   [P1] lain42.top reading note (abstract; summary "core method" bullets).
 *   [P2] aiplusplus.yigather.com explainer (sections "core idea" and
 *        "key technical points" 1-4).
 *   [P3] auturnal.com analytical guide "paged-attention-serving" (sections
 *        1-6, "Equations and derivations" Eq. (1)-(3), "Verification protocol").
 *   [P4] cayang0802.github.io blog "paged-attention" (KV block and block
 *        table figure, beam-search sharing, preemption by swapping).
 *
 * Two halves:
 *   - a host block pool (pkv_pool_*, pkv_seq_*, pkv_append_tokens,
 *     pkv_block_tables, pkv_swap_out / pkv_swap_in): fixed-size blocks,
 *     per-sequence block tables, on-demand allocation, refcounted sharing,
 *     copy-on-write, and an optional host tier for preemption by swapping.
 *     Host memory only; no GPU is touched, so these calls also work on a
 *     machine without one.
 *   - device calls (pkv_reshape_and_cache, pkv_copy_blocks, pkv_swap_blocks,
 *     pkv_paged_attention_decode, pkv_decode_step): HIP kernels enqueued on
 *     the caller's stream.  Every pointer they take is caller-owned memory the
 *     GPU can reach; they allocate nothing, never synchronise, validate
 *     arguments on the host and return the error synchronously; a failed
 *     launch returns PKV_ERR_HIP.
 *
 * Status codes: 0 on success, negative on error.  On any error from the
 * pool, the pool's state is unchanged.
 *
 * Physical cache layout (one key cache and one value cache per layer):
 *   key cache    K[num_blocks][H_kv][d / X][B][X],   X = 16 / bytes_per_scalar
 *   value cache  V[num_blocks][H_kv][d][B]
 * Each (block, KV head) owns one contiguous tile of B * d scalars.  In a key
 * tile, a token's d values are split into 16-byte pieces and piece j of all B
 * tokens is stored together; a value tile is stored transposed, one row of B
 * token values per head dimension.  Token position t of a sequence whose
 * table is bt lives in block bt[t / B] at offset t % B; its slot is
 * bt[t / B] * B + t % B.  Scalars are fp32 or bf16 (PKV_F32 / PKV_BF16).
 *
 * Supported shapes: head_dim d in {64, 128}; block size B in {16, 32};
 * H_q / H_kv in {1, 2, 4, 8}; fp32 or bf16 scalars.  Others give
 * PKV_ERR_UNSUPPORTED.
 *
 * Threading: a pool is not thread-safe; the caller serialises calls on one
 * pool.  Device calls are safe to issue from any thread.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;

enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,   /* bad pointer, size, id or shape */
  PKV_ERR_OUT_OF_BLOCKS = -2, /* the pool cannot hold the whole batch */
  PKV_ERR_NO_SUCH_SEQ = -3,   /* sequence id unknown or already freed */
  PKV_ERR_REFCOUNT = -4,      /* pkv_pool_validate found a broken invariant */
  PKV_ERR_UNSUPPORTED = -5,   /* shape or dtype outside the supported set */
  PKV_ERR_HIP = -6,           /* a kernel launch failed */
  PKV_ERR_WORKSPACE = -7,     /* attention workspace missing or too small */
  PKV_ERR_SWAPPED = -8        /* the sequence is on the other tier (swapped out, or not) */
};

enum { PKV_F32 = 0, PKV_BF16 = 1 };

typedef struct pkv_pool pkv_pool; /* opaque; owns host metadata only */

typedef struct pkv_stats {
  int64_t num_blocks;      /* pool capacity */
  int64_t free_blocks;     /* blocks in the free queue */
  int64_t used_blocks;     /* physical blocks with refcount > 0 */
  int64_t sum_refcount;    /* equals logical_blocks while the pool is sound */
  int64_t num_seqs;        /* live sequences, swapped out or not */
  int64_t logical_tokens;  /* sum of the lengths of live sequences on the device */
  int64_t logical_blocks;  /* sum of their block-table lengths */
  int64_t allocated_slots; /* used_blocks * B: Eq. (2)'s A_B summed, [P3] */
  int64_t table_bytes;     /* 4 * logical_blocks */
  int64_t host_blocks;      /* host tier capacity (0: no host tier) */
  int64_t host_free_blocks; /* host blocks in the host free queue */
  int64_t host_used_blocks; /* host blocks with refcount > 0 */
  int64_t swapped_seqs;     /* live sequences on the host tier */
  int64_t swapped_tokens;   /* sum of their lengths */
  int64_t cached_blocks;      /* device blocks findable by prefix key */
  int64_t cached_free_blocks; /* of those, blocks waiting in the free queue */
} pkv_stats;

/* Human-readable name of a status code (static string). */
const char* pkv_status_string(pkv_status status);

/* Interface version; bumped whenever a signature, an entry point or the cache
 * layout changes. */
int32_t pkv_abi_version(void);

/* ---------------------------------------------------------------------------
 * Host block pool
 * ------------------------------------------------------------------------- */

/* Create a pool of num_blocks blocks of block_size token slots.
 * [P2] core idea items 1 and 4: fixed-size blocks, allocated on demand.
 * free_order: a permutation of [0, num_blocks) giving the initial order of the
 *   free queue (host array, read only, copied), or NULL for 0, 1, 2, ...
 *   Blocks are taken from the head of the queue and freed blocks join its tail
 *   (FIFO), so a freed block is reused as late as possible.
 * out: receives the pool; destroy it with pkv_pool_destroy.
 * Errors: INVALID_ARG (non-positive sizes, free_order not a permutation). */
pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                           pkv_pool** out);

/* Destroy a pool and every sequence in it.  NULL is ignored.  A utility with
 * no passage of its own: it releases the host metadata the pool owns. */
void pkv_pool_destroy(pkv_pool* pool);

/* Create an empty sequence (0 tokens, 0 blocks): a new request holds no
 * block until it grows onto one ([P2] core idea item 4 and [P1] core method,
 * allocation on demand).  Ids are 0, 1, 2, ... in creation
 * order (forks included) and are never reused. */
pkv_status pkv_seq_create(pkv_pool* pool, int32_t* out_seq);

/* Create a child that shares every block of parent: the child's table is a copy
 * of the parent's and each block's refcount rises by one.  [P4] beam-search
 * sharing; [P3] section 3 (sharing needs identical tokens and positions, which
 * a fork guarantees).  Errors: NO_SUCH_SEQ. */
pkv_status pkv_seq_fork(pkv_pool* pool, int32_t parent, int32_t* out_child);

/* Release a sequence (finish, cancel or time-out, [P2] key technical point 2,
 * [P3] section 3): refcounts drop in logical order and blocks that reach zero
 * join the tail of the free queue.  Errors: NO_SUCH_SEQ. */
pkv_status pkv_seq_free(pkv_pool* pool, int32_t seq);

/* Append counts[i] tokens to seqs[i] for i < n, in that order, all or nothing.
 * [P1]/[P2]: a sequence takes a new block only when it grows onto one.
 * [P3] section 3: a branch writing into a shared block that is not full copies
 * it first.  Per sequence with current length L and count c > 0:
 *   1. if L % B != 0 and the last block's refcount > 1: pop a fresh block,
 *      record the pair (old, new), decrement old, point the table at new;
 *   2. for each position p in [L, L + c): if p % B == 0 pop a fresh block;
 *      emit slot table[p / B] * B + p % B.
 * A block popped from the free queue loses its prefix key (eviction).
 * token_ids: host int32[sum(counts)], the new tokens' ids, sequence-major, or
 *   NULL.  With ids, each block the batch fills is registered for automatic
 *   prefix caching ([P4] prefix-caching paragraph) under
 *     key = FNV-1a-64( parent key as 8 little-endian bytes,
 *                      the block's B ids as 4-byte little-endian integers ),
 *   parent key = the previous block's key, 0 for a sequence's first block,
 *   unless that key is already registered; keys are registered after every
 *   block of the batch has been taken.  Without ids, the listed sequences
 *   (count > 0) stop being keyed for the rest of their life.
 * out_slots: host int64[slots_cap] receiving sum(counts) slots, sequence-major
 *   and in position order.
 * out_cow_pairs: host int32[2 * cow_cap] receiving (src, dst) block pairs; the
 *   caller must run pkv_copy_blocks on them before writing the new tokens.
 *   At most one pair per sequence, so cow_cap >= n always suffices.
 * out_n_cow: receives the number of pairs.
 * Errors (pool unchanged): INVALID_ARG (n < 0, NULL arrays, negative count,
 *   a sequence listed twice, slots_cap < sum(counts), cow_cap too small; in
 *   the last case *out_n_cow holds the number needed), NO_SUCH_SEQ,
 *   OUT_OF_BLOCKS (the batch needs more blocks than are free). */
pkv_status pkv_append_tokens(pkv_pool* pool, const int32_t* seqs, const int32_t* counts, int32_t n,
                             const int32_t* token_ids, int64_t* out_slots, int64_t slots_cap,
                             int32_t* out_cow_pairs, int32_t cow_cap, int32_t* out_n_cow);

/* Automatic prefix caching ([P4] the note that identical KV blocks can be
 * shared, and the prefix-caching paragraph; [P2] section 3, sharing of a
 * common prompt).  Create a sequence for a prompt of n_tokens ids (host
 * int32[n_tokens]) that starts with the longest run of its leading full
 * blocks already registered, at most (n_tokens - 1) / B of them so that at
 * least one prompt token is left to compute.  Block i hits when the key
 * chained from the hits before it is registered and the block holding it
 * stored the same parent key and the same B ids (a hash collision is a miss).
 * Each hit block's refcount rises by one; a hit block with refcount 0 leaves
 * the free queue from wherever it sits.  *out_cached_tokens receives the
 * tokens mapped (a multiple of B); the caller appends the remaining ids with
 * pkv_append_tokens (token_ids given) and writes only their keys and values.
 * A freed block keeps its key while it waits in the free queue; it loses it
 * when popped for new use or moved to the host tier (blocks brought back from
 * the host are not registered again).
 * Errors: INVALID_ARG (NULL pointers, n_tokens < 0). */
pkv_status pkv_seq_create_prefixed(pkv_pool* pool, const int32_t* token_ids, int32_t n_tokens, int32_t* out_seq,
                                   int32_t* out_cached_tokens);

/* The registered prefix keys and their device blocks, in increasing key order:
 * host out_keys[cap], out_blocks[cap]; *out_n = their number.
 * Errors: INVALID_ARG (cap too small; *out_n is still set). */
pkv_status pkv_pool_cached_blocks(const pkv_pool* pool, uint64_t* out_keys, int32_t* out_blocks, int32_t cap,
                                  int32_t* out_n);

/* Roll a sequence back to its first new_len tokens (speculative decoding
 * stages KV positions and drops the ones verification rejects, [P3] section
 * 5).  The table keeps ceil(new_len / B) blocks; the others are released in
 * logical order as pkv_seq_free releases them.  The sequence stops being keyed
 * for prefix caching.  A block left partly filled keeps its bytes (and any
 * prefix key) until the next append writes into it: a shared one is copied on
 * write, an unshared one is written in place and loses its key then.
 * new_len == current length changes nothing.
 * Errors: NO_SUCH_SEQ, SWAPPED, INVALID_ARG (new_len outside [0, length]). */
pkv_status pkv_seq_truncate(pkv_pool* pool, int32_t seq, int32_t new_len);

/* Dense block tables for seqs[0..n): host int32 out_tables[n][max_blocks],
 * row i = the physical blocks of seqs[i] in logical order, padded with -1;
 * out_context_lens[i] = its length in tokens ([P2] key technical point 1).
 * Errors: INVALID_ARG (a table longer than max_blocks, NULL arrays),
 * NO_SUCH_SEQ, SWAPPED (a sequence is swapped out: its blocks are host
 * blocks, which the device calls cannot read). */
pkv_status pkv_block_tables(const pkv_pool* pool, const int32_t* seqs, int32_t n, int32_t max_blocks,
                            int32_t* out_tables, int32_t* out_context_lens);

/* Length in tokens and number of blocks of one sequence (either tier).
 * Errors: NO_SUCH_SEQ. */
pkv_status pkv_seq_info(const pkv_pool* pool, int32_t seq, int32_t* out_len, int32_t* out_num_blocks);

/* Pool counters ([P3] Eq. (2)-(3) and section 6's accounting categories). */
pkv_status pkv_pool_stats(const pkv_pool* pool, pkv_stats* out);

/* Refcount of one physical block, or -1 for an id out of range: the number
 * of block tables that map it ([P3] section 3: a shared block's lifetime is
 * tied to a reference count; [P4] beam-search sharing). */
int32_t pkv_block_refcount(const pkv_pool* pool, int32_t block);

/* Copy the free queue, head first, into host out[cap]; *out_n = its length.
 * Errors: INVALID_ARG if cap < the queue length. */
pkv_status pkv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* out_n);

/* Check the pool's invariants, per tier: each block's refcount equals the
 * number of live tables of that tier holding it; a free block has refcount 0
 * and appears once; free plus used equals capacity; each table has
 * ceil(length / B) entries; the prefix-key map and the keyed blocks match one
 * to one.  [P3] section 3 asks tests to check refcounts and
 * reuse.  Errors: REFCOUNT. */
pkv_status pkv_pool_validate(const pkv_pool* pool);

/* Preemption by swapping ([P2] section 4: waiting sequences' KV cache moves
 * out to CPU memory and comes back when needed, like an operating system's
 * swap; [P4] "Preemption": swapping, which moves poorly with small blocks).
 *
 * pkv_pool_set_host_blocks: give the pool a host tier of num_host_blocks
 * blocks of the same size, ids 0..num_host_blocks-1, free queue in id order.
 * Allowed while no sequence is swapped out (it resets the host tier).
 * Errors: INVALID_ARG. */
pkv_status pkv_pool_set_host_blocks(pkv_pool* pool, int32_t num_host_blocks);

/* Move seqs[0..n) to the host tier (pkv_swap_out) or back (pkv_swap_in), all
 * or nothing.  The list must be a whole sharing group: every holder of each of
 * its blocks is listed (beams of one request move together).  The blocks are
 * met in list order, then logical order; each distinct block takes the next
 * block from the other tier's free queue, which inherits its refcount, and the
 * block it leaves joins the tail of its own tier's free queue.  The tables are
 * renamed to the new ids.
 * out_pairs: host int32[2 * pairs_cap] receiving (from, to) block pairs in the
 *   order met: (device, host) for a swap-out, (host, device) for a swap-in.
 *   The caller copies the blocks with pkv_swap_blocks before the blocks left
 *   behind are written again (a swap-out's device blocks are free at once).
 * out_n_pairs: receives the number of pairs.
 * Errors (pool unchanged): INVALID_ARG (n < 0, NULL arrays, a sequence listed
 *   twice, a block also held by an unlisted sequence, pairs_cap too small, in
 *   which case *out_n_pairs holds the number needed), NO_SUCH_SEQ, SWAPPED (a
 *   sequence already on the target tier), OUT_OF_BLOCKS (the target tier has
 *   too few free blocks). */
pkv_status pkv_swap_out(pkv_pool* pool, const int32_t* seqs, int32_t n, int32_t* out_pairs, int32_t pairs_cap,
                        int32_t* out_n_pairs);
pkv_status pkv_swap_in(pkv_pool* pool, const int32_t* seqs, int32_t n, int32_t* out_pairs, int32_t pairs_cap,
                       int32_t* out_n_pairs);

/* One sequence's table in its current tier: host int32 out[cap] receives its
 * block ids in logical order, *out_n their number, *out_on_host (may be NULL)
 * 1 if it is swapped out, else 0.  Errors: NO_SUCH_SEQ, INVALID_ARG (cap too
 * small; *out_n is still set). */
pkv_status pkv_seq_table(const pkv_pool* pool, int32_t seq, int32_t* out, int32_t cap, int32_t* out_n,
                         int32_t* out_on_host);

/* Refcount of one host block, or -1 for an id out of range. */
int32_t pkv_host_block_refcount(const pkv_pool* pool, int32_t block);

/* Copy the host free queue, head first (as pkv_pool_free_list). */
pkv_status pkv_pool_host_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* out_n);

/* ---------------------------------------------------------------------------
 * Device calls (HIP, gfx950).  All pointers are device memory owned by the
 * caller, 16-byte aligned (pkv_swap_blocks also takes page-locked host
 * memory); `stream` may be NULL (the default stream).
 *
 * Debug mode: with the environment variable PKV_DEBUG set to anything but ""
 * or "0" (read once per process), pkv_reshape_and_cache and pkv_copy_blocks
 * also copy their slots / pairs to the host, wait for the stream, and return
 * INVALID_ARG when two of them would write the same slot / block.
 * ------------------------------------------------------------------------- */

/* Write token i's key and value (k_new, v_new: [num_tokens][H_kv][d], the
 * cache's scalar type) into slot slots[i] of the caches, in the layout above.
 * Decoding computes only the new token's K/V and reads the rest from the cache
 * ([P4] KV-cache introduction; [P2] core idea item 3).
 * slots: device int64[num_tokens]; a slot of -1 is skipped, a slot at or past
 * num_blocks * B is skipped as well.  Slots must be distinct within a call
 * (two writers of one slot race; checked in debug mode).
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
pkv_status pkv_reshape_and_cache(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 const int64_t* slots, int32_t num_tokens, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 int32_t kv_dtype, hipStream_t stream);

/* Copy whole blocks (every head and slot of both caches) src -> dst for each
 * pair: the device half of copy-on-write ([P3] section 3).
 * pairs: device int32[n_pairs][2] as returned by pkv_append_tokens.  Every pair
 * is copied at once, so the dst blocks must be distinct and no dst may also
 * be a src in the same call, its own pair's included (the pool never produces
 * either; debug mode refuses both with INVALID_ARG).  Pairs with an id out of
 * [0, num_blocks) are skipped.
 * block_bytes: bytes of one block in one cache, H_kv * B * d * scalar size.
 * Errors: INVALID_ARG (block_bytes not a positive multiple of 16), HIP. */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t n_pairs,
                           int32_t num_blocks, int64_t block_bytes, hipStream_t stream);

/* Copy whole blocks between two cache pairs: for each pair (i, j),
 * dst_k block j <- src_k block i and dst_v block j <- src_v block i.  The
 * device half of swapping: src on the device and dst in host memory for a
 * swap-out, the reverse for a swap-in ([P2] section 4; [P4] "Preemption").
 * One kernel moves every pair, whatever the block size.
 * src_k, src_v, dst_k, dst_v: 16-byte aligned; each either device memory or
 *   page-locked host memory from the HIP allocator (hipHostMalloc; a pinned
 *   torch tensor), which the kernel reads or writes over the host link.
 *   Other host memory is refused.  The source and destination ranges must not
 *   overlap.
 * pairs: int32[n_pairs][2] in device or page-locked host memory, as returned
 *   by pkv_swap_out / pkv_swap_in; a pair with an id outside [0, src_blocks) or
 *   [0, dst_blocks) is skipped.  Destination blocks must be distinct.
 * block_bytes: bytes of one block in one cache (a positive multiple of 16).
 * Errors: INVALID_ARG (sizes, alignment, memory the GPU cannot reach), HIP. */
pkv_status pkv_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v, const int32_t* pairs,
                           int32_t n_pairs, int32_t src_blocks, int32_t dst_blocks, int64_t block_bytes,
                           hipStream_t stream);

/* Bytes of workspace pkv_paged_attention_decode, pkv_decode_step and the
 * two-stage calls need for these sizes (0 when no sequence can span more than
 * one partition, i.e. partition_size == 0 or max_context_len <= it).  A
 * utility with no passage of its own: the pages describe no split of a
 * context; splitting long contexts across workgroups and combining them by
 * log-sum-exp weights is this library's way to fill the GPU with few
 * sequences.  With up to 4096 sequences the workspace holds two records per
 * workgroup of the persistent grid (at most 2048 workgroups): about
 * 2 * min(2048, sequences * H_kv * partitions) * ((H_q / H_kv) * (d + 2) * 4 + 32)
 * bytes whatever the lengths (17 MB at most for 64/8 heads and d 128); above
 * 4096 sequences it holds one slot per (sequence, query head, partition).
 * Errors: 0 for invalid sizes. */
size_t pkv_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                     int32_t partition_size);

/* Decode attention, one query token per sequence, reading K/V through block
 * tables ([P2] key technical point 1; [P1] "custom kernel fusing table lookup,
 * block fetch and attention"; [P3] section 1: paging changes storage, not the
 * result).  For sequence s, query head h and g = h / (H_q / H_kv):
 *   out[s][h] = sum_{t < n_s} softmax_t(scale * q[s][h] . K_s[t][g]) V_s[t][g]
 * where K_s[t] is the key of token position t read through block_tables[s].
 *   out: fp32 [num_seqs][H_q][d].
 *   q: [num_seqs][H_q][d] in the cache's scalar type.
 *   block_tables: device int32 [num_seqs][max_blocks] (entries past the
 *     sequence's last block are not read).
 *   context_lens: device int32 [num_seqs]; n_s counts the token just written.
 *     n_s == 0 gives an all-zero output row; n_s < 0, n_s > max_context_len,
 *     n_s > max_blocks * B, or a block id outside [0, num_blocks) gives NaN.
 *   scale: any finite value (negative and zero included).
 *   partition_size: tokens per context partition (a multiple of B), or 0 for
 *     one partition per sequence.  The work is split at partition boundaries
 *     (or inside a partition when every workgroup has plenty of work): a
 *     sequence is computed as one or more segments, and the segments' partial
 *     results are combined by log-sum-exp weights (split context).  With up
 *     to 4096 sequences the combination happens in the same kernel: the
 *     workgroup that computes a sequence's last segment waits for the others'
 *     partials and combines them in token order; above that, a second kernel
 *     does.  Splitting needs `workspace` (device, workspace_bytes >=
 *     pkv_attention_workspace_bytes(...), 16-byte aligned) whenever a
 *     sequence can span more than one partition.  Its contents are private
 *     and need no initialisation (the hand-over between workgroups matches a
 *     64-bit value derived from what the previous call left, so stale or
 *     arbitrary contents do not leak into results, except with probability
 *     2^-64 per record); one workspace serves one call at a time, so calls
 *     in flight on different streams need different workspaces.
 * Arithmetic: fp32 accumulation; bf16 inputs are multiplied exactly and summed
 * in fp32 (probabilities enter the value product as two bf16 terms whose sum
 * is within 2^-16 of the fp32 value).  Errors: INVALID_ARG, UNSUPPORTED,
 * WORKSPACE, HIP. */
pkv_status pkv_paged_attention_decode(float* out, const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks, int32_t max_context_len, float scale,
                                      int32_t partition_size, void* workspace, size_t workspace_bytes,
                                      int32_t kv_dtype, hipStream_t stream);

/* One decode step: write each sequence's new token, then attend.  k_new and
 * v_new: device [num_seqs][H_kv][d] in the cache's scalar type, the key and
 * value of the token at position n_s - 1 of sequence s.  Equivalent to
 * pkv_reshape_and_cache with slot = block_tables[s][(n_s - 1) / B] * B +
 * (n_s - 1) % B (the allocator's slot for that token; sequences with an
 * invalid length or block id are not written), followed by
 * pkv_paged_attention_decode with the remaining arguments (k_cache and v_cache
 * serve both); the output and the caches are bit for bit those of the two
 * calls.  With up to 4096 sequences the write happens inside the attention
 * kernel: the tokens are stored at the start of the launch, and the
 * workgroup that reads a sequence's last token takes that token's key and
 * value from k_new and v_new, so no read waits for the stores (bf16 with
 * B = 32: each workgroup stores the tokens it reads first and waits for
 * them) ([P2] key technical point 1: the kernel fetches blocks through the
 * table; [P2] core idea: each step appends one token per sequence).
 * Errors: as pkv_paged_attention_decode, and INVALID_ARG for a missing or
 * misaligned k_new / v_new. */
pkv_status pkv_decode_step(const void* k_new, const void* v_new, float* out, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, int32_t max_blocks, int32_t max_context_len,
                           float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                           int32_t kv_dtype, hipStream_t stream);

/* pkv_decode_step for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid it): the same
 * kernels and results, with the split-context workspace taken from a static
 * device array of the library (18 MiB, one per GPU, held until the process
 * ends) instead of a caller argument.  It covers every batch of up to 4096
 * sequences with at most 2048 KV heads (whose workspace is at most about
 * 17 MB); a batch that needs more returns WORKSPACE before any device work.
 * The array needs no clearing between calls, but every call on one GPU uses
 * it: calls that overlap on one GPU (different streams, threads or
 * processes' streams on the same device) race and must be serialised.  No
 * hipMalloc, hipFree or other allocation happens inside.  Other errors as
 * pkv_decode_step. */
pkv_status pkv_decode_step_static(const void* k_new, const void* v_new, float* out, const void* q,
                                  const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t max_blocks, int32_t max_context_len, float scale, int32_t partition_size,
                                  int32_t kv_dtype, hipStream_t stream);

/* Runs of causal queries over the paged cache ([P3] section 5: blockwise
 * attention composes with paging, and speculative decoding stages KV positions
 * that verification keeps or rolls back; [P4] "Preemption": a whole prompt's
 * KV is computed in one parallel pass).  Sequence s owns query rows
 * query_start[s] .. query_start[s+1] - 1, a run of q_s rows that are its last
 * q_s positions; row i is at position p = n_s - q_s + i and, for query head h
 * and g = h / (H_q / H_kv),
 *   out[row][h] = sum_{t <= p} softmax_t(scale * q[row][h] . K_s[t][g]) V_s[t][g].
 * q_s = n_s is a prompt's own attention; a shorter run is the rest of a prompt
 * whose leading blocks came from the prefix cache, or a set of speculated
 * tokens under verification.  Every row's K/V (the run's own included) must
 * already be in the cache (pkv_reshape_and_cache at the run's slots).
 *   out: fp32 [num_query_rows][H_q][d]; q: [num_query_rows][H_q][d] in the
 *     cache's scalar type.
 *   query_start: device int32 [num_seqs + 1], non-decreasing.
 *   block_tables, context_lens: as for pkv_paged_attention_decode.
 *   seq_order: device int32 [num_seqs], a permutation of the sequences giving
 *     the order in which their work starts (longest first evens out the end
 *     of a ragged batch), or NULL for 0, 1, 2, ...  It changes scheduling
 *     only, never the results.  An entry outside [0, num_seqs) is skipped;
 *     on the runs kernel (see Paths), a sequence the order leaves out is not
 *     computed (its rows are left as they were, or unspecified when the call
 *     splits contexts); the decode kernel's pass ignores the order.
 *   max_query_len: a bound on every q_s (it sizes the launch).
 *   workspace: device memory of workspace_bytes >= the value of
 *     pkv_attention_multi_workspace_bytes(...) for these sizes, 16-byte
 *     aligned, or NULL; with it, long contexts of few (sequence, KV head)
 *     pairs are split (see there).  Its contents are private.
 * Rows of a run with q_s > n_s, q_s > max_query_len, n_s > max_context_len or
 * n_s > max_blocks * B are NaN (for q_s > max_query_len, only its first
 * max_query_len rows are written); a row that reads a block id outside
 * [0, num_blocks) is NaN, and so may be the rows computed with it; a run with
 * query_start[s] < 0 or query_start[s+1] > num_query_rows is not written.
 * Supported shapes and dtypes as for decode.  Arithmetic: fp32 accumulation,
 * products on the matrix cores; bf16 probabilities enter the value product as
 * two bf16 terms.  Allocates nothing.
 * Paths: runs of at most 16 / G queries (max_query_len * H_q / H_kv <= 16;
 * speculative verification) with at most 4096 sequences go to the decode
 * kernel's listed pass, the queries of a run as further matrix-core columns of
 * one persistent, cost-balanced pass over 512-token partitions (256 for a
 * small batch: num_seqs * ceil(max_context_len / 16) under 6 * (512 / H_kv)
 * * 40); that path needs the workspace when a context exceeds a partition,
 * and without one the call uses the runs kernel, unsplit.  Other batches use the runs kernel,
 * except a batch with max_query_len > 16 / G and num_query_rows <
 * num_seqs * max_query_len (some runs are shorter than the longest: prompt
 * chunks beside decodes in one step), which takes two launches on the
 * stream: the runs of at most 16 / G queries on the decode kernel's pass
 * (when it fits, as above), then the longer ones on the runs kernel.  The
 * environment variable PKV_MULTI_PATH set to "runs" (read at each call) keeps
 * every run on the runs kernel.  Both paths meet the same contract and
 * tolerances; their rows differ in rounding.
 * Tuning: where a pair has more than 64 rows, a workgroup serves 128 rows
 * (two row tiles per wave) when the batch's rows fill the GPU, else 64; the
 * environment variable PKV_MULTI_TILES set to "1" or "2" (read at each call)
 * forces the choice.  Both give the same rows.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE (given but smaller than
 * pkv_attention_multi_workspace_bytes for these sizes, or misaligned), HIP. */
pkv_status pkv_paged_attention_multi(float* out, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     const int32_t* query_start, const int32_t* seq_order, int32_t num_seqs,
                                     int32_t num_query_rows,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int32_t num_blocks, int32_t max_blocks,
                                     int32_t max_context_len, int32_t max_query_len, float scale, void* workspace,
                                     size_t workspace_bytes, int32_t kv_dtype, hipStream_t stream);

/* Bytes of workspace pkv_paged_attention_multi uses to split long contexts (0
 * when it would not split them): the larger of the two paths' needs.  The
 * decode kernel's path (runs of at most 16 / G queries, see there) cuts
 * contexts into 512- or 256-token partitions and between workgroups, with
 * records per workgroup.  On the runs
 * kernel a context is split when every run's rows (max_query_len * H_q / H_kv)
 * fit one 64-row block and the batch has too few (sequence, KV head) pairs to
 * fill the GPU: each pair's context is cut into splits of at least 256 tokens,
 * computed apart and combined with log-sum-exp weights.  With no workspace the
 * call does not split. */
size_t pkv_attention_multi_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t max_context_len, int32_t max_query_len);

/* pkv_paged_attention_decode as two launches, for callers that schedule or
 * time the combination separately.  Same arguments and errors; issue
 * `partitions` then `reduce` on one stream, with the same workspace; the
 * output has the same bits as the one-call path.
 * pkv_paged_attention_partitions: one pass over every (sequence, KV head,
 *   segment); writes the final rows of sequences computed in one segment, and
 *   the (acc, max, sum) of every other segment with its extent into the
 *   workspace.
 * pkv_paged_attention_reduce: combines the segments of every sequence that
 *   has more than one (log-sum-exp weights); a no-op when none has. */
pkv_status pkv_paged_attention_partitions(float* out, const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_tables, const int32_t* context_lens,
                                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                          int32_t max_blocks, int32_t max_context_len, float scale,
                                          int32_t partition_size, void* workspace, size_t workspace_bytes,
                                          int32_t kv_dtype, hipStream_t stream);
pkv_status pkv_paged_attention_reduce(float* out, const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_blocks, int32_t max_blocks,
                                      int32_t max_context_len, float scale, int32_t partition_size,
                                      void* workspace, size_t workspace_bytes, int32_t kv_dtype,
                                      hipStream_t stream);

/* Calibration: read `bytes` (a multiple of 16) of device memory once with a
 * plain streaming kernel (16-byte loads, 16 in flight per thread) and discard
 * the data.  Used to measure the practical HBM read ceiling next to the
 * attention kernel's KV read rate.  sink: device uint32[1], never written in
 * practice.  Errors: INVALID_ARG, HIP. */
pkv_status pkv_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
