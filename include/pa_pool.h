/*
 * pa_pool.h - host-side KV block pool and step-input builder of libpa.so.
 *
 * The bookkeeping half of PagedAttention, on the CPU, in the calling process
 * (llm-stack-book 7.3 "vLLM: Architecture, PagedAttention & Internals",
 * sections "The free list and the block table", "Copy-on-write for shared
 * blocks" and "The forward step in detail"; modernaiengineering.com lesson
 * 13.15 "vLLM: High-Throughput Serving with PagedAttention", sections "How
 * PagedAttention stores a request" and "How PagedAttention shares memory"):
 *
 *  - the pool is a free list of physical block ids; the block at the end of
 *    the list is handed out first and a released block goes back onto the end;
 *  - a sequence of n tokens holds ceil(n / block_size) blocks, taken as it
 *    grows, never ahead of need;
 *  - every held block has a reference count: sharing (parallel samples, beam
 *    search, a reused prompt prefix) raises it, releasing lowers it, and a
 *    block goes back to the free list when nobody holds it;
 *  - a sequence about to write into a block others hold gets a private copy
 *    first (copy-on-write): the caller then copies the block's K/V on the GPU
 *    (pa_copy_blocks in pa.h);
 *  - pa_prepare_step turns the tables into what the GPU kernels take: a slot
 *    per token being written, its position, padded block tables and context
 *    lengths.
 *
 * All pointers here are HOST pointers owned by the caller. A pool is not
 * thread-safe: one owner at a time. Every call validates first and changes
 * nothing when it returns an error (pa_status from pa.h; PA_ERR_NO_BLOCKS
 * when the pool has too few free blocks).
 */
#ifndef PA_POOL_H_
#define PA_POOL_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_pool pa_pool;

/*
 * pa_pool_create - a pool of num_blocks blocks of block_size tokens.
 *   free_order   optional permutation of [0, num_blocks): the initial free list,
 *                its last entry handed out first. NULL: 0, 1, ..., num_blocks-1
 *                (block num_blocks-1 handed out first).
 *   out          receives the pool (release it with pa_pool_destroy).
 * PA_ERR_INVALID_ARG for a bad shape or an order that is not a permutation.
 */
int pa_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, pa_pool** out);

/* pa_pool_destroy - frees the pool (NULL is ignored). */
void pa_pool_destroy(pa_pool* pool);

/* pa_pool_num_free - free blocks, or -1 for a NULL pool. */
int32_t pa_pool_num_free(const pa_pool* pool);

/* pa_pool_ref_count - holders of `block` (0 when free), -1 for a bad id. */
int32_t pa_pool_ref_count(const pa_pool* pool, int32_t block);

/* pa_pool_blocks_for - ceil(num_tokens / block_size) (0 for num_tokens <= 0). */
int64_t pa_pool_blocks_for(const pa_pool* pool, int64_t num_tokens);

/*
 * pa_pool_allocate - a fresh block table for num_tokens tokens, all or
 * nothing: table[0 .. *num_blocks) receives the blocks in the order taken.
 *   capacity     entries table can hold (PA_ERR_INVALID_ARG if too few).
 */
int pa_pool_allocate(pa_pool* pool, int64_t num_tokens, int32_t* table, int32_t capacity,
                     int32_t* num_blocks);

/*
 * pa_pool_append_slot - make the table cover token position cur_len (the token
 * about to be written), appending blocks to table[*table_len ...] and updating
 * *table_len. *taken receives the last block taken, or -1 when the table
 * already covered the position (every decode step except the ones that start
 * a block).
 */
int pa_pool_append_slot(pa_pool* pool, int32_t* table, int32_t* table_len, int32_t capacity,
                        int64_t cur_len, int32_t* taken);

/* pa_pool_share - one more holder for each of blocks[0 .. n) (all must be held). */
int pa_pool_share(pa_pool* pool, const int32_t* blocks, int32_t n);

/* pa_pool_release - one holder fewer for each block, in order; blocks nobody
 * holds go back onto the free list. */
int pa_pool_release(pa_pool* pool, const int32_t* blocks, int32_t n);

/*
 * pa_pool_make_writable - copy-on-write for table[idx], 0 <= idx < table_len.
 * If others hold that block, table[idx] becomes a fresh block and
 * (*src, *dst) = (old, new) is the block copy the caller must run on the GPU
 * before writing; otherwise *src = *dst = -1.
 */
int pa_pool_make_writable(pa_pool* pool, int32_t* table, int32_t table_len, int32_t idx, int32_t* src,
                          int32_t* dst);

/*
 * pa_prepare_step - inputs of one engine step. Sequence i has the block table
 * tables[table_offsets[i] .. table_offsets[i+1]) and processes num_new[i]
 * tokens (a prompt chunk, or 1 for decode) after num_computed[i] stored ones.
 * For every such token, in sequence order:
 *     positions[t]    = p = num_computed[i] + j
 *     slot_mapping[t] = table[p / block_size] * block_size + p % block_size
 * block_tables [num_seqs, max_blocks] receives each table padded with -1, and
 * context_lens[i] = num_computed[i] + num_new[i]. *num_tokens receives the
 * token count. PA_ERR_INVALID_ARG if a table is longer than max_blocks, does
 * not cover its tokens, a length exceeds INT32_MAX, or token_capacity is too
 * small.
 */
int pa_prepare_step(int32_t num_seqs, const int32_t* tables, const int64_t* table_offsets,
                    const int64_t* num_computed, const int64_t* num_new, int32_t block_size,
                    int32_t max_blocks, int64_t* slot_mapping, int64_t* positions, int32_t* block_tables,
                    int32_t* context_lens, int64_t token_capacity, int64_t* num_tokens);

#ifdef __cplusplus
}
#endif

#endif /* PA_POOL_H_ */
