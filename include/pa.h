/*
 * pa.h - C ABI of libpa.so: paged KV-cache decode attention for AMD MI355X (gfx950).
 *
 * The library holds the data-plane half of PagedAttention as the pages describe
 * it: a per-layer KV pool carved into fixed-size blocks, a block table per
 * sequence mapping logical blocks to physical ones, a slot mapping telling
 * where each new token's K/V is written, and a decode kernel that follows the
 * block table (llm-stack-book 7.3 "vLLM: Architecture, PagedAttention &
 * Internals", sections "PagedAttention in one paragraph" and "The forward step
 * in detail"; stanleyjacob.dev "vLLM", Part V "The attention backend dispatch
 * layer": a backend runs attention given the query, the paged KV pool and the
 * block tables).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor arguments are DEVICE pointers, row-major and contiguous, owned
 *    by the caller. The library never allocates, frees or synchronises; every
 *    launch goes on the caller's `stream` (a hipStream_t passed as void*, NULL
 *    for the default stream) and returns immediately. Work on one stream is
 *    ordered, so reshape_and_cache followed by a decode on the same stream sees
 *    the new token.
 *  - Base pointers of tensors must be 16-byte aligned.
 *  - Element type (`dtype`): PA_DTYPE_F32 (IEEE float32) or PA_DTYPE_BF16
 *    (bfloat16 stored as 16-bit words). Query, caches, new K/V and `out` share
 *    it; accumulation is always float32.
 *  - Layouts:
 *        query, out        [num_seqs, num_heads, head_size]
 *        key_cache,
 *        value_cache       [num_blocks, block_size, num_kv_heads, head_size]
 *        block_tables      int32 [num_seqs, max_blocks_per_seq]
 *        context_lens      int32 [num_seqs]   (tokens stored, including the
 *                                              token written this step)
 *        key, value        [num_tokens, num_kv_heads, head_size]
 *        slot_mapping      int64 [num_tokens]
 *  - Supported shapes: block_size == 16; head_size in {64, 128};
 *    num_heads % num_kv_heads == 0 and num_heads / num_kv_heads <= 16;
 *    num_kv_heads * head_size * 4 < 2^24 (a token row under 16 MiB).
 *  - Host-side checks (shapes, enums, null or misaligned pointers, workspace
 *    size) return a non-zero pa_status before any GPU work is queued. Device
 *    CONTENTS are the caller's contract: block ids in [0, num_blocks),
 *    context_lens[i] <= max_blocks_per_seq * block_size, distinct slots. The
 *    kernels clamp out-of-range block ids and lengths, and skip out-of-range
 *    slots, so bad contents give unspecified numbers, never an out-of-bounds
 *    access.
 *  - Query head h reads kv head h / (num_heads / num_kv_heads) (contiguous GQA
 *    groups).
 *  - No entry point uses atomics; results are bit-identical run to run and do
 *    not depend on where the physical blocks sit in the pool.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_dtype {
  PA_DTYPE_F32 = 0,
  PA_DTYPE_BF16 = 1
} pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, negative size, bad enum   */
  PA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (block_size, head_size)   */
  PA_ERR_WORKSPACE = 3,    /* workspace smaller than pa_decode_split_workspace_bytes */
  PA_ERR_HIP = 4,          /* the HIP runtime refused a launch                     */
  PA_ERR_NO_BLOCKS = 5     /* a block pool (pa_pool.h) has too few free blocks     */
} pa_status;

/*
 * pa_reshape_and_cache - write each new token's K and V into its cache slot.
 *
 * The freshly computed K and V of every token are scattered into the paged
 * pool at slot_mapping (llm-stack-book 7.3, "The forward step in detail"),
 * where a slot is physical_block * block_size + offset.
 *
 *   key, value        [num_tokens, num_kv_heads, head_size], read.
 *   key_cache,
 *   value_cache       [num_blocks, block_size, num_kv_heads, head_size], written
 *                     at rows slot_mapping[t] only; every other row is untouched.
 *   slot_mapping      int64 [num_tokens]. slot < 0 marks a padding token and is
 *                     skipped; slot >= num_blocks*block_size is skipped too.
 *                     Two tokens with the same slot is a caller error.
 *   num_tokens        may be 0 (nothing is launched).
 *
 * The copy is bitwise: no conversion, no rounding.
 * Returns PA_OK or an error status (see conventions).
 */
int pa_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                         const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                         int32_t dtype, void* stream);

/*
 * FP8 KV caches.
 *
 * The pages name an FP8 KV cache as a way to enlarge the pool (llm-stack-book
 * 7.3, "The knobs that actually matter", item 5) without fixing a format. This
 * library's reading: caches hold OCP FP8 E4M3 codes (1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits; largest finite 448; S.1111.111 is NaN; no
 * infinity), one code per element, in the same [num_blocks, block_size,
 * num_kv_heads, head_size] layout, with one float32 scale per cache (k_scale,
 * v_scale > 0). A value x is stored as the code nearest to float32(x)/scale
 * (IEEE float32 division; ties to even; magnitudes above 448, infinities
 * included, saturate to 448; NaN is stored as a NaN code with x's sign) and
 * reads back as value(code) * scale.
 */

/*
 * pa_reshape_and_cache_fp8 - pa_reshape_and_cache into FP8 caches: each new
 * token's K and V (dtype: PA_DTYPE_BF16 or PA_DTYPE_F32, 16-byte aligned) are
 * quantized with k_scale / v_scale and written to their slot (caches 8-byte
 * aligned). Negative and out-of-pool slots are skipped.
 */
int pa_reshape_and_cache_fp8(const void* key, const void* value, uint8_t* key_cache, uint8_t* value_cache,
                             const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                             int32_t block_size, int32_t num_kv_heads, int32_t head_size, int32_t dtype,
                             float k_scale, float v_scale, void* stream);

/*
 * pa_decode_fp8 - pa_decode over FP8 caches: attention on the caches' values
 * value(code) * scale. Query and out are bf16 (dtype PA_DTYPE_BF16; anything
 * else is PA_ERR_UNSUPPORTED); lse_out and seq_order as for pa_decode. The
 * keys' scale folds into the scores (s_t = scale * k_scale * <q, K_code_t>),
 * the values' into the normalised output; every code converts exactly to
 * bf16/float32, so this reads half the bytes of a bf16 cache for the same
 * arithmetic on the stored values.
 */
int pa_decode_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                  const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                  int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int64_t num_blocks,
                  int32_t block_size, float scale, float k_scale, float v_scale, int32_t dtype, float* lse_out,
                  const int32_t* seq_order, void* stream);

/*
 * pa_reshape_and_decode_fp8 - pa_reshape_and_cache_fp8 of one decode step's
 * new tokens followed by pa_decode_fp8, in one launch: the FP8 counterpart of
 * pa_reshape_and_decode (same three slot cases). key, value [num_seqs, H_kv,
 * head_size] are bf16 (dtype PA_DTYPE_BF16, like query and out); each row is
 * quantized with k_scale / v_scale exactly as pa_reshape_and_cache_fp8 does,
 * written to slot_mapping[i], and used as position n - 1's codes when the
 * slot is that position's. Other arguments as pa_decode_fp8.
 */
int pa_reshape_and_decode_fp8(void* out, const void* query, const void* key, const void* value,
                              const int64_t* slot_mapping, uint8_t* key_cache, uint8_t* value_cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                              int64_t num_blocks, int32_t block_size, float scale, float k_scale, float v_scale,
                              int32_t dtype, float* lse_out, const int32_t* seq_order, void* stream);

/*
 * pa_copy_blocks - whole-block copies: the GPU half of copy-on-write.
 *
 * When a sequence must write into a block that others still read, it gets a
 * fresh block holding a copy of the shared one (llm-stack-book 7.3, section
 * "Copy-on-write for shared blocks"; the host side is pa_pool_make_writable in
 * pa_pool.h). For every pair p, block block_mapping[p][1] of both caches
 * receives block block_mapping[p][0] (all block_size token rows, all kv
 * heads), bitwise.
 *
 *   key_cache,
 *   value_cache       [num_blocks, block_size, num_kv_heads, head_size], device.
 *   block_mapping     int64 [num_pairs, 2] (source, destination), device. A
 *                     pair naming a block outside [0, num_blocks) is skipped.
 *                     Destinations must be distinct and must not be the source
 *                     of another pair (the pairs run in parallel).
 *   num_pairs         may be 0 (nothing is launched).
 * Returns PA_OK or an error status.
 */
int pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping, int64_t num_pairs,
                   int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                   int32_t dtype, void* stream);

/*
 * pa_decode - one decode step of paged attention, one pass over each context.
 *
 * For every sequence i and query head h, with n = context_lens[i] and
 * kvh = h / (num_heads / num_kv_heads):
 *     K_t = key_cache[block_tables[i][t / block_size]][t % block_size][kvh]
 *     s_t = scale * <query[i][h], K_t>            for t in [0, n)
 *     out[i][h] = sum_t softmax(s)_t * V_t
 * The arithmetic is ordinary attention; only the addressing goes through the
 * block table (llm-stack-book 7.3, "PagedAttention in one paragraph"). The
 * softmax is evaluated online over the streamed blocks (stanleyjacob.dev
 * "vLLM", Part IV "Stage 6: The forward pass").
 *
 * Work is cut into jobs of one (sequence, kv head): one workgroup of the tile
 * kernel (the multi-query kernel with one new token per sequence, P*V on the
 * matrix cores) per job, handed out by the hardware in seq_order; 8-wave
 * workgroups when every resident 4-wave workgroup would get at most one job,
 * 4-wave ones otherwise (PA_OPT_TILE_WAVES).
 *
 *   out               [num_seqs, num_heads, head_size], written (dtype).
 *   lse_out           optional float32 [num_seqs, num_heads]: ln sum_t exp(s_t).
 *                     NULL to skip.
 *   seq_order         optional int32 [num_seqs], a permutation of the sequence
 *                     indices: the order in which sequences are handed out.
 *                     Longest-first evens out the work of the workgroups. It is
 *                     a schedule only: every output is bit-identical to the
 *                     NULL (natural order) result. Entries outside
 *                     [0, num_seqs) are clamped.
 *   n = 0             gives out = 0 and lse = -inf.
 *   Table entries at index >= ceil(n / block_size) never affect the result
 *                     and no cache block they name is read, but the first 16
 *                     entries of a row may be read before n is known (the
 *                     row holds max_blocks_per_seq entries, so this stays
 *                     inside the table).
 * Returns PA_OK or an error status.
 */
int pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
              const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
              int32_t num_kv_heads, int32_t head_size, int64_t num_blocks, int32_t block_size,
              float scale, int32_t dtype, float* lse_out, const int32_t* seq_order, void* stream);

/*
 * pa_multi_query_fp8 - pa_multi_query over FP8 (E4M3) caches: attention on
 * value(code) * scale, bf16 query and out (dtype PA_DTYPE_BF16, anything else
 * is PA_ERR_UNSUPPORTED), k_scale folded into the scores and v_scale into the
 * normalised output, as in pa_decode_fp8. Other arguments as pa_multi_query.
 */
int pa_multi_query_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                       const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_size, int64_t num_blocks, int32_t block_size, float scale,
                       float k_scale, float v_scale, int32_t dtype, float* lse_out, void* stream);

/*
 * pa_multi_query_split_workspace_bytes - workspace pa_multi_query_split needs:
 * float32 partials [num_tokens, num_heads, slots, head_size], then float32
 * log-sum-exps [num_tokens, num_heads, slots], each 256-byte aligned, with
 * slots = ceil(max_context_len / partition_size). Returns 0 for invalid
 * arguments.
 */
size_t pa_multi_query_split_workspace_bytes(int32_t num_tokens, int32_t num_heads, int32_t head_size,
                                            int32_t max_context_len, int32_t partition_size);

/*
 * pa_multi_query_split_partition_size - partition length (tokens, a multiple
 * of 256) for pa_multi_query_split on this device, or 0 when the plain
 * pa_multi_query should be used: the step's tiles already give at least one
 * workgroup per compute unit, or the longest context is not longer than one
 * partition would be. Cuts to about six workgroups per compute unit
 * otherwise. Shape arguments as pa_multi_query; returns 0 for invalid ones.
 */
int32_t pa_multi_query_split_partition_size(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                            int32_t num_kv_heads, int32_t head_size, int32_t dtype,
                                            int32_t max_context_len);

/*
 * pa_multi_query_split - the same result as pa_multi_query, with every
 * context cut into partitions of partition_size tokens (P) merged by the
 * log-sum-exp rule of pa_merge_partitions: each tile of new tokens (see
 * pa_multi_query) is one workgroup per (tile, partition, kv head), so long
 * contexts no longer set the time of a step that has few tiles. Partition p
 * of a tile covers keys [p*P, (p+1)*P); each of its columns sees those below
 * its own causal limit, and writes its normalised output and log-sum-exp to
 * slot p of its (token, head) row in the workspace. A second kernel on the
 * same stream merges, for the token at position x of its sequence, slots
 * 0 .. ceil(min(x + 1, C) / P) - 1 into out (C = slots * P, also capped by the
 * block table: positions past it are ignored); rows of tokens that belong
 * to no sequence get zeros and a log-sum-exp of -inf. The merge rests on the same
 * softmax normaliser identity as pa_decode_split (stanleyjacob.dev "vLLM",
 * Part V "The attention backend dispatch layer").
 *
 *   max_context_len   host-side upper bound of context_lens (sizes the grid
 *                     and the workspace without reading the lengths back).
 *   partition_size    P: multiple of block_size, > 0.
 *   workspace         device memory of at least
 *                     pa_multi_query_split_workspace_bytes(...) bytes,
 *                     256-byte aligned, owned by the caller.
 * Other arguments as pa_multi_query. Returns PA_OK or an error status.
 */
int pa_multi_query_split(void* out, const void* query, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                         const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_size, int64_t num_blocks, int32_t block_size,
                         float scale, int32_t dtype, int32_t max_context_len, int32_t partition_size,
                         void* workspace, size_t workspace_bytes, float* lse_out, void* stream);

/*
 * pa_decode_prefix_workspace_bytes - workspace pa_decode_prefix needs: float32
 * [num_seqs, num_heads, head_size] outputs and float32 [num_seqs, num_heads]
 * log-sum-exps of the prefix pass, each at a 256-byte aligned offset.
 * Returns 0 for invalid arguments.
 */
size_t pa_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_size);

/*
 * pa_decode_prefix - pa_decode for a batch whose sequences share a prefix.
 *
 * Sequences forked from one prompt (parallel sampling, beam search) or served
 * from one cached system prompt point their first block-table entries at the
 * same physical blocks (llm-stack-book 7.3, sections "Copy-on-write for shared
 * blocks" and "Automatic prefix caching"; modernaiengineering.com lesson
 * 13.15, "How PagedAttention shares memory"). This call reads those shared
 * blocks once for the whole batch instead of once per sequence: a first pass
 * attends every sequence's query over the shared blocks (one context, all
 * queries at once, on the matrix cores), a second pass attends each sequence
 * over its own remaining blocks and merges the two parts exactly with their
 * log-sum-exps. The result is the pa_decode result.
 *
 *   prefix_blocks     the number of leading block-table entries shared by every
 *                     sequence: entries [0, prefix_blocks) of every row must
 *                     equal row 0's (caller contract; the shared part is read
 *                     through row 0). A sequence with n_i < prefix_blocks *
 *                     block_size sees its first n_i keys. 0 runs pa_decode.
 *   workspace         device memory of at least
 *                     pa_decode_prefix_workspace_bytes(...) bytes, 256-byte
 *                     aligned, owned by the caller.
 * Other arguments as pa_decode. Two kernels are queued on `stream`.
 * Returns PA_OK or an error status (PA_ERR_WORKSPACE for a short or misaligned
 * workspace).
 */
int pa_decode_prefix(void* out, const void* query, const void* key_cache, const void* value_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                     int64_t num_blocks, int32_t block_size, float scale, int32_t dtype, int32_t prefix_blocks,
                     void* workspace, size_t workspace_bytes, float* lse_out, const int32_t* seq_order,
                     void* stream);

/*
 * pa_reshape_and_decode - pa_reshape_and_cache of one decode step's new
 * tokens followed by pa_decode, in one launch.
 *
 * Token i is sequence i's new token: its K/V (key, value [num_seqs, H_kv,
 * head_size]) are written to slot_mapping[i] and the step's attention is
 * computed as pa_decode computes it (the forward step of llm-stack-book 7.3,
 * "The forward step in detail": scatter the new K/V, then attend).
 *
 *   slot_mapping      int64 [num_seqs], device. Three cases per sequence i,
 *                     with n = context_lens[i]:
 *                     - the slot the block table gives position n - 1
 *                       (block_tables[i][(n-1)/block_size] * block_size +
 *                       (n-1) % block_size), the usual decode step: the row is
 *                       written and the attention uses the new K/V at
 *                       position n - 1. The workgroup that reads that slot
 *                       writes it with the very lanes that hold it, so the
 *                       write needs no extra pass or fence.
 *                     - negative or >= num_blocks * block_size: nothing is
 *                       written (as pa_reshape_and_cache).
 *                     - any other slot (n = 0 included): the row is written,
 *                       and the attention reads what the cache holds at every
 *                       position, position n - 1 included. The result equals
 *                       pa_reshape_and_cache followed by pa_decode only if no
 *                       context of this step reads that slot (e.g. a free
 *                       block); otherwise whether a reader sees the old or the
 *                       new row is unspecified.
 * Runs on the tile kernel for every batch size. Other arguments as pa_decode
 * and pa_reshape_and_cache (same dtype for key, value, query, out and caches).
 * Returns PA_OK or an error status.
 */
int pa_reshape_and_decode(void* out, const void* query, const void* key, const void* value,
                          const int64_t* slot_mapping, void* key_cache, void* value_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                          int64_t num_blocks, int32_t block_size, float scale, int32_t dtype, float* lse_out,
                          const int32_t* seq_order, void* stream);

/*
 * pa_multi_query - paged attention for several new tokens per sequence.
 *
 * One step may give a sequence more than one new token: a slice of a long
 * prompt (chunked prefill) or the k+1 positions of a speculative step, mixed
 * freely with one-token decodes of other sequences (llm-stack-book 7.3,
 * sections "Prefill, decode, and chunked prefill" and "Speculative decoding
 * support"). The new tokens' K/V are written first (pa_reshape_and_cache), so
 * with n = context_lens[i] tokens stored and q_i = query_start_loc[i+1] -
 * query_start_loc[i] of them new, the new token in row t = query_start_loc[i]
 * + j sits at position p = n - q_i + j, and for every query head h:
 *     s_u = scale * <query[t][h], K_u>            for u in [0, p]
 *     out[t][h] = sum_u softmax(s)_u * V_u
 * with K_u, V_u found through block_tables[i] as in pa_decode. A token with
 * p < 0 (more new tokens than stored ones) gets out = 0 and lse = -inf. With
 * every q_i = 1 this is pa_decode.
 *
 * Work is cut into tiles of one sequence and kv head covering 16 or 32
 * (new token, query head) pairs; each tile reads the keys up to its last
 * token's position once.
 *
 *   out, query        [num_tokens, num_heads, head_size] (dtype), device.
 *   query_start_loc   int32 [num_seqs + 1], device: non-decreasing, starting at
 *                     0 and ending at num_tokens. Entries are clamped to
 *                     [0, num_tokens]; other violations give unspecified
 *                     output rows, never an out-of-bounds access.
 *   num_tokens        rows of query/out (host value); 0 launches nothing.
 *   lse_out           optional float32 [num_tokens, num_heads]; NULL to skip.
 *   scale             > 0 and finite.
 * Other arguments as pa_decode. Returns PA_OK or an error status.
 */
int pa_multi_query(void* out, const void* query, const void* key_cache, const void* value_cache,
                   const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                   const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                   int32_t num_kv_heads, int32_t head_size, int64_t num_blocks, int32_t block_size, float scale,
                   int32_t dtype, float* lse_out, void* stream);

/*
 * pa_decode_split_workspace_bytes - workspace pa_decode_split needs.
 *
 * slots = ceil(max_context_len / partition_size) + 1. The workspace holds, each
 * part at a 256-byte aligned offset: float32 partials o_p
 * [num_seqs, num_heads, slots, head_size], float32 lse_p
 * [num_seqs, num_heads, slots], and a header (int64 total_blocks, int64
 * num_ranges, int32 block prefix [num_seqs + 1]) describing the pieces.
 * Returns 0 for invalid arguments.
 */
size_t pa_decode_split_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                       int32_t max_context_len, int32_t partition_size);

/*
 * pa_decode_split - the same result as pa_decode, computed over context
 * pieces and merged exactly with the log-sum-exp rule of pa_merge_partitions.
 * The merge rests on the softmax normaliser identity the pages lean on for
 * streaming (stanleyjacob.dev "vLLM", Part V "The attention backend dispatch
 * layer": tiling plus online softmax). The work is cut one of two ways
 * (pa_decode_split_part_tokens says which):
 *
 * Partitions (the default for groups H_q / H_kv <= 16): with P' = k * P tokens
 * (pa_decode_split_part_tokens: k >= 1 grows with the grid the call would
 * launch, so every workgroup streams long enough) and C = ceil(max_context_len
 * / P) * P, partition p of sequence i is its keys [p*P', min((p+1)*P', n_i, C)),
 * p < ceil(C / P'). One workgroup of the multi-query kernel per (sequence,
 * partition, kv head), handed out by the hardware dispatcher, writes the
 * partition's normalised output and log-sum-exp for the group's query heads
 * to slot p of o_p / lse_p; partitions past n_i write nothing. A second kernel
 * on the same stream merges the slots of every (sequence, head) that hold a
 * partition into out. The header is not written.
 *
 * Pieces (groups above 16; with float32 caches, groups of at most 4 when
 * num_seqs * H_kv is below the number of resident tile workgroups, i.e. a few
 * long contexts; or PA_OPT_SPLIT_CUT = 2): the kv heads are taken
 * in groups of up to 8 (one persistent workgroup has one wave per kv head of
 * its group, all walking the same blocks). Per head group, the blocks of all
 * sequences are laid end to end (sequence i has nb_i = ceil(n_i / block_size)
 * blocks; total_blocks T = groups * sum nb_i, group-major) and cut into
 * num_ranges R equal contiguous ranges, one per workgroup, so long and short
 * contexts share the GPU evenly: range r is blocks [r*T/R, (r+1)*T/R). R is at
 * most the number of resident workgroups and at most T / (partition_size /
 * block_size), so every range spans at least partition_size tokens. The piece
 * of (sequence i, head group) inside range r gets slot r - r0 (r0 the range of
 * the sequence's first block); its normalised output and log-sum-exp go to
 * o_p / lse_p of the query heads of that group. A sequence that one range
 * covers whole is written straight to `out`; a second kernel merges the
 * pieces of the others. The header describes the cut.
 *
 *   max_context_len   host-side upper bound of context_lens (sizes the
 *                     workspace and the grid without reading the lengths
 *                     back). Positions past ceil(max_context_len / P) * P are
 *                     ignored, so it must be >= every length.
 *   partition_size    P: multiple of block_size, > 0.
 *   workspace         device memory of at least
 *                     pa_decode_split_workspace_bytes(...) bytes, 256-byte
 *                     aligned, owned by the caller. Slots that the cut does not
 *                     use are left untouched.
 *   lse_out           optional float32 [num_seqs, num_heads]; NULL to skip.
 * The pieces cut keeps num_seqs + 1 block counts in 64 KiB of LDS
 * (num_seqs <= 16383). Other arguments as pa_decode. Returns PA_OK or an
 * error status.
 */
int pa_decode_split(void* out, const void* query, const void* key_cache, const void* value_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                    int32_t num_kv_heads, int32_t head_size, int64_t num_blocks,
                    int32_t block_size, float scale, int32_t dtype, int32_t max_context_len,
                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                    float* lse_out, void* stream);

/*
 * pa_decode_split_noalloc - pa_decode_split without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). Same arguments,
 * result and kernels as pa_decode_split, minus workspace / workspace_bytes:
 * the partials, log-sum-exps and pieces header live in a device array inside
 * the library, PA_DECODE_SPLIT_NOALLOC_MAX_BYTES large, one per GPU the
 * library runs on, held until the process ends. No device memory is
 * allocated or freed by the call (the array's device address is looked up
 * once per device, on the first call there).
 *
 *   Limit: pa_decode_split_workspace_bytes(num_seqs, num_heads, head_size,
 *          max_context_len, partition_size) must not exceed
 *          PA_DECODE_SPLIT_NOALLOC_MAX_BYTES; otherwise PA_ERR_WORKSPACE and
 *          nothing is launched.
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps the
 *          last call's contents (nothing in it needs to start at zero). Calls
 *          whose work overlaps on one GPU (different streams, or other host
 *          threads) race on it; serialise them (one stream, or events).
 * Returns PA_OK or an error status (PA_ERR_HIP if the array's address cannot
 * be found on the current device).
 */
#define PA_DECODE_SPLIT_NOALLOC_MAX_BYTES (64u << 20)

int pa_decode_split_noalloc(void* out, const void* query, const void* key_cache, const void* value_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                            int32_t num_kv_heads, int32_t head_size, int64_t num_blocks,
                            int32_t block_size, float scale, int32_t dtype, int32_t max_context_len,
                            int32_t partition_size, float* lse_out, void* stream);

/*
 * pa_decode_split_part_tokens - the cut pa_decode_split makes for these
 * arguments on the current device: the partition length P' (a multiple of
 * partition_size) of the partition cut, 0 for the pieces cut, -1 for invalid
 * arguments, with the options PA_OPT_SPLIT_CUT and PA_OPT_SPLIT_PART_FACTOR
 * as they stand. dtype: the caches' element type. Queries the device's CU
 * count, launches nothing.
 */
int32_t pa_decode_split_part_tokens(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t max_context_len, int32_t partition_size, int32_t dtype);

/*
 * pa_merge_partitions - exact log-sum-exp merge of partial attention results.
 *
 * A softmax over a whole context can be carried piecewise as a running maximum
 * and normaliser, so attention computed separately over pieces of a context
 * recombines exactly (stanleyjacob.dev "vLLM", Part V "The attention backend
 * dispatch layer": tiling plus online softmax; Part IV "Stage 6: The forward
 * pass"). For each (sequence, head): M = max_p lse_p, w_p = exp(lse_p - M),
 *     out = sum_p w_p o_p / sum_p w_p,   lse = M + ln sum_p w_p.
 * Partitions with lse_p = -inf carry no weight and their o_p is never used
 * (it may hold anything). If all are -inf: out = 0, lse = -inf.
 *
 *   o_parts           float32 [num_seqs, num_heads, num_parts, head_size]
 *   lse_parts         float32 [num_seqs, num_heads, num_parts]
 *   out               [num_seqs, num_heads, head_size] in dtype, written.
 *   lse_out           optional float32 [num_seqs, num_heads]; NULL to skip.
 * Returns PA_OK or an error status.
 */
int pa_merge_partitions(void* out, float* lse_out, const float* o_parts, const float* lse_parts,
                        int32_t num_seqs, int32_t num_heads, int32_t num_parts,
                        int32_t head_size, int32_t dtype, void* stream);

/*
 * Kernel-choice overrides.
 *
 * Every entry point picks its launch shape from the call's arguments and the
 * device (the defaults are the measured choices). These process-wide options
 * force one of the alternatives instead, so that tests can cover every path
 * and measurements can compare them; each choice computes the same result up
 * to rounding order. An option applies to calls made after it is set; which
 * value a call made concurrently from another thread sees is unspecified.
 *
 *   PA_OPT_TILE_WAVES        waves per workgroup of the tile kernel (16-column
 *                            tiles of 16-bit and FP8 caches): 0 = 8 when the
 *                            launch has at most one job per resident 4-wave
 *                            workgroup, else 4 (default); or 4, or 8.
 *   PA_OPT_TILE_COLUMNS      columns per multi-query tile: 0 = 32 when the step
 *                            averages more new tokens per sequence than a
 *                            16-column tile holds, else 16 (default); or 16,
 *                            or 32.
 *   PA_OPT_SPLIT_CUT         pa_decode_split's cut: 0 = by shape (default),
 *                            1 = partitions (groups <= 16), 2 = pieces.
 *   PA_OPT_SPLIT_PART_FACTOR the partition cut's factor k (partitions of
 *                            k * partition_size tokens): 0 = by grid size
 *                            (default), or k >= 1 (capped at
 *                            ceil(max_context_len / partition_size)).
 *   PA_OPT_MERGE_ROWS        (sequence, head) rows per workgroup of the merge
 *                            kernels: 0 = by row count (default), or 1, 2, 4.
 *
 * pa_set_option returns PA_OK, or PA_ERR_INVALID_ARG for an unknown option or
 * a value outside its range (the option keeps its value). pa_get_option
 * returns the value, or -1 for an unknown option.
 */
typedef enum pa_option {
  PA_OPT_TILE_WAVES = 0,
  PA_OPT_TILE_COLUMNS = 1,
  PA_OPT_SPLIT_CUT = 2,
  PA_OPT_SPLIT_PART_FACTOR = 3,
  PA_OPT_MERGE_ROWS = 4
} pa_option;

int pa_set_option(int option, int value);
int pa_get_option(int option);

/* pa_status_string - static, NUL-terminated description of a status code. */
const char* pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
