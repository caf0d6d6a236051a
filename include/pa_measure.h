/*
 * pa_measure.h - measurement kernels of libpa.so (not part of the attention
 * path): the read rates that bound the paged decode on this GPU, measured in
 * the same process as the decode itself.
 *
 * The pages bound a decode step by the bytes it must read (AI Infrastructure
 * part 17, "Why can one GPU step serve many users?": every step streams the
 * weights and each request's KV cache), so a decode kernel is judged against
 * what the memory system delivers. These two calls give that rate for a plain
 * streaming read and for the decode's own access pattern.
 *
 * Conventions as in pa.h: device pointers owned by the caller, 16-byte
 * aligned; work queued on `stream`; nothing allocated or synchronised; an int
 * status (pa_status). Both kernels fold everything they read into a checksum
 * and write sink[0] only when the checksum equals one fixed value (which data
 * drawn from a continuous distribution practically never gives), so the loads
 * cannot be optimised away and the only write traffic is that one word.
 */
#ifndef PA_MEASURE_H_
#define PA_MEASURE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pa_stream_read - read `bytes` contiguous bytes at `src` (a multiple of 16)
 * once, in the pattern this GPU streams fastest at (measured: each workgroup
 * reads one contiguous range with non-temporal 16-byte loads, 16 per thread
 * in flight). The time of this call over bytes is the plain streaming-read
 * ceiling.
 *   sink   uint32 [1], device, written only as described above.
 */
int pa_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * pa_stream_kv - the decode's memory traffic without its arithmetic: exactly
 * the K and V loads pa_decode issues (the same tile kernel layout, job map,
 * chunking, look-ahead and workgroup size, seq_order honoured), each
 * (sequence, kv head) job reading its context's rows through the block table.
 * The time of this call is the ceiling of the decode's access pattern.
 *   cache_kind   0: float32 caches, 1: bfloat16, 2: FP8 (one byte per element).
 * Other arguments as pa_decode. Returns PA_OK or an error status.
 */
int pa_stream_kv(const void* key_cache, const void* value_cache, const int32_t* block_tables,
                 int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                 int32_t head_size, int64_t num_blocks, int32_t block_size, int32_t cache_kind,
                 const int32_t* seq_order, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_MEASURE_H_ */
