// Launchers shared between the library's translation units (not part of the
// C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Shared-prefix pass of pa_decode_prefix: every sequence's decode query
// attends over the first prefix_blocks blocks of block table row 0 (at most
// context_lens[i] keys), writing normalised float32 outputs to part_o
// [num_seqs, num_heads, head_size] and log-sum-exps to part_lse
// [num_seqs, num_heads]. Arguments are validated by the caller.
int launch_prefix_pass(const void* query, const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                       int64_t num_blocks, int32_t prefix_blocks, float scale, int32_t dtype, float* part_o,
                       float* part_lse, hipStream_t stream);

}  // namespace pa
