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

// One-token-per-sequence decode through the multi-query kernel (P*V on the
// matrix cores; one workgroup per (sequence, kv head), dispatched in
// seq_order): scale_log2 = scale * log2(e), times k_scale for FP8 caches.
// With skip_blocks > 0 it is the suffix pass of the shared-prefix decode
// (prefix_o / prefix_lse as the decode kernel's). Arguments are validated by
// the caller.
int launch_decode_multi(void* out, const void* query, const void* key_cache, const void* value_cache,
                        const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                        int64_t num_blocks, float scale_log2, float v_scale, int32_t dtype, bool fp8_cache,
                        float* lse_out, const int32_t* seq_order, int32_t skip_blocks, const float* prefix_o,
                        const float* prefix_lse, hipStream_t stream);

// Context partitions of a one-token-per-sequence decode on the multi-query
// kernel: partition p of sequence i (keys [p * P, min((p + 1) * P, n_i,
// part_cap)), P = 16 * part_blocks, p < num_parts) writes the normalised
// float32 output and log-sum-exp of each query head h to o_parts / lse_parts
// row (i * num_heads + h) * parts_stride + p; partitions past a context's end
// write nothing. g = num_heads / num_kv_heads must be at most 16. Arguments are
// validated by the caller.
int launch_split_tiles(const void* query, const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                       int64_t num_blocks, float scale, int32_t dtype, int32_t part_blocks, int32_t num_parts,
                       int32_t part_cap, int32_t parts_stride, float* o_parts, float* lse_parts,
                       hipStream_t stream);

// Merge of pa_multi_query_split: output row (token t, head h) combines the
// partitions 0 .. ceil(min(position(t) + 1, cap) / partition_size) - 1 of
// its row in o_parts / lse_parts ([num_tokens, num_heads, num_parts(, D)]);
// position(t) follows from query_start_loc and context_lens. Arguments are
// validated by the caller.
int launch_merge_mq_parts(void* out, float* lse_out, const float* o_parts, const float* lse_parts,
                          const int32_t* query_start_loc, const int32_t* context_lens, int num_seqs,
                          int num_tokens, int num_heads, int cap, int max_blocks, int partition_size,
                          int num_parts, int head_size, int dtype, hipStream_t stream);

// Compute units of the current device (256 when it cannot be queried).
int device_cus();

// True when scale is a power of two in [2^-120, 2^120]; then *inv is its
// exact reciprocal and x * inv equals the correctly rounded x / scale.
inline bool exact_reciprocal(float scale, float* inv) {
  int e = 0;
  const float m = __builtin_frexpf(scale, &e);
  if (m != 0.5f || e < -119 || e > 121) return false;
  *inv = __builtin_ldexpf(1.0f, 1 - e);
  return true;
}

// Current value of a kernel-choice option (pa_option in pa.h); 0 = the
// default choice.
int option_value(int option);

}  // namespace pa
