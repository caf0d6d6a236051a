// Measurement kernels (include/pa_measure.h): the streaming-read ceiling and
// the decode's memory traffic without its arithmetic. Neither is on the
// attention path; the bench times them beside the decode to say how close the
// decode comes to what the memory system delivers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_measure.h"
#include "pa_tiles.h"

namespace pa {

constexpr uint32_t kSinkMagic = 0x9E3779B9u;

__device__ __forceinline__ uint32_t fold4(u32x4_t v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// Plain streaming read: workgroup b reads the contiguous 16-byte pieces
// [b * per, (b + 1) * per), U loads per thread in flight, non-temporal (the
// data is used once). On MI355X this pattern measured 7.0 TB/s, against
// 6.1-6.3 TB/s for plain loads and 5.3-5.7 TB/s for a grid-stride walk.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + (U - 1) * 256 < hi; i += U * 256) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&src[i + u * 256]);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= fold4(v[u]);
  }
  for (; i < hi; i += 256) acc ^= fold4(__builtin_nontemporal_load(&src[i]));
  if (acc == kSinkMagic) sink[0] = acc;
}

struct StreamKvArgs {
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* seq_order;
  uint32_t* sink;
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_kv_heads;
};

template <typename T, int D, int CB, bool F8>
__device__ __forceinline__ uint32_t fold_chunk(const Chunk<T, D, 16, CB, F8>& f) {
  using S = DecodeShape<T, D, 16, CB, F8>;
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < CB; ++i) {
#pragma unroll
    for (int s = 0; s < S::kKSeg; ++s) acc ^= fold4(f.k[i][s]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int w = 0; w < S::kVDw; ++w) acc ^= f.v[i][r][w];
  }
  return acc;
}

// The tile kernel's decode mode (paged_multi_query_kernel with one new token
// per sequence) with the arithmetic taken out: the same workgroup per
// (sequence, kv head) in the same dispatch order, chunk c of CB blocks to wave
// c % W, one chunk of look-ahead in registers, the same non-temporal loads
// (load_chunk, K row by row through LDS for 16-bit caches).
template <typename T, int D, int CB, bool F8, int W>
__global__ __launch_bounds__(W * kWave, W == 4 ? 2 : 1) void stream_kv_kernel(StreamKvArgs a) {
  using S = DecodeShape<T, D, 16, CB, F8>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int slot, kvh;
  slot_and_head(blockIdx.x, a.num_kv_heads, slot, kvh);
  if (slot >= a.num_seqs) return;
  int seq = slot;
  if (a.seq_order != nullptr) {
    const uint32_t o = static_cast<uint32_t>(a.seq_order[slot]);
    seq = static_cast<int>(o < static_cast<uint32_t>(a.num_seqs) ? o : a.num_seqs - 1);
  }
  const int max_tokens = a.max_blocks * kBlockTokens;
  // As the decode: the first chunk's table entries with the length (16-bit caches).
  int32_t first_ids[CB] = {};
  if constexpr (!F8) first_chunk_ids<CB>(first_ids, a.block_tables + static_cast<int64_t>(seq) * a.max_blocks,
                                         wave * CB, a.max_blocks);
  int n = a.context_lens[seq];
  n = n < 0 ? 0 : (n > max_tokens ? max_tokens : n);
  const uint32_t tok_stride = static_cast<uint32_t>(a.num_kv_heads) * D * S::kElemBytes;
  const int64_t blk_stride = static_cast<int64_t>(tok_stride) * kBlockTokens;
  const int64_t head_off = static_cast<int64_t>(kvh) * D * S::kElemBytes;
  const char* kc = static_cast<const char*>(a.key_cache);
  const char* vc = static_cast<const char*>(a.value_cache);
  const int32_t* bt_row = a.block_tables + static_cast<int64_t>(seq) * a.max_blocks;
  const int blk_end = (n + kBlockTokens - 1) / kBlockTokens;
  const int nchunk = (blk_end + CB - 1) / CB;
  const int blk_last = blk_end - 1;
  const int last_rows = n - blk_last * kBlockTokens;
  const int mine = wave < nchunk ? (nchunk - wave + W - 1) / W : 0;
  auto blk_of = [&](int i) { return (wave + i * W) * CB; };
  // 16-bit caches: row-wise K through each wave's LDS area, as the decode does.
  constexpr bool kRowK = S::kRowKCapable;
  __shared__ u32x4_t s_stage[W][kRowK ? CB * kBlockTokens * S::kRowPieces : 1];
  uint32_t acc = 0;
  Chunk<T, D, 16, CB, F8> fa, fb;
  auto fold = [&](Chunk<T, D, 16, CB, F8>& f) {
    if constexpr (kRowK) k_rows_to_mfma<T, D, 16, CB, F8>(f, s_stage[wave], lane);
    return fold_chunk<T, D, CB, F8>(f);
  };
  if (mine > 0) {
    load_chunk<T, D, 16, CB, F8, true, kRowK>(fa, kc, vc, bt_row, blk_of(0), blk_last, a.num_blocks, tok_stride,
                                              blk_stride, head_off, lane, last_rows, first_ids, !F8);
    int i = 0;
    for (; i + 2 < mine; i += 2) {
      load_chunk<T, D, 16, CB, F8, true, kRowK>(fb, kc, vc, bt_row, blk_of(i + 1), blk_last, a.num_blocks, tok_stride,
                                   blk_stride, head_off, lane, last_rows);
      __builtin_amdgcn_sched_barrier(0);
      acc ^= fold(fa);
      __builtin_amdgcn_sched_barrier(0);
      load_chunk<T, D, 16, CB, F8, true, kRowK>(fa, kc, vc, bt_row, blk_of(i + 2), blk_last, a.num_blocks, tok_stride,
                                   blk_stride, head_off, lane, last_rows);
      __builtin_amdgcn_sched_barrier(0);
      acc ^= fold(fb);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (i + 1 < mine) {
      load_chunk<T, D, 16, CB, F8, true, kRowK>(fb, kc, vc, bt_row, blk_of(i + 1), blk_last, a.num_blocks, tok_stride,
                                   blk_stride, head_off, lane, last_rows);
      __builtin_amdgcn_sched_barrier(0);
      acc ^= fold(fa);
      acc ^= fold(fb);
    } else {
      acc ^= fold(fa);
    }
  }
  if (acc == kSinkMagic) a.sink[0] = acc;
}

}  // namespace pa

using namespace pa;

namespace {

typedef void (*StreamKvKernel)(StreamKvArgs);

// Blocks per chunk as the tile kernel takes them for 16-column tiles.
template <typename T, int D, bool F8>
StreamKvKernel stream_kv_for(int W) {
  constexpr int kElem = F8 ? 1 : static_cast<int>(sizeof(T));
  constexpr int CB = D * kElem / 8 <= 32 ? 2 : 1;
  if constexpr (sizeof(T) == 2) {
    if (W == 8) return stream_kv_kernel<T, D, CB, F8, 8>;
  }
  return stream_kv_kernel<T, D, CB, F8, 4>;
}

}  // namespace

extern "C" int pa_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return PA_OK;
  if (src == nullptr || sink == nullptr || (bytes & 15u) != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return PA_ERR_INVALID_ARG;
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  // 16 workgroups of 256 threads per compute unit (4,096 on MI355X), but no
  // more than one per 4 KiB.
  int64_t grid = 16 * static_cast<int64_t>(device_cus());
  if (grid > (n16 + 255) / 256) grid = (n16 + 255) / 256;
  hipLaunchKernelGGL(stream_read_kernel<16>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" int pa_stream_kv(const void* key_cache, const void* value_cache, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_kv_heads, int32_t head_size, int64_t num_blocks, int32_t block_size,
                            int32_t cache_kind, const int32_t* seq_order, uint32_t* sink, void* stream) {
  if (num_seqs < 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if (cache_kind < 0 || cache_kind > 2) return PA_ERR_INVALID_ARG;
  if (block_size != kBlockTokens) return PA_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!key_cache || !value_cache || !block_tables || !context_lens || !sink) return PA_ERR_INVALID_ARG;
  if (((reinterpret_cast<uintptr_t>(key_cache) | reinterpret_cast<uintptr_t>(value_cache)) & 15u) != 0)
    return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_blocks_per_seq) * kBlockTokens > INT32_MAX) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(num_kv_heads) * head_size * 4 >= (int64_t{1} << 24)) return PA_ERR_UNSUPPORTED;
  const int64_t grid = (static_cast<int64_t>(num_seqs) + 7) / 8 * 8 * num_kv_heads;
  if (grid > INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
  // Waves per workgroup as the decode picks them.
  int W = option_value(PA_OPT_TILE_WAVES);
  if (W != 4 && W != 8)
    W = static_cast<int64_t>(num_seqs) * num_kv_heads <= 2 * static_cast<int64_t>(device_cus()) ? 8 : 4;
  StreamKvKernel k;
  if (cache_kind == 2) {
    k = head_size == 128 ? stream_kv_for<bf16_t, 128, true>(W) : stream_kv_for<bf16_t, 64, true>(W);
  } else if (cache_kind == 1) {
    k = head_size == 128 ? stream_kv_for<bf16_t, 128, false>(W) : stream_kv_for<bf16_t, 64, false>(W);
  } else {
    W = 4;
    k = head_size == 128 ? stream_kv_for<float, 128, false>(W) : stream_kv_for<float, 64, false>(W);
  }
  StreamKvArgs a{key_cache, value_cache, block_tables, context_lens, seq_order, sink,
                 num_blocks, max_blocks_per_seq, num_seqs, num_kv_heads};
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(grid)), dim3(W * kWave), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
