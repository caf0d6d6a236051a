// pa_reshape_and_cache for gfx950: scatter new K/V rows into their cache slots.
//
// Each token's K and V row ([H_kv, d_h], contiguous) is copied to row `slot` of
// the flattened pool [num_blocks * block_size, H_kv, d_h], where the slot is
// physical_block * block_size + offset (llm-stack-book 7.3 "vLLM: Architecture,
// PagedAttention & Internals", section "The forward step in detail"). One
// thread moves one 16-byte piece of K and the matching piece of V, so a wave
// copies 1 KiB of each with fully coalesced loads and stores. The copy is
// bitwise.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(const u32x4_t* __restrict__ key,
                                                                const u32x4_t* __restrict__ value,
                                                                u32x4_t* __restrict__ key_cache,
                                                                u32x4_t* __restrict__ value_cache,
                                                                const int64_t* __restrict__ slot_mapping,
                                                                int64_t num_tokens, int64_t num_slots,
                                                                int row_pieces) {
  const int64_t total = num_tokens * row_pieces;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t t = i / row_pieces;
    const int64_t piece = i - t * row_pieces;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;  // padding token, or a slot outside the pool
    key_cache[slot * row_pieces + piece] = key[i];
    value_cache[slot * row_pieces + piece] = value[i];
  }
}

// pa_reshape_and_cache_fp8: the quantizing scatter. A thread turns 8 values
// of a token row (bf16 or float32) into 8 E4M3 codes with quantize4_e4m3
// (pa_device.h), the encoding the one-launch FP8 decode step uses too.
template <typename T, bool POW2>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(const T* __restrict__ key,
                                                                    const T* __restrict__ value,
                                                                    u32x2_t* __restrict__ key_cache,
                                                                    u32x2_t* __restrict__ value_cache,
                                                                    const int64_t* __restrict__ slot_mapping,
                                                                    int64_t num_tokens, int64_t num_slots,
                                                                    int row_groups, float k_scale, float v_scale,
                                                                    float k_inv, float v_inv) {
  // One group = 8 consecutive elements of a token row = one 8-byte piece of
  // its cache row.
  const int64_t total = num_tokens * row_groups;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t t = i / row_groups;
    const int64_t grp = i - t * row_groups;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;  // padding token, or a slot outside the pool
    float k[8], v[8];
    if constexpr (sizeof(T) == 2) {
      const u32x4_t kw = reinterpret_cast<const u32x4_t*>(key)[i];
      const u32x4_t vw = reinterpret_cast<const u32x4_t*>(value)[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k[2 * e] = bf16_lo(kw[e]);
        k[2 * e + 1] = bf16_hi(kw[e]);
        v[2 * e] = bf16_lo(vw[e]);
        v[2 * e + 1] = bf16_hi(vw[e]);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4_t kw = reinterpret_cast<const u32x4_t*>(key)[2 * i + h];
        const u32x4_t vw = reinterpret_cast<const u32x4_t*>(value)[2 * i + h];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k[4 * h + e] = as_float(kw[e]);
          v[4 * h + e] = as_float(vw[e]);
        }
      }
    }
    const int64_t dst = slot * row_groups + grp;
    key_cache[dst] = u32x2_t{quantize4_e4m3<POW2>(k[0], k[1], k[2], k[3], k_scale, k_inv),
                             quantize4_e4m3<POW2>(k[4], k[5], k[6], k[7], k_scale, k_inv)};
    value_cache[dst] = u32x2_t{quantize4_e4m3<POW2>(v[0], v[1], v[2], v[3], v_scale, v_inv),
                               quantize4_e4m3<POW2>(v[4], v[5], v[6], v[7], v_scale, v_inv)};
  }
}

// pa_copy_blocks: workgroup (pair, cache) copies one whole block, source to
// destination (the GPU half of copy-on-write: llm-stack-book 7.3, section
// "Copy-on-write for shared blocks"). Each of the 512 threads keeps
// kCopyBatch 16-byte pieces in flight before storing them (a 32 KiB block in
// one batch); the pair's ids are wave-uniform scalar loads. Pairs naming a
// block outside the pool are skipped. The source is read with non-temporal
// loads (read once) and the destination written with plain stores: on 4,096
// pairs of the batch-256 pool 102.2 us, against 106.7 us with non-temporal
// stores too, 104.4 us with plain loads and non-temporal stores, 111.2 us
// with plain loads and stores, and 103.2 us with 256 threads of 8 pieces.
constexpr int kCopyBatch = 4;
constexpr int kCopyThreads = 512;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(u32x4_t* __restrict__ key_cache,
                                                                   u32x4_t* __restrict__ value_cache,
                                                                   const int64_t* __restrict__ block_mapping,
                                                                   int64_t num_blocks, int64_t block_pieces) {
  const int64_t src = block_mapping[2 * static_cast<int64_t>(blockIdx.x)];
  const int64_t dst = block_mapping[2 * static_cast<int64_t>(blockIdx.x) + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  u32x4_t* cache = blockIdx.y == 0 ? key_cache : value_cache;
  const u32x4_t* from = cache + src * block_pieces;
  u32x4_t* to = cache + dst * block_pieces;
  const int64_t step = static_cast<int64_t>(blockDim.x) * kCopyBatch;
  for (int64_t base = threadIdx.x; base < block_pieces; base += step) {
    u32x4_t v[kCopyBatch];
#pragma unroll
    for (int i = 0; i < kCopyBatch; ++i) {
      const int64_t j = base + static_cast<int64_t>(i) * blockDim.x;
      if (j < block_pieces) v[i] = __builtin_nontemporal_load(&from[j]);
    }
#pragma unroll
    for (int i = 0; i < kCopyBatch; ++i) {
      const int64_t j = base + static_cast<int64_t>(i) * blockDim.x;
      if (j < block_pieces) to[j] = v[i];
    }
  }
}

}  // namespace pa

using namespace pa;

extern "C" int pa_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                                    const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                                    int32_t block_size, int32_t num_kv_heads, int32_t head_size, int32_t dtype,
                                    void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PA_ERR_INVALID_ARG;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_INVALID_ARG;
  if (block_size != kBlockTokens) return PA_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value) |
                        reinterpret_cast<uintptr_t>(key_cache) | reinterpret_cast<uintptr_t>(value_cache);
  if (mis & 15u) return PA_ERR_INVALID_ARG;
  const int64_t row_bytes = static_cast<int64_t>(num_kv_heads) * head_size * (dtype == PA_DTYPE_F32 ? 4 : 2);
  const int64_t row_pieces = row_bytes / 16;  // head_size in {64,128} makes rows whole 16-byte pieces
  if (row_pieces > INT32_MAX) return PA_ERR_UNSUPPORTED;
  const int64_t total = num_tokens * row_pieces;
  constexpr int kThreads = 256;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;  // grid-stride loop covers the rest
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(key),
                     static_cast<const u32x4_t*>(value), static_cast<u32x4_t*>(key_cache),
                     static_cast<u32x4_t*>(value_cache), slot_mapping, num_tokens,
                     num_blocks * kBlockTokens, static_cast<int>(row_pieces));
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or dtype)";
    case PA_ERR_UNSUPPORTED: return "unsupported shape (block_size must be 16, head_size 64 or 128, "
                                    "num_heads/num_kv_heads at most 16)";
    case PA_ERR_WORKSPACE: return "workspace smaller than pa_decode_split_workspace_bytes()";
    case PA_ERR_HIP: return "HIP runtime refused the launch";
    case PA_ERR_NO_BLOCKS: return "the block pool has too few free blocks";
    default: return "unknown status";
  }
}

extern "C" int pa_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                              int64_t num_pairs, int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                              int32_t head_size, int32_t dtype, void* stream) {
  if (num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PA_ERR_INVALID_ARG;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_INVALID_ARG;
  if (block_size != kBlockTokens) return PA_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !block_mapping) return PA_ERR_INVALID_ARG;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(key_cache) | reinterpret_cast<uintptr_t>(value_cache);
  if (mis & 15u) return PA_ERR_INVALID_ARG;
  if (num_pairs > INT32_MAX) return PA_ERR_UNSUPPORTED;
  const int64_t block_bytes =
      static_cast<int64_t>(kBlockTokens) * num_kv_heads * head_size * (dtype == PA_DTYPE_F32 ? 4 : 2);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<unsigned>(num_pairs), 2), dim3(kCopyThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4_t*>(key_cache),
                     static_cast<u32x4_t*>(value_cache), block_mapping, num_blocks, block_bytes / 16);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

extern "C" int pa_reshape_and_cache_fp8(const void* key, const void* value, uint8_t* key_cache,
                                        uint8_t* value_cache, const int64_t* slot_mapping, int64_t num_tokens,
                                        int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                                        int32_t head_size, int32_t dtype, float k_scale, float v_scale,
                                        void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PA_ERR_INVALID_ARG;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_INVALID_ARG;
  if (block_size != kBlockTokens) return PA_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale == __builtin_inff() || v_scale == __builtin_inff())
    return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value);
  if ((mis & 15u) || ((reinterpret_cast<uintptr_t>(key_cache) | reinterpret_cast<uintptr_t>(value_cache)) & 7u))
    return PA_ERR_INVALID_ARG;
  const int64_t row_groups = static_cast<int64_t>(num_kv_heads) * head_size / 8;
  if (row_groups > INT32_MAX) return PA_ERR_UNSUPPORTED;
  const int64_t total = num_tokens * row_groups;
  constexpr int kThreads = 256;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  float k_inv = 0.f, v_inv = 0.f;
  const bool pow2 = exact_reciprocal(k_scale, &k_inv) && exact_reciprocal(v_scale, &v_inv);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  auto* kd = reinterpret_cast<u32x2_t*>(key_cache);
  auto* vd = reinterpret_cast<u32x2_t*>(value_cache);
  const int64_t ns = num_blocks * kBlockTokens;
  const int rg = static_cast<int>(row_groups);
  if (dtype == PA_DTYPE_BF16) {
    const auto* k = static_cast<const bf16_t*>(key);
    const auto* v = static_cast<const bf16_t*>(value);
    if (pow2)
      hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<bf16_t, true>), grid, block, 0, s, k, v, kd, vd, slot_mapping,
                         num_tokens, ns, rg, k_scale, v_scale, k_inv, v_inv);
    else
      hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<bf16_t, false>), grid, block, 0, s, k, v, kd, vd, slot_mapping,
                         num_tokens, ns, rg, k_scale, v_scale, k_inv, v_inv);
  } else {
    const auto* k = static_cast<const float*>(key);
    const auto* v = static_cast<const float*>(value);
    if (pow2)
      hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<float, true>), grid, block, 0, s, k, v, kd, vd, slot_mapping,
                         num_tokens, ns, rg, k_scale, v_scale, k_inv, v_inv);
    else
      hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<float, false>), grid, block, 0, s, k, v, kd, vd, slot_mapping,
                         num_tokens, ns, rg, k_scale, v_scale, k_inv, v_inv);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
