// Device-side helpers shared by the paged-attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pa {

typedef uint16_t bf16_t;  // bfloat16 storage
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;  // MFMA bf16 operand
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr int kWave = 64;
constexpr int kBlockTokens = 16;  // tokens per KV block; also the MFMA M dimension
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// Lane H of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int H>
__device__ __forceinline__ float row_bcast(float x) {
  static_assert(H >= 0 && H < 16, "row lane");
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + H, 0xF, 0xF, false));
}

__device__ __forceinline__ float xor_shfl(float x, int mask) { return __shfl_xor(x, mask, kWave); }

// Combine each lane's value with lane l^16 (resp. l^32) on the VALU
// (v_permlane16_swap / v_permlane32_swap give every lane both values of its
// pair); unlike a shuffle through LDS this does not wait on the LDS/scalar
// memory counter. Addition is commutative, so both lanes of a pair get the
// same bits.
__device__ __forceinline__ float pair16_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, static_cast<uint32_t>(r[0])), __builtin_bit_cast(float, static_cast<uint32_t>(r[1])));
}
__device__ __forceinline__ float pair32_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, static_cast<uint32_t>(r[0])), __builtin_bit_cast(float, static_cast<uint32_t>(r[1])));
}
__device__ __forceinline__ float pair16_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, static_cast<uint32_t>(r[0])) + __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, static_cast<uint32_t>(r[0])) + __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
}
// Sum / max over the four 16-lane rows (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float rows_sum(float x) { return pair32_sum(pair16_sum(x)); }
__device__ __forceinline__ float rows_max(float x) { return pair32_max(pair16_max(x)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// A wave-uniform pointer passed through readfirstlane: the compiler keeps it in
// scalar registers and does not fold per-lane offsets into it, so loads use the
// scalar-base + 32-bit-lane-offset addressing form.
typedef __attribute__((address_space(1))) const char gchar_t;  // global-memory byte

__device__ __forceinline__ const gchar_t* uniform_ptr(const char* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return reinterpret_cast<const gchar_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Load of a 16-byte vector from global memory.
__device__ __forceinline__ u32x4_t gload16(const gchar_t* p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) u32x4_t*>(p);
}

// The same load, plain (STREAM = false) or non-temporal (STREAM = true: the
// data is read once, so the caches need not keep it). On MI355X a stream of
// 16-byte non-temporal loads reads 7.0 TB/s against 6.2 TB/s for plain ones,
// and the decode's K/V loads gain 10% from it; data that other workgroups
// read again (a shared prefix, the keys of a sequence's other tiles) must
// stay cached and uses plain loads.
template <bool STREAM>
__device__ __forceinline__ u32x4_t gload16s(const gchar_t* p) {
  const auto* q = reinterpret_cast<const __attribute__((address_space(1))) u32x4_t*>(p);
  if constexpr (STREAM) return __builtin_nontemporal_load(q);
  return *q;
}

__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }

// FP8 E4M3 (OCP) codes to float32, two at a time with the hardware converter:
// bytes 0,1 (hi = false) or 2,3 (hi = true) of w. On gfx950 the converter reads
// the OCP E4M3 format (finite values up to 448, S.1111.111 = NaN) and every
// code's value is exact in float32.
template <bool HI>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t w, float& a, float& b) {
  const auto v = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), HI);
  a = v[0];
  b = v[1];
}

// Eight FP8 codes (two dwords) to eight bf16 values, the MFMA operand. Every
// E4M3 value is exact in bfloat16 (3 mantissa bits, exponents 2^-9 .. 2^8);
// gfx950 converts two codes straight to two bf16 (scale 1, exact).
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{fp8x2_to_bf16x2(w0, false), fp8x2_to_bf16x2(w0, true),
                                              fp8x2_to_bf16x2(w1, false), fp8x2_to_bf16x2(w1, true)});
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Four values to four FP8 E4M3 codes (byte i = value i): x / scale in float32
// (IEEE division, round to nearest), magnitudes above 448 (infinities
// included) clamped to 448, NaN written as S.1111.111 with x's sign, and the
// rest converted by the hardware to the nearest code, ties to even. The format
// and the scale are this library's reading: the pages name an FP8 KV cache
// without fixing one (llm-stack-book 7.3, "The knobs that actually matter",
// item 5). POW2: scale is a power of two and inv its exact reciprocal, so
// x * inv is the correctly rounded quotient x / scale (both round the same
// exact value once) at the cost of one multiplication instead of a division.
template <bool POW2>
__device__ __forceinline__ uint32_t quantize4_e4m3(float a, float b, float c, float d, float scale, float inv) {
  float v[4];
  if constexpr (POW2) {
    v[0] = a * inv;
    v[1] = b * inv;
    v[2] = c * inv;
    v[3] = d * inv;
  } else {
    v[0] = __fdiv_rn(a, scale);
    v[1] = __fdiv_rn(b, scale);
    v[2] = __fdiv_rn(c, scale);
    v[3] = __fdiv_rn(d, scale);
  }
  uint32_t nan_bits = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (v[i] != v[i]) {
      nan_bits |= ((__builtin_bit_cast(uint32_t, v[i]) >> 31) << 7 | 0x7Fu) << (8 * i);
      v[i] = 0.f;
    } else {
      v[i] = fminf(fmaxf(v[i], -448.f), 448.f);
    }
  }
  uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false));
  w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], static_cast<int>(w), true));
  // NaN lanes were converted as zero (code 0): OR in their NaN code.
  return w | nan_bits;
}

// Two dwords of bf16 (four values, low halves first) to four E4M3 codes.
template <bool POW2>
__device__ __forceinline__ uint32_t quantize_bf16x4_e4m3(uint32_t w0, uint32_t w1, float scale, float inv) {
  return quantize4_e4m3<POW2>(__builtin_bit_cast(float, w0 << 16), __builtin_bit_cast(float, w0 & 0xFFFF0000u),
                              __builtin_bit_cast(float, w1 << 16), __builtin_bit_cast(float, w1 & 0xFFFF0000u),
                              scale, inv);
}

// float32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ void store_elem(T* p, float x);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_elem<bf16_t>(bf16_t* p, float x) { *p = f32_to_bf16(x); }

// Two consecutive elements (p 4-byte aligned for bf16, 8-byte for float).
template <typename T>
__device__ __forceinline__ void store_pair(T* p, float x, float y);
template <>
__device__ __forceinline__ void store_pair<float>(float* p, float x, float y) {
  *reinterpret_cast<u32x2_t*>(p) = u32x2_t{__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y)};
}
template <>
__device__ __forceinline__ void store_pair<bf16_t>(bf16_t* p, float x, float y) {
  *reinterpret_cast<uint32_t*>(p) = static_cast<uint32_t>(f32_to_bf16(x)) | (static_cast<uint32_t>(f32_to_bf16(y)) << 16);
}

// N consecutive elements from floats (bf16: rounded to nearest even), as
// 16-byte stores where the run allows (p aligned to the run's size, up to 16
// bytes).
template <typename T, int N>
__device__ __forceinline__ void store_run(T* p, const float (&x)[N]) {
  constexpr int kWords = N * static_cast<int>(sizeof(T)) / 4;
  uint32_t w[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) {
    if constexpr (sizeof(T) == 4)
      w[i] = __builtin_bit_cast(uint32_t, x[i]);
    else
      w[i] = static_cast<uint32_t>(f32_to_bf16(x[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(x[2 * i + 1])) << 16);
  }
  uint32_t* q = reinterpret_cast<uint32_t*>(p);
  if constexpr (kWords % 4 == 0) {
#pragma unroll
    for (int i = 0; i < kWords; i += 4)
      *reinterpret_cast<u32x4_t*>(q + i) = u32x4_t{w[i], w[i + 1], w[i + 2], w[i + 3]};
  } else if constexpr (kWords % 2 == 0) {
#pragma unroll
    for (int i = 0; i < kWords; i += 2) *reinterpret_cast<u32x2_t*>(q + i) = u32x2_t{w[i], w[i + 1]};
  } else {
#pragma unroll
    for (int i = 0; i < kWords; ++i) q[i] = w[i];
  }
}

// Load `NDW` dwords (4, 8, 16 or 32 bytes) that are 16-byte (or 8- or
// 4-byte) aligned; STREAM as for gload16s.
template <int NDW, bool STREAM = false>
__device__ __forceinline__ void load_dwords(uint32_t (&dst)[NDW], const gchar_t* src) {
  if constexpr (NDW == 1) {
    const auto* q = reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(src);
    if constexpr (STREAM) dst[0] = __builtin_nontemporal_load(q);
    else dst[0] = *q;
  } else if constexpr (NDW == 2) {
    const auto* q = reinterpret_cast<const __attribute__((address_space(1))) u32x2_t*>(src);
    u32x2_t v;
    if constexpr (STREAM) v = __builtin_nontemporal_load(q);
    else v = *q;
    dst[0] = v[0];
    dst[1] = v[1];
  } else {
    static_assert(NDW % 4 == 0, "16-byte granules");
#pragma unroll
    for (int i = 0; i < NDW / 4; ++i) {
      u32x4_t v = gload16s<STREAM>(src + 16 * i);
      dst[4 * i + 0] = v[0];
      dst[4 * i + 1] = v[1];
      dst[4 * i + 2] = v[2];
      dst[4 * i + 3] = v[3];
    }
  }
}

// Workgroup id -> (slot, kv head) for grids of one workgroup per (slot, kv
// head). Consecutive ids go to the 8 XCDs in turn, and the kv heads of one
// slot share an XCD (ids x, x+8, x+16, ...), so each XCD reads whole token
// rows. Within an XCD the dispatcher deals workgroups to its 4 shader engines
// in turn and strictly in order. With a fixed head per dispatch position each
// engine would always get the same heads, and heads do not stream at the same
// rate (their byte offset in the token row decides where their rows fall in
// the memory system; on the Llama-3-8B layout two of the 8 heads run 15-40%
// slower). The engine holding the slow heads would then stall the in-order
// dispatch of its whole XCD, so the heads of consecutive slots are rotated
// and every engine sees every head.
__device__ __forceinline__ void slot_and_head(int id, int num_kv_heads, int& slot, int& kvh) {
  const int xcd = id & 7;
  const int k = id >> 3;
  const int group = k / num_kv_heads;
  const int span = num_kv_heads >= 4 ? 1 : 4 / num_kv_heads;
  kvh = (k - group * num_kv_heads + group / span) % num_kv_heads;
  slot = group * 8 + xcd;
}

// Workgroup id -> (slot, kv head) for launches whose consecutive slots share
// keys (several tiles of new tokens of one sequence). Each XCD walks its slots
// in phases of kPhase slot groups: within a phase it serves one kv head for
// all the phase's slots before the next head, so the tiles that re-read a
// sequence's keys of one head run on one XCD close together and find them in
// its L2, instead of every XCD holding every head (on the batch-256 step with
// a 1,024-token chunk, phases of 16, 32 and 64 groups ran 259, 243 and 238 us;
// 64 holds that whole grid). Heads are rotated by XCD
// and by phase so that no XCD keeps the slower heads. `grid` must be
// ceil(slots / 8) * 8 * num_kv_heads; the map is a bijection onto
// [0, grid / num_kv_heads) x [0, num_kv_heads).
__device__ __forceinline__ void slot_and_head_phased(int id, int grid, int num_kv_heads, int& slot, int& kvh) {
  constexpr int kPhase = 64;
  const int xcd = id & 7;
  const int k = id >> 3;
  const int groups = (grid >> 3) / num_kv_heads;  // slot groups of 8 (one slot per XCD)
  const int span = kPhase * num_kv_heads;
  const int phase = k / span;
  const int full = groups / kPhase;
  const int f = phase < full ? kPhase : groups - full * kPhase;  // groups in this phase
  const int r = k - phase * span;
  const int h = r / f;
  kvh = (h + xcd + phase) % num_kv_heads;
  slot = (phase * kPhase + (r - h * f)) * 8 + xcd;
}

}  // namespace pa
