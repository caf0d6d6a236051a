// K/V tile loads and the MFMA score tile shared by the paged-attention
// kernels (gfx950 only). Layout of one tile (16 tokens of one block, one kv
// head): for the score MFMA, lane l holds K row (l % 16), 16-byte pieces at
// byte offset s*64 + (l/16)*16 (16-bit caches load K row by row and reach
// this layout through LDS: k_rows_to_mfma); for the value side, lane l holds
// rows 4*(l/16) .. 4*(l/16)+3, elements (l%16)*D/16 .. (l%16+1)*D/16 - 1 of
// each.
#pragma once

#include "pa_device.h"

namespace pa {

// T: query/output element; F8: the caches hold FP8 E4M3 codes (with bf16
// queries) instead of T.
template <typename T, int D, int G, int CB, bool F8 = false>
struct DecodeShape {
  static constexpr int kElemBytes = F8 ? 1 : static_cast<int>(sizeof(T));  // cache element
  static constexpr int kKSeg = D * kElemBytes / 64;  // 16-byte K loads per lane per block
  static constexpr int kQSeg = F8 ? 2 * kKSeg : kKSeg;  // 16-byte query pieces per lane (MFMA k-steps)
  static constexpr int kVec = D / 16;                // V elements per lane per token
  static constexpr int kVDw = kVec * kElemBytes / 4; // ... as dwords
  // 16-bit caches can load K row by row (each load instruction covers whole
  // token rows) and pass it through LDS into the MFMA operand layout; see
  // load_chunk (ROWK) and k_rows_to_mfma. (FP8 caches measured slower that
  // way: 100.2 vs 94.0 us for the batch-256 step.)
  static constexpr bool kRowKCapable = !F8 && sizeof(T) == 2;
  static constexpr int kRowPieces = D * kElemBytes / 16;  // 16-byte pieces per K row
  static constexpr int kRowsPerLoad = kWave / kRowPieces;  // K rows per load instruction
  static_assert(kKSeg >= 1 && kVDw >= 1, "shape");
  static_assert(G >= 1 && G <= 16, "group");
  static_assert(!F8 || sizeof(T) == 2, "FP8 caches take bf16 queries");
};

template <typename T, int D, int G, int CB, bool F8 = false>
struct Chunk {
  using S = DecodeShape<T, D, G, CB, F8>;
  u32x4_t k[CB][S::kKSeg];
  uint32_t v[CB][4][S::kVDw];
};

// Loads one chunk (CB blocks) of K and V for this wave's kv head. Block ids
// are wave-uniform, so each load is a scalar base (block, head, row) plus a
// 32-bit per-lane offset. Block blk_last holds only last_rows valid rows: its
// lanes for later rows read the last valid row again (same lines, no extra
// memory traffic); those rows are masked out by the caller (16-bit and FP8
// caches). STREAM: non-temporal loads (data no other workgroup reads again).
// ROWK (16-bit caches): K loaded row by row, for k_rows_to_mfma. use_ids:
// ids[i] is the table entry of block blk0 + i, read in advance (used where the
// block is not clamped to blk_last).
template <typename T, int D, int G, int CB, bool F8 = false, bool STREAM = false, bool ROWK = false>
__device__ __forceinline__ void load_chunk(Chunk<T, D, G, CB, F8>& f, const char* kc, const char* vc,
                                           const int32_t* bt_row, int blk0, int blk_last,
                                           int64_t num_blocks, uint32_t tok_stride_bytes,
                                           int64_t blk_stride_bytes, int64_t head_off_bytes,
                                           int lane, int last_rows, const int32_t (&ids)[CB], bool use_ids) {
  using S = DecodeShape<T, D, G, CB, F8>;
  const int tok = lane & 15;
  const int j = lane >> 4;
  const int lr = last_rows - 1;
  const uint32_t vcol = tok * (S::kVDw * 4);
  const uint32_t koff = tok * tok_stride_bytes + j * 16;                      // K: row tok, piece j
  const uint32_t koff_last = min(tok, lr) * tok_stride_bytes + j * 16;
  const uint32_t voff = (4 * j) * tok_stride_bytes + vcol;                   // V: rows 4j.., piece tok
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int b = min(blk0 + i, blk_last);
    const bool last = b == blk_last;
    // Out-of-range ids (negative included) are clamped so a bad table never
    // leads to an out-of-bounds access.
    const int32_t id = (use_ids && blk0 + i <= blk_last) ? ids[i] : bt_row[b];
    uint64_t phys = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(id));
    phys = phys < static_cast<uint64_t>(num_blocks) ? phys : static_cast<uint64_t>(num_blocks - 1);
    const int64_t base = static_cast<int64_t>(phys) * blk_stride_bytes + head_off_bytes;
    const gchar_t* kb = uniform_ptr(kc + base);
    const gchar_t* vb = uniform_ptr(vc + base);
    static_assert(!ROWK || S::kRowKCapable, "row-wise K needs 16-bit caches");
    if constexpr (ROWK) {
      // K: load s covers rows kRowsPerLoad * s + lane / kRowPieces; lane l
      // takes piece (l - row) mod kRowPieces of its row, so that the pieces
      // land rotated by the row in LDS (k_rows_to_mfma) and the MFMA-layout
      // reads hit distinct banks. Rows past the last valid one of the
      // context's last block read that row again (the wave-uniform limit
      // `lim` is 15 elsewhere). Offsets stay unsigned 32-bit so that the loads
      // take the scalar-base + lane-offset form, and row * stride is a 24-bit
      // multiply (row <= 15; the callers keep a token row under 2^24 bytes).
      const uint32_t lim = static_cast<uint32_t>(last ? lr : kBlockTokens - 1);
#pragma unroll
      for (int s = 0; s < S::kKSeg; ++s) {
        const uint32_t row = static_cast<uint32_t>(S::kRowsPerLoad * s + lane / S::kRowPieces);
        const uint32_t piece = static_cast<uint32_t>(lane - static_cast<int>(row)) & (S::kRowPieces - 1);
        f.k[i][s] = gload16s<STREAM>(kb + (__umul24(min(row, lim), tok_stride_bytes) + piece * 16u));
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // V: rows 4j + r, piece tok.
        const uint32_t row = min(static_cast<uint32_t>(4 * j + r), lim);
        load_dwords<S::kVDw, STREAM>(f.v[i][r], vb + (__umul24(row, tok_stride_bytes) + vcol));
      }
    } else if constexpr (S::kElemBytes <= 2) {
      const uint32_t ko = last ? koff_last : koff;
#pragma unroll
      for (int s = 0; s < S::kKSeg; ++s) f.k[i][s] = gload16s<STREAM>(kb + s * 64 + ko);
      // V: rows 4j + r, piece tok, clamped to the wave-uniform limit; unsigned
      // 32-bit offsets with a 24-bit row multiply, as in the row-wise K loads.
      const uint32_t lim = static_cast<uint32_t>(last ? lr : kBlockTokens - 1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t row = min(static_cast<uint32_t>(4 * j + r), lim);
        load_dwords<S::kVDw, STREAM>(f.v[i][r], vb + (__umul24(row, tok_stride_bytes) + vcol));
      }
    } else {
      // fp32 caches (the small workloads) read whole blocks: the per-row
      // offsets would spill registers there.
#pragma unroll
      for (int s = 0; s < S::kKSeg; ++s) f.k[i][s] = gload16s<STREAM>(kb + s * 64 + koff);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        load_dwords<S::kVDw, STREAM>(f.v[i][r], vb + r * tok_stride_bytes + voff);
    }
  }
}

template <typename T, int D, int G, int CB, bool F8 = false, bool STREAM = false, bool ROWK = false>
__device__ __forceinline__ void load_chunk(Chunk<T, D, G, CB, F8>& f, const char* kc, const char* vc,
                                           const int32_t* bt_row, int blk0, int blk_last,
                                           int64_t num_blocks, uint32_t tok_stride_bytes,
                                           int64_t blk_stride_bytes, int64_t head_off_bytes,
                                           int lane, int last_rows = kBlockTokens) {
  const int32_t none[CB] = {};
  load_chunk<T, D, G, CB, F8, STREAM, ROWK>(f, kc, vc, bt_row, blk0, blk_last, num_blocks, tok_stride_bytes,
                                            blk_stride_bytes, head_off_bytes, lane, last_rows, none, false);
}

// Table entries of a wave's first chunk (blocks blk0 .. blk0 + CB - 1, kept
// inside the row), requested before the context length is known: the first
// K/V loads then wait for one scalar round trip fewer.
template <int CB>
__device__ __forceinline__ void first_chunk_ids(int32_t (&ids)[CB], const int32_t* bt_row, int blk0, int max_blocks) {
#pragma unroll
  for (int i = 0; i < CB; ++i) ids[i] = bt_row[min(blk0 + i, max_blocks - 1)];
}

// K rows of a chunk loaded row by row (16-bit caches) into the MFMA operand
// layout (lane l: row l % 16, piece 4 s + l / 16 at k-step s), through this
// wave's LDS area `kt` (CB blocks of 16 x kRowPieces 16-byte pieces). Each lane
// stores its pieces at consecutive addresses; piece p of row t sits at
// position (p + t) mod kRowPieces of the row, so the 16 lanes reading one
// k-step's piece of rows 0..15 use distinct banks. Only this wave touches
// `kt`, and a wave's LDS operations complete in order, so no barrier is needed.
template <typename T, int D, int G, int CB, bool F8>
__device__ __forceinline__ void k_rows_to_mfma(Chunk<T, D, G, CB, F8>& f, u32x4_t* kt, int lane) {
  using S = DecodeShape<T, D, G, CB, F8>;
  constexpr int kBlockPieces = kBlockTokens * S::kRowPieces;
#pragma unroll
  for (int i = 0; i < CB; ++i)
#pragma unroll
    for (int s = 0; s < S::kKSeg; ++s) kt[i * kBlockPieces + s * kWave + lane] = f.k[i][s];
  const int t = lane & 15;
  const int j = lane >> 4;
#pragma unroll
  for (int i = 0; i < CB; ++i)
#pragma unroll
    for (int s = 0; s < S::kKSeg; ++s)
      f.k[i][s] = kt[i * kBlockPieces + t * S::kRowPieces + ((4 * s + j + t) & (S::kRowPieces - 1))];
}

// Scores of one chunk: s[i][r] = scale*log2(e) * <q, K> for token 4*(lane/16)+r
// of block i and head lane % 16.
template <typename T, int D, int G, int CB, bool F8 = false>
__device__ __forceinline__ void qk_chunk(float (&s)[CB][4], const Chunk<T, D, G, CB, F8>& f,
                                         const u32x4_t (&q)[DecodeShape<T, D, G, CB, F8>::kQSeg],
                                         float scale_log2) {
  using S = DecodeShape<T, D, G, CB, F8>;
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sg = 0; sg < S::kKSeg; ++sg) {
      if constexpr (F8) {
        // 16 codes per load: dwords 0-1 feed k-step 2*sg, dwords 2-3 k-step
        // 2*sg+1, converted exactly to bf16 (the query uses the same d order).
#pragma unroll
        for (int h = 0; h < 2; ++h)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(f.k[i][sg][2 * h], f.k[i][sg][2 * h + 1]),
                                                      __builtin_bit_cast(bf16x8_t, q[2 * sg + h]), c, 0, 0, 0);
      } else if constexpr (sizeof(T) == 2) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f.k[i][sg]),
                                                    __builtin_bit_cast(bf16x8_t, q[sg]), c, 0, 0, 0);
      } else {
        // Vector elements are read into scalars first: bit-casting a vector
        // element in place is not reliable.
#pragma unroll
        for (int e = 0; e < 4; ++e)
          c = __builtin_amdgcn_mfma_f32_16x16x4f32(as_float(f.k[i][sg][e]), as_float(q[sg][e]), c, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) s[i][r] = c[r] * scale_log2;
  }
}

}  // namespace pa
