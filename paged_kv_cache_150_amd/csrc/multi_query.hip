// Multi-query paged attention for gfx950: pa_multi_query.
//
// What is computed (llm-stack-book 7.3 "vLLM: Architecture, PagedAttention &
// Internals", sections "Prefill, decode, and chunked prefill", "The forward
// step in detail" and "Speculative decoding support"): one step may hand a
// sequence several new tokens (a prompt chunk, or the k+1 positions a
// speculative step verifies). Their K/V are already in the cache, so with n
// tokens stored and q of them new, new token j sits at position n - q + j and
// attends over positions 0 .. n - q + j of the sequence's paged context.
//
// Work decomposition: a workgroup takes one tile of one sequence and one kv
// head. A tile is 16*NT "columns", each a (new token, query head) pair: the
// group's g heads for 16*NT/g consecutive new tokens. Its 4 waves split the
// tile's key range into chunks of CB blocks (chunk c to wave c % 4) and merge
// through LDS at the end, as in the decode kernel.
//  * Scores: the decode kernel's 16x16 MFMA tile, A = 16 K rows of a block,
//    B = 16 columns; lane l gets the scores of keys 4*(l/16)+r of the block for
//    column l % 16.
//  * Causal limit per column: column (token j, head h) sees keys up to its own
//    position. Only the last one to three chunks of a tile reach past the first
//    token's position, and each is the last chunk of its wave.
//  * P*V on MFMA, without moving data between lanes: lane l already holds V
//    rows 4*(l/16)..+3, elements (l%16)*D/16 .. +D/16 of each (the decode
//    tile layout), and the probabilities of the same four keys for column
//    l % 16. Taking element t of each lane's piece gives the A operand of a
//    16x16 MFMA whose rows are d = (D/16)*m + t, contracted over the keys
//    (K = 4 keys of a block, or 8 keys of two blocks), with B = the
//    probabilities. Lane l ends up owning output elements
//    d in [(l/16)*D/4, (l/16+1)*D/4) of column l % 16.
//  * Probabilities enter the bf16 MFMA rounded to bf16 (relative error at
//    most 2^-8 per weight, so an output moves by at most 2^-8 * max |v|);
//    the normaliser and the log-sum-exp use the fp32 values. fp32 caches use the fp32 MFMA and keep fp32 probabilities.
//  * Online softmax in base 2, per column, with a reference point that moves
//    only when a chunk's maximum exceeds it by more than 2^8 in weight; a
//    column with no visible key yet keeps weight 0.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_tiles.h"

namespace pa {

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4_t;

// Waves per workgroup: 4 (two workgroups per CU), or 8 (one per CU) when a
// launch has at most one job per resident 4-wave workgroup, so that each job
// is split over twice the waves.

struct MultiArgs {
  const void* query;              // [num_tokens, num_heads, D]
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;    // tokens stored per sequence, new ones included
  const int32_t* query_start_loc; // [num_seqs + 1]: sequence i's new tokens are rows [loc[i], loc[i+1]);
                                  // null: one new token per sequence, row i (decode)
  const int32_t* seq_order;       // decode only, optional: slot i takes sequence seq_order[i]
  void* out;                      // [num_tokens, num_heads, D]
  float* lse_out;                 // optional [num_tokens, num_heads]
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;        // H_q / H_kv
  int32_t tile_tokens;  // new tokens per tile: 16 * NT / group
  int32_t num_slots;    // tile slots: num_tokens / tile_tokens + num_seqs
  float scale_log2;     // scale * log2(e) (times k_scale for FP8 caches)
  float v_scale;        // multiplies the normalised output: v_scale for FP8 caches, else 1
  // Shared-prefix pass (prefix_keys > 0): one context, the first
  // prefix_keys / 16 blocks of block table row 0, attended by num_tokens
  // queries, query row t being sequence t's decode query; column (t, h) sees
  // min(context_lens[t], prefix_keys) keys. Normalised float32 outputs and
  // log-sum-exps go to part_o [num_tokens, num_heads, D] / part_lse.
  int32_t prefix_keys;
  float* part_o;
  float* part_lse;
  // Decode mode as the suffix pass of the shared-prefix decode: keys of
  // blocks < skip_blocks were attended by the prefix pass, whose normalised
  // output and log-sum-exp per (sequence, query head) join the final merge.
  int32_t skip_blocks;
  const float* prefix_o;    // [num_seqs, num_heads, D]
  const float* prefix_lse;  // [num_seqs, num_heads]
  // Decode mode with the new tokens' write folded in: sequence i's new K/V
  // (new_key/new_value row i, [num_seqs, H_kv, D]) go to slot_mapping[i]
  // first. Null: the caches already hold them.
  const void* new_key;             // query dtype (bf16 for FP8 caches)
  const void* new_value;
  const int64_t* slot_mapping;
  float k_scale;                   // FP8 caches: the write's scales (codes = value / scale)
  float v_scale_write;
  float k_inv, v_inv;              // their exact reciprocals when scales_pow2
  int32_t scales_pow2;             // both scales are powers of two
  // Decode mode cut into context partitions (part_blocks > 0): slot
  // p * num_seqs + j attends the keys [p * P, min((p + 1) * P, n)) of sequence
  // i = (j - p) mod num_seqs (P = 16 * part_blocks) and writes the normalised
  // float32 output and the log-sum-exp of each query head h to part_o /
  // part_lse row (i * num_heads + h) * parts_stride + p. Partitions past the
  // context end write nothing. First partitions (full ones) are dispatched
  // first; the rotation by p moves each sequence to another XCD from one
  // partition to the next, so every XCD gets a share of every context.
  int32_t part_blocks;
  int32_t num_parts;
  int32_t parts_stride;
  int32_t part_cap;  // keys at or past this position are ignored
  // Multi-query mode cut into context partitions (part_blocks > 0 with
  // query_start_loc): slot p * tile_slots + j is partition p of tile slot
  // (j - p) mod tile_slots; each column sees the partition's keys below its
  // own limit, and its normalised output and log-sum-exp go to part_o /
  // part_lse row (token row * num_heads + head) * parts_stride + p.
  int32_t tile_slots;
};

// Tile slots: sequence i owns slots [B_i, B_{i+1}) with
// B_i = loc[i] / tile_tokens + i. That is at least ceil(q_i / tile_tokens)
// slots (at most one more), B is non-decreasing, and B_S is a host-known
// bound, so a slot's sequence is the number of i >= 1 with B_i <= slot.
__device__ __forceinline__ int clamp_loc(int v, int num_tokens) { return v < 0 ? 0 : (v > num_tokens ? num_tokens : v); }

__device__ __forceinline__ int slot_owner(const MultiArgs& a, int slot, int lane) {
  int count = 0;
  for (int base = 1; base <= a.num_seqs; base += kWave) {
    const int i = base + lane;
    bool le = false;
    if (i <= a.num_seqs) le = clamp_loc(a.query_start_loc[i], a.num_tokens) / a.tile_tokens + i <= slot;
    const uint64_t m = __ballot(le);
    count += __popcll(m);
    if (m != ~0ull) break;  // B is non-decreasing: no later i qualifies
  }
  return count;
}

template <typename T, int D, int CB, int NT>
struct MqState {
  static constexpr int kTiles = D / 16;  // output d-tiles: tile t holds d = (D/16)*m + t
  float m[NT];              // running max (base-2 scaled) of column lane%16 of part p
  float l[NT];              // partial normaliser over this lane's keys
  f32x4_t acc[NT][kTiles];  // d = (D/16)*(4*(lane/16) + r) + t, column lane%16
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v_t{a, b}, bf16x2v_t));
}
// Element t of a lane's bf16 piece, taken from two rows, packed (row a low):
// one byte permute (bytes 0-3 of x, 4-7 of y).
template <int T_>
__device__ __forceinline__ uint32_t pick_bf16(const uint32_t* ra, const uint32_t* rb) {
  return __builtin_amdgcn_perm(rb[T_ / 2], ra[T_ / 2], (T_ & 1) ? 0x07060302u : 0x05040100u);
}

// One chunk of the online softmax and P*V. MASK: the chunk reaches past some
// column's last visible key (a compile-time choice, so the chunks that need no
// mask carry none of its selects).
template <typename T, int D, int CB, int NT, bool F8, bool MASK>
__device__ __forceinline__ void mq_chunk(MqState<T, D, CB, NT>& st, const Chunk<T, D, 16, CB, F8>& f,
                                         const u32x4_t (&q)[NT][DecodeShape<T, D, 16, CB, F8>::kQSeg],
                                         float scale_log2, int tok0, const int (&lim)[NT], int key_end, int lane) {
  using S = DecodeShape<T, D, 16, CB, F8>;
  constexpr int kTiles = D / 16;
  const int rg = lane >> 4;
  uint32_t vz[CB][4][S::kVDw];
#pragma unroll
  for (int i = 0; i < CB; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int w = 0; w < S::kVDw; ++w) vz[i][r][w] = f.v[i][r][w];
  // Raw scores <q, K>; scale*log2(e) is applied inside the exponent.
  float s[NT][CB][4];
#pragma unroll
  for (int p = 0; p < NT; ++p) qk_chunk<T, D, 16, CB, F8>(s[p], f, q[p], 1.0f);
  if constexpr (MASK) {
    // Keys at or past the tile's last position: weight 0 for every column,
    // and their V rows (possibly stale or poisoned) are replaced by 0.
#pragma unroll
    for (int i = 0; i < CB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = tok0 + i * 16 + 4 * rg + r;
#pragma unroll
        for (int p = 0; p < NT; ++p) s[p][i][r] = key < lim[p] ? s[p][i][r] : -__builtin_inff();
        const bool live = key < key_end;
#pragma unroll
        for (int w = 0; w < S::kVDw; ++w) vz[i][r][w] = live ? vz[i][r][w] : 0u;
      }
  }
  // Online softmax with a lazily moved reference point: a column's reference
  // m only moves (and its partial sums are rescaled) when the chunk maximum
  // exceeds it by more than kLazy (base-2 units), so weights stay below
  // 2^kLazy and most chunks skip the rescaling of the accumulators. A
  // column with no visible key yet keeps m = -inf and weight 0.
  constexpr float kLazy = 8.0f;
  float alpha[NT];
  bool any = false;
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    float mx = s[p][0][0];
#pragma unroll
    for (int i = 0; i < CB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[p][i][r]);
    mx = rows_max(mx) * scale_log2;
    const bool move = mx > st.m[p] + kLazy;
    alpha[p] = move ? st.m[p] - mx : 0.f;  // log2 of the rescale factor
    st.m[p] = move ? mx : st.m[p];
    any = any || move;
  }
  if (__builtin_amdgcn_ballot_w64(any) != 0) {
#pragma unroll
    for (int p = 0; p < NT; ++p) {
      alpha[p] = fast_exp2(alpha[p]);
      st.l[p] *= alpha[p];
#pragma unroll
      for (int t = 0; t < kTiles; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.acc[p][t][r] *= alpha[p];
    }
  }
  float pw[NT][CB][4];
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    const float neg_m = st.m[p] == -__builtin_inff() ? 0.f : -st.m[p];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < CB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pw[p][i][r] = fast_exp2(fmaf(s[p][i][r], scale_log2, neg_m));
        psum += pw[p][i][r];
      }
    st.l[p] += psum;
  }

  if constexpr (sizeof(T) == 2) {
    // bf16: probabilities rounded to bf16, contracted with V over 8 keys of
    // two blocks per MFMA, or 4 keys of the odd block out. FP8 V codes are
    // first converted to bf16 (exact), giving the same per-lane rows.
    constexpr int kBW = D / 32;  // bf16 dwords of a lane's piece of one row
    // Element t of rows ra and rb of block i as a bf16 pair (row ra low). FP8
    // codes are first byte-permuted into (ra, rb) pairs, then converted: one
    // permute serves two elements.
    auto vpair = [&](int i, int ra, int rb, auto tc) __attribute__((always_inline)) {
      constexpr int t = decltype(tc)::value;
      if constexpr (F8) {
        const uint32_t p = __builtin_amdgcn_perm(vz[i][rb][t / 4], vz[i][ra][t / 4],
                                                 (t % 4) < 2 ? 0x05010400u : 0x07030602u);
        return fp8x2_to_bf16x2(p, (t & 1) != 0);
      } else {
        static_assert(kBW == S::kVDw, "bf16 piece");
        return pick_bf16<t>(&vz[i][ra][0], &vz[i][rb][0]);
      }
    };
#pragma unroll
    for (int i = 0; i < CB; i += 2) {
      if (i + 1 < CB) {
        u32x4_t b[NT];
#pragma unroll
        for (int p = 0; p < NT; ++p) {
          b[p] = u32x4_t{pack_bf16(pw[p][i][0], pw[p][i][1]), pack_bf16(pw[p][i][2], pw[p][i][3]),
                         pack_bf16(pw[p][i + 1][0], pw[p][i + 1][1]), pack_bf16(pw[p][i + 1][2], pw[p][i + 1][3])};
        }
        static_for<kTiles>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          const u32x4_t av = {vpair(i, 0, 1, tc), vpair(i, 2, 3, tc), vpair(i + 1, 0, 1, tc), vpair(i + 1, 2, 3, tc)};
#pragma unroll
          for (int p = 0; p < NT; ++p)
            st.acc[p][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                                   __builtin_bit_cast(bf16x8_t, b[p]),
                                                                   st.acc[p][t], 0, 0, 0);
        });
      } else {
        u32x2_t b[NT];
#pragma unroll
        for (int p = 0; p < NT; ++p) {
          b[p] = u32x2_t{pack_bf16(pw[p][i][0], pw[p][i][1]), pack_bf16(pw[p][i][2], pw[p][i][3])};
        }
        static_for<kTiles>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          const u32x2_t av = {vpair(i, 0, 1, tc), vpair(i, 2, 3, tc)};
#pragma unroll
          for (int p = 0; p < NT; ++p)
            st.acc[p][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, av),
                                                                     __builtin_bit_cast(bf16x4_t, b[p]),
                                                                     st.acc[p][t], 0, 0, 0);
        });
      }
    }
  } else {
    // fp32: one key per lane per MFMA (K = 4: keys 4*(l/16) + r of a block).
#pragma unroll
    for (int i = 0; i < CB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < kTiles; ++t)
#pragma unroll
          for (int p = 0; p < NT; ++p)
            st.acc[p][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(as_float(vz[i][r][t]), pw[p][i][r], st.acc[p][t],
                                                                0, 0, 0);
  }
}


// The new token's bf16 K and V pieces of one lane (kraw: two 16-byte loads per
// 16-code K piece; vraw: the V piece) to E4M3 codes in the layout the FP8
// chunk loads use (kn: 16 codes per K piece, vn: 4 codes per dword).
// KQ: the K pieces to quantize (all KS, or just the first with row-wise K).
template <bool POW2, int KQ, int KS, int VD>
__device__ __forceinline__ void quantize_rows(u32x4_t (&kn)[KS], uint32_t (&vn)[VD], const u32x4_t (&kraw)[2 * KS],
                                              const uint32_t (&vraw)[2 * VD], float k_scale, float k_inv,
                                              float v_scale, float v_inv) {
#pragma unroll
  for (int sg = 0; sg < KQ; ++sg) {
    const u32x4_t lo = kraw[2 * sg], hi = kraw[2 * sg + 1];
    kn[sg] = u32x4_t{quantize_bf16x4_e4m3<POW2>(lo[0], lo[1], k_scale, k_inv),
                     quantize_bf16x4_e4m3<POW2>(lo[2], lo[3], k_scale, k_inv),
                     quantize_bf16x4_e4m3<POW2>(hi[0], hi[1], k_scale, k_inv),
                     quantize_bf16x4_e4m3<POW2>(hi[2], hi[3], k_scale, k_inv)};
  }
#pragma unroll
  for (int w = 0; w < VD; ++w) vn[w] = quantize_bf16x4_e4m3<POW2>(vraw[2 * w], vraw[2 * w + 1], v_scale, v_inv);
}

// Query fragments of a tile's columns: column c = 16 p + (lane % 16) is new
// token c / g (row `row0` + c / g) and head head0 + c % g; columns past the
// tile's `ncols` get zeros. Same d order as the K operand of qk_chunk.
template <typename T, int D, int CB, int NT, bool F8>
__device__ __forceinline__ void load_query_cols(const void* query, int64_t row0, int num_heads, int head0, int g,
                                                int ncols, int lane,
                                                u32x4_t (&q)[NT][DecodeShape<T, D, 16, CB, F8>::kQSeg]) {
  using S = DecodeShape<T, D, 16, CB, F8>;
  constexpr int kQBytes = static_cast<int>(sizeof(T));
  const int j = lane >> 4;
  const gchar_t* qb = uniform_ptr(static_cast<const char*>(query) + (row0 * num_heads + head0) * D * kQBytes);
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    const int c = 16 * p + (lane & 15);
    const bool valid = c < ncols;
    const int tok = c / g;
    const uint32_t qoff = valid ? static_cast<uint32_t>((tok * num_heads + c - tok * g) * D * kQBytes) : 0u;
#pragma unroll
    for (int sg = 0; sg < S::kQSeg; ++sg) {
      // The K operand's d order: 32 sg + 8 j + e for bf16/fp32 caches; for
      // FP8 caches (16 codes per lane per load) 64 (sg/2) + 16 j + 8 (sg%2) + e.
      const uint32_t off = F8 ? 128 * (sg / 2) + 32 * j + 16 * (sg % 2) : sg * 64 + j * 16;
      u32x4_t v = gload16(qb + off + qoff);
      q[p][sg] = valid ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
}

// One workgroup of W waves per (tile slot, kv head); slot ids follow the
// decode kernel's XCD-aware order (id % 8 names the XCD; the kv heads of a
// slot share it).
template <typename T, int D, int CB, int NT, bool F8, int W>
__global__ __launch_bounds__(W * kWave, W == 4 ? 2 : 1) void paged_multi_query_kernel(MultiArgs a) {
  constexpr int kMqWaves = W;
  using S = DecodeShape<T, D, 16, CB, F8>;
  constexpr int kCols = 16 * NT;
  constexpr int kRow = D + 4;  // LDS row stride in floats: 16-byte rows, the 16 columns on distinct banks
  // s_acc also holds each wave's K staging area (k_rows_to_mfma) during the
  // chunk loop; a barrier separates the two uses.
  __shared__ __attribute__((aligned(16))) float s_acc[kMqWaves][kCols][kRow];
  __shared__ float s_m[kMqWaves][kCols];
  __shared__ float s_l[kMqWaves][kCols];
  __shared__ float s_w[kMqWaves + 1][kCols];  // merge weights per column (last: the prefix part)
  __shared__ float s_L[kCols];                // normaliser per column
  __shared__ float s_lse[kCols];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = a.group;
  // 16-column tiles of 16-bit caches load K row by row (k_rows_to_mfma); the
  // 32-column ones keep the direct operand loads (the staging pushes them
  // past the register budget).
  constexpr bool kRowK = S::kRowKCapable && NT == 1;
  constexpr int kStagePieces = CB * kBlockTokens * S::kRowPieces;  // 16-byte pieces per wave
  static_assert(!kRowK || sizeof(s_acc) >= sizeof(u32x4_t) * kStagePieces * kMqWaves, "K staging fits s_acc");
  u32x4_t* k_stage = reinterpret_cast<u32x4_t*>(&s_acc[0][0][0]) + wave * kStagePieces;

  int slot, kvh;
  if (a.query_start_loc != nullptr && a.part_blocks == 0 && a.prefix_keys == 0)
    slot_and_head_phased(blockIdx.x, gridDim.x, a.num_kv_heads, slot, kvh);
  else
    slot_and_head(blockIdx.x, a.num_kv_heads, slot, kvh);
  if (slot >= a.num_slots) return;
  const int max_tokens = a.max_blocks * kBlockTokens;
  auto clamp_len = [&](int v) { return v < 0 ? 0 : (v > max_tokens ? max_tokens : v); };
  // The tile reads keys [16 * blk_begin, key_end); column p of this lane sees
  // keys below lim[p]; min_lim is the smallest limit of the tile's columns.
  int seq, q0, tok0, ntok, key_end, min_lim, blk_begin = 0, part = -1;
  int lim[NT];
  // One-pass decode with 16-bit caches: the first chunk's table entries are
  // requested with the context length (FP8 caches measured slower with it).
  int32_t first_ids[CB] = {};
  bool have_first = false;
  if (a.prefix_keys > 0) {
    // Shared-prefix pass: tile `slot` of the queries, all over row 0's prefix.
    seq = 0;
    q0 = 0;
    tok0 = slot * a.tile_tokens;
    if (tok0 >= a.num_tokens) return;
    ntok = min(a.tile_tokens, a.num_tokens - tok0);
    // Each lane reads its columns' lengths (one round trip); the tile's key
    // range and smallest limit are reductions over the 16 columns of a row.
    int hi = 0, lo = a.prefix_keys;
#pragma unroll
    for (int p = 0; p < NT; ++p) {
      const int c = 16 * p + (lane & 15);
      const bool valid = c < ntok * g;
      lim[p] = valid ? min(clamp_len(a.context_lens[tok0 + c / g]), a.prefix_keys) : 0;
      hi = max(hi, lim[p]);
      lo = valid ? min(lo, lim[p]) : lo;
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) {
      hi = max(hi, __shfl_xor(hi, m, kWave));
      lo = min(lo, __shfl_xor(lo, m, kWave));
    }
    key_end = __builtin_amdgcn_readfirstlane(hi);
    min_lim = __builtin_amdgcn_readfirstlane(lo);
  } else {
    int q1, r;
    if (a.query_start_loc == nullptr) {
      // One new token per sequence (decode): slot i is sequence i (or
      // seq_order[i], clamped), query row = sequence; with partitions, slot
      // p * num_seqs + j is partition p of sequence (j - p) mod num_seqs.
      if (a.part_blocks > 0) {
        part = slot / a.num_seqs;
        const int j = slot - part * a.num_seqs;
        const int rot = part % a.num_seqs;
        seq = j >= rot ? j - rot : j - rot + a.num_seqs;
        blk_begin = part * a.part_blocks;
      } else {
        if (slot >= a.num_seqs) return;
        seq = slot;
        if (a.seq_order != nullptr) {
          const uint32_t o = static_cast<uint32_t>(a.seq_order[slot]);
          seq = static_cast<int>(o < static_cast<uint32_t>(a.num_seqs) ? o : a.num_seqs - 1);
        }
        blk_begin = a.skip_blocks;
        if constexpr (!F8) {
          first_chunk_ids<CB>(first_ids, a.block_tables + static_cast<int64_t>(seq) * a.max_blocks,
                              blk_begin + wave * CB, a.max_blocks);
          have_first = true;
        }
      }
      q0 = seq;
      q1 = seq + 1;
      r = 0;
    } else {
      int tslot = slot;
      if (a.part_blocks > 0) {
        part = slot / a.tile_slots;
        const int j = slot - part * a.tile_slots;
        const int rot = part % a.tile_slots;
        tslot = j >= rot ? j - rot : j - rot + a.tile_slots;
        blk_begin = part * a.part_blocks;
      }
      seq = __builtin_amdgcn_readfirstlane(slot_owner(a, tslot, lane));
      if (seq >= a.num_seqs) return;
      q0 = clamp_loc(a.query_start_loc[seq], a.num_tokens);
      q1 = clamp_loc(a.query_start_loc[seq + 1], a.num_tokens);
      r = tslot - (q0 / a.tile_tokens + seq);
    }
    const int ql = q1 - q0;
    if (ql <= 0) return;
    const int ntiles = (ql + a.tile_tokens - 1) / a.tile_tokens;
    if (r < 0 || r >= ntiles) return;
    // Later tiles see longer contexts: they take the lower slots of the sequence.
    const int tile = ntiles - 1 - r;
    tok0 = tile * a.tile_tokens;                               // first new token of the tile
    ntok = min(a.tile_tokens, ql - tok0);
    const int n = clamp_len(a.context_lens[seq]);
    const int pos0 = n - ql + tok0;                            // position of the tile's first token
    key_end = max(0, pos0 + ntok);                             // keys [0, key_end) are read
    min_lim = pos0 + 1;
#pragma unroll
    for (int p = 0; p < NT; ++p) {
      const int c = 16 * p + (lane & 15);
      lim[p] = c < ntok * g ? pos0 + c / g + 1 : 0;
    }
    if (part >= 0) {
      // Keys of the partition, each column up to its own limit.
      key_end = min(key_end, a.part_cap);
      if (key_end <= blk_begin * kBlockTokens) return;
      key_end = min(key_end, (blk_begin + a.part_blocks) * kBlockTokens);
      min_lim = min(min_lim, key_end);
#pragma unroll
      for (int p = 0; p < NT; ++p) lim[p] = lim[p] > 0 ? min(lim[p], key_end) : 0;
    }
  }
  const int ncols = ntok * g;

  const uint32_t tok_stride = static_cast<uint32_t>(a.num_kv_heads) * D * S::kElemBytes;
  const int64_t blk_stride = static_cast<int64_t>(tok_stride) * kBlockTokens;
  const int64_t head_off = static_cast<int64_t>(kvh) * D * S::kElemBytes;
  const char* kc = static_cast<const char*>(a.key_cache);
  const char* vc = static_cast<const char*>(a.value_cache);
  const int32_t* bt_row = a.block_tables + static_cast<int64_t>(seq) * a.max_blocks;
  const int blk_end = (key_end + kBlockTokens - 1) / kBlockTokens;
  const int nchunk = blk_end > blk_begin ? (blk_end - blk_begin + CB - 1) / CB : 0;
  const int blk_last = blk_end - 1;
  const int last_rows = key_end - blk_last * kBlockTokens;  // valid rows of the last block
  const int mine = wave < nchunk ? (nchunk - wave + kMqWaves - 1) / kMqWaves : 0;
  auto blk_of = [&](int i) { return blk_begin + (wave + i * kMqWaves) * CB; };
  auto tok_of = [&](int i) { return blk_of(i) * kBlockTokens; };

  // Decode with the new token's write folded in. When the slot is the one the
  // block table gives position n - 1 (the decode step's own token), the wave
  // whose last chunk holds that position loads the new rows, swaps them into
  // that chunk's registers before using it, and stores them to the slot once
  // its chunks are done; nothing in this launch reads the slot from memory
  // after the store, so no ordering is needed. Any other slot (an empty
  // context included) is only written, by wave 0: attention then uses what
  // the cache holds at position n - 1. FP8 caches get the new rows quantized
  // (quantize4_e4m3, the encoding of pa_reshape_and_cache_fp8) in the same
  // register layout as the codes the chunks load. (Decode mode always runs
  // 16-column tiles; the 32-column instantiations leave this out.)
  constexpr bool kFusedWrite = NT == 1;
  u32x4_t kn[S::kKSeg];
  uint32_t vn[S::kVDw];
  u32x4_t kraw[2 * S::kKSeg];  // FP8 caches: the new bf16 rows before quantizing
  uint32_t vraw[2 * S::kVDw];
  bool own_new = false;    // this wave stores the new rows
  bool patch_own = false;  // ... and uses them in place of position n - 1
  int new_ib = 0, new_r0 = 0;
  int64_t new_slot = -1;
  if constexpr (kFusedWrite) {
    if (a.slot_mapping != nullptr) {
      new_slot = a.slot_mapping[seq];
      if (new_slot >= 0 && new_slot < a.num_blocks * kBlockTokens) {
        const int pos = key_end - 1;
        const bool on_pos = pos >= 0 && static_cast<int64_t>(bt_row[pos / kBlockTokens]) * kBlockTokens +
                                            pos % kBlockTokens == new_slot;
        if (on_pos) {
          const int c_last = (pos / kBlockTokens) / CB;
          own_new = c_last % kMqWaves == wave;
          patch_own = own_new;
          new_ib = pos / kBlockTokens - c_last * CB;
          new_r0 = pos % kBlockTokens;
        } else {
          own_new = wave == 0;
        }
      }
    }
    if (own_new) {
      // Only the storing wave reads the new rows (query dtype).
      const int64_t src_off = (static_cast<int64_t>(seq) * a.num_kv_heads + kvh) * D * sizeof(T);
      const gchar_t* ksrc = uniform_ptr(static_cast<const char*>(a.new_key) + src_off);
      const gchar_t* vsrc = uniform_ptr(static_cast<const char*>(a.new_value) + src_off);
      if constexpr (F8) {
        // Elements 64 sg + 16 (lane / 16) .. +15 (K) and (lane % 16) * D/16
        // .. +D/16 - 1 (V): the elements of the codes this lane holds.
        static_assert(!kRowK, "FP8 tiles load K in the operand layout");
#pragma unroll
        for (int sg = 0; sg < S::kKSeg; ++sg) {
          const gchar_t* kp = ksrc + 2 * (sg * 64 + (lane >> 4) * 16);
          kraw[2 * sg] = gload16(kp);
          kraw[2 * sg + 1] = gload16(kp + 16);
        }
        load_dwords<2 * S::kVDw>(vraw, vsrc + 2 * (lane & 15) * S::kVec);
      } else if constexpr (kRowK) {
        // The piece of row new_r0 this lane holds in the row-wise K layout.
        kn[0] = gload16(ksrc + ((lane - new_r0) & (S::kRowPieces - 1)) * 16);
        load_dwords<S::kVDw>(vn, vsrc + (lane & 15) * (S::kVDw * 4));
      } else {
#pragma unroll
        for (int sg = 0; sg < S::kKSeg; ++sg) kn[sg] = gload16(ksrc + sg * 64 + (lane >> 4) * 16);
        load_dwords<S::kVDw>(vn, vsrc + (lane & 15) * (S::kVDw * 4));
      }
    }
  }
  // FP8 caches: the storing wave turns the new rows into codes (the encoding
  // of pa_reshape_and_cache_fp8). Called once the wave's first chunk loads are
  // in flight, so the IEEE divisions overlap their latency.
  auto quantize_new = [&]() __attribute__((always_inline)) {
    if constexpr (kFusedWrite && F8) {
      if (own_new) {
        constexpr int kKQ = kRowK ? 1 : S::kKSeg;
        if (a.scales_pow2)
          quantize_rows<true, kKQ>(kn, vn, kraw, vraw, a.k_scale, a.k_inv, a.v_scale_write, a.v_inv);
        else
          quantize_rows<false, kKQ>(kn, vn, kraw, vraw, a.k_scale, a.k_inv, a.v_scale_write, a.v_inv);
      }
    }
  };
  // K row new_r0 of block new_ib lives in lanes with lane % 16 == new_r0; V row
  // new_r0 in lanes with lane / 16 == new_r0 / 4, register row new_r0 % 4.
  // With row-wise K (16-bit caches) row new_r0 sits in load new_r0 /
  // kRowsPerLoad, lanes with lane / kRowPieces == new_r0 % kRowsPerLoad.
  auto patch_new = [&](Chunk<T, D, 16, CB, F8>& f) {
    const bool krow = kRowK ? lane / S::kRowPieces == new_r0 % S::kRowsPerLoad : (lane & 15) == new_r0;
    const bool vrow = (lane >> 4) == new_r0 / 4;
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      if (i != new_ib) continue;
#pragma unroll
      for (int sg = 0; sg < S::kKSeg; ++sg) {
        if constexpr (kRowK) {
          if (sg == new_r0 / S::kRowsPerLoad) f.k[i][sg] = krow ? kn[0] : f.k[i][sg];
        } else {
          f.k[i][sg] = krow ? kn[sg] : f.k[i][sg];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r != new_r0 % 4) continue;
#pragma unroll
        for (int w = 0; w < S::kVDw; ++w) f.v[i][r][w] = vrow ? vn[w] : f.v[i][r][w];
      }
    }
  };

  // Output row of column c; the epilogue's split of a tile's outputs over the
  // threads (kTpc threads per column, kPer consecutive elements each).
  auto out_row = [&](int c) {
    const int tok = c / g;
    return (static_cast<int64_t>(q0) + tok0 + tok) * a.num_heads + kvh * g + (c - tok * g);
  };
  constexpr int kTpc = kMqWaves * kWave / kCols;
  constexpr int kPer = D / kTpc;
  static_assert(kPer >= 2 && kPer % 2 == 0 && kPer * kTpc == D, "epilogue split");
  // Suffix pass of the shared-prefix decode (16-column tiles of 16-bit
  // caches): the prefix part of this thread's outputs, and of its column's
  // weight, is read now, so that the epilogue does not wait for it.
  constexpr bool kPrefetchPrefix = NT == 1 && sizeof(T) == 2;
  float pre_o[kPrefetchPrefix ? kPer : 1];
  float pre_lse = -__builtin_inff();
  if constexpr (kPrefetchPrefix) {
    if (a.prefix_o != nullptr) {
      if (static_cast<int>(threadIdx.x) < ncols) pre_lse = a.prefix_lse[out_row(threadIdx.x)];
      const int c = threadIdx.x / kTpc;
      if (c < ncols) {
        const float* src = a.prefix_o + out_row(c) * D + (threadIdx.x % kTpc) * kPer;
#pragma unroll
        for (int e = 0; e < kPer; ++e) pre_o[e] = src[e];
      }
    }
  }

  u32x4_t q[NT][S::kQSeg];
  load_query_cols<T, D, CB, NT, F8>(a.query, q0 + tok0, a.num_heads, kvh * g, g, ncols, lane, q);

  MqState<T, D, CB, NT> st;
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    st.m[p] = -__builtin_inff();
    st.l[p] = 0.f;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) st.acc[p][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Register double buffer with unconditional steady-state loads and a peeled
  // tail, as in the decode kernel. For new tokens of one sequence only a
  // wave's last chunk can need a mask; in the shared-prefix pass columns may
  // stop anywhere, so every chunk checks. A decode launch (one new token per
  // sequence, whole contexts or partitions) reads every key once and streams
  // it with non-temporal loads; multi-query launches keep plain loads (the
  // keys of a sequence cut into several tiles are re-read from L2 by its other
  // tiles: the batch-256 step with a 1,024-token chunk ran 255 vs 238 us with
  // its one-tile sequences streamed), and so do both passes of the
  // shared-prefix decode (the suffix pass measured 55.5 vs 57.8 us per step on
  // the 70B-shaped workload).
  const bool stream_keys = a.query_start_loc == nullptr && a.prefix_keys == 0 && a.prefix_o == nullptr;
  // Chunk i of this wave with the mask applied or not (compile time). In a
  // decode or multi-query launch only a wave's last chunk can reach past some
  // column's limit, so the loop below runs the unmasked chunk everywhere else
  // (no selects) and the masked one last. In the shared-prefix pass a column
  // may stop anywhere when a context is shorter than the prefix; such tiles
  // (min_lim < key_end) mask every chunk.
  auto run_chunks = [&](auto stream_tag, auto all_masked_tag) {
    constexpr bool kStream = decltype(stream_tag)::value;
    constexpr bool kAllMasked = decltype(all_masked_tag)::value;
    Chunk<T, D, 16, CB, F8> fa, fb;
    auto load = [&](Chunk<T, D, 16, CB, F8>& f, int i) {
      load_chunk<T, D, 16, CB, F8, kStream, kRowK>(f, kc, vc, bt_row, blk_of(i), blk_last, a.num_blocks,
                                                   tok_stride, blk_stride, head_off, lane, last_rows, first_ids,
                                                   i == 0 && have_first);
    };
    auto compute = [&](Chunk<T, D, 16, CB, F8>& f, int i, auto mask_tag) {
      if constexpr (kRowK) k_rows_to_mfma<T, D, 16, CB, F8>(f, k_stage, lane);
      mq_chunk<T, D, CB, NT, F8, decltype(mask_tag)::value || kAllMasked>(st, f, q, a.scale_log2, tok_of(i), lim,
                                                                          key_end, lane);
    };
    if (mine > 0) load(fa, 0);
    // The write is folded only into decode launches, and those always stream
    // (stream_keys), so only the streaming loop quantizes.
    if constexpr (kStream) quantize_new();
    if (mine <= 0) return;
    int i = 0;
    for (; i + 2 < mine; i += 2) {
      load(fb, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(fa, i, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      load(fa, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(fb, i + 1, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
    if (i + 1 < mine) {
      load(fb, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(fa, i, std::false_type{});
      if constexpr (kFusedWrite) {
        if (patch_own) patch_new(fb);
      }
      compute(fb, i + 1, std::true_type{});
    } else {
      if constexpr (kFusedWrite) {
        if (patch_own) patch_new(fa);
      }
      compute(fa, i, std::true_type{});
    }
  };
  if (stream_keys)
    run_chunks(std::true_type{}, std::false_type{});
  else if (a.prefix_keys > 0 && min_lim < key_end)
    run_chunks(std::false_type{}, std::true_type{});
  else
    run_chunks(std::false_type{}, std::false_type{});
  if (kFusedWrite && own_new) {
    // The new token's slice to its slot (the lanes that hold it).
    typedef __attribute__((address_space(1))) char gwchar_t;
    const int64_t dst_off = (new_slot / kBlockTokens) * blk_stride + (new_slot % kBlockTokens) * tok_stride + head_off;
    gwchar_t* kdst = reinterpret_cast<gwchar_t*>(reinterpret_cast<uintptr_t>(kc + dst_off));
    gwchar_t* vdst = reinterpret_cast<gwchar_t*>(reinterpret_cast<uintptr_t>(vc + dst_off));
    if constexpr (kRowK) {
      if (lane < S::kRowPieces)
        *reinterpret_cast<__attribute__((address_space(1))) u32x4_t*>(
            kdst + ((lane - new_r0) & (S::kRowPieces - 1)) * 16) = kn[0];
    } else if ((lane & 15) == 0) {
#pragma unroll
      for (int sg = 0; sg < S::kKSeg; ++sg)
        *reinterpret_cast<__attribute__((address_space(1))) u32x4_t*>(kdst + sg * 64 + (lane >> 4) * 16) = kn[sg];
    }
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int w = 0; w < S::kVDw; ++w)
        reinterpret_cast<__attribute__((address_space(1))) uint32_t*>(vdst + (lane & 15) * (S::kVDw * 4))[w] = vn[w];
    }
  }

  // Every wave is done with its K staging area before s_acc takes the partials.
  if constexpr (kRowK) __syncthreads();
  // Wave partials to LDS: per column the running max and normaliser, and the
  // lane's D/4 output elements.
  const int j = lane >> 4;
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    const float l = rows_sum(st.l[p]);
    const int c = 16 * p + (lane & 15);
    if (lane < 16) {
      s_m[wave][c] = st.m[p];
      s_l[wave][c] = l;
    }
    // Columns past the tile's last (token, head) pair are never read back.
    if (c < ncols) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int t0 = 0; t0 < D / 16; t0 += 4)
          *reinterpret_cast<f32x4_t*>(&s_acc[wave][c][(D / 16) * (4 * j + rr) + t0]) =
              f32x4_t{st.acc[p][t0][rr], st.acc[p][t0 + 1][rr], st.acc[p][t0 + 2][rr], st.acc[p][t0 + 3][rr]};
    }
  }
  __syncthreads();

  // Merge weights per column, once: wave w's part weighs 2^(m_w - M), and
  // the normaliser is L = sum_w 2^(m_w - M) l_w. A prefix-pass result joins
  // as one more part: l = 1, acc = its output, m = its log-sum-exp in base 2.
  for (int c = threadIdx.x; c < ncols; c += kMqWaves * kWave) {
    float M = -__builtin_inff();
#pragma unroll
    for (int v = 0; v < kMqWaves; ++v) M = fmaxf(M, s_m[v][c]);
    float pm = -__builtin_inff();
    if (a.prefix_o != nullptr) pm = (kPrefetchPrefix ? pre_lse : a.prefix_lse[out_row(c)]) * kLog2e;
    M = fmaxf(M, pm);
    float L = 0.f;
    float w[kMqWaves + 1];
#pragma unroll
    for (int v = 0; v < kMqWaves; ++v) {
      w[v] = M == -__builtin_inff() ? 0.f : fast_exp2(s_m[v][c] - M);
      L = fmaf(w[v], s_l[v][c], L);
    }
    w[kMqWaves] = pm == -__builtin_inff() ? 0.f : fast_exp2(pm - M);
    L += w[kMqWaves];
#pragma unroll
    for (int v = 0; v <= kMqWaves; ++v) s_w[v][c] = w[v];
    s_L[c] = L;
    s_lse[c] = M == -__builtin_inff() ? -__builtin_inff() : (M + fast_log2(L)) * kLn2;
  }
  __syncthreads();

  // Each column's row: kTpc threads per column, each a contiguous run of kPer
  // elements (vector LDS reads and stores; the column's row, weights and
  // normaliser read once). out = (sum_w weight_w acc_w) / L times v_scale (0
  // for a column with no visible key).
  const int oc = threadIdx.x / kTpc;
  if (oc < ncols) {
    const int d0 = (threadIdx.x % kTpc) * kPer;
    const int64_t row = out_row(oc);
    float o[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) o[e] = 0.f;
    const float L = s_L[oc];
    if (L != 0.f) {
#pragma unroll
      for (int v = 0; v < kMqWaves; ++v) {
        const float wv = s_w[v][oc];
        const float* src = &s_acc[v][oc][d0];
#pragma unroll
        for (int e = 0; e < kPer; ++e) o[e] = fmaf(wv, src[e], o[e]);
      }
      if (a.prefix_o != nullptr) {
        const float wp = s_w[kMqWaves][oc];
        if (wp != 0.f) {
          const float* src = a.prefix_o + row * D + d0;
#pragma unroll
          for (int e = 0; e < kPer; ++e) o[e] = fmaf(wp, kPrefetchPrefix ? pre_o[e] : src[e], o[e]);
        }
      }
      // Divided, not multiplied by 1/L: a one-key context returns its V row
      // exactly.
#pragma unroll
      for (int e = 0; e < kPer; ++e) o[e] = o[e] / L * a.v_scale;
    }
    if (a.part_o != nullptr) {
      const int64_t orow = part >= 0 ? row * a.parts_stride + part : row;
      store_run<float, kPer>(a.part_o + orow * D + d0, o);
      if (d0 == 0) a.part_lse[orow] = s_lse[oc];
    } else {
      store_run<T, kPer>(static_cast<T*>(a.out) + row * D + d0, o);
      if (a.lse_out != nullptr && d0 == 0) a.lse_out[row] = s_lse[oc];
    }
  }
}

}  // namespace pa

// ------------------------------------------------------------------ host side
namespace {

using namespace pa;

typedef void (*MultiKernel)(MultiArgs);

template <typename T, int D, int NT, bool F8>
MultiKernel multi_kernel_for(int W) {
  constexpr int kElem = F8 ? 1 : static_cast<int>(sizeof(T));
  constexpr int kRegsPerBlock = D * kElem / 8;  // K + V dwords per lane
  constexpr int CB = (kRegsPerBlock <= 32 && NT == 1) ? 2 : 1;
  // 8-wave workgroups for 16-column tiles of 16-bit and FP8 caches; fp32
  // caches (the small workloads) and 32-column tiles (137 KB of LDS at 8
  // waves) keep 4.
  if constexpr (sizeof(T) == 2 && NT == 1) {
    if (W == 8) return paged_multi_query_kernel<T, D, CB, NT, F8, 8>;
  }
  return paged_multi_query_kernel<T, D, CB, NT, F8, 4>;
}

template <typename T, bool F8>
MultiKernel pick_multi_t(int D, int NT, int W) {
  if (D == 128) return NT == 1 ? multi_kernel_for<T, 128, 1, F8>(W) : multi_kernel_for<T, 128, 2, F8>(W);
  return NT == 1 ? multi_kernel_for<T, 64, 1, F8>(W) : multi_kernel_for<T, 64, 2, F8>(W);
}

// fp32 caches with 128-element heads keep 16-column tiles (32 would spill).
// Returns the kernel and sets W to the waves per workgroup it was built for.
MultiKernel pick_multi(int dtype, int D, int NT, bool fp8_cache, int& W) {
  if ((dtype == PA_DTYPE_F32 && !fp8_cache) || NT != 1) W = 4;
  if (fp8_cache) return pick_multi_t<bf16_t, true>(D, NT, W);
  if (dtype == PA_DTYPE_BF16) return pick_multi_t<bf16_t, false>(D, NT, W);
  if (D == 128) return multi_kernel_for<float, 128, 1, false>(W);
  return NT == 1 ? multi_kernel_for<float, 64, 1, false>(W) : multi_kernel_for<float, 64, 2, false>(W);
}

// Waves per workgroup for a launch of `jobs` workgroups: 8 when every
// resident 4-wave workgroup (two per CU) would get at most one job, else 4;
// PA_OPT_TILE_WAVES forces one. (pick_multi keeps 4 where no 8-wave kernel is
// built.)
int pick_waves(int64_t jobs) {
  const int v = option_value(PA_OPT_TILE_WAVES);
  if (v == 4 || v == 8) return v;
  return jobs <= 2 * static_cast<int64_t>(device_cus()) ? 8 : 4;
}

int max_tiles(int dtype, int D) { return (dtype == PA_DTYPE_F32 && D == 128) ? 1 : 2; }

inline bool aligned16_mq(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Tiles of 32 columns when the step averages more new tokens per sequence
// than one 16-column tile holds: prompt chunks and longer speculative runs
// then read each key once per 32 columns instead of per 16
// (PA_OPT_TILE_COLUMNS forces a width).
int pick_tiles(int num_tokens, int num_seqs, int group) {
  const int v = option_value(PA_OPT_TILE_COLUMNS);
  if (v == 16 || v == 32) return v / 16;
  return static_cast<int64_t>(num_tokens) * group > static_cast<int64_t>(num_seqs) * 16 ? 2 : 1;
}

// Shared host checks of the multi-query entry points.
int check_multi(const void* out, const void* query, const void* key_cache, const void* value_cache,
                const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                int32_t num_seqs, int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                int64_t num_blocks, int32_t block_size, float scale, int32_t dtype) {
  if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0)
    return PA_ERR_INVALID_ARG;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (num_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != kBlockTokens) return PA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || scale == __builtin_inff()) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (!aligned16_mq(out) || !aligned16_mq(query) || !aligned16_mq(key_cache) || !aligned16_mq(value_cache))
    return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_blocks_per_seq) * kBlockTokens > INT32_MAX) return PA_ERR_INVALID_ARG;
  // A token row (all kv heads) must stay under 2^24 bytes (24-bit row offsets).
  if (static_cast<int64_t>(num_kv_heads) * head_size * 4 >= (int64_t{1} << 24)) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// One multi-query launch. query_start_loc == nullptr: one new token per
// sequence (query row i is sequence i's), 16-column tiles.
int launch_multi(void* out, const void* query, const void* key_cache, const void* value_cache,
                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                 const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                 int32_t num_kv_heads, int32_t head_size, int64_t num_blocks, float scale_log2, float v_scale,
                 int32_t dtype, bool fp8_cache, float* lse_out, const int32_t* seq_order, hipStream_t stream,
                 int32_t skip_blocks = 0, const float* prefix_o = nullptr, const float* prefix_lse = nullptr,
                 const void* new_key = nullptr, const void* new_value = nullptr,
                 const int64_t* slot_mapping = nullptr, float write_k_scale = 1.0f,
                 float write_v_scale = 1.0f) {
  const int g = num_heads / num_kv_heads;
  int NT = query_start_loc == nullptr ? 1 : pick_tiles(num_tokens, num_seqs, g);
  NT = NT < max_tiles(dtype, head_size) ? NT : max_tiles(dtype, head_size);
  MultiArgs a{};
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.seq_order = query_start_loc == nullptr ? seq_order : nullptr;
  a.out = out;
  a.lse_out = lse_out;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = g;
  a.tile_tokens = 16 * NT / g;
  const int64_t slots =
      query_start_loc == nullptr ? num_seqs : static_cast<int64_t>(num_tokens) / a.tile_tokens + num_seqs;
  const int64_t grid = (slots + 7) / 8 * 8 * num_kv_heads;
  if (grid > INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
  // Jobs that do work: about ceil(mean new tokens per sequence / tile) tiles
  // per sequence (the slot bound counts one spare slot per sequence).
  const int64_t per_seq = query_start_loc == nullptr ? 1
      : (static_cast<int64_t>(num_tokens) + static_cast<int64_t>(num_seqs) * a.tile_tokens - 1) /
            (static_cast<int64_t>(num_seqs) * a.tile_tokens);
  int W = pick_waves(static_cast<int64_t>(num_seqs) * per_seq * num_kv_heads);
  MultiKernel k = pick_multi(dtype, head_size, NT, fp8_cache, W);
  a.num_slots = static_cast<int32_t>(slots);
  a.scale_log2 = scale_log2;
  a.v_scale = v_scale;
  a.skip_blocks = skip_blocks;
  a.prefix_o = prefix_o;
  a.prefix_lse = prefix_lse;
  a.new_key = new_key;
  a.new_value = new_value;
  a.slot_mapping = slot_mapping;
  a.k_scale = write_k_scale;
  a.v_scale_write = write_v_scale;
  a.scales_pow2 = exact_reciprocal(write_k_scale, &a.k_inv) && exact_reciprocal(write_v_scale, &a.v_inv);
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(grid)), dim3(W * kWave), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

int pa::launch_prefix_pass(const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                           int64_t num_blocks, int32_t prefix_blocks, float scale, int32_t dtype, float* part_o,
                           float* part_lse, hipStream_t stream) {
  const int g = num_heads / num_kv_heads;
  int NT = pick_tiles(num_seqs, 1, g);
  NT = NT < max_tiles(dtype, head_size) ? NT : max_tiles(dtype, head_size);
  MultiArgs a{};
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = 1;
  a.num_tokens = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = g;
  a.tile_tokens = 16 * NT / g;
  const int64_t slots = (static_cast<int64_t>(num_seqs) + a.tile_tokens - 1) / a.tile_tokens;
  const int64_t grid = (slots + 7) / 8 * 8 * num_kv_heads;
  if (grid > INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
  int W = pick_waves(slots * num_kv_heads);
  MultiKernel k = pick_multi(dtype, head_size, NT, false, W);
  a.num_slots = static_cast<int32_t>(slots);
  a.scale_log2 = scale * kLog2e;
  a.v_scale = 1.0f;
  a.prefix_keys = prefix_blocks * kBlockTokens;
  a.part_o = part_o;
  a.part_lse = part_lse;
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(grid)), dim3(W * kWave), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa::device_cus() {
  // Cached per device (every caller on a device stores the same value).
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const bool slot = dev >= 0 && dev < 64;
  if (slot) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  if (slot) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int pa::launch_split_tiles(const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                           int64_t num_blocks, float scale, int32_t dtype, int32_t part_blocks, int32_t num_parts,
                           int32_t part_cap, int32_t parts_stride, float* o_parts, float* lse_parts,
                           hipStream_t stream) {
  const int g = num_heads / num_kv_heads;
  if (g > 16 || part_blocks <= 0 || num_parts <= 0 || parts_stride < num_parts) return PA_ERR_UNSUPPORTED;
  MultiArgs a{};
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_tokens = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = g;
  a.tile_tokens = 16 / g;
  const int64_t slots = static_cast<int64_t>(num_seqs) * num_parts;
  const int64_t grid = (slots + 7) / 8 * 8 * num_kv_heads;
  if (grid > INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
  int W = pick_waves(slots * num_kv_heads);
  MultiKernel k = pick_multi(dtype, head_size, 1, false, W);
  a.num_slots = static_cast<int32_t>(slots);
  a.scale_log2 = scale * kLog2e;
  a.v_scale = 1.0f;
  a.part_o = o_parts;
  a.part_lse = lse_parts;
  a.part_blocks = part_blocks;
  a.num_parts = num_parts;
  a.parts_stride = parts_stride;
  a.part_cap = part_cap;
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(grid)), dim3(W * kWave), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

namespace {

// Workspace of pa_multi_query_split: float32 partials [num_tokens, num_heads,
// slots, head_size] then float32 log-sum-exps [num_tokens, num_heads, slots],
// each 256-byte aligned; slots = ceil(max_context_len / partition_size).
struct MqSplitLayout {
  int64_t slots = 0;
  size_t lse_off = 0, total = 0;
};

bool mq_split_layout(int64_t num_tokens, int64_t num_heads, int64_t head_size, int64_t max_context_len,
                     int64_t partition_size, MqSplitLayout& L) {
  if (num_tokens < 0 || num_heads <= 0 || head_size <= 0 || max_context_len < 0 || partition_size <= 0) return false;
  L.slots = (max_context_len + partition_size - 1) / partition_size;
  if (L.slots < 1) L.slots = 1;
  const size_t rows = static_cast<size_t>(num_tokens) * static_cast<size_t>(num_heads) * static_cast<size_t>(L.slots);
  auto a256 = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  L.lse_off = a256(rows * static_cast<size_t>(head_size) * sizeof(float));
  L.total = L.lse_off + a256(rows * sizeof(float));
  return L.slots <= INT32_MAX;
}

}  // namespace

extern "C" size_t pa_multi_query_split_workspace_bytes(int32_t num_tokens, int32_t num_heads, int32_t head_size,
                                                       int32_t max_context_len, int32_t partition_size) {
  MqSplitLayout L;
  return mq_split_layout(num_tokens, num_heads, head_size, max_context_len, partition_size, L) ? L.total : 0;
}

// One round of the plain launch has at most tile_slots * H_kv workgroups,
// each over a whole context. When that is fewer than the compute units, the
// contexts are cut so that about three rounds of two resident workgroups per
// compute unit remain (as for the decode partition cut), in multiples of
// 256 tokens so that each partition still streams long enough.
extern "C" int32_t pa_multi_query_split_partition_size(int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                                       int32_t num_kv_heads, int32_t head_size, int32_t dtype,
                                                       int32_t max_context_len) {
  if (num_seqs <= 0 || num_tokens <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      max_context_len <= 0 || (head_size != 64 && head_size != 128))
    return 0;
  const int g = num_heads / num_kv_heads;
  if (g > 16) return 0;
  int NT = pick_tiles(num_tokens, num_seqs, g);
  NT = NT < max_tiles(dtype, head_size) ? NT : max_tiles(dtype, head_size);
  const int64_t tile_tokens = 16 * NT / g;
  const int64_t jobs = (static_cast<int64_t>(num_tokens) / tile_tokens + num_seqs) * num_kv_heads;
  const int64_t cus = device_cus();
  if (jobs >= cus) return 0;
  const int64_t parts = (3 * 2 * cus + jobs - 1) / jobs;
  int64_t P = (static_cast<int64_t>(max_context_len) + parts - 1) / parts;
  P = (P + 255) / 256 * 256;
  return P >= max_context_len ? 0 : static_cast<int32_t>(P);
}

extern "C" int pa_multi_query_split(void* out, const void* query, const void* key_cache, const void* value_cache,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, const int32_t* query_start_loc, int32_t num_seqs,
                                    int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                    int64_t num_blocks, int32_t block_size, float scale, int32_t dtype,
                                    int32_t max_context_len, int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, float* lse_out, void* stream) {
  int st = check_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_tokens, num_heads, num_kv_heads, head_size, num_blocks, block_size, scale, dtype);
  if (st != PA_OK) return st;
  if (partition_size <= 0 || partition_size % kBlockTokens != 0 || max_context_len < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!query_start_loc) return PA_ERR_INVALID_ARG;
  MqSplitLayout L;
  if (!mq_split_layout(num_tokens, num_heads, head_size, max_context_len, partition_size, L))
    return PA_ERR_UNSUPPORTED;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_INVALID_ARG;
  if (workspace_bytes < L.total) return PA_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  float* o_parts = static_cast<float*>(workspace);
  float* lse_parts = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.lse_off);
  const int num_parts = static_cast<int>(L.slots);
  const int64_t cap = min(static_cast<int64_t>(max_blocks_per_seq) * kBlockTokens,
                          static_cast<int64_t>(partition_size) * num_parts);
  if (cap > INT32_MAX) return PA_ERR_UNSUPPORTED;

  const int g = num_heads / num_kv_heads;
  int NT = pick_tiles(num_tokens, num_seqs, g);
  NT = NT < max_tiles(dtype, head_size) ? NT : max_tiles(dtype, head_size);
  MultiArgs a{};
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = g;
  a.tile_tokens = 16 * NT / g;
  const int64_t tile_slots = static_cast<int64_t>(num_tokens) / a.tile_tokens + num_seqs;
  const int64_t slots = tile_slots * num_parts;
  const int64_t grid = (slots + 7) / 8 * 8 * num_kv_heads;
  if (tile_slots > INT32_MAX || grid > INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
  const int64_t per_seq = (static_cast<int64_t>(num_tokens) + static_cast<int64_t>(num_seqs) * a.tile_tokens - 1) /
                          (static_cast<int64_t>(num_seqs) * a.tile_tokens);
  int W = pick_waves(static_cast<int64_t>(num_seqs) * per_seq * num_parts * num_kv_heads);
  MultiKernel k = pick_multi(dtype, head_size, NT, false, W);
  a.num_slots = static_cast<int32_t>(slots);
  a.tile_slots = static_cast<int32_t>(tile_slots);
  a.scale_log2 = scale * kLog2e;
  a.v_scale = 1.0f;
  a.part_o = o_parts;
  a.part_lse = lse_parts;
  a.part_blocks = partition_size / kBlockTokens;
  a.num_parts = num_parts;
  a.parts_stride = num_parts;
  a.part_cap = static_cast<int32_t>(cap);
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(grid)), dim3(W * kWave), 0, s, a);
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  return launch_merge_mq_parts(out, lse_out, o_parts, lse_parts, query_start_loc, context_lens, num_seqs,
                               num_tokens, num_heads, static_cast<int>(cap), max_blocks_per_seq, partition_size,
                               num_parts, head_size, dtype, s);
}

int pa::launch_decode_multi(void* out, const void* query, const void* key_cache, const void* value_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                            int64_t num_blocks, float scale_log2, float v_scale, int32_t dtype, bool fp8_cache,
                            float* lse_out, const int32_t* seq_order, int32_t skip_blocks, const float* prefix_o,
                            const float* prefix_lse, hipStream_t stream) {
  return launch_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens, nullptr,
                      num_seqs, num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale_log2, v_scale,
                      dtype, fp8_cache, lse_out, seq_order, stream, skip_blocks, prefix_o, prefix_lse);
}

extern "C" int pa_multi_query(void* out, const void* query, const void* key_cache, const void* value_cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                              const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int64_t num_blocks,
                              int32_t block_size, float scale, int32_t dtype, float* lse_out, void* stream) {
  int st = check_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_tokens, num_heads, num_kv_heads, head_size, num_blocks, block_size, scale, dtype);
  if (st != PA_OK || num_seqs == 0 || num_tokens == 0) return st;
  if (!query_start_loc) return PA_ERR_INVALID_ARG;
  return launch_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                      query_start_loc, num_seqs, num_tokens, num_heads, num_kv_heads, head_size, num_blocks,
                      scale * kLog2e, 1.0f, dtype, false, lse_out, nullptr, static_cast<hipStream_t>(stream));
}

extern "C" int pa_multi_query_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, const int32_t* query_start_loc, int32_t num_seqs,
                                  int32_t num_tokens, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                  int64_t num_blocks, int32_t block_size, float scale, float k_scale, float v_scale,
                                  int32_t dtype, float* lse_out, void* stream) {
  int st = check_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_tokens, num_heads, num_kv_heads, head_size, num_blocks, block_size, scale, dtype);
  if (st != PA_OK || num_seqs == 0 || num_tokens == 0) return st;
  if (dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale == __builtin_inff() || v_scale == __builtin_inff())
    return PA_ERR_INVALID_ARG;
  if (!query_start_loc) return PA_ERR_INVALID_ARG;
  return launch_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                      query_start_loc, num_seqs, num_tokens, num_heads, num_kv_heads, head_size, num_blocks,
                      scale * k_scale * kLog2e, v_scale, dtype, true, lse_out, nullptr,
                      static_cast<hipStream_t>(stream));
}

extern "C" int pa_reshape_and_decode(void* out, const void* query, const void* key, const void* value,
                                     const int64_t* slot_mapping, void* key_cache, void* value_cache,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                     int32_t num_kv_heads, int32_t head_size, int64_t num_blocks, int32_t block_size,
                                     float scale, int32_t dtype, float* lse_out, const int32_t* seq_order,
                                     void* stream) {
  int st = check_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_seqs, num_heads, num_kv_heads, head_size, num_blocks, block_size, scale, dtype);
  if (st != PA_OK || num_seqs == 0) return st;
  if (!key || !value || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned16_mq(key) || !aligned16_mq(value)) return PA_ERR_INVALID_ARG;
  return launch_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens, nullptr,
                      num_seqs, num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale * kLog2e, 1.0f,
                      dtype, false, lse_out, seq_order, static_cast<hipStream_t>(stream), 0, nullptr, nullptr, key,
                      value, slot_mapping);
}

extern "C" int pa_reshape_and_decode_fp8(void* out, const void* query, const void* key, const void* value,
                                         const int64_t* slot_mapping, uint8_t* key_cache, uint8_t* value_cache,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                         int32_t num_kv_heads, int32_t head_size, int64_t num_blocks,
                                         int32_t block_size, float scale, float k_scale, float v_scale, int32_t dtype,
                                         float* lse_out, const int32_t* seq_order, void* stream) {
  int st = check_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_seqs, num_heads, num_kv_heads, head_size, num_blocks, block_size, scale, dtype);
  if (st != PA_OK || num_seqs == 0) return st;
  if (dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale == __builtin_inff() || v_scale == __builtin_inff())
    return PA_ERR_INVALID_ARG;
  if (!key || !value || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned16_mq(key) || !aligned16_mq(value)) return PA_ERR_INVALID_ARG;
  return launch_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens, nullptr,
                      num_seqs, num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale * k_scale * kLog2e,
                      v_scale, dtype, true, lse_out, seq_order, static_cast<hipStream_t>(stream), 0, nullptr, nullptr,
                      key, value, slot_mapping, k_scale, v_scale);
}
