// Paged decode attention for gfx950: the decode entry points (pa_decode,
// pa_decode_fp8, pa_decode_prefix, pa_decode_split, pa_merge_partitions), the
// pieces cut of the split path, and the log-sum-exp merges.
//
// What is computed (llm-stack-book 7.3 "vLLM: Architecture, PagedAttention &
// Internals", sections "PagedAttention in one paragraph" and "The forward step
// in detail"): for each sequence and query head, ordinary attention of the one
// new query over the sequence's whole context, with K/V rows found through the
// block table instead of in one contiguous tensor. The softmax runs online over
// streamed blocks (stanleyjacob.dev "vLLM", Part IV "Stage 6: The forward
// pass"); a context split into pieces is recombined exactly with log-sum-exp
// weights (Part V, "The attention backend dispatch layer": tiling plus online
// softmax).
//
// The one-pass decode runs on the tile kernel of multi_query.hip (one new
// token per sequence). This file holds the pieces kernel of pa_decode_split
// (persistent workgroups over an even cut of all blocks, one wave per kv head):
//  * A wave streams chunks of CB consecutive 16-token blocks. All g = H_q/H_kv
//    query heads of the kv head share every K/V tile the wave loads.
//  * Scores: one 16x16 MFMA tile per block, A = K rows (M = the block's 16
//    tokens), B = the group's query rows (N = up to 16 heads), contracted over
//    head_size. Each lane loads its K operand straight from HBM: token
//    (lane % 16), 16-byte pieces at byte offset s*64 + (lane/16)*16 of the row,
//    so every load instruction reads one aligned 64-byte segment of each of the
//    16 rows of the tile. The query fragment uses the same d ordering.
//  * The MFMA result leaves lane l with the scores of tokens 4*(l/16)+r,
//    r = 0..3, for head l % 16. The V load uses exactly those tokens: lane l
//    reads head_size/16 contiguous elements (d = (l%16)*head_size/16 ...) of
//    the 4 rows, so each load instruction covers 4 whole rows, and the
//    probabilities a lane needs come from its own 16-lane row by DPP broadcast.
//  * P*V runs on the VALU in fp32.
//  * Online softmax per chunk with base-2 exponentials (scale*log2(e) folded
//    into the scores); the chunk maximum is reduced across the 4 row groups.
// Reduction order depends only on logical token positions and CB, never on
// physical block ids, so results do not change when blocks move or are shared.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_tiles.h"

namespace pa {

template <typename T, int D, int G, int CB>
struct WaveState {
  using S = DecodeShape<T, D, G, CB>;
  float m;                  // running max (base-2 scaled) for head lane%16
  float l;                  // partial sum of weights, this lane's tokens
  float acc[G][S::kVec];    // partial P*V, this lane's tokens and d range
};

// Online-softmax update and P*V for one chunk whose scores are in s.
template <typename T, int D, int G, int CB, bool F8 = false>
__device__ __forceinline__ void softmax_pv_chunk(WaveState<T, D, G, CB>& st, const Chunk<T, D, G, CB, F8>& f,
                                                 float (&s)[CB][4], int tok0, int t_end, bool mask, int lane) {
  using S = DecodeShape<T, D, G, CB, F8>;
  const int rg = lane >> 4;
  // The chunk that straddles the end of the context: positions >= t_end get
  // weight exactly 0 and their V rows (stale or poisoned) are replaced by 0.
  uint32_t vz[CB][4][S::kVDw];
#pragma unroll
  for (int i = 0; i < CB; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int w = 0; w < S::kVDw; ++w) vz[i][r][w] = f.v[i][r][w];
  if (mask) {
#pragma unroll
    for (int i = 0; i < CB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool valid = tok0 + i * 16 + 4 * rg + r < t_end;
        s[i][r] = valid ? s[i][r] : -__builtin_inff();
#pragma unroll
        for (int w = 0; w < S::kVDw; ++w) vz[i][r][w] = valid ? vz[i][r][w] : 0u;
      }
  }
  float mx = s[0][0];
#pragma unroll
  for (int i = 0; i < CB; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[i][r]);
  mx = rows_max(mx);
  const float m_new = fmaxf(st.m, mx);
  const float alpha = fast_exp2(st.m - m_new);
  st.m = m_new;
  float p[CB][4];
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < CB; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[i][r] = fast_exp2(s[i][r] - m_new);
      psum += p[i][r];
    }
  st.l = st.l * alpha + psum;

  static_for<G>([&](auto hc) {
    constexpr int h = decltype(hc)::value;
    const float a = row_bcast<h>(alpha);
#pragma unroll
    for (int e = 0; e < S::kVec; ++e) st.acc[h][e] *= a;
  });
#pragma unroll
  for (int i = 0; i < CB; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float vf[S::kVec];
      if constexpr (F8) {
#pragma unroll
        for (int w = 0; w < S::kVDw; ++w) {
          fp8x2_to_f32<false>(vz[i][r][w], vf[4 * w], vf[4 * w + 1]);
          fp8x2_to_f32<true>(vz[i][r][w], vf[4 * w + 2], vf[4 * w + 3]);
        }
      } else if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int w = 0; w < S::kVDw; ++w) {
          vf[2 * w] = bf16_lo(vz[i][r][w]);
          vf[2 * w + 1] = bf16_hi(vz[i][r][w]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < S::kVDw; ++w) vf[w] = as_float(vz[i][r][w]);
      }
      const float pr = p[i][r];
      static_for<G>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const float ph = row_bcast<h>(pr);
#pragma unroll
        for (int e = 0; e < S::kVec; ++e) st.acc[h][e] = fmaf(ph, vf[e], st.acc[h][e]);
      });
    }
}

template <typename T, int D, int G, int CB, bool F8 = false>
__device__ __forceinline__ void load_query(const void* query, int seq, int num_heads, int head0, int g, int lane,
                                           u32x4_t (&q)[DecodeShape<T, D, G, CB, F8>::kQSeg]) {
  using S = DecodeShape<T, D, G, CB, F8>;
  constexpr int kQBytes = static_cast<int>(sizeof(T));
  const int hq = lane & 15;
  const int j = lane >> 4;
  const gchar_t* qb = uniform_ptr(static_cast<const char*>(query) +
                                  (static_cast<int64_t>(seq) * num_heads + head0) * D * kQBytes);
  const uint32_t qoff = (hq < g ? hq : 0) * (D * kQBytes);
#pragma unroll
  for (int sg = 0; sg < S::kQSeg; ++sg) {
    // Same d order as the K operand: for bf16 caches k-step sg holds
    // d = 32 sg + 8 j + e; for FP8 caches (16 codes per lane per load)
    // d = 64 (sg / 2) + 16 j + 8 (sg % 2) + e.
    const uint32_t off = F8 ? 128 * (sg / 2) + 32 * j + 16 * (sg % 2) : sg * 64 + j * 16;
    u32x4_t v = gload16(qb + off + qoff);
    q[sg] = hq < g ? v : u32x4_t{0u, 0u, 0u, 0u};
  }
}

// ------------------------------------------------------------------ partitioned path
// Persistent workgroups over an exactly balanced split of the work. A
// workgroup has one wave per kv head of a head group (up to 8 kv heads); its
// waves walk the same blocks at the same time, each computing its own kv head,
// so a CU reads whole token rows of every block it touches (2 KiB for 8 kv
// heads of 128 bf16). The blocks of all sequences are laid end to end, per
// head group, and workgroup r of R takes the contiguous range
// [r*T/R, (r+1)*T/R) of the T blocks: every workgroup reads the same amount
// (to within one block). Where a range cuts a sequence, each piece's
// normalised output and log-sum-exp go to a workspace slot and a merge kernel
// combines them; a sequence that one range covers whole is written straight to
// the output. R is capped so that every range holds at least partition_size
// tokens, which bounds the pieces of a sequence by ceil(n / partition_size) + 1.
// Each wave streams its chunks back to back with the next chunk (possibly of
// the next sequence) in flight; no LDS traffic or barriers inside the loop.
constexpr int kMaxHeadsPerGroup = 8;

struct SplitArgs {
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* lse_out;
  float* o_parts;     // [S, H_q, slots, D]
  float* lse_parts;   // [S, H_q, slots]
  int64_t* header;    // [0] T, [1] R; followed by int32 prefix of blocks per sequence [S + 1]
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t heads_per_group;  // kv heads per workgroup (= waves), <= 8
  int32_t num_groups;       // ceil(num_kv_heads / heads_per_group)
  int32_t part_tokens;      // minimum piece length, multiple of 16
  int32_t slots;            // ceil(max_context_len / part_tokens) + 1
  float scale_log2;
};

// Tokens of a sequence the partitioned path covers: clamped to the block
// table and to what the workspace slots can hold.
__device__ __forceinline__ int split_tokens(const int32_t* context_lens, int seq, int max_blocks, int part_tokens,
                                            int slots) {
  const int n = context_lens[seq];
  const int64_t cap = min(static_cast<int64_t>(max_blocks) * kBlockTokens,
                          static_cast<int64_t>(part_tokens) * (slots - 1));
  return n < 0 ? 0 : static_cast<int>(n > cap ? cap : n);
}

// Range holding flattened block x when T blocks are split into R ranges.
__device__ __forceinline__ int64_t range_of(int64_t x, int64_t T, int64_t R) { return (x * R + R - 1) / T; }

struct PieceCursor {
  int64_t x;      // flattened index of the piece's first block; -1 when done
  int64_t x_end;  // end of this workgroup's range
  int seq;
  int kvh;        // this wave's kv head (head group * heads_per_group + wave)
  int nb;         // blocks of the sequence
  int b_lo, b_hi; // piece = blocks [b_lo, b_hi) of the sequence
  int t_end;      // exclusive end position of the piece
  int nchunk, c;
  int slot;       // partial slot of this piece, -1 when the piece is the whole sequence
};

template <int CB>
__device__ __forceinline__ void cursor_set_piece(PieceCursor& u, const SplitArgs& a, const int* s_pre, int64_t T,
                                                 int64_t R, int wave) {
  if (u.x >= u.x_end) { u.x = -1; return; }
  const int64_t Tseq = __builtin_amdgcn_readfirstlane(s_pre[a.num_seqs]);
  const int gi = static_cast<int>(u.x / Tseq);
  const int64_t xs = u.x - static_cast<int64_t>(gi) * Tseq;
  int lo = 0, hi = a.num_seqs;  // largest seq with s_pre[seq] <= xs
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (__builtin_amdgcn_readfirstlane(s_pre[mid]) <= xs) lo = mid; else hi = mid;
  }
  u.seq = __builtin_amdgcn_readfirstlane(lo);
  const int pre = __builtin_amdgcn_readfirstlane(s_pre[u.seq]);
  u.nb = __builtin_amdgcn_readfirstlane(s_pre[u.seq + 1]) - pre;
  u.kvh = gi * a.heads_per_group + wave;
  u.b_lo = static_cast<int>(xs - pre);
  u.b_hi = static_cast<int>(min(static_cast<int64_t>(u.nb), u.b_lo + (u.x_end - u.x)));
  const int n = __builtin_amdgcn_readfirstlane(
      split_tokens(a.context_lens, u.seq, a.max_blocks, a.part_tokens, a.slots));
  u.t_end = min(n, u.b_hi * kBlockTokens);
  u.nchunk = (u.b_hi - u.b_lo + CB - 1) / CB;
  u.c = 0;
  if (u.b_lo == 0 && u.b_hi == u.nb) {
    u.slot = -1;
  } else {
    u.slot = static_cast<int>(range_of(u.x, T, R) - range_of(u.x - u.b_lo, T, R));
  }
}

template <int CB>
__device__ __forceinline__ void cursor_next(PieceCursor& u, const SplitArgs& a, const int* s_pre, int64_t T,
                                            int64_t R, int wave) {
  if (++u.c < u.nchunk) return;
  u.x += u.b_hi - u.b_lo;
  cursor_set_piece<CB>(u, a, s_pre, T, R, wave);
}

// Close a piece: sum over row groups, normalise, write the partial or the
// final output. After the reduction every row group holds the totals, so row
// group rg writes heads h with h % 4 == rg.
template <typename T, int D, int G, int CB>
__device__ __forceinline__ void finish_piece(WaveState<T, D, G, CB>& st, const SplitArgs& a, const PieceCursor& u,
                                             int lane) {
  using S = DecodeShape<T, D, G, CB>;
  const int head0 = u.kvh * a.group;
  const float l = rows_sum(st.l);
  const float lse_col = (st.m + fast_log2(l)) * kLn2;  // head lane % 16
  const int rg = lane >> 4;
  const int c = lane & 15;
  const bool whole = u.slot < 0;
  const bool slot_ok = u.slot < a.slots;  // always true by construction; guards the writes
  static_for<G>([&](auto hc) {
    constexpr int h = decltype(hc)::value;
    const float inv = 1.f / row_bcast<h>(l);
    float o[S::kVec];
#pragma unroll
    for (int e = 0; e < S::kVec; ++e) o[e] = rows_sum(st.acc[h][e]) * inv;
    if ((h & 3) == rg && h < a.group) {
      const int64_t row = static_cast<int64_t>(u.seq) * a.num_heads + head0 + h;
      if (whole) {
        T* dst = static_cast<T*>(a.out) + row * D + c * S::kVec;
#pragma unroll
        for (int e = 0; e < S::kVec; ++e) store_elem<T>(dst + e, o[e]);
      } else if (slot_ok) {
        float* dst = a.o_parts + (row * a.slots + u.slot) * D + c * S::kVec;
#pragma unroll
        for (int e = 0; e < S::kVec; e += 4)
          *reinterpret_cast<f32x4_t*>(dst + e) = f32x4_t{o[e], o[e + 1], o[e + 2], o[e + 3]};
      }
    }
  });
  if (rg == 0 && c < a.group) {
    const int64_t row = static_cast<int64_t>(u.seq) * a.num_heads + head0 + c;
    if (whole) {
      if (a.lse_out != nullptr) a.lse_out[row] = lse_col;
    } else if (slot_ok) {
      a.lse_parts[row * a.slots + u.slot] = lse_col;
    }
  }
  st.m = -__builtin_inff();
  st.l = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < S::kVec; ++e) st.acc[h][e] = 0.f;
}

template <typename T, int D, int G, int CB>
__global__ __launch_bounds__(64 * kMaxHeadsPerGroup, 1) void paged_decode_split_kernel(SplitArgs a) {
  using S = DecodeShape<T, D, G, CB>;
  extern __shared__ int s_pre[];  // [num_seqs + 1] blocks per sequence, exclusive prefix
  __shared__ int s_run[64 * kMaxHeadsPerGroup];
  const int lane = threadIdx.x & 63;
  // Wave-uniform by construction; readfirstlane lets the compiler keep all
  // per-wave indexing (pieces, block ids, base addresses) in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Prefix sum of blocks per sequence: thread t sums a contiguous run of
  // sequences, the run totals are scanned in LDS.
  {
    const int per = (a.num_seqs + blockDim.x - 1) / blockDim.x;
    const int s0 = threadIdx.x * per;
    const int s1 = min(a.num_seqs, s0 + per);
    int run = 0;
    for (int i = s0; i < s1; ++i) {
      const int n = split_tokens(a.context_lens, i, a.max_blocks, a.part_tokens, a.slots);
      run += (n + kBlockTokens - 1) / kBlockTokens;
    }
    s_run[threadIdx.x] = run;
    __syncthreads();
    for (int off = 1; off < static_cast<int>(blockDim.x); off <<= 1) {
      const int v = static_cast<int>(threadIdx.x) >= off ? s_run[threadIdx.x - off] : 0;
      __syncthreads();
      s_run[threadIdx.x] += v;
      __syncthreads();
    }
    int base = s_run[threadIdx.x] - run;
    for (int i = s0; i < s1; ++i) {
      s_pre[i] = base;
      const int n = split_tokens(a.context_lens, i, a.max_blocks, a.part_tokens, a.slots);
      base += (n + kBlockTokens - 1) / kBlockTokens;
    }
    if (threadIdx.x == blockDim.x - 1) s_pre[a.num_seqs] = s_run[threadIdx.x];
    __syncthreads();
  }

  const int64_t nblk = static_cast<int64_t>(a.num_groups) * __builtin_amdgcn_readfirstlane(s_pre[a.num_seqs]);
  int64_t R = min(static_cast<int64_t>(gridDim.x), nblk / (a.part_tokens / kBlockTokens));
  if (R < 1) R = 1;
  if (blockIdx.x == 0) {
    // Layout of the pieces, for the merge kernel.
    if (threadIdx.x == 0) {
      a.header[0] = nblk;
      a.header[1] = R;
    }
    int* pre_out = reinterpret_cast<int*>(a.header + 2);
    for (int i = threadIdx.x; i <= a.num_seqs; i += blockDim.x) pre_out[i] = s_pre[i];
  }
  const int64_t r = blockIdx.x;
  if (nblk == 0 || r >= R) return;

  PieceCursor cur;
  cur.x = r * nblk / R;
  cur.x_end = (r + 1) * nblk / R;
  cursor_set_piece<CB>(cur, a, s_pre, nblk, R, wave);
  if (cur.x < 0) return;

  const int g = a.group;
  const uint32_t tok_stride = static_cast<uint32_t>(a.num_kv_heads) * D * S::kElemBytes;
  const int64_t blk_stride = static_cast<int64_t>(tok_stride) * kBlockTokens;
  const char* kc = static_cast<const char*>(a.key_cache);
  const char* vc = static_cast<const char*>(a.value_cache);
  auto bt_row = [&](int seq) { return a.block_tables + static_cast<int64_t>(seq) * a.max_blocks; };
  // An idle wave (kv head past the last) reads kv head 0 and writes nothing.
  auto live = [&](const PieceCursor& u) { return u.kvh < a.num_kv_heads; };
  auto head_off = [&](const PieceCursor& u) {
    return static_cast<int64_t>(live(u) ? u.kvh : 0) * D * S::kElemBytes;
  };

  WaveState<T, D, G, CB> st;
  st.m = -__builtin_inff();
  st.l = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < S::kVec; ++e) st.acc[h][e] = 0.f;

  u32x4_t q[S::kKSeg];
  load_query<T, D, G, CB>(a.query, cur.seq, a.num_heads, (live(cur) ? cur.kvh : 0) * g, g, lane, q);
  Chunk<T, D, G, CB> fa, fb;
  load_chunk<T, D, G, CB, false, true>(fa, kc, vc, bt_row(cur.seq), cur.b_lo, cur.b_hi - 1, a.num_blocks, tok_stride,
                          blk_stride, head_off(cur), lane);
  PieceCursor nx = cur;
  cursor_next<CB>(nx, a, s_pre, nblk, R, wave);

  // Computes the current chunk (fcur) and closes its piece when it is the
  // piece's last chunk.
  auto compute = [&](Chunk<T, D, G, CB>& fcur) {
    const int tok0 = (cur.b_lo + cur.c * CB) * kBlockTokens;
    const bool last = cur.c == cur.nchunk - 1;
    float sc[CB][4];
    qk_chunk<T, D, G, CB>(sc, fcur, q, a.scale_log2);
    // The query of the next piece is fetched as soon as this piece's last
    // scores are out, so its latency hides behind the P*V work.
    if (last && nx.x >= 0)
      load_query<T, D, G, CB>(a.query, nx.seq, a.num_heads, (live(nx) ? nx.kvh : 0) * g, g, lane, q);
    softmax_pv_chunk<T, D, G, CB>(st, fcur, sc, tok0, cur.t_end, tok0 + CB * kBlockTokens > cur.t_end, lane);
    if (last) {
      if (live(cur)) {
        finish_piece<T, D, G, CB>(st, a, cur, lane);
      } else {
        st.m = -__builtin_inff();
        st.l = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < S::kVec; ++e) st.acc[h][e] = 0.f;
      }
    }
  };
  // The lookahead load is issued unconditionally inside the loop (the exit
  // test comes first), so the hardware wait before the current chunk's use
  // leaves the lookahead in flight; the scheduling barriers keep the loads
  // ahead of the arithmetic. Every block is read by one wave only, so the
  // loads are non-temporal.
  auto advance = [&](Chunk<T, D, G, CB>& fcur, Chunk<T, D, G, CB>& fnext) -> bool {
    if (nx.x < 0) {
      compute(fcur);
      return false;
    }
    load_chunk<T, D, G, CB, false, true>(fnext, kc, vc, bt_row(nx.seq), nx.b_lo + nx.c * CB, nx.b_hi - 1, a.num_blocks,
                            tok_stride, blk_stride, head_off(nx), lane);
    __builtin_amdgcn_sched_barrier(0);
    compute(fcur);
    __builtin_amdgcn_sched_barrier(0);
    cur = nx;
    cursor_next<CB>(nx, a, s_pre, nblk, R, wave);
    return true;
  };
  while (advance(fa, fb) && advance(fb, fa)) {
  }
}

// Log-sum-exp merge of np partials of one (sequence, head) row by one wave.
// Lane j owns output elements [j*D/64, (j+1)*D/64); lane p holds lse_p (lanes
// stride over p when np > 64). The first 32 partials are requested together
// with the lse values, before the maximum is known, and later ones 32 at a
// time, so a row costs one or two memory round trips instead of one per
// eight partials. A partial whose lse_p is -inf has weight 0 and its o_p (which
// may hold anything) does not enter the sum.
template <typename T, int D>
__device__ __forceinline__ void merge_row(T* out, float* lse_out, const float* o_row, const float* lse_row, int np,
                                          int lane) {
  constexpr int kPer = D / kWave;
  constexpr int kBatch = 32;
  const float lv0 = lane < np ? lse_row[lane] : -__builtin_inff();
  const float* op = o_row + lane * kPer;
  float v[kBatch][kPer];
#pragma unroll
  for (int u = 0; u < kBatch; ++u)
#pragma unroll
    for (int e = 0; e < kPer; ++e) v[u][e] = u < np ? op[u * D + e] : 0.f;
  float M = lv0;
  for (int p = lane + kWave; p < np; p += kWave) M = fmaxf(M, lse_row[p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, xor_shfl(M, off));
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float L = 0.f;
  if (M != -__builtin_inff()) {
    for (int p0 = 0; p0 < np; p0 += kWave) {
      const float lv = p0 == 0 ? lv0 : (p0 + lane < np ? lse_row[p0 + lane] : -__builtin_inff());
      const float w = lv == -__builtin_inff() ? 0.f : fast_exp2((lv - M) * kLog2e);
      float wsum = w;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) wsum += xor_shfl(wsum, off);
      L += wsum;
      const int cnt = min(kWave, np - p0);
      for (int i = 0; i < cnt; i += kBatch) {
        if (p0 != 0 || i != 0) {
#pragma unroll
          for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int e = 0; e < kPer; ++e) v[u][e] = i + u < cnt ? op[(p0 + i + u) * D + e] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), i + u));
          if (wu > 0.f) {
#pragma unroll
            for (int e = 0; e < kPer; ++e) acc[e] = fmaf(wu, v[u][e], acc[e]);
          }
        }
      }
    }
  }
  const bool empty = (M == -__builtin_inff());
#pragma unroll
  for (int e = 0; e < kPer; ++e) store_elem<T>(out + lane * kPer + e, empty ? 0.f : acc[e] / L);
  if (lse_out != nullptr && lane == 0) *lse_out = empty ? -__builtin_inff() : M + fast_log2(L) * kLn2;
}

// Merge for the partitioned path: row (sequence, head) combines the pieces its
// (sequence, kv head) pair was cut into. Pairs covered by one piece were
// written directly by the split kernel; an empty context gives 0 / -inf.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_pieces_kernel(T* __restrict__ out, float* __restrict__ lse_out,
                                                           const float* __restrict__ o_parts,
                                                           const float* __restrict__ lse_parts,
                                                           const int64_t* __restrict__ header, int num_seqs,
                                                           int num_heads, int num_kv_heads, int heads_per_group,
                                                           int slots) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= static_cast<int64_t>(num_seqs) * num_heads) return;
  const int seq = static_cast<int>(row / num_heads);
  const int kvh = static_cast<int>(row - static_cast<int64_t>(seq) * num_heads) / (num_heads / num_kv_heads);
  const int gi = kvh / heads_per_group;
  const int64_t nblk = header[0];
  const int64_t R = header[1];
  const int* pre = reinterpret_cast<const int*>(header + 2);
  const int64_t Tseq = pre[num_seqs];
  const int nb = pre[seq + 1] - pre[seq];
  int np = 0;
  if (nb > 0) {
    const int64_t x0 = static_cast<int64_t>(gi) * Tseq + pre[seq];
    np = static_cast<int>(range_of(x0 + nb - 1, nblk, R) - range_of(x0, nblk, R)) + 1;
  }
  if (np == 1) return;
  if (np > slots) np = slots;
  merge_row<T, D>(out + row * D, lse_out != nullptr ? lse_out + row : nullptr, o_parts + row * slots * D,
                  lse_parts + row * slots, np, lane);
}

// One wave per (sequence, head) row: out = sum_p w_p o_p / sum_p w_p with
// w_p = exp(lse_p - max lse); partitions at -inf are skipped outright.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_partitions_kernel(T* __restrict__ out, float* __restrict__ lse_out,
                                                               const float* __restrict__ o_parts,
                                                               const float* __restrict__ lse_parts,
                                                               int64_t num_rows, int num_parts) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= num_rows) return;
  merge_row<T, D>(out + row * D, lse_out != nullptr ? lse_out + row : nullptr, o_parts + row * num_parts * D,
                  lse_parts + row * num_parts, num_parts, lane);
}

// Merge for the partition path: row (sequence, head) combines the
// min(ceil(n_i / P), num_parts) partitions its sequence was cut into (partial
// rows spaced `slots` apart); an empty context gives 0 / -inf.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_parts_kernel(T* __restrict__ out, float* __restrict__ lse_out,
                                                          const float* __restrict__ o_parts,
                                                          const float* __restrict__ lse_parts,
                                                          const int32_t* __restrict__ context_lens, int num_seqs,
                                                          int num_heads, int max_tokens, int part_tokens,
                                                          int num_parts, int slots) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= static_cast<int64_t>(num_seqs) * num_heads) return;
  const int seq = static_cast<int>(row / num_heads);
  int n = context_lens[seq];
  n = n < 0 ? 0 : (n > max_tokens ? max_tokens : n);
  const int np = min((n + part_tokens - 1) / part_tokens, num_parts);
  merge_row<T, D>(out + row * D, lse_out != nullptr ? lse_out + row : nullptr, o_parts + row * slots * D,
                  lse_parts + row * slots, np, lane);
}

// Merge of the multi-query partitions: one wave per (token, head) row. The
// token's sequence is found by binary search over query_start_loc; the token
// at position n - q + j of its sequence sees keys below that position + 1,
// i.e. the first ceil(min(position + 1, cap) / P) partitions.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_mq_parts_kernel(T* __restrict__ out, float* __restrict__ lse_out,
                                                             const float* __restrict__ o_parts,
                                                             const float* __restrict__ lse_parts,
                                                             const int32_t* __restrict__ loc,
                                                             const int32_t* __restrict__ context_lens, int num_seqs,
                                                             int num_tokens, int num_heads, int cap, int max_tokens,
                                                             int part_tokens, int num_parts) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= static_cast<int64_t>(num_tokens) * num_heads) return;
  const int t = static_cast<int>(row / num_heads);
  auto cl = [&](int v) { return v < 0 ? 0 : (v > num_tokens ? num_tokens : v); };
  int lo = 0, hi = num_seqs;  // largest seq with loc[seq] <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cl(loc[mid]) <= t) lo = mid; else hi = mid;
  }
  const int q0 = cl(loc[lo]), q1 = cl(loc[lo + 1]);
  int np = 0;
  if (t >= q0 && t < q1) {
    int n = context_lens[lo];
    n = n < 0 ? 0 : (n > max_tokens ? max_tokens : n);
    int lim = n - (q1 - q0) + (t - q0) + 1;
    lim = lim < 0 ? 0 : (lim > cap ? cap : lim);
    np = min((lim + part_tokens - 1) / part_tokens, num_parts);
  }
  merge_row<T, D>(out + row * D, lse_out != nullptr ? lse_out + row : nullptr, o_parts + row * num_parts * D,
                  lse_parts + row * num_parts, np, lane);
}

// ------------------------------------------------------------------ host side
namespace {

// Rows (one wave each) per workgroup of the merge kernels: one for merges of
// up to eight rows per compute unit, so that a small merge (a few hundred to
// a few thousand rows of long partial lists) spreads its loads over every
// compute unit instead of a quarter of them; PA_OPT_MERGE_ROWS forces a count.
int merge_rows_per_block(int64_t rows) {
  const int v = option_value(PA_OPT_MERGE_ROWS);
  if (v == 1 || v == 2 || v == 4) return v;
  return rows <= 8 * static_cast<int64_t>(device_cus()) ? 1 : 4;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int next_pow2_group(int g) {
  int G = 1;
  while (G < g) G <<= 1;
  return G;
}

int check_common(const void* out, const void* query, const void* key_cache, const void* value_cache,
                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                 int64_t num_blocks, int32_t block_size, int32_t dtype) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return PA_ERR_INVALID_ARG;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_INVALID_ARG;
  if (num_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (num_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != kBlockTokens) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
    return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_blocks_per_seq) * kBlockTokens > INT32_MAX) return PA_ERR_INVALID_ARG;
  // A token row (all kv heads) must stay under 2^24 bytes (24-bit row offsets).
  if (static_cast<int64_t>(num_kv_heads) * head_size * 4 >= (int64_t{1} << 24)) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// Workgroups of `kernel` with `threads` threads that fit on the device at once.
int resident_groups(const void* kernel, int threads, size_t lds) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess) return 0;
  return cus * (per_cu > 0 ? per_cu : 1);
}

typedef void (*SplitKernel)(SplitArgs);

// The partitioned path keeps a cursor and the next piece's state live across
// its loop, so it streams one block per chunk.
template <typename T, int D, int G>
SplitKernel split_kernel_for() {
  return paged_decode_split_kernel<T, D, G, 1>;
}

template <typename T, int D>
SplitKernel pick_split_group(int G) {
  switch (G) {
    case 1: return split_kernel_for<T, D, 1>();
    case 2: return split_kernel_for<T, D, 2>();
    case 4: return split_kernel_for<T, D, 4>();
    case 8: return split_kernel_for<T, D, 8>();
    case 16: return split_kernel_for<T, D, 16>();
    default: return nullptr;
  }
}

SplitKernel pick_split(int dtype, int D, int G) {
  if (dtype == PA_DTYPE_BF16) return D == 128 ? pick_split_group<bf16_t, 128>(G) : pick_split_group<bf16_t, 64>(G);
  return D == 128 ? pick_split_group<float, 128>(G) : pick_split_group<float, 64>(G);
}

int launch_split(const SplitArgs& args, int dtype, int head_size, hipStream_t stream) {
  const int G = next_pow2_group(args.group);
  SplitKernel k = pick_split(dtype, head_size, G);
  if (!k) return PA_ERR_UNSUPPORTED;
  const int threads = kWave * args.heads_per_group;
  const size_t lds = (static_cast<size_t>(args.num_seqs) + 1) * sizeof(int);
  const int resident = resident_groups(reinterpret_cast<const void*>(k), threads, lds);
  if (resident <= 0) return PA_ERR_HIP;
  // Persistent grid: as many workgroups as fit at once, and no more than the
  // work can use (each range spans at least partition_size tokens).
  const int64_t blocks_bound = static_cast<int64_t>(args.num_seqs) * args.max_blocks * args.num_groups;
  const int64_t useful = blocks_bound / (args.part_tokens / kBlockTokens) + 1;
  int64_t grid = resident;
  if (grid > useful) grid = useful;
  if (grid < 1) grid = 1;
  if (grid > INT32_MAX) return PA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(grid)), dim3(threads), lds, stream, args);
  if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  const int64_t rows = static_cast<int64_t>(args.num_seqs) * args.num_heads;
  const int kRowsPerBlock = merge_rows_per_block(rows);
  const int64_t mgrid = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (mgrid > INT32_MAX) return PA_ERR_UNSUPPORTED;
  dim3 g(static_cast<unsigned>(mgrid)), b(kRowsPerBlock * kWave);
#define PA_MERGE_PIECES(TT, DD)                                                                                    \
  hipLaunchKernelGGL((merge_pieces_kernel<TT, DD>), g, b, 0, stream, static_cast<TT*>(args.out), args.lse_out,   \
                     args.o_parts, args.lse_parts, args.header, args.num_seqs, args.num_heads, args.num_kv_heads, \
                     args.heads_per_group, args.slots)
  if (dtype == PA_DTYPE_BF16) {
    if (head_size == 128) PA_MERGE_PIECES(bf16_t, 128); else PA_MERGE_PIECES(bf16_t, 64);
  } else {
    if (head_size == 128) PA_MERGE_PIECES(float, 128); else PA_MERGE_PIECES(float, 64);
  }
#undef PA_MERGE_PIECES
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int launch_merge(void* out, float* lse_out, const float* o_parts, const float* lse_parts, int64_t rows,
                 int num_parts, int head_size, int dtype, hipStream_t stream) {
  if (rows <= 0) return PA_OK;
  const int kRowsPerBlock = merge_rows_per_block(rows);
  const int64_t grid = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (grid > INT32_MAX) return PA_ERR_UNSUPPORTED;
  dim3 g(static_cast<unsigned>(grid)), b(kRowsPerBlock * kWave);
  if (dtype == PA_DTYPE_BF16) {
    if (head_size == 128)
      hipLaunchKernelGGL((merge_partitions_kernel<bf16_t, 128>), g, b, 0, stream, static_cast<bf16_t*>(out),
                         lse_out, o_parts, lse_parts, rows, num_parts);
    else
      hipLaunchKernelGGL((merge_partitions_kernel<bf16_t, 64>), g, b, 0, stream, static_cast<bf16_t*>(out),
                         lse_out, o_parts, lse_parts, rows, num_parts);
  } else {
    if (head_size == 128)
      hipLaunchKernelGGL((merge_partitions_kernel<float, 128>), g, b, 0, stream, static_cast<float*>(out),
                         lse_out, o_parts, lse_parts, rows, num_parts);
    else
      hipLaunchKernelGGL((merge_partitions_kernel<float, 64>), g, b, 0, stream, static_cast<float*>(out),
                         lse_out, o_parts, lse_parts, rows, num_parts);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int launch_merge_parts(void* out, float* lse_out, const float* o_parts, const float* lse_parts,
                       const int32_t* context_lens, int num_seqs, int num_heads, int max_tokens, int part_tokens,
                       int num_parts, int slots, int head_size, int dtype, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_heads;
  if (rows <= 0) return PA_OK;
  const int kRowsPerBlock = merge_rows_per_block(rows);
  const int64_t grid = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (grid > INT32_MAX) return PA_ERR_UNSUPPORTED;
  dim3 g(static_cast<unsigned>(grid)), b(kRowsPerBlock * kWave);
#define PA_MERGE_PARTS(TT, DD)                                                                                   \
  hipLaunchKernelGGL((merge_parts_kernel<TT, DD>), g, b, 0, stream, static_cast<TT*>(out), lse_out, o_parts,     \
                     lse_parts, context_lens, num_seqs, num_heads, max_tokens, part_tokens, num_parts, slots)
  if (dtype == PA_DTYPE_BF16) {
    if (head_size == 128) PA_MERGE_PARTS(bf16_t, 128); else PA_MERGE_PARTS(bf16_t, 64);
  } else {
    if (head_size == 128) PA_MERGE_PARTS(float, 128); else PA_MERGE_PARTS(float, 64);
  }
#undef PA_MERGE_PARTS
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// pa_decode_split's cut: context partitions on the multi-query kernel (one
// workgroup per (sequence, partition, kv head), from the hardware
// dispatcher) when its 16-column tiles hold the group; pieces on the
// persistent split kernel, whose workgroups read whole token rows (one wave
// per kv head), for groups above 16 and, with float32 caches, for groups of
// at most 4 when the batch has fewer (sequence, kv head) pairs than resident
// tile workgroups (2 per CU): long contexts of a few sequences. With 16-bit
// caches the tile kernel's row-wise K loads made the partitions faster there
// too (batch of 8, contexts 16k-32k: 134.3 vs 141.4 us). (Larger groups keep
// the tiles: the piece kernel's per-lane accumulators spill registers from a
// group of 8 up.) PA_OPT_SPLIT_CUT forces a cut.
bool split_by_tiles(int group, int num_seqs, int num_kv_heads, int dtype) {
  if (group > 16) return false;
  const int v = option_value(PA_OPT_SPLIT_CUT);
  if (v == 1) return true;
  if (v == 2) return false;
  if (group > 4 || dtype == PA_DTYPE_BF16) return true;
  return static_cast<int64_t>(num_seqs) * num_kv_heads >= 2 * static_cast<int64_t>(device_cus());
}

// Partition length of the partition cut: k * P with k the largest factor
// that still leaves about three rounds of resident tile workgroups for the
// longest possible batch (num_seqs contexts of max_context_len tokens), so
// each workgroup streams long enough to amortise its start; at most the
// longest context. PA_OPT_SPLIT_PART_FACTOR forces k.
int split_part_tokens(int num_seqs, int num_kv_heads, int max_context_len, int P) {
  const int64_t n_p = (static_cast<int64_t>(max_context_len) + P - 1) / P;
  if (n_p <= 1) return P;
  int64_t k = option_value(PA_OPT_SPLIT_PART_FACTOR);
  if (k <= 0) {
    const int64_t target = 3 * 2 * static_cast<int64_t>(device_cus());  // 2 tile workgroups per CU
    k = static_cast<int64_t>(num_seqs) * n_p * num_kv_heads / target;
  }
  k = k < 1 ? 1 : (k > n_p ? n_p : k);
  return static_cast<int>(k * P);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

int launch_merge_mq_parts(void* out, float* lse_out, const float* o_parts, const float* lse_parts,
                              const int32_t* query_start_loc, const int32_t* context_lens, int num_seqs,
                              int num_tokens, int num_heads, int cap, int max_blocks, int partition_size,
                              int num_parts, int head_size, int dtype, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(num_tokens) * num_heads;
  if (rows <= 0) return PA_OK;
  const int kRowsPerBlock = merge_rows_per_block(rows);
  const int64_t grid = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (grid > INT32_MAX) return PA_ERR_UNSUPPORTED;
  const int max_tokens = max_blocks * kBlockTokens;
  dim3 g(static_cast<unsigned>(grid)), b(kRowsPerBlock * kWave);
#define PA_MERGE_MQ(TT, DD)                                                                                      \
  hipLaunchKernelGGL((merge_mq_parts_kernel<TT, DD>), g, b, 0, stream, static_cast<TT*>(out), lse_out, o_parts,  \
                     lse_parts, query_start_loc, context_lens, num_seqs, num_tokens, num_heads, cap, max_tokens,  \
                     partition_size, num_parts)
  if (dtype == PA_DTYPE_BF16) {
    if (head_size == 128) PA_MERGE_MQ(bf16_t, 128); else PA_MERGE_MQ(bf16_t, 64);
  } else {
    if (head_size == 128) PA_MERGE_MQ(float, 128); else PA_MERGE_MQ(float, 64);
  }
#undef PA_MERGE_MQ
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa

using namespace pa;

extern "C" int pa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_size, int64_t num_blocks, int32_t block_size,
                         float scale, int32_t dtype, float* lse_out, const int32_t* seq_order, void* stream) {
  int st = check_common(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                        num_seqs, num_heads, num_kv_heads, head_size, num_blocks, block_size, dtype);
  if (st != PA_OK || num_seqs == 0) return st;
  return launch_decode_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                             num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale * kLog2e, 1.0f, dtype,
                             false, lse_out, seq_order, 0, nullptr, nullptr, static_cast<hipStream_t>(stream));
}

extern "C" int32_t pa_decode_split_part_tokens(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                               int32_t max_context_len, int32_t partition_size, int32_t dtype) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return -1;
  if (max_context_len < 0 || partition_size <= 0 || partition_size % kBlockTokens != 0) return -1;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return -1;
  if (!split_by_tiles(num_heads / num_kv_heads, num_seqs, num_kv_heads, dtype)) return 0;
  return split_part_tokens(num_seqs, num_kv_heads, max_context_len, partition_size);
}

extern "C" size_t pa_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_size) {
  if (num_seqs < 0 || num_heads <= 0 || head_size <= 0) return 0;
  const size_t rows = static_cast<size_t>(num_seqs) * num_heads;
  return align256(rows * head_size * sizeof(float)) + align256(rows * sizeof(float));
}

extern "C" int pa_decode_prefix(void* out, const void* query, const void* key_cache, const void* value_cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_size, int64_t num_blocks, int32_t block_size,
                                float scale, int32_t dtype, int32_t prefix_blocks, void* workspace,
                                size_t workspace_bytes, float* lse_out, const int32_t* seq_order, void* stream) {
  int st = check_common(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                        num_seqs, num_heads, num_kv_heads, head_size, num_blocks, block_size, dtype);
  if (st != PA_OK) return st;
  if (prefix_blocks < 0 || prefix_blocks > max_blocks_per_seq) return PA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || scale == __builtin_inff()) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (prefix_blocks == 0)
    return pa_decode(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                     num_heads, num_kv_heads, head_size, num_blocks, block_size, scale, dtype, lse_out, seq_order,
                     stream);
  const size_t need = pa_decode_prefix_workspace_bytes(num_seqs, num_heads, head_size);
  if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return PA_ERR_WORKSPACE;
  const size_t rows = static_cast<size_t>(num_seqs) * num_heads;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(rows * head_size * sizeof(float)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_prefix_pass(query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                          num_heads, num_kv_heads, head_size, num_blocks, prefix_blocks, scale, dtype, part_o,
                          part_lse, s);
  if (st != PA_OK) return st;
  return launch_decode_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                             num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale * kLog2e, 1.0f, dtype,
                             false, lse_out, seq_order, prefix_blocks, part_o, part_lse, s);
}

extern "C" int pa_decode_fp8(void* out, const void* query, const uint8_t* key_cache, const uint8_t* value_cache,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                             int32_t num_kv_heads, int32_t head_size, int64_t num_blocks, int32_t block_size,
                             float scale, float k_scale, float v_scale, int32_t dtype, float* lse_out,
                             const int32_t* seq_order, void* stream) {
  int st = check_common(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                        num_seqs, num_heads, num_kv_heads, head_size, num_blocks, block_size, dtype);
  if (st != PA_OK || num_seqs == 0) return st;
  if (dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale == __builtin_inff() || v_scale == __builtin_inff())
    return PA_ERR_INVALID_ARG;
  // Keys are code values times k_scale: the scale folds into the scores'.
  return launch_decode_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                             num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale * k_scale * kLog2e,
                             v_scale, dtype, true, lse_out, seq_order, 0, nullptr, nullptr,
                             static_cast<hipStream_t>(stream));
}

// Workspace layout: o_p [S, H_q, slots, D] float32 | lse_p [S, H_q, slots]
// float32 | header: int64 T, int64 R, int32 blocks prefix [S + 1]; each part
// 256-byte aligned.
struct SplitLayout {
  int64_t slots = 0;
  size_t lse_off = 0, header_off = 0, total = 0;
};

bool split_layout(int32_t num_seqs, int32_t num_heads, int32_t head_size, int32_t max_context_len,
                  int32_t partition_size, SplitLayout& L) {
  if (num_seqs < 0 || num_heads <= 0 || head_size <= 0 || max_context_len < 0 || partition_size <= 0) return false;
  L.slots = (static_cast<int64_t>(max_context_len) + partition_size - 1) / partition_size + 1;
  const size_t rows = static_cast<size_t>(num_seqs) * num_heads * static_cast<size_t>(L.slots);
  L.lse_off = align256(rows * head_size * sizeof(float));
  L.header_off = L.lse_off + align256(rows * sizeof(float));
  L.total = L.header_off + align256(2 * sizeof(int64_t) + (static_cast<size_t>(num_seqs) + 1) * sizeof(int32_t));
  return L.slots <= INT32_MAX;
}

extern "C" size_t pa_decode_split_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_size,
                                                  int32_t max_context_len, int32_t partition_size) {
  SplitLayout L;
  return split_layout(num_seqs, num_heads, head_size, max_context_len, partition_size, L) ? L.total : 0;
}

namespace {

// The work of pa_decode_split once the arguments and the layout are checked:
// partials, log-sum-exps and the pieces header go to `workspace`.
int decode_split_launch(void* out, const void* query, const void* key_cache, const void* value_cache,
                        const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                        int64_t num_blocks, float scale, int32_t dtype, int32_t max_context_len,
                        int32_t partition_size, const SplitLayout& L, void* workspace, float* lse_out,
                        void* stream) {
  int st = PA_OK;

  SplitArgs args{};
  args.query = query;
  args.key_cache = key_cache;
  args.value_cache = value_cache;
  args.block_tables = block_tables;
  args.context_lens = context_lens;
  args.out = out;
  args.lse_out = lse_out;
  args.o_parts = static_cast<float*>(workspace);
  args.lse_parts = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.lse_off);
  args.header = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + L.header_off);
  args.num_blocks = num_blocks;
  args.max_blocks = max_blocks_per_seq;
  args.num_seqs = num_seqs;
  args.num_heads = num_heads;
  args.num_kv_heads = num_kv_heads;
  args.group = num_heads / num_kv_heads;
  args.heads_per_group = num_kv_heads < kMaxHeadsPerGroup ? num_kv_heads : kMaxHeadsPerGroup;
  args.num_groups = (num_kv_heads + args.heads_per_group - 1) / args.heads_per_group;
  args.part_tokens = partition_size;
  args.slots = static_cast<int32_t>(L.slots);
  args.scale_log2 = scale * kLog2e;
  if (split_by_tiles(args.group, num_seqs, num_kv_heads, dtype)) {
    // Partitions of pt = k * P tokens; positions past ceil(max_context_len / P) * P
    // are ignored, as with the pieces cut.
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int pt = split_part_tokens(num_seqs, num_kv_heads, max_context_len, partition_size);
    const int64_t cap = min(static_cast<int64_t>(max_blocks_per_seq) * kBlockTokens,
                            static_cast<int64_t>(partition_size) * (L.slots - 1));
    const int num_parts = static_cast<int>((cap + pt - 1) / pt);
    if (num_parts > 0) {
      st = launch_split_tiles(query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                              num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale, dtype,
                              pt / kBlockTokens, num_parts, static_cast<int>(cap), args.slots, args.o_parts,
                              args.lse_parts, s);
      if (st != PA_OK) return st;
    }
    return launch_merge_parts(out, lse_out, args.o_parts, args.lse_parts, context_lens, num_seqs, num_heads,
                              static_cast<int>(cap), pt, num_parts, args.slots, head_size, dtype, s);
  }
  return launch_split(args, dtype, head_size, static_cast<hipStream_t>(stream));
}

// Host checks shared by pa_decode_split and pa_decode_split_noalloc; on PA_OK
// with num_seqs > 0, L holds the workspace layout.
int check_split(const void* out, const void* query, const void* key_cache, const void* value_cache,
                const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size, int64_t num_blocks,
                int32_t block_size, int32_t dtype, int32_t max_context_len, int32_t partition_size,
                SplitLayout& L) {
  int st = check_common(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                        num_seqs, num_heads, num_kv_heads, head_size, num_blocks, block_size, dtype);
  if (st != PA_OK) return st;
  if (partition_size <= 0 || partition_size % kBlockTokens != 0 || max_context_len < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (!split_layout(num_seqs, num_heads, head_size, max_context_len, partition_size, L)) return PA_ERR_UNSUPPORTED;
  if ((static_cast<size_t>(num_seqs) + 1) * sizeof(int) > 64 * 1024) return PA_ERR_UNSUPPORTED;  // LDS prefix
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_split(void* out, const void* query, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_size, int64_t num_blocks,
                               int32_t block_size, float scale, int32_t dtype, int32_t max_context_len,
                               int32_t partition_size, void* workspace, size_t workspace_bytes,
                               float* lse_out, void* stream) {
  SplitLayout L;
  const int st = check_split(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                             num_seqs, num_heads, num_kv_heads, head_size, num_blocks, block_size, dtype,
                             max_context_len, partition_size, L);
  if (st != PA_OK || num_seqs == 0) return st;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_INVALID_ARG;
  if (workspace_bytes < L.total) return PA_ERR_WORKSPACE;
  return decode_split_launch(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                             num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale, dtype,
                             max_context_len, partition_size, L, workspace, lse_out, stream);
}

// ------------------------------------------------------------------ pa_decode_split_noalloc
// The workspace of pa_decode_split_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in); it passes the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[PA_DECODE_SPLIT_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    p = ptr;
  }
  return p;
}

}  // namespace

extern "C" int pa_decode_split_noalloc(void* out, const void* query, const void* key_cache, const void* value_cache,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_size, int64_t num_blocks,
                                       int32_t block_size, float scale, int32_t dtype, int32_t max_context_len,
                                       int32_t partition_size, float* lse_out, void* stream) {
  SplitLayout L;
  const int st = check_split(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                             num_seqs, num_heads, num_kv_heads, head_size, num_blocks, block_size, dtype,
                             max_context_len, partition_size, L);
  if (st != PA_OK || num_seqs == 0) return st;
  if (L.total > static_cast<size_t>(PA_DECODE_SPLIT_NOALLOC_MAX_BYTES)) return PA_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return PA_ERR_HIP;
  return decode_split_launch(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                             num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale, dtype,
                             max_context_len, partition_size, L, ws, lse_out, stream);
}

extern "C" int pa_merge_partitions(void* out, float* lse_out, const float* o_parts, const float* lse_parts,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_parts, int32_t head_size,
                                   int32_t dtype, void* stream) {
  if (num_seqs < 0 || num_heads <= 0 || num_parts <= 0) return PA_ERR_INVALID_ARG;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_INVALID_ARG;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!out || !o_parts || !lse_parts) return PA_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(o_parts)) return PA_ERR_INVALID_ARG;
  return launch_merge(out, lse_out, o_parts, lse_parts, static_cast<int64_t>(num_seqs) * num_heads, num_parts,
                      head_size, dtype, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ kernel-choice options
namespace {

constexpr int kNumOptions = 5;
std::atomic<int> g_options[kNumOptions];

bool option_ok(int option, int value) {
  switch (option) {
    case PA_OPT_TILE_WAVES: return value == 0 || value == 4 || value == 8;
    case PA_OPT_TILE_COLUMNS: return value == 0 || value == 16 || value == 32;
    case PA_OPT_SPLIT_CUT: return value >= 0 && value <= 2;
    case PA_OPT_SPLIT_PART_FACTOR: return value >= 0;
    case PA_OPT_MERGE_ROWS: return value == 0 || value == 1 || value == 2 || value == 4;
    default: return false;
  }
}

}  // namespace

int pa::option_value(int option) {
  return option >= 0 && option < kNumOptions ? g_options[option].load(std::memory_order_relaxed) : 0;
}

extern "C" int pa_set_option(int option, int value) {
  if (option < 0 || option >= kNumOptions || !option_ok(option, value)) return PA_ERR_INVALID_ARG;
  g_options[option].store(value, std::memory_order_relaxed);
  return PA_OK;
}

extern "C" int pa_get_option(int option) {
  if (option < 0 || option >= kNumOptions) return -1;
  return g_options[option].load(std::memory_order_relaxed);
}
