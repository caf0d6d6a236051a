// Paged decode attention for gfx950: pa_decode, pa_decode_split, pa_merge_partitions.
//
// What is computed (llm-stack-book 7.3 "vLLM: Architecture, PagedAttention &
// Internals", sections "PagedAttention in one paragraph" and "The forward step
// in detail"): for each sequence and query head, ordinary attention of the one
// new query over the sequence's whole context, with K/V rows found through the
// block table instead of in one contiguous tensor. The softmax runs online over
// streamed blocks (stanleyjacob.dev "vLLM", Part IV "Stage 6: The forward
// pass"); a context split into partitions is recombined exactly with
// log-sum-exp weights.
//
// Work decomposition (one workgroup per (sequence, kv head, context
// partition), W waves per workgroup):
//  * A wave handles "chunks" of CB consecutive 16-token blocks; chunk c goes to
//    wave c % W. All g = H_q/H_kv query heads of the kv head share every K/V
//    tile the wave loads.
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
//  * P*V runs on the VALU in fp32 (the V tile would need a transpose for MFMA).
//  * Online softmax per chunk with base-2 exponentials (scale*log2(e) folded
//    into the scores); the chunk maximum is reduced across the 4 row groups.
//  * At the end each wave reduces its partial sums across row groups and the W
//    waves merge through LDS with log-sum-exp weights.
// Reduction order depends only on logical token positions, W and CB, never on
// physical block ids, so results do not change when blocks move or are shared.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_tiles.h"

namespace pa {

struct DecodeArgs {
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* lse_out;            // optional
  const int32_t* seq_order;  // optional processing order of sequences
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;        // H_q / H_kv
  int32_t num_jobs;     // job ids: ceil(num_seqs / 8) * 8 * num_kv_heads
  float scale_log2;     // scale * log2(e) (times k_scale for FP8 caches)
  float v_scale;        // multiplies the normalised output: v_scale for FP8 caches, else 1
  // Suffix pass of the shared-prefix decode: keys of blocks < skip_blocks were
  // attended by the prefix pass, whose normalised float32 output and
  // log-sum-exp per (sequence, query head) join the final merge. Zero / null
  // for a plain decode.
  int32_t skip_blocks;
  const float* prefix_o;    // [num_seqs, num_heads, D]
  const float* prefix_lse;  // [num_seqs, num_heads]
};

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
__device__ __forceinline__ void compute_chunk(WaveState<T, D, G, CB>& st, const Chunk<T, D, G, CB, F8>& f,
                                              const u32x4_t (&q)[DecodeShape<T, D, G, CB, F8>::kQSeg],
                                              float scale_log2, int tok0, int t_end, bool mask, int lane) {
  float s[CB][4];
  qk_chunk<T, D, G, CB, F8>(s, f, q, scale_log2);
  softmax_pv_chunk<T, D, G, CB, F8>(st, f, s, tok0, t_end, mask, lane);
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

// One decode job is one (sequence, kv head); job ids follow the XCD-aware
// order of slot_and_head (id % 8 names the XCD meant to run it, and all kv
// heads of a sequence share it), and ids past the last sequence are padding.
struct DecodeJob {
  int seq;  // -1 for a padding id
  int kvh;
  int n;    // context tokens, clamped to the block table
};

__device__ __forceinline__ DecodeJob decode_job(const DecodeArgs& a, int id) {
  DecodeJob j;
  int seq, kvh;
  slot_and_head(id, a.num_kv_heads, seq, kvh);
  j.kvh = kvh;
  j.seq = -1;
  j.n = 0;
  if (seq >= a.num_seqs) return j;
  if (a.seq_order != nullptr) {
    // Schedule hint: the j-th dispatched sequence is seq_order[j]. Out-of-range
    // entries are clamped (wrong output for that caller, never a bad access).
    const uint32_t o = static_cast<uint32_t>(a.seq_order[seq]);
    seq = static_cast<int>(o < static_cast<uint32_t>(a.num_seqs) ? o : a.num_seqs - 1);
  }
  const int max_tokens = a.max_blocks * kBlockTokens;
  const int n = a.context_lens[seq];
  j.n = n < 0 ? 0 : (n > max_tokens ? max_tokens : n);
  j.seq = seq;
  return j;
}

// Job k of persistent workgroup w out of `grid`: rounds of `grid` consecutive
// ids, walked forwards in even rounds and backwards in odd ones, so that with
// jobs in longest-first order every workgroup gets a similar total. grid is a
// multiple of 8, so the kv heads of one sequence (ids equal mod 8) still run on
// one XCD.
__device__ __forceinline__ int job_of(int k, int w, int grid) {
  const int base = k * grid;
  return (k & 1) ? base + grid - 1 - w : base + w;
}

// This wave's share of one job: chunks wave, wave + W, ... of the context.
struct JobPlan {
  const int32_t* bt_row;
  int64_t head_off;
  int blk_last;    // last block of the context
  int mine;        // chunks of this wave
  int mask_chunk;  // the chunk that reaches past the context end, or -1
};

// Chunk c of a job starts at block skip_blocks + c * CB.

template <int EB, int D, int CB>  // EB: bytes per cache element
__device__ __forceinline__ JobPlan plan_job(const DecodeArgs& a, const DecodeJob& j, int wave, int nwaves) {
  JobPlan p;
  p.bt_row = a.block_tables + static_cast<int64_t>(j.seq < 0 ? 0 : j.seq) * a.max_blocks;
  p.head_off = static_cast<int64_t>(j.kvh) * D * EB;
  const int blk_end = (j.n + kBlockTokens - 1) / kBlockTokens;
  const int nchunk = blk_end > a.skip_blocks ? (blk_end - a.skip_blocks + CB - 1) / CB : 0;
  p.blk_last = blk_end - 1;
  p.mine = (j.seq >= 0 && wave < nchunk) ? (nchunk - wave + nwaves - 1) / nwaves : 0;
  p.mask_chunk = ((a.skip_blocks + nchunk * CB) * kBlockTokens > j.n) ? nchunk - 1 : -1;
  return p;
}

// Persistent workgroups, each taking the jobs job_of(0, w), job_of(1, w), ...
// While a job's waves merge their partial results, the next job's query and
// first chunk are already being loaded, so no workgroup waits on a cold start
// between jobs.
// Two workgroups per CU (at most 256 registers per lane); the 16-head group
// needs more registers and runs one workgroup per CU.
template <typename T, int D, int G, int CB, bool PF, bool F8 = false>
__global__ __launch_bounds__(G >= 16 ? 256 : 512, 1) void paged_decode_kernel(DecodeArgs a) {
  using S = DecodeShape<T, D, G, CB, F8>;
  extern __shared__ float s_acc[];  // [W][G][D]
  __shared__ float s_m[8][16];
  __shared__ float s_l[8][16];

  const int lane = threadIdx.x & 63;
  // Wave-uniform by construction; readfirstlane lets the compiler keep all
  // per-wave indexing (units, block ids, base addresses) in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int grid = gridDim.x;
  const int w = blockIdx.x;
  const int g = a.group;

  const uint32_t tok_stride = static_cast<uint32_t>(a.num_kv_heads) * D * S::kElemBytes;
  const int64_t blk_stride = static_cast<int64_t>(tok_stride) * kBlockTokens;
  const char* kc = static_cast<const char*>(a.key_cache);
  const char* vc = static_cast<const char*>(a.value_cache);

  int k = 0;
  const int id0 = job_of(0, w, grid);
  DecodeJob cur;
  cur.seq = -1;
  cur.kvh = 0;
  cur.n = 0;
  if (id0 < a.num_jobs) cur = decode_job(a, id0);
  JobPlan pc = plan_job<S::kElemBytes, D, CB>(a, cur, wave, nwaves);
  // Block of this wave's i-th chunk of a job.
  auto blk_of = [&](int i) { return a.skip_blocks + (wave + i * nwaves) * CB; };

  u32x4_t q[S::kQSeg];
  Chunk<T, D, G, CB, F8> fa;
  if (cur.n > 0 && cur.seq >= 0) {
    load_query<T, D, G, CB, F8>(a.query, cur.seq, a.num_heads, cur.kvh * g, g, lane, q);
    if (PF && pc.mine > 0)
      load_chunk<T, D, G, CB, F8>(fa, kc, vc, pc.bt_row, blk_of(0), pc.blk_last, a.num_blocks, tok_stride,
                              blk_stride, pc.head_off, lane);
  }
  int id = id0;
  while (id < a.num_jobs) {
    // The next job is known now: its metadata is fetched a whole job ahead.
    const int id_next = job_of(k + 1, w, grid);
    DecodeJob nxt;
    nxt.seq = -1;
    nxt.kvh = 0;
    nxt.n = 0;
    if (id_next < a.num_jobs) nxt = decode_job(a, id_next);

    WaveState<T, D, G, CB> st;
    st.m = -__builtin_inff();
    st.l = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < S::kVec; ++e) st.acc[h][e] = 0.f;

    const int mine = pc.mine;
    auto tok_of = [&](int i) { return blk_of(i) * kBlockTokens; };
    auto is_mask = [&](int i) { return wave + i * nwaves == pc.mask_chunk; };
    if constexpr (PF) {
      // One chunk of lookahead, fa already in flight. The steady-state loop
      // issues its lookahead loads unconditionally and the last one or two
      // chunks are peeled off: with a conditional load inside the loop the
      // hardware wait counts on the two paths differ and the wait before the
      // current chunk's use would also cover the lookahead. The scheduling
      // barriers keep the loads ahead of the current chunk's arithmetic (left
      // alone, the scheduler sinks them to shorten register live ranges).
      // Only the final chunk of the context, a wave's last, can need a mask.
      Chunk<T, D, G, CB, F8> fb;
      if (mine > 0) {
        int i = 0;
        for (; i + 2 < mine; i += 2) {
          load_chunk<T, D, G, CB, F8>(fb, kc, vc, pc.bt_row, blk_of(i + 1), pc.blk_last, a.num_blocks, tok_stride,
                                  blk_stride, pc.head_off, lane);
          __builtin_amdgcn_sched_barrier(0);
          compute_chunk<T, D, G, CB, F8>(st, fa, q, a.scale_log2, tok_of(i), cur.n, false, lane);
          __builtin_amdgcn_sched_barrier(0);
          load_chunk<T, D, G, CB, F8>(fa, kc, vc, pc.bt_row, blk_of(i + 2), pc.blk_last, a.num_blocks, tok_stride,
                                  blk_stride, pc.head_off, lane);
          __builtin_amdgcn_sched_barrier(0);
          compute_chunk<T, D, G, CB, F8>(st, fb, q, a.scale_log2, tok_of(i + 1), cur.n, false, lane);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (i + 1 < mine) {
          load_chunk<T, D, G, CB, F8>(fb, kc, vc, pc.bt_row, blk_of(i + 1), pc.blk_last, a.num_blocks, tok_stride,
                                  blk_stride, pc.head_off, lane);
          __builtin_amdgcn_sched_barrier(0);
          compute_chunk<T, D, G, CB, F8>(st, fa, q, a.scale_log2, tok_of(i), cur.n, false, lane);
          compute_chunk<T, D, G, CB, F8>(st, fb, q, a.scale_log2, tok_of(i + 1), cur.n, is_mask(i + 1), lane);
        } else {
          compute_chunk<T, D, G, CB, F8>(st, fa, q, a.scale_log2, tok_of(i), cur.n, is_mask(i), lane);
        }
      }
    } else {
      for (int i = 0; i < mine; ++i) {
        load_chunk<T, D, G, CB, F8>(fa, kc, vc, pc.bt_row, blk_of(i), pc.blk_last, a.num_blocks, tok_stride,
                                blk_stride, pc.head_off, lane);
        compute_chunk<T, D, G, CB, F8>(st, fa, q, a.scale_log2, tok_of(i), cur.n, is_mask(i), lane);
      }
    }

    // The next job's query and first chunk go out before this job's merge.
    const JobPlan pn = plan_job<S::kElemBytes, D, CB>(a, nxt, wave, nwaves);
    if (nxt.n > 0 && nxt.seq >= 0) {
      load_query<T, D, G, CB, F8>(a.query, nxt.seq, a.num_heads, nxt.kvh * g, g, lane, q);
      if (PF && pn.mine > 0)
        load_chunk<T, D, G, CB, F8>(fa, kc, vc, pn.bt_row, blk_of(0), pn.blk_last, a.num_blocks, tok_stride,
                                blk_stride, pn.head_off, lane);
    }

    // Sum this wave's partials over the 4 row groups (lanes l, l^16, l^32, l^48).
    st.l = rows_sum(st.l);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < S::kVec; ++e) st.acc[h][e] = rows_sum(st.acc[h][e]);
    if (lane < 16) {
      s_m[wave][lane] = st.m;
      s_l[wave][lane] = st.l;
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < S::kVec; ++e) s_acc[(wave * G + h) * D + lane * S::kVec + e] = st.acc[h][e];
    }
    __syncthreads();

    if (cur.seq >= 0) {
      // Merge the waves: weights 2^(m_w - M). A prefix-pass result joins as
      // one more part with l = 1, acc = its output and m = its lse in base 2.
      const int head0 = cur.kvh * g;
      for (int idx = threadIdx.x; idx < g * D; idx += blockDim.x) {
        const int h = idx / D;
        const int d = idx - h * D;
        const int64_t row = static_cast<int64_t>(cur.seq) * a.num_heads + head0 + h;
        float M = -__builtin_inff();
        for (int v = 0; v < nwaves; ++v) M = fmaxf(M, s_m[v][h]);
        float pm = -__builtin_inff();
        if (a.prefix_o != nullptr) {
          pm = a.prefix_lse[row] * kLog2e;
          M = fmaxf(M, pm);
        }
        float o = 0.f, L = 0.f;
        if (M != -__builtin_inff()) {
          for (int v = 0; v < nwaves; ++v) {
            const float wt = fast_exp2(s_m[v][h] - M);
            L = fmaf(wt, s_l[v][h], L);
            o = fmaf(wt, s_acc[(v * G + h) * D + d], o);
          }
          if (pm != -__builtin_inff()) {
            const float wt = fast_exp2(pm - M);
            L += wt;
            o = fmaf(wt, a.prefix_o[row * D + d], o);
          }
          o = o / L * a.v_scale;
        }
        const float lse = (M == -__builtin_inff()) ? -__builtin_inff() : (M + fast_log2(L)) * kLn2;
        store_elem<T>(static_cast<T*>(a.out) + row * D + d, o);
        if (a.lse_out != nullptr && d == 0) a.lse_out[row] = lse;
      }
    }
    __syncthreads();  // the next job rewrites the LDS partials

    id = id_next;
    cur = nxt;
    pc = pn;
    ++k;
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
  load_chunk<T, D, G, CB>(fa, kc, vc, bt_row(cur.seq), cur.b_lo, cur.b_hi - 1, a.num_blocks, tok_stride,
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
  // ahead of the arithmetic.
  auto advance = [&](Chunk<T, D, G, CB>& fcur, Chunk<T, D, G, CB>& fnext) -> bool {
    if (nx.x < 0) {
      compute(fcur);
      return false;
    }
    load_chunk<T, D, G, CB>(fnext, kc, vc, bt_row(nx.seq), nx.b_lo + nx.c * CB, nx.b_hi - 1, a.num_blocks,
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
// compute unit instead of a quarter of them. PA_MERGE_ROWS=1|2|4 overrides.
int merge_rows_per_block(int64_t rows) {
  if (const char* e = getenv("PA_MERGE_ROWS")) {
    const int v = atoi(e);
    if (v == 1 || v == 2 || v == 4) return v;
  }
  return rows <= 8 * static_cast<int64_t>(device_cus()) ? 1 : 4;
}

// Blocks per chunk (CB) and one-chunk register lookahead (PF), chosen per
// shape so a wave fits in 256 VGPRs without spilling (2 waves per SIMD).
template <typename T, int D, int G, bool F8 = false>
struct Policy {
  static constexpr int kElemBytes = F8 ? 1 : static_cast<int>(sizeof(T));
  static constexpr int kRegsPerBlock = D * kElemBytes / 8;  // K + V dwords per lane
  static constexpr int kAcc = G * D / 16;
  // FP8 blocks take half the registers; small groups use twice the blocks per
  // chunk (larger ones would spill the conversion temporaries).
  static constexpr int CB = (kRegsPerBlock <= 16 && G <= 2) ? 4 : (kRegsPerBlock <= 32 && G <= 4) ? 2 : 1;
  static constexpr bool PF = 2 * CB * kRegsPerBlock + kAcc <= 160;
};

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int next_pow2_group(int g) {
  int G = 1;
  while (G < g) G <<= 1;
  return G;
}

// Waves per workgroup forced through PA_DECODE_WAVES (1, 2, 4 or 8), else 0.
int waves_override() {
  static int w = [] {
    const char* e = getenv("PA_DECODE_WAVES");
    int v = e ? atoi(e) : 0;
    return (v == 1 || v == 2 || v == 4 || v == 8) ? v : 0;
  }();
  return w;
}


typedef void (*DecodeKernel)(DecodeArgs);

template <typename T, int D, int G, bool F8 = false>
DecodeKernel kernel_for() {
  using P = Policy<T, D, G, F8>;
  return paged_decode_kernel<T, D, G, P::CB, P::PF, F8>;
}

template <int D>
DecodeKernel pick_group_fp8(int G) {
  switch (G) {
    case 1: return kernel_for<bf16_t, D, 1, true>();
    case 2: return kernel_for<bf16_t, D, 2, true>();
    case 4: return kernel_for<bf16_t, D, 4, true>();
    case 8: return kernel_for<bf16_t, D, 8, true>();
    case 16: return kernel_for<bf16_t, D, 16, true>();
    default: return nullptr;
  }
}

template <typename T, int D>
DecodeKernel pick_group(int G) {
  switch (G) {
    case 1: return kernel_for<T, D, 1>();
    case 2: return kernel_for<T, D, 2>();
    case 4: return kernel_for<T, D, 4>();
    case 8: return kernel_for<T, D, 8>();
    case 16: return kernel_for<T, D, 16>();
    default: return nullptr;
  }
}

DecodeKernel pick_decode(int dtype, int D, int G) {
  if (dtype == PA_DTYPE_BF16) return D == 128 ? pick_group<bf16_t, 128>(G) : pick_group<bf16_t, 64>(G);
  return D == 128 ? pick_group<float, 128>(G) : pick_group<float, 64>(G);
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

// Which kernel serves a decode step: the tile kernel (the multi-query kernel
// with one token per sequence: P*V on the matrix cores, one workgroup per
// (sequence, kv head) handed out by the hardware in seq_order, with 8-wave
// workgroups when the grid is a single round) measured faster on every
// workload; the persistent kernel is kept as the alternative.
// PA_DECODE_KERNEL=persistent|tiles forces one (the tests run both).
bool decode_by_tiles(int group) {
  if (const char* e = getenv("PA_DECODE_KERNEL")) {
    if (e[0] == 'p') return false;
  }
  return group <= 16;
}

int launch_decode(DecodeArgs args, int num_seqs, int dtype, int head_size, hipStream_t stream,
                  bool fp8_cache = false) {
  const int G = next_pow2_group(args.group);
  DecodeKernel k = fp8_cache ? (head_size == 128 ? pick_group_fp8<128>(G) : pick_group_fp8<64>(G))
                             : pick_decode(dtype, head_size, G);
  if (!k) return PA_ERR_UNSUPPORTED;
  // Job ids padded to whole XCD rounds (a multiple of 8).
  const int64_t jobs = (static_cast<int64_t>(num_seqs) + 7) / 8 * 8 * args.num_kv_heads;
  if (jobs <= 0) return PA_OK;
  if (jobs > INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
  // Four waves per workgroup (two workgroups per CU), unless every workgroup
  // would get at most one job: then eight waves (one workgroup per CU) split
  // each job twice as finely, which narrows the spread of finishing times
  // (batch 64: 76 -> 71 us). The 16-head group fits 4 waves only.
  int W = waves_override();
  if (W == 0 || (W == 8 && G >= 16)) {
    W = 4;
    if (G < 16) {
      const int64_t resident4 = resident_groups(reinterpret_cast<const void*>(k), 4 * kWave,
                                                static_cast<size_t>(4) * G * head_size * sizeof(float));
      if (resident4 > 0 && jobs <= resident4) W = 8;
    }
  }
  const size_t lds = static_cast<size_t>(W) * G * head_size * sizeof(float);
  // Persistent grid: the workgroups that fit at once, a multiple of 8 (one
  // round over the XCDs), and no more than there are jobs.
  int64_t grid = resident_groups(reinterpret_cast<const void*>(k), W * kWave, lds);
  if (grid <= 0) return PA_ERR_HIP;
  if (grid >= 8) grid -= grid % 8;
  if (grid > jobs) grid = jobs;

  args.num_jobs = static_cast<int32_t>(jobs);
  hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(grid)), dim3(W * kWave), lds, stream, args);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
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
// per kv head), for groups above 16 and for groups of at most 4 when the
// batch has fewer (sequence, kv head) pairs than resident tile workgroups (2
// per CU): long contexts of a few sequences, where the pieces measured faster.
// (Larger groups keep the tiles: the piece kernel's per-lane accumulators
// spill registers from a group of 8 up.) PA_SPLIT_KERNEL=pieces|tiles
// overrides.
bool split_by_tiles(int group, int num_seqs, int num_kv_heads) {
  if (group > 16) return false;
  if (const char* e = getenv("PA_SPLIT_KERNEL")) {
    if (e[0] == 'p') return false;
    if (e[0] == 't') return true;
  }
  if (group > 4) return true;
  return static_cast<int64_t>(num_seqs) * num_kv_heads >= 2 * static_cast<int64_t>(device_cus());
}

// Partition length of the partition cut: k * P with k the largest factor
// that still leaves about three rounds of resident tile workgroups for the
// longest possible batch (num_seqs contexts of max_context_len tokens), so
// each workgroup streams long enough to amortise its start; at most the
// longest context. PA_SPLIT_PART_FACTOR=k overrides k.
int split_part_tokens(int num_seqs, int num_kv_heads, int max_context_len, int P) {
  const int64_t n_p = (static_cast<int64_t>(max_context_len) + P - 1) / P;
  if (n_p <= 1) return P;
  int64_t k = 0;
  if (const char* e = getenv("PA_SPLIT_PART_FACTOR")) k = atoi(e);
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
  if (decode_by_tiles(num_heads / num_kv_heads))
    return launch_decode_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                               num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale * kLog2e, 1.0f,
                               dtype, false, lse_out, seq_order, 0, nullptr, nullptr,
                               static_cast<hipStream_t>(stream));
  DecodeArgs args{};
  args.query = query;
  args.key_cache = key_cache;
  args.value_cache = value_cache;
  args.block_tables = block_tables;
  args.context_lens = context_lens;
  args.out = out;
  args.lse_out = lse_out;
  args.seq_order = seq_order;
  args.num_blocks = num_blocks;
  args.max_blocks = max_blocks_per_seq;
  args.num_seqs = num_seqs;
  args.num_heads = num_heads;
  args.num_kv_heads = num_kv_heads;
  args.group = num_heads / num_kv_heads;
  args.scale_log2 = scale * kLog2e;
  args.v_scale = 1.0f;
  return launch_decode(args, num_seqs, dtype, head_size, static_cast<hipStream_t>(stream));
}

extern "C" int pa_decode_uses_tiles(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                                    int32_t dtype, int32_t fp8_cache) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return -1;
  if (num_heads / num_kv_heads > 16 || (head_size != 64 && head_size != 128)) return -1;
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return -1;
  return decode_by_tiles(num_heads / num_kv_heads) ? 1 : 0;
}

extern "C" int32_t pa_decode_split_part_tokens(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                               int32_t max_context_len, int32_t partition_size) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return -1;
  if (max_context_len < 0 || partition_size <= 0 || partition_size % kBlockTokens != 0) return -1;
  if (!split_by_tiles(num_heads / num_kv_heads, num_seqs, num_kv_heads)) return 0;
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
  if (decode_by_tiles(num_heads / num_kv_heads))
    return launch_decode_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                               num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale * kLog2e, 1.0f,
                               dtype, false, lse_out, seq_order, prefix_blocks, part_o, part_lse, s);
  DecodeArgs args{};
  args.query = query;
  args.key_cache = key_cache;
  args.value_cache = value_cache;
  args.block_tables = block_tables;
  args.context_lens = context_lens;
  args.out = out;
  args.lse_out = lse_out;
  args.seq_order = seq_order;
  args.num_blocks = num_blocks;
  args.max_blocks = max_blocks_per_seq;
  args.num_seqs = num_seqs;
  args.num_heads = num_heads;
  args.num_kv_heads = num_kv_heads;
  args.group = num_heads / num_kv_heads;
  args.scale_log2 = scale * kLog2e;
  args.v_scale = 1.0f;
  args.skip_blocks = prefix_blocks;
  args.prefix_o = part_o;
  args.prefix_lse = part_lse;
  return launch_decode(args, num_seqs, dtype, head_size, s);
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
  if (decode_by_tiles(num_heads / num_kv_heads))
    return launch_decode_multi(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                               num_seqs, num_heads, num_kv_heads, head_size, num_blocks, scale * k_scale * kLog2e,
                               v_scale, dtype, true, lse_out, seq_order, 0, nullptr, nullptr,
                               static_cast<hipStream_t>(stream));
  DecodeArgs args{};
  args.query = query;
  args.key_cache = key_cache;
  args.value_cache = value_cache;
  args.block_tables = block_tables;
  args.context_lens = context_lens;
  args.out = out;
  args.lse_out = lse_out;
  args.seq_order = seq_order;
  args.num_blocks = num_blocks;
  args.max_blocks = max_blocks_per_seq;
  args.num_seqs = num_seqs;
  args.num_heads = num_heads;
  args.num_kv_heads = num_kv_heads;
  args.group = num_heads / num_kv_heads;
  // Keys are code values times k_scale: the scale folds into the scores'.
  args.scale_log2 = scale * k_scale * kLog2e;
  args.v_scale = v_scale;
  return launch_decode(args, num_seqs, dtype, head_size, static_cast<hipStream_t>(stream), true);
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

extern "C" int pa_decode_split(void* out, const void* query, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_size, int64_t num_blocks,
                               int32_t block_size, float scale, int32_t dtype, int32_t max_context_len,
                               int32_t partition_size, void* workspace, size_t workspace_bytes,
                               float* lse_out, void* stream) {
  int st = check_common(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                        num_seqs, num_heads, num_kv_heads, head_size, num_blocks, block_size, dtype);
  if (st != PA_OK) return st;
  if (partition_size <= 0 || partition_size % kBlockTokens != 0 || max_context_len < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  SplitLayout L;
  if (!split_layout(num_seqs, num_heads, head_size, max_context_len, partition_size, L)) return PA_ERR_UNSUPPORTED;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_INVALID_ARG;
  if (workspace_bytes < L.total) return PA_ERR_WORKSPACE;
  if ((static_cast<size_t>(num_seqs) + 1) * sizeof(int) > 64 * 1024) return PA_ERR_UNSUPPORTED;  // LDS prefix

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
  if (split_by_tiles(args.group, num_seqs, num_kv_heads)) {
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
