// Host-side KV block pool and step-input builder (see pa_pool.h).
//
// The pool keeps the free list as a stack (the pages hand out the block at the
// end of the list and put released blocks back there) and one reference count
// per physical block, so every operation is O(blocks touched) with no search
// (llm-stack-book 7.3 "vLLM: Architecture, PagedAttention & Internals",
// sections "The free list and the block table" and "Copy-on-write for shared
// blocks"). Every entry point checks its arguments and the pool's state in full
// before it changes anything.
#include <stdint.h>

#include <algorithm>
#include <limits>
#include <new>
#include <vector>

#include "pa.h"
#include "pa_pool.h"

struct pa_pool {
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refs;        // holders per block; 0 = on the free list
};

namespace {

bool valid_block(const pa_pool* p, int32_t b) {
  return b >= 0 && static_cast<size_t>(b) < p->refs.size();
}

int64_t blocks_for(int64_t tokens, int32_t block_size) {
  return tokens <= 0 ? 0 : (tokens + block_size - 1) / block_size;
}

int32_t take(pa_pool* p) {
  const int32_t b = p->free_stack.back();
  p->free_stack.pop_back();
  p->refs[b] = 1;
  return b;
}

// True when every id is a held block.
bool all_held(const pa_pool* p, const int32_t* blocks, int32_t n) {
  for (int32_t i = 0; i < n; ++i)
    if (!valid_block(p, blocks[i]) || p->refs[blocks[i]] <= 0) return false;
  return true;
}

}  // namespace

extern "C" int pa_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                              pa_pool** out) {
  if (out == nullptr || num_blocks < 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  pa_pool* p = new (std::nothrow) pa_pool;
  if (p == nullptr) return PA_ERR_INVALID_ARG;
  p->block_size = block_size;
  p->refs.assign(static_cast<size_t>(num_blocks), 0);
  p->free_stack.resize(static_cast<size_t>(num_blocks));
  if (free_order == nullptr) {
    for (int32_t i = 0; i < num_blocks; ++i) p->free_stack[i] = i;
  } else {
    std::vector<char> seen(static_cast<size_t>(num_blocks), 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return PA_ERR_INVALID_ARG;
      }
      seen[b] = 1;
      p->free_stack[i] = b;
    }
  }
  *out = p;
  return PA_OK;
}

extern "C" void pa_pool_destroy(pa_pool* pool) { delete pool; }

extern "C" int32_t pa_pool_num_free(const pa_pool* pool) {
  return pool == nullptr ? -1 : static_cast<int32_t>(pool->free_stack.size());
}

extern "C" int32_t pa_pool_ref_count(const pa_pool* pool, int32_t block) {
  if (pool == nullptr || !valid_block(pool, block)) return -1;
  return pool->refs[block];
}

extern "C" int64_t pa_pool_blocks_for(const pa_pool* pool, int64_t num_tokens) {
  return pool == nullptr ? -1 : blocks_for(num_tokens, pool->block_size);
}

extern "C" int pa_pool_allocate(pa_pool* pool, int64_t num_tokens, int32_t* table, int32_t capacity,
                                int32_t* num_blocks) {
  if (pool == nullptr || num_blocks == nullptr || capacity < 0 || num_tokens < 0) return PA_ERR_INVALID_ARG;
  const int64_t n = blocks_for(num_tokens, pool->block_size);
  if (n > capacity || (n > 0 && table == nullptr)) return PA_ERR_INVALID_ARG;
  if (n > static_cast<int64_t>(pool->free_stack.size())) return PA_ERR_NO_BLOCKS;
  for (int64_t i = 0; i < n; ++i) table[i] = take(pool);
  *num_blocks = static_cast<int32_t>(n);
  return PA_OK;
}

extern "C" int pa_pool_append_slot(pa_pool* pool, int32_t* table, int32_t* table_len, int32_t capacity,
                                   int64_t cur_len, int32_t* taken) {
  if (pool == nullptr || table_len == nullptr || taken == nullptr || cur_len < 0 || *table_len < 0 ||
      *table_len > capacity)
    return PA_ERR_INVALID_ARG;
  const int64_t need = cur_len / pool->block_size + 1;  // blocks covering position cur_len
  const int64_t have = *table_len;
  *taken = -1;
  if (have >= need) return PA_OK;
  if (need > capacity || table == nullptr) return PA_ERR_INVALID_ARG;
  if (need - have > static_cast<int64_t>(pool->free_stack.size())) return PA_ERR_NO_BLOCKS;
  for (int64_t i = have; i < need; ++i) table[i] = take(pool);
  *table_len = static_cast<int32_t>(need);
  *taken = table[need - 1];
  return PA_OK;
}

extern "C" int pa_pool_share(pa_pool* pool, const int32_t* blocks, int32_t n) {
  if (pool == nullptr || n < 0 || (n > 0 && blocks == nullptr)) return PA_ERR_INVALID_ARG;
  if (!all_held(pool, blocks, n)) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    if (pool->refs[blocks[i]] == std::numeric_limits<int32_t>::max()) return PA_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) ++pool->refs[blocks[i]];
  return PA_OK;
}

extern "C" int pa_pool_release(pa_pool* pool, const int32_t* blocks, int32_t n) {
  if (pool == nullptr || n < 0 || (n > 0 && blocks == nullptr)) return PA_ERR_INVALID_ARG;
  if (!all_held(pool, blocks, n)) return PA_ERR_INVALID_ARG;
  // A block listed more often than it has holders would go negative: check
  // the multiset against the counts before touching anything.
  std::vector<int32_t> sorted(blocks, blocks + n);
  std::sort(sorted.begin(), sorted.end());
  for (size_t i = 0; i < sorted.size();) {
    size_t j = i;
    while (j < sorted.size() && sorted[j] == sorted[i]) ++j;
    if (static_cast<int64_t>(j - i) > pool->refs[sorted[i]]) return PA_ERR_INVALID_ARG;
    i = j;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    if (--pool->refs[b] == 0) pool->free_stack.push_back(b);
  }
  return PA_OK;
}

extern "C" int pa_pool_make_writable(pa_pool* pool, int32_t* table, int32_t table_len, int32_t idx,
                                     int32_t* src, int32_t* dst) {
  if (pool == nullptr || table == nullptr || src == nullptr || dst == nullptr || idx < 0 || idx >= table_len)
    return PA_ERR_INVALID_ARG;
  const int32_t b = table[idx];
  if (!valid_block(pool, b) || pool->refs[b] <= 0) return PA_ERR_INVALID_ARG;
  *src = *dst = -1;
  if (pool->refs[b] == 1) return PA_OK;
  if (pool->free_stack.empty()) return PA_ERR_NO_BLOCKS;
  const int32_t fresh = take(pool);
  --pool->refs[b];
  table[idx] = fresh;
  *src = b;
  *dst = fresh;
  return PA_OK;
}

extern "C" int pa_prepare_step(int32_t num_seqs, const int32_t* tables, const int64_t* table_offsets,
                               const int64_t* num_computed, const int64_t* num_new, int32_t block_size,
                               int32_t max_blocks, int64_t* slot_mapping, int64_t* positions,
                               int32_t* block_tables, int32_t* context_lens, int64_t token_capacity,
                               int64_t* num_tokens) {
  if (num_seqs < 0 || block_size <= 0 || max_blocks < 0 || token_capacity < 0 || num_tokens == nullptr)
    return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (table_offsets == nullptr || num_computed == nullptr || num_new == nullptr ||
                       block_tables == nullptr || context_lens == nullptr))
    return PA_ERR_INVALID_ARG;
  // Validate everything first.
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t len = table_offsets[i + 1] - table_offsets[i];
    if (table_offsets[i] < 0 || len < 0 || len > max_blocks) return PA_ERR_INVALID_ARG;
    if (len > 0 && tables == nullptr) return PA_ERR_INVALID_ARG;
    if (num_computed[i] < 0 || num_new[i] < 0) return PA_ERR_INVALID_ARG;
    const int64_t end = num_computed[i] + num_new[i];
    if (end > std::numeric_limits<int32_t>::max()) return PA_ERR_INVALID_ARG;
    if (num_new[i] > 0 && blocks_for(end, block_size) > len) return PA_ERR_INVALID_ARG;
    total += num_new[i];
  }
  if (total > token_capacity || (total > 0 && (slot_mapping == nullptr || positions == nullptr)))
    return PA_ERR_INVALID_ARG;
  int64_t t = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t* table = tables + table_offsets[i];
    const int64_t len = table_offsets[i + 1] - table_offsets[i];
    for (int64_t p = num_computed[i]; p < num_computed[i] + num_new[i]; ++p, ++t) {
      positions[t] = p;
      slot_mapping[t] = static_cast<int64_t>(table[p / block_size]) * block_size + p % block_size;
    }
    int32_t* row = block_tables + static_cast<int64_t>(i) * max_blocks;
    for (int64_t j = 0; j < max_blocks; ++j) row[j] = j < len ? table[j] : -1;
    context_lens[i] = static_cast<int32_t>(num_computed[i] + num_new[i]);
  }
  *num_tokens = total;
  return PA_OK;
}
