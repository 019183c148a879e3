// Host block manager: per-sequence block lists and token counts over the
// pool's free-block stack.  Host memory only.
//
//   growth per block   -- "KV Cache and Attention Mechanisms", section 2
//                         ("Zero-Waste Allocation"); "Paged KV-Cache Memory
//                         Management", "Memory Waste Analysis".
//   admission          -- "KV Cache and Attention Mechanisms", section 3.1
//                         ("Cache Block Pool").
//   free-block stack   -- "Paged KV-Cache Memory Management", "Python
//                         Implementation: Physical Block Pool".

#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "internal.h"

struct kv_block_manager {
  kv_pool* pool;   // null once the pool has been destroyed
  int max_blocks;
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t tokens = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;
  int64_t blocks_used = 0;
  int64_t tokens = 0;
};

namespace {

int64_t blocks_for(int64_t tokens, int block_size) {
  return (tokens + block_size - 1) / block_size;
}

// Validate a step and count the blocks it needs.  Negative = status.
int64_t step_need(const kv_block_manager* m, int n, const int64_t* ids, const int32_t* counts) {
  if (!m || !m->pool || n < 0) return PAGEDKV_ERR_INVALID_ARG;
  if (n == 0) return 0;
  if (!ids || !counts) return PAGEDKV_ERR_INVALID_ARG;
  std::unordered_set<int64_t> seen;
  seen.reserve((size_t)n * 2);
  int64_t need = 0;
  for (int i = 0; i < n; ++i) {
    const auto it = m->seqs.find(ids[i]);
    if (it == m->seqs.end() || counts[i] < 0 || !seen.insert(ids[i]).second)
      return PAGEDKV_ERR_INVALID_ARG;
    const int64_t tokens = it->second.tokens + counts[i];
    const int64_t after = blocks_for(tokens, m->pool->block_size);
    if (after > m->max_blocks || tokens > INT32_MAX) return PAGEDKV_ERR_INVALID_ARG;
    need += after - (int64_t)it->second.blocks.size();
  }
  return need;
}

void release_blocks(kv_block_manager* m, kv_block_manager::Seq& s) {
  for (const int32_t b : s.blocks) kv_pool_free_block(m->pool, b);   // logical order
  m->blocks_used -= (int64_t)s.blocks.size();
  m->tokens -= s.tokens;
}

}  // namespace

// The pool is going away: forget it (the manager's later calls fail).
void kv_manager_detach(kv_block_manager* m) { m->pool = nullptr; }

extern "C" {

int kv_manager_create(kv_block_manager_t** out, kv_pool_t* pool, int max_blocks_per_seq) {
  if (!out) return PAGEDKV_ERR_INVALID_ARG;
  *out = nullptr;
  if (!pool || max_blocks_per_seq < 1) return PAGEDKV_ERR_INVALID_ARG;
  kv_block_manager* m = new (std::nothrow) kv_block_manager;
  if (!m) return PAGEDKV_ERR_INVALID_ARG;
  m->pool = pool;
  m->max_blocks = max_blocks_per_seq;
  try {
    pool->managers.push_back(m);
  } catch (...) {
    delete m;
    return PAGEDKV_ERR_INVALID_ARG;
  }
  *out = m;
  return PAGEDKV_OK;
}

int kv_manager_destroy(kv_block_manager_t* mgr) {
  if (!mgr) return PAGEDKV_OK;
  if (mgr->pool) {
    for (auto& kv : mgr->seqs) release_blocks(mgr, kv.second);
    auto& list = mgr->pool->managers;
    for (size_t i = 0; i < list.size(); ++i)
      if (list[i] == mgr) {
        list[i] = list.back();
        list.pop_back();
        break;
      }
  }
  delete mgr;
  return PAGEDKV_OK;
}

int kv_manager_add_sequence(kv_block_manager_t* mgr, int64_t seq_id) {
  if (!mgr || !mgr->pool) return PAGEDKV_ERR_INVALID_ARG;
  try {
    if (!mgr->seqs.emplace(seq_id, kv_block_manager::Seq{}).second) return PAGEDKV_ERR_INVALID_ARG;
  } catch (...) {
    return PAGEDKV_ERR_INVALID_ARG;
  }
  return PAGEDKV_OK;
}

int64_t kv_manager_blocks_needed(const kv_block_manager_t* mgr, int n, const int64_t* seq_ids,
                                 const int32_t* counts) {
  try {
    return step_need(mgr, n, seq_ids, counts);
  } catch (...) {
    return PAGEDKV_ERR_INVALID_ARG;
  }
}

int kv_manager_reserve(kv_block_manager_t* mgr, int n, const int64_t* seq_ids,
                       const int32_t* counts, int32_t* start_positions) {
  int64_t need;
  try {
    need = step_need(mgr, n, seq_ids, counts);
  } catch (...) {
    return PAGEDKV_ERR_INVALID_ARG;
  }
  if (need < 0) return (int)need;
  if (need > (int64_t)mgr->pool->free_stack.size()) return PAGEDKV_ERR_OUT_OF_BLOCKS;
  const int bs = mgr->pool->block_size;
  // make room first, so that nothing below can throw once blocks move
  try {
    for (int i = 0; i < n; ++i) {
      kv_block_manager::Seq& s = mgr->seqs.find(seq_ids[i])->second;
      s.blocks.reserve((size_t)blocks_for(s.tokens + counts[i], bs));
    }
  } catch (...) {
    return PAGEDKV_ERR_INVALID_ARG;
  }
  for (int i = 0; i < n; ++i) {
    kv_block_manager::Seq& s = mgr->seqs.find(seq_ids[i])->second;
    const int64_t after = blocks_for(s.tokens + counts[i], bs);
    while ((int64_t)s.blocks.size() < after) {
      int32_t id = -1;
      kv_pool_alloc_block(mgr->pool, &id);   // cannot fail: need <= free blocks
      s.blocks.push_back(id);                // capacity: after <= max_blocks
      ++mgr->blocks_used;
    }
    if (start_positions) start_positions[i] = (int32_t)s.tokens;
    s.tokens += counts[i];
    mgr->tokens += counts[i];
  }
  return PAGEDKV_OK;
}

int kv_manager_release(kv_block_manager_t* mgr, int64_t seq_id) {
  if (!mgr || !mgr->pool) return PAGEDKV_ERR_INVALID_ARG;
  const auto it = mgr->seqs.find(seq_id);
  if (it == mgr->seqs.end()) return PAGEDKV_ERR_INVALID_ARG;
  release_blocks(mgr, it->second);
  mgr->seqs.erase(it);
  return PAGEDKV_OK;
}

int kv_manager_block_tables(const kv_block_manager_t* mgr, int n, const int64_t* seq_ids,
                            int32_t* tables, int32_t* context_lens) {
  if (!mgr || !mgr->pool || n < 0) return PAGEDKV_ERR_INVALID_ARG;
  if (n == 0) return PAGEDKV_OK;
  if (!seq_ids || !tables) return PAGEDKV_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (mgr->seqs.find(seq_ids[i]) == mgr->seqs.end()) return PAGEDKV_ERR_INVALID_ARG;
  const int mb = mgr->max_blocks;
  for (int i = 0; i < n; ++i) {
    const kv_block_manager::Seq& s = mgr->seqs.find(seq_ids[i])->second;
    int32_t* row = tables + (int64_t)i * mb;
    const int nb = (int)s.blocks.size();
    for (int j = 0; j < nb; ++j) row[j] = s.blocks[j];
    for (int j = nb; j < mb; ++j) row[j] = -1;
    if (context_lens) context_lens[i] = (int32_t)s.tokens;
  }
  return PAGEDKV_OK;
}

int kv_manager_stats(const kv_block_manager_t* mgr, kv_manager_stats_t* out) {
  if (!mgr || !mgr->pool || !out) return PAGEDKV_ERR_INVALID_ARG;
  out->sequences = (int64_t)mgr->seqs.size();
  out->blocks_total = mgr->pool->num_blocks;
  out->blocks_free = (int64_t)mgr->pool->free_stack.size();
  out->blocks_used = mgr->blocks_used;
  out->tokens = mgr->tokens;
  out->slots = mgr->blocks_used * mgr->pool->block_size;
  out->waste_slots = out->slots - out->tokens;
  out->waste_ratio = out->tokens ? (double)out->waste_slots / (double)out->tokens : 0.0;
  return PAGEDKV_OK;
}

}  // extern "C"
