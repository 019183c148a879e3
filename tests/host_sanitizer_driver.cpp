// Host-only exercise of the pool handle, free-block stack, block manager and
// argument validation under AddressSanitizer (no device work is issued).
#include <stdio.h>
#include <stdlib.h>
#include <vector>
#include "pagedkv.h"

int main() {
  void* fake = (void*)0x7F0000000000ull;
  int fails = 0;
  for (int round = 0; round < 50; ++round) {
    const int nb = 8 + round * 3, bs = 4 + (round % 3) * 4, mb = 6;
    kv_pool_t* pool = nullptr;
    if (kv_pool_create(&pool, nb, bs, 2, 2, 64, PAGEDKV_BF16, fake,
                       kv_pool_bytes(nb, bs, 2, 2, 64, PAGEDKV_BF16)) != 0) return 1;
    kv_block_manager_t* m = nullptr;
    if (kv_manager_create(&m, pool, mb) != 0) return 2;
    std::vector<int64_t> live;
    unsigned seed = 1234u + round;
    for (int step = 0; step < 2000; ++step) {
      seed = seed * 1103515245u + 12345u;
      const unsigned r = (seed >> 8) % 100;
      if (r < 15 || live.empty()) {
        const int64_t id = (int64_t)step * 7919 - 100000;
        if (kv_manager_add_sequence(m, id) == 0) live.push_back(id);
      } else if (r < 25) {
        const size_t i = (seed >> 3) % live.size();
        kv_manager_release(m, live[i]);
        live[i] = live.back();
        live.pop_back();
      } else {
        const int n = 1 + (int)((seed >> 5) % live.size());
        std::vector<int64_t> ids(live.begin(), live.begin() + n);
        std::vector<int32_t> counts(n), starts(n);
        for (int i = 0; i < n; ++i) counts[i] = (int32_t)((seed >> (i % 16)) % 9);
        kv_manager_blocks_needed(m, n, ids.data(), counts.data());
        kv_manager_reserve(m, n, ids.data(), counts.data(), starts.data());
        std::vector<int32_t> tables((size_t)n * mb), lens(n);
        if (kv_manager_block_tables(m, n, ids.data(), tables.data(), lens.data()) != 0) ++fails;
      }
      kv_manager_stats_t st;
      kv_manager_stats(m, &st);
      if (st.blocks_free + st.blocks_used != nb) ++fails;
    }
    // bad arguments
    kv_manager_reserve(m, -1, nullptr, nullptr, nullptr);
    kv_manager_block_tables(m, 3, nullptr, nullptr, nullptr);
    int32_t id;
    kv_pool_alloc_block(pool, &id);
    kv_pool_free_block(pool, -5);
    kv_pool_free_block(pool, nb + 10);
    if (round % 2) {            // destroy the pool first: the manager is detached
      kv_pool_destroy(pool);
      if (kv_manager_add_sequence(m, 1) == 0) ++fails;
      kv_manager_destroy(m);
    } else {
      kv_manager_destroy(m);
      kv_pool_destroy(pool);
    }
  }
  // entry-point validation without a GPU
  kv_pool_t* pool = nullptr;
  kv_pool_create(&pool, 8, 16, 2, 2, 64, PAGEDKV_BF16, fake, kv_pool_bytes(8, 16, 2, 2, 64, PAGEDKV_BF16));
  if (kv_append(pool, 5, fake, fake, (int32_t*)fake, 4, (int32_t*)fake, 4, nullptr) != PAGEDKV_ERR_INVALID_ARG) ++fails;
  if (paged_attention_decode(fake, fake, pool, 0, (int32_t*)fake, 4, (int32_t*)fake, 4, 7, 0.1f, fake, 1 << 20, 0u, nullptr) != PAGEDKV_ERR_INVALID_ARG) ++fails;
  kv_pool_destroy(pool);
  printf("host checks done, %d failures\n", fails);
  return fails ? 3 : 0;
}
