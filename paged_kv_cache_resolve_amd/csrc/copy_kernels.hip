// Bit-exact copy kernels: KV append into the tail block, batched paged-KV
// gather into contiguous tensors, and the stand-alone block-table resolver.
//
//   append  -- "KV Cache and Attention Mechanisms", section 2 (blocks are
//              filled one token at a time as generation proceeds);
//              "Paged KV-Cache Memory Management", section "The Solution".
//   gather  -- "Paged KV-Cache Memory Management", section "Zero-Copy
//              Batched Attention Gather".
//   resolve -- "vllmini", section "PagedAttention Metaphor".
//
// All copies move 16-byte units (a pool row of head_dim elements is a
// whole number of units: head_dim is a multiple of 8 for bf16 and of 4 for
// fp32), so every load and store is a dwordx4.

#include "internal.h"

namespace pagedkv {
namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// One thread per 16-byte unit of the new K and V rows.
__global__ __launch_bounds__(256) void append_kernel(PoolGeom pool, int layer, int elem,
                                                     const char* __restrict__ k_new,
                                                     const char* __restrict__ v_new,
                                                     const int32_t* __restrict__ tables, int mb,
                                                     const int32_t* __restrict__ positions,
                                                     int batch) {
  const int units = pool.head_dim * elem / 16;          // per (b, g) row
  const int64_t total = (int64_t)batch * pool.kv_heads * 2 * units;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int u = (int)(i % units);
  int64_t r = i / units;
  const int kv = (int)(r & 1);
  r >>= 1;
  const int g = (int)(r % pool.kv_heads);
  const int b = (int)(r / pool.kv_heads);
  const int pos = positions[b];
  if (pos < 0) return;
  const int phys = tables[(int64_t)b * mb + pos / pool.block_size];
  const int64_t dst_elem = (int64_t)phys * pool.block_stride + kv * pool.kv_stride +
                           (int64_t)layer * pool.layer_stride + (int64_t)g * pool.head_stride +
                           (int64_t)(pos % pool.block_size) * pool.head_dim;
  const char* src = (kv ? v_new : k_new) + ((int64_t)b * pool.kv_heads + g) * pool.head_dim * elem;
  char* dst = const_cast<char*>(pool.base) + dst_elem * elem;
  reinterpret_cast<uint4*>(dst)[u] = reinterpret_cast<const uint4*>(src)[u];
}

// All-layer append: one thread per 16-byte unit of every layer's new K and V
// rows; k_new / v_new are [batch][layers][kv_heads][head_dim].
__global__ __launch_bounds__(256) void append_layers_kernel(PoolGeom pool, int layers, int elem,
                                                            const char* __restrict__ k_new,
                                                            const char* __restrict__ v_new,
                                                            const int32_t* __restrict__ tables,
                                                            int mb,
                                                            const int32_t* __restrict__ positions,
                                                            int batch) {
  const int units = pool.head_dim * elem / 16;
  const int64_t total = (int64_t)batch * layers * pool.kv_heads * 2 * units;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int u = (int)(i % units);
  int64_t r = i / units;
  const int kv = (int)(r & 1);
  r >>= 1;
  const int g = (int)(r % pool.kv_heads);
  r /= pool.kv_heads;
  const int layer = (int)(r % layers);
  const int b = (int)(r / layers);
  const int pos = positions[b];
  if (pos < 0) return;
  const int phys = tables[(int64_t)b * mb + pos / pool.block_size];
  const int64_t dst_elem = (int64_t)phys * pool.block_stride + kv * pool.kv_stride +
                           (int64_t)layer * pool.layer_stride + (int64_t)g * pool.head_stride +
                           (int64_t)(pos % pool.block_size) * pool.head_dim;
  const char* src = (kv ? v_new : k_new) +
                    (((int64_t)b * layers + layer) * pool.kv_heads + g) * pool.head_dim * elem;
  char* dst = const_cast<char*>(pool.base) + dst_elem * elem;
  reinterpret_cast<uint4*>(dst)[u] = reinterpret_cast<const uint4*>(src)[u];
}

// Multi-token append: one thread per 16-byte unit of every new row.  Rows
// offsets[b] .. offsets[b+1]-1 of k_new / v_new ([total][kv_heads][head_dim])
// belong to sequence b and go to positions starts[b], starts[b] + 1, ...
__global__ __launch_bounds__(256) void append_tokens_kernel(PoolGeom pool, int layer, int elem,
                                                            const char* __restrict__ k_new,
                                                            const char* __restrict__ v_new,
                                                            const int32_t* __restrict__ tables,
                                                            int mb,
                                                            const int32_t* __restrict__ starts,
                                                            const int32_t* __restrict__ offsets,
                                                            int batch, int64_t total_rows) {
  const int units = pool.head_dim * elem / 16;
  const int64_t total = total_rows * pool.kv_heads * 2 * units;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int u = (int)(i % units);
  int64_t r = i / units;
  const int kv = (int)(r & 1);
  r >>= 1;
  const int g = (int)(r % pool.kv_heads);
  const int64_t row = r / pool.kv_heads;
  // the sequence of this row: the largest b in [0, batch) with offsets[b] <= row
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= row) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int start = starts[b];
  if (start < 0) return;
  const int t = start + (int)(row - offsets[b]);
  const int phys = tables[(int64_t)b * mb + t / pool.block_size];
  const int64_t dst_elem = (int64_t)phys * pool.block_stride + kv * pool.kv_stride +
                           (int64_t)layer * pool.layer_stride + (int64_t)g * pool.head_stride +
                           (int64_t)(t % pool.block_size) * pool.head_dim;
  const char* src = (kv ? v_new : k_new) + (row * pool.kv_heads + g) * pool.head_dim * elem;
  char* dst = const_cast<char*>(pool.base) + dst_elem * elem;
  reinterpret_cast<uint4*>(dst)[u] = reinterpret_cast<const uint4*>(src)[u];
}

// Workgroup = 256 threads = (256 / units) tokens x units of one KV head.
// grid = (ceil(max_len / tokens_per_iter), kv_heads, batch); each workgroup
// walks kTokIters token tiles.
constexpr int kTokIters = 4;

__global__ __launch_bounds__(256) void gather_kernel(PoolGeom pool, int layer, int elem,
                                                     char* __restrict__ k_out,
                                                     char* __restrict__ v_out,
                                                     uint8_t* __restrict__ mask,
                                                     const int32_t* __restrict__ tables, int mb,
                                                     const int32_t* __restrict__ lens,
                                                     int max_len, int units_log2) {
  const int units = 1 << units_log2;
  const int u = threadIdx.x & (units - 1);
  const int tl = threadIdx.x >> units_log2;
  const int tiles = 256 >> units_log2;                  // tokens per iteration
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int T = lens[b];
  const int H = pool.kv_heads;
  const int64_t row_bytes = (int64_t)pool.head_dim * elem;   // = units * 16
  for (int it = 0; it < kTokIters; ++it) {
    const int t = (blockIdx.x * kTokIters + it) * tiles + tl;
    if (t >= max_len) return;
    u32x4_t kk = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (t < T) {
      const int phys = tables[(int64_t)b * mb + t / pool.block_size];
      const int64_t src_elem = (int64_t)phys * pool.block_stride + (int64_t)layer * pool.layer_stride +
                               (int64_t)g * pool.head_stride + (int64_t)(t % pool.block_size) * pool.head_dim;
      const u32x4_t* ks = reinterpret_cast<const u32x4_t*>(pool.base + src_elem * elem);
      const u32x4_t* vs = reinterpret_cast<const u32x4_t*>(pool.base + (src_elem + pool.kv_stride) * elem);
      // each pool row is read once: non-temporal loads keep it out of the caches
      kk = __builtin_nontemporal_load(ks + u);
      vv = __builtin_nontemporal_load(vs + u);
    }
    const int64_t dst = (((int64_t)b * max_len + t) * H + g) * row_bytes;
    __builtin_nontemporal_store(kk, reinterpret_cast<u32x4_t*>(k_out + dst) + u);
    __builtin_nontemporal_store(vv, reinterpret_cast<u32x4_t*>(v_out + dst) + u);
    if (g == 0 && u == 0) mask[(int64_t)b * max_len + t] = t < T ? 1 : 0;
  }
}

__global__ __launch_bounds__(256) void resolve_kernel(int64_t* __restrict__ slots,
                                                      const int32_t* __restrict__ tables, int mb,
                                                      const int32_t* __restrict__ lens,
                                                      int block_size, int max_len) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= max_len) return;
  const int T = lens[b];
  int64_t v = -1;
  if (t < T) v = (int64_t)tables[(int64_t)b * mb + t / block_size] * block_size + t % block_size;
  slots[(int64_t)b * max_len + t] = v;
}

}  // namespace

hipError_t launch_append(const kv_pool* pool, int layer, const void* k_new, const void* v_new,
                         const int32_t* tables, int mb, const int32_t* positions, int batch,
                         hipStream_t s) {
  const PoolGeom g = geom_of(pool);
  const int elem = elem_size(pool->dtype);
  const int64_t total = (int64_t)batch * pool->kv_heads * 2 * (pool->head_dim * elem / 16);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, g, layer, elem,
                     static_cast<const char*>(k_new), static_cast<const char*>(v_new), tables, mb,
                     positions, batch);
  return hipGetLastError();
}

hipError_t launch_append_layers(const kv_pool* pool, const void* k_new, const void* v_new,
                                const int32_t* tables, int mb, const int32_t* positions, int batch,
                                hipStream_t s) {
  const int elem = elem_size(pool->dtype);
  const int units = pool->head_dim * elem / 16;
  const int64_t total = (int64_t)batch * pool->layers * pool->kv_heads * 2 * units;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(append_layers_kernel, dim3((unsigned)blocks), dim3(256), 0, s, geom_of(pool),
                     pool->layers, elem, static_cast<const char*>(k_new),
                     static_cast<const char*>(v_new), tables, mb, positions, batch);
  return hipGetLastError();
}

hipError_t launch_append_tokens(const kv_pool* pool, int layer, const void* k_new,
                                const void* v_new, const int32_t* tables, int mb,
                                const int32_t* starts, const int32_t* offsets, int batch,
                                int64_t total_rows, hipStream_t s) {
  const int elem = elem_size(pool->dtype);
  const int units = pool->head_dim * elem / 16;
  const int64_t total = total_rows * pool->kv_heads * 2 * units;
  if (total == 0 || batch == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(append_tokens_kernel, dim3((unsigned)blocks), dim3(256), 0, s, geom_of(pool),
                     layer, elem, static_cast<const char*>(k_new), static_cast<const char*>(v_new),
                     tables, mb, starts, offsets, batch, total_rows);
  return hipGetLastError();
}

hipError_t launch_gather(void* k_out, void* v_out, uint8_t* mask, const kv_pool* pool, int layer,
                         const int32_t* tables, int mb, const int32_t* lens, int batch, int max_len,
                         hipStream_t s) {
  if (batch == 0 || max_len == 0) return hipSuccess;
  const PoolGeom g = geom_of(pool);
  const int elem = elem_size(pool->dtype);
  const int units = pool->head_dim * elem / 16;
  int units_log2 = 0;
  while ((1 << units_log2) < units) ++units_log2;
  if ((1 << units_log2) != units || units > 256) return hipErrorInvalidValue;
  const int tiles = 256 >> units_log2;
  const int per_block = tiles * kTokIters;
  const dim3 grid((max_len + per_block - 1) / per_block, pool->kv_heads, batch);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, s, g, layer, elem,
                     static_cast<char*>(k_out), static_cast<char*>(v_out), mask, tables, mb, lens,
                     max_len, units_log2);
  return hipGetLastError();
}

hipError_t launch_resolve(int64_t* slots, const int32_t* tables, int mb, const int32_t* lens,
                          int batch, int block_size, int max_len, hipStream_t s) {
  if (batch == 0 || max_len == 0) return hipSuccess;
  const dim3 grid((max_len + 255) / 256, batch);
  hipLaunchKernelGGL(resolve_kernel, grid, dim3(256), 0, s, slots, tables, mb, lens, block_size,
                     max_len);
  return hipGetLastError();
}

}  // namespace pagedkv
