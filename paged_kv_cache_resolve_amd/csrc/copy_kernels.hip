// Bit-exact copy kernels: KV appends (one token, one token for every layer,
// several tokens of a prompt), batched paged-KV gather into contiguous
// tensors, and the stand-alone block-table resolver.
//
//   append  -- "KV Cache and Attention Mechanisms", section 2 (blocks are
//              filled one token at a time as generation proceeds; a prompt
//              fills whole blocks and only the last is partly filled);
//              "Paged KV-Cache Memory Management", section "The Solution"
//              (a block holds its tokens' K and V for all layers).
//   gather  -- "Paged KV-Cache Memory Management", section "Zero-Copy
//              Batched Attention Gather".
//   resolve -- "vllmini", section "PagedAttention Metaphor".
//
// All copies move 16-byte units (a pool row of head_dim elements is a
// whole number of units: head_dim is a multiple of 8 for bf16 and fp16 and
// of 4 for fp32), so every load and store is a dwordx4.

#include "internal.h"

namespace pagedkv {
namespace {

// Appends.  A "row" is what one sequence writes at one logical position:
// its new K and V for `nl` consecutive layers starting at `layer0`, every
// KV head.  The source holds rows as k[row][nl][kv_heads][head_dim] (and the
// same for v).  Three callers share the kernel:
//   single token   row b -> (sequence b, position pos[b]), nl = 1;
//   all layers     row b -> (sequence b, position pos[b]), nl = layers;
//   several tokens row r -> (sequence b with off[b] <= r < off[b+1],
//                            position start[b] + r - off[b]), nl = 1.
// A row whose position is negative is skipped.
//
// Each workgroup owns 256 * VPT consecutive 16-byte units of the launch
// piece ([kv][layer][head][unit] inside a row).  It first issues all its
// source loads (VPT per thread, so that enough bytes are in flight to cover
// HBM latency), then resolves each of its rows once -- sequence, position,
// block-table entry -- into a pool offset in LDS, then stores.  All per-unit
// index arithmetic is 32-bit: the host splits launches so that one piece
// holds fewer than 2^31 units.  Large launches take VPT = 8; small ones take
// fewer units per thread so that the grid still spreads over every CU.
constexpr int kAppendMaxVpt = 8;

struct AppendArgs {
  PoolGeom pool;
  const uint4* k;
  const uint4* v;
  const int32_t* tables;
  const int32_t* pos;       // positions[batch], or start positions
  const int32_t* offsets;   // row offsets[batch + 1] (several-token form only)
  int mb;
  int batch;
  int layer0;
  int elem;
  uint32_t units;           // 16-byte units per (layer, head) row of head_dim
  uint32_t hu;              // units per (row, K or V) = nl * kv_heads * units
  uint32_t lhu;             // units per layer of a row = kv_heads * units
  int row0;                 // first row of this launch piece
  uint32_t piece_units;     // rows_in_piece * 2 * hu
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <bool TOKENS, int VPT>
__global__ __launch_bounds__(256) void append_rows_kernel(AppendArgs a) {
  constexpr uint32_t kUnits = 256 * VPT;
  __shared__ int64_t dst_row[kUnits / 2 + 2];   // element offset, -1 = skip (a row has >= 2 units)
  const uint32_t j0 = blockIdx.x * kUnits;
  const uint32_t j1 = min(j0 + kUnits, a.piece_units);
  const uint32_t w = 2 * a.hu;                  // units per row
  const uint32_t rl0 = j0 / w;

  uint4 val[VPT];
  uint32_t row_l[VPT], kv[VPT], rem[VPT];
#pragma unroll
  for (int x = 0; x < VPT; ++x) {
    const uint32_t j = j0 + x * 256 + threadIdx.x;
    const uint32_t q = j / a.hu;                // 2 * row + kv
    row_l[x] = q >> 1;
    kv[x] = q & 1;
    rem[x] = j - q * a.hu;
    if (j < j1) {
      const uint4* src = (kv[x] ? a.v : a.k) + (size_t)(a.row0 + row_l[x]) * a.hu + rem[x];
      val[x] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                             reinterpret_cast<const u32x4_t*>(src)));
    }
  }

  // one thread per row of this workgroup: sequence, position, block
  const uint32_t nrows = (j1 - 1) / w - rl0 + 1;
  for (uint32_t k = threadIdx.x; k < nrows; k += 256) {
    const int row = a.row0 + (int)(rl0 + k);
    int b, t;
    if (TOKENS) {
      // the last b with offsets[b] <= row
      int lo = 0, hi = a.batch;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.offsets[mid] <= row) lo = mid; else hi = mid;
      }
      b = lo;
      const int start = a.pos[b];
      t = start < 0 ? -1 : start + (row - a.offsets[b]);
    } else {
      b = row;
      t = a.pos[b];
    }
    int64_t d = -1;
    if (t >= 0) {
      const int phys = a.tables[(int64_t)b * a.mb + t / a.pool.block_size];
      d = (int64_t)phys * a.pool.block_stride + (int64_t)a.layer0 * a.pool.layer_stride +
          (int64_t)(t % a.pool.block_size) * a.pool.head_dim;
    }
    dst_row[k] = d;
  }
  __syncthreads();

  char* base = const_cast<char*>(a.pool.base);
#pragma unroll
  for (int x = 0; x < VPT; ++x) {
    const uint32_t j = j0 + x * 256 + threadIdx.x;
    if (j >= j1) continue;
    const int64_t d = dst_row[row_l[x] - rl0];
    if (d < 0) continue;
    const uint32_t l = rem[x] / a.lhu;
    const uint32_t r2 = rem[x] - l * a.lhu;
    const uint32_t g = r2 / a.units;
    const uint32_t u = r2 - g * a.units;
    const int64_t e = d + kv[x] * a.pool.kv_stride + (int64_t)l * a.pool.layer_stride +
                      (int64_t)g * a.pool.head_stride;
    reinterpret_cast<uint4*>(base + e * a.elem)[u] = val[x];
  }
}

// Workgroup = 256 threads = floor(256 / units) tokens x units (16-byte row
// pieces) of one KV head; threads past the last whole token idle (rows of
// 12 units, head_dim 96 in bf16, leave 4 of 256).  grid = (ceil(max_len /
// tokens_per_iter), kv_heads, batch); each workgroup walks kTokIters token
// tiles.
constexpr int kTokIters = 4;

__global__ __launch_bounds__(256) void gather_kernel(PoolGeom pool, int layer, int elem,
                                                     char* __restrict__ k_out,
                                                     char* __restrict__ v_out,
                                                     uint8_t* __restrict__ mask,
                                                     const int32_t* __restrict__ tables, int mb,
                                                     const int32_t* __restrict__ lens,
                                                     int max_len, int units) {
  const int tiles = 256 / units;                        // tokens per iteration
  if ((int)threadIdx.x >= tiles * units) return;
  const int tl = threadIdx.x / units;
  const int u = threadIdx.x - tl * units;
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

namespace {

// Launch the rows [0, rows) in pieces of fewer than 2^31 units.
template <bool TOKENS>
hipError_t launch_rows(const kv_pool* pool, int layer0, int nl, const void* k_new,
                       const void* v_new, const int32_t* tables, int mb, const int32_t* pos,
                       const int32_t* offsets, int batch, int rows, hipStream_t s) {
  AppendArgs a;
  a.pool = geom_of(pool);
  a.k = static_cast<const uint4*>(k_new);
  a.v = static_cast<const uint4*>(v_new);
  a.tables = tables;
  a.pos = pos;
  a.offsets = offsets;
  a.mb = mb;
  a.batch = batch;
  a.layer0 = layer0;
  a.elem = elem_size(pool->dtype);
  a.units = (uint32_t)(pool->head_dim * a.elem / 16);
  a.lhu = (uint32_t)pool->kv_heads * a.units;
  a.hu = (uint32_t)nl * a.lhu;
  const int64_t w = 2 * (int64_t)a.hu;
  const int64_t rows_per_piece = ((int64_t)1 << 31) / w - 1;
  if (rows_per_piece < 1) return hipErrorInvalidValue;
  for (int64_t r0 = 0; r0 < rows; r0 += rows_per_piece) {
    const int64_t n = rows - r0 < rows_per_piece ? rows - r0 : rows_per_piece;
    a.row0 = (int)r0;
    a.piece_units = (uint32_t)(n * w);
    // the most units per thread that still gives >= 8 workgroups per CU
    const uint32_t want = 8u * (uint32_t)device_cus();
    int vpt = kAppendMaxVpt;
    while (vpt > 1 && (a.piece_units + 256u * vpt - 1) / (256u * vpt) < want) vpt >>= 1;
    const uint32_t blocks = (a.piece_units + 256u * vpt - 1) / (256u * vpt);
    switch (vpt) {
      case 8: hipLaunchKernelGGL((append_rows_kernel<TOKENS, 8>), dim3(blocks), dim3(256), 0, s, a); break;
      case 4: hipLaunchKernelGGL((append_rows_kernel<TOKENS, 4>), dim3(blocks), dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL((append_rows_kernel<TOKENS, 2>), dim3(blocks), dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((append_rows_kernel<TOKENS, 1>), dim3(blocks), dim3(256), 0, s, a); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_append(const kv_pool* pool, int layer, const void* k_new, const void* v_new,
                         const int32_t* tables, int mb, const int32_t* positions, int batch,
                         hipStream_t s) {
  if (batch == 0) return hipSuccess;
  return launch_rows<false>(pool, layer, 1, k_new, v_new, tables, mb, positions, nullptr, batch,
                            batch, s);
}

hipError_t launch_append_layers(const kv_pool* pool, const void* k_new, const void* v_new,
                                const int32_t* tables, int mb, const int32_t* positions, int batch,
                                hipStream_t s) {
  if (batch == 0) return hipSuccess;
  return launch_rows<false>(pool, 0, pool->layers, k_new, v_new, tables, mb, positions, nullptr,
                            batch, batch, s);
}

hipError_t launch_append_tokens(const kv_pool* pool, int layer, const void* k_new,
                                const void* v_new, const int32_t* tables, int mb,
                                const int32_t* starts, const int32_t* offsets, int batch,
                                int64_t total_rows, hipStream_t s) {
  if (batch == 0 || total_rows == 0) return hipSuccess;
  return launch_rows<true>(pool, layer, 1, k_new, v_new, tables, mb, starts, offsets, batch,
                           (int)total_rows, s);
}

hipError_t launch_gather(void* k_out, void* v_out, uint8_t* mask, const kv_pool* pool, int layer,
                         const int32_t* tables, int mb, const int32_t* lens, int batch, int max_len,
                         hipStream_t s) {
  if (batch == 0 || max_len == 0) return hipSuccess;
  const PoolGeom g = geom_of(pool);
  const int elem = elem_size(pool->dtype);
  const int units = pool->head_dim * elem / 16;
  if (units < 1 || units > 256 || units * 16 != pool->head_dim * elem) return hipErrorInvalidValue;
  const int tiles = 256 / units;
  const int per_block = tiles * kTokIters;
  const dim3 grid((max_len + per_block - 1) / per_block, pool->kv_heads, batch);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, s, g, layer, elem,
                     static_cast<char*>(k_out), static_cast<char*>(v_out), mask, tables, mb, lens,
                     max_len, units);
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
