// Internal declarations shared by the host entry points and the kernel
// launchers of libpagedkv.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "pagedkv.h"

struct kv_pool {
  int num_blocks;
  int block_size;
  int layers;
  int kv_heads;
  int head_dim;
  pagedkv_dtype_t dtype;
  char* base;          // device address of element [0][0][0][0][0][0]
  size_t bytes;
  std::vector<int32_t> free_stack;   // top = back()
  std::vector<uint8_t> is_free;
  std::vector<kv_block_manager*> managers;   // detached when the pool is destroyed
};

// Called by kv_pool_destroy for every manager still attached to the pool.
void kv_manager_detach(kv_block_manager* m);

namespace pagedkv {

// Geometry of the pool passed to kernels by value.  Strides in elements.
struct PoolGeom {
  const char* base;
  int64_t block_stride;  // 2 * layers * kv_heads * block_size * head_dim
  int64_t kv_stride;     // layers * kv_heads * block_size * head_dim
  int64_t layer_stride;  // kv_heads * block_size * head_dim
  int64_t head_stride;   // block_size * head_dim
  int block_size;
  int head_dim;
  int kv_heads;
  int num_blocks;
};

inline PoolGeom geom_of(const kv_pool* p) {
  PoolGeom g;
  g.base = p->base;
  g.head_stride = (int64_t)p->block_size * p->head_dim;
  g.layer_stride = g.head_stride * p->kv_heads;
  g.kv_stride = g.layer_stride * p->layers;
  g.block_stride = g.kv_stride * 2;
  g.block_size = p->block_size;
  g.head_dim = p->head_dim;
  g.kv_heads = p->kv_heads;
  g.num_blocks = p->num_blocks;
  return g;
}

inline int elem_size(pagedkv_dtype_t t) { return t == PAGEDKV_F32 ? 4 : 2; }

// ---------------------------------------------------------------------------
// Decode work split.
//
// A "chunk" is CT consecutive tokens of one sequence; sequence b has
// n_b = ceil(T_b / CT) chunks, and the sequences' chunks laid end to end form
// a chunk space of C = sum_b n_b entries.  Wavefronts come in head groups:
// wavefront w serves KV head w % kv_heads for unit w / kv_heads, and unit u
// takes the contiguous, equal-sized range [u*C/U_eff, (u+1)*C/U_eff) of the
// chunk space.  The kv_heads wavefronts of a unit therefore stream the same
// blocks at the same time, and since the pool stores the heads of a block
// side by side, HBM sees long contiguous runs.  A wavefront that sees a
// whole (sequence, head) pair writes the output directly; otherwise it
// leaves a partial (max, sum, unnormalised output) in the workspace slot
// (b + u) * kv_heads + g, and the merge kernel combines the partials of
// every pair that was split between units.
// ---------------------------------------------------------------------------
// Unsigned division by a divisor d >= 1 fixed for a launch, as a
// multiply-high, an add and a shift (the round-up method:
// s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1, n / d =
// (mulhi(n, m) + n) >> s), exact for every 0 <= n < 2^31.  The kernels use
// it for the block size and the virtual KV head count, where the
// compiler's expansion of a division by a run-time value costs some twenty
// scalar instructions, which the wavefronts of a CU issue one at a time.
struct FastDiv {
  uint32_t m;
  uint32_t s;
};
inline FastDiv make_fast_div(uint32_t d) {
  uint32_t s = 0;
  while (((uint64_t)1 << s) < d) ++s;
  const uint64_t m = (((uint64_t)1 << 32) * (((uint64_t)1 << s) - d)) / d + 1;
  return FastDiv{(uint32_t)m, s};
}

struct DecodeParams {
  PoolGeom pool;
  const void* q;
  void* out;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t* ws_prefix;     // [batch + 1]: prefix sums of n_b (written by pass 1)
  float* ws_ml;           // [slots][G][2]: running max (log2 units) and sum
  float* ws_o;            // [slots][G][D]: unnormalised partial outputs
  int layer;
  int max_blocks_per_seq;
  int batch;
  int num_q_heads;
  int group;              // G = num_q_heads / kv_heads
  float scale_log2;       // scale * log2(e)
  int units;              // units (head groups of wavefronts) launched; the
                          // number that receives work is derived on device
  int min_chunks;         // minimum chunks per unit
  pagedkv_dtype_t dtype;  // element type of pool, q and out
  // Fused append (all null for a plain decode): the new token of sequence b
  // sits at position positions[b] (negative = none).  Pass 1 reads its K/V
  // rows from k_new / v_new ([batch][kv_heads][head_dim]) instead of the
  // pool, and the merge pass writes them into the pool afterwards.
  const void* k_new;
  const void* v_new;
  const int32_t* positions;
  // More query heads per KV head than one wavefront serves (16, or 32 for
  // the two-column-group MFMA stream): each KV head is served as qsplit
  // virtual KV heads (vheads = kv_heads * qsplit) of at most `group`
  // consecutive query heads each (vhead_rows in decode_split.h).  Work
  // split, q/out rows and partial slots use the virtual head; pool
  // addressing uses virtual / qsplit.  kv_group = num_q_heads / kv_heads.
  int vheads;
  int qsplit;
  int kv_group;
  // Dense decode (null for the paged forms): K and V as [batch][dense_len]
  // [kv_heads][head_dim], token t of sequence b attended where mask[b][t] != 0.
  const void* k_dense;
  const void* v_dense;
  const uint8_t* mask;
  int dense_len;
  // In: non-zero lets small batches run as one workgroup per (sequence,
  // virtual KV head) pair, which merges its own pieces.  Out (set by the
  // pass-1 launcher): non-zero if that kernel ran, so no merge pass follows.
  int pair_mode;
  // Set by the pass-1 launcher: division by pool.block_size and by vheads.
  FastDiv bs_div;
  FastDiv vh_div;
};

constexpr int kMaxWaves = 8192;          // upper bound on wavefronts (256 CUs x 32)
constexpr int kMaxGroup = 16;            // query heads per MFMA column group / VALU wavefront
constexpr int kDecodeWgPerCu = 1;        // decode workgroups (4 wavefronts) per CU
constexpr int kGenericChunk = 64;        // tokens per chunk, VALU kernel
constexpr int kMaxBatchLds = 16384;      // sequences whose prefix fits in LDS

// How the query heads of one KV head are spread over virtual KV heads of at
// most max_group query heads each (api.cpp).
struct HeadSplit {
  int qsplit;   // virtual heads per KV head
  int group;    // query heads per virtual head, at most (slot stride)
  int vheads;   // kv_heads * qsplit
};
HeadSplit head_split(int kv_heads, int group, int max_group);

size_t decode_workspace_bytes(int batch, int kv_heads, int group, int head_dim);
void decode_workspace_carve(void* ws, int batch, int kv_heads, int group,
                            int head_dim, int32_t** prefix, float** ml,
                            float** o);

// Launchers (return a hipError_t-derived status via hipGetLastError).
hipError_t launch_append(const kv_pool* pool, int layer, const void* k_new,
                         const void* v_new, const int32_t* tables, int mb,
                         const int32_t* positions, int batch, hipStream_t s);
hipError_t launch_append_layers(const kv_pool* pool, const void* k_new, const void* v_new,
                                const int32_t* tables, int mb, const int32_t* positions, int batch,
                                hipStream_t s);
hipError_t launch_append_tokens(const kv_pool* pool, int layer, const void* k_new,
                                const void* v_new, const int32_t* tables, int mb,
                                const int32_t* starts, const int32_t* offsets, int batch,
                                int64_t total_rows, hipStream_t s);
hipError_t launch_gather(void* k_out, void* v_out, uint8_t* mask,
                         const kv_pool* pool, int layer, const int32_t* tables,
                         int mb, const int32_t* lens, int batch, int max_len,
                         hipStream_t s);
hipError_t launch_resolve(int64_t* slots, const int32_t* tables, int mb,
                          const int32_t* lens, int batch, int block_size,
                          int max_len, hipStream_t s);

// Workgroups the device holds at once for kernel `fn` (cached per device).
hipError_t resident_workgroups(const void* fn, int threads, size_t lds, int* out);
// Decode pass-1 workgroups to launch: kDecodeWgPerCu per CU (a build with
// -DPAGEDKV_LAUNCH_SWEEP takes the count from PAGEDKV_DECODE_WG_PER_CU, for
// launch-shape sweeps), never more than `resident`.
int decode_workgroups(int resident);
// Compute units of the current device (0 if the runtime cannot tell).
int device_cus();

// Decode pass 1 variants and pass 2.  The *_supported predicates say which
// shapes each pass-1 kernel handles.
bool mfma_supported(const kv_pool* pool, int group);
int mfma_max_group(const kv_pool* pool);
bool generic_supported(const kv_pool* pool, int group);
hipError_t launch_decode_mfma(DecodeParams& p, hipStream_t s);
hipError_t launch_decode_generic(DecodeParams& p, hipStream_t s);
hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t s);

}  // namespace pagedkv
