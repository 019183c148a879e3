// extern "C" entry points of libpagedkv: argument validation, the host
// free-block stack, workspace layout and kernel dispatch.

#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>

#include "internal.h"

using namespace pagedkv;

namespace {

bool valid_dtype(pagedkv_dtype_t t) {
  return t == PAGEDKV_F32 || t == PAGEDKV_BF16 || t == PAGEDKV_F16;
}

size_t pool_bytes_checked(int nb, int bs, int layers, int hkv, int d, pagedkv_dtype_t t) {
  if (nb < 1 || bs < 1 || layers < 1 || hkv < 1 || d < 1 || !valid_dtype(t)) return 0;
  const unsigned __int128 n = (unsigned __int128)nb * 2 * layers * hkv * bs * d * elem_size(t);
  if (n > (unsigned __int128)INT64_MAX) return 0;
  return (size_t)n;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PAGEDKV_OK : PAGEDKV_ERR_HIP; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Row arrays (q, out, new K/V rows, gather outputs) are moved in 16-byte units.
bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

namespace pagedkv {

// Workspace: [prefix: batch+1 int32][ml: slots*G*2 f32][o: slots*G*D f32],
// each section 256-byte aligned; slots = batch*kv_heads + kMaxWaves.
size_t decode_workspace_bytes(int batch, int kv_heads, int group, int head_dim) {
  const size_t slots = (size_t)batch * kv_heads + kMaxWaves;
  return align256(sizeof(int32_t) * (size_t)(batch + 1)) +
         align256(sizeof(float) * slots * group * 2) +
         align256(sizeof(float) * slots * group * head_dim);
}

void decode_workspace_carve(void* ws, int batch, int kv_heads, int group, int head_dim,
                            int32_t** prefix, float** ml, float** o) {
  const size_t slots = (size_t)batch * kv_heads + kMaxWaves;
  char* p = static_cast<char*>(ws);
  *prefix = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * (size_t)(batch + 1));
  *ml = reinterpret_cast<float*>(p);
  p += align256(sizeof(float) * slots * group * 2);
  *o = reinterpret_cast<float*>(p);
}

// Query heads per KV head beyond what one wavefront serves (max_group: 32
// for the two-column-group MFMA stream, else 16; MQA, wide GQA groups): the
// kernels serve each KV head as qsplit = ceil(group / max_group) "virtual"
// KV heads of floor or ceil(group / qsplit) consecutive query heads each.
// Every virtual head streams its KV head's rows itself, so K/V are
// requested qsplit times.
HeadSplit head_split(int kv_heads, int group, int max_group) {
  const int q = (group + max_group - 1) / max_group;
  return HeadSplit{q, (group + q - 1) / q, kv_heads * q};
}

namespace {
// The split the paged decode uses: as wide as the kernel that will run takes.
HeadSplit paged_split(const kv_pool* pool, int num_q_heads) {
  const int group = num_q_heads / pool->kv_heads;
  const int cap = mfma_supported(pool, 1) ? mfma_max_group(pool) : kMaxGroup;
  return head_split(pool->kv_heads, group, cap);
}
}  // namespace

}  // namespace pagedkv

extern "C" {

size_t kv_pool_bytes(int num_blocks, int block_size, int layers, int kv_heads, int head_dim,
                     pagedkv_dtype_t dtype) {
  return pool_bytes_checked(num_blocks, block_size, layers, kv_heads, head_dim, dtype);
}

int kv_pool_create(kv_pool_t** out, int num_blocks, int block_size, int layers, int kv_heads,
                   int head_dim, pagedkv_dtype_t dtype, void* device_base, size_t device_bytes) {
  if (!out) return PAGEDKV_ERR_INVALID_ARG;
  *out = nullptr;
  const size_t need = pool_bytes_checked(num_blocks, block_size, layers, kv_heads, head_dim, dtype);
  if (need == 0 || !device_base || device_bytes < need) return PAGEDKV_ERR_INVALID_ARG;
  if (head_dim % (dtype == PAGEDKV_F32 ? 4 : 8) != 0) return PAGEDKV_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(device_base) % 16 != 0) return PAGEDKV_ERR_INVALID_ARG;
  kv_pool* p = new (std::nothrow) kv_pool;
  if (!p) return PAGEDKV_ERR_INVALID_ARG;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->layers = layers;
  p->kv_heads = kv_heads;
  p->head_dim = head_dim;
  p->dtype = dtype;
  p->base = static_cast<char*>(device_base);
  p->bytes = device_bytes;
  try {
    p->free_stack.resize(num_blocks);
    p->is_free.assign(num_blocks, 1);
  } catch (...) {
    delete p;
    return PAGEDKV_ERR_INVALID_ARG;
  }
  for (int i = 0; i < num_blocks; ++i) p->free_stack[i] = i;   // top = num_blocks - 1
  *out = p;
  return PAGEDKV_OK;
}

int kv_pool_destroy(kv_pool_t* pool) {
  if (pool)
    for (kv_block_manager* m : pool->managers) kv_manager_detach(m);
  delete pool;
  return PAGEDKV_OK;
}

int kv_pool_geometry(const kv_pool_t* pool, int* num_blocks, int* block_size, int* layers,
                     int* kv_heads, int* head_dim, pagedkv_dtype_t* dtype, void** device_base) {
  if (!pool) return PAGEDKV_ERR_INVALID_ARG;
  if (num_blocks) *num_blocks = pool->num_blocks;
  if (block_size) *block_size = pool->block_size;
  if (layers) *layers = pool->layers;
  if (kv_heads) *kv_heads = pool->kv_heads;
  if (head_dim) *head_dim = pool->head_dim;
  if (dtype) *dtype = pool->dtype;
  if (device_base) *device_base = pool->base;
  return PAGEDKV_OK;
}

int kv_pool_alloc_block(kv_pool_t* pool, int32_t* block_id) {
  if (!pool || !block_id) return PAGEDKV_ERR_INVALID_ARG;
  if (pool->free_stack.empty()) return PAGEDKV_ERR_OUT_OF_BLOCKS;
  const int32_t id = pool->free_stack.back();
  pool->free_stack.pop_back();
  pool->is_free[id] = 0;
  *block_id = id;
  return PAGEDKV_OK;
}

int kv_pool_free_block(kv_pool_t* pool, int32_t block_id) {
  if (!pool || block_id < 0 || block_id >= pool->num_blocks) return PAGEDKV_ERR_INVALID_ARG;
  if (pool->is_free[block_id]) return PAGEDKV_ERR_INVALID_ARG;
  pool->is_free[block_id] = 1;
  pool->free_stack.push_back(block_id);
  return PAGEDKV_OK;
}

int kv_pool_num_free(const kv_pool_t* pool) {
  if (!pool) return PAGEDKV_ERR_INVALID_ARG;
  return (int)pool->free_stack.size();
}

int kv_append(kv_pool_t* pool, int layer, const void* k_new, const void* v_new,
              const int32_t* block_tables, int max_blocks_per_seq, const int32_t* positions,
              int batch, void* stream) {
  if (!pool || batch < 0 || layer < 0 || layer >= pool->layers || max_blocks_per_seq < 1)
    return PAGEDKV_ERR_INVALID_ARG;
  if (batch == 0) return PAGEDKV_OK;
  if (!k_new || !v_new || !block_tables || !positions) return PAGEDKV_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return PAGEDKV_ERR_INVALID_ARG;
  return hip_status(launch_append(pool, layer, k_new, v_new, block_tables, max_blocks_per_seq,
                                  positions, batch, static_cast<hipStream_t>(stream)));
}

int kv_append_layers(kv_pool_t* pool, const void* k_new, const void* v_new,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* positions, int batch, void* stream) {
  if (!pool || batch < 0 || max_blocks_per_seq < 1) return PAGEDKV_ERR_INVALID_ARG;
  if (batch == 0) return PAGEDKV_OK;
  if (!k_new || !v_new || !block_tables || !positions) return PAGEDKV_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return PAGEDKV_ERR_INVALID_ARG;
  return hip_status(launch_append_layers(pool, k_new, v_new, block_tables, max_blocks_per_seq,
                                         positions, batch, static_cast<hipStream_t>(stream)));
}

int kv_append_tokens(kv_pool_t* pool, int layer, const void* k_new, const void* v_new,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* start_positions, const int32_t* token_offsets, int batch,
                     int total_tokens, void* stream) {
  if (!pool || batch < 0 || total_tokens < 0 || layer < 0 || layer >= pool->layers ||
      max_blocks_per_seq < 1)
    return PAGEDKV_ERR_INVALID_ARG;
  if (batch == 0 || total_tokens == 0) return PAGEDKV_OK;
  if (!k_new || !v_new || !block_tables || !start_positions || !token_offsets)
    return PAGEDKV_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return PAGEDKV_ERR_INVALID_ARG;
  return hip_status(launch_append_tokens(pool, layer, k_new, v_new, block_tables,
                                         max_blocks_per_seq, start_positions, token_offsets,
                                         batch, total_tokens, static_cast<hipStream_t>(stream)));
}

int paged_kv_gather(void* k_out, void* v_out, uint8_t* mask, const kv_pool_t* pool, int layer,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* context_lens, int batch, int max_len, void* stream) {
  if (!pool || batch < 0 || max_len < 0 || layer < 0 || layer >= pool->layers ||
      max_blocks_per_seq < 1 || batch > 65535)
    return PAGEDKV_ERR_INVALID_ARG;
  if (batch == 0 || max_len == 0) return PAGEDKV_OK;
  if (!k_out || !v_out || !mask || !block_tables || !context_lens) return PAGEDKV_ERR_INVALID_ARG;
  if (!aligned16(k_out) || !aligned16(v_out)) return PAGEDKV_ERR_INVALID_ARG;
  if (pool->head_dim * elem_size(pool->dtype) > 256 * 16) return PAGEDKV_ERR_UNSUPPORTED;
  return hip_status(launch_gather(k_out, v_out, mask, pool, layer, block_tables,
                                  max_blocks_per_seq, context_lens, batch, max_len,
                                  static_cast<hipStream_t>(stream)));
}

size_t paged_attention_workspace_bytes(const kv_pool_t* pool, int batch, int num_q_heads) {
  if (!pool || batch < 0 || num_q_heads < 1 || num_q_heads % pool->kv_heads != 0) return 0;
  const HeadSplit hs = paged_split(pool, num_q_heads);
  return decode_workspace_bytes(batch, hs.vheads, hs.group, pool->head_dim);
}

}  // extern "C"

namespace {

// Device scratch of paged_attention_decode_noalloc: one copy per GPU, held
// from module load to process end.  Host code must not use the array's name
// as a device address: every use goes through the address returned by
// hipGetSymbolAddress on that device (scratch_address below).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kScratchDevices];
std::mutex g_scratch_mu;

// Device address of the current GPU's scratch array, looked up once per
// device with that device current.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PAGEDKV_ERR_HIP;
  if (dev < 0 || dev >= kScratchDevices) return PAGEDKV_ERR_UNSUPPORTED;
  void* a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!a) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    a = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!a) {
      void* sym = nullptr;
      if (hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch)) != hipSuccess || !sym)
        return PAGEDKV_ERR_HIP;
      g_scratch_addr[dev].store(sym, std::memory_order_release);
      a = sym;
    }
  }
  *out = a;
  return PAGEDKV_OK;
}

// Shared body of the decode entry points.  With k_new != nullptr the call
// also appends each sequence's new token (the fused form).  With
// use_scratch the workspace is the library's static device scratch (the
// workspace arguments are ignored).
int decode_call(void* out, const void* q, const kv_pool_t* pool, int layer,
                const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                int batch, int num_q_heads, float scale, void* workspace, size_t workspace_bytes,
                unsigned flags, void* stream, const void* k_new, const void* v_new,
                const int32_t* positions, bool use_scratch = false) {
  if (!pool || batch < 0 || layer < 0 || layer >= pool->layers || max_blocks_per_seq < 1 ||
      num_q_heads < 1 || num_q_heads % pool->kv_heads != 0 || !isfinite(scale) ||
      (flags & ~PAGEDKV_DECODE_CHUNKS) != 0)
    return PAGEDKV_ERR_INVALID_ARG;
  if (batch == 0) return PAGEDKV_OK;
  if (!out || !q || !block_tables || !context_lens) return PAGEDKV_ERR_INVALID_ARG;
  const bool append = k_new != nullptr || v_new != nullptr || positions != nullptr;
  if (append && (!k_new || !v_new || !positions)) return PAGEDKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || (append && (!aligned16(k_new) || !aligned16(v_new))))
    return PAGEDKV_ERR_INVALID_ARG;
  if (batch > kMaxBatchLds) return PAGEDKV_ERR_UNSUPPORTED;
  // The kernels keep chunk counts and their prefix sums in int32: the
  // longest sequence the tables allow, cut into 16-token chunks (the
  // smallest chunk of any kernel), times the batch must fit.
  const int64_t max_tokens = (int64_t)max_blocks_per_seq * pool->block_size;
  if ((int64_t)batch * ((max_tokens + 15) / 16) > INT32_MAX) return PAGEDKV_ERR_UNSUPPORTED;
  const HeadSplit hs = paged_split(pool, num_q_heads);
  const bool use_mfma = mfma_supported(pool, hs.group);
  if (!use_mfma && !generic_supported(pool, hs.group)) return PAGEDKV_ERR_UNSUPPORTED;
  const size_t need = decode_workspace_bytes(batch, hs.vheads, hs.group, pool->head_dim);
  if (use_scratch) {
    if (need > kScratchBytes) return PAGEDKV_ERR_SCRATCH;
    const int st = scratch_address(&workspace);
    if (st != PAGEDKV_OK) return st;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace || workspace_bytes < need) return PAGEDKV_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return PAGEDKV_ERR_WORKSPACE;

  DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.pool = geom_of(pool);
  p.q = q;
  p.out = out;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  decode_workspace_carve(workspace, batch, hs.vheads, hs.group, pool->head_dim, &p.ws_prefix,
                         &p.ws_ml, &p.ws_o);
  p.layer = layer;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.group = hs.group;
  p.vheads = hs.vheads;
  p.qsplit = hs.qsplit;
  p.kv_group = num_q_heads / pool->kv_heads;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.dtype = pool->dtype;
  p.min_chunks = 0;   // launcher default
  p.pair_mode = use_mfma && (flags & PAGEDKV_DECODE_CHUNKS) == 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (use_mfma) {
    // (the merge kernel stores each new row with one 16-byte unit per lane)
    if (append && 2 * pool->head_dim * elem_size(pool->dtype) > 64 * 16) return PAGEDKV_ERR_UNSUPPORTED;
    if (append) {
      p.k_new = k_new;
      p.v_new = v_new;
      p.positions = positions;
    }
    e = launch_decode_mfma(p, s);
    if (e == hipSuccess && p.pair_mode) return PAGEDKV_OK;   // merged in its own workgroups
  } else {
    // the VALU kernel reads the pool only: append first, as its own launch
    if (append) {
      e = launch_append(pool, layer, k_new, v_new, block_tables, max_blocks_per_seq, positions,
                        batch, s);
      if (e != hipSuccess) return PAGEDKV_ERR_HIP;
    }
    e = launch_decode_generic(p, s);
  }
  if (e != hipSuccess) return PAGEDKV_ERR_HIP;
  return hip_status(launch_decode_merge(p, s));
}

}  // namespace

extern "C" {

int paged_attention_decode(void* out, const void* q, const kv_pool_t* pool, int layer,
                           const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, int batch, int num_q_heads, float scale,
                           void* workspace, size_t workspace_bytes, unsigned flags,
                           void* stream) {
  return decode_call(out, q, pool, layer, block_tables, max_blocks_per_seq, context_lens, batch,
                     num_q_heads, scale, workspace, workspace_bytes, flags, stream, nullptr,
                     nullptr, nullptr);
}

int paged_attention_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                                  const int32_t* positions, kv_pool_t* pool, int layer,
                                  const int32_t* block_tables, int max_blocks_per_seq,
                                  const int32_t* context_lens, int batch, int num_q_heads,
                                  float scale, void* workspace, size_t workspace_bytes,
                                  unsigned flags, void* stream) {
  if (batch > 0 && (!k_new || !v_new || !positions)) return PAGEDKV_ERR_INVALID_ARG;
  return decode_call(out, q, pool, layer, block_tables, max_blocks_per_seq, context_lens, batch,
                     num_q_heads, scale, workspace, workspace_bytes, flags, stream, k_new, v_new,
                     positions);
}

int paged_attention_decode_noalloc(void* out, const void* q, const kv_pool_t* pool, int layer,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* context_lens, int batch, int num_q_heads,
                                   float scale, unsigned flags, void* stream) {
  return decode_call(out, q, pool, layer, block_tables, max_blocks_per_seq, context_lens, batch,
                     num_q_heads, scale, nullptr, 0, flags, stream, nullptr, nullptr, nullptr,
                     /*use_scratch=*/true);
}

size_t dense_attention_workspace_bytes(int batch, int kv_heads, int num_q_heads, int head_dim) {
  if (batch < 0 || kv_heads < 1 || num_q_heads < 1 || num_q_heads % kv_heads != 0 || head_dim < 1)
    return 0;
  const HeadSplit hs = head_split(kv_heads, num_q_heads / kv_heads, kMaxGroup);
  return decode_workspace_bytes(batch, hs.vheads, hs.group, head_dim);
}

int dense_attention_decode(void* out, const void* q, const void* k, const void* v,
                           const uint8_t* mask, int batch, int max_len, int kv_heads,
                           int head_dim, int num_q_heads, pagedkv_dtype_t dtype, float scale,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0 || max_len < 0 || kv_heads < 1 || num_q_heads < 1 ||
      num_q_heads % kv_heads != 0 || !isfinite(scale) || !valid_dtype(dtype) || head_dim < 1)
    return PAGEDKV_ERR_INVALID_ARG;
  if (batch == 0) return PAGEDKV_OK;
  if (!out || !q || (max_len > 0 && (!k || !v || !mask))) return PAGEDKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v))
    return PAGEDKV_ERR_INVALID_ARG;
  const HeadSplit hs = head_split(kv_heads, num_q_heads / kv_heads, kMaxGroup);
  if ((dtype != PAGEDKV_BF16 && dtype != PAGEDKV_F16) ||
      (head_dim != 64 && head_dim != 96 && head_dim != 128 && head_dim != 256) ||
      batch > kMaxBatchLds)
    return PAGEDKV_ERR_UNSUPPORTED;
  // chunk count (16-token chunks at the smallest) must fit the kernel's int32 prefix
  if ((int64_t)batch * ((max_len + 15) / 16) > INT32_MAX) return PAGEDKV_ERR_UNSUPPORTED;
  const size_t need = decode_workspace_bytes(batch, hs.vheads, hs.group, head_dim);
  if (!workspace || workspace_bytes < need) return PAGEDKV_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return PAGEDKV_ERR_WORKSPACE;

  DecodeParams p;
  memset(&p, 0, sizeof(p));
  // only the head geometry of the "pool" is used; K/V come from k and v
  p.pool.kv_heads = kv_heads;
  p.pool.head_dim = head_dim;
  p.pool.block_size = 16;
  p.max_blocks_per_seq = max_len > 0 ? (max_len + 15) / 16 : 1;
  p.q = q;
  p.out = out;
  decode_workspace_carve(workspace, batch, hs.vheads, hs.group, head_dim, &p.ws_prefix, &p.ws_ml,
                         &p.ws_o);
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.group = hs.group;
  p.vheads = hs.vheads;
  p.qsplit = hs.qsplit;
  p.kv_group = num_q_heads / kv_heads;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.dtype = dtype;
  p.k_dense = k ? k : q;   // max_len == 0: never read
  p.v_dense = v ? v : q;
  p.mask = mask;
  p.dense_len = max_len;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_decode_mfma(p, s) != hipSuccess) return PAGEDKV_ERR_HIP;
  return hip_status(launch_decode_merge(p, s));
}

int paged_kv_resolve(int64_t* slots, const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* context_lens, int batch, int block_size, int max_len,
                     void* stream) {
  if (batch < 0 || max_len < 0 || block_size < 1 || max_blocks_per_seq < 1 || batch > 65535)
    return PAGEDKV_ERR_INVALID_ARG;
  if (batch == 0 || max_len == 0) return PAGEDKV_OK;
  if (!slots || !block_tables || !context_lens) return PAGEDKV_ERR_INVALID_ARG;
  return hip_status(launch_resolve(slots, block_tables, max_blocks_per_seq, context_lens, batch,
                                   block_size, max_len, static_cast<hipStream_t>(stream)));
}

const char* pagedkv_status_string(int status) {
  switch (status) {
    case PAGEDKV_OK: return "ok";
    case PAGEDKV_ERR_INVALID_ARG: return "invalid argument";
    case PAGEDKV_ERR_OUT_OF_BLOCKS: return "no free block left in the pool";
    case PAGEDKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PAGEDKV_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case PAGEDKV_ERR_HIP: return "HIP runtime error";
    case PAGEDKV_ERR_SCRATCH:
      return "call needs more than the 64 MiB static scratch of paged_attention_decode_noalloc";
    default: return "unknown status";
  }
}

}  // extern "C"
