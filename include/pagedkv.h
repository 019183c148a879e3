/*
 * pagedkv.h -- paged KV-cache attention decode for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpagedkv.so.  Plain pointers and sizes only.
 *
 * Sources (three web pages on paged KV caches):
 *   [vllmini]    "vllmini: Building a Minimalist PagedAttention and KV Cache
 *                Engine", sections "PagedAttention Metaphor" and "The CUDA
 *                Block Kernel".
 *   [kv-cache]   "KV Cache and Attention Mechanisms: PagedAttention and vLLM",
 *                section 2 "PagedAttention Architecture".
 *   [mini-infer] "Paged KV-Cache Memory Management", sections "The Solution",
 *                "Python Implementation: Physical Block Pool & Batched
 *                Paging" and "Zero-Copy Batched Attention Gather".
 *
 * Conventions shared by every call
 *   - Device memory is owned by the caller (PyTorch in the Python binding).
 *     The library never allocates or frees device memory and never
 *     synchronises; GPU work is enqueued on the given stream (a hipStream_t
 *     passed as void*; NULL = the default stream) and is asynchronous.
 *   - Every call returns an int status: PAGEDKV_OK (0) or a negative code.
 *     No exception crosses the ABI.
 *   - Pool layout ([mini-infer] "Python Implementation: Physical Block
 *     Pool"): one contiguous array
 *         [num_blocks][2 (0 = K, 1 = V)][layers][kv_heads][block_size][head_dim]
 *     of the pool dtype, row-major.  One physical block holds block_size
 *     tokens of K and V for every layer and KV head.
 *   - Block tables ([vllmini] "PagedAttention Metaphor"; [mini-infer] "The
 *     Solution"): int32, row-major [batch][max_blocks_per_seq]; entry j of
 *     row b is the physical block holding tokens j*block_size ..
 *     j*block_size + block_size - 1 of sequence b.  One row serves all heads
 *     and layers.  Entries at j >= ceil(T_b / block_size) are never read.
 *   - context_lens: int32 [batch], T_b = number of cached tokens of sequence
 *     b, counting the token appended in the same step.
 *   - Values that live in device memory (block ids, context lengths,
 *     positions) are not validated: checking them would need a
 *     synchronisation.  Block ids outside [0, num_blocks) or lengths beyond
 *     max_blocks_per_seq * block_size are undefined behaviour.  Every
 *     host-visible argument is validated before anything is enqueued.
 *   - Row arrays (q, out, new K/V rows, gather outputs) are moved in 16-byte
 *     units and must be 16-byte aligned; a misaligned pointer is rejected
 *     with PAGEDKV_ERR_INVALID_ARG.
 *   - Calls that share a workspace or write the same output must not run
 *     concurrently on different streams.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define PAGEDKV_OK 0
#define PAGEDKV_ERR_INVALID_ARG (-1)   /* null pointer, out-of-range size or index */
#define PAGEDKV_ERR_OUT_OF_BLOCKS (-2) /* free-block stack empty */
#define PAGEDKV_ERR_UNSUPPORTED (-3)   /* shape/dtype combination with no kernel */
#define PAGEDKV_ERR_WORKSPACE (-4)     /* workspace missing or too small */
#define PAGEDKV_ERR_HIP (-5)           /* a HIP runtime call or launch failed */
#define PAGEDKV_ERR_SCRATCH (-6)       /* call needs more than the library's static scratch */

/* Element types of the pool (and of q / out / new tokens / gather output). */
typedef enum {
  PAGEDKV_F32 = 0,
  PAGEDKV_BF16 = 1,
  PAGEDKV_F16 = 2    /* IEEE binary16 */
} pagedkv_dtype_t;

/* Opaque host handle describing a pool.  It records the geometry and the
 * device address of the pool storage and keeps the host free-block stack.
 * It does not own the device memory. */
typedef struct kv_pool kv_pool_t;

/* Bytes of device storage a pool of this geometry needs:
 * num_blocks * 2 * layers * kv_heads * block_size * head_dim * sizeof(dtype).
 * Returns 0 for invalid arguments. */
size_t kv_pool_bytes(int num_blocks, int block_size, int layers, int kv_heads,
                     int head_dim, pagedkv_dtype_t dtype);

/* Describe a pool over caller-owned device memory of at least
 * kv_pool_bytes(...) bytes at device_base (any 16-byte-aligned device
 * allocation; its contents are left untouched).  All num_blocks ids start on
 * the free-block stack in ascending order, so the first allocation returns
 * num_blocks - 1 ([mini-infer] "Python Implementation: Physical Block Pool":
 * the free list is a stack popped from its end).
 * Requirements: all sizes >= 1, head_dim a multiple of 8 (bf16, fp16) or 4
 * (fp32), so that a row is a whole number of 16-byte units.
 * On success *out receives a handle to release with kv_pool_destroy. */
int kv_pool_create(kv_pool_t** out, int num_blocks, int block_size, int layers,
                   int kv_heads, int head_dim, pagedkv_dtype_t dtype,
                   void* device_base, size_t device_bytes);

/* Release the handle (not the device memory).  NULL is accepted. */
int kv_pool_destroy(kv_pool_t* pool);

/* Geometry query; any output pointer may be NULL. */
int kv_pool_geometry(const kv_pool_t* pool, int* num_blocks, int* block_size,
                     int* layers, int* kv_heads, int* head_dim,
                     pagedkv_dtype_t* dtype, void** device_base);

/* Pop a free physical block id from the top of the host stack
 * ([mini-infer] "Python Implementation": allocation fails once no block is
 * free).  Returns PAGEDKV_ERR_OUT_OF_BLOCKS when the stack is empty. */
int kv_pool_alloc_block(kv_pool_t* pool, int32_t* block_id);

/* Push block_id back onto the stack.  Unlike the page's list, ids outside
 * [0, num_blocks) and ids that are already free are rejected with
 * PAGEDKV_ERR_INVALID_ARG. */
int kv_pool_free_block(kv_pool_t* pool, int32_t block_id);

/* Number of free blocks, or a negative status. */
int kv_pool_num_free(const kv_pool_t* pool);

/* ---- Host block manager (host memory only; never touches the GPU) ----
 *
 * Tracks which physical blocks each sequence holds and how many tokens it
 * has, drawing blocks from and returning them to the pool's free stack:
 *   - blocks are added one at a time as a sequence grows, so only its last
 *     block can be partly filled ([kv-cache] section 2, "Zero-Waste
 *     Allocation"; [mini-infer] "Memory Waste Analysis");
 *   - a step is admitted only if the pool holds every block it needs
 *     ([kv-cache] section 3.1, "Cache Block Pool"); otherwise nothing changes;
 *   - a finished sequence returns its blocks in logical order, so its last
 *     block is the next one the stack hands out.
 * Sequences are named by caller-chosen int64 ids.  Not thread-safe: calls on
 * one manager, and on its pool's free stack, must not overlap.  Destroying
 * the pool detaches its managers: their later calls return
 * PAGEDKV_ERR_INVALID_ARG, and kv_manager_destroy only frees the manager. */
typedef struct kv_block_manager kv_block_manager_t;

typedef struct {
  int64_t sequences;     /* live sequences */
  int64_t blocks_total;  /* pool blocks */
  int64_t blocks_free;   /* on the pool's free stack */
  int64_t blocks_used;   /* held by this manager's sequences */
  int64_t tokens;        /* tokens held */
  int64_t slots;         /* blocks_used * block_size */
  int64_t waste_slots;   /* slots - tokens: at most block_size - 1 per sequence */
  double waste_ratio;    /* waste_slots / tokens (0 when no tokens) */
} kv_manager_stats_t;

/* max_blocks_per_seq: width of the block-table rows the manager writes; a
 * sequence may not grow past it. */
int kv_manager_create(kv_block_manager_t** out, kv_pool_t* pool, int max_blocks_per_seq);

/* Releases every live sequence's blocks to the pool, then frees the
 * manager.  NULL is accepted. */
int kv_manager_destroy(kv_block_manager_t* mgr);

/* Register an empty sequence (no blocks).  An id already live is
 * PAGEDKV_ERR_INVALID_ARG. */
int kv_manager_add_sequence(kv_block_manager_t* mgr, int64_t seq_id);

/* The admission figure of a step: free blocks needed to grow sequence
 * seq_ids[i] by counts[i] tokens for every i (a decode step: counts all 1;
 * a prompt or a chunk of one: its length).  Returns the count (>= 0) or a
 * negative status: unknown id, an id twice, a negative count or growth past
 * max_blocks_per_seq blocks is PAGEDKV_ERR_INVALID_ARG. */
int64_t kv_manager_blocks_needed(const kv_block_manager_t* mgr, int n, const int64_t* seq_ids,
                                 const int32_t* counts);

/* Admit and apply a step: allocate the blocks kv_manager_blocks_needed
 * counts (sequences in the order given, each one's blocks in logical order),
 * grow every sequence, and write its first new position (its token count
 * before the step) to start_positions[i] (may be NULL).  If the pool has
 * too few free blocks, returns PAGEDKV_ERR_OUT_OF_BLOCKS and changes
 * nothing; argument errors as for kv_manager_blocks_needed. */
int kv_manager_reserve(kv_block_manager_t* mgr, int n, const int64_t* seq_ids,
                       const int32_t* counts, int32_t* start_positions);

/* Finish a sequence: its blocks go back to the pool's free stack in logical
 * order and the id is forgotten. */
int kv_manager_release(kv_block_manager_t* mgr, int64_t seq_id);

/* Host block tables for a batch: tables[i][j] (row-major [n][max_blocks_per_seq],
 * -1 past the sequence's blocks) and context_lens[i] = its token count.  Ready
 * to be copied to the device for kv_append* and paged_attention_decode*. */
int kv_manager_block_tables(const kv_block_manager_t* mgr, int n, const int64_t* seq_ids,
                            int32_t* tables, int32_t* context_lens);

/* Blocks and tokens held, and the internal-fragmentation waste
 * ([mini-infer] "Memory Waste Analysis"). */
int kv_manager_stats(const kv_block_manager_t* mgr, kv_manager_stats_t* out);

/* Append one token per sequence into its tail block
 * ([kv-cache] section 2: blocks are filled per block as generation
 * proceeds; [mini-infer] "The Solution": a block stores K and V of B
 * tokens for every layer).
 *   k_new, v_new : device, [batch][kv_heads][head_dim], pool dtype.
 *   block_tables : device, [batch][max_blocks_per_seq] int32.
 *   positions    : device, [batch] int32; token index written for sequence b
 *                  (normally T_b - 1).  A negative position skips b.
 * Writes pool[table[b][pos/B]][0|1][layer][g][pos%B][:] for every g.  The
 * copy is bit-exact.  The caller must have placed the tail block in the
 * table (allocate when pos % block_size == 0). */
int kv_append(kv_pool_t* pool, int layer, const void* k_new, const void* v_new,
              const int32_t* block_tables, int max_blocks_per_seq,
              const int32_t* positions, int batch, void* stream);

/* Append one token per sequence for every layer at once ([mini-infer] "The
 * Solution": a block holds its tokens' K and V for all layers, so one slot
 * serves every layer).
 *   k_new, v_new : device, [batch][layers][kv_heads][head_dim], pool dtype.
 *   positions    : device, [batch] int32; negative = skip b.
 * Equal to kv_append(pool, l, k_new[:, l], v_new[:, l], ...) for every layer
 * l, in one launch.  Bit-exact. */
int kv_append_layers(kv_pool_t* pool, const void* k_new, const void* v_new,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* positions, int batch, void* stream);

/* Append several consecutive tokens per sequence for one layer, e.g. a
 * prompt or a chunk of one ([kv-cache] section 2: a prompt fills whole blocks
 * and only the last one is partly filled).
 *   k_new, v_new   : device, [total_tokens][kv_heads][head_dim], pool dtype;
 *                    rows token_offsets[b] .. token_offsets[b+1]-1 belong to
 *                    sequence b.
 *   start_positions: device, [batch] int32; row token_offsets[b] + i goes to
 *                    logical position start_positions[b] + i.  Negative = skip b.
 *   token_offsets  : device, [batch + 1] int32, non-decreasing, from 0 to
 *                    total_tokens (total_tokens itself is passed by value).
 * Row r belongs to the last b with token_offsets[b] <= r, so an empty
 * sequence (equal neighbouring offsets) receives nothing.  The caller must
 * have placed in the table every block the new positions fall into; like
 * kv_append, the kernel trusts offsets, positions and table entries.
 * Bit-exact. */
int kv_append_tokens(kv_pool_t* pool, int layer, const void* k_new, const void* v_new,
                     const int32_t* block_tables, int max_blocks_per_seq,
                     const int32_t* start_positions, const int32_t* token_offsets,
                     int batch, int total_tokens, void* stream);

/* Batched gather of paged K/V into contiguous tensors
 * ([mini-infer] "Zero-Copy Batched Attention Gather").
 *   k_out, v_out : device, [batch][max_len][kv_heads][head_dim], pool dtype.
 *   mask         : device, [batch][max_len] uint8: 1 for t < T_b, else 0.
 *   context_lens : device, [batch] int32, each <= max_len.
 * Positions t >= T_b are written as zero bits.  Bit-exact copy. */
int paged_kv_gather(void* k_out, void* v_out, uint8_t* mask,
                    const kv_pool_t* pool, int layer,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* context_lens, int batch, int max_len,
                    void* stream);

/* Bytes of device workspace paged_attention_decode needs for this call
 * shape (independent of the context lengths' values).  0 on invalid
 * arguments. */
size_t paged_attention_workspace_bytes(const kv_pool_t* pool, int batch,
                                       int num_q_heads);

/* Paged-attention decode for one layer
 * ([vllmini] "The CUDA Block Kernel": for each (sequence, head) the kernel
 * resolves the sequence's logical token positions through its block table
 * into physical pages and computes dot-product attention over them;
 * [kv-cache] section 2: the kernel fetches the physical blocks named by the
 * block table).
 *   out, q       : device, [batch][num_q_heads][head_dim], pool dtype.
 *   num_q_heads  : a multiple of kv_heads; query head h reads KV head
 *                  h / (num_q_heads / kv_heads).
 *   scale        : multiplies q.k before the softmax.
 *   workspace    : device, >= paged_attention_workspace_bytes(...) bytes,
 *                  256-byte aligned; contents need no initialisation.  Calls
 *                  that share a workspace must not overlap.
 * out[b][h] = sum_t softmax_t(scale * q[b][h] . K_t) V_t over t < T_b,
 * computed with fp32 accumulation; bf16 and fp16 outputs are rounded to
 * nearest even.  T_b = 0 gives a zero row.  Work is split evenly over all
 * wavefronts the GPU holds at once; a sequence split across wavefronts is
 * merged by a second kernel on the same stream (log-sum-exp weights).
 * Small batches on the MFMA kernels instead run one workgroup of 8
 * wavefronts per (sequence, KV head) pair, which merges its own pieces, so
 * one kernel does the whole call.  That applies at head_dim 64, 96 or 128
 * with at most 16 query heads per wavefront, when every pair's workgroup is
 * resident at once and the longest sequence the block tables allow,
 * max_blocks_per_seq * block_size tokens, holds at most 512 KiB of K and V
 * per KV head at head_dim 64 in bf16 or fp16 with block_size a multiple of
 * 16 (2048 tokens; these pairs stage K and V through LDS, and while at
 * most 128 such pairs are launched each runs as two workgroups that take
 * one half of V's dims each), else 256 KiB
 * (1024 tokens at head_dim 64 in bf16 or fp16 with 4- or 8-token blocks,
 * 512 at 128; 512 and 256 in fp32); flags = PAGEDKV_DECODE_CHUNKS keeps
 * every call on the chunk split (below).
 * Kernels: MFMA for head_dim 64 or 128 with block_size a multiple of 16
 * (bf16, fp16, fp32), and in bf16 and fp16 also for head_dim 96 and 256 and
 * for block_size 4 or 8; a VALU kernel for head_dim up to 256 in steps of 4
 * and any block size.  At most 16384 sequences per call; otherwise
 * PAGEDKV_ERR_UNSUPPORTED.  Any number of query heads per KV head, G =
 * num_q_heads / kv_heads: one wavefront serves up to W of them (W = 32 for
 * bf16/fp16 at head_dim 64 or 128 with block_size a multiple of 16, else
 * 16), reading K/V once for all; a larger G is served as q = ceil(G/W)
 * "virtual" KV heads of floor or ceil(G/q) query heads, each of which
 * requests the KV head's rows itself. */
int paged_attention_decode(void* out, const void* q, const kv_pool_t* pool,
                           int layer, const int32_t* block_tables,
                           int max_blocks_per_seq, const int32_t* context_lens,
                           int batch, int num_q_heads, float scale,
                           void* workspace, size_t workspace_bytes,
                           unsigned flags, void* stream);

/* One decode step: append each sequence's new token, then decode
 * ([kv-cache] section 2: generation fills the tail block one token at a
 * time; [vllmini] "The CUDA Block Kernel": attention over the blocks the
 * table names).  The result, in `out` and in the pool, equals
 *     kv_append(pool, layer, k_new, v_new, block_tables, max_blocks_per_seq,
 *               positions, batch, stream);
 *     paged_attention_decode(out, q, pool, layer, block_tables, ...);
 * for every input, positions included (negative = no token for b; a
 * position at or past T_b is written but not attended, as in the two-call
 * form).  Arguments are those of the two calls; k_new, v_new and positions
 * must all be non-null when batch > 0.
 * Where the MFMA kernel runs (see paged_attention_decode) it reads each new
 * K/V row from k_new / v_new instead of the pool and
 * the merge kernel stores them into the pool afterwards, which saves the
 * separate append launch; other shapes run the two launches. */
int paged_attention_decode_append(void* out, const void* q, const void* k_new,
                                  const void* v_new, const int32_t* positions,
                                  kv_pool_t* pool, int layer,
                                  const int32_t* block_tables,
                                  int max_blocks_per_seq,
                                  const int32_t* context_lens, int batch,
                                  int num_q_heads, float scale, void* workspace,
                                  size_t workspace_bytes, unsigned flags, void* stream);

/* Flags of paged_attention_decode, paged_attention_decode_append and
 * paged_attention_decode_noalloc, per call; any other bit set is
 * PAGEDKV_ERR_INVALID_ARG.
 *   0                     : per-pair workgroups where the shape allows (see
 *                           paged_attention_decode), else the chunk split.
 *   PAGEDKV_DECODE_CHUNKS : always the persistent chunk split.
 * The two splits agree within the decode tolerances but not bit for bit,
 * since the softmax sums are taken in a different order.  Each split is
 * deterministic: the same inputs and flags give the same bits. */
#define PAGEDKV_DECODE_CHUNKS 1u

/* paged_attention_decode without a workspace argument, for callers that
 * cannot allocate device memory: code recorded under HIP graph capture,
 * serving loops and harnesses that forbid allocation.  The call allocates
 * nothing.  Its scratch (what the workspace holds for
 * paged_attention_decode: chunk prefix, partial results of split
 * sequences) is a static device array of 64 MiB inside the library, one per
 * GPU, which exists from the loading of the library's device code until the
 * process ends; its address is looked up once per GPU (hipGetSymbolAddress)
 * on the first call made with that GPU current.
 *   - A call whose paged_attention_workspace_bytes(pool, batch,
 *     num_q_heads) exceeds 64 MiB returns PAGEDKV_ERR_SCRATCH before
 *     anything is enqueued (e.g. batch 64 with 8 KV heads of 4 query heads
 *     at head_dim 128 needs 18 MB; batch 256 with 8 KV heads of 8 query
 *     heads, 42 MB).
 *   - Every call on one GPU uses that GPU's one array and leaves its
 *     contents behind; the kernels need no clearing between calls.  Calls
 *     on one stream are ordered and safe; calls that overlap on one GPU
 *     (several streams, or host threads without ordering) race on the array
 *     and give undefined results.
 * Arguments, results and other errors as paged_attention_decode. */
int paged_attention_decode_noalloc(void* out, const void* q, const kv_pool_t* pool,
                                   int layer, const int32_t* block_tables,
                                   int max_blocks_per_seq, const int32_t* context_lens,
                                   int batch, int num_q_heads, float scale,
                                   unsigned flags, void* stream);

/* Bytes of device workspace dense_attention_decode needs (0 for invalid
 * arguments). */
size_t dense_attention_workspace_bytes(int batch, int kv_heads, int num_q_heads, int head_dim);

/* Decode over gathered, padded K/V: the attention that follows
 * paged_kv_gather in [mini-infer] "Zero-Copy Batched Attention Gather"
 * (the v0.2.0 path), kept to compare with the paged decode, which reads the
 * pool in place.
 *   out, q : device, [batch][num_q_heads][head_dim], dtype.
 *   k, v   : device, [batch][max_len][kv_heads][head_dim], dtype (the gather's
 *            outputs; values must be finite).
 *   mask   : device, [batch][max_len] uint8; token t of sequence b takes part
 *            iff mask[b][t] != 0.  A sequence with no such token gives zeros.
 * Every one of the max_len rows is read, padding included.  Same arithmetic
 * and tolerances as paged_attention_decode.  bf16 and fp16, head_dim 64, 96,
 * 128 or 256, any number of query heads per KV head (split as in
 * paged_attention_decode); otherwise PAGEDKV_ERR_UNSUPPORTED.
 * workspace as for paged_attention_decode (256-byte aligned). */
int dense_attention_decode(void* out, const void* q, const void* k, const void* v,
                           const uint8_t* mask, int batch, int max_len, int kv_heads,
                           int head_dim, int num_q_heads, pagedkv_dtype_t dtype, float scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Block-table resolution on its own ([vllmini] "PagedAttention Metaphor":
 * logical offsets resolved to physical page offsets on the fly).
 *   slots : device, [batch][max_len] int64; slots[b][t] =
 *           table[b][t / block_size] * block_size + t % block_size for
 *           t < T_b, else -1.
 * Bit-exact; exists so the resolver can be checked on its own. */
int paged_kv_resolve(int64_t* slots, const int32_t* block_tables,
                     int max_blocks_per_seq, const int32_t* context_lens,
                     int batch, int block_size, int max_len, void* stream);

/* Static description of a status code. */
const char* pagedkv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
