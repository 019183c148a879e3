/*
 * pagedkv_probe.h -- HBM read-ceiling probe (measurement helper, not part of
 * the decode library's ABI).  Built as libpagedkv_probe.so beside
 * libpagedkv.so.
 *
 * Paged decode streams every cached K/V row once per step, so its speed is
 * set by HBM read bandwidth ("vllmini: Building a Minimalist PagedAttention
 * and KV Cache Engine", introduction: memory bandwidth is the bottleneck of
 * decoding; "KV Cache and Attention Mechanisms", section 1).  This probe
 * measures what a plain read kernel reaches on the machine for a given
 * access pattern: the same 16-byte non-temporal loads as the decode kernel,
 * over fixed-size slabs visited in a caller-given order (sequential, or a
 * random permutation, like the blocks a block table names), with no
 * arithmetic beyond folding the loaded words into one value per thread.
 */
#ifndef PAGEDKV_PROBE_H
#define PAGEDKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read n_slabs slabs of slab_bytes each from the device buffer `base`
 * (buffer_bytes long): slab i of the visit order starts at byte
 * slab_ids[i] * slab_bytes.  The visit order is cut into `workgroups` x 4
 * equal contiguous ranges, one per wavefront; each wavefront reads its
 * slabs 1 KiB (64 lanes x 16 bytes) at a time with 32 loads per lane in
 * flight.  Each thread folds what it read into one word of sink
 * (device, workgroups * 256 uint32), so no load is dead.
 *   slab_ids    : device, int32 [n_slabs]; values are clamped to
 *                 [0, buffer_bytes / slab_bytes - 1], so any value stays in
 *                 the buffer.
 *   slab_bytes  : a power of two, at least 1024.
 *   workgroups  : 1 .. 65535 (256 threads each).
 * Returns 0, -1 for invalid arguments, -5 if the launch failed.
 * Asynchronous on `stream` (a hipStream_t; NULL = the default stream). */
int pagedkv_read_probe(const void* base, size_t buffer_bytes, const int32_t* slab_ids,
                       int64_t n_slabs, int slab_bytes, int workgroups, uint32_t* sink,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_PROBE_H */
