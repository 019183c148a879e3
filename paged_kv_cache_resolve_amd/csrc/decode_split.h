// Device helpers for the decode work split (see DecodeParams in internal.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace pagedkv {

// n / d for 0 <= n < 2^31, with f = make_fast_div(d).
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

__device__ __forceinline__ int chunks_of(int T, int ct) {
  return T > 0 ? (T + ct - 1) / ct : 0;
}

// prefix[b] = sum_{b' < b} chunks_of(T_b', ct) for b in [0, batch], computed by
// one workgroup of NT threads (a multiple of 64) into LDS.  Thread t sums a
// contiguous run of sequences; the runs' totals are scanned within each
// wavefront with lane shuffles, and the wavefront totals (NT / 64 ints of
// `scan`, LDS) are added after one barrier.  Every thread of the workgroup
// must call this; it ends with a barrier.
template <int NT>
__device__ void block_chunk_prefix(const int32_t* __restrict__ lens, int batch,
                                   int ct, int32_t* prefix, int32_t* scan) {
  static_assert(NT % 64 == 0, "whole wavefronts");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int per = (batch + NT - 1) / NT;
  const int lo = min(batch, tid * per);
  const int hi = min(batch, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) {
    const int n = chunks_of(lens[i], ct);
    prefix[i + 1] = n;
    local += n;
  }
  int incl = local;   // inclusive scan of the run totals across the wavefront
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int up = __shfl_up(incl, d, 64);
    if (lane >= d) incl += up;
  }
  if (lane == 63) scan[tid >> 6] = incl;
  __syncthreads();
  int run = incl - local;   // exclusive offset of this thread's run
  for (int w = 0; w < (tid >> 6); ++w) run += scan[w];
  for (int i = lo; i < hi; ++i) {
    run += prefix[i + 1];
    prefix[i + 1] = run;
  }
  if (tid == 0) prefix[0] = 0;
  __syncthreads();
}

// Number of wavefronts that receive work: all W, unless that would leave
// fewer than min_chunks chunks per wavefront.
__device__ __forceinline__ int64_t waves_eff(int64_t C, int W, int min_chunks) {
  if (C <= 0) return 0;
  const int64_t cap = (C + min_chunks - 1) / min_chunks;
  return cap < W ? cap : W;
}

__device__ __forceinline__ int64_t wave_begin(int64_t w, int64_t C, int64_t We) {
  return w * C / We;
}

// The wavefront whose range holds chunk c (largest w with begin(w) <= c).
__device__ __forceinline__ int64_t wave_of_chunk(int64_t c, int64_t C, int64_t We) {
  return ((c + 1) * We - 1) / C;
}

// Largest b in [0, batch) with prefix[b] <= c, which is the sequence that
// holds chunk c (an empty sequence has prefix[b + 1] == prefix[b] and is
// skipped).  Requires c < prefix[batch].
__device__ __forceinline__ int seq_of_chunk(const int32_t* prefix, int batch, int64_t c) {
  int lo = 0, hi = batch;   // invariant: answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= c) lo = mid; else hi = mid;
  }
  return lo;
}

// Partial slot of (sequence b, KV head g) written by unit u.  For a fixed g
// both b and u increase along the chunk space, so b + u is unique per g.
__device__ __forceinline__ int64_t partial_slot(int b, int g, int64_t u, int kv_heads) {
  return ((int64_t)b + u) * kv_heads + g;
}

// Query heads of virtual KV head g.  The kv_group query heads of a pool KV
// head are split over qsplit virtual heads, virtual head k taking the
// floor-bounded range [k*kv_group/qsplit, (k+1)*kv_group/qsplit): sizes
// differ by at most one and none is empty (qsplit <= kv_group).
// Pool KV head of virtual head g.
__device__ __forceinline__ int vhead_pool_head(int g, int qsplit) {
  return qsplit == 1 ? g : g / qsplit;
}

struct VHead {
  int first;   // first query head (absolute index)
  int count;   // query heads served
};
__device__ __forceinline__ VHead vhead_rows(int g, int qsplit, int kv_group) {
  if (qsplit == 1) return VHead{g * kv_group, kv_group};   // the usual case: no divisions
  const int gp = g / qsplit;
  const int k = g - gp * qsplit;
  const int lo = k * kv_group / qsplit;
  const int hi = (k + 1) * kv_group / qsplit;
  return VHead{gp * kv_group + lo, hi - lo};
}

// The inverse: virtual head g of query head h and h's index within it.
__device__ __forceinline__ void vhead_of(int h, int qsplit, int kv_group, int* g, int* hn) {
  if (qsplit == 1) {
    *g = h / kv_group;
    *hn = h - *g * kv_group;
    return;
  }
  const int gp = h / kv_group;
  const int r = h - gp * kv_group;
  const int k = ((r + 1) * qsplit - 1) / kv_group;   // largest k with k*kv_group/qsplit <= r
  *g = gp * qsplit + k;
  *hn = r - k * kv_group / qsplit;
}

}  // namespace pagedkv
