// Paged-attention decode, merge pass: combine the partial results of every
// (sequence, KV head) pair whose chunks were split across work units.
//
// A partial k holds, per query head, the running max m_k (log2 units), the
// sum l_k of exp2(s - m_k) and the unnormalised output o_k over its chunks.
// With M = max_k m_k and w_k = exp2(m_k - M):
//     out = (sum_k w_k o_k) / (sum_k w_k l_k),
// the softmax-weighted V sum over the whole context, accumulated here with
// an online (running-max) update.  Empty sequences (T_b = 0) get zero rows,
// and so does a (sequence, head) with nothing attended (a dense batch whose
// mask is all zero): partials with m_k = -inf are skipped.
//
// For a fused append, this pass also stores each sequence's new K/V rows
// into the pool: pass 1 read them from the k_new / v_new inputs, so the pool
// copy is only needed by later calls.

#include <math.h>

#include <type_traits>

#include "decode_split.h"
#include "internal.h"

namespace pagedkv {
namespace {

constexpr int kDimsPerLane = 4;   // head_dim <= 256

template <typename TS> __device__ __forceinline__ TS out_cast(float x);
template <> __device__ __forceinline__ float out_cast<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t out_cast<uint16_t>(float x) {   // bf16
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
template <> __device__ __forceinline__ _Float16 out_cast<_Float16>(float x) { return (_Float16)x; }

// One wavefront per (sequence b, query head h).  Every lane reads the same
// (m_k, l_k) of each partial and its own dims of o_k, eight or sixteen
// partials per round of loads, and folds them in with an online
// log-sum-exp; there is no cross-lane traffic at all.
template <typename TS>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p) {
  const int H = p.vheads;   // (virtual) KV heads
  const int G = p.group;    // partial slot stride
  const int D = p.pool.head_dim;
  const int lane = threadIdx.x;
  const int b = blockIdx.x / p.num_q_heads;
  const int h = blockIdx.x - b * p.num_q_heads;
  int g, hn;   // virtual KV head of h and h's column in it
  vhead_of(h, p.qsplit, p.kv_group, &g, &hn);
  const int gp = vhead_pool_head(g, p.qsplit);   // the pool's KV head
  TS* out = static_cast<TS*>(p.out) + ((int64_t)b * p.num_q_heads + h) * D;

  // Independent loads first: the sequence's chunk range and, for a fused
  // append, its position and the new K/V row (one 16-byte unit per lane;
  // fused appends come with head_dim * element size <= 256 bytes, so one
  // pass of 64 lanes covers both rows).
  const bool app =
      p.positions != nullptr && hn == 0 && (p.qsplit == 1 || g % p.qsplit == 0);
  const int units = D * (int)sizeof(TS) / 16;   // 16-byte units per row
  const int kv = lane >= units;
  const int u = lane - kv * units;
  int pos = -1;
  uint4 row_unit = make_uint4(0, 0, 0, 0);
  if (app) {
    pos = p.positions[b];
    if (lane < 2 * units)
      row_unit = reinterpret_cast<const uint4*>(static_cast<const TS*>(kv ? p.v_new : p.k_new) +
                                                ((int64_t)b * p.pool.kv_heads + gp) * D)[u];
  }
  const int pb = p.ws_prefix[b];
  const int nb = p.ws_prefix[b + 1] - pb;
  const int64_t C = p.ws_prefix[p.batch];
  // the first wave of each (b, pool head) stores the new token of that head; the
  // store is made at every exit so that the table load overlaps the merge
  const bool store_row = app && pos >= 0 && lane < 2 * units;
  const int phys =
      store_row ? p.block_tables[(int64_t)b * p.max_blocks_per_seq + pos / p.pool.block_size] : 0;
  auto append_row = [&]() {
    if (!store_row) return;
    const int64_t row = (int64_t)phys * p.pool.block_stride + (int64_t)p.layer * p.pool.layer_stride +
                        (int64_t)gp * p.pool.head_stride + (int64_t)(pos % p.pool.block_size) * D;
    reinterpret_cast<uint4*>(reinterpret_cast<TS*>(const_cast<char*>(p.pool.base)) + row +
                             kv * p.pool.kv_stride)[u] = row_unit;
  };
  if (nb == 0) {
    for (int d = lane; d < D; d += 64) out[d] = out_cast<TS>(0.f);
    append_row();
    return;
  }
  const int64_t Ue = waves_eff(C, p.units, p.min_chunks);
  const int64_t uf = wave_of_chunk(pb, C, Ue);
  const int64_t ul = wave_of_chunk(pb + nb - 1, C, Ue);
  if (uf == ul) {   // one unit saw the whole sequence and wrote `out`
    append_row();
    return;
  }
  const int K = (int)(ul - uf + 1);

  // partials of (b, g) from units uf..ul sit H slots apart
  const int64_t slot0 = partial_slot(b, g, uf, H);
  const int64_t stride_o = (int64_t)H * G * D;
  const int64_t stride_m = (int64_t)H * G * 2;
  const float* ob = p.ws_o + (slot0 * G + hn) * (int64_t)D;
  const float* mb = p.ws_ml + (slot0 * G + hn) * 2;

  float M = -INFINITY, L = 0.f, a[kDimsPerLane];
#pragma unroll
  for (int i = 0; i < kDimsPerLane; ++i) a[i] = 0.f;

  // One round: the loads of partials k0 .. k0+N-1 are issued together, then
  // folded in order.  Up to 8 partials (the usual case) take one round of 8;
  // more take rounds of 16, one memory round trip per 16 partials.
  auto fold_round = [&](int k0, auto n) {
    constexpr int N = decltype(n)::value;
    float mv[N], lv[N], ov[N][kDimsPerLane];
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int k = min(k0 + u, K - 1);   // duplicates past K are skipped below
      mv[u] = mb[(int64_t)k * stride_m];
      lv[u] = mb[(int64_t)k * stride_m + 1];
#pragma unroll
      for (int i = 0; i < kDimsPerLane; ++i) {
        const int d = lane + 64 * i;
        ov[u][i] = d < D ? ob[(int64_t)k * stride_o + d] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < N; ++u) {
      if (k0 + u >= K) break;
      if (mv[u] == -INFINITY) continue;   // a partial with every token masked (dense decode)
      const float Mn = fmaxf(M, mv[u]);
      const float sc = __builtin_amdgcn_exp2f(M - Mn);
      const float w = __builtin_amdgcn_exp2f(mv[u] - Mn);
      L = L * sc + w * lv[u];
#pragma unroll
      for (int i = 0; i < kDimsPerLane; ++i) a[i] = a[i] * sc + w * ov[u][i];
      M = Mn;
    }
  };
  int k0 = 0;
  for (; K - k0 > 8; k0 += 16) fold_round(k0, std::integral_constant<int, 16>());
  for (; k0 < K; k0 += 8) fold_round(k0, std::integral_constant<int, 8>());
  const float inv = L > 0.f ? 1.0f / L : 0.f;   // nothing attended: zeros
#pragma unroll
  for (int i = 0; i < kDimsPerLane; ++i) {
    const int d = lane + 64 * i;
    if (d < D) out[d] = out_cast<TS>(a[i] * inv);
  }
  append_row();
}

}  // namespace

hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.batch * p.num_q_heads;
  if (blocks == 0) return hipSuccess;
  if (p.dtype == PAGEDKV_F32)
    hipLaunchKernelGGL(decode_merge_kernel<float>, dim3((unsigned)blocks), dim3(64), 0, s, p);
  else if (p.dtype == PAGEDKV_F16)
    hipLaunchKernelGGL(decode_merge_kernel<_Float16>, dim3((unsigned)blocks), dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(decode_merge_kernel<uint16_t>, dim3((unsigned)blocks), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace pagedkv
