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

// Each lane merges four consecutive dims of one query head (a float4 of the
// partials): a head takes lph = head_dim / 4 lanes and a wavefront serves
// hpp = 64 / lph heads of one (sequence, virtual KV head) pair (two at
// head_dim 128, four at 64), so a pair of G query heads takes ceil(G / hpp)
// wavefronts.
__device__ __forceinline__ int merge_lanes_per_head(int head_dim) { return head_dim >> 2; }
__device__ __forceinline__ int merge_heads_per_wave(int head_dim) { return 64 / (head_dim >> 2); }

template <typename TS> __device__ __forceinline__ void store4(TS* dst, float4 v);
template <> __device__ __forceinline__ void store4<float>(float* dst, float4 v) {
  *reinterpret_cast<float4*>(dst) = v;
}
template <> __device__ __forceinline__ void store4<uint16_t>(uint16_t* dst, float4 v) {   // bf16
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  bf16x4_t r;
  r[0] = (__bf16)v.x;
  r[1] = (__bf16)v.y;
  r[2] = (__bf16)v.z;
  r[3] = (__bf16)v.w;
  *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, r);
}
template <> __device__ __forceinline__ void store4<_Float16>(_Float16* dst, float4 v) {
  typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
  f16x4_t r;
  r[0] = (_Float16)v.x;
  r[1] = (_Float16)v.y;
  r[2] = (_Float16)v.z;
  r[3] = (_Float16)v.w;
  *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, r);
}

// One wavefront per hpp query heads of a (sequence b, virtual KV head g)
// pair.  Each lane reads the (m_k, l_k) of its head and its four dims of
// o_k for every partial, eight or sixteen partials per round of loads, and
// folds them in with an online log-sum-exp; there is no cross-lane traffic.
template <typename TS>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p) {
  const int H = p.vheads;   // (virtual) KV heads
  const int G = p.group;    // partial slot stride (most query heads per virtual head)
  const int D = p.pool.head_dim;
  const int lane = threadIdx.x;
  const int lph = merge_lanes_per_head(D);
  const int hpp = merge_heads_per_wave(D);
  const int wpv = (G + hpp - 1) / hpp;   // wavefronts per virtual head
  int x = blockIdx.x;
  const int wi = x % wpv;
  x /= wpv;
  const int b = x / H;
  const int g = x - b * H;
  const int gp = vhead_pool_head(g, p.qsplit);   // the pool's KV head
  const VHead vh = vhead_rows(g, p.qsplit, p.kv_group);
  const int hs = lane / lph;            // this lane's head among the wavefront's
  const int dg = lane - hs * lph;       // and its dims 4*dg .. 4*dg + 3
  const int hc0 = wi * hpp + hs;        // head column within the virtual head
  const bool mine = hs < hpp && hc0 < vh.count;
  const int hc = mine ? hc0 : 0;        // idle lanes read head 0 and store nothing
  TS* out = static_cast<TS*>(p.out) + ((int64_t)b * p.num_q_heads + vh.first + hc) * D + 4 * dg;

  // Independent loads first: the sequence's chunk range and, for a fused
  // append, its position and the new K/V row (one 16-byte unit per lane;
  // fused appends come with head_dim * element size <= 256 bytes, so one
  // pass of 64 lanes covers both rows).
  const bool app =
      p.positions != nullptr && wi == 0 && (p.qsplit == 1 || g % p.qsplit == 0);
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
    if (mine) store4<TS>(out, make_float4(0.f, 0.f, 0.f, 0.f));
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
  const float* ob = p.ws_o + (slot0 * G + hc) * (int64_t)D + 4 * dg;
  const float* mb = p.ws_ml + (slot0 * G + hc) * 2;

  float M = -INFINITY, L = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);

  // One round: the loads of partials k0 .. k0+N-1 are issued together, then
  // folded in order.  Up to 8 partials (the usual case) take one round of 8;
  // more take rounds of 16, one memory round trip per 16 partials.
  auto fold_round = [&](int k0, auto n) {
    constexpr int N = decltype(n)::value;
    float mv[N], lv[N];
    float4 ov[N];
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int k = min(k0 + u, K - 1);   // duplicates past K are skipped below
      mv[u] = mb[(int64_t)k * stride_m];
      lv[u] = mb[(int64_t)k * stride_m + 1];
      ov[u] = *reinterpret_cast<const float4*>(ob + (int64_t)k * stride_o);
    }
#pragma unroll
    for (int u = 0; u < N; ++u) {
      if (k0 + u >= K) break;
      if (mv[u] == -INFINITY) continue;   // a partial with every token masked (dense decode)
      const float Mn = fmaxf(M, mv[u]);
      const float sc = __builtin_amdgcn_exp2f(M - Mn);
      const float w = __builtin_amdgcn_exp2f(mv[u] - Mn);
      L = L * sc + w * lv[u];
      a.x = a.x * sc + w * ov[u].x;
      a.y = a.y * sc + w * ov[u].y;
      a.z = a.z * sc + w * ov[u].z;
      a.w = a.w * sc + w * ov[u].w;
      M = Mn;
    }
  };
  int k0 = 0;
  for (; K - k0 > 8; k0 += 16) fold_round(k0, std::integral_constant<int, 16>());
  for (; k0 < K; k0 += 8) fold_round(k0, std::integral_constant<int, 8>());
  const float inv = L > 0.f ? 1.0f / L : 0.f;   // nothing attended: zeros
  if (mine) store4<TS>(out, make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv));
  append_row();
}

}  // namespace

hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t s) {
  const int hpp = 64 / (p.pool.head_dim / 4);   // query heads per wavefront
  const int64_t blocks = (int64_t)p.batch * p.vheads * ((p.group + hpp - 1) / hpp);
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
