// Paged-attention decode, merge pass: combine the partial results of every
// (sequence, KV head) pair whose chunks were split across work units.
//
// A partial k holds, per query head, the running max m_k (log2 units), the
// sum l_k of exp2(s - m_k) and the unnormalised output o_k over its chunks.
// With M = max_k m_k and w_k = exp2(m_k - M):
//     out = (sum_k w_k o_k) / (sum_k w_k l_k),
// the softmax-weighted V sum over the whole context.  M is found first, so
// every partial row can then be loaded independently (eight per thread in
// flight).  Pairs of empty sequences (T_b = 0) get zero rows.

#include <math.h>

#include "decode_split.h"
#include "internal.h"

namespace pagedkv {
namespace {

constexpr int kThreads = 256;

template <typename TS> __device__ __forceinline__ TS out_cast(float x);
template <> __device__ __forceinline__ float out_cast<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t out_cast<uint16_t>(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// One workgroup per (pair, query head of the pair's group).  Thread t owns
// dim t % D of every partial k with k % S == t / D (S = 256 / D threads share
// a dim), so up to S * 8 partial rows are in flight at once.
template <typename TS>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecodeParams p) {
  __shared__ float red[kThreads];
  __shared__ float red_l[kThreads];
  const int H = p.pool.kv_heads;
  const int G = p.group;
  const int D = p.pool.head_dim;
  const int pair = blockIdx.x / G;
  const int hn = blockIdx.x - pair * G;
  const int b = pair / H;
  const int g = pair - b * H;
  TS* out = static_cast<TS*>(p.out) + ((int64_t)b * p.num_q_heads + (int64_t)g * G + hn) * D;

  const int pb = p.ws_prefix[b];
  const int nb = p.ws_prefix[b + 1] - pb;
  if (nb == 0) {
    for (int i = threadIdx.x; i < D; i += kThreads) out[i] = out_cast<TS>(0.f);
    return;
  }
  const int64_t C = p.ws_prefix[p.batch];
  const int64_t Ue = waves_eff(C, p.units, p.min_chunks);
  const int64_t uf = wave_of_chunk(pb, C, Ue);
  const int64_t ul = wave_of_chunk(pb + nb - 1, C, Ue);
  if (uf == ul) return;   // one unit saw the whole sequence and wrote `out`
  const int K = (int)(ul - uf + 1);
  // partials of (b, g) from units uf..ul sit kv_heads slots apart
  const int64_t slot0 = partial_slot(b, g, uf, H);

  // global max of the partials' running maxima
  float M = -INFINITY;
  for (int k = threadIdx.x; k < K; k += kThreads)
    M = fmaxf(M, p.ws_ml[((slot0 + (int64_t)k * H) * G + hn) * 2]);
  red[threadIdx.x] = M;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  M = red[0];
  __syncthreads();

  const int S = kThreads / D;            // threads per dim (D <= 256)
  const int d = threadIdx.x % D;
  const int sp = threadIdx.x / D;
  float a = 0.f, L = 0.f;
  if (sp < S) {
    const int64_t stride_o = (int64_t)H * G * D;   // next unit's partial of (b, g)
    const int64_t stride_m = (int64_t)H * G * 2;
    const float* ob = p.ws_o + (slot0 * G + hn) * (int64_t)D + d;
    const float* mb = p.ws_ml + (slot0 * G + hn) * 2;
    int k = sp;
    for (; k + 7 * S < K; k += 8 * S) {
      float ov[8], mv[8], lv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ov[u] = ob[(int64_t)(k + u * S) * stride_o];
        mv[u] = mb[(int64_t)(k + u * S) * stride_m];
        lv[u] = mb[(int64_t)(k + u * S) * stride_m + 1];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = __builtin_amdgcn_exp2f(mv[u] - M);
        a += w * ov[u];
        L += w * lv[u];
      }
    }
    for (; k < K; k += S) {
      const float w = __builtin_amdgcn_exp2f(mb[(int64_t)k * stride_m] - M);
      a += w * ob[(int64_t)k * stride_o];
      L += w * mb[(int64_t)k * stride_m + 1];
    }
  }
  red[threadIdx.x] = a;
  red_l[threadIdx.x] = L;
  __syncthreads();
  if (threadIdx.x < D) {
    float at = 0.f, lt = 0.f;
    for (int s2 = 0; s2 < S; ++s2) {
      at += red[s2 * D + threadIdx.x];
      lt += red_l[s2 * D + threadIdx.x];
    }
    out[threadIdx.x] = out_cast<TS>(at / lt);
  }
}

}  // namespace

hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t s) {
  const int64_t blocks = (int64_t)p.batch * p.pool.kv_heads * p.group;
  if (blocks == 0) return hipSuccess;
  if (p.dtype == PAGEDKV_F32)
    hipLaunchKernelGGL(decode_merge_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(decode_merge_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       p);
  return hipGetLastError();
}

}  // namespace pagedkv
