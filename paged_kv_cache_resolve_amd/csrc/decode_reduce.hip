// Paged-attention decode, pass 2: merge the partial results of every
// (sequence, KV head) pair whose chunks were split across wavefronts.
//
// Each partial k holds, per query head, the running max m_k (log2 units),
// the sum l_k of exp2(s - m_k) and the unnormalised output o_k over its
// chunks.  With M = max_k m_k and w_k = exp2(m_k - M):
//     out = (sum_k w_k o_k) / (sum_k w_k l_k),
// which equals the softmax-weighted V sum over the whole context.  A pair
// with no tokens (T_b = 0) gets a zero output row.

#include <math.h>

#include "decode_split.h"
#include "internal.h"

namespace pagedkv {
namespace {

template <typename TS> __device__ __forceinline__ TS out_cast(float x);
template <> __device__ __forceinline__ float out_cast<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t out_cast<uint16_t>(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <typename TS>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeParams p, int ct) {
  const int H = p.pool.kv_heads;
  const int pair = blockIdx.x;
  const int b = pair / H;
  const int g = pair - b * H;
  const int G = p.group;
  const int D = p.pool.head_dim;
  TS* out = static_cast<TS*>(p.out) + ((int64_t)b * p.num_q_heads + (int64_t)g * G) * D;

  const int pb = p.ws_prefix[b];
  const int nb = p.ws_prefix[b + 1] - pb;
  if (nb == 0) {
    for (int i = threadIdx.x; i < G * D; i += blockDim.x) out[i] = out_cast<TS>(0.f);
    return;
  }
  const int64_t C = (int64_t)H * p.ws_prefix[p.batch];
  const int64_t We = waves_eff(C, p.waves, p.min_chunks);
  const int64_t first = (int64_t)H * pb + (int64_t)g * nb;
  const int64_t wf = wave_of_chunk(first, C, We);
  const int64_t wl = wave_of_chunk(first + nb - 1, C, We);
  if (wf == wl) return;   // one wavefront covered the pair and wrote `out`

  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int n = i / D;
    const int d = i - n * D;
    float M = -INFINITY;
    for (int64_t w = wf; w <= wl; ++w) M = fmaxf(M, p.ws_ml[((pair + w) * G + n) * 2]);
    float L = 0.f, acc = 0.f;
    for (int64_t w = wf; w <= wl; ++w) {
      const int64_t slot = pair + w;
      const float sc = __builtin_amdgcn_exp2f(p.ws_ml[(slot * G + n) * 2] - M);
      L += sc * p.ws_ml[(slot * G + n) * 2 + 1];
      acc += sc * p.ws_o[(slot * G + n) * D + d];
    }
    out[i] = out_cast<TS>(acc / L);
  }
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeParams& p, int chunk_tokens, hipStream_t s) {
  const int pairs = p.batch * p.pool.kv_heads;
  if (pairs == 0) return hipSuccess;
  if (p.dtype == PAGEDKV_F32)
    hipLaunchKernelGGL(decode_reduce_kernel<float>, dim3(pairs), dim3(256), 0, s, p, chunk_tokens);
  else
    hipLaunchKernelGGL(decode_reduce_kernel<uint16_t>, dim3(pairs), dim3(256), 0, s, p, chunk_tokens);
  return hipGetLastError();
}

}  // namespace pagedkv
