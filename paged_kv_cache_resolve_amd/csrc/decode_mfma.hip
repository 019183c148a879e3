// Paged-attention decode, pass 1, bf16 pools, MFMA tiles on gfx950.
//
// What is computed ("vllmini: Building a Minimalist PagedAttention and KV
// Cache Engine", section "The CUDA Block Kernel"; "KV Cache and Attention
// Mechanisms", section 2): for every (sequence, query head) the logical
// token positions are resolved through the sequence's block table into
// physical blocks of the pool, and scaled q.K scores, a max-subtracted
// softmax and the weighted sum of V rows are formed.
//
// Mapping onto CDNA4.  One wavefront streams a contiguous range of 16-token
// chunks of one or more (sequence, KV head) pairs (decode_split.h).  All G
// query heads of the KV head are computed from the same K/V bytes, so each
// K/V byte is read from HBM once.  Per chunk:
//   * K tile [16 tokens x D] is loaded straight into the A-operand layout of
//     v_mfma_f32_16x16x32_bf16 (row = token = lane % 16, eight consecutive
//     dims per lane); Q^T (16 head columns, G used, rest zero) is the B
//     operand.  The result holds score(token 4*(lane/16)+r, head lane%16).
//   * Online softmax over those scores in fp32 (exp2 domain), with a
//     wave-uniform rescale only when some head's running max grows.
//   * The probabilities, rounded to bf16, are already in the B-operand
//     layout of v_mfma_f32_16x16x16_bf16 (k = token); V is loaded with
//     fully coalesced 16-byte rows (lane = token 4*(lane/16)+r, dims
//     VD*(lane%16)..) and transposed to the A operand with v_perm_b32.
//     The accumulator holds out^T: lane = head lane%16, 4*VD contiguous dims.
// The partition's block-table entries are prefetched into a VGPR (one entry
// per lane, the next window loaded one window ahead) and read back with
// v_readlane, so chunk addresses come from scalar registers.

#include <math.h>

#include "decode_split.h"
#include "internal.h"

namespace pagedkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D> struct VRow;
template <> struct VRow<128> { using type = uint4; };   // 8 bf16 per lane
template <> struct VRow<64> { using type = uint2; };    // 4 bf16 per lane

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ uint32_t dword_of(const uint2& v, int i) {
  return i == 0 ? v.x : v.y;
}

// Round two floats to bf16 (nearest even) and pack: lo = a, hi = b.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

template <int D>
struct ChunkBuf {
  uint4 k[D / 32];
  typename VRow<D>::type v[4];
};

template <int D>
__device__ __forceinline__ void zero_row(typename VRow<D>::type& v);
template <> __device__ __forceinline__ void zero_row<128>(uint4& v) { v = make_uint4(0, 0, 0, 0); }
template <> __device__ __forceinline__ void zero_row<64>(uint2& v) { v = make_uint2(0, 0); }

template <int D>
__device__ __forceinline__ void store_out_row(uint16_t* dst, const float* vals);
// 32 bf16 = 4 x 16-byte stores.
template <>
__device__ __forceinline__ void store_out_row<128>(uint16_t* dst, const float* v) {
  uint4* d = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d[i] = make_uint4(pack_bf16x2(v[8 * i + 0], v[8 * i + 1]), pack_bf16x2(v[8 * i + 2], v[8 * i + 3]),
                      pack_bf16x2(v[8 * i + 4], v[8 * i + 5]), pack_bf16x2(v[8 * i + 6], v[8 * i + 7]));
}
// 16 bf16 = 2 x 16-byte stores.
template <>
__device__ __forceinline__ void store_out_row<64>(uint16_t* dst, const float* v) {
  uint4* d = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    d[i] = make_uint4(pack_bf16x2(v[8 * i + 0], v[8 * i + 1]), pack_bf16x2(v[8 * i + 2], v[8 * i + 3]),
                      pack_bf16x2(v[8 * i + 4], v[8 * i + 5]), pack_bf16x2(v[8 * i + 6], v[8 * i + 7]));
}

template <int D>
struct Segment {
  static constexpr int NK = D / 32;   // K loads (16 B) per lane per chunk
  static constexpr int VD = D / 16;   // V dims per lane
  static constexpr int NW = VD / 2;   // dwords per lane per V row

  const DecodeParams& p;
  const int lane, n, quad;
  const int b, g, j0, j1, T;
  const char* khead;        // K slab of (layer, g) in block 0, in bytes
  const int32_t* trow;
  int tb0;                  // first logical block held in `tbl`
  int tbl, tbl_next;        // block-table window (one entry per lane)
  int last_blk;

  bf16x8_t qop[NK];
  f32x4_t acc[VD];
  float m, l;

  __device__ Segment(const DecodeParams& p_, int lane_, int b_, int g_, int j0_, int j1_)
      : p(p_), lane(lane_), n(lane_ & 15), quad(lane_ >> 4), b(b_), g(g_), j0(j0_), j1(j1_),
        T(p_.context_lens[b_]) {
    const int BS = p.pool.block_size;
    khead = p.pool.base + 2 * ((int64_t)p.layer * p.pool.layer_stride + (int64_t)g * p.pool.head_stride);
    trow = p.block_tables + (int64_t)b * p.max_blocks_per_seq;
    tb0 = (j0 * 16) / BS;
    last_blk = (j1 * 16 - 1) / BS;
    tbl = tb0 + lane <= last_blk ? trow[tb0 + lane] : 0;
    tbl_next = tb0 + 64 + lane <= last_blk ? trow[tb0 + 64 + lane] : 0;

    const int G = p.group;
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                           ((int64_t)b * p.num_q_heads + (int64_t)g * G + n) * D + 8 * quad;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < G) v = *reinterpret_cast<const uint4*>(qrow + 32 * j);
      qop[j] = as_bf16x8(v);
    }
#pragma unroll
    for (int c = 0; c < VD; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }

  // Byte address of the K slab rows of chunk j (tokens 16j .. 16j+15).
  __device__ __forceinline__ const char* chunk_base(int j) {
    const int BS = p.pool.block_size;
    const int blk = (j * 16) / BS;
    if (blk - tb0 >= 64) {           // uniform: slide the table window
      tb0 += 64;
      tbl = tbl_next;
      tbl_next = tb0 + 64 + lane <= last_blk ? trow[tb0 + 64 + lane] : 0;
    }
    const int phys = __builtin_amdgcn_readlane(tbl, blk - tb0);
    return khead + 2 * ((int64_t)phys * p.pool.block_stride + (int64_t)((j * 16) % BS) * D);
  }

  __device__ __forceinline__ void load(ChunkBuf<D>& cb, int j) {
    const char* kb = chunk_base(j);
    const char* vb = kb + 2 * p.pool.kv_stride;
    const char* kl = kb + 2 * (n * D + 8 * quad);
#pragma unroll
    for (int i = 0; i < NK; ++i) cb.k[i] = *reinterpret_cast<const uint4*>(kl + 64 * i);
    const char* vl = vb + 2 * (4 * quad * D + VD * n);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      cb.v[r] = *reinterpret_cast<const typename VRow<D>::type*>(vl + 2 * r * D);
  }

  __device__ __forceinline__ void compute(ChunkBuf<D>& cb, int j) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NK; ++i)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cb.k[i]), qop[i], s, 0, 0, 0);

    const int tok0 = j * 16 + 4 * quad;
    const bool tail = j * 16 + 16 > T;   // uniform
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = s[r] * p.scale_log2;
      if (tail && tok0 + r >= T) sv[r] = -INFINITY;
    }
    float bmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    if (__any(bmax > m)) {
      const float mn = fmaxf(m, bmax);
      const float alpha = exp2f(m - mn);
#pragma unroll
      for (int c = 0; c < VD; ++c) acc[c] *= alpha;
      l *= alpha;
      m = mn;
    }
    const uint32_t p01 = pack_bf16x2(exp2f(sv[0] - m), exp2f(sv[1] - m));
    const uint32_t p23 = pack_bf16x2(exp2f(sv[2] - m), exp2f(sv[3] - m));
    l += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
    const s16x4_t pop = __builtin_bit_cast(s16x4_t, make_uint2(p01, p23));

    if (tail) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (tok0 + r >= T) zero_row<D>(cb.v[r]);
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t v0 = dword_of(cb.v[0], w), v1 = dword_of(cb.v[1], w);
      const uint32_t v2 = dword_of(cb.v[2], w), v3 = dword_of(cb.v[3], w);
      const uint2 ev = make_uint2(__builtin_amdgcn_perm(v1, v0, 0x05040100u),
                                  __builtin_amdgcn_perm(v3, v2, 0x05040100u));
      const uint2 od = make_uint2(__builtin_amdgcn_perm(v1, v0, 0x07060302u),
                                  __builtin_amdgcn_perm(v3, v2, 0x07060302u));
      acc[2 * w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          __builtin_bit_cast(s16x4_t, ev), pop, acc[2 * w], 0, 0, 0);
      acc[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          __builtin_bit_cast(s16x4_t, od), pop, acc[2 * w + 1], 0, 0, 0);
    }
  }

  __device__ void run() {
    ChunkBuf<D> c0, c1;
    load(c0, j0);
    for (int j = j0; j < j1; j += 2) {
      if (j + 1 < j1) load(c1, j + 1);
      compute(c0, j);
      if (j + 1 >= j1) break;
      if (j + 2 < j1) load(c0, j + 2);
      compute(c1, j + 1);
    }
  }

  __device__ void finish(int nb, int64_t wave) {
    const int G = p.group;
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    if (n >= G) return;
    // lane holds dims 4*VD*quad + VD*r + c of head n as acc[c][r]
    float vals[4 * VD];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < VD; ++c) vals[VD * r + c] = acc[c][r];
    const int pair = b * p.pool.kv_heads + g;
    if (j0 == 0 && j1 == nb) {
      const float inv = 1.0f / lt;
#pragma unroll
      for (int i = 0; i < 4 * VD; ++i) vals[i] *= inv;
      uint16_t* dst = static_cast<uint16_t*>(p.out) +
                      ((int64_t)b * p.num_q_heads + (int64_t)g * G + n) * D + 4 * VD * quad;
      store_out_row<D>(dst, vals);
    } else {
      const int64_t slot = pair + wave;
      float4* o = reinterpret_cast<float4*>(p.ws_o + (slot * G + n) * D + 4 * VD * quad);
#pragma unroll
      for (int i = 0; i < VD; ++i)
        o[i] = make_float4(vals[4 * i], vals[4 * i + 1], vals[4 * i + 2], vals[4 * i + 3]);
      if (quad == 0) {
        p.ws_ml[(slot * G + n) * 2 + 0] = m;
        p.ws_ml[(slot * G + n) * 2 + 1] = lt;
      }
    }
  }
};

template <int D>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeParams p) {
  extern __shared__ int32_t prefix[];
  __shared__ int32_t scan[256];
  block_chunk_prefix<256>(p.context_lens, p.batch, kMfmaChunk, prefix, scan);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= p.batch; i += 256) p.ws_prefix[i] = prefix[i];

  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H = p.pool.kv_heads;
  const int64_t C = (int64_t)H * prefix[p.batch];
  const int64_t We = waves_eff(C, p.waves, p.min_chunks);
  if (wave >= We) return;
  int64_t c = wave_begin(wave, C, We);
  const int64_t c_end = wave_begin(wave + 1, C, We);
  int b = seq_of_chunk(prefix, p.batch, c, H);
  while (c < c_end) {
    const int pb = prefix[b];
    const int nb = prefix[b + 1] - pb;
    const int64_t base = (int64_t)H * pb;
    const int rel = (int)(c - base);
    const int g = rel / nb;
    const int j0 = rel - g * nb;
    const int64_t left = c_end - c;
    const int j1 = left < (int64_t)(nb - j0) ? j0 + (int)left : nb;
    {
      Segment<D> seg(p, lane, b, g, j0, j1);
      seg.run();
      seg.finish(nb, wave);
    }
    c += j1 - j0;
    if (c >= base + (int64_t)H * nb) {
      ++b;
      while (b < p.batch && prefix[b + 1] == prefix[b]) ++b;
    }
  }
}

}  // namespace

bool mfma_supported(const kv_pool* pool, int group) {
  return pool->dtype == PAGEDKV_BF16 && (pool->head_dim == 64 || pool->head_dim == 128) &&
         pool->block_size % 16 == 0 && group >= 1 && group <= kMaxGroup;
}

hipError_t launch_decode_mfma(DecodeParams& p, hipStream_t s) {
  const size_t lds = sizeof(int32_t) * (p.batch + 1);
  const void* fn = p.pool.head_dim == 128 ? reinterpret_cast<const void*>(&decode_mfma_kernel<128>)
                                          : reinterpret_cast<const void*>(&decode_mfma_kernel<64>);
  int wgs = 0;
  hipError_t e = resident_workgroups(fn, 256, lds, &wgs);
  if (e != hipSuccess) return e;
  int waves = wgs * 4;
  if (waves > kMaxWaves) waves = kMaxWaves;
  p.waves = waves;
  if (p.min_chunks < 1) p.min_chunks = 4;
  const dim3 grid((waves + 3) / 4), block(256);
  if (p.pool.head_dim == 128)
    hipLaunchKernelGGL(decode_mfma_kernel<128>, grid, block, lds, s, p);
  else
    hipLaunchKernelGGL(decode_mfma_kernel<64>, grid, block, lds, s, p);
  return hipGetLastError();
}

}  // namespace pagedkv
