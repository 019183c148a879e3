// Paged-attention decode, pass 1, general shapes (fp32, bf16 or fp16 pools, any
// block size, head_dim a multiple of 4 up to 256, up to 16 query heads per
// wavefront; larger groups arrive split into virtual KV heads), plain VALU
// arithmetic.
//
// Same computation as the MFMA kernel ("vllmini", section "The CUDA Block
// Kernel": per (sequence, head), resolve logical positions through the block
// table and attend over the physical pages) and the same head-group work
// split (internal.h), with 64-token chunks and one wavefront per workgroup:
//   * scores: lane t owns token t of the chunk, resolves its own block-table
//     entry, and forms the G dot products against q (held in LDS, already
//     multiplied by scale*log2(e));
//   * online softmax per head with wavefront max/sum reductions;
//   * weighted V sum: lane owns dims lane, lane+64, ...; token rows are
//     walked in order with addresses broadcast by v_readlane.
// Loads are issued in batches (16 K pieces per lane, then 32 / DPL V rows)
// so that a chunk costs a few memory round trips, not one per load.

#include <math.h>

#include "decode_split.h"
#include "internal.h"

namespace pagedkv {
namespace {

constexpr int kGenDimsPerLane = 4;   // head_dim <= 256
constexpr int kKBatch = 16;          // 4-element K pieces per lane in flight

// Storage types: float (fp32), uint16_t (bf16 bit patterns), _Float16 (fp16).
template <typename TS> __device__ __forceinline__ float to_f32(TS x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) {
  return __uint_as_float((uint32_t)x << 16);
}
template <> __device__ __forceinline__ float to_f32<_Float16>(_Float16 x) { return (float)x; }
template <typename TS> __device__ __forceinline__ TS from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }

// Four consecutive K elements as floats (16-byte or 8-byte load).  K and V
// are streamed once, so their loads are non-temporal.
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 load4(const float* p) {
  const f32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const u32x2_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(p));
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}
// fp16 from its 16 bits.  The halves are taken out of each loaded dword with
// integer shifts: bit-casting the loaded vector's elements straight to half
// pairs made this compiler load one dword and use it for both pairs.
__device__ __forceinline__ float half_bits(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}
__device__ __forceinline__ float4 load4(const _Float16* p) {
  const u32x2_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(p));
  return make_float4(half_bits(v.x & 0xffffu), half_bits(v.x >> 16), half_bits(v.y & 0xffffu),
                     half_bits(v.y >> 16));
}
__device__ __forceinline__ float load1(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float load1(const _Float16* p) {
  return half_bits(__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p)));
}
__device__ __forceinline__ float load1(const uint16_t* p) {
  return __uint_as_float((uint32_t)__builtin_nontemporal_load(p) << 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// DPL = dims per lane in the V sum (head_dim <= 64 * DPL).
template <typename TS, int DPL>
__device__ __forceinline__ void generic_segment(const DecodeParams& p, float* qs, float* ps, int lane,
                                int64_t unit, int b, int g, int j0, int j1, int nb) {
  constexpr int VB = 32 / DPL;   // V rows in flight per batch
  const int GS = p.group;   // partial slot stride
  const VHead vh = vhead_rows(g, p.qsplit, p.kv_group);
  const int G = vh.count;   // query heads of this (virtual) KV head
  const int D = p.pool.head_dim;
  const int BS = p.pool.block_size;
  const int T = p.context_lens[b];
  const TS* pool = reinterpret_cast<const TS*>(p.pool.base);
  // g is a virtual KV head; the pool's head is g / qsplit
  const int64_t head_off =
      (int64_t)p.layer * p.pool.layer_stride + (int64_t)vhead_pool_head(g, p.qsplit) * p.pool.head_stride;
  const int32_t* trow = p.block_tables + (int64_t)b * p.max_blocks_per_seq;

  // q rows of the group, pre-multiplied by scale*log2(e)
  const TS* q = static_cast<const TS*>(p.q) + ((int64_t)b * p.num_q_heads + vh.first) * D;
  for (int i = lane; i < G * D; i += 64) qs[i] = to_f32<TS>(q[i]) * p.scale_log2;
  __syncthreads();

  float acc[kMaxGroup][DPL];
  float m[kMaxGroup], l[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[h][i] = 0.f;
  }

  for (int j = j0; j < j1; ++j) {
    const int tok = j * kGenericChunk + lane;
    const bool valid = tok < T;
    int64_t row = 0;   // element offset of this lane's token row (K); V adds kv_stride
    if (valid) {
      const int phys = trow[tok / BS];
      row = (int64_t)phys * p.pool.block_stride + head_off + (int64_t)(tok % BS) * D;
    }
    float s[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) s[h] = 0.f;
    for (int d0 = 0; d0 < D; d0 += 4 * kKBatch) {
      // Unconditional loads (a lane past T reads row 0 of the pool, a piece
      // past D re-reads the row's last piece; both are discarded below), so
      // that the whole batch is in flight before the first use.
      float4 kk[kKBatch];
#pragma unroll
      for (int u = 0; u < kKBatch; ++u) kk[u] = load4(pool + row + min(d0 + 4 * u, D - 4));
#pragma unroll
      for (int u = 0; u < kKBatch; ++u) {
        const int d = d0 + 4 * u;
        if (d < D) {
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h) {
            if (h < G) {
              const float4 qq = *reinterpret_cast<const float4*>(qs + h * D + d);
              s[h] += qq.x * kk[u].x + qq.y * kk[u].y + qq.z * kk[u].z + qq.w * kk[u].w;
            }
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < G) {
        const float sv = valid ? s[h] : -INFINITY;
        const float mn = fmaxf(m[h], wave_max(sv));
        const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
        const float pv = __builtin_amdgcn_exp2f(sv - mn);
        l[h] = l[h] * alpha + wave_sum(pv);
        m[h] = mn;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[h][i] *= alpha;
        ps[h * 64 + lane] = pv;
      }
    }
    __syncthreads();
    const int ntok = min(64, T - j * kGenericChunk);
    const uint32_t row_lo = (uint32_t)(row & 0xffffffffu);
    const uint32_t row_hi = (uint32_t)(row >> 32);
    // V rows VB at a time: the loads of a batch are independent, so they are
    // in flight together instead of one round trip per token.
    for (int t0 = 0; t0 < ntok; t0 += VB) {
      float v[VB][DPL];
#pragma unroll
      for (int u = 0; u < VB; ++u) {
        const int t = min(t0 + u, ntok - 1);   // repeats past ntok are skipped below
        const int64_t r = ((int64_t)(uint32_t)__builtin_amdgcn_readlane((int)row_hi, t) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)row_lo, t);
        const TS* vrow = pool + r + p.pool.kv_stride;
#pragma unroll
        for (int i = 0; i < DPL; ++i) v[u][i] = load1(vrow + min(lane + 64 * i, D - 1));
      }
#pragma unroll
      for (int u = 0; u < VB; ++u) {
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h)
          if (h < G && t0 + u < ntok) {
            const float pw = ps[h * 64 + t0 + u];
#pragma unroll
            for (int i = 0; i < DPL; ++i) acc[h][i] += pw * v[u][i];
          }
      }
    }
    __syncthreads();
  }

  const bool whole = (j0 == 0 && j1 == nb);
  const int64_t slot = partial_slot(b, g, unit, p.vheads);
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h >= G) continue;
    if (whole) {
      TS* o = static_cast<TS*>(p.out) + ((int64_t)b * p.num_q_heads + vh.first + h) * D;
      const float inv = 1.0f / l[h];
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int d = lane + 64 * i;
        if (d < D) o[d] = from_f32<TS>(acc[h][i] * inv);
      }
    } else {
      float* o = p.ws_o + (slot * GS + h) * D;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int d = lane + 64 * i;
        if (d < D) o[d] = acc[h][i];
      }
      if (lane == 0) {
        p.ws_ml[(slot * GS + h) * 2 + 0] = m[h];
        p.ws_ml[(slot * GS + h) * 2 + 1] = l[h];
      }
    }
  }
}

template <typename TS, int DPL>
__global__ __launch_bounds__(64) void decode_generic_kernel(DecodeParams p) {
  extern __shared__ int32_t lds[];
  __shared__ int32_t scan[1];
  int32_t* prefix = lds;
  // q (G x D floats) and probabilities (G x 64 floats) after the prefix
  const int pre_words = ((p.batch + 1) + 3) & ~3;
  float* qs = reinterpret_cast<float*>(lds + pre_words);
  float* ps = qs + p.group * p.pool.head_dim;

  block_chunk_prefix<64>(p.context_lens, p.batch, kGenericChunk, prefix, scan);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= p.batch; i += 64) p.ws_prefix[i] = prefix[i];

  const int lane = threadIdx.x;
  const int H = p.vheads;
  const int64_t unit = blockIdx.x / H;
  const int g = (int)(blockIdx.x - unit * H);
  const int64_t C = prefix[p.batch];
  const int64_t Ue = waves_eff(C, p.units, p.min_chunks);
  if (unit >= Ue) return;
  int64_t c = wave_begin(unit, C, Ue);
  const int64_t c_end = wave_begin(unit + 1, C, Ue);
  int b = seq_of_chunk(prefix, p.batch, c);
  while (c < c_end) {
    const int pb = prefix[b];
    const int nb = prefix[b + 1] - pb;
    const int j0 = (int)(c - pb);
    const int64_t left = c_end - c;
    const int j1 = left < (int64_t)(nb - j0) ? j0 + (int)left : nb;
    generic_segment<TS, DPL>(p, qs, ps, lane, unit, b, g, j0, j1, nb);
    __syncthreads();
    c += j1 - j0;
    if (j1 == nb) {
      ++b;
      while (b < p.batch && prefix[b + 1] == prefix[b]) ++b;
    }
  }
}

}  // namespace

bool generic_supported(const kv_pool* pool, int group) {
  return group >= 1 && group <= kMaxGroup && pool->head_dim % 4 == 0 &&
         pool->head_dim <= 64 * kGenDimsPerLane;
}

hipError_t launch_decode_generic(DecodeParams& p, hipStream_t s) {
  const int pre_words = ((p.batch + 1) + 3) & ~3;
  const size_t lds = sizeof(int32_t) * pre_words +
                     sizeof(float) * (size_t)p.group * (p.pool.head_dim + 64);
  const bool f32 = p.dtype == PAGEDKV_F32;
  const bool f16 = p.dtype == PAGEDKV_F16;
  const int dpl = p.pool.head_dim <= 64 ? 1 : p.pool.head_dim <= 128 ? 2 : 4;
  const void* fn = f32 ? reinterpret_cast<const void*>(&decode_generic_kernel<float, 4>)
                   : f16 ? reinterpret_cast<const void*>(&decode_generic_kernel<_Float16, 4>)
                         : reinterpret_cast<const void*>(&decode_generic_kernel<uint16_t, 4>);
  int wgs = 0;
  hipError_t e = resident_workgroups(fn, 64, lds, &wgs);
  if (e != hipSuccess) return e;
  int waves = wgs;
  if (waves > kMaxWaves) waves = kMaxWaves;
  p.units = waves / p.vheads;   // head groups
  if (p.units < 1) {
    p.units = 1;
    waves = p.vheads;
  }
  if (p.min_chunks < 1) p.min_chunks = 2;
  // no more units than the largest possible chunk count can keep busy
  const int64_t max_chunks = (int64_t)p.batch *
      (((int64_t)p.max_blocks_per_seq * p.pool.block_size + kGenericChunk - 1) / kGenericChunk);
  const int64_t useful = (max_chunks + p.min_chunks - 1) / p.min_chunks;
  if (useful < p.units) {
    p.units = (int)(useful < 1 ? 1 : useful);
    waves = p.units * p.vheads;
  }
  const dim3 grid(waves), block(64);
  if (f32) {
    if (dpl == 1) hipLaunchKernelGGL((decode_generic_kernel<float, 1>), grid, block, lds, s, p);
    else if (dpl == 2) hipLaunchKernelGGL((decode_generic_kernel<float, 2>), grid, block, lds, s, p);
    else hipLaunchKernelGGL((decode_generic_kernel<float, 4>), grid, block, lds, s, p);
  } else if (f16) {
    if (dpl == 1) hipLaunchKernelGGL((decode_generic_kernel<_Float16, 1>), grid, block, lds, s, p);
    else if (dpl == 2) hipLaunchKernelGGL((decode_generic_kernel<_Float16, 2>), grid, block, lds, s, p);
    else hipLaunchKernelGGL((decode_generic_kernel<_Float16, 4>), grid, block, lds, s, p);
  } else {
    if (dpl == 1) hipLaunchKernelGGL((decode_generic_kernel<uint16_t, 1>), grid, block, lds, s, p);
    else if (dpl == 2) hipLaunchKernelGGL((decode_generic_kernel<uint16_t, 2>), grid, block, lds, s, p);
    else hipLaunchKernelGGL((decode_generic_kernel<uint16_t, 4>), grid, block, lds, s, p);
  }
  return hipGetLastError();
}

}  // namespace pagedkv
