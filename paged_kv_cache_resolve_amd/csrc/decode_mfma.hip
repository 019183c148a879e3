// Paged-attention decode, pass 1, on MFMA tiles (gfx950): one persistent
// kernel body (decode_mfma_kernel<S>) over three stream types S.
//   Stream<E, D, 2, ...>  bf16 / fp16 pools (E = Bf16Ops, F16Ops), 32-token
//                         chunks of two 16x16 tiles (head_dim 256: 16-token
//                         chunks of one tile); its DENSE form reads
//                         the padded [batch][max_len][kv_heads][head_dim]
//                         tensors a batched gather writes, under a mask;
//   StreamF32<D, ...>     fp32 pools, 16-token chunks (described at the type).
//
// What is computed ("vllmini: Building a Minimalist PagedAttention and KV
// Cache Engine", section "The CUDA Block Kernel"; "KV Cache and Attention
// Mechanisms", section 2): for every (sequence, query head) the logical
// token positions are resolved through the sequence's block table into
// physical blocks of the pool, and scaled q.K scores, a max-subtracted
// softmax and the weighted sum of V rows are formed.
//
// Mapping onto CDNA4 (16-bit stream; the fp32 stream differs in the operand
// layouts only).
//  * Work split (internal.h, decode_split.h): the kv_heads wavefronts of a
//    head group take the same contiguous, equal-sized range of chunks of the
//    sequences laid end to end, one KV head each, and stream through it
//    without stopping at sequence boundaries.  All G query heads of a KV head
//    are computed from the same K/V bytes, so each byte is read from HBM
//    once, and the group reads each block's heads side by side.
//  * Per chunk:
//      - the K tiles [16 tokens x D] are loaded straight into the A-operand
//        layout of the 16x16x32 MFMA (row = token = lane % 16, eight
//        consecutive dims per lane) and multiplied by Q^T (16 head columns, G
//        used), giving score(token 4*(lane/16)+r, head lane%16);
//      - online softmax in fp32 in the exp2 domain (the accumulator is
//        rescaled branch-free; the factor is 1 unless a running max grew);
//      - the probabilities, rounded to the pool type, already sit in the
//        B-operand layout of the PV MFMA (k = token); V rows are loaded fully
//        coalesced (lane = token 4*(lane/16)+r, dims VD*(lane%16)..; at
//        head_dim 256 eight dims from each half of the row) and transposed
//        to the A operand with v_perm_b32.  The accumulator holds out^T:
//        lane = head lane%16, 4*VD contiguous dims (two runs of 32 at 256);
//      - the next chunk's K and V (and, at a sequence boundary, the next
//        sequence's q) are in flight while this chunk is computed; the
//        block-table entry of the chunk after that is already being fetched
//        by a scalar load.
//  * When a (sequence, KV head) ends inside the wavefront's range the
//    normalised output is written directly; one cut by a range edge leaves a
//    partial (running max, sum, unnormalised output) in the workspace, and
//    the merge kernel (decode_merge.hip) combines the partials.

#include <math.h>

#include "decode_split.h"
#include "internal.h"

namespace pagedkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;           // independent wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
#ifndef PAGEDKV_TILES_PER_STEP
#define PAGEDKV_TILES_PER_STEP 2
#endif
constexpr int kTilesPerStep = PAGEDKV_TILES_PER_STEP;   // 16-token MFMA tiles per chunk
#ifndef PAGEDKV_TILES_D256
#define PAGEDKV_TILES_D256 1
#endif
// head_dim 256: a 16-token tile already moves as many K/V bytes as a 32-token
// chunk at head_dim 128, and one tile keeps the K/V registers at that size
constexpr int kTilesD256 = PAGEDKV_TILES_D256;

template <int D> struct VRow;
template <> struct VRow<128> { using type = uint4; };   // 8 elements per lane
template <> struct VRow<96> { using type = uint3; };    // 6 elements per lane
template <> struct VRow<64> { using type = uint2; };    // 4 elements per lane
struct u32x8_t {   // 16 elements per lane (head_dim 256): two 16-byte halves
  uint4 lo, hi;
};
template <> struct VRow<256> { using type = u32x8_t; };

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// K and V are streamed once and never reused by this call, so their loads
// are non-temporal: they do not displace cache lines that are reused (block
// tables, q, the context lengths).  Measured: ~11% less time per call on the
// Llama-shaped and long-context workloads.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));
template <typename X8>
__device__ __forceinline__ X8 stream_load8(const char* p) {
  return __builtin_bit_cast(X8, __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p)));
}
__device__ __forceinline__ void stream_load(uint4& d, const char* p) {
  d = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p)));
}
// 12-byte rows (head_dim 96) are only 4-byte aligned
typedef unsigned int u32x3_nt __attribute__((ext_vector_type(3), aligned(4)));
__device__ __forceinline__ void stream_load(uint3& d, const char* p) {
  const u32x3_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x3_nt*>(p));
  d = make_uint3(v.x, v.y, v.z);
}
__device__ __forceinline__ void stream_load(uint2& d, const char* p) {
  d = __builtin_bit_cast(uint2, __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(p)));
}
// head_dim 256: a lane's 16 elements are 8 from each half of the row (the
// halves start 256 bytes apart), so that 16 lanes read each half as one
// contiguous 256-byte run
__device__ __forceinline__ void stream_load(u32x8_t& d, const char* p) {
  stream_load(d.lo, p);
  stream_load(d.hi, p + 256);
}

// Block tables are read-only while a decode runs; reading them through the
// constant address space lets uniform indices become scalar loads.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;


__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ uint32_t dword_of(const uint3& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : v.z;
}
__device__ __forceinline__ uint32_t dword_of(const uint2& v, int i) { return i == 0 ? v.x : v.y; }
__device__ __forceinline__ uint32_t dword_of(const u32x8_t& v, int i) {
  return i < 4 ? dword_of(v.lo, i) : dword_of(v.hi, i - 4);
}

// Element operations of the two 16-bit pool types: the MFMA forms, rounding
// of two floats to a packed pair (nearest even; lo = a, hi = b) and widening
// of either half of a pair.  Probabilities are multiplied by 2^kPScaleLog2
// before rounding: fp16 would lose small weights to its subnormal range, and
// the output and the normaliser carry the same factor, so it cancels (bf16
// has fp32's exponent range and needs none).
struct Bf16Ops {
  using x8 = bf16x8_t;
  using elem = __bf16;
  static constexpr float kPScaleLog2 = 0.f;
  static __device__ __forceinline__ f32x4_t mma32(x8 a, x8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mma16(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                     __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float lo(uint32_t x) { return __uint_as_float(x << 16); }
  static __device__ __forceinline__ float hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
};

struct F16Ops {
  using x8 = f16x8_t;
  using elem = _Float16;
  static constexpr float kPScaleLog2 = 15.f;   // p <= 2^15 < 65504
  static __device__ __forceinline__ f32x4_t mma32(x8 a, x8 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mma16(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    f16x2_t v;
    v[0] = (_Float16)a;
    v[1] = (_Float16)b;
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float lo(uint32_t x) { return (float)__builtin_bit_cast(f16x2_t, x)[0]; }
  static __device__ __forceinline__ float hi(uint32_t x) { return (float)__builtin_bit_cast(f16x2_t, x)[1]; }
};

// Combine a value with the lane 16 (resp. 32) apart, on the VALU.
__device__ __forceinline__ float max_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// K and V registers of one step: TILES tiles of 16 tokens.
template <typename E, int D, int TILES>
struct ChunkBuf {
  uint32_t mk[TILES];   // dense batches: the mask bytes of the lane's 4 score tokens per tile (loaded with V)
  typename E::x8 k[TILES][D / 32];
  typename VRow<D>::type v[TILES][4];
};

template <int D> __device__ __forceinline__ void zero_row(typename VRow<D>::type& v);
template <> __device__ __forceinline__ void zero_row<128>(uint4& v) { v = make_uint4(0, 0, 0, 0); }
template <> __device__ __forceinline__ void zero_row<96>(uint3& v) { v = make_uint3(0, 0, 0); }
template <> __device__ __forceinline__ void zero_row<64>(uint2& v) { v = make_uint2(0, 0); }
template <> __device__ __forceinline__ void zero_row<256>(u32x8_t& v) {
  v.lo = make_uint4(0, 0, 0, 0);
  v.hi = make_uint4(0, 0, 0, 0);
}

// Position in the chunk space of one KV head: chunk j of sequence b, which
// has nb chunks and T tokens; pos is b's appended token (fused append only,
// else -1).  All fields are wave-uniform.
struct Cursor {
  int b, j, nb, T, pos;
  int dense_T;   // length of every sequence of a dense batch (lens is null then)

  __device__ __forceinline__ void load_seq(const int32_t* prefix, const_i32_ptr lens,
                                           const_i32_ptr positions) {
    nb = uni(prefix[b + 1] - prefix[b]);
    T = lens ? uni(lens[b]) : dense_T;
    pos = positions ? uni(positions[b]) : -1;
  }

  // Step to the next chunk.  The caller guarantees one exists.
  __device__ __forceinline__ void advance(const int32_t* prefix, const_i32_ptr lens,
                                          const_i32_ptr positions, int batch) {
    if (++j < nb) return;
    j = 0;
    do { ++b; } while (b < batch - 1 && prefix[b + 1] == prefix[b]);
    b = uni(b);
    load_seq(prefix, lens, positions);
  }
};

// One wavefront's stream over its chunk range for KV head g.  A chunk is
// TILES x 16 tokens; tile t of chunk j holds tokens 16 * (TILES * j + t) ...
// With APPEND, the row of a sequence's appended token is read from k_new /
// v_new instead of the pool (a per-lane address choice; the pool row is
// written by the merge pass).
// With DENSE, K and V are the contiguous, padded [batch][max_len][kv_heads]
// [head_dim] tensors a batched gather produces, every sequence is max_len
// long, and a token takes part only where its mask byte is non-zero (the
// gather-then-attend path, for comparison with the paged one).
// With SMALL, blocks hold 4 or 8 tokens, so a 16-token tile spans several
// blocks: each lane looks up the block of its own K row and of its four V
// rows (which never straddle a block), one vector load each per tile.
//
// With NC = 2, a wavefront serves up to 32 query heads of its KV head as two
// groups of 16 MFMA columns: each K tile feeds one QK MFMA per group and each
// V operand one PV MFMA per group, so K/V are read once for all of them.
template <typename E, int D, int TILES, bool APPEND, bool DENSE = false, bool SMALL = false,
          int NC = 1>
struct Stream {
  static constexpr int kTiles = TILES;
  static constexpr int kCols = NC;            // groups of 16 query-head columns
  static constexpr int kChunk = 16 * TILES;   // tokens per chunk
  static constexpr bool kAppend = APPEND;
  static constexpr bool kDense = DENSE;
  static constexpr int kPh = SMALL ? 2 * TILES : TILES;   // block entries held per chunk
  using x8 = typename E::x8;
  using OutElem = typename E::elem;   // element type of q, out and the pool
  // fits the per-pair kernel's 256 registers per lane without spilling
  static constexpr bool kPairs = !DENSE && D <= 128 && NC == 1;
  static constexpr int kDim = D;
  using Buf = ChunkBuf<E, D, TILES>;
  static constexpr int NK = D / 32;   // 16-byte K loads per lane per tile
  static constexpr int VD = D / 16;   // V dims per lane
  static constexpr int NW = VD / 2;   // dwords per lane per V row
  // Where a lane's VD elements of a V row sit.  Lane n holds elements
  // kVLane*n + i (i < VD), except at head_dim 256, where it holds 8n + i and
  // 128 + 8n + (i - 8) (the two halves of the row, each read contiguously
  // by the 16 lanes).  In the output, accumulator i of the lane with quad q
  // and row r is dim kQuadDims*q + kRowDims*r + i (+ 120 for i >= 8 at 256).
  static constexpr bool kSplitRow = D == 256;
  static constexpr int kVLane = kSplitRow ? 8 : VD;
  static constexpr int kQuadDims = 4 * kVLane;
  static constexpr int kRowDims = kVLane;
  static constexpr int kHalfDims = kSplitRow ? 128 : 8;   // offset of element group i / 8

  const DecodeParams& p;
  const int lane, n, quad;
  const int g;              // (virtual) KV head served by this wavefront
  const int gp;             // the pool's KV head it reads
  int qh0, gw;              // its query heads: qh0 .. qh0 + gw - 1
  const int64_t unit;       // head group (chunk range) of this wavefront

  x8 qop[NC][NK];
  f32x4_t acc[NC][VD];
  float m[NC], l[NC];
  // LDS-staged stream only: the normaliser of column n summed over every
  // token by one MFMA per chunk (A operand all ones), in each of the four
  // rows a lane holds, so it needs no cross-lane sum at the end.
  f32x4_t lacc[NC];

  __device__ Stream(const DecodeParams& p_, int lane_, int g_, int64_t unit_)
      : p(p_), lane(lane_), n(lane_ & 15), quad(lane_ >> 4), g(g_),
        gp(vhead_pool_head(g_, p_.qsplit)), unit(unit_) {
    const VHead v = vhead_rows(g_, p_.qsplit, p_.kv_group);
    qh0 = v.first;
    gw = v.count;
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
#pragma unroll
      for (int c = 0; c < VD; ++c) acc[cg][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      lacc[cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m[cg] = -INFINITY;
      l[cg] = 0.f;
    }
  }

  // q of the sequence's gw query heads of this (virtual) KV head in the
  // B-operand layout: column n of group cg is head 16*cg + n.  Columns at or
  // past gw carry a copy of the last head: every column goes through its own
  // softmax and accumulator and only columns below gw are ever written, so
  // the copies cost nothing and need neither a branch nor masking.
  __device__ __forceinline__ void load_q(const Cursor& c) {
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
      const uint16_t* qrow =
          static_cast<const uint16_t*>(p.q) +
          ((int64_t)c.b * p.num_q_heads + qh0 + min(16 * cg + n, gw - 1)) * D + 8 * quad;
#pragma unroll
      for (int i = 0; i < NK; ++i) qop[cg][i] = *reinterpret_cast<const x8*>(qrow + 32 * i);
    }
  }

  // Physical blocks of chunk c's tiles: scalar loads of block-table
  // entries.  A tile that starts at or past T (the sequence's last chunk can
  // be partly empty) reuses tile 0's block: its loads stay inside the pool
  // and all of its tokens are masked.
  __device__ __forceinline__ void fetch_phys(const Cursor& c, int* ph) const {
    if constexpr (DENSE) {
#pragma unroll
      for (int t = 0; t < TILES; ++t) ph[t] = 0;
      return;
    }
    if constexpr (SMALL) {
      // tokens at or past T look up the block of token T-1: their loads stay
      // inside the pool and they are masked
      const int32_t* trow = p.block_tables + (int64_t)c.b * p.max_blocks_per_seq;
      const int sh = __builtin_ctz(p.pool.block_size);
      const int tok0 = c.j * (16 * TILES);
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        ph[2 * t] = trow[min(tok0 + 16 * t + n, c.T - 1) >> sh];
        ph[2 * t + 1] = trow[min(tok0 + 16 * t + 4 * quad, c.T - 1) >> sh];
      }
      return;
    }
    const const_i32_ptr trow = (const_i32_ptr)(p.block_tables + (int64_t)c.b * p.max_blocks_per_seq);
    const int tok0 = c.j * (16 * TILES);
    ph[0] = uni(trow[fdiv(tok0, p.bs_div)]);
#pragma unroll
    for (int t = 1; t < TILES; ++t) {
      const int tok = tok0 + 16 * t;
      ph[t] = tok < c.T ? uni(trow[fdiv(tok, p.bs_div)]) : ph[0];
    }
  }

  // Byte address of the K rows of tile t of chunk c.
  __device__ __forceinline__ const char* tile_base(const Cursor& c, const int* ph, int t) const {
    return tile_addr(ph[t], c.j * (16 * TILES) + 16 * t);
  }
  // Byte address of the K row of token tok, which lies in block phys.
  __device__ __forceinline__ const char* tile_addr(int phys, int tok) const {
    const int off = tok - (int)fdiv(tok, p.bs_div) * p.pool.block_size;   // tok % block_size
    return p.pool.base + 2 * ((int64_t)p.layer * p.pool.layer_stride +
                              (int64_t)gp * p.pool.head_stride +
                              (int64_t)phys * p.pool.block_stride + (int64_t)off * D);
  }

  // SMALL blocks: byte address of token tok's K (kv = 0) or V (kv = 1) row
  // in block phys.
  __device__ __forceinline__ const char* row_addr(int phys, int tok, int kv) const {
    return p.pool.base + 2 * ((int64_t)p.layer * p.pool.layer_stride +
                              (int64_t)gp * p.pool.head_stride +
                              (int64_t)phys * p.pool.block_stride + (int64_t)kv * p.pool.kv_stride +
                              (int64_t)(tok & (p.pool.block_size - 1)) * D);
  }

  // Row of the new token of (c.b, g) in k_new (kv = 0) or v_new (kv = 1).
  __device__ __forceinline__ const char* new_row(const Cursor& c, int kv) const {
    return static_cast<const char*>(kv ? p.v_new : p.k_new) +
           2 * ((int64_t)c.b * p.pool.kv_heads + gp) * D;
  }

  // Dense batches: byte address of token tok's row of head g (tokens past
  // the end re-read the last row; they are masked).
  __device__ __forceinline__ const char* dense_row(const void* base, const Cursor& c,
                                                   int tok) const {
    const int tc = min(tok, c.T - 1);
    return static_cast<const char*>(base) +
           2 * ((((int64_t)c.b * p.dense_len + tc) * p.pool.kv_heads + gp) * D);
  }

  __device__ __forceinline__ void issue_k(Buf& cb, const Cursor& c,
                                          const int* ph) const {
    if constexpr (DENSE) {
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const int tok0 = c.j * (16 * TILES) + 16 * t;
        const char* kl = dense_row(p.k_dense, c, tok0 + n) + 2 * 8 * quad;
#pragma unroll
        for (int i = 0; i < NK; ++i) cb.k[t][i] = stream_load8<x8>(kl + 64 * i);
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const char* kl;
      if constexpr (SMALL)
        kl = row_addr(ph[2 * t], c.j * (16 * TILES) + 16 * t + n, 0) + 2 * 8 * quad;
      else
        kl = tile_base(c, ph, t) + (uint32_t)(2 * (n * D + 8 * quad));
      if constexpr (APPEND) {
        const int tok = c.j * (16 * TILES) + 16 * t + n;
        if (tok == c.pos) kl = new_row(c, 0) + 2 * 8 * quad;
      }
#pragma unroll
      for (int i = 0; i < NK; ++i) cb.k[t][i] = stream_load8<x8>(kl + 64 * i);
    }
  }
  __device__ __forceinline__ void issue_v(Buf& cb, const Cursor& c,
                                          const int* ph) const {
    if constexpr (DENSE) {
      // The mask bytes of the lane's score tokens travel with V: the next
      // chunk's V (and mask) is issued only after this chunk's softmax,
      // while its K is issued before it.
      const uint8_t* mrow = p.mask + (int64_t)c.b * p.dense_len;
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        uint32_t bits = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = c.j * (16 * TILES) + 16 * t + 4 * quad + r;
          stream_load(cb.v[t][r], dense_row(p.v_dense, c, tok) + 2 * kVLane * n);
          bits |= (uint32_t)mrow[min(tok, c.T - 1)] << (8 * r);
        }
        cb.mk[t] = bits;
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const char* vl = SMALL ? nullptr
                             : tile_base(c, ph, t) + 2 * p.pool.kv_stride +
                                   (uint32_t)(2 * (4 * quad * D + kVLane * n));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const char* row;
        if constexpr (SMALL)
          row = row_addr(ph[2 * t + 1], c.j * (16 * TILES) + 16 * t + 4 * quad + r, 1) +
                2 * kVLane * n;
        else
          row = vl + 2 * r * D;
        if constexpr (APPEND) {
          const int tok = c.j * (16 * TILES) + 16 * t + 4 * quad + r;
          if (tok == c.pos) row = new_row(c, 1) + 2 * kVLane * n;
        }
        stream_load(cb.v[t][r], row);
      }
    }
  }

  // LDS-staged streaming (the per-pair kernel at head_dim 64, see
  // stream_pair_lds): a chunk's K and V rows are copied into an LDS slot by
  // LDS-direct loads (global_load_lds_dwordx4, 16 bytes per lane), which
  // need no registers while in flight, and read into the Buf registers when
  // the chunk is computed.
  static constexpr bool kLdsStream = !DENSE && !SMALL && D == 64 && NC == 1 && TILES == 2;
  static constexpr uint32_t kSlotBytes = 2 * TILES * 16 * D * 2;   // K then V of one chunk
  // With VS (one of two workgroups of a pair, each with half of V's dims):
  // K and that half of V
  template <bool VS>
  static constexpr uint32_t slot_bytes() { return VS ? kSlotBytes / 4 * 3 : kSlotBytes; }
  // LDS-direct loads per chunk
  template <bool VS>
  static constexpr int chunk_loads() { return VS ? 6 : 8; }

  // Copy chunk c into the slot at LDS byte address `slot`.  Tile t's K rows
  // go to slot + t * 2 KiB, its V rows to slot + (TILES + t) * 2 KiB: 16
  // rows of 128 bytes, row r's 16-byte column q stored at column q ^ (r & 7)
  // (so that the reads below hit distinct banks).  Unit u = 64 h + lane of
  // instruction h is LDS column u & 7 of row u >> 3.  With VS only half
  // `dhalf` of each V row is copied (dims 32 dhalf .. 32 dhalf + 31, 64
  // bytes, four 16-byte columns), tile t to slot + TILES * 2 KiB + t * 1 KiB
  // in one load: unit u = lane holds column u & 3 of row 4 ((u >> 2) & 3) +
  // (u >> 4), so that the rows a read instruction takes (4 quad + r for the
  // four quads) sit in different banks.  The appended token's row comes
  // from k_new / v_new, as in issue_k / issue_v; whether the chunk holds it
  // is wave-uniform, so other chunks take the form without the per-lane
  // choice.
  template <bool OVR, bool VS>
  __device__ __forceinline__ void dma_tiles(const Cursor& c, const char* const* tb, uint32_t slot,
                                            int dhalf) const {
    typedef __attribute__((address_space(3))) void* lds_ptr;
#pragma unroll
    for (int kv = 0; kv < (VS ? 1 : 2); ++kv)
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int u = 64 * h + lane;
          const int r = u >> 3;
          const int col = (u & 7) ^ (r & 7);
          const char* src =
              tb[t] + (kv ? 2 * p.pool.kv_stride : 0) + (uint32_t)(2 * r * D + 16 * col);
          if constexpr (OVR) {
            if (c.j * kChunk + 16 * t + r == c.pos) src = new_row(c, kv) + 16 * col;
          }
          __builtin_amdgcn_global_load_lds(
              src, (lds_ptr)(uintptr_t)(slot + (uint32_t)((kv * TILES + t) * 2048 + h * 1024)), 16, 0, 0);
        }
    if constexpr (VS) {
      const int r = 4 * ((lane >> 2) & 3) + (lane >> 4);
      const int q = lane & 3;
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const char* src = tb[t] + 2 * p.pool.kv_stride +
                          (uint32_t)(2 * r * D + 64 * dhalf + 16 * q);
        if constexpr (OVR) {
          if (c.j * kChunk + 16 * t + r == c.pos) src = new_row(c, 1) + 64 * dhalf + 16 * q;
        }
        __builtin_amdgcn_global_load_lds(
            src, (lds_ptr)(uintptr_t)(slot + (uint32_t)(TILES * 2048 + t * 1024)), 16, 0, 0);
      }
    }
  }
  template <bool VS = false>
  __device__ __forceinline__ void dma_chunk(const Cursor& c, const char* const* tb, uint32_t slot,
                                            int dhalf = 0) const {
    if (APPEND && (unsigned)(c.pos - c.j * kChunk) < (unsigned)kChunk)
      dma_tiles<APPEND, VS>(c, tb, slot, dhalf);
    else
      dma_tiles<false, VS>(c, tb, slot, dhalf);
  }

  // A lane's LDS read addresses in slot 0 of its wavefront; the other slot
  // and the tiles are immediate offsets.  Lane (n, quad) takes K row n,
  // columns quad and quad + 4 of each tile, and V rows 4 quad + r, bytes
  // 8n .. 8n+7: the layouts issue_k and issue_v load.  With VS, lane
  // (n, quad) takes dims 32 dhalf + 2n and + 1 of V rows 4 quad + r (4 bytes
  // of the staged half row), for the two-column PV product of attend.
  struct LdsLane {
    uint32_t k[2], v[4];
  };
  template <bool VS = false>
  __device__ __forceinline__ LdsLane lds_lane(uint32_t slot0, int dhalf = 0) const {
    LdsLane a;
#pragma unroll
    for (int i = 0; i < 2; ++i) a.k[i] = slot0 + (uint32_t)((n * 8 + ((quad + 4 * i) ^ (n & 7))) * 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * quad + r;
      if constexpr (VS) {
        a.v[r] = slot0 + (uint32_t)(TILES * 2048 + (16 * r + 4 * quad + (n >> 2)) * 16 + (n & 3) * 4);
      } else {
        a.v[r] = slot0 + (uint32_t)(TILES * 2048 + (row * 8 + ((n >> 1) ^ (row & 7))) * 16 + (n & 1) * 8);
      }
    }
    return a;
  }

  // Read the chunk in slot SLOT into the Buf registers.  The reads are
  // written as asm with their wait inside, because the compiler would
  // otherwise wait for every LDS-direct load in flight (it cannot tell the
  // slots apart) before each LDS read.  K and V go out together under one
  // wait: a wait between them cost the churned-pool call 0.2 us.
  template <int SLOT, bool VS = false>
  __device__ __forceinline__ void read_chunk(Buf& cb, const LdsLane& a) const {
    static_assert(TILES == 2, "two tiles per chunk");
    constexpr int O = SLOT * (int)slot_bytes<VS>();
    constexpr int OV1 = O + (VS ? 1024 : 2048);   // V tile 1
    typedef unsigned u32x4_v __attribute__((ext_vector_type(4)));
    typedef unsigned u32x2_v __attribute__((ext_vector_type(2)));
    u32x4_v k[TILES][2];
    if constexpr (VS) {
      uint32_t v[TILES][4];
      asm volatile(
          "ds_read_b128 %0, %12 offset:%18\n\t"
          "ds_read_b128 %1, %13 offset:%18\n\t"
          "ds_read_b128 %2, %12 offset:%19\n\t"
          "ds_read_b128 %3, %13 offset:%19\n\t"
          "ds_read_b32 %4, %14 offset:%18\n\t"
          "ds_read_b32 %5, %15 offset:%18\n\t"
          "ds_read_b32 %6, %16 offset:%18\n\t"
          "ds_read_b32 %7, %17 offset:%18\n\t"
          "ds_read_b32 %8, %14 offset:%20\n\t"
          "ds_read_b32 %9, %15 offset:%20\n\t"
          "ds_read_b32 %10, %16 offset:%20\n\t"
          "ds_read_b32 %11, %17 offset:%20\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k[0][0]), "=&v"(k[0][1]), "=&v"(k[1][0]), "=&v"(k[1][1]),
            "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]),
            "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3])
          : "v"(a.k[0]), "v"(a.k[1]), "v"(a.v[0]), "v"(a.v[1]), "v"(a.v[2]), "v"(a.v[3]),
            "i"(O), "i"(O + 2048), "i"(OV1)
          : "memory");
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) cb.v[t][r] = make_uint2(v[t][r], 0u);
    } else {
      u32x2_v v[TILES][4];
      asm volatile(
          "ds_read_b128 %0, %12 offset:%18\n\t"
          "ds_read_b128 %1, %13 offset:%18\n\t"
          "ds_read_b128 %2, %12 offset:%19\n\t"
          "ds_read_b128 %3, %13 offset:%19\n\t"
          "ds_read_b64 %4, %14 offset:%18\n\t"
          "ds_read_b64 %5, %15 offset:%18\n\t"
          "ds_read_b64 %6, %16 offset:%18\n\t"
          "ds_read_b64 %7, %17 offset:%18\n\t"
          "ds_read_b64 %8, %14 offset:%20\n\t"
          "ds_read_b64 %9, %15 offset:%20\n\t"
          "ds_read_b64 %10, %16 offset:%20\n\t"
          "ds_read_b64 %11, %17 offset:%20\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k[0][0]), "=&v"(k[0][1]), "=&v"(k[1][0]), "=&v"(k[1][1]),
            "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]),
            "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3])
          : "v"(a.k[0]), "v"(a.k[1]), "v"(a.v[0]), "v"(a.v[1]), "v"(a.v[2]), "v"(a.v[3]),
            "i"(O), "i"(O + 2048), "i"(OV1)
          : "memory");
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) cb.v[t][r] = make_uint2(v[t][r].x, v[t][r].y);
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int i = 0; i < 2; ++i) cb.k[t][i] = __builtin_bit_cast(x8, k[t][i]);
  }

  // s[cg * TILES + t]: scores of tile t against column group cg.
  __device__ __forceinline__ void qk(const Buf& cb, f32x4_t* s) const {
#pragma unroll
    for (int cg = 0; cg < NC; ++cg)
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        f32x4_t& st = s[cg * TILES + t];
        st = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NK; ++i) st = E::mma32(cb.k[t][i], qop[cg][i], st);
      }
  }

  // Online softmax of column group cg over one chunk: rescales its m, l and
  // acc and returns the probabilities rounded to the pool type, packed in
  // pairs (the B-operand layout of the PV product).
  // LAZY (the LDS-staged stream): the normaliser is summed by the MFMA unit
  // (lacc, in attend), and m, acc and lacc are rescaled only when some
  // column's chunk maximum exceeds its running max by more than kLazyLog2.
  // Until then the older max stays the common reference of acc, lacc and the
  // probabilities, which stay below 2^kLazyLog2 (times 2^kPScaleLog2), so
  // the result is the same up to rounding; fp16 takes 0 (its probabilities
  // already use the range up to 2^15), which still skips every chunk that
  // raises no column's max.
  static constexpr float kLazyLog2 = E::kPScaleLog2 == 0.f ? 8.f : 0.f;
  // VS (half of V's dims, two dims per lane): acc[cg][0..1] only
  template <bool TAIL, bool LAZY = false, bool VS = false>
  __device__ __forceinline__ void softmax_cols(const f32x4_t* s, const Buf& cb, const Cursor& c,
                                               int cg, uint32_t (&pw)[TILES][2]) {
    float sv[TILES][4];
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[t][r] = s[t][r] * p.scale_log2;
        if (TAIL && c.j * (16 * TILES) + 16 * t + 4 * quad + r >= c.T) sv[t][r] = -INFINITY;
        if (DENSE && ((cb.mk[t] >> (8 * r)) & 0xffu) == 0) sv[t][r] = -INFINITY;
      }
    float bmax = fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3]));
#pragma unroll
    for (int t = 1; t < TILES; ++t)
      bmax = fmaxf(bmax, fmaxf(fmaxf(sv[t][0], sv[t][1]), fmaxf(sv[t][2], sv[t][3])));
    bmax = max_x32(max_x16(bmax));
    // A dense batch can present chunks with every token masked: while the
    // running max is still -inf, exponents are taken against 0 instead
    // (acc and l are zero then, and the weights of masked tokens are 0).
    float mref;
    if constexpr (LAZY) {
      static_assert(!DENSE, "every chunk of a paged sequence holds a token");
      if (__builtin_amdgcn_ballot_w64(bmax > m[cg] + kLazyLog2) != 0) {
        const float mn = fmaxf(m[cg], bmax);
        const float alpha = __builtin_amdgcn_exp2f(m[cg] - mn);
#pragma unroll
        for (int i = 0; i < (VS ? 2 : VD); ++i) acc[cg][i] *= alpha;
        lacc[cg] *= alpha;
        m[cg] = mn;
      }
      mref = m[cg];
    } else {
      // branch-free rescale (alpha = 1 when no running max grows)
      const float mn = fmaxf(m[cg], bmax);
      mref = DENSE && mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m[cg] - mref);
#pragma unroll
      for (int i = 0; i < VD; ++i) acc[cg][i] *= alpha;
      l[cg] *= alpha;
      m[cg] = mn;
    }
    const float mp = mref - E::kPScaleLog2;
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      pw[t][0] = E::pack2(__builtin_amdgcn_exp2f(sv[t][0] - mp), __builtin_amdgcn_exp2f(sv[t][1] - mp));
      pw[t][1] = E::pack2(__builtin_amdgcn_exp2f(sv[t][2] - mp), __builtin_amdgcn_exp2f(sv[t][3] - mp));
      if constexpr (!LAZY)
        l[cg] += (E::lo(pw[t][0]) + E::hi(pw[t][0])) + (E::lo(pw[t][1]) + E::hi(pw[t][1]));
    }
  }

  // Scores -> probabilities in the pool type (already in the B-operand layout of the PV
  // product), then the weighted V sum; updates m, l, acc.  TAIL masks tokens
  // at or past T; masked V rows are zeroed, not weighted by zero, so unused
  // pool slots never reach the sum.
  // VS (LDS-staged stream, half `dhalf` of V's dims per workgroup): the
  // lane's V words hold dims 2n and 2n + 1 of its half for its eight tokens,
  // so one 16x16x32 product per dim parity e takes row n as dim
  // 32 dhalf + 2n + e, and acc[cg][e][r] is dim 32 dhalf + 8 quad + 2r + e.
  template <bool TAIL, bool LAZY = false, bool VS = false>
  __device__ __forceinline__ void attend(const f32x4_t* s, Buf& cb, const Cursor& c) {
    static_assert(!LAZY || TILES == 2, "the lazy form sums the normaliser with the 16x16x32 MFMA");
    static_assert(!VS || (LAZY && NC == 1), "VS: LDS-staged stream only");
    uint32_t pw[NC][TILES][2];
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) softmax_cols<TAIL, LAZY, VS>(s + cg * TILES, cb, c, cg, pw[cg]);
    if (TAIL && !DENSE) {   // dense rows past the end repeat a real row; their weight is 0
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (c.j * (16 * TILES) + 16 * t + 4 * quad + r >= c.T) zero_row<D>(cb.v[t][r]);
    }
    if constexpr (TILES == 1) {
      // k = 4 tokens per lane: the 16x16x16 MFMA
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const uint32_t v0 = dword_of(cb.v[0][0], w), v1 = dword_of(cb.v[0][1], w);
        const uint32_t v2 = dword_of(cb.v[0][2], w), v3 = dword_of(cb.v[0][3], w);
        const uint2 ev = make_uint2(__builtin_amdgcn_perm(v1, v0, 0x05040100u),
                                    __builtin_amdgcn_perm(v3, v2, 0x05040100u));
        const uint2 od = make_uint2(__builtin_amdgcn_perm(v1, v0, 0x07060302u),
                                    __builtin_amdgcn_perm(v3, v2, 0x07060302u));
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) {
          const uint2 pop = make_uint2(pw[cg][0][0], pw[cg][0][1]);
          acc[cg][2 * w] = E::mma16(ev, pop, acc[cg][2 * w]);
          acc[cg][2 * w + 1] = E::mma16(od, pop, acc[cg][2 * w + 1]);
        }
      }
    } else {
      // k = 8 tokens per lane (4 of each tile, in the order the lane holds
      // its scores): the 16x16x32 MFMA
      x8 pop[NC];
#pragma unroll
      for (int cg = 0; cg < NC; ++cg)
        pop[cg] = __builtin_bit_cast(
            x8, make_uint4(pw[cg][0][0], pw[cg][0][1], pw[cg][1][0], pw[cg][1][1]));
      if constexpr (LAZY) {   // column sums of the rounded probabilities
        const uint32_t one2 = E::pack2(1.f, 1.f);
        const x8 ones = __builtin_bit_cast(x8, make_uint4(one2, one2, one2, one2));
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) lacc[cg] = E::mma32(ones, pop[cg], lacc[cg]);
      }
      if constexpr (VS) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t sel = e ? 0x07060302u : 0x05040100u;
          uint32_t a[4];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            a[2 * t] = __builtin_amdgcn_perm(cb.v[t][1].x, cb.v[t][0].x, sel);
            a[2 * t + 1] = __builtin_amdgcn_perm(cb.v[t][3].x, cb.v[t][2].x, sel);
          }
          acc[0][e] = E::mma32(__builtin_bit_cast(x8, make_uint4(a[0], a[1], a[2], a[3])), pop[0],
                               acc[0][e]);
        }
        return;
      }
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        uint32_t ev[4], od[4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t v0 = dword_of(cb.v[t][0], w), v1 = dword_of(cb.v[t][1], w);
          const uint32_t v2 = dword_of(cb.v[t][2], w), v3 = dword_of(cb.v[t][3], w);
          ev[2 * t] = __builtin_amdgcn_perm(v1, v0, 0x05040100u);
          ev[2 * t + 1] = __builtin_amdgcn_perm(v3, v2, 0x05040100u);
          od[2 * t] = __builtin_amdgcn_perm(v1, v0, 0x07060302u);
          od[2 * t + 1] = __builtin_amdgcn_perm(v3, v2, 0x07060302u);
        }
        const x8 eva = __builtin_bit_cast(x8, make_uint4(ev[0], ev[1], ev[2], ev[3]));
        const x8 oda = __builtin_bit_cast(x8, make_uint4(od[0], od[1], od[2], od[3]));
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) {
          acc[cg][2 * w] = E::mma32(eva, pop[cg], acc[cg][2 * w]);
          acc[cg][2 * w + 1] = E::mma32(oda, pop[cg], acc[cg][2 * w + 1]);
        }
      }
    }
  }

  template <bool LAZY = false, bool VS = false>
  __device__ __forceinline__ void attend_chunk(const f32x4_t* s, Buf& cb,
                                               const Cursor& c) {
    if (DENSE || (c.j == c.nb - 1 && (c.T % (16 * TILES)) != 0))
      attend<true, LAZY, VS>(s, cb, c);
    else
      attend<false, LAZY, VS>(s, cb, c);
  }

  // End of this wavefront's part of sequence c.b: normalised output if it
  // saw the whole sequence, else a partial in its (sequence, head, unit) slot.
  __device__ void flush(const Cursor& c, bool whole) {
    float lt[NC];
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) lt[cg] = sum_x32(sum_x16(l[cg]));
#pragma unroll
    for (int cg = 0; cg < NC; ++cg)
      if (16 * cg + n < gw) flush_cols(c, whole, cg, lt[cg]);
  }

  // Per-pair kernel with LDS staging: the partial (unnormalised output of
  // the gw heads, then their (max, sum)) into LDS at byte address `base`,
  // laid out [head][D] floats then [head][2], for the workgroup's merge.
  __device__ __forceinline__ void flush_lds(uint32_t base) {
    static_assert(NC == 1 && VD % 4 == 0, "LDS partials: one column group");
    typedef __attribute__((address_space(3))) float lds_float;
    const float lt = lacc[0][0];
    if (n >= gw) return;
    lds_float* of = (lds_float*)(uintptr_t)base + n * D + kQuadDims * quad;
    const f32x4_t* a = acc[0];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int h = 0; h < VD / 4; ++h) {
        lds_float* d = of + kRowDims * r + kHalfDims * (h / 2) + 4 * (h % 2);
        d[0] = a[4 * h][r];
        d[1] = a[4 * h + 1][r];
        d[2] = a[4 * h + 2][r];
        d[3] = a[4 * h + 3][r];
      }
    if (quad == 0) {
      lds_float* ml = (lds_float*)(uintptr_t)base + gw * D + 2 * n;
      ml[0] = m[0];
      ml[1] = lt;
    }
  }

  // VS: the partial of this workgroup's half of V's dims, in flush_lds's
  // layout (the other half's dims are left as they are: the fold does not
  // read them).  Lane (n, quad) holds dims 32 dhalf + 8 quad .. + 7.
  __device__ __forceinline__ void flush_lds_vs(uint32_t base, int dhalf) {
    typedef __attribute__((address_space(3))) float lds_float;
    const float lt = lacc[0][0];
    if (n >= gw) return;
    lds_float* of = (lds_float*)(uintptr_t)base + n * D + 32 * dhalf + 8 * quad;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      of[2 * r] = acc[0][0][r];
      of[2 * r + 1] = acc[0][1][r];
    }
    if (quad == 0) {
      lds_float* ml = (lds_float*)(uintptr_t)base + gw * D + 2 * n;
      ml[0] = m[0];
      ml[1] = lt;
    }
  }

  // VS, a sequence this wavefront saw whole: its half of head n's output
  // row, 8 dims per lane in one 16-byte store.
  __device__ __forceinline__ void flush_whole_vs(const Cursor& c, float lt, int dhalf) {
    if (n >= gw) return;
    const float inv = 1.0f / lt;
    uint16_t* dst = static_cast<uint16_t*>(p.out) +
                    ((int64_t)c.b * p.num_q_heads + qh0 + n) * D + 32 * dhalf + 8 * quad;
    const f32x4_t* a = acc[0];
    *reinterpret_cast<uint4*>(dst) =
        make_uint4(E::pack2(a[0][0] * inv, a[1][0] * inv), E::pack2(a[0][1] * inv, a[1][1] * inv),
                   E::pack2(a[0][2] * inv, a[1][2] * inv), E::pack2(a[0][3] * inv, a[1][3] * inv));
  }

  // Column group cg's share of flush: head 16*cg + n of this (virtual) KV head.
  __device__ __forceinline__ void flush_cols(const Cursor& c, bool whole, int cg, float lt) {
    const int G = p.group;   // partial slot stride
    const int hc = 16 * cg + n;
    const f32x4_t* a = acc[cg];
    // lane holds dims kQuadDims*quad + kRowDims*r + (i % 8) + kHalfDims*(i / 8)
    // of head hc as a[i][r]
    if (whole) {
      const float inv = DENSE && lt == 0.f ? 0.f : 1.0f / lt;   // dense: all masked -> zeros
      uint16_t* dst = static_cast<uint16_t*>(p.out) +
                      ((int64_t)c.b * p.num_q_heads + qh0 + hc) * D + kQuadDims * quad;
      if constexpr (VD % 8 == 0) {   // VD / 8 16-byte stores per r
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int h = 0; h < VD / 8; ++h)
            *reinterpret_cast<uint4*>(dst + kRowDims * r + kHalfDims * h) =
                make_uint4(E::pack2(a[8 * h][r] * inv, a[8 * h + 1][r] * inv),
                           E::pack2(a[8 * h + 2][r] * inv, a[8 * h + 3][r] * inv),
                           E::pack2(a[8 * h + 4][r] * inv, a[8 * h + 5][r] * inv),
                           E::pack2(a[8 * h + 6][r] * inv, a[8 * h + 7][r] * inv));
      } else if constexpr (VD == 6) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {   // 12 bytes per r: three dword stores
          uint32_t* d1 = reinterpret_cast<uint32_t*>(dst + VD * r);
          d1[0] = E::pack2(a[0][r] * inv, a[1][r] * inv);
          d1[1] = E::pack2(a[2][r] * inv, a[3][r] * inv);
          d1[2] = E::pack2(a[4][r] * inv, a[5][r] * inv);
        }
      } else {
        uint2* d2 = reinterpret_cast<uint2*>(dst);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          d2[r] = make_uint2(E::pack2(a[0][r] * inv, a[1][r] * inv),
                             E::pack2(a[2][r] * inv, a[3][r] * inv));
      }
    } else {
      const int64_t slot = partial_slot(c.b, g, unit, p.vheads);
      float* of = p.ws_o + (slot * G + hc) * D + kQuadDims * quad;
      if constexpr (VD % 4 == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int h = 0; h < VD / 4; ++h)
            *reinterpret_cast<float4*>(of + kRowDims * r + kHalfDims * (h / 2) + 4 * (h % 2)) =
                make_float4(a[4 * h][r], a[4 * h + 1][r], a[4 * h + 2][r], a[4 * h + 3][r]);
      } else {
        float2* o = reinterpret_cast<float2*>(of);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int h = 0; h < VD / 2; ++h)
            o[r * (VD / 2) + h] = make_float2(a[2 * h][r], a[2 * h + 1][r]);
      }
      if (quad == 0) {
        p.ws_ml[(slot * G + hc) * 2 + 0] = m[cg];
        p.ws_ml[(slot * G + hc) * 2 + 1] = lt;
      }
    }
  }
};

// fp32 pools: v_mfma_f32_16x16x4_f32 (full fp32 products), one 16-token
// tile per chunk, so that a chunk moves as many bytes as a bf16 one.
//  * QK: the sum over head_dim is taken in the order (i, c): at step (i, c)
//    lane (token n, quad) feeds K[n][16*i + 4*quad + c] and lane (head n,
//    quad) feeds q[n][16*i + 4*quad + c].  Load i of a lane is then the
//    float4 at dim 16*i + 4*quad of its row, and the four quads of a row
//    read 64 contiguous bytes per instruction.  Four accumulators (one per
//    c) keep the dependent MFMA chains short.
//  * PV: step r (0..3) takes tokens 4*quad + r.  Its B operand is the lane's
//    own probability of token 4*quad + r (the score layout, so no data moves
//    between lanes) and its A operand holds V dims 4*n + e + 64*h of those
//    tokens for output block (h, e): each lane reads float4s at dims
//    4*n + 64*h of its four rows.  Block (h, e) accumulates out^T rows i ->
//    dim 64*h + 4*i + e, so lane (head n, quad) ends with dims
//    64*h + 16*quad + 4*r + e: 16 contiguous dims per h.
//  * Probabilities stay in fp32.
template <int D, bool APPEND>
struct StreamF32 {
  static constexpr int kTiles = 1;
  static constexpr int kCols = 1;
  static constexpr int kChunk = 16;
  static constexpr bool kAppend = APPEND;
  static constexpr bool kDense = false;
  static constexpr int kPh = 1;
  static constexpr int KQ = D / 4;    // K floats per lane per tile
  static constexpr int NH = D / 64;   // float4 V loads per row per lane
  static constexpr int NB = D / 16;   // output blocks (h, e)
  using OutElem = float;
  static constexpr bool kPairs = true;
  static constexpr bool kLdsStream = false;
  static constexpr uint32_t kSlotBytes = 0;
  __device__ __forceinline__ void flush_lds(uint32_t) {}
  static constexpr int kDim = D;
  struct Buf {
    float4 k[KQ / 4];
    float4 v[4][NH];
  };

  const DecodeParams& p;
  const int lane, n, quad;
  const int g;              // (virtual) KV head served by this wavefront
  const int gp;             // the pool's KV head it reads
  int qh0, gw;              // its query heads: qh0 .. qh0 + gw - 1
  const int64_t unit;

  float qop[KQ];
  f32x4_t acc[NB];
  float m, l;

  __device__ StreamF32(const DecodeParams& p_, int lane_, int g_, int64_t unit_)
      : p(p_), lane(lane_), n(lane_ & 15), quad(lane_ >> 4), g(g_),
        gp(vhead_pool_head(g_, p_.qsplit)), unit(unit_) {
    const VHead v = vhead_rows(g_, p_.qsplit, p_.kv_group);
    qh0 = v.first;
    gw = v.count;
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }

  // Columns n >= gw repeat the last head (see the 16-bit stream).
  __device__ __forceinline__ void load_q(const Cursor& c) {
    const float4* qrow = reinterpret_cast<const float4*>(
        static_cast<const float*>(p.q) +
        ((int64_t)c.b * p.num_q_heads + qh0 + min(n, gw - 1)) * D + 4 * quad);
#pragma unroll
    for (int i = 0; i < KQ / 4; ++i) {
      const float4 v = qrow[4 * i];   // dims 16*i + 4*quad .. + 3
      qop[4 * i] = v.x;
      qop[4 * i + 1] = v.y;
      qop[4 * i + 2] = v.z;
      qop[4 * i + 3] = v.w;
    }
  }

  __device__ __forceinline__ void fetch_phys(const Cursor& c, int* ph) const {
    const const_i32_ptr trow = (const_i32_ptr)(p.block_tables + (int64_t)c.b * p.max_blocks_per_seq);
    ph[0] = uni(trow[fdiv(c.j * 16, p.bs_div)]);
  }

  __device__ __forceinline__ const char* tile_base(const Cursor& c, const int* ph) const {
    const int tok = c.j * 16;
    const int off = tok - (int)fdiv(tok, p.bs_div) * p.pool.block_size;   // tok % block_size
    return p.pool.base + 4 * ((int64_t)p.layer * p.pool.layer_stride +
                              (int64_t)gp * p.pool.head_stride +
                              (int64_t)ph[0] * p.pool.block_stride + (int64_t)off * D);
  }

  __device__ __forceinline__ const char* new_row(const Cursor& c, int kv) const {
    return static_cast<const char*>(kv ? p.v_new : p.k_new) +
           4 * ((int64_t)c.b * p.pool.kv_heads + gp) * D;
  }

  __device__ __forceinline__ void issue_k(Buf& cb, const Cursor& c, const int* ph) const {
    const char* kl = tile_base(c, ph) + (uint32_t)(4 * (n * D + 4 * quad));
    if constexpr (APPEND) {
      if (c.j * 16 + n == c.pos) kl = new_row(c, 0) + 4 * 4 * quad;
    }
#pragma unroll
    for (int i = 0; i < KQ / 4; ++i) {
      uint4 u;
      stream_load(u, kl + 64 * i);
      cb.k[i] = __builtin_bit_cast(float4, u);
    }
  }

  __device__ __forceinline__ void issue_v(Buf& cb, const Cursor& c, const int* ph) const {
    const char* vl = tile_base(c, ph) + 4 * p.pool.kv_stride + (uint32_t)(4 * (4 * quad * D + 4 * n));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const char* row = vl + 4 * r * D;
      if constexpr (APPEND) {
        if (c.j * 16 + 4 * quad + r == c.pos) row = new_row(c, 1) + 4 * 4 * n;
      }
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        uint4 u;
        stream_load(u, row + 4 * 64 * h);
        cb.v[r][h] = __builtin_bit_cast(float4, u);
      }
    }
  }

  __device__ __forceinline__ void qk(const Buf& cb, f32x4_t* s) const {
    f32x4_t a[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) a[w] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KQ / 4; ++i) {
      a[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(cb.k[i].x, qop[4 * i], a[0], 0, 0, 0);
      a[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(cb.k[i].y, qop[4 * i + 1], a[1], 0, 0, 0);
      a[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(cb.k[i].z, qop[4 * i + 2], a[2], 0, 0, 0);
      a[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(cb.k[i].w, qop[4 * i + 3], a[3], 0, 0, 0);
    }
    s[0] = (a[0] + a[1]) + (a[2] + a[3]);
  }

  template <bool TAIL>
  __device__ __forceinline__ void attend(const f32x4_t* s, Buf& cb, const Cursor& c) {
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = s[0][r] * p.scale_log2;
      if (TAIL && c.j * 16 + 4 * quad + r >= c.T) sv[r] = -INFINITY;
    }
    float bmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    bmax = max_x32(max_x16(bmax));
    {
      const float mn = fmaxf(m, bmax);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[i] *= alpha;
      l *= alpha;
      m = mn;
    }
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(sv[r] - m);
    l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    if (TAIL) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (c.j * 16 + 4 * quad + r >= c.T)
#pragma unroll
          for (int h = 0; h < NH; ++h) cb.v[r][h] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        acc[4 * h + 0] = __builtin_amdgcn_mfma_f32_16x16x4f32(cb.v[r][h].x, pr[r], acc[4 * h + 0], 0, 0, 0);
        acc[4 * h + 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(cb.v[r][h].y, pr[r], acc[4 * h + 1], 0, 0, 0);
        acc[4 * h + 2] = __builtin_amdgcn_mfma_f32_16x16x4f32(cb.v[r][h].z, pr[r], acc[4 * h + 2], 0, 0, 0);
        acc[4 * h + 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(cb.v[r][h].w, pr[r], acc[4 * h + 3], 0, 0, 0);
      }
  }

  __device__ __forceinline__ void attend_chunk(const f32x4_t* s, Buf& cb, const Cursor& c) {
    if (c.j == c.nb - 1 && (c.T % 16) != 0)
      attend<true>(s, cb, c);
    else
      attend<false>(s, cb, c);
  }

  __device__ void flush(const Cursor& c, bool whole) {
    const int G = p.group;   // partial slot stride
    const float lt = sum_x32(sum_x16(l));
    if (n >= gw) return;
    // lane holds dim 64*h + 16*quad + 4*r + e of head n as acc[4*h + e][r]
    if (whole) {
      const float inv = 1.0f / lt;
      float* dst = static_cast<float*>(p.out) +
                   ((int64_t)c.b * p.num_q_heads + qh0 + n) * D + 16 * quad;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<float4*>(dst + 64 * h + 4 * r) =
              make_float4(acc[4 * h][r] * inv, acc[4 * h + 1][r] * inv, acc[4 * h + 2][r] * inv,
                          acc[4 * h + 3][r] * inv);
    } else {
      const int64_t slot = partial_slot(c.b, g, unit, p.vheads);
      float* o = p.ws_o + (slot * G + n) * D + 16 * quad;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<float4*>(o + 64 * h + 4 * r) =
              make_float4(acc[4 * h][r], acc[4 * h + 1][r], acc[4 * h + 2][r], acc[4 * h + 3][r]);
      if (quad == 0) {
        p.ws_ml[(slot * G + n) * 2 + 0] = m;
        p.ws_ml[(slot * G + n) * 2 + 1] = lt;
      }
    }
  }
};

// One wavefront's pass over rem >= 1 consecutive chunks of the chunk space
// for KV head g, starting at cur: the range may cross into later sequences
// (prefix, lens and poss are read only at such a boundary).  Each sequence
// it touches is flushed, as a normalised output if the wavefront saw it from
// chunk 0 to its last chunk, else as a partial in the slot of `unit`.
template <typename S>
__device__ __forceinline__ void stream_chunks(const DecodeParams& p, int lane, int g, int64_t unit,
                                              const int32_t* prefix, const_i32_ptr lens,
                                              const_i32_ptr poss, Cursor cur, int rem) {
  S st(p, lane, g, unit);
  st.reset();
  st.load_q(cur);
  typename S::Buf cb;
  int ph[S::kPh], ph_nx[S::kPh], ph_n2[S::kPh];
  st.fetch_phys(cur, ph);
  st.issue_k(cb, cur, ph);
  st.issue_v(cb, cur, ph);
  Cursor nx = cur;
#pragma unroll
  for (int t = 0; t < S::kPh; ++t) ph_nx[t] = 0;
  if (rem > 1) {
    nx.advance(prefix, lens, poss, p.batch);
    st.fetch_phys(nx, ph_nx);
  }
  bool whole_start = cur.j == 0;   // this wave has seen the current sequence from chunk 0

  f32x4_t s[S::kCols * S::kTiles];
  for (int i = 0; i + 1 < rem; ++i) {
    st.qk(cb, s);
    __builtin_amdgcn_sched_barrier(0);
    st.issue_k(cb, nx, ph_nx);
    // q is dead until the next chunk's QK, so a new sequence's q loads in place
    const bool sw = nx.b != cur.b;
    if (sw) st.load_q(nx);
    __builtin_amdgcn_sched_barrier(0);
    Cursor n2 = nx;
#pragma unroll
    for (int t = 0; t < S::kPh; ++t) ph_n2[t] = 0;
    if (i + 2 < rem) {
      n2.advance(prefix, lens, poss, p.batch);
      st.fetch_phys(n2, ph_n2);
    }
    st.attend_chunk(s, cb, cur);
    __builtin_amdgcn_sched_barrier(0);
    st.issue_v(cb, nx, ph_nx);
    __builtin_amdgcn_sched_barrier(0);
    if (sw) {
      st.flush(cur, whole_start);
      st.reset();
      whole_start = true;
    }
    cur = nx;
    nx = n2;
#pragma unroll
    for (int t = 0; t < S::kPh; ++t) ph_nx[t] = ph_n2[t];
  }
  st.qk(cb, s);
  st.attend_chunk(s, cb, cur);
  st.flush(cur, whole_start && cur.j == cur.nb - 1);
}

// Wait until at most N vector-memory operations of this wavefront are in
// flight (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// left at their maxima, so they are not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most `newer` chunk copies (LPC LDS-direct loads each)
// issued after the oldest one are still in flight, for newer in [0, K].
template <int K, int LPC>
__device__ __forceinline__ void wait_newer_chunks(int newer) {
  if constexpr (K == 0) {
    wait_vmcnt<0>();
  } else {
    if (newer >= K)
      wait_vmcnt<LPC * K>();
    else
      wait_newer_chunks<K - 1, LPC>(newer);
  }
}

// One wavefront of the per-pair kernel over chunks cur.j, cur.j + stride,
// ... (rem of them) of one sequence, its K and V staged through NS LDS slots
// of slot_bytes<VS>() from `slot0`: while the wavefront computes chunk i
// from registers, chunks i + 1 .. i + NS are in flight or waiting in LDS.  A
// chunk's copy is chunk_loads<VS>() LDS-direct loads (K and V, or K and half
// of V, two tiles, 1 KiB of lanes each), and vector-memory operations
// complete in issue order, so chunk i is in LDS once at most the loads of
// the chunks copied after it are still in flight.  Lane 2k + t of `ent`
// holds the block-table entry of tile t of the wavefront's k-th chunk
// (loaded by the caller with the sequence's length), so the loop makes no
// table loads: a scalar load issued in one step would be waited for by the
// next step's LDS reads (s_waitcnt lgkmcnt counts both), which put its
// latency on every chunk.  The loop runs NS chunks per pass so that each
// read has its slot as an immediate offset.
template <int P> struct SlotTag { static constexpr int value = P; };

// Chunks of one wavefront of the per-pair LDS-staged stream: w, w + A,
// w + 2A, ... for the A = min(n, NW) of the workgroup's NW wavefronts that
// have chunks.  They are w, w + NW, w + 2 NW, ... whatever the pair's chunk
// count n (with A < NW each wavefront has at most one), so their table
// entries can be loaded before n is known.  (Rounds that gave
// wavefronts 0..3, the first of each SIMD, four chunks for every three of
// the others were slower: churned pool 10.75 -> 11.5 us.)
struct PairChunks {
  int w, stride;
  __device__ __forceinline__ int at(int i) const { return w + i * stride; }
};

// With VS the workgroup stages half `dhalf` of V's dims (the other half is
// its partner workgroup's) and writes only those dims of the output.
template <typename S, int NS, bool VS>
__device__ __forceinline__ void stream_pair_lds(const DecodeParams& p, int lane, int g, int64_t unit,
                                                Cursor cur, PairChunks pc, int rem, int ent,
                                                uint32_t slot0, int dhalf) {
  static_assert(NS == 1 || NS == 2 || NS == 4, "slots per wavefront");
  S st(p, lane, g, unit);
  st.reset();
  st.load_q(cur);
  const typename S::LdsLane la = st.template lds_lane<VS>(slot0, dhalf);
  typename S::Buf cb;
  constexpr uint32_t SB = S::template slot_bytes<VS>();
  constexpr int LPC = S::template chunk_loads<VS>();
  const bool whole = cur.nb == 1;
  static_assert(S::kPh == 2, "two tiles per chunk");
  // the entries arrive before the first copy is issued: waiting for them
  // here, on every path, keeps the compiler from waiting for all vector
  // memory (copies included) at a later use
  asm volatile("" ::"v"(ent));
  // lane 2k + t: address of tile t of the wavefront's k-th chunk, worked
  // out once for all chunks, so that a chunk's copies take four lane reads
  // instead of ~30 scalar operations (0.17 us on the churned-pool call); a
  // tile that starts at or past T takes the block of the chunk's first tile
  // (its rows are masked)
  const int tokl = pc.at(lane >> 1) * S::kChunk + 16 * (lane & 1);
  const int ent0 = __builtin_amdgcn_update_dpp(0, ent, 0xA0, 0xf, 0xf, false);   // lane & ~1
  const uint64_t tla = (uint64_t)(uintptr_t)st.tile_addr(tokl < cur.T ? ent : ent0, tokl);
  const uint32_t tlo = (uint32_t)tla, thi = (uint32_t)(tla >> 32);
  auto chunk_blocks = [&](int k, const char** tb) {
    const int e = (2 * k) & 63;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      tb[t] = (const char*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(thi, e + t) << 32) |
                                       (uint32_t)__builtin_amdgcn_readlane(tlo, e + t));
  };
#pragma unroll
  for (int k = 0; k < NS; ++k)
    if (k < rem) {
      Cursor c = cur;
      c.j = pc.at(k);
      const char* tb[2];
      chunk_blocks(k, tb);
      st.template dma_chunk<VS>(c, tb, slot0 + k * SB, dhalf);
    }
  f32x4_t s[S::kTiles];
  auto step = [&](auto tag, int i) {
    constexpr int P = decltype(tag)::value;
    wait_newer_chunks<NS - 1, LPC>(rem - 1 - i);
    st.template read_chunk<P, VS>(cb, la);
    st.qk(cb, s);
    if (i + NS < rem) {   // chunk i + NS into the slot just read
      Cursor c = cur;
      c.j = pc.at(i + NS);
      const char* tb[2];
      chunk_blocks(i + NS, tb);
      st.template dma_chunk<VS>(c, tb, slot0 + P * SB, dhalf);
    }
    cur.j = pc.at(i);
    st.template attend_chunk<true, VS>(s, cb, cur);
  };
  for (int i = 0; i < rem; i += NS) {
    step(SlotTag<0>{}, i);
    if constexpr (NS >= 2)
      if (i + 1 < rem) step(SlotTag<1>{}, i + 1);
    if constexpr (NS == 4) {
      if (i + 2 < rem) step(SlotTag<2>{}, i + 2);
      if (i + 3 < rem) step(SlotTag<3>{}, i + 3);
    }
  }
  if (whole) {
    if constexpr (VS)
      st.flush_whole_vs(cur, st.lacc[0][0], dhalf);
    else if (st.n < st.gw)
      st.flush_cols(cur, true, 0, st.lacc[0][0]);
  } else {   // the partial goes to this wavefront's own (now free) slots
    if constexpr (VS)
      st.flush_lds_vs(slot0, dhalf);
    else
      st.flush_lds(slot0);
  }
}

// One persistent kernel for every stream type S (16-bit or fp32 elements).
template <typename S>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeParams p) {
  extern __shared__ int32_t prefix[];
  __shared__ int32_t scan[kThreads / 64];
  const int H = p.vheads;   // (virtual) KV heads

  if constexpr (S::kDense) {   // every sequence is dense_len tokens long
    const int nc = chunks_of(p.dense_len, S::kChunk);
    for (int i = threadIdx.x; i <= p.batch; i += kThreads) prefix[i] = i * nc;
    __syncthreads();
  } else {
    block_chunk_prefix<kThreads>(p.context_lens, p.batch, S::kChunk, prefix, scan);
  }
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= p.batch; i += kThreads) p.ws_prefix[i] = prefix[i];

  const int lane = threadIdx.x & 63;
  // A unit's H wavefronts span npu = H / kWaves workgroups.  Those workgroups
  // are blockIdx u, u + grid/npu, ...: workgroups go to the XCDs round-robin,
  // so a unit's workgroups share an XCD when grid/npu is a multiple of 8.
  int64_t unit;
  int g;
  const int w = uni(threadIdx.x >> 6);
  const int npu = H / kWaves;
  if (H % kWaves == 0 && npu > 1 && gridDim.x % npu == 0) {
    const int stride = gridDim.x / npu;
    const int k = blockIdx.x / stride;
    unit = blockIdx.x - k * stride;
    g = k * kWaves + w;
  } else {
    // With one (virtual) KV head a unit is one wavefront, and the units that
    // get work (fewer than launched when chunks are few) go round-robin over
    // the workgroups rather than filling the first ones, so that they spread
    // over every CU: one KV head for 32 query heads at batch 64 went from
    // 34.6 to 30.4 us per call.
    const int64_t wave = H == 1 ? (int64_t)w * gridDim.x + blockIdx.x
                                : (int64_t)blockIdx.x * kWaves + w;
    unit = fdiv((uint32_t)wave, p.vh_div);
    g = (int)(wave - unit * H);
  }
  const int64_t C = uni(prefix[p.batch]);
  const int64_t Ue = waves_eff(C, p.units, p.min_chunks);
  if (unit >= Ue) return;
  const int64_t c0 = wave_begin(unit, C, Ue);
  const int rem = (int)(wave_begin(unit + 1, C, Ue) - c0);   // >= 1

  const const_i32_ptr lens = S::kDense ? nullptr : (const_i32_ptr)p.context_lens;
  const const_i32_ptr poss = S::kAppend ? (const_i32_ptr)p.positions : nullptr;
  Cursor cur;
  cur.dense_T = p.dense_len;
  cur.b = uni(seq_of_chunk(prefix, p.batch, c0));
  cur.load_seq(prefix, lens, poss);
  cur.j = uni((int)(c0 - prefix[cur.b]));
  stream_chunks<S>(p, lane, g, unit, prefix, lens, poss, cur, rem);
}

// Small batches: one workgroup of NW wavefronts per (sequence b, virtual KV
// head g) pair, so that the split of a sequence and the merge of its pieces
// stay inside one workgroup and no merge launch follows.  Of the pair's n
// chunks, wavefront w < A = min(n, NW) streams [w*n/A, (w+1)*n/A) and
// leaves a partial (running max, sum, unnormalised output) in slot
// (kPairWaves*b + w)*vheads + g of the workspace; with the LDS-staged
// stream it takes chunks w, w + A, w + 2A, ... and leaves its partial in
// its own LDS slots.  After a barrier the wavefronts combine the A partials
// of each query head with the same log-sum-exp update as the merge pass and
// write the output rows.  A pair one wavefront sees whole (n == 1) is
// written directly; an empty one (T_b = 0) gets zero rows.  With a fused
// append the workgroup of the pool head's first virtual head also stores
// the new K/V rows into the pool: this call reads them from k_new / v_new
// only, so the store may come at any time.
constexpr int kPairWaves = 8;   // NW of the register stream
// NW of the LDS-staged stream, and its slots per wavefront
constexpr int kLdsWaves = 8;
constexpr int kLdsSlots = 2;
template <typename S>
constexpr int pair_waves() { return S::kLdsStream ? kLdsWaves : kPairWaves; }
// K/V bytes per wavefront up to which the per-pair kernel is used.  Measured
// (batches of 4 to 64 sequences, head_dim 64 and 128, bf16 and fp32): one
// workgroup per pair is 15-25% faster than the chunk split and merge kernel
// up to ~32 KB per wavefront, and slower beyond: a pair's bytes then all go
// through one CU, which streams only ~27 GB/s however many wavefronts it
// runs (16 wavefronts per pair were slower than 8 at the same length).
constexpr int64_t kPairBytesPerWave = 32 << 10;
// K/V bytes per pair up to which the LDS-staged stream (head_dim 64,
// 16-bit, blocks of a multiple of 16 tokens) is used; it keeps several
// chunks in flight per wavefront without registers and merges through LDS.
constexpr int64_t kPairBytesLds = 512 << 10;
// Chunks (32 tokens of head_dim 64 in 16 bits: 8 KiB) per wavefront at most
// on the LDS-staged stream with NW wavefronts: kPairBytesLds of K and V over
// NW, rounded up.
template <int NW>
constexpr int lds_chunks_per_wave() {
  return (int)((kPairBytesLds / (8 << 10) + NW - 1) / NW);
}
static_assert(2 * lds_chunks_per_wave<kLdsWaves>() <= 64, "one table entry per lane");

// VS (LDS-staged stream only): two workgroups per pair, each staging K and
// half of V's dims and writing those dims of the output rows; the halves of
// pair pr are workgroups 16 (pr / 8) + pr % 8 and that + 8, which share an
// XCD (workgroups go to the 8 XCDs round-robin), so their K reads meet in
// one L2.  The grid is twice the pair count rounded up to a multiple of 8.
template <typename S, bool VS = false>
__global__ __launch_bounds__(64 * pair_waves<S>()) void decode_pair_kernel(DecodeParams p) {
  using Out = typename S::OutElem;
  constexpr int NW = pair_waves<S>();
  static_assert(!VS || S::kLdsStream, "split V only with the LDS-staged stream");
  // The kernel-argument fields the prologue reads, requested before its
  // first branch: their loads then go out in one batch, not in a second
  // one after the early exit, which would wait a round trip of its own.
  asm volatile("" ::"s"(p.block_tables), "s"(p.context_lens), "s"(p.positions),
               "s"(p.max_blocks_per_seq), "s"(p.pool.block_size), "s"(p.batch), "s"(p.vheads));
  const int H = p.vheads;
  int pr = blockIdx.x, dhalf = 0;
  if constexpr (VS) {
    pr = (int)(blockIdx.x >> 4) * 8 + (int)(blockIdx.x & 7);
    dhalf = (int)(blockIdx.x >> 3) & 1;
    if (pr >= p.batch * H) return;
  }
  const int b = (int)fdiv((uint32_t)pr, p.vh_div);
  const int g = pr - b * H;
  const int lane = threadIdx.x & 63;
  const int w = uni(threadIdx.x >> 6);
  const const_i32_ptr lens = (const_i32_ptr)p.context_lens;
  const const_i32_ptr poss = S::kAppend ? (const_i32_ptr)p.positions : nullptr;
  Cursor cur;
  cur.dense_T = 0;
  cur.b = b;
  // LDS-staged stream: wavefront w < min(n, NW) takes chunks w, w + NW, ...
  // (so its chunks are known before the length is), and one vector load
  // issued together with the length brings the table entries of all of
  // them: lane 2k + t takes tile t of chunk w + NW k, for the at most
  // lds_chunks_per_wave<NW>() chunks a wavefront gets.  Indices are clamped into the
  // table row; an entry of a chunk that does not exist is never used.
  int ent = 0;
  if constexpr (S::kLdsStream) {
    const int32_t* trow = p.block_tables + (int64_t)b * p.max_blocks_per_seq;
    const unsigned last = (unsigned)p.max_blocks_per_seq - 1;
    if (lane < 2 * lds_chunks_per_wave<NW>())
      ent = trow[min(fdiv((uint32_t)((w + NW * (lane >> 1)) * S::kChunk + 16 * (lane & 1)), p.bs_div),
                     last)];
  }
  cur.T = uni(lens[b]);
  cur.pos = poss ? uni(poss[b]) : -1;
  cur.nb = chunks_of(cur.T, S::kChunk);
  const int n = cur.nb;
  const int A = min(n, NW);   // wavefronts with chunks (uniform over the workgroup)
  // Fused append: the last wavefront stores the new K/V rows of the pool
  // head (one 16-byte unit per lane) once the workgroup is done; its loads
  // are issued here so that they are in hand by then.
  constexpr int D = S::kDim;
  const int row_units = D * (int)sizeof(Out) / 16;   // 16-byte units per row
  const bool app_row = S::kAppend && w == NW - 1 && cur.pos >= 0 && dhalf == 0 &&
                       (p.qsplit == 1 || g % p.qsplit == 0);
  uint4 row_unit = make_uint4(0, 0, 0, 0);
  int row_phys = 0;
  if (app_row) {
    const int gp = vhead_pool_head(g, p.qsplit);
    const int kv = lane >= row_units;
    if (lane < 2 * row_units)
      row_unit = reinterpret_cast<const uint4*>(
          static_cast<const Out*>(kv ? p.v_new : p.k_new) +
          ((int64_t)b * p.pool.kv_heads + gp) * D)[lane - kv * row_units];
    row_phys = p.block_tables[(int64_t)b * p.max_blocks_per_seq + fdiv(cur.pos, p.bs_div)];
  }
  if (w < A) {
    // unit 7b + w makes partial_slot() give slot (8b + w) * vheads + g
    if constexpr (S::kLdsStream) {
      extern __shared__ __attribute__((aligned(16))) unsigned char pair_lds[];
      const uint32_t slot0 =
          (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)pair_lds +
          (uint32_t)w * kLdsSlots * S::template slot_bytes<VS>();
      PairChunks pc;
      pc.w = w;
      pc.stride = A;
      cur.j = w;
      stream_pair_lds<S, kLdsSlots, VS>(p, lane, g, (int64_t)(kPairWaves - 1) * b + w, cur, pc,
                                        A == NW ? (n - 1 - w) / NW + 1 : 1, ent, slot0, dhalf);
    } else {
      cur.j = w * n / A;
      stream_chunks<S>(p, lane, g, (int64_t)(kPairWaves - 1) * b + w, nullptr, lens, poss, cur,
                       (w + 1) * n / A - cur.j);
    }
  }

  const VHead vh = vhead_rows(g, p.qsplit, p.kv_group);
  constexpr int DPL = (D + 63) / 64;   // dims per lane in the merge
  Out* out = static_cast<Out*>(p.out) + ((int64_t)b * p.num_q_heads + vh.first) * D;
  if (A == 0) {
    for (int hn = w; hn < vh.count; hn += NW)
      for (int d = lane; d < D; d += 64)
        if (!VS || d / 32 == dhalf) out[(int64_t)hn * D + d] = (Out)0.f;
  } else if (A > 1) {
    __syncthreads();   // the A partials are written (workgroup-scope release and acquire)
    const int G = p.group;   // partial slot stride
    for (int hn = w; hn < vh.count; hn += NW) {
      float mv[NW], lv[NW], ov[NW][DPL];
#pragma unroll
      for (int u = 0; u < NW; ++u) {
        const int k = min(u, A - 1);   // copies past A are not folded
        if constexpr (S::kLdsStream) {   // wavefront k's partial, in its LDS slots
          extern __shared__ __attribute__((aligned(16))) unsigned char pair_lds[];
          const float* part = reinterpret_cast<const float*>(
              pair_lds + (size_t)k * kLdsSlots * S::template slot_bytes<VS>());
          mv[u] = part[vh.count * D + 2 * hn];
          lv[u] = part[vh.count * D + 2 * hn + 1];
#pragma unroll
          for (int i = 0; i < DPL; ++i) {
            const int d = lane + 64 * i;
            ov[u][i] = d < D ? part[hn * D + d] : 0.f;
          }
        } else {
          const int64_t e = (((int64_t)kPairWaves * b + k) * H + g) * G + hn;
          mv[u] = p.ws_ml[2 * e];
          lv[u] = p.ws_ml[2 * e + 1];
#pragma unroll
          for (int i = 0; i < DPL; ++i) {
            const int d = lane + 64 * i;
            ov[u][i] = d < D ? p.ws_o[e * D + d] : 0.f;
          }
        }
      }
      float M = -INFINITY, L = 0.f, a[DPL];
#pragma unroll
      for (int i = 0; i < DPL; ++i) a[i] = 0.f;
#pragma unroll
      for (int u = 0; u < NW; ++u) {
        if (u < A) {
          const float Mn = fmaxf(M, mv[u]);
          const float sc = __builtin_amdgcn_exp2f(M - Mn);
          const float wt = __builtin_amdgcn_exp2f(mv[u] - Mn);
          L = L * sc + wt * lv[u];
#pragma unroll
          for (int i = 0; i < DPL; ++i) a[i] = a[i] * sc + wt * ov[u][i];
          M = Mn;
        }
      }
      const float inv = 1.0f / L;   // every piece holds at least one token
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const int d = lane + 64 * i;
        if (d < D && (!VS || d / 32 == dhalf)) out[(int64_t)hn * D + d] = (Out)(a[i] * inv);
      }
    }
  }

  if constexpr (S::kAppend) {
    if (app_row && lane < 2 * row_units) {
      const int kv = lane >= row_units;
      const int gp = vhead_pool_head(g, p.qsplit);
      const int64_t row = (int64_t)row_phys * p.pool.block_stride +
                          (int64_t)p.layer * p.pool.layer_stride + (int64_t)gp * p.pool.head_stride +
                          (int64_t)(cur.pos - (int)fdiv(cur.pos, p.bs_div) * p.pool.block_size) * D +
                          kv * p.pool.kv_stride;
      reinterpret_cast<uint4*>(reinterpret_cast<Out*>(const_cast<char*>(p.pool.base)) + row)[lane - kv * row_units] =
          row_unit;
    }
  }
}

size_t mfma_lds_bytes(int batch) { return sizeof(int32_t) * (size_t)(batch + 1); }

}  // namespace

// Query heads one wavefront can serve: 32 (two column groups) for 16-bit
// pools at head_dim 64 or 128 with blocks of a multiple of 16 tokens, else 16.
int mfma_max_group(const kv_pool* pool) {
  const int d = pool->head_dim;
  const bool wide = pool->dtype != PAGEDKV_F32 && (d == 64 || d == 128) &&
                    pool->block_size % 16 == 0;
  return wide ? 2 * kMaxGroup : kMaxGroup;
}

bool mfma_supported(const kv_pool* pool, int group) {
  const int d = pool->head_dim, bs = pool->block_size;
  const bool half = pool->dtype != PAGEDKV_F32;
  const bool dim_ok = d == 64 || d == 128 || ((d == 96 || d == 256) && half);
  const bool bs_ok = bs % 16 == 0 || ((bs == 4 || bs == 8) && half);
  return dim_ok && bs_ok && group >= 1 && group <= mfma_max_group(pool);
}

int mfma_chunk_tokens(int head_dim) { return 16 * (head_dim == 256 ? kTilesD256 : kTilesPerStep); }

namespace {
// Launch the per-pair kernel if its instantiation for S runs without scratch
// (register spills), the pieces' slots fit the workspace and every pair's
// workgroup is resident at once.
template <typename S>
bool launch_pairs(const DecodeParams& p, int64_t pairs, hipStream_t s) {
  if constexpr (S::kLdsStream) {
    // two workgroups per pair (each with half of V's dims) while they all
    // fit on the device at once
    const void* fv = reinterpret_cast<const void*>(&decode_pair_kernel<S, true>);
    static const bool spill_free_v = [fv] {
      hipFuncAttributes a;
      return hipFuncGetAttributes(&a, fv) == hipSuccess && a.localSizeBytes == 0;
    }();
    constexpr int NWV = pair_waves<S>();
    const size_t ldsv = (size_t)NWV * kLdsSlots * S::template slot_bytes<true>();
    const int64_t grid = 2 * ((pairs + 7) / 8 * 8);
    int resident = 0;
    if (spill_free_v && resident_workgroups(fv, 64 * NWV, ldsv, &resident) == hipSuccess &&
        grid <= resident) {
      hipLaunchKernelGGL((decode_pair_kernel<S, true>), dim3((unsigned)grid), dim3(64 * NWV), ldsv,
                         s, p);
      return true;
    }
  }
  const void* fn = reinterpret_cast<const void*>(&decode_pair_kernel<S>);
  static const bool spill_free = [fn] {
    hipFuncAttributes a;
    return hipFuncGetAttributes(&a, fn) == hipSuccess && a.localSizeBytes == 0;
  }();
  constexpr int NW = pair_waves<S>();
  const size_t lds = S::kLdsStream ? (size_t)NW * kLdsSlots * S::kSlotBytes : 0;
  int resident = 0;
  if (!spill_free || (kPairWaves - 1) * pairs > kMaxWaves ||
      resident_workgroups(fn, 64 * NW, lds, &resident) != hipSuccess || pairs > resident)
    return false;
  hipLaunchKernelGGL((decode_pair_kernel<S>), dim3((unsigned)pairs), dim3(64 * NW), lds, s, p);
  return true;
}

// Pass 1 for stream type S.  When p.pair_mode asks for it, the per-pair
// kernel runs if the longest sequence the block tables allow holds at most
// kPairWaves * kPairBytesPerWave of K and V per pair (kPairBytesLds for the
// LDS-staged stream); otherwise p.pair_mode is cleared and the persistent
// kernel runs on wgs workgroups.
template <typename S>
void launch_one(DecodeParams& p, int wgs, size_t lds, hipStream_t s) {
  if constexpr (S::kPairs) {
    if (p.pair_mode) {
      const int64_t pairs = (int64_t)p.batch * p.vheads;
      const int64_t bytes = 2 * (int64_t)p.max_blocks_per_seq * p.pool.block_size *
                            p.pool.head_dim * (p.dtype == PAGEDKV_F32 ? 4 : 2);
      const int64_t limit = S::kLdsStream ? kPairBytesLds : kPairWaves * kPairBytesPerWave;
      if (bytes <= limit && launch_pairs<S>(p, pairs, s)) return;
    }
  }
  p.pair_mode = 0;
  hipLaunchKernelGGL((decode_mfma_kernel<S>), dim3(wgs), dim3(kThreads), lds, s, p);
}

template <typename E>
void launch_typed(DecodeParams& p, int wgs, size_t lds, hipStream_t s) {
  const bool append = p.positions != nullptr;
  constexpr int T = kTilesPerStep;
  constexpr int T2 = kTilesD256;
  if (p.k_dense) {
    if (p.pool.head_dim == 256) launch_one<Stream<E, 256, T2, false, true>>(p, wgs, lds, s);
    else if (p.pool.head_dim == 128) launch_one<Stream<E, 128, T, false, true>>(p, wgs, lds, s);
    else if (p.pool.head_dim == 96) launch_one<Stream<E, 96, T, false, true>>(p, wgs, lds, s);
    else launch_one<Stream<E, 64, T, false, true>>(p, wgs, lds, s);
    return;
  }
  if (p.pool.block_size < 16) {   // 4 or 8 tokens per block
    if (p.pool.head_dim == 256) {
      if (append) launch_one<Stream<E, 256, T2, true, false, true>>(p, wgs, lds, s);
      else launch_one<Stream<E, 256, T2, false, false, true>>(p, wgs, lds, s);
    } else if (p.pool.head_dim == 128) {
      if (append) launch_one<Stream<E, 128, T, true, false, true>>(p, wgs, lds, s);
      else launch_one<Stream<E, 128, T, false, false, true>>(p, wgs, lds, s);
    } else if (p.pool.head_dim == 96) {
      if (append) launch_one<Stream<E, 96, T, true, false, true>>(p, wgs, lds, s);
      else launch_one<Stream<E, 96, T, false, false, true>>(p, wgs, lds, s);
    } else {
      if (append) launch_one<Stream<E, 64, T, true, false, true>>(p, wgs, lds, s);
      else launch_one<Stream<E, 64, T, false, false, true>>(p, wgs, lds, s);
    }
    return;
  }
  if (p.group > kMaxGroup) {   // two column groups (head_dim 64 or 128)
    if (p.pool.head_dim == 128) {
      if (append) launch_one<Stream<E, 128, T, true, false, false, 2>>(p, wgs, lds, s);
      else launch_one<Stream<E, 128, T, false, false, false, 2>>(p, wgs, lds, s);
    } else {
      if (append) launch_one<Stream<E, 64, T, true, false, false, 2>>(p, wgs, lds, s);
      else launch_one<Stream<E, 64, T, false, false, false, 2>>(p, wgs, lds, s);
    }
    return;
  }
  if (p.pool.head_dim == 256) {
    if (append) launch_one<Stream<E, 256, T2, true>>(p, wgs, lds, s);
    else launch_one<Stream<E, 256, T2, false>>(p, wgs, lds, s);
  } else if (p.pool.head_dim == 128) {
    if (append) launch_one<Stream<E, 128, T, true>>(p, wgs, lds, s);
    else launch_one<Stream<E, 128, T, false>>(p, wgs, lds, s);
  } else if (p.pool.head_dim == 96) {
    if (append) launch_one<Stream<E, 96, T, true>>(p, wgs, lds, s);
    else launch_one<Stream<E, 96, T, false>>(p, wgs, lds, s);
  } else {
    if (append) launch_one<Stream<E, 64, T, true>>(p, wgs, lds, s);
    else launch_one<Stream<E, 64, T, false>>(p, wgs, lds, s);
  }
}

void launch_f32(DecodeParams& p, int wgs, size_t lds, hipStream_t s) {
  const bool append = p.positions != nullptr;
  if (p.pool.head_dim == 128) {
    if (append) launch_one<StreamF32<128, true>>(p, wgs, lds, s);
    else launch_one<StreamF32<128, false>>(p, wgs, lds, s);
  } else {
    if (append) launch_one<StreamF32<64, true>>(p, wgs, lds, s);
    else launch_one<StreamF32<64, false>>(p, wgs, lds, s);
  }
}
}  // namespace

hipError_t launch_decode_mfma(DecodeParams& p, hipStream_t s) {
  p.bs_div = make_fast_div((uint32_t)p.pool.block_size);
  p.vh_div = make_fast_div((uint32_t)p.vheads);
  const size_t lds = mfma_lds_bytes(p.batch);
  // The grid is kDecodeWgPerCu (1) workgroup per CU, capped by what one
  // instantiation of this head_dim holds at once.  Every instantiation holds
  // at least one workgroup per CU (its registers fit one wavefront per SIMD),
  // so the grid is resident whichever one runs, although they differ in
  // registers: the two-column-group streams hold one wavefront per SIMD
  // where the others hold two to four.
  const void* fn =
      p.pool.head_dim == 256
          ? reinterpret_cast<const void*>(&decode_mfma_kernel<Stream<Bf16Ops, 256, kTilesD256, false>>)
      : p.pool.head_dim == 128
          ? reinterpret_cast<const void*>(&decode_mfma_kernel<Stream<Bf16Ops, 128, kTilesPerStep, false>>)
          : reinterpret_cast<const void*>(&decode_mfma_kernel<Stream<Bf16Ops, 64, kTilesPerStep, false>>);
  const int chunk = p.dtype == PAGEDKV_F32 ? 16 : mfma_chunk_tokens(p.pool.head_dim);
  int wgs = 0;
  hipError_t e = resident_workgroups(fn, kThreads, lds, &wgs);
  if (e != hipSuccess) return e;
  const int dev_wgs = wgs;
  wgs = decode_workgroups(dev_wgs);
  p.units = wgs * kWaves / p.vheads;   // head groups
  if (p.units < 1) {                   // more KV heads than resident waves
    p.units = 1;
    wgs = (p.vheads + kWaves - 1) / kWaves;
  }
  // Each piece of a split sequence leaves a partial of group x head_dim fp32
  // values: group / 32 of one 32-token 16-bit chunk's K/V bytes.  At least
  // group / 4 chunks per unit (2 up to 11 query heads) keeps the partials
  // under 1/8 of the K/V a piece reads; measured on one KV head serving 32
  // query heads at batch 64: 38.8 -> 37.0 us per call.
  if (p.min_chunks < 1) p.min_chunks = p.group / 4 > 2 ? p.group / 4 : 2;
  // no more units than the largest possible chunk count can keep busy
  const int64_t max_chunks = (int64_t)p.batch *
      (((int64_t)p.max_blocks_per_seq * p.pool.block_size + chunk - 1) / chunk);
  const int64_t useful = (max_chunks + p.min_chunks - 1) / p.min_chunks;
  if (useful < p.units) {
    p.units = (int)(useful < 1 ? 1 : useful);
    wgs = (p.units * p.vheads + kWaves - 1) / kWaves;
  }
  if (p.dtype == PAGEDKV_F32)
    launch_f32(p, wgs, lds, s);
  else if (p.dtype == PAGEDKV_F16)
    launch_typed<F16Ops>(p, wgs, lds, s);
  else
    launch_typed<Bf16Ops>(p, wgs, lds, s);
  return hipGetLastError();
}

}  // namespace pagedkv
