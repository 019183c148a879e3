// HBM read-ceiling probe: a plain streaming read over slabs in a given order
// (pagedkv_probe.h).  It shares no code with the decode library; it exists
// to give the decode's bandwidth a measured denominator beside the 8 TB/s
// nameplate.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv_probe.h"

namespace {

constexpr int kLoadsInFlight = 32;   // 1 KiB lines per wavefront in flight

typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

// Address of this lane's 16 bytes of 1 KiB line `line` (wave-uniform) of the
// visit order.
__device__ __forceinline__ const u32x4_nt* line_addr(const char* base, const_i32_ptr ids,
                                                     int64_t line, int lines_shift,
                                                     int slab_shift, int max_id, int lane) {
  int slab = ids[line >> lines_shift];   // uniform index: a scalar load
  slab = slab < 0 ? 0 : (slab > max_id ? max_id : slab);
  const int64_t lines_mask = ((int64_t)1 << lines_shift) - 1;
  return reinterpret_cast<const u32x4_nt*>(base + ((int64_t)slab << slab_shift) +
                                           ((line & lines_mask) << 10) + 16 * lane);
}

__global__ __launch_bounds__(256) void read_probe_kernel(const char* __restrict__ base,
                                                         const int32_t* __restrict__ ids,
                                                         int64_t n_lines, int lines_shift,
                                                         int slab_shift, int max_id,
                                                         uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int64_t l0 = wave * n_lines / waves;
  const int64_t l1 = (wave + 1) * n_lines / waves;
  const const_i32_ptr sid = (const_i32_ptr)ids;
  uint32_t acc = 0;
  int64_t l = l0;
  // whole groups: every load of the group issued before any is consumed
  for (; l + kLoadsInFlight <= l1; l += kLoadsInFlight) {
    u32x4_nt v[kLoadsInFlight];
#pragma unroll
    for (int j = 0; j < kLoadsInFlight; ++j)
      v[j] = __builtin_nontemporal_load(
          line_addr(base, sid, l + j, lines_shift, slab_shift, max_id, lane));
    __builtin_amdgcn_sched_barrier(0);   // keep every load of the group ahead of its use
#pragma unroll
    for (int j = 0; j < kLoadsInFlight; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; l < l1; ++l) {   // the rest of the range, a line at a time
    const u32x4_nt v = __builtin_nontemporal_load(
        line_addr(base, sid, l, lines_shift, slab_shift, max_id, lane));
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

int log2_exact(int64_t x) {
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int s = 0;
  while ((int64_t(1) << s) < x) ++s;
  return s;
}

}  // namespace

extern "C" int pagedkv_read_probe(const void* base, size_t buffer_bytes, const int32_t* slab_ids,
                                  int64_t n_slabs, int slab_bytes, int workgroups, uint32_t* sink,
                                  void* stream) {
  const int slab_shift = log2_exact(slab_bytes);
  if (!base || !slab_ids || !sink || n_slabs < 1 || slab_bytes < 1024 || slab_shift < 0 ||
      workgroups < 1 || workgroups > 65535 || reinterpret_cast<uintptr_t>(base) % 16 != 0)
    return -1;
  const uint64_t slabs_in_buffer = buffer_bytes / (uint64_t)slab_bytes;
  if (slabs_in_buffer < 1 || (uint64_t)n_slabs > slabs_in_buffer ||
      slabs_in_buffer - 1 > (uint64_t)INT32_MAX)
    return -1;
  const int lines_shift = slab_shift - 10;
  hipLaunchKernelGGL(read_probe_kernel, dim3(workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(base), slab_ids,
                     n_slabs << lines_shift, lines_shift, slab_shift,
                     (int)(slabs_in_buffer - 1), sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
