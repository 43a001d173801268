// probes.hip -- measurement probes for the benchmark (not part of the layer):
//   probe_stream_read : read a buffer once with 16-byte loads (HBM ceiling)
//   probe_empty       : an empty kernel, for launch-gap measurements
//   probe_spin        : one wave that busy-waits a given number of microseconds
//                       (keeps the queue ahead of the host before a timed region)
//   probe_handoff     : an all-to-all hand-off through 16-byte records: every
//                       workgroup stores one record, one wave of every
//                       workgroup polls all of them (device-coherent loads and
//                       stores, as the one-token kernels' hand-offs)
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ p, int64_t n16,
                                                      uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // practically never: keeps the loads alive
}

__global__ void k_empty() {}

// Bounded: the wave leaves once the 100 MHz wall clock has advanced `ticks`.
__global__ void k_spin(uint64_t ticks) {
  const uint64_t w0 = wall_clock64();
  while (wall_clock64() - w0 < ticks) __builtin_amdgcn_s_sleep(8);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Grid <= 512: lane l of wave 0 polls records l + 64 v, v < 8.  Every wait is
// bounded by `limit` ticks of the 100 MHz wall clock.  st[2 b], st[2 b + 1]:
// workgroup b's start and the time it had seen every record (0 if it gave up).
__global__ __launch_bounds__(256) void k_handoff(u32x4_t* rec, uint32_t ep, uint64_t limit,
                                                 uint64_t* st) {
  const int t = threadIdx.x, b = blockIdx.x, n = gridDim.x, lane = t & 63;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(rec, 0, n * 16, 0x00020000);
  const uint64_t t0 = wall_clock64();
  if (t == 0) {
    const u32x4_t v = {(uint32_t)b, ep, 0u, ep ^ (uint32_t)b ^ 0x55u};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, b * 16, 0, 16);
  }
  bool ok = true;
  if (t < 64) {
    bool done[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) done[v] = lane + 64 * v >= n;
    for (;;) {
      u32x4_t x[8];
#pragma unroll
      for (int v = 0; v < 8; ++v)
        if (!done[v]) x[v] = __builtin_amdgcn_raw_buffer_load_b128(r, (lane + 64 * v) * 16, 0, 16);
      bool pending = false;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        if (done[v]) continue;
        const uint32_t e = (uint32_t)(lane + 64 * v);
        if (x[v][1] == ep && x[v][3] == (ep ^ e ^ 0x55u)) done[v] = true;
        else pending = true;
      }
      if (!__any(pending)) break;
      if (wall_clock64() - t0 > limit) { ok = false; break; }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  ok = __syncthreads_and(ok);
  if (t == 0) {
    st[2 * b] = t0;
    st[2 * b + 1] = ok ? wall_clock64() : 0;
  }
}

}  // namespace

extern "C" int probe_handoff(void* rec, int grid, uint32_t ep, void* st, void* stream) {
  if (grid < 1 || grid > 512) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_handoff, dim3(grid), dim3(256), 0, (hipStream_t)stream, (u32x4_t*)rec, ep,
                     (uint64_t)1000000, (uint64_t*)st);   // 10 ms bound
  return (int)hipGetLastError();
}

extern "C" int probe_stream_read(const void* p, int64_t bytes, void* sink, int grid, void* stream) {
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)p, bytes / 16, (uint32_t*)sink);
  return (int)hipGetLastError();
}

extern "C" int probe_empty(int grid, void* stream) {
  hipLaunchKernelGGL(k_empty, dim3(grid), dim3(64), 0, (hipStream_t)stream);
  return (int)hipGetLastError();
}

extern "C" int probe_spin(int us, void* stream) {
  if (us < 0) us = 0;
  if (us > 100000) us = 100000;
  hipLaunchKernelGGL(k_spin, dim3(1), dim3(64), 0, (hipStream_t)stream, (uint64_t)us * 100u);
  return (int)hipGetLastError();
}
