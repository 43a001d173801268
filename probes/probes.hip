// probes.hip -- measurement probes for the benchmark (not part of the layer):
//   probe_stream_read : read a buffer once with 16-byte loads (HBM ceiling)
//   probe_empty       : an empty kernel, for launch-gap measurements
//   probe_spin        : one wave that busy-waits a given number of microseconds
//                       (keeps the queue ahead of the host before a timed region)
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

}  // namespace

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
