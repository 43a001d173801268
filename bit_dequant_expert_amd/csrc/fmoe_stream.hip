// fmoe_stream.hip -- host-tier expert streaming: the routed experts' slabs
// copied from pinned host memory into their HBM slots, driven by the routing
// indices on the device.
//
// [WAS] "1. SSD-Experten-Streaming mit macOS Page Cache" and [HADA] "SSD Expert
// Streaming": only the experts a layer selects are read from the slower tier,
// in parallel, and a cache keeps what was read recently.  Here the slower tier
// is pinned host memory (for expert sets larger than HBM), read by the GPU over
// its host link, and the fast tier is the layer's slab array in HBM: slot e
// holds expert e of whichever layer last fetched it, recorded in tags[e].  The
// indices never go to the host: a workgroup per (selected expert, 64 KiB piece
// of its slab) skips the piece when the slot already holds that expert for
// this tag or when an earlier entry of the list names the same expert, and
// copies it otherwise; a second launch then records the tags.
#include "fmoe_device.h"
#include "fmoe_internal.h"

namespace fmoe {

namespace {

typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));
constexpr int kStThreads = 256;
constexpr int64_t kStPiece = 64 * 1024;   // bytes per workgroup

// The expert of entry j of the fetch list: idx[j] for j < n, then the shared one.
__device__ __forceinline__ int st_expert(const FetchArgs& a, int j) {
  return j < a.n_idx ? a.idx[j] : a.shared;
}

// Whether entry j is the first entry that names its expert and the slot does
// not already hold it for this tag (workgroup-uniform).
__device__ __forceinline__ bool st_needed(const FetchArgs& a, int j, int e) {
  if (e < 0 || e >= a.n_slots) return false;   // out-of-range indices copy nothing
  if (a.tags[e] == a.tag) return false;
  for (int i = 0; i < j; ++i)
    if (st_expert(a, i) == e) return false;
  return true;
}

__global__ __launch_bounds__(kStThreads) void k_fetch(FetchArgs a) {
  const int64_t pieces = (a.slab_bytes + kStPiece - 1) / kStPiece;
  const int j = (int)(blockIdx.x / pieces);
  const int64_t pc = blockIdx.x - (int64_t)j * pieces;
  const int e = st_expert(a, j);
  if (!st_needed(a, j, e)) return;
  const int64_t off = pc * kStPiece;
  const int64_t nb = min(kStPiece, a.slab_bytes - off);   // a multiple of 16
  const u32v4* src = reinterpret_cast<const u32v4*>(a.host + (int64_t)e * a.stride + off);
  u32v4* dst = reinterpret_cast<u32v4*>(a.dev + (int64_t)e * a.stride + off);
  const int n16 = (int)(nb / 16);
  constexpr int U = 4;   // loads in flight per thread
  for (int i0 = threadIdx.x; i0 < n16; i0 += kStThreads * U) {
    u32v4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kStThreads;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kStThreads;
      if (i < n16) dst[i] = v[u];
    }
  }
  if (pc == 0 && threadIdx.x == 0 && a.n_copied) atomicAdd(a.n_copied, 1);
}

// After every piece is in: the fetched slots now hold this tag.
__global__ __launch_bounds__(kStThreads) void k_fetch_tags(FetchArgs a) {
  for (int j = threadIdx.x; j < a.n_idx + (a.shared >= 0 ? 1 : 0); j += kStThreads) {
    const int e = st_expert(a, j);
    if (e >= 0 && e < a.n_slots) a.tags[e] = a.tag;
  }
}

}  // namespace

hipError_t launch_fetch(const FetchArgs& a, hipStream_t st) {
  const int n = a.n_idx + (a.shared >= 0 ? 1 : 0);
  if (n == 0) return hipSuccess;
  const int64_t pieces = (a.slab_bytes + kStPiece - 1) / kStPiece;
  const int64_t grid = (int64_t)n * pieces;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_fetch, dim3((unsigned)grid), dim3(kStThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_fetch_tags, dim3(1), dim3(kStThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace fmoe
