// fmoe_inst.hip -- instantiates the format-templated kernels for one
// (bits, group) pair, given by FMOE_BITS and FMOE_GROUP at compile time.  The
// build compiles this file once per pair, in parallel.
#include "fmoe_mfma.h"
#include "fmoe_chain.h"

#if !defined(FMOE_BITS) || !defined(FMOE_GROUP)
#error "FMOE_BITS and FMOE_GROUP must be defined"
#endif

#define FMOE_CAT2(a, b, c) a##b##_##c
#define FMOE_CAT(a, b, c) FMOE_CAT2(a, b, c)
#define FMOE_VARIANT FMOE_CAT(run_variant_, FMOE_BITS, FMOE_GROUP)

namespace fmoe {

namespace {

// Raises a matrix-core kernel's dynamic LDS limit to everything the CU has
// beside its static LDS; done on the first launch of each kernel only.
template <int G, int SB, int MODE>
hipError_t allow_all_lds() {
  static const hipError_t once = [] {
    const void* fn = reinterpret_cast<const void*>(&k_moe_mfma<G, SB, MODE>);
    hipFuncAttributes at{};
    hipError_t e = hipFuncGetAttributes(&at, fn);
    if (e != hipSuccess) return e;
    const int dyn = kLdsPerCu - (int)at.sharedSizeBytes;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
  }();
  return once;
}

template <int SB, int NS>
hipError_t run_one(const VCall& c) {
  constexpr int B = FMOE_BITS, G = FMOE_GROUP;
  switch (c.kind) {
    case VCall::GEMV: {
      const int rpi = rows_per_iter(c.K, B);
      int U = c.N / (4 * rpi * 256);
      U = U < 1 ? 1 : (U > kUMax ? kUMax : U);
      const int rwg = 4 * rpi * U;
      const int grid = (c.N + rwg - 1) / rwg;
      hipLaunchKernelGGL((k_gemv<B, G, SB, NS>), dim3(grid), dim3(kThreads), xprep_bytes(c.K),
                         c.st, c.q, c.s, c.b, c.N, c.K, c.x, c.y, U);
      break;
    }
    case VCall::GEMV_SWIGLU: {
      const int rpi = rows_per_iter(c.K, B);
      int U = c.N / (4 * rpi * 256);
      U = U < 1 ? 1 : (U > kUMax ? kUMax : U);
      const int rwg = 4 * rpi * U;
      const int grid = (c.N + rwg - 1) / rwg;
      hipLaunchKernelGGL((k_gemv_swiglu<B, G, SB, NS>), dim3(grid), dim3(kThreads),
                         xprep_bytes(c.K), c.st, c.q, c.s, c.b, c.q2, c.s2, c.b2, c.N, c.K, c.x,
                         c.y, U);
      break;
    }
    case VCall::GATEUP:
      if (c.gu->U == 2)
        hipLaunchKernelGGL((k_gateup<B, G, SB, NS, 2>), dim3(c.grid), dim3(kThreads),
                           xprep_bytes(c.gu->H), c.st, *c.gu);
      else
        hipLaunchKernelGGL((k_gateup<B, G, SB, NS, 1>), dim3(c.grid), dim3(kThreads),
                           xprep_bytes(c.gu->H), c.st, *c.gu);
      break;
    case VCall::DOWN_COMBINE: {
      const size_t lds = (size_t)c.d->nbatch * xprep_bytes(c.d->I);
      const dim3 grid(c.d->nrb), blk(kThreads);
      if (c.d->U == 2) {
        if (c.d->nbatch > 4)
          hipLaunchKernelGGL((k_down_combine<B, G, SB, NS, 2, 8>), grid, blk, lds, c.st, *c.d);
        else
          hipLaunchKernelGGL((k_down_combine<B, G, SB, NS, 2, 4>), grid, blk, lds, c.st, *c.d);
      } else {
        if (c.d->nbatch > 4)
          hipLaunchKernelGGL((k_down_combine<B, G, SB, NS, 1, 8>), grid, blk, lds, c.st, *c.d);
        else
          hipLaunchKernelGGL((k_down_combine<B, G, SB, NS, 1, 4>), grid, blk, lds, c.st, *c.d);
      }
      break;
    }
    case VCall::DOWN_SLOTS:
      if (c.d->U == 2)
        hipLaunchKernelGGL((k_down_slots<B, G, SB, NS, 2>), dim3(c.grid), dim3(kThreads),
                           xprep_bytes(c.d->I), c.st, *c.d);
      else
        hipLaunchKernelGGL((k_down_slots<B, G, SB, NS, 1>), dim3(c.grid), dim3(kThreads),
                           xprep_bytes(c.d->I), c.st, *c.d);
      break;
    case VCall::EXPERT_MFMA:
      if constexpr (B != 4) {
        return hipErrorNotSupported;
      } else {
        // More than 64 KB of dynamic LDS must be allowed per kernel first
        // (once per kernel, for all the LDS a workgroup can have).
        const size_t lds = moe_mfma_lds(c.mode, c.mf->H, c.mf->I, G, SB);
        hipError_t e = c.mode == 0 ? allow_all_lds<G, SB, 0>() : allow_all_lds<G, SB, 1>();
        if (e != hipSuccess) return e;
        if (c.mode == 0)
          hipLaunchKernelGGL((k_moe_mfma<G, SB, 0>), dim3(c.grid), dim3(kThreads), lds, c.st, *c.mf);
        else
          hipLaunchKernelGGL((k_moe_mfma<G, SB, 1>), dim3(c.grid), dim3(kThreads), lds, c.st, *c.mf);
      }
      break;
    case VCall::FUSED1: {
      if constexpr (NS > 2) {
        return hipErrorNotSupported;
      } else {
        const dim3 blk(kThreads), grid(c.grid);
        if (c.fu->E <= 512)
          hipLaunchKernelGGL((k_layer1<B, G, SB, NS, 8>), grid, blk, c.lds, c.st, *c.fu);
        else
          hipLaunchKernelGGL((k_layer1<B, G, SB, NS, 32>), grid, blk, c.lds, c.st, *c.fu);
      }
      break;
    }
    case VCall::TOK1: {
      if constexpr (NS > 2) {
        return hipErrorNotSupported;
      } else {
        const dim3 blk(kThreads), grid(c.grid);
        const Tok1Args& t = *c.t1;
        if (t.E <= 512)
          hipLaunchKernelGGL((k_layer1t<B, G, SB, NS, 8>), grid, blk, c.lds, c.st, t.x, t.Wr,
                             t.area, t.wsg, t.slabs, t);
        else
          hipLaunchKernelGGL((k_layer1t<B, G, SB, NS, 32>), grid, blk, c.lds, c.st, t.x, t.Wr,
                             t.area, t.wsg, t.slabs, t);
      }
      break;
    }
    case VCall::CHAIN1: {
      if constexpr (NS > 2) {
        return hipErrorNotSupported;
      } else {
        const dim3 blk(kThreads), grid(c.grid);
        const Tok1Args& t = *c.t1;   // E <= 512 (launch_chain1 checks it)
        hipLaunchKernelGGL((k_chain1t<B, G, SB, NS, 8>), grid, blk, c.lds, c.st, t.x, t.area, t,
                           *c.ch);
      }
      break;
    }
    case VCall::EXPERT1: {
      if constexpr (NS > 2) {
        return hipErrorNotSupported;
      } else {
        hipLaunchKernelGGL((k_expert1<B, G, SB, NS>), dim3(c.grid), dim3(kThreads), c.lds, c.st, *c.ex);
      }
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Resident workgroups of the fused kernel per CU (queried once per variant).
template <int SB, int NS, int V>
int fused_occupancy(size_t lds) {
  static int cached = -1;
  if (cached < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&k_layer1<FMOE_BITS, FMOE_GROUP, SB, NS, V>),
            kThreads, lds) != hipSuccess || n < 1)
      n = 1;
    cached = n;
  }
  return cached;
}

// Resident workgroups of the one-token layer kernel per CU (queried once per variant).
template <int SB, int NS, int V>
int tok1_occupancy(size_t lds) {
  static int cached = -1;
  if (cached < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&k_layer1t<FMOE_BITS, FMOE_GROUP, SB, NS, V>),
            kThreads, lds) != hipSuccess || n < 1)
      n = 0;
    cached = n;
  }
  return cached;
}

// Resident workgroups of the chained one-token kernel per CU.
template <int SB, int NS, int V>
int chain1_occupancy(size_t lds) {
  static int cached = -1;
  if (cached < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&k_chain1t<FMOE_BITS, FMOE_GROUP, SB, NS, V>),
            kThreads, lds) != hipSuccess || n < 1)
      n = 0;
    cached = n;
  }
  return cached;
}

// Resident workgroups of the one-launch expert kernel per CU.
template <int SB, int NS>
int expert1_occupancy(size_t lds) {
  static int cached = -1;
  if (cached < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&k_expert1<FMOE_BITS, FMOE_GROUP, SB, NS>), kThreads,
            lds) != hipSuccess || n < 1)
      n = 0;
    cached = n;
  }
  return cached;
}

}  // namespace

int FMOE_CAT(expert1_occupancy_, FMOE_BITS, FMOE_GROUP)(int sb, int ns, size_t lds) {
  if (sb == 4 && ns == 1) return expert1_occupancy<4, 1>(lds);
  if (sb == 4 && ns == 2) return expert1_occupancy<4, 2>(lds);
  if (sb == 2 && ns == 1) return expert1_occupancy<2, 1>(lds);
  if (sb == 2 && ns == 2) return expert1_occupancy<2, 2>(lds);
  return 0;
}

int FMOE_CAT(tok1_occupancy_, FMOE_BITS, FMOE_GROUP)(int sb, int ns, int E, size_t lds) {
  if (sb == 4 && ns == 1) return E <= 512 ? tok1_occupancy<4, 1, 8>(lds) : tok1_occupancy<4, 1, 32>(lds);
  if (sb == 4 && ns == 2) return E <= 512 ? tok1_occupancy<4, 2, 8>(lds) : tok1_occupancy<4, 2, 32>(lds);
  if (sb == 2 && ns == 1) return E <= 512 ? tok1_occupancy<2, 1, 8>(lds) : tok1_occupancy<2, 1, 32>(lds);
  if (sb == 2 && ns == 2) return E <= 512 ? tok1_occupancy<2, 2, 8>(lds) : tok1_occupancy<2, 2, 32>(lds);
  return 0;
}

int FMOE_CAT(chain1_occupancy_, FMOE_BITS, FMOE_GROUP)(int sb, int ns, int E, size_t lds) {
  if (E > 512) return 0;
  if (sb == 4 && ns == 1) return chain1_occupancy<4, 1, 8>(lds);
  if (sb == 4 && ns == 2) return chain1_occupancy<4, 2, 8>(lds);
  if (sb == 2 && ns == 1) return chain1_occupancy<2, 1, 8>(lds);
  if (sb == 2 && ns == 2) return chain1_occupancy<2, 2, 8>(lds);
  return 0;
}

int FMOE_CAT(fused_occupancy_, FMOE_BITS, FMOE_GROUP)(int sb, int ns, int E, size_t lds) {
  if (sb == 4 && ns == 1) return E <= 512 ? fused_occupancy<4, 1, 8>(lds) : fused_occupancy<4, 1, 32>(lds);
  if (sb == 4 && ns == 2) return E <= 512 ? fused_occupancy<4, 2, 8>(lds) : fused_occupancy<4, 2, 32>(lds);
  if (sb == 2 && ns == 1) return E <= 512 ? fused_occupancy<2, 1, 8>(lds) : fused_occupancy<2, 1, 32>(lds);
  if (sb == 2 && ns == 2) return E <= 512 ? fused_occupancy<2, 2, 8>(lds) : fused_occupancy<2, 2, 32>(lds);
  return 1;
}

hipError_t FMOE_VARIANT(const VCall& c) {
#define FMOE_SN(S, N) \
  if (c.f.sb == S && c.ns == N) return run_one<S, N>(c);
  FMOE_SN(4, 1) FMOE_SN(4, 2) FMOE_SN(4, 4) FMOE_SN(2, 1) FMOE_SN(2, 2) FMOE_SN(2, 4)
#undef FMOE_SN
  return hipErrorInvalidValue;
}

}  // namespace fmoe
