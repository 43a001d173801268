// fmoe_kernels.h -- HIP kernels of the quantised MoE decode layer (gfx950).
//
// Page keys:
//   [WAS]  "Was ist Flash-MoE? 397B-Parameter-KI-Modelle auf einem Laptop
//          laufen lassen" (a2a-mcp.org, German, and translations)
//   [HADA] "Flash-MoE - Ein 397-Milliarden-Parameter-Modell auf einem
//          Notebook ausfuehren" (news.hada.io)
//
// Kernels, in the order a layer runs them:
//   k_route_logits, k_route_select (fmoe_route.h)   router product (fp64),
//                  top-k, softmax weights, shared gate, activation prep and
//                  the active-expert list (indices stay on the device)
//   k_gateup       gathered gate/up dequant-GEMV over the active slabs, SwiGLU
//                  epilogue; the last writer of each 32-row block prepares it
//                  as the down projection's input
//   k_down_combine (one token) gathered down dequant-GEMV over all active
//                  slabs, weighted combine + sigmoid-gated shared expert +
//                  residual in registers; last workgroup applies RMSNorm
//   k_down_slots + k_combine_norm   the same for several tokens
//   k_gemv         a single dequant-GEMV (fmoe_dequant_gemv)
#pragma once

#include <limits.h>

#include "fmoe_device.h"
#include "fmoe_internal.h"

namespace fmoe {

constexpr int kThreads = 256;
constexpr int kUMax = 4;


// =================================================================== gemv
// [WAS] "3. Handoptimierte Metal Compute-Shader": a tiled 4-bit / 2-bit
// matrix-vector product with cached inputs and a SIMD reduction.  Here: the
// workgroup prepares x once in LDS, each lane keeps its slice of it in
// registers, rows stream through 16-byte loads and wave shuffles reduce.
template <int BITS, int G, int SB, int NS>
__global__ __launch_bounds__(kThreads) void k_gemv(const uint8_t* __restrict__ q,
                                                   const uint8_t* __restrict__ s,
                                                   const uint8_t* __restrict__ b, int N, int K,
                                                   const float* __restrict__ x,
                                                   float* __restrict__ y, int U) {
  extern __shared__ __align__(16) uint8_t lds[];
  using TileT = Tile<BITS, G, SB, NS>;
  const RowGeo geo(K, BITS);
  const int wave = threadIdx.x >> 6;
  const int rpw = U * geo.RPI;
  int64_t n = ((int64_t)blockIdx.x * 4 + wave) * rpw + geo.lane_row;

  TileT cur;
  if (n < N) cur.load(q, s, b, K, n, geo); else cur.zero();

  prep_vector<BITS, kThreads>(x, lds, K);
  __syncthreads();
  XRegs<BITS, NS> xr;
  xr.load(lds, K, geo);

  for (int it = 0; it < U; ++it) {
    TileT nxt;
    const bool more = it + 1 < U;
    const int64_t nn = n + geo.RPI;
    if (more) {
      if (nn < N) nxt.load(q, s, b, K, nn, geo); else nxt.zero();
    }
    const float v = sum_lanes(tile_dot(cur, xr), geo.LPR);
    if (n < N && geo.lane_seg == geo.LPR - 1) y[n] = v;
    if (more) { cur = nxt; n = nn; }
  }
}

// Gate and up of one expert against one vector, SwiGLU applied: the same
// structure as k_gemv with a pair of tiles per row ([WAS] "3. Handoptimierte
// Metal Compute-Shader": dequant matrix-vector products with the SwiGLU
// activation fused).
template <int BITS, int G, int SB, int NS>
__global__ __launch_bounds__(kThreads) void k_gemv_swiglu(
    const uint8_t* __restrict__ gq, const uint8_t* __restrict__ gs, const uint8_t* __restrict__ gb,
    const uint8_t* __restrict__ uq, const uint8_t* __restrict__ us, const uint8_t* __restrict__ ub,
    int N, int K, const float* __restrict__ x, float* __restrict__ y, int U) {
  extern __shared__ __align__(16) uint8_t lds[];
  using TileT = Tile<BITS, G, SB, NS>;
  const RowGeo geo(K, BITS);
  const int wave = threadIdx.x >> 6;
  const int rpw = U * geo.RPI;
  int64_t n = ((int64_t)blockIdx.x * 4 + wave) * rpw + geo.lane_row;

  TileT cg, cu;
  if (n < N) { cg.load(gq, gs, gb, K, n, geo); cu.load(uq, us, ub, K, n, geo); }
  else { cg.zero(); cu.zero(); }

  prep_vector<BITS, kThreads>(x, lds, K);
  __syncthreads();
  XRegs<BITS, NS> xr;
  xr.load(lds, K, geo);

  for (int it = 0; it < U; ++it) {
    TileT ng, nu;
    const bool more = it + 1 < U;
    const int64_t nn = n + geo.RPI;
    if (more) {
      if (nn < N) { ng.load(gq, gs, gb, K, nn, geo); nu.load(uq, us, ub, K, nn, geo); }
      else { ng.zero(); nu.zero(); }
    }
    const float g = sum_lanes(tile_dot(cg, xr), geo.LPR);
    const float u = sum_lanes(tile_dot(cu, xr), geo.LPR);
    if (n < N && geo.lane_seg == geo.LPR - 1) y[n] = silu(g) * u;
    if (more) { cg = ng; cu = nu; n = nn; }
  }
}

// ================================================================== route
__device__ __forceinline__ uint64_t order_key(double v) {
  // Monotone map of fp64 to uint64 (larger value -> larger key).
  const uint64_t b = __double_as_longlong(v);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ uint64_t max_lanes_u64(uint64_t v) {
  for (int d = 1; d < kWave; d <<= 1) {
    const uint64_t o = __shfl_xor(v, d);
    v = o > v ? o : v;
  }
  return v;
}

// Exclusive scan of per-thread values over the workgroup (256 threads).
__device__ __forceinline__ int block_exscan(int v, int* scratch, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
  for (int w = 0; w < kThreads / kWave; ++w) {
    if (w < wave) before += scratch[w];
    total += scratch[w];
  }
  __syncthreads();
  return before + inc - v;
}

// ================================================================ gate/up
// [WAS] "3. Handoptimierte Metal Compute-Shader": dequant matrix-vector
// products with the SwiGLU activation fused.  One launch covers every active
// expert: workgroup (a, rb) reads rows rb*RWG.. of gate and up of active
// expert a and applies them to every token routed there.
template <int BITS, int G, int SB, int NS, int UT>
__global__ __launch_bounds__(kThreads) void k_gateup(GUArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_flag[2];
  using TileT = Tile<BITS, G, SB, NS>;
  const ActView av{a.act, a.maxA};
  const int ai = blockIdx.x / a.nrb, rb = blockIdx.x % a.nrb;
  if (ai >= av.base[0]) return;
  const int cnt = av.cnt()[ai];
  if (cnt >= a.mfma_thr) return;
  const int64_t e = av.e()[ai];
  const int eoff = av.off()[ai];
  const uint8_t* base = a.src.base + e * a.src.stride;
  const uint8_t *gq = base + a.src.off[0], *gs = base + a.src.off[1], *gb = base + a.src.off[2];
  const uint8_t *uq = base + a.src.off[3], *us = base + a.src.off[4], *ub = base + a.src.off[5];

  const RowGeo geo(a.H, BITS);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rpw = UT * geo.RPI, RWG = 4 * rpw;
  const int n0 = rb * RWG, wrow0 = n0 + wave * rpw;
  const int64_t xb = xprep_bytes(a.H), ab = xprep_bytes(a.I);
  const int nchunk = a.I / 32;

  TileT tg[UT], tu[UT];
#pragma unroll
  for (int u = 0; u < UT; ++u) {
    const int n = wrow0 + u * geo.RPI + geo.lane_row;
    if (n < a.I) {
      tg[u].load(gq, gs, gb, a.H, n, geo);
      tu[u].load(uq, us, ub, a.H, n, geo);
    } else {
      tg[u].zero();
      tu[u].zero();
    }
  }

  for (int jt = 0; jt < cnt; ++jt) {
    const int p = av.entries()[eoff + jt];
    const int t = p / a.kp1;
    if (jt > 0) __syncthreads();
    copy_image_to_lds<BITS, QF<BITS>::CPS>(reinterpret_cast<uint4*>(lds),
                                            reinterpret_cast<const uint4*>(a.xprep + (int64_t)t * xb),
                                            a.H, kThreads);
    __syncthreads();
    XRegs<BITS, NS> xr;
    xr.load(lds, a.H, geo);
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      {
        const float gsum = sum_lanes(tile_dot(tg[u], xr), geo.LPR);
        const float usum = sum_lanes(tile_dot(tu[u], xr), geo.LPR);
        const int n = wrow0 + u * geo.RPI + geo.lane_row;
        if (n < a.I && geo.lane_seg == geo.LPR - 1)
          st_agent(a.abuf + (int64_t)p * a.I + n, silu(gsum) * usum);
      }
    }
    vm_drain();
    __syncthreads();
    if (tid == 0) {
      const int rows_in = RWG < 32 ? RWG : 32;
      s_flag[0] = -1;
      s_flag[1] = -1;
      const int nend = min(n0 + RWG, a.I);
      for (int c = n0 / 32, qi = 0; c * 32 < nend && qi < 2; ++c, ++qi) {
        const int old = add_agent(a.ccnt + (int64_t)p * nchunk + c, rows_in);
        s_flag[qi] = (old + rows_in == 32) ? c : -1;
      }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int qi = 0; qi < 2; ++qi) {
        const int c = s_flag[qi];
        if (c >= 0) {
          prep_blocks<BITS, true>(a.abuf + (int64_t)p * a.I, a.aprep + (int64_t)p * ab, a.I,
                                  lane < 8 ? c : -1);
          if (lane == 0) st_agent(a.ccnt + (int64_t)p * nchunk + c, 0);
        }
      }
    }
  }
}

// ======================================================== down + combine
// One token.  [WAS] "3. Handoptimierte Metal Compute-Shader": MoE combine,
// residual and sigmoid gating in one pass, and a two-phase RMSNorm (sum of
// squares, then apply); [HADA] "Deferred GPU Expert Compute": the result goes
// straight on to the next layer.  Workgroup rb owns output rows rb*RWG..; it
// reads those rows of the down matrix of every active expert (a gather over
// the slabs), combines them with the routing weights and the shared gate,
// adds the residual, and the last workgroup to finish normalises.
template <int BITS, int G, int SB, int NS, int UT, int MAXS>
__global__ __launch_bounds__(kThreads) void k_down_combine(DArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float s_part[kThreads / kWave];
  __shared__ int s_last;
  using TileT = Tile<BITS, G, SB, NS>;
  const ActView av{a.act, a.maxA};
  const RowGeo geo(a.I, BITS);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rpw = UT * geo.RPI, RWG = 4 * rpw;
  const int m0 = blockIdx.x * RWG, wrow0 = m0 + wave * rpw;
  const int64_t ab = xprep_bytes(a.I);
  const int nact = av.base[0];

  float acc[UT];
#pragma unroll
  for (int u = 0; u < UT; ++u) acc[u] = 0.f;

  for (int s0 = 0; s0 < nact; s0 += a.nbatch) {
    const int ns = min(a.nbatch, nact - s0);
    TileT tl[MAXS][UT];
#pragma unroll
    for (int sl = 0; sl < MAXS; ++sl) {
      const uint8_t* base = nullptr;
      if (sl < ns) base = a.src.base + (int64_t)av.e()[s0 + sl] * a.src.stride;
#pragma unroll
      for (int u = 0; u < UT; ++u) {
        const int m = wrow0 + u * geo.RPI + geo.lane_row;
        if (sl < ns && m < a.H)
          tl[sl][u].load(base + a.src.off[6], base + a.src.off[7], base + a.src.off[8], a.I, m,
                         geo);
        else
          tl[sl][u].zero();
      }
    }
    if (s0 > 0) __syncthreads();
    for (int sl = 0; sl < ns; ++sl) {
      const int p = av.entries()[av.off()[s0 + sl]];
      copy_image_to_lds<BITS, QF<BITS>::CPS>(reinterpret_cast<uint4*>(lds + sl * ab),
                                              reinterpret_cast<const uint4*>(a.aprep + (int64_t)p * ab),
                                              a.I, kThreads);
    }
    __syncthreads();
#pragma unroll
    for (int sl = 0; sl < MAXS; ++sl) {
      if (sl < ns) {
        const int p = av.entries()[av.off()[s0 + sl]];
        const int t = p / a.kp1, i = p % a.kp1;
        const float coef = i < a.k ? a.w_ws[(int64_t)t * a.k + i] : a.g_ws[t];
        XRegs<BITS, NS> xr;
        xr.load(lds + sl * ab, a.I, geo);
#pragma unroll
        for (int u = 0; u < UT; ++u) {
          {
            const float v = sum_lanes(tile_dot(tl[sl][u], xr), geo.LPR);
            acc[u] = fmaf(coef, v, acc[u]);
          }
        }
      }
    }
  }

  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < UT; ++u) {
    const int m = wrow0 + u * geo.RPI + geo.lane_row;
    if (m < a.H && geo.lane_seg == geo.LPR - 1) {
      const float h = a.resid[m] + acc[u];
      st_agent(a.h_out + m, h);
      if (a.moe_out) a.moe_out[m] = acc[u];
      ss = fmaf(h, h, ss);
    }
  }
  ss = sum_lanes(ss, kWave);
  if (lane == kWave - 1) s_part[wave] = ss;
  vm_drain();
  __syncthreads();
  if (tid == 0) {
    float tot = 0.f;
    for (int w = 0; w < kThreads / kWave; ++w) tot += s_part[w];
    st_agent(a.partials + blockIdx.x, tot);
    vm_drain();
    s_last = (add_agent(a.ncnt, 1) == (int)gridDim.x - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // Last workgroup: total sum of squares in a fixed order, then apply.
  float part = 0.f;
  for (int r = tid; r < (int)gridDim.x; r += kThreads) part += ld_agent(a.partials + r);
  part = sum_lanes(part, kWave);
  if (lane == kWave - 1) s_part[wave] = part;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < kThreads / kWave; ++w) tot += s_part[w];
  const float inv = 1.f / sqrtf(tot / (float)a.H + a.eps);
  for (int m0 = 0; m0 < a.H; m0 += 8 * kThreads) {
    float hv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {   // all loads first (clamped addresses)
      const int m = m0 + j * kThreads + tid;
      hv[j] = ld_agent(a.h_out + (m < a.H ? m : 0));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = m0 + j * kThreads + tid;
      if (m < a.H) a.y_out[m] = a.gamma[m] * hv[j] * inv;
    }
  }
  if (tid == 0) st_agent(a.ncnt, 0);
}

// ============================================================ down, slots
// Several tokens: workgroup (a, rb) reads rows rb*RWG.. of active expert a's
// down matrix once and applies them to each token routed there, writing one
// output row block per (token, slot) entry.
template <int BITS, int G, int SB, int NS, int UT>
__global__ __launch_bounds__(kThreads) void k_down_slots(DArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  using TileT = Tile<BITS, G, SB, NS>;
  const ActView av{a.act, a.maxA};
  const int ai = blockIdx.x / a.nrb, rb = blockIdx.x % a.nrb;
  if (ai >= av.base[0]) return;
  const int cnt = av.cnt()[ai];
  if (cnt >= a.mfma_thr) return;
  const uint8_t* base = a.src.base + (int64_t)av.e()[ai] * a.src.stride;
  const int eoff = av.off()[ai];
  const RowGeo geo(a.I, BITS);
  const int tid = threadIdx.x, wave = tid >> 6;
  const int rpw = UT * geo.RPI, RWG = 4 * rpw;
  const int wrow0 = rb * RWG + wave * rpw;
  const int64_t ab = xprep_bytes(a.I);

  TileT tl[UT];
#pragma unroll
  for (int u = 0; u < UT; ++u) {
    const int m = wrow0 + u * geo.RPI + geo.lane_row;
    if (m < a.H)
      tl[u].load(base + a.src.off[6], base + a.src.off[7], base + a.src.off[8], a.I, m, geo);
    else
      tl[u].zero();
  }
  for (int jt = 0; jt < cnt; ++jt) {
    const int p = av.entries()[eoff + jt];
    if (jt > 0) __syncthreads();
    copy_image_to_lds<BITS, QF<BITS>::CPS>(reinterpret_cast<uint4*>(lds),
                                            reinterpret_cast<const uint4*>(a.aprep + (int64_t)p * ab),
                                            a.I, kThreads);
    __syncthreads();
    XRegs<BITS, NS> xr;
    xr.load(lds, a.I, geo);
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      {
        const float v = sum_lanes(tile_dot(tl[u], xr), geo.LPR);
        const int m = wrow0 + u * geo.RPI + geo.lane_row;
        if (m < a.H && geo.lane_seg == geo.LPR - 1) a.yslot[(int64_t)p * a.H + m] = v;
      }
    }
  }
}

}  // namespace fmoe
