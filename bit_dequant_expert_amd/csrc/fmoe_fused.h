// fmoe_fused.h -- the whole one-token MoE layer in one persistent launch.
//
// [HADA] "Deferred GPU Expert Compute" describes the engine handing combine,
// norm and residual straight to the next layer without a host round trip, and
// [WAS] "3. Handoptimierte Metal Compute-Shader" fuses each step into a
// kernel.  On MI355X the one-token layer is latency-bound (tens of MB in a few
// microseconds), so every step runs inside one launch.  Workgroups take work
// items in dependency order
//
//   router rows (fp64 logits) -> gate/up of the shared expert
//   -> gate/up of the routed experts -> down + combine + residual (+ RMSNorm)
//
// from 8 interleaved sub-queues (item i lives in sub-queue i mod 8 and each
// sub-queue hands out its items in increasing order), so the lowest unfinished
// item is always held by a running workgroup and an item only ever waits for
// lower items: no deadlock, whatever the number of resident workgroups.
//
// Hardware facts this layout answers (measured on MI355X): atomics on one
// address serialise at ~10 ns each and a hot line slows every stream that
// touches its channel, so every counter is split into 8 sub-counters plus a
// top counter, each on its own 256-byte line, and phase completion is
// broadcast through 64 flags on separate lines (each waiting workgroup polls
// its own).  Every waiting consumer recomputes the top-k from the published
// logits (same inputs, same result) instead of waiting for a published
// choice.  The last workgroup to leave resets counters and flags.
#pragma once

#include "fmoe_fused_args.h"
#include "fmoe_kernels.h"

namespace fmoe {

constexpr int kFusedMaxSlots = 6;   // active slots whose down tiles are held at once
constexpr int kFusedUG = 2;         // gate/up rows per wave per item (long rows)
constexpr int kFusedUD = 2;         // down iterations per wave per item
constexpr int kSpinLimit = 1 << 22;

// Counter block layout, in 256-byte lines (64 ints) of the workspace.
constexpr int kLine = 64;
constexpr int kQHeadLine = 0;       // 8 sub-queue heads
constexpr int kRouterSubLine = 8;   // 8 router arrive sub-counters, then the top counter
constexpr int kGuSubLine = 17;
constexpr int kDownSubLine = 26;
constexpr int kExitSubLine = 35;
constexpr int kTimeoutLine = 44;
constexpr int kRouterFlagLine = 48;   // 64 flags
constexpr int kGuFlagLine = 112;      // 64 flags

__device__ __forceinline__ int* ctr_line(int* base, int line) { return base + kLine * line; }

// Arrival number idx of n at a hierarchical counter; true for the very last.
// Each sub-counter resets itself once its last arrival is in.
__device__ __forceinline__ bool arrive(int* ctr, int sub_line, int idx, int n) {
  const int s = idx & 7;
  const int sub_total = n / 8 + ((s < n % 8) ? 1 : 0);
  const int nsub = n < 8 ? n : 8;
  int* sub = ctr_line(ctr, sub_line + s);
  if (add_agent(sub, 1) != sub_total - 1) return false;
  st_agent(sub, 0);
  int* top = ctr_line(ctr, sub_line + 8);
  if (add_agent(top, 1) != nsub - 1) return false;
  st_agent(top, 0);
  return true;
}

__device__ __forceinline__ void raise_flags(int* ctr, int flag_line) {
  for (int j = 0; j < 64; ++j) st_agent(ctr_line(ctr, flag_line + j), 1);
}

// Thread-level bounded wait on this workgroup's flag; a timeout is recorded
// in the workspace instead of hanging.
__device__ __forceinline__ void wait_flag(int* ctr, int flag_line) {
  int* f = ctr_line(ctr, flag_line + (blockIdx.x & 63));
  int spins = 0;
  while (ld_agent(f) == 0) {
    __builtin_amdgcn_s_sleep(4);
    if (++spins > kSpinLimit) {
      st_agent(ctr_line(ctr, kTimeoutLine), 1);
      break;
    }
  }
}

// ------------------------------------------------------------ wave max (u64)
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xF, true);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over the wave, returned in every lane (keys are unsigned; the DPP
// lanes outside a row mask read 0, which never wins).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp_u64<kDppXor1>(v));
  v = umax64(v, dpp_u64<kDppXor2>(v));
  v = umax64(v, dpp_u64<kDppHalfMirror>(v));
  v = umax64(v, dpp_u64<kDppMirror>(v));
  v = umax64(v, dpp_u64<kDppBcast15, 0xA>(v));
  v = umax64(v, dpp_u64<kDppBcast31, 0xC>(v));
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Per-workgroup cache of the routing decision.
struct RouteCache {
  int ready;
  int sel[16];
  float coef[17];   // routing weights, then the shared gate
};

// Wave 0: top-k over the logits staged in LDS (ties: lower index), weights =
// softmax over the selected logits, shared gate = sigmoid of logit E.
template <int VMAX>
__device__ __forceinline__ void fused_topk(const FusedArgs& a, const double* lg, RouteCache& rc) {
  const int lane = threadIdx.x & 63;
  uint64_t key[VMAX];
#pragma unroll
  for (int v = 0; v < VMAX; ++v) {
    const int e = lane * VMAX + v;
    const uint64_t kk = order_key(lg[e < a.E ? e : 0]);
    key[v] = e < a.E ? kk : 0ull;
  }
  int sel_e = 0;
  for (int r = 0; r < a.k; ++r) {
    uint64_t best = 0;
    int bv = 0;
#pragma unroll
    for (int v = 0; v < VMAX; ++v) {
      if (key[v] > best) { best = key[v]; bv = v; }
    }
    const uint64_t m = wave_max_u64(best);
    const uint64_t ball = __ballot(best == m);
    const int L = __ffsll((unsigned long long)ball) - 1;
    const int win = __builtin_amdgcn_readlane(lane * VMAX + bv, L);
#pragma unroll
    for (int v = 0; v < VMAX; ++v)
      if (lane == L && v == bv) key[v] = 0ull;
    if (lane == r) sel_e = win;
  }
  const double l = lg[lane < a.k ? sel_e : 0];
  const double l0 = lg[__builtin_amdgcn_readlane(sel_e, 0)];
  const float ex = lane < a.k ? expf((float)(l - l0)) : 0.f;
  const float z = wave_sum(ex);
  if (lane < a.k) {
    rc.sel[lane] = sel_e;
    rc.coef[lane] = ex / z;
  }
  if (lane == 0) rc.coef[a.k] = 1.f / (1.f + expf(-(float)lg[a.E]));
}

template <int BITS, int G, int SB, int NSH, int VMAX>
__global__ __launch_bounds__(kThreads) void k_layer1(FusedArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_item;
  __shared__ int s_flag;
  __shared__ float s_part[kThreads / kWave];
  __shared__ RouteCache rc;
  using TileH = Tile<BITS, G, SB, NSH>;
  using TileI = Tile<BITS, G, SB, 1>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int kp1 = a.k + 1;
  const int64_t xbH = xprep_bytes(a.H), xbI = xprep_bytes(a.I);
  // LDS: phase-1 regions [x fp32 | x prepared | logits]; the down stage reuses
  // the first two (a workgroup never returns to phase 1 after a down item).
  float* lds_x = reinterpret_cast<float*>(lds);
  uint8_t* lds_xp = lds + (int64_t)a.H * 4;
  uint8_t* lds_lg = lds_xp + xbH;
  uint8_t* lds_ap = lds;
  const int nGUs = a.I / a.gu_rows;               // gate/up items per slot
  const int n_items = a.nR + a.nGU + a.nD;
  int* ctr = a.ctr;
  const int subq = blockIdx.x & 7;
  bool have_x = false, have_xp = false;
  if (tid == 0) rc.ready = 0;

  auto ensure_routing = [&]() {
    if (rc.ready) return;  // workgroup-uniform (shared, read after a barrier)
    if (tid == 0) wait_flag(ctr, kRouterFlagLine);
    __syncthreads();
    copy_to_lds_agent(reinterpret_cast<uint64_t*>(lds_lg),
                      reinterpret_cast<const uint64_t*>(a.lg64), a.E + 1, kThreads);
    __syncthreads();
    if (wave == 0) fused_topk<VMAX>(a, reinterpret_cast<const double*>(lds_lg), rc);
    __syncthreads();
    if (tid == 0) rc.ready = 1;
    __syncthreads();
  };

  for (;;) {
    __syncthreads();
    if (tid == 0) s_item = subq + 8 * add_agent(ctr_line(ctr, kQHeadLine + subq), 1);
    __syncthreads();
    const int item = s_item;
    if (item >= n_items) break;

    if (item < a.nR) {
      // ------------------------------------------------ router rows (fp64)
      const int e = item * 4 + wave;
      const bool live = e <= a.E;
      const float* wrow = (live && e < a.E) ? a.Wr + (int64_t)e * a.H : a.wsg;
      const int nf4 = a.H / 4;
      double acc = 0.0;
      for (int c0 = 0; c0 < nf4; c0 += 16 * kWave) {
        float4 wv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int f = c0 + j * kWave + lane;
          wv[j] = (live && f < nf4) ? ld_nt(reinterpret_cast<const float4*>(wrow) + f)
                                    : make_float4(0, 0, 0, 0);
        }
        if (!have_x) {   // x staging overlaps the row loads
          copy_to_lds(reinterpret_cast<uint4*>(lds_x), reinterpret_cast<const uint4*>(a.x),
                      nf4, kThreads);
          have_x = true;
          __syncthreads();
        }
        if (live) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int f = c0 + j * kWave + lane;
            if (f < nf4) {
              const float4 xv = reinterpret_cast<const float4*>(lds_x)[f];
              acc = fma((double)wv[j].x, (double)xv.x, acc);
              acc = fma((double)wv[j].y, (double)xv.y, acc);
              acc = fma((double)wv[j].z, (double)xv.z, acc);
              acc = fma((double)wv[j].w, (double)xv.w, acc);
            }
          }
        }
      }
      acc = sum_lanes64(acc);
      if (live && lane == 0) st_agent(a.lg64 + e, acc);
      vm_drain();
      __syncthreads();
      if (tid == 0 && arrive(ctr, kRouterSubLine, item, a.nR)) raise_flags(ctr, kRouterFlagLine);
    } else if (item < a.nR + a.nGU) {
      // ------------------------------------------------ gate/up + SwiGLU
      const int g = item - a.nR;
      const int so = g / nGUs, rb = g % nGUs;
      const int slot = so == 0 ? a.k : so - 1;          // shared expert first
      if (slot < a.k) ensure_routing();
      const int64_t e = slot < a.k ? rc.sel[slot] : a.E;
      const uint8_t* base = a.src.base + e * a.src.stride;
      const RowGeo geo(a.H, BITS);
      const int n0 = rb * a.gu_rows + wave * kFusedUG;
      TileH tg[kFusedUG], tu[kFusedUG];
#pragma unroll
      for (int u = 0; u < kFusedUG; ++u) {
        tg[u].load(base + a.src.off[0], base + a.src.off[1], base + a.src.off[2], a.H, n0 + u, geo);
        tu[u].load(base + a.src.off[3], base + a.src.off[4], base + a.src.off[5], a.H, n0 + u, geo);
      }
      if (!have_xp) {
        prep_vector<BITS, kThreads, false>(a.x, lds_xp, a.H);
        have_xp = true;
        __syncthreads();
      }
      XRegs<BITS, NSH> xr;
      xr.load(lds_xp, a.H, geo);
      float* arow = a.abuf + (int64_t)slot * a.I;
#pragma unroll
      for (int u = 0; u < kFusedUG; ++u) {
        const float gs = sum_lanes(tile_dot(tg[u], xr), kWave);
        const float us = sum_lanes(tile_dot(tu[u], xr), kWave);
        if (lane == kWave - 1) st_agent(arow + n0 + u, silu(gs) * us);
      }
      vm_drain();
      __syncthreads();
      if (tid == 0 && arrive(ctr, kGuSubLine, g, a.nGU)) raise_flags(ctr, kGuFlagLine);
    } else {
      // ------------------------------------------------ down + combine
      const int d = item - a.nR - a.nGU;
      ensure_routing();
      const RowGeo geo(a.I, BITS);
      const int rpw = kFusedUD * geo.RPI;
      const int wrow0 = d * a.d_rows + wave * rpw;
      float acc[kFusedUD];
#pragma unroll
      for (int u = 0; u < kFusedUD; ++u) acc[u] = 0.f;
      for (int s0 = 0; s0 < kp1; s0 += kFusedMaxSlots) {
        const int ns = min(kFusedMaxSlots, kp1 - s0);
        TileI tl[kFusedMaxSlots][kFusedUD];
#pragma unroll
        for (int sl = 0; sl < kFusedMaxSlots; ++sl) {
          const int slot = s0 + sl;
          const int64_t e = slot < a.k ? rc.sel[slot < a.k ? slot : 0] : a.E;
          const uint8_t* base = a.src.base + e * a.src.stride;
#pragma unroll
          for (int u = 0; u < kFusedUD; ++u) {
            const int m = wrow0 + u * geo.RPI + geo.lane_row;
            if (sl < ns && m < a.H)
              tl[sl][u].load(base + a.src.off[6], base + a.src.off[7], base + a.src.off[8], a.I,
                             m, geo);
            else
              tl[sl][u].zero();
          }
        }
        if (s0 == 0 && tid == 0) wait_flag(ctr, kGuFlagLine);
        __syncthreads();
        // prepare this batch's SwiGLU outputs (written by other workgroups)
        prep_vectors<BITS, kThreads, true>(a.abuf + (int64_t)s0 * a.I, lds_ap, a.I, ns);
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < kFusedMaxSlots; ++sl) {
          if (sl < ns) {
            const float coef = rc.coef[s0 + sl];
            XRegs<BITS, 1> xr;
            xr.load(lds_ap + sl * xbI, a.I, geo);
#pragma unroll
            for (int u = 0; u < kFusedUD; ++u) {
              const float v = sum_lanes(tile_dot(tl[sl][u], xr), geo.LPR);
              acc[u] = fmaf(coef, v, acc[u]);
            }
          }
        }
      }
      float ss = 0.f;
#pragma unroll
      for (int u = 0; u < kFusedUD; ++u) {
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
        st_agent(a.partials + d, tot);
        vm_drain();
        s_flag = arrive(ctr, kDownSubLine, d, a.nD);
      }
      __syncthreads();
      if (s_flag) {
        // Last down item: RMSNorm over the whole row, routing outputs.
        float part = 0.f;
        for (int r0 = 0; r0 < a.nD; r0 += 4 * kThreads) {
          float pv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = r0 + j * kThreads + tid;
            pv[j] = ld_agent(a.partials + (r < a.nD ? r : 0));
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (r0 + j * kThreads + tid < a.nD) part += pv[j];
        }
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
        if (tid < a.k) {
          if (a.idx_out) a.idx_out[tid] = rc.sel[tid];
          if (a.w_out) a.w_out[tid] = rc.coef[tid];
        }
      }
    }
  }

  // Leave; the last workgroup out resets queue heads and flags.
  if (tid == 0) {
    vm_drain();
    if (arrive(ctr, kExitSubLine, blockIdx.x, gridDim.x)) {
      for (int s = 0; s < 8; ++s) st_agent(ctr_line(ctr, kQHeadLine + s), 0);
      for (int j = 0; j < 64; ++j) {
        st_agent(ctr_line(ctr, kRouterFlagLine + j), 0);
        st_agent(ctr_line(ctr, kGuFlagLine + j), 0);
      }
    }
  }
}

}  // namespace fmoe
