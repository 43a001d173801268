// fmoe_fused.h -- the whole one-token MoE layer in one persistent launch.
//
// [HADA] "Deferred GPU Expert Compute" describes the engine handing combine,
// norm and residual straight to the next layer without a host round trip, and
// [WAS] "3. Handoptimierte Metal Compute-Shader" fuses each step into a
// kernel.  On MI355X the one-token layer is latency-bound (tens of MB in a few
// microseconds), so every step runs inside one launch, and the launch is laid
// out so that all expert weights are in flight as soon as the routing is known.
//
// Work items.  Workgroup b first takes item b (no atomic on the way in); items
// past the grid, if any, are handed out in order from 64 interleaved
// sub-queues.  Item f carries up to four parts:
//
//   router rows f, f + nRr, ... below E   fp64 logits, a quarter row per wave;
//                        nRr = min(grid, E), so every router row belongs to a
//                        first item; item E mod nRr also computes row E, the
//                        shared-expert gate, after the routing is published
//   shared gate/up part f   a block of the shared expert's gate and up rows
//   routed gate/up part f   the same for routed expert slot f / nGUs
//   down part f          a block of down rows of EVERY active expert,
//                        combined with the routing weights, plus the residual
//
// A gate/up part publishes its SwiGLU outputs as prepared fp16 blocks (one
// power-of-two scale per code word of the down rows), so no consumer converts
// them.  An item requests its router row and x, publishes the logits, computes
// its shared gate/up part while the routing completes, recomputes the top-k
// from the published logits (same inputs, same result in every workgroup),
// computes and publishes its routed gate/up part, arrives, and only then
// requests its down tiles, which load while the other parts finish; the item
// flag (every item arrived) releases the down parts.  A down part waits for
// the flag only when every item of the queue is held by a running workgroup:
// each gate/up part then finishes without waiting on any down part.
// Otherwise (fewer resident workgroups than items) it defers its down part to
// a list worked off once the queue is empty; the flag counts every item's
// decision, so after it the list is complete.  Each down part publishes the
// sum of squares of its rows; once all are in, every workgroup scales its own
// rows (RMSNorm).  With a queue, the last workgroup to leave resets it.
//
// Hardware facts this layout answers (measured on MI355X): atomics on one
// address serialise at ~11 ns each (far slower while HBM is saturated), so
// every phase counter is split into 64 sub-counters, each on its own 256-byte
// line, and phase completion is a done line of 64 words (one per sub-counter)
// kept in 8 copies, so that few workgroups poll each copy.  A wave's loads
// complete in issue order, so a small load the critical path needs is never
// issued behind bulk loads it does not need (the down tiles go out after the
// gate/up part is published).  A load whose data is used at once behind a
// branch costs a full memory round trip each, so every batch of loads here is
// issued on every path (clamped addresses).
#pragma once

#include "fmoe_fused_args.h"
#include "fmoe_kernels.h"

namespace fmoe {

constexpr int kFusedMaxSlots = 5;   // active experts whose down tiles are held at once
constexpr int kFusedImgPer = 4;     // 8-byte words per thread of one SwiGLU image
constexpr int kSpinLimit = 1 << 22;

// Counter block layout, in 256-byte lines (64 ints) of the workspace.  A
// phase's arrivals go to kSubs sub-counters on lines of their own (a device-
// scope atomic on one address serialises at ~11 ns, and far worse while HBM
// is saturated); the last arrival of a sub-counter resets it and stamps word
// s of the phase's done line, written in kDoneCopies copies so that each
// waiting workgroup polls one line shared with few others.  The stamp is the
// call's epoch: one more than the down-phase stamp the previous call left
// (which no workgroup of this call can change before every workgroup has read
// it), so done lines are never reset.
constexpr int kSubs = 64;
constexpr int kLine = 64;
constexpr int kDoneCopies = 8;
constexpr int kQHeadLine = 0;                          // kSubs sub-queue heads
constexpr int kStartLine = kQHeadLine + kSubs;         // kSubs started counters
constexpr int kRouterSubLine = kStartLine + kSubs;     // kSubs each
constexpr int kItemSubLine = kRouterSubLine + kSubs;
constexpr int kDownSubLine = kItemSubLine + kSubs;
constexpr int kExitSubLine = kDownSubLine + kSubs;     // kSubs subs + top
constexpr int kTimeoutLine = kExitSubLine + kSubs + 1;
constexpr int kDefHeadLine = kTimeoutLine + 1;         // deferred down parts: next one to take
constexpr int kDefTailLine = kTimeoutLine + 2;         // deferred down parts: how many
constexpr int kRouterDoneLine = kTimeoutLine + 3;      // kDoneCopies lines each
constexpr int kItemDoneLine = kRouterDoneLine + kDoneCopies;
constexpr int kDownDoneLine = kItemDoneLine + kDoneCopies;
static_assert(kDownDoneLine + kDoneCopies <= kFusedCtrLines, "counter block too small");
constexpr int kMaxDoneParts = kFusedMaxNormParts;      // down parts one workgroup may finish

// LDS of one workgroup: [x fp32 | x prepared | down-stage activation images].
inline size_t fused_lds_bytes(int H, int I, int bits) {
  return (size_t)H * 4 + (size_t)xprep_bytes(H) + (size_t)kFusedMaxSlots * wimg_bytes(I, bits);
}

__device__ __forceinline__ int* ctr_line(int* base, int line) { return base + kLine * line; }

// Arrival number idx of n at a hierarchical counter; true for the very last.
// Each sub-counter resets itself once its last arrival is in.
__device__ __forceinline__ bool arrive(int* ctr, int sub_line, int idx, int n) {
  const int s = idx % kSubs;
  const int sub_total = n / kSubs + ((s < n % kSubs) ? 1 : 0);
  const int nsub = n < kSubs ? n : kSubs;
  int* sub = ctr_line(ctr, sub_line + s);
  if (add_agent(sub, 1) != sub_total - 1) return false;
  st_agent(sub, 0);
  int* top = ctr_line(ctr, sub_line + kSubs);
  if (add_agent(top, 1) != nsub - 1) return false;
  st_agent(top, 0);
  return true;
}

// Arrival number idx of n at a phase: the last arrival of its sub-counter
// resets it and stamps the phase's done line (all copies) with ep.
__device__ __forceinline__ void arrive_done(int* ctr, int sub_line, int done_line, int idx, int n,
                                            int ep) {
  const int s = idx % kSubs;
  const int sub_total = n / kSubs + ((s < n % kSubs) ? 1 : 0);
  int* sub = ctr_line(ctr, sub_line + s);
  if (add_agent(sub, 1) != sub_total - 1) return;
  st_agent(sub, 0);
  for (int c = 0; c < kDoneCopies; ++c) st_agent(ctr_line(ctr, done_line + c) + s, ep);
}

// One whole wave: bounded wait until every sub-counter of a phase with n
// arrivals has stamped ep (lane s reads word s of this workgroup's copy).  A
// timeout is recorded in the workspace instead of hanging.
__device__ __forceinline__ void wait_done(int* ctr, int done_line, int n, int ep) {
  const int lane = tid_x() & 63, nsub = n < kSubs ? n : kSubs;
  const int* w = ctr_line(ctr, done_line + (int)(blockIdx.x % kDoneCopies)) + lane;
  for (int spins = 0;; ++spins) {
    if (__all(lane >= nsub || ld_agent(w) == ep)) break;
    if (spins > kSpinLimit) {
      st_agent(ctr_line(ctr, kTimeoutLine), 1);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}
// The same by one thread (word after word).
__device__ __forceinline__ void wait_done_thread(int* ctr, int done_line, int n, int ep) {
  const int nsub = n < kSubs ? n : kSubs;
  const int* w = ctr_line(ctr, done_line + (int)(blockIdx.x % kDoneCopies));
  for (int s = 0, spins = 0; s < nsub; ++spins) {
    if (ld_agent(w + s) == ep) {
      ++s;
      continue;
    }
    if (spins > kSpinLimit) {
      st_agent(ctr_line(ctr, kTimeoutLine), 1);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Whether every item of the queue is held by a running workgroup: every
// workgroup has started (so holds its first item, item blockIdx.x) and every
// later item (n_main - gridDim.x of them, in kSubs sub-queues) was handed out.
// One wave: lane s reads started counter s and sub-queue head s.
struct QueueView {
  int started, head;
};
__device__ __forceinline__ QueueView load_queue(int* ctr) {
  const int s = tid_x() & 63;
  return {ld_agent(ctr_line(ctr, kStartLine + s)), ld_agent(ctr_line(ctr, kQHeadLine + s))};
}
__device__ __forceinline__ bool queue_drained(QueueView q, int n_main) {
  const int s = tid_x() & 63, g = (int)gridDim.x, nd = n_main - g;
  const int want_started = g / kSubs + (s < g % kSubs ? 1 : 0);
  const int want_head = nd > 0 ? nd / kSubs + (s < nd % kSubs ? 1 : 0) : 0;
  return __ballot(q.started < want_started || q.head < want_head) == 0;
}

// ------------------------------------------------------------ wave max (u32)
// Maximum over the wave, returned in every lane, on DPP maxima.  DPP lanes
// outside a row mask read 0, which never wins (unsigned keys).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor1, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor2, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppHalfMirror, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppMirror, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppBcast15, 0xA, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppBcast31, 0xC, 0xF, true));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// The logit a key of order_key was made from.
__device__ __forceinline__ double key_value(uint64_t k) {
  const uint64_t b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)b);
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Per-workgroup cache of the routing decision.  Down slot 0 is the shared
// expert, slot 1 + i the i-th selected expert; coef follows the slots.
struct RouteCache {
  int ready;
  int sel[16];
  float coef[17];   // shared gate (set by the first down batch), then routing weights
};

// Top-k of the published logits (ties: lower index) by the whole workgroup.
// Wave w holds logits w*64*VW .. (w+1)*64*VW-1 (VW per lane, agent-scope
// loads: other workgroups wrote them) and takes its k largest in k rounds of
// a wave maximum; a round compares the high 32 bits of the keys only, unless
// several lanes share the largest high half.  Wave 0 then ranks the 4k
// candidates against each other (lane c holds candidate c and counts those
// that beat it), so the merge takes no serial rounds.  Weights = softmax over
// the selected logits.  Called by all threads, in two halves: the loads, then
// (with other loads possibly issued in between) the selection.
struct TopkCand {
  uint64_t key[64];
  int idx[64];
};
template <int VW>
__device__ __forceinline__ void topk_keys(const FusedArgs& a, double (&l)[VW]) {
  const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int v = 0; v < VW; ++v) {
    const int e = (wave * 64 + lane) * VW + v;
    l[v] = ld_agent(a.lg64 + (e < a.E ? e : a.E - 1));
  }
}
template <int VW>
__device__ __forceinline__ void topk_select(const FusedArgs& a, const double (&l)[VW],
                                            RouteCache& rc, TopkCand& tc) {
  const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
  // 1 <= k <= 16 (checked on the host); without it the compiler keeps a path
  // where the logit loads stay unconsumed and then waits for them much later.
  __builtin_assume(a.k >= 1);
  __builtin_assume(a.k <= 16);
  uint64_t key[VW];
#pragma unroll
  for (int v = 0; v < VW; ++v)
    key[v] = (wave * 64 + lane) * VW + v < a.E ? order_key(l[v]) : 0ull;
  for (int r = 0; r < a.k; ++r) {
    uint64_t best = 0;
    int bv = 0;
#pragma unroll
    for (int v = 0; v < VW; ++v) {
      if (key[v] > best) { best = key[v]; bv = v; }
    }
    const uint32_t hi = (uint32_t)(best >> 32);
    const uint32_t mh = wave_max_u32(hi);
    uint64_t ball = __ballot(hi == mh);
    if (__popcll(ball) != 1) {   // the high halves tie: full keys of those lanes
      const uint32_t ml = wave_max_u32(hi == mh ? (uint32_t)best : 0u);
      ball = __ballot(best == (((uint64_t)mh << 32) | ml));
    }
    const int L = __ffsll((unsigned long long)ball) - 1;
    const uint32_t wl = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)best, L);
    const int we = __builtin_amdgcn_readlane((wave * 64 + lane) * VW + bv, L);
#pragma unroll
    for (int v = 0; v < VW; ++v)
      if (lane == L && v == bv) key[v] = 0ull;
    if (lane == 0) {
      tc.key[wave * a.k + r] = ((uint64_t)mh << 32) | wl;
      tc.idx[wave * a.k + r] = we;
    }
  }
  // Candidates past 4k up to the next multiple of 16 lose every comparison
  // (key 0, largest index), so the ranking needs no per-candidate guard.
  {
    const int nc = 4 * a.k;
    if (wave == 0 && lane >= nc && lane < ((nc + 15) & ~15)) {
      tc.key[lane] = 0ull;
      tc.idx[lane] = 0x7FFFFFFF;
    }
  }
  lds_barrier();
  if (wave == 0) {
    const int nc = 4 * a.k;
    const bool c = lane < nc;
    const uint64_t ck = c ? tc.key[lane] : 0ull;
    const int ce = c ? tc.idx[lane] : 0x7FFFFFFF;
    // All 16 candidates of a block are read before any comparison, and the
    // comparison has no short circuit: a branch per candidate would make
    // each LDS read a round trip of its own.
    int rank = 0;
    for (int j0 = 0; j0 < nc; j0 += 16) {
      uint64_t kj[16];
      int ej[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        kj[t] = tc.key[j0 + t];
        ej[t] = tc.idx[j0 + t];
      }
#pragma unroll
      for (int t = 0; t < 16; ++t)
        rank += (int)((kj[t] > ck) | ((kj[t] == ck) & (ej[t] < ce)));
    }
    const bool sel = c && rank < a.k;
    const int L0 = __ffsll((unsigned long long)__ballot(c && rank == 0)) - 1;
    const double l = key_value(ck);
    const double l0 = readlane_f64(l, L0);
    const float ex = sel ? expf((float)(l - l0)) : 0.f;
    const float z = wave_sum(ex);
    if (sel) {
      rc.sel[rank] = ce;
      rc.coef[1 + rank] = ex / z;
    }
  }
}

// ------------------------------------------------------------ down parts
// Tiles of down rows wrow0 + u*RPI + lane_row (u < kFusedUD) of down slots
// s0 + sl for sl in [SL0, SL1) (slot 0 = the shared expert, slot 1 + i =
// selected expert i); slots past the last active one repeat it (never read).
// The launcher admits only hidden sizes that are a multiple of the part's
// rows, so every row exists.  Every load is issued on every path: the
// compiler's waits count the loads issued after the one waited for, and a
// load skipped on some path makes it wait for everything on all of them.
template <int BITS, int G, int SB, int SL0, int SL1>
__device__ __forceinline__ void down_load(Tile<BITS, G, SB, 1> (&tl)[kFusedMaxSlots][kFusedUD],
                                          const FusedArgs& a, const RouteCache& rc, int wrow0,
                                          int s0, const RowGeo& geo) {
#pragma unroll
  for (int sl = SL0; sl < SL1; ++sl) {
    const int ds = min(s0 + sl, a.k);
    const int64_t e = ds == 0 ? a.E : rc.sel[ds > 0 ? ds - 1 : 0];
    const uint8_t* base = a.src.base + e * a.src.stride;
#pragma unroll
    for (int u = 0; u < kFusedUD; ++u) {
      const int m = wrow0 + u * geo.RPI + geo.lane_row;
      tl[sl][u].load(base + a.src.off[6], base + a.src.off[7], base + a.src.off[8], a.I, m, geo);
    }
  }
}

// acc[u] += sum over the batch's down slots of coef * (down row . SwiGLU
// output).  The batch's word-blocked SwiGLU images (published by the gate/up
// parts before the item flag) are copied to LDS first (all threads); the first
// batch also takes the shared-expert gate from its logit.
template <int BITS, class TileT>
__device__ __forceinline__ void down_dot(const TileT (&tl)[kFusedMaxSlots][kFusedUD],
                                         float (&acc)[kFusedUD], const FusedArgs& a,
                                         RouteCache& rc, uint8_t* lds_ap, int s0, int ns,
                                         const RowGeo& geo) {
  const int64_t ib = wimg_bytes(a.I, BITS);
  const double gl = ld_agent(a.lg64 + a.E);
  copy_wimgs_to_lds_agent<BITS, kThreads, kFusedMaxSlots, kFusedImgPer>(
      reinterpret_cast<uint64_t*>(lds_ap),
      reinterpret_cast<const uint64_t*>(reinterpret_cast<const uint8_t*>(a.abuf) + s0 * ib), a.I,
      ns);
  if (s0 == 0 && tid_x() == 0) rc.coef[0] = 1.f / (1.f + expf(-(float)gl));
  lds_barrier();
  // Lane shares weighted by coef first, one cross-lane sum per row at the end.
  float part[kFusedUD];
#pragma unroll
  for (int u = 0; u < kFusedUD; ++u) part[u] = 0.f;
#pragma unroll
  for (int sl = 0; sl < kFusedMaxSlots; ++sl) {
    if (sl < ns) {
      const float coef = rc.coef[s0 + sl];
      XRegsW<BITS> xr;
      xr.load(lds_ap + sl * ib, a.I, geo);
#pragma unroll
      for (int u = 0; u < kFusedUD; ++u) part[u] = fmaf(coef, tile_dot_w(tl[sl][u], xr), part[u]);
    }
    __builtin_amdgcn_sched_barrier(0);   // one expert's activations in registers at a time
  }
#pragma unroll
  for (int u = 0; u < kFusedUD; ++u) acc[u] += sum_lanes(part[u], geo.LPR);
  lds_barrier();   // lds_ap is reused by the next batch
}

// The experts from s_begin on, tiles loaded here (deferred parts, and experts
// past the first kFusedMaxSlots).
template <int BITS, int G, int SB>
__device__ __forceinline__ void down_batches(float (&acc)[kFusedUD], const FusedArgs& a,
                                             RouteCache& rc, uint8_t* lds_ap, int wrow0,
                                             int s_begin, const RowGeo& geo) {
  const int kp1 = a.k + 1;
  for (int s0 = s_begin; s0 < kp1; s0 += kFusedMaxSlots) {
    const int ns = min(kFusedMaxSlots, kp1 - s0);
    Tile<BITS, G, SB, 1> tl[kFusedMaxSlots][kFusedUD];
    down_load<BITS, G, SB, 0, kFusedMaxSlots>(tl, a, rc, wrow0, s0, geo);
    down_dot<BITS>(tl, acc, a, rc, lds_ap, s0, ns, geo);
  }
}

// Residual and gamma of the part's rows.
__device__ __forceinline__ void down_vectors(const FusedArgs& a, int wrow0, int rpi, int lane_row,
                                             float (&rv)[kFusedUD], float (&gv)[kFusedUD]) {
#pragma unroll
  for (int u = 0; u < kFusedUD; ++u) {
    const int m = wrow0 + u * rpi + lane_row;
    rv[u] = a.resid[m];
    gv[u] = a.gamma[m];
  }
}

// h = residual + combined expert output for the part's rows (writer lanes),
// kept as gamma*h in hy; the part's sum of h^2 is published and the part
// arrives at the down phase.  Called by the whole workgroup.
__device__ __forceinline__ void down_publish(const FusedArgs& a, int d,
                                             const float (&acc)[kFusedUD],
                                             const float (&rv)[kFusedUD],
                                             const float (&gv)[kFusedUD], float (&hy)[kFusedUD],
                                             int wrow0, int rpi, int lane_row, bool writer,
                                             float* s_part, int ep) {
  const int tid = tid_x(), wave = tid >> 6, lane = tid & 63;
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < kFusedUD; ++u) {
    const int m = wrow0 + u * rpi + lane_row;
    const float h = rv[u] + acc[u];
    hy[u] = gv[u] * h;
    if (writer) {
      a.h_out[m] = h;
      if (a.moe_out) a.moe_out[m] = acc[u];
      ss = fmaf(h, h, ss);
    }
  }
  ss = sum_lanes(ss, kWave);
  if (lane == kWave - 1) s_part[wave] = ss;
  lds_barrier();
  if (tid == 0) {
    float tot = 0.f;
    for (int w = 0; w < kThreads / kWave; ++w) tot += s_part[w];
    st_agent(a.partials + d, tot);
    vm_drain();
    arrive_done(a.ctr, kDownSubLine, kDownDoneLine, d, a.nD, ep);
  }
}

// 1/rms of h from the nD partial sums (all published; the same order of
// additions in every workgroup).  Called by the whole workgroup.
__device__ __forceinline__ float norm_scale(const FusedArgs& a, float* s_part) {
  constexpr int J = kFusedMaxNormParts / kThreads;
  const int tid = tid_x(), wave = tid >> 6, lane = tid & 63;
  float pv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int r = j * kThreads + tid;
    pv[j] = ld_agent(a.partials + (r < a.nD ? r : a.nD - 1));
  }
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (j * kThreads + tid < a.nD) part += pv[j];
  part = sum_lanes(part, kWave);
  lds_barrier();
  if (lane == kWave - 1) s_part[wave] = part;
  lds_barrier();
  float tot = 0.f;
  for (int w = 0; w < kThreads / kWave; ++w) tot += s_part[w];
  return 1.f / sqrtf(tot / (float)a.H + a.eps);
}

// The persistent loop's body is large and its address arithmetic depends on
// nothing but the arguments and the lane, so the compiler would hoist all of it
// in front of the loop and keep it live in VGPRs across every path (well over a
// hundred registers).  Re-reading the arguments through an empty asm at the top
// of each item makes them opaque there, so that arithmetic stays inside the
// path that needs it.  (The asm moves nothing: the values live in SGPRs.)
// Pointers keep their global address space through the asm (a generic pointer
// would turn every access into a FLAT one, which may alias LDS).
template <typename T>
__device__ __forceinline__ void opaque_s(T& v) {
  asm volatile("" : "+s"(v));
}
template <typename T>
__device__ __forceinline__ void opaque_g(T*& p) {
  uint64_t v = reinterpret_cast<uint64_t>(p);
  asm volatile("" : "+s"(v));
  p = (T*)((__attribute__((address_space(1))) T*)v);
}
__device__ __forceinline__ void opaque_args(FusedArgs& a) {
  opaque_g(a.src.base);
  opaque_g(a.Wr); opaque_g(a.wsg); opaque_g(a.x); opaque_g(a.resid); opaque_g(a.gamma);
  opaque_g(a.h_out); opaque_g(a.y_out); opaque_g(a.moe_out); opaque_g(a.w_out);
  opaque_g(a.idx_out); opaque_g(a.lg64); opaque_g(a.abuf); opaque_g(a.gh);
  opaque_g(a.partials); opaque_g(a.dlist); opaque_g(a.ctr);
  opaque_s(a.H); opaque_s(a.I); opaque_s(a.E); opaque_s(a.k); opaque_s(a.eps);
  opaque_s(a.nRr); opaque_s(a.nGUs); opaque_s(a.nD); opaque_s(a.nF);
  opaque_s(a.gu_rows); opaque_s(a.d_rows);
  opaque_s(a.src.stride);
#pragma unroll
  for (int m = 0; m < 9; ++m) opaque_s(a.src.off[m]);
}

template <int BITS, int G, int SB, int NSH, int VMAX>
__global__ __launch_bounds__(kThreads) void k_layer1(FusedArgs a_in) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_item;
  __shared__ int s_defer;
  __shared__ int s_ndone;                  // down parts finished before the last one
  __shared__ int s_done[kMaxDoneParts];
  __shared__ float s_act[kWave];
  __shared__ float s_part[kThreads / kWave];
  __shared__ RouteCache rc;
  __shared__ TopkCand s_tc;
  __shared__ double s_rp[kFusedWaves];
  using TileH = Tile<BITS, G, SB, NSH>;
  using TileI = Tile<BITS, G, SB, 1>;
  constexpr int kUG = fused_ug(NSH);
  // float4 per lane of a quarter hidden row, and of x per thread: the hidden
  // size is NSH*8192/BITS (the launcher admits 64 or 128 segments per row).
  constexpr int kQ = 8 * NSH / BITS;
  const int subq = blockIdx.x % kSubs;
  bool have_x = false;                    // LDS already holds x (fp32 and prepared)
  bool drained = false;                   // wave 0: every queue item handed out
  bool first = true;                      // first item not yet taken
  bool listing = false;                   // thread 0: now taking deferred down parts
  int ndef = 0;                           // thread 0: length of the deferred list
  // The call's epoch (stamp of the done lines).  It is loaded together with
  // x on the first item (every workgroup stages x before its first arrival,
  // so before any done line of this call is stamped): a load of its own at
  // entry would be a round trip ahead of the first weight loads.
  int ep = 0;
  auto get_ep = [&]() { return ep; };
  // gamma*h of the last down part of this workgroup (writer lanes) and its index
  float hy[kFusedUD];
  int last_d = -1;
  if (tid_x() == 0) {
    rc.ready = 0;
    s_ndone = 0;
  }

  for (;;) {
    FusedArgs a = a_in;
    opaque_args(a);
    const int tid = tid_x(), lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kp1 = a.k + 1;
    float* lds_x = reinterpret_cast<float*>(lds);
    uint8_t* lds_xp = lds + (int64_t)a.H * 4;
    uint8_t* lds_ap = lds_xp + xprep_bytes(a.H);
    const int n_main = a.nF;
    const bool queued = n_main > (int)gridDim.x;   // items past the grid: queue and deferral
    int* ctr = a.ctr;

    // Next piece of work: first item blockIdx.x, then item < n_main from the
    // queue of the items past the grid; once that is empty, n_main + d for
    // deferred down part d (after the item flag, when the list is complete);
    // -1 when there is nothing left.  The first item is blockIdx.x, known to
    // every thread: nothing to drain or hand over.  Later ones: nothing of the
    // last item is still in flight; the wait says so to the compiler, which
    // otherwise assumes loads of skipped paths pending and waits for them
    // inside the phases.
    int item;
    if (first) {
      first = false;
      item = blockIdx.x;
      if (queued && tid == 0)
        __hip_atomic_fetch_add(ctr_line(ctr, kStartLine + subq), 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);   // result unused: no round trip
    } else {
      vm_drain();
      lds_barrier();
      if (tid == 0) {
        int it = -1;
        if (queued && !listing) {
          it = (int)gridDim.x + subq + kSubs * add_agent(ctr_line(ctr, kQHeadLine + subq), 1);
          if (it >= n_main) {
            listing = true;
            wait_done_thread(ctr, kItemDoneLine, n_main, get_ep());
            ndef = ld_agent(ctr_line(ctr, kDefTailLine));
          }
        }
        if (listing) {
          it = -1;
          if (ndef > 0) {
            const int j = add_agent(ctr_line(ctr, kDefHeadLine), 1);
            if (j < ndef) it = n_main + ld_agent(a.dlist + j);
          }
        }
        s_item = it;
      }
      lds_barrier();
      item = s_item;
    }
    if (item < 0) break;

    // What the item holds (all workgroup-uniform): router rows item,
    // item + nRr, ... below E (item < nRr) and, for item E mod nRr, the
    // shared-expert gate row E; shared gate/up part item; routed gate/up part
    // item (expert slot item / nGUs); down part item.
    int spart = -1, gslot = -1, gpart = 0, dpart = -1;
    const bool deferred = item >= n_main;
    const bool routes = !deferred && item < a.nRr;
    if (deferred) {
      dpart = item - n_main;
    } else {
      if (item < a.nGUs) spart = item;
      if (item < a.k * a.nGUs) { gslot = item / a.nGUs; gpart = item - gslot * a.nGUs; }
      if (item < a.nD) dpart = item;
    }
    const RowGeo geoH(a.H, BITS), geoI(a.I, BITS);

    // Gate/up part `part` of expert e: SwiGLU of its rows, published as one
    // block of word-blocked prepared image per code word of the down rows
    // (image slot = down slot: 0 shared, 1 + i selected expert i).
    auto gu_load = [&](TileH (&tg)[kUG], TileH (&tu)[kUG], int64_t e, int part) {
      const uint8_t* base = a.src.base + e * a.src.stride;
      const int n0 = part * a.gu_rows + wave * kUG;
#pragma unroll
      for (int u = 0; u < kUG; ++u) {
        tg[u].load(base + a.src.off[0], base + a.src.off[1], base + a.src.off[2], a.H, n0 + u,
                   geoH);
        tu[u].load(base + a.src.off[3], base + a.src.off[4], base + a.src.off[5], a.H, n0 + u,
                   geoH);
      }
    };
    auto gu_finish = [&](const TileH (&tg)[kUG], const TileH (&tu)[kUG], int islot, int part) {
      lds_barrier();   // prepared x visible; s_act free
      XRegs<BITS, NSH> xr;
      xr.load(lds_xp, a.H, geoH);
#pragma unroll
      for (int u = 0; u < kUG; ++u) {
        const float gs = sum_lanes(tile_dot(tg[u], xr), kWave);
        const float us = sum_lanes(tile_dot(tu[u], xr), kWave);
        if (lane == kWave - 1) s_act[wave * kUG + u] = silu(gs) * us;
      }
      lds_barrier();
      if (wave == 0) {   // the part's rows are whole code-word blocks of the image
        uint8_t* img = reinterpret_cast<uint8_t*>(a.abuf) + islot * wimg_bytes(a.I, BITS);
        const bool live = lane < a.gu_rows;
        wimg_publish<BITS>(s_act[live ? lane : 0], live, img, a.I, part * a.gu_rows + lane);
      }
    };
    // A quarter of router row e per wave (row E is the shared-expert gate).
    auto router_load = [&](float4 (&wv)[kQ], int e) {
      const float4* row = reinterpret_cast<const float4*>(e < a.E ? a.Wr + (int64_t)e * a.H : a.wsg);
      const int q0 = wave * (a.H / 16) + lane;
#pragma unroll
      for (int q = 0; q < kQ; ++q) wv[q] = ld_nt(row + q0 + q * 64);
    };
    // fp64 logit of the row in wv against x in LDS, stored by thread 0.
    auto router_dot = [&](const float4 (&wv)[kQ], int e) {
      const float4* xl = reinterpret_cast<const float4*>(lds_x) + wave * (a.H / 16) + lane;
      double racc = 0.0;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const float4 xv = xl[q * 64];
        racc = fma((double)wv[q].x, (double)xv.x, racc);
        racc = fma((double)wv[q].y, (double)xv.y, racc);
        racc = fma((double)wv[q].z, (double)xv.z, racc);
        racc = fma((double)wv[q].w, (double)xv.w, racc);
      }
      racc = sum_lanes_f64(racc);
      if (lane == kWave - 1) s_rp[wave] = racc;
      lds_barrier();
      if (tid == 0) st_agent(a.lg64 + e, ((s_rp[0] + s_rp[1]) + s_rp[2]) + s_rp[3]);
    };

    // Phases of an item, each a straight run of loads then their use (no
    // join between a load and its use, where the compiler would wait):
    //   1. x staged in LDS; router rows -> logits published, router arrival
    //   2. the shared expert's gate/up part, in the time the routing takes
    //   3. the routing (the shared expert's down tile is requested between
    //      the logits and the selection); the routed gate/up part computed and
    //      published
    //   4. arrival; the selected experts' down tiles requested; once every
    //      item has arrived, the down part from the held tiles
    TileI tl[kFusedMaxSlots][kFusedUD];
    float acc[kFusedUD], rv[kFusedUD], gv[kFusedUD];
    const int wrow0 = (dpart >= 0 ? dpart : 0) * a.d_rows + wave * (kFusedUD * geoI.RPI);
#pragma unroll
    for (int u = 0; u < kFusedUD; ++u) acc[u] = 0.f;
    if (!deferred) {
      // x is read only here, before this item arrives, and every h_out write
      // waits until every item has arrived, so h_out may alias x.
      if (routes || !have_x) {
        // x (and the epoch) first: x is staged and prepared while the
        // router rows are still streaming in.
        float4 wv[kQ];
        float4 xq[kQ];
        int ep_v = 0;
        if (!have_x) {
#pragma unroll
          for (int q = 0; q < kQ; ++q) xq[q] = reinterpret_cast<const float4*>(a.x)[q * kThreads + tid];
          ep_v = ld_agent(ctr_line(ctr, kDownDoneLine));
        }
        if (routes) router_load(wv, item);
        if (!have_x) {
#pragma unroll
          for (int q = 0; q < kQ; ++q) {
            reinterpret_cast<float4*>(lds_x)[q * kThreads + tid] = xq[q];
            prep_x4<BITS, false, true>(xq[q], lds_xp, a.H, q * (kThreads / 8) + tid / 8);
          }
          ep = __builtin_amdgcn_readfirstlane(ep_v) + 1;
          have_x = true;
          lds_barrier();
        }
        if (routes) {
          for (int e = item;;) {
            router_dot(wv, e);
            e += a.nRr;
            if (e >= a.E) break;
            router_load(wv, e);
            lds_barrier();   // s_rp is reused
          }
          if (tid == 0) {
            vm_drain();
            arrive_done(ctr, kRouterSubLine, kRouterDoneLine, item, a.nRr, get_ep());
          }
          if (item == a.E % a.nRr) {
            // The shared-expert gate is first needed by the down parts, after
            // the item flag, which this item's arrival (after this store) gates.
            router_load(wv, a.E);
            lds_barrier();   // s_rp is reused
            router_dot(wv, a.E);
          }
        }
      }
      if (spart >= 0) {
        TileH tg[kUG], tu[kUG];
        gu_load(tg, tu, a.E, spart);
        gu_finish(tg, tu, 0, spart);
      }
      // The routing: logits first, then the shared expert's down tile, so
      // that neither the selection nor the tile waits for the other.
      double lg[VMAX / 4];
      const bool route_now = !rc.ready;   // workgroup-uniform (shared, read after a barrier)
      if (route_now) {
        if (wave == 0) wait_done(ctr, kRouterDoneLine, a.nRr, get_ep());
        lds_barrier();
        topk_keys<VMAX / 4>(a, lg);
      }
      down_load<BITS, G, SB, 0, 1>(tl, a, rc, wrow0, 0, geoI);
      if (route_now) {
        topk_select<VMAX / 4>(a, lg, rc, s_tc);
        if (tid == 0) rc.ready = 1;
        lds_barrier();
        if (blockIdx.x == 0 && tid < a.k) {   // the routing outputs
          if (a.idx_out) a.idx_out[tid] = rc.sel[tid];
          if (a.w_out) a.w_out[tid] = rc.coef[1 + tid];
        }
      }
      {
        // All of this phase's loads on every path (the part clamped for items
        // without one; see down_load), so that the gate/up compute waits for
        // its own tiles only.  With a queue, the queue view rides along for
        // the decision (without one, 512 agent-scope loads per workgroup that
        // nothing needs: measured 0.6 us per layer).
        TileH tg[kUG], tu[kUG];
        gu_load(tg, tu, rc.sel[gslot >= 0 ? gslot : 0], gslot >= 0 ? gpart : 0);
        const QueueView qv = queued ? load_queue(ctr) : QueueView{0, 0};
        if (gslot >= 0) gu_finish(tg, tu, gslot + 1, gpart);
        if (wave == 0 && !drained) drained = !queued || queue_drained(qv, n_main);
      }
      // Every item arrives once, after its gate/up parts (published: wave 0
      // drains its stores) and its decision to wait for the item flag or to
      // defer its down part.
      if (wave == 0) vm_drain();
      lds_barrier();
      if (wave == 0) {
        bool defer = false;
        if (queued && dpart >= 0 && !drained) {
          drained = queue_drained(load_queue(ctr), n_main);
          defer = !drained;
        }
        if (lane == 0) {
          s_defer = defer;
          if (defer) {
            const int j = add_agent(ctr_line(ctr, kDefTailLine), 1);
            st_agent(a.dlist + j, dpart);
            vm_drain();
          }
          arrive_done(ctr, kItemSubLine, kItemDoneLine, item, n_main, get_ep());
        }
      }
      lds_barrier();
      if (dpart < 0 || s_defer) continue;
      // The selected experts' down tiles load while the other parts finish.
      down_load<BITS, G, SB, 1, kFusedMaxSlots>(tl, a, rc, wrow0, 0, geoI);
      down_vectors(a, wrow0, geoI.RPI, geoI.lane_row, rv, gv);
      if constexpr (BITS == 4) {
        // 4-bit tiles turn into fp16 pairs as soon as they arrive, before the
        // wait, so that only the dot2s remain once the images are in.
        TileDq4<G, SB> tq[kFusedMaxSlots][kFusedUD];
#pragma unroll
        for (int sl = 0; sl < kFusedMaxSlots; ++sl)
#pragma unroll
          for (int u = 0; u < kFusedUD; ++u) tq[sl][u].from(tl[sl][u]);
        if (wave == 0) wait_done(ctr, kItemDoneLine, n_main, get_ep());
        lds_barrier();
        down_dot<BITS>(tq, acc, a, rc, lds_ap, 0, min(kFusedMaxSlots, kp1), geoI);
      } else {
        if (wave == 0) wait_done(ctr, kItemDoneLine, n_main, get_ep());
        lds_barrier();
        down_dot<BITS>(tl, acc, a, rc, lds_ap, 0, min(kFusedMaxSlots, kp1), geoI);
      }
      if (kp1 > kFusedMaxSlots)
        down_batches<BITS, G, SB>(acc, a, rc, lds_ap, wrow0, kFusedMaxSlots, geoI);
    } else {
      // deferred (the item flag is up already): tiles loaded here
      down_vectors(a, wrow0, geoI.RPI, geoI.lane_row, rv, gv);
      down_batches<BITS, G, SB>(acc, a, rc, lds_ap, wrow0, 0, geoI);
    }
    // A down part before this one keeps gamma*h in gh for the norm at exit.
    if (last_d >= 0) {
      const bool writer = geoI.lane_seg == geoI.LPR - 1;
      const int w0 = last_d * a.d_rows + wave * (kFusedUD * geoI.RPI);
#pragma unroll
      for (int u = 0; u < kFusedUD; ++u)
        if (writer) a.gh[w0 + u * geoI.RPI + geoI.lane_row] = hy[u];
      if (tid == 0) s_done[s_ndone++] = last_d;
    }
    down_publish(a, dpart, acc, rv, gv, hy, wrow0, geoI.RPI, geoI.lane_row,
                 geoI.lane_seg == geoI.LPR - 1, s_part, get_ep());
    last_d = dpart;
    // Without a queue a workgroup holds one item: straight to the norm, with
    // no drain of this part's stores and no barrier ahead of the wait.
    if (!queued) break;
  }

  // RMSNorm of this workgroup's rows once every down part is in; then leave.
  // With items past the grid, the last workgroup out resets the queue.
  {
    FusedArgs a = a_in;
    opaque_args(a);
    const int tid = tid_x(), wave = tid >> 6;
    if (last_d >= 0) {   // workgroup-uniform
      const RowGeo geoI(a.I, BITS);
      const bool writer = geoI.lane_seg == geoI.LPR - 1;
      if (wave == 0) wait_done(a.ctr, kDownDoneLine, a.nD, get_ep());
      lds_barrier();
      const float inv = norm_scale(a, s_part);
      const int w0 = last_d * a.d_rows + wave * (kFusedUD * geoI.RPI);
#pragma unroll
      for (int u = 0; u < kFusedUD; ++u)
        if (writer) a.y_out[w0 + u * geoI.RPI + geoI.lane_row] = hy[u] * inv;
      for (int i = 0; i < s_ndone; ++i) {
        const int w1 = s_done[i] * a.d_rows + wave * (kFusedUD * geoI.RPI);
#pragma unroll
        for (int u = 0; u < kFusedUD; ++u) {
          const int m = w1 + u * geoI.RPI + geoI.lane_row;
          if (writer) a.y_out[m] = a.gh[m] * inv;
        }
      }
    }
    if (tid == 0 && a.nF > (int)gridDim.x) {
      int* ctr = a.ctr;
      vm_drain();
      if (arrive(ctr, kExitSubLine, blockIdx.x, gridDim.x)) {
        for (int s = 0; s < kSubs; ++s) {
          st_agent(ctr_line(ctr, kQHeadLine + s), 0);
          st_agent(ctr_line(ctr, kStartLine + s), 0);
        }
        st_agent(ctr_line(ctr, kDefHeadLine), 0);
        st_agent(ctr_line(ctr, kDefTailLine), 0);
      }
    }
  }
}

// ------------------------------------------------------------ one expert
// The single-expert FFN y = down . (silu(gate . x) * (up . x)) in one launch
// ([WAS] "3. Handoptimierte Metal Compute-Shader": gate/up with SwiGLU, then
// down).  Workgroup b: gate/up part b (rows b*gu_rows .. of gate and up, for
// b < nGU), published as a word-blocked SwiGLU image; then down part b (rows
// b*d_rows .., for b < nD), whose tiles are requested and converted before
// the wait for the image.  Every workgroup arrives once (after its gate/up
// part, if any).  The call's epoch is the stamp of the workgroup's own
// sub-counter plus one: that word cannot change in this call before this
// workgroup has arrived (another sub-counter's word can), and every call of
// this kernel uses all kSubs sub-counters (grid >= 128), so all words hold the
// last call's epoch when a call starts.  The counter lines are this kernel's
// own: its epochs never mix with the layer kernel's on a shared workspace.
// The launcher admits grids whose workgroups are all resident at once.
constexpr int kExpSubLine = kDownDoneLine + kDoneCopies;   // kSubs sub-counters
constexpr int kExpDoneLine = kExpSubLine + kSubs;          // kDoneCopies lines
static_assert(kExpDoneLine + kDoneCopies <= kFusedCtrLines, "counter block too small");

inline size_t expert1_lds_bytes(int H, int I, int bits) {
  return (size_t)xprep_bytes(H) + (size_t)wimg_bytes(I, bits);
}

template <int BITS, int G, int SB, int NSH>
__global__ __launch_bounds__(kThreads) void k_expert1(Expert1Args a) {
  extern __shared__ __align__(16) uint8_t lds[];   // [x prepared | SwiGLU image]
  __shared__ float s_act[kWave];
  using TileH = Tile<BITS, G, SB, NSH>;
  using TileI = Tile<BITS, G, SB, 1>;
  constexpr int kUG = fused_ug(NSH);
  constexpr int kQ = 8 * NSH / BITS;   // float4 of x per thread
  const int tid = tid_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x;
  const RowGeo geoH(a.H, BITS), geoI(a.I, BITS);
  uint8_t* lds_xp = lds;
  uint8_t* lds_ap = lds + xprep_bytes(a.H);
  int* ctr = a.ctr;
  int ep;
  if (b < a.nGU) {   // workgroup-uniform
    // x first (it is staged while the tiles stream in), then the tiles.
    float4 xq[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) xq[q] = reinterpret_cast<const float4*>(a.x)[q * kThreads + tid];
    TileH tg[kUG], tu[kUG];
    const int n0 = b * a.gu_rows + wave * kUG;
#pragma unroll
    for (int u = 0; u < kUG; ++u) {
      tg[u].load(a.gq, a.gs, a.gb, a.H, n0 + u, geoH);
      tu[u].load(a.uq, a.us, a.ub, a.H, n0 + u, geoH);
    }
    const int ep_v = ld_agent(ctr_line(ctr, kExpDoneLine) + b % kSubs);
#pragma unroll
    for (int q = 0; q < kQ; ++q) prep_x4<BITS, false, true>(xq[q], lds_xp, a.H, q * (kThreads / 8) + tid / 8);
    lds_barrier();
    XRegs<BITS, NSH> xr;
    xr.load(lds_xp, a.H, geoH);
#pragma unroll
    for (int u = 0; u < kUG; ++u) {
      const float gs = sum_lanes(tile_dot(tg[u], xr), kWave);
      const float us = sum_lanes(tile_dot(tu[u], xr), kWave);
      if (lane == kWave - 1) s_act[wave * kUG + u] = silu(gs) * us;
    }
    lds_barrier();
    if (wave == 0) {   // the part's rows are whole code-word blocks of the image
      const bool live = lane < a.gu_rows;
      wimg_publish<BITS>(s_act[live ? lane : 0], live, a.img, a.I, b * a.gu_rows + lane);
    }
    ep = __builtin_amdgcn_readfirstlane(ep_v) + 1;
  } else {
    ep = __builtin_amdgcn_readfirstlane(ld_agent(ctr_line(ctr, kExpDoneLine) + b % kSubs)) + 1;
  }
  // Arrival (wave 0's image stores drained first).
  if (wave == 0) vm_drain();
  lds_barrier();
  if (tid == 0) arrive_done(ctr, kExpSubLine, kExpDoneLine, b, (int)gridDim.x, ep);
  if (b >= a.nD) return;   // workgroup-uniform
  const int m = b * a.d_rows + wave * geoI.RPI + geoI.lane_row;
  TileI tl;
  tl.load(a.dq, a.ds, a.db, a.I, m, geoI);
  float v;
  auto finish = [&](const auto& t) {
    if (wave == 0) wait_done(ctr, kExpDoneLine, (int)gridDim.x, ep);
    lds_barrier();
    copy_wimgs_to_lds_agent<BITS, kThreads, 1, kFusedImgPer>(
        reinterpret_cast<uint64_t*>(lds_ap), reinterpret_cast<const uint64_t*>(a.img), a.I, 1);
    lds_barrier();
    XRegsW<BITS> xw;
    xw.load(lds_ap, a.I, geoI);
    v = sum_lanes(tile_dot_w(t, xw), geoI.LPR);
  };
  if constexpr (BITS == 4) {
    TileDq4<G, SB> tq;   // fp16 pairs before the wait: only the dot2s remain after it
    tq.from(tl);
    finish(tq);
  } else {
    finish(tl);
  }
  if (geoI.lane_seg == geoI.LPR - 1) a.y[m] = v;
}

}  // namespace fmoe
