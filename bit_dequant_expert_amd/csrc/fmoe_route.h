// fmoe_route.h -- router of the multi-launch path (any number of tokens).
//
// [WAS] "Verstaendnis von Mixture-of-Experts (MoE) ...": the router scores
// every expert for every token and keeps the k best, plus the shared expert.
// Two kernels:
//   k_route_logits  logits = Wr . x for all tokens as one fp64 matrix product
//                   on the matrix cores (v_mfma_f64_16x16x4_f64).  Every
//                   product of two fp32 values is exact in fp64, so the sums
//                   do not depend on their order beyond fp64 rounding.  A
//                   workgroup takes 16 router rows x 32 tokens over one slice
//                   of the hidden dim (its 4 waves split the slice again and
//                   add in a fixed order through LDS); partial sums per slice
//                   go to the workspace.  Extra workgroups prepare the
//                   activations of the gate/up products (GEMV form, or the
//                   matrix-core images: one wave per token) and take the
//                   shared expert's gate logit wsg . x (one wave per token).
//   k_route_select  one workgroup per token: adds the slices in a fixed
//                   order, picks the top k (larger logit first, lower index on
//                   ties), the softmax weights over the selection and the
//                   shared expert's sigmoid gate; the last workgroup groups
//                   the token slots by expert (histogram, scans, stable
//                   scatter) for the expert kernels.
#pragma once

#include "fmoe_mfma.h"    // image_row, wave_max_u32 (and the common kernels)

namespace fmoe {

// Phase stamps of the FMOE_TRACE build: one thread per workgroup writes the
// 100 MHz wall clock at its marks (the select kernel's workgroups first).
#ifdef FMOE_TRACE
#define ROUTE_MARK(base, ev, cond)                                                  \
  do {                                                                              \
    if ((cond) && a.trace) a.trace[(base) + (ev)] = wall_clock64();                 \
  } while (0)
#else
#define ROUTE_MARK(base, ev, cond) do {} while (0)
#endif

typedef double f64x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void k_route_logits(RouteArgs a) {
  __shared__ f64x4 s_red[3][2][kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrt = (a.rows + 15) / 16, ntp = (a.T + 31) / 32;
  const int nlog = nrt * ntp * a.ksplit;

  // Workgroups: T token workgroups first (their loads go out ahead of the
  // bulk), then the logit tiles, then the GEMV-form preparation.
  const int nx = (a.ximg || a.gl) ? a.T : 0;
  const int bi = (int)blockIdx.x - nx;
  if (bi < 0) {
    // ---- one workgroup per token: wave 0 writes the matrix-core image of x
    // (fp16 pairs in unpack order, one power-of-two scale); waves 1 and 2 take
    // the shared expert's gate logit wsg . x in fp64 (every product of two
    // fp32 values is exact): each lane sums its float4 chunks in order, then
    // the lanes, then the two halves in wave order.
    __shared__ double s_gh;
    const int t = (int)blockIdx.x;
    const int XB = a.T * kRouteTraceSel + nlog * kRouteTraceLog + t * 2;
    ROUTE_MARK(XB, 0, tid == 0);
    const bool gate = a.wsg && a.gl;
    double acc = 0.0;
    if (wave == 0) {
      if (a.ximg) {
        const float sc = image_row<64, kMfmaMaxH / 512>(a.x + (int64_t)t * a.H, a.H,
                                                        a.ximg + (int64_t)t * (a.H / 8), nullptr);
        if (lane == 0) a.xsc[t] = sc;
      }
    } else if (wave <= 2 && gate) {
      const float4* w4 = reinterpret_cast<const float4*>(a.wsg);
      const float4* x4 = reinterpret_cast<const float4*>(a.x + (int64_t)t * a.H);
      const int nq = a.H / 4, half = (nq + 1) / 2;
      const int q_lo = wave == 1 ? 0 : half, q_hi = wave == 1 ? half : nq;
      constexpr int kGQ = 8;   // float4 chunks a lane has in flight
      for (int q0 = q_lo + lane; q0 < q_hi; q0 += kGQ * kWave) {
        float4 wv[kGQ], xv[kGQ];
#pragma unroll
        for (int j = 0; j < kGQ; ++j) {
          const int q = q0 + j * kWave;
          wv[j] = q < q_hi ? w4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
          xv[j] = q < q_hi ? x4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < kGQ; ++j)
          acc += (double)wv[j].x * xv[j].x + (double)wv[j].y * xv[j].y +
                 (double)wv[j].z * xv[j].z + (double)wv[j].w * xv[j].w;
      }
      acc = sum_lanes64(acc);
      if (wave == 2 && lane == 0) s_gh = acc;
    }
    __syncthreads();
    if (gate && wave == 1 && lane == 0) a.gl[t] = acc + s_gh;
    ROUTE_MARK(XB, 1, tid == 0);
    return;
  }
  if (bi >= nlog) {
    // ---- activation prep for the gate/up products (independent of routing)
    if (!a.xprep) return;
    const int pb = bi - nlog;
    // The gate/up kernel's completion counters live in the workspace's data
    // region, where a call of another shape may have left data: clear them
    // here, one launch ahead of their first use.
    for (int i = pb * kThreads + tid; i < a.n_ccnt; i += a.n_prep_wgs * kThreads) a.ccnt[i] = 0;
    const int per_tok = a.H / 32;
    const int gb = pb * (kThreads / 8) + (tid >> 3);
    const bool ok = gb < a.T * per_tok;
    const int t = ok ? gb / per_tok : 0, blk = ok ? gb % per_tok : -1;
    const float* src = a.x + (int64_t)t * a.H;
    uint8_t* dst = a.xprep + (int64_t)t * xprep_bytes(a.H);
    if (a.bits == 4) prep_blocks<4, false>(src, dst, a.H, blk);
    else prep_blocks<2, false>(src, dst, a.H, blk);
    return;
  }

  const int LB = a.T * kRouteTraceSel + bi * kRouteTraceLog;
  ROUTE_MARK(LB, 0, tid == 0);
  const int ks = bi % a.ksplit;
  const int rest = bi / a.ksplit;
  const int rt = rest % nrt, tp = rest / nrt;
  // Operand lanes: lane = m + 16 g supplies row m of the A tile (router rows)
  // and column m of the B tile (tokens) at the k index of group g.
  const int m = lane & 15, g = lane >> 4;
  const int row = rt * 16 + m;
  const float* wrow = a.Wr + (int64_t)(row < a.rows ? row : 0) * a.H;
  const bool wok = row < a.rows;
  const int t0 = tp * 32 + m, t1 = t0 + 16;
  const bool ok0 = t0 < a.T, ok1 = t1 < a.T;
  const float* x0 = a.x + (int64_t)(ok0 ? t0 : 0) * a.H;
  const float* x1 = a.x + (int64_t)(ok1 ? t1 : 0) * a.H;

  // Hidden dim in blocks of 64; slice s of NS gets blocks [b0, b1).
  const int nblk = (a.H + 63) / 64, NS = a.ksplit * 4, s = ks * 4 + wave;
  const int b0 = (int)((int64_t)s * nblk / NS), b1 = (int)((int64_t)(s + 1) * nblk / NS);

  f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
  // Lane group g takes elements 16 j + 4 g .. + 3 of the block (j < 4) of its
  // row and of its tokens: each load covers 64 contiguous bytes of 16 rows.
  auto load_block = [&](int b, float4 (&wv)[4], float4 (&xa)[4], float4 (&xb)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = b * 64 + 16 * j + 4 * g;
      const bool in = kk < a.H;   // H % 4 == 0: a float4 is wholly in or out
      const int kc = in ? kk : 0;
      wv[j] = ld_nt(reinterpret_cast<const float4*>(wrow + kc));
      xa[j] = *reinterpret_cast<const float4*>(x0 + kc);
      xb[j] = *reinterpret_cast<const float4*>(x1 + kc);
      if (!(in && wok)) wv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (!(in && ok0)) xa[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (!(in && ok1)) xb[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto mul_block = [&](const float4 (&wv)[4], const float4 (&xa)[4], const float4 (&xb)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float w4[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
      const float a4[4] = {xa[j].x, xa[j].y, xa[j].z, xa[j].w};
      const float c4[4] = {xb[j].x, xb[j].y, xb[j].z, xb[j].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double wd = (double)w4[c];
        acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(wd, (double)a4[c], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(wd, (double)c4[c], acc1, 0, 0, 0);
      }
    }
  };
  // Two blocks in flight: the loads of block b+1 go out before block b's products.
  for (int b = b0; b < b1; b += 2) {
    float4 wv0[4], xa0[4], xb0[4], wv1[4], xa1[4], xb1[4];
    load_block(b, wv0, xa0, xb0);
    load_block(min(b + 1, b1 - 1), wv1, xa1, xb1);
    mul_block(wv0, xa0, xb0);
    ROUTE_MARK(LB, 1, tid == 0 && b == b0);
    if (b + 1 < b1) mul_block(wv1, xa1, xb1);
  }
  ROUTE_MARK(LB, 2, tid == 0);

  // Waves 1..3 hand their tiles to wave 0, which adds them in wave order.
  if (wave > 0) {
    s_red[wave - 1][0][lane] = acc0;
    s_red[wave - 1][1][lane] = acc1;
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    acc0 += s_red[w][0][lane];
    acc1 += s_red[w][1][lane];
  }
  // Result lane layout of the fp64 16x16 product: element r of lane
  // (m + 16 g) is row g + 4 r of the tile, token column m (unlike the fp32
  // products, whose element r is row 4 g + r).  Through LDS into
  // [token][row] order, then each token's 16 rows go out as one 128-byte run.
  double* s_t = reinterpret_cast<double*>(&s_red[0][0][0]);   // [32][16], reuses s_red
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s_t[m * 16 + g + 4 * r] = acc0[r];
    s_t[(m + 16) * 16 + g + 4 * r] = acc1[r];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  ROUTE_MARK(LB, 3, tid == 0);
  double* part = a.part + (int64_t)ks * a.T * a.rows;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int i = q * 64 + lane, tt = i >> 4, rr = rt * 16 + (i & 15), t = tp * 32 + tt;
    if (t < a.T && rr < a.rows) part[(int64_t)t * a.rows + rr] = s_t[i];
  }
}

// One workgroup per token; the last one to finish groups the slots by expert.
template <int VMAX>
__global__ __launch_bounds__(kThreads) void k_route_select(RouteArgs a) {
  extern __shared__ __align__(16) double lds_d[];
  __shared__ int s_last;
  __shared__ uint64_t s_wsum[kThreads / kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  const int SB = t * kRouteTraceSel;
  ROUTE_MARK(SB, 0, tid == 0);
  // The shared gate's logit, requested with the partial sums.
  const double glt = a.g_ws && a.gl && tid == 0 ? a.gl[t] : 0.0;

  // Logits of this token: the slices added in slice order.
  double* s_lg = lds_d;   // [rows]
  for (int e0 = 0; e0 < a.rows; e0 += 4 * kThreads) {
    // Every slice's loads first (clamped; slices past ksplit are not added),
    // then the sums in slice order.
    double pv[kRouteMaxSplit][4];
#pragma unroll
    for (int ks = 0; ks < kRouteMaxSplit; ++ks) {
      const double* p = a.part + ((int64_t)min(ks, a.ksplit - 1) * a.T + t) * a.rows;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + j * kThreads + tid;
        pv[ks][j] = p[e < a.rows ? e : 0];
      }
    }
    double v[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < kRouteMaxSplit; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = ks < a.ksplit ? v[j] + pv[ks][j] : v[j];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + j * kThreads + tid;
      if (e < a.rows) {
        s_lg[e] = v[j];
        if (a.logits_out && e < a.E) a.logits_out[(int64_t)t * a.E + e] = (float)v[j];
      }
    }
  }
  __syncthreads();
  ROUTE_MARK(SB, 1, tid == 0);

  if (wave == 0) {
    uint64_t key[VMAX];
#pragma unroll
    for (int v = 0; v < VMAX; ++v) {
      const int e = lane * VMAX + v;
      key[v] = e < a.E ? order_key(s_lg[e]) : 0ull;
    }
    int sel_e = 0;
    for (int r = 0; r < a.k; ++r) {
      uint64_t best = 0;
      int bv = -1;
#pragma unroll
      for (int v = 0; v < VMAX; ++v) {
        if (key[v] > best) { best = key[v]; bv = v; }
      }
      // Wave maximum on DPP row operations: the high halves first, the low
      // halves only among lanes that tie on them.
      const uint32_t hi = (uint32_t)(best >> 32);
      const uint32_t mh = wave_max_u32(hi);
      const uint32_t ml = wave_max_u32(hi == mh ? (uint32_t)best : 0u);
      const uint64_t mx = ((uint64_t)mh << 32) | ml;
      // Equal keys: the lowest lane holds the lowest index (indices ascend
      // with lane, then with v, and the first maximum in v order is kept).
      const uint64_t ball = __ballot(bv >= 0 && best == mx);
      const int L = ball ? __ffsll((unsigned long long)ball) - 1 : 0;
      const int win = __builtin_amdgcn_readlane(lane * VMAX + (bv < 0 ? 0 : bv), L);
#pragma unroll
      for (int v = 0; v < VMAX; ++v)
        if (lane == L && v == bv) key[v] = 0ull;
      if (lane == r) sel_e = win;
    }
    // Weights: softmax over the selected logits, in fp32 from the fp64 logits
    // (the one-token kernel's arithmetic).
    const double l = lane < a.k ? s_lg[sel_e] : 0.0;
    const double l0 = readlane_f64(l, 0);
    const float ex = lane < a.k ? expf((float)(l - l0)) : 0.f;
    const float z = wave_sum(ex);
    if (lane < a.k) {
      const float w = ex / z;
      const int64_t o = (int64_t)t * a.k + lane;
      if (a.idx_out) a.idx_out[o] = sel_e;
      if (a.w_out) a.w_out[o] = w;
      if (a.w_ws) a.w_ws[o] = w;
      if (a.sel_ws) st_agent(a.sel_ws + o, sel_e);
    }
    if (lane == 0 && a.g_ws && a.gl) a.g_ws[t] = 1.f / (1.f + expf(-(float)glt));
    // The grouping reads this wave's selections: drain its stores, then count
    // the token in.
    ROUTE_MARK(SB, 2, lane == 0);
    if (a.act) {
      vm_drain();
      if (lane == 0) s_last = (add_agent(a.counter, 1) == a.T - 1);
      ROUTE_MARK(SB, 3, lane == 0);
    }
  }
  if (!a.act) return;
  __syncthreads();
  if (!s_last) return;
  ROUTE_MARK(SB, 5, tid == 0);

  // ---- last workgroup: group token slots by expert.
  int32_t* act = a.act;
  int32_t* act_e = act + 2;
  int32_t* act_off = act_e + a.maxA;
  int32_t* act_cnt = act_off + a.maxA;
  int32_t* act_mf = act_cnt + a.maxA;
  int32_t* entries = act_mf + a.maxA;
  const int nsel = a.T * a.k;
  // LDS: per-expert token masks [E] (T <= 64), then the selections [T*k] and
  // per-expert counts, active positions and first entries [E] x 3.
  const bool masks = a.T <= 64;
  uint64_t* s_msk = reinterpret_cast<uint64_t*>(lds_d);
  int* s_sel = reinterpret_cast<int*>(s_msk + (masks ? a.E : 0));
  for (int j = tid; j < nsel; j += kThreads) s_sel[j] = ld_agent(a.sel_ws + j);
  int* s_cnt = s_sel + nsel;   // [E]
  int* s_pos = s_cnt + a.E;    // [E] rank among active experts
  int* s_off = s_pos + a.E;    // [E] first entry
  for (int e = tid; e < a.E; e += kThreads) {
    s_cnt[e] = 0;
    if (masks) s_msk[e] = 0ull;
  }
  __syncthreads();
  for (int j = tid; j < nsel; j += kThreads) {
    atomicAdd(&s_cnt[s_sel[j]], 1);
    if (masks) atomicOr(reinterpret_cast<unsigned long long*>(&s_msk[s_sel[j]]), 1ull << (j / a.k));
  }
  __syncthreads();
  ROUTE_MARK(SB, 6, tid == 0);
  // Per thread a run of experts: active ones, slots, and matrix-core ones,
  // scanned over the workgroup as one packed 64-bit value (16 | 16 | 32 bits).
  const int per = (a.E + kThreads - 1) / kThreads;
  const int e0 = tid * per, e1 = min(a.E, e0 + per);
  uint64_t pk = 0;
  for (int e = e0; e < e1; ++e)
    pk += (uint64_t)(s_cnt[e] > 0) | ((uint64_t)(s_cnt[e] >= a.mfma_thr) << 16) |
          ((uint64_t)s_cnt[e] << 32);
  uint64_t inc = pk;
  for (int d = 1; d < kWave; d <<= 1) {
    const uint64_t o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  if (lane == kWave - 1) s_wsum[wave] = inc;
  __syncthreads();
  uint64_t before = 0, total = 0;
  for (int w = 0; w < kThreads / kWave; ++w) {
    if (w < wave) before += s_wsum[w];
    total += s_wsum[w];
  }
  const uint64_t ex = before + inc - pk;
  int bf = (int)(ex & 0xFFFF), bc = (int)(ex >> 32);
  const int sh = a.T >= a.mfma_thr ? 1 : 0;
  int bm = (int)((ex >> 16) & 0xFFFF) + sh;
  const int tf = (int)(total & 0xFFFF), tm = (int)((total >> 16) & 0xFFFF);
  // The shared expert (all T tokens: the most work) takes active index 0 so
  // that the expert kernels start its workgroups first; routed experts follow
  // in expert order at 1 .. tf.  Matrix-core list: the shared expert, then the
  // routed experts at or above the threshold in expert order.
  for (int e = e0; e < e1; ++e) {
    s_pos[e] = bf + 1;
    s_off[e] = bc;
    if (s_cnt[e] > 0) {
      act_e[bf + 1] = e;
      act_off[bf + 1] = bc;
      act_cnt[bf + 1] = s_cnt[e];
      if (s_cnt[e] >= a.mfma_thr) act_mf[bm++] = bf + 1;
      ++bf;
    }
    bc += s_cnt[e];
  }
  __syncthreads();
  // Stable scatter: a slot's rank among the slots of its expert is the number
  // of earlier slots (token order, then selection order) with that expert.  A
  // token selects an expert at most once, so with the token masks that is the
  // number of earlier tokens in the expert's mask.
  const int4* s_sel4 = reinterpret_cast<const int4*>(s_sel);
  for (int j = tid; j < nsel; j += kThreads) {
    const int e = s_sel[j], tj = j / a.k;
    int rank = 0;
    if (masks) {
      rank = __popcll(s_msk[e] & ((1ull << tj) - 1ull));
    } else {
      int jj = 0;
#pragma unroll 4
      for (; jj + 4 <= j; jj += 4) {   // four slots per LDS read
        const int4 v = s_sel4[jj >> 2];
        rank += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
      }
      for (; jj < j; ++jj) rank += (s_sel[jj] == e);
    }
    entries[s_off[e] + rank] = tj * a.kp1 + (j % a.k);
  }
  for (int tt = tid; tt < a.T; tt += kThreads) entries[nsel + tt] = tt * a.kp1 + a.k;
  if (tid == 0) {
    act_e[0] = a.E;
    act_off[0] = nsel;
    act_cnt[0] = a.T;
    if (sh) act_mf[0] = 0;
    act[0] = tf + 1;
    act[1] = tm + sh;
    st_agent(a.counter, 0);
  }
  ROUTE_MARK(SB, 7, tid == 0);
}

}  // namespace fmoe
