// fmoe_chain.h -- batch-1 decode through a chain of MoE layers in one launch.
//
// [HADA] "Deferred GPU Expert Compute": the combine, norm and residual of a
// layer go straight into the next layer with no host round trip.  Here the
// whole chain is one persistent launch of the one-token layer (fmoe_tok1.h):
// each workgroup runs layer after layer, and the hand-off between layers is
// the last hand-off of a layer.  Every down part publishes its d_rows values of
// h and their sum of squares, three words a record; every workgroup polls all
// of them (it needs every sum anyway for the norm), so when the norm is known
// it holds the whole of h and builds the next layer's input
// x_{l+1} = gamma_l * h_l / rms(h_l) in its own LDS.  What a launch per layer
// costs -- the launch gap, the workgroups' start, loading x and writing y
// before the next layer reads it -- is gone; the next layer's residual h_l
// stays in the registers of the waves that computed it (each workgroup keeps
// the same down part in every layer).  The sums of squares are added in the
// one-token kernel's order and x_{l+1} is computed as y_l is, so a chain gives
// the same bits as one one-token launch per layer.
//
// Records of layer l live in record area l mod 2 with epoch base + 1 + l.  A
// workgroup writes layer l + 2's records into area l mod 2 only after it has
// polled every part record of layer l + 1, which every workgroup publishes
// after finishing layer l: no workgroup still reads area l mod 2 for layer l.
// (Each record position is written by the same wave in every layer, so two
// layers' stores to one position land in program order.)  This needs every
// workgroup to own a down part (grid = down parts); the launcher checks it.
#pragma once

#include "fmoe_tok1.h"

namespace fmoe {

// Phase trace of the FMOE_TRACE build: the second layer of a chain (the first
// of a chain of one) stamps the wall clock at these marks, kTok1TraceEvents
// per workgroup.
#ifdef FMOE_TRACE
#define CHAIN_MARK(ev, w)                                                                 \
  do {                                                                                    \
    if (l == (ch.n > 1 ? 1 : 0) && tid_x() == 64 * (w) && a.trace)                        \
      a.trace[blockIdx.x * kTok1TraceEvents + (ev)] = wall_clock64();                     \
  } while (0)
#else
#define CHAIN_MARK(ev, w) do {} while (0)
#endif

template <int BITS, int G, int SB, int NSH, int VW>
__global__ __launch_bounds__(kThreads, 2) void k_chain1t(const float* __restrict__ x_in,
                                                         uint8_t* area_in, Tok1Args a,
                                                         Tok1Chain ch) {
  a.x = x_in;
  a.area = area_in;
  // LDS: [x fp32 | x prepared | images]; the x area also stages the shared
  // SwiGLU values (phase C) and then collects h (phase D).
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ Tok1Shared sh;
  __shared__ float s_hrow[16];   // the part's values of h (d_rows <= 16)
  using TileH = Tile<BITS, G, SB, NSH>;
  using TileI = Tile<BITS, G, SB, 1>;
  constexpr int kUG = fused_ug(NSH);
  constexpr int kQ = 8 * NSH / BITS;
  constexpr int W = 32 / BITS;
  constexpr int kUD = 2;
  // Lane-dependent values are taken from tid_x() inside each layer (it sits
  // behind an empty asm), so that none of them stays live across the layer
  // loop in the role that does not use it.
  const int wave = __builtin_amdgcn_readfirstlane(tid_x() >> 6);
  const bool holder = wave >= 2, writer_wave = wave == 3;
  const int b = blockIdx.x, nwg = gridDim.x;
  const int H = a.H, I = a.I, E = a.E, k = a.k, kp1 = k + 1;
  // records per down part: words 0 .. d_rows-1 carry h, word d_rows the sum of squares
  const int dr = a.d_rows, R = (dr + 3) / 3;
  float* lds_x = reinterpret_cast<float*>(lds);
  uint8_t* lds_xp = lds + (int64_t)H * 4;
  uint8_t* lds_ap = lds_xp + xprep_bytes(H);
  const int64_t ib = wimg_bytes(I, BITS);
  int* epoch_word = reinterpret_cast<int*>(a.area);
  if (tid_x() == 0) sh.fail = 0;
  const int ep_raw = ld_agent(epoch_word);
  const uint32_t ep_base = (uint32_t)__builtin_amdgcn_readfirstlane(ep_raw);

  // Rows of this workgroup's down part (the same in every layer), held by
  // waves 2-3: rows b*d_rows + (w-2)*kUD*RPI + u*RPI + lane_row.
  auto down_rows = [&](int (&drow)[kUD], const RowGeo& geoI) {
#pragma unroll
    for (int u = 0; u < kUD; ++u)
      drow[u] = b * dr + (holder ? wave - 2 : 0) * kUD * geoI.RPI + u * geoI.RPI + geoI.lane_row;
  };
  float rv[kUD];   // the residual of the next layer, in the holders
  // layer 0's input and residual from memory; later layers' x is built in LDS
  {
    const int tid = tid_x();
    int drow[kUD];
    down_rows(drow, RowGeo(I, BITS));
#pragma unroll
    for (int u = 0; u < kUD; ++u) rv[u] = a.resid[drow[u]];
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      reinterpret_cast<float4*>(lds_x)[q * kThreads + tid] =
          reinterpret_cast<const float4*>(a.x)[q * kThreads + tid];
  }
  lds_barrier();

  // The first loads of a layer's phase A (router row b, the shared-gate value
  // of this thread, and in wave 3 the shared row pair b) do not depend on x:
  // they are issued
  // for layer 0 here and for layer l + 1 at the start of layer l's phase D,
  // so that they are in flight while the last hand-off of layer l completes.
  // (The last layer issues its own loads again: a load issued on every path
  // keeps the registers of the earlier one dead through phases B-C.)
  const int n_sp = I / 2;
  float4 wv[kQ];
  TileH ts[2][2];   // wave 3: the shared expert's [row 2 sp + r][gate, up]
  float wsg_v;
  auto first_loads = [&](const Tok1ChainLayer& Ln) {
    const int tid = tid_x(), lane = tid & 63;
    const RowGeo geoH(H, BITS);
    const int e = min(b, E - 1);
    const float4* row = reinterpret_cast<const float4*>(Ln.Wr + (int64_t)e * H);
    const int q0 = wave * (H / 16) + lane;
#pragma unroll
    for (int q = 0; q < kQ; ++q) wv[q] = ld_nt(row + q0 + q * 64);
    wsg_v = Ln.wsg[min((int)((int64_t)e * H / E) + tid, H - 1)];
    if (writer_wave) {
      const uint8_t* base = Ln.slabs + (int64_t)E * a.stride;
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int m = 0; m < 2; ++m)
          ts[r][m].load(base + a.off[3 * m], base + a.off[3 * m + 1], base + a.off[3 * m + 2], H,
                        2 * min(b, n_sp - 1) + r, geoH);
    }
  };
  first_loads(ch.layer[0]);

  for (int l = 0; l < ch.n; ++l) {
    const Tok1ChainLayer L = ch.layer[l];
    const int tid = tid_x(), lane = tid & 63;
    const RowGeo geoH(H, BITS), geoI(I, BITS);
    int drow[kUD];
    down_rows(drow, geoI);
    uint8_t* area = a.area + (size_t)(l & 1) * kTok1AreaBytes;
    const rsrc_t rlog = rec_rsrc(area + kTok1LogitOff, (uint32_t)(16 * E));
    const rsrc_t rsh = rec_rsrc(area + kTok1SharedOff, (uint32_t)(16 * (I / 2)));
    const rsrc_t rpart = rec_rsrc(area + kTok1PartOff, (uint32_t)(16 * R * a.nD));
    const rsrc_t rimg = rec_rsrc(area + kTok1ImgOff, (uint32_t)(kp1 * (I / W) * ImgBlk<BITS>::BYTES));
    uint32_t ep = (ep_base + 1u + (uint32_t)l) & 0x7FFFFFFFu;
    if (ep == 0) ep = 1;

    // ------------------------------------------------------------ phase A
    auto router_load = [&](float4 (&wv)[kQ], int e) {
      const float4* row = reinterpret_cast<const float4*>(L.Wr + (int64_t)e * H);
      const int q0 = wave * (H / 16) + lane;
#pragma unroll
      for (int q = 0; q < kQ; ++q) wv[q] = ld_nt(row + q0 + q * 64);
    };
    auto gate_slice = [&](int e, int& lo, int& hi) {
      lo = (int)((int64_t)e * H / E);
      hi = (int)((int64_t)(e + 1) * H / E);
    };
    CHAIN_MARK(0, 0);   // layer start
    auto shared_load = [&](int sp) {
      const uint8_t* base = L.slabs + (int64_t)E * a.stride;
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int m = 0; m < 2; ++m)
          ts[r][m].load(base + a.off[3 * m], base + a.off[3 * m + 1], base + a.off[3 * m + 2], H,
                        2 * sp + r, geoH);
    };
    auto down_tile = [&](TileI& t, int64_t e, int u) {
      const uint8_t* base = L.slabs + e * a.stride;
      t.load(base + a.off[6], base + a.off[7], base + a.off[8], I, drow[u], geoI);
    };
    TileI td[kFusedMaxSlots][kUD];

    // x is in lds_x (staged above, or built at the end of the last layer)
    for (int e = b; e < E; e += nwg) {
      const float4* xl = reinterpret_cast<const float4*>(lds_x) + wave * (H / 16) + lane;
      double racc = 0.0;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const float4 xv = xl[q * 64];
        racc = fma((double)wv[q].x, (double)xv.x, racc);
        racc = fma((double)wv[q].y, (double)xv.y, racc);
        racc = fma((double)wv[q].z, (double)xv.z, racc);
        racc = fma((double)wv[q].w, (double)xv.w, racc);
      }
      int lo, hi;
      gate_slice(e, lo, hi);
      double gacc = 0.0;
      if (e == b) {
        if (lo + tid < hi) gacc = (double)wsg_v * (double)lds_x[lo + tid];
        for (int j = lo + kThreads + tid; j < hi; j += kThreads)
          gacc = fma((double)L.wsg[j], (double)lds_x[j], gacc);
      } else {
        for (int j = lo + tid; j < hi; j += kThreads) gacc = fma((double)L.wsg[j], (double)lds_x[j], gacc);
      }
      if (e + nwg < E) router_load(wv, e + nwg);
      racc = sum_lanes_f64(racc);
      gacc = sum_lanes_f64(gacc);
      if (lane == kWave - 1) {
        sh.rp[wave] = racc;
        sh.gp[wave] = gacc;
      }
      lds_barrier();
      if (writer_wave && lane == 0) {
        const double lg = ((sh.rp[0] + sh.rp[1]) + sh.rp[2]) + sh.rp[3];
        const float gsl = (float)(((sh.gp[0] + sh.gp[1]) + sh.gp[2]) + sh.gp[3]);
        const uint64_t bits = (uint64_t)__double_as_longlong(lg);
        const uint32_t w0 = (uint32_t)bits, w1 = (uint32_t)(bits >> 32), w2 = __float_as_uint(gsl);
        rec_st(rlog, (uint32_t)(16 * e),
               u32x4_t{w0, w1, w2, rec_check(ep, w0, w1, w2, pos_salt(kSaltLogit, e))});
      }
      lds_barrier();
    }
    CHAIN_MARK(1, 3);   // logits stored

    // x prepared as fp16 pairs for the gate/up rows
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      prep_x4<BITS, false, true>(reinterpret_cast<const float4*>(lds_x)[q * kThreads + tid], lds_xp,
                                 H, q * (kThreads / 8) + tid / 8);
    lds_barrier();

    // ------------------------------------------------------------ phase B
    // wave 0: the top-k; wave 3 meanwhile: the shared expert's SwiGLU values
    XRegs<BITS, NSH> xr;
    if (wave == 0) {
      const bool ok = topk_wave<VW>(rlog, E, k, ep, a.spin_ticks, sh);
      if (!ok && lane == 0) sh.fail = 1;
    } else if (writer_wave) {
      for (int sp = b; sp < n_sp; sp += nwg) {
        if (sp != b) shared_load(sp);
        xr.load(lds_xp, H, geoH);
        uint32_t v[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const float g = wave_sum(tile_dot(ts[r][0], xr));
          const float u = wave_sum(tile_dot(ts[r][1], xr));
          v[r] = __float_as_uint(silu(g) * u);
        }
        if (lane == 0)
          rec_st(rsh, (uint32_t)(16 * sp),
                 u32x4_t{v[0], v[1], 0u, rec_check(ep, v[0], v[1], 0u, pos_salt(kSaltShared, sp))});
      }
      CHAIN_MARK(2, 3);   // shared SwiGLU published
    }
    lds_barrier();
    CHAIN_MARK(3, 0);   // top-k known
    if (b == 0 && tid < k) {
      if (a.idx_out) a.idx_out[(int64_t)l * k + tid] = sh.sel[tid];
      if (a.w_out) a.w_out[(int64_t)l * k + tid] = sh.coef[1 + tid];
    }
    const int n_gu = k * a.nGUs;
    TileH tg[kUG], tu[kUG];
    auto gu_load = [&](int64_t e, int part) {
      const uint8_t* base = L.slabs + e * a.stride;
      const int n0 = part * a.gu_rows + wave * kUG;
#pragma unroll
      for (int u = 0; u < kUG; ++u) {
        tg[u].load(base + a.off[0], base + a.off[1], base + a.off[2], H, n0 + u, geoH);
        tu[u].load(base + a.off[3], base + a.off[4], base + a.off[5], H, n0 + u, geoH);
      }
    };
    auto gu_dots = [&]() {
      xr.load(lds_xp, H, geoH);
#pragma unroll
      for (int u = 0; u < kUG; ++u) {
        const float gs = sum_lanes(tile_dot(tg[u], xr), kWave);
        const float us = sum_lanes(tile_dot(tu[u], xr), kWave);
        if (lane == kWave - 1) sh.act[wave * kUG + u] = silu(gs) * us;
      }
    };
    auto gu_publish = [&](int part) {
      lds_barrier();
      if (writer_wave)
        publish_blocks<BITS>(sh.act[lane < a.gu_rows ? lane : 0], a.gu_rows,
                             (part % a.nGUs) * a.gu_rows, 1 + part / a.nGUs, I, rimg, ep,
                             sh.fail != 0, sh);
      lds_barrier();
    };

    // ---- phase D (all four waves): every part's h and sum of squares, R
    // records a part, kPer records per thread a pass; h into lds_x, the sums
    // into lds_ss (the prepared-x area, free by now).  False if the wait gave
    // up.
    auto poll_parts = [&]() -> bool {
      constexpr int kPer = 1;   // small poll rounds finish sooner than one round of six
      const int t = tid_x();
      const int nrec = R * a.nD;
      float* lds_ss = reinterpret_cast<float*>(lds_xp);
      bool ok_all = true;
      for (int base = 0; base < nrec; base += kPer * kThreads) {
        bool done[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) done[j] = base + j * kThreads + t >= nrec;
        const uint64_t t0 = now_ticks();
        for (;;) {
          u32x4_t r[kPer];
#pragma unroll
          for (int j = 0; j < kPer; ++j) {
            const int ri = min(base + j * kThreads + t, nrec - 1);
            if (!done[j]) r[j] = rec_ld(rpart, (uint32_t)(16 * ri));
          }
          bool pending = false;
#pragma unroll
          for (int j = 0; j < kPer; ++j) {
            if (done[j]) continue;
            const int ri = base + j * kThreads + t;
            if (!rec_ok(r[j], ep, pos_salt(kSaltPart, ri))) { pending = true; continue; }
            done[j] = true;
            const int d = ri / R, c = ri - d * R;
#pragma unroll
            for (int i = 0; i < 3; ++i) {
              const int w = 3 * c + i;
              if (w < dr) lds_x[d * dr + w] = __uint_as_float(r[j][i]);
              else if (w == dr) lds_ss[d] = __uint_as_float(r[j][i]);
            }
          }
          if (!__any(pending)) break;
          if (now_ticks() - t0 > a.spin_ticks) { ok_all = false; break; }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      return ok_all;
    };

    if (holder) {
      // ---- waves 2-3: routed gate/up rows, the down rows, h, the next x
      float gv[kUD];
      for (int part = b; part < n_gu; part += nwg) {
        gu_load(sh.sel[part / a.nGUs], part % a.nGUs);
        gu_dots();
        gu_publish(part);
      }
      CHAIN_MARK(4, 3);   // routed SwiGLU published
      // the down rows of every active expert (slot 0: the shared one), in
      // flight while the pollers wait for the images
#pragma unroll
      for (int sl = 0; sl < kFusedMaxSlots; ++sl)
#pragma unroll
        for (int u = 0; u < kUD; ++u)
          down_tile(td[sl][u], sl == 0 ? (int64_t)E : (int64_t)sh.sel[min(sl, k) - 1], u);
#pragma unroll
      for (int u = 0; u < kUD; ++u) gv[u] = L.gamma[drow[u]];
      CHAIN_MARK(9, 3);   // down rows requested

      // ---- phase C (one batch: k + 1 <= kFusedMaxSlots)
      lds_barrier();   // images polled
      lds_barrier();   // shared image built
      float acc[kUD];
#pragma unroll
      for (int u = 0; u < kUD; ++u) acc[u] = 0.f;
#pragma unroll
      for (int sl = 0; sl < kFusedMaxSlots; ++sl) {
        if (sl < kp1) {
          XRegsW<BITS> xw;
          xw.load(lds_ap + sl * ib, I, geoI);
          const float c = sh.coef[sl];
#pragma unroll
          for (int u = 0; u < kUD; ++u) {
            pin_tile(td[sl][u]);
            acc[u] = fmaf(c, tile_dot_w(td[sl][u], xw), acc[u]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);   // one expert's activations in registers at a time
      }
#pragma unroll
      for (int u = 0; u < kUD; ++u) acc[u] = sum_lanes(acc[u], geoI.LPR);
      CHAIN_MARK(10, 3);   // down rows computed
      const bool writer = geoI.lane_seg == geoI.LPR - 1;
      const bool bad = sh.fail != 0;
      float hval[kUD];
      float ss = 0.f;
#pragma unroll
      for (int u = 0; u < kUD; ++u) {
        hval[u] = bad ? __builtin_nanf("") : rv[u] + acc[u];
        if (writer) {
          a.h_out[(int64_t)l * H + drow[u]] = hval[u];
          s_hrow[drow[u] - b * dr] = hval[u];
          ss = fmaf(hval[u], hval[u], ss);
        }
      }
      ss = sum_lanes(ss, kWave);
      if (lane == kWave - 1) sh.part[wave] = ss;
      lds_barrier();
      // the part's values of h and their sum of squares: R records
      if (writer_wave && lane < R && b != a.stall_part) {
        const float tot = sh.part[2] + sh.part[3];
        uint32_t d[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const int w = 3 * lane + i;
          d[i] = w < dr ? __float_as_uint(s_hrow[w]) : w == dr ? __float_as_uint(tot) : 0u;
        }
        const int ri = R * b + lane;
        rec_st(rpart, (uint32_t)(16 * ri),
               u32x4_t{d[0], d[1], d[2], rec_check(ep, d[0], d[1], d[2], pos_salt(kSaltPart, ri))});
      }
      CHAIN_MARK(6, 3);   // part published
      // gamma of this layer for the next x (all H), then the next layer's
      // first loads, in flight during phase D
      constexpr int kG4 = kQ * 2;   // float4 per holder thread: H / 4 / 128
      float4 gq[kG4];
#pragma unroll
      for (int q = 0; q < kG4; ++q)
        gq[q] = reinterpret_cast<const float4*>(L.gamma)[q * 128 + (tid - 128)];
      first_loads(ch.layer[min(l + 1, ch.n - 1)]);
      if (!poll_parts()) sh.fail = 1;
      lds_barrier();   // every part's h and sum in LDS
      lds_barrier();   // phase D polled: h in lds_x, the sum of squares in sh.part[0..1]
      const float tot = sh.part[0] + sh.part[1];
      const float inv = 1.f / sqrtf(tot / (float)H + a.eps);
      const bool bad2 = sh.fail != 0;
#pragma unroll
      for (int u = 0; u < kUD; ++u) {
        if (writer) a.y_out[(int64_t)l * H + drow[u]] = bad2 ? __builtin_nanf("") : gv[u] * hval[u] * inv;
        rv[u] = hval[u];
      }
      // the next layer's x = gamma * h * inv, in place
#pragma unroll
      for (int q = 0; q < kG4; ++q) {
        float4* p = reinterpret_cast<float4*>(lds_x) + q * 128 + (tid - 128);
        const float4 hv = *p;
        *p = bad2 ? make_float4(__builtin_nanf(""), 0.f, 0.f, 0.f)
                  : make_float4(gq[q].x * hv.x * inv, gq[q].y * hv.y * inv, gq[q].z * hv.z * inv,
                                gq[q].w * hv.w * inv);
      }
      if (bad2 && writer_wave && lane == 0) st_agent(a.timeout, 1);
      lds_barrier();   // next x complete
    } else {
      // ---- waves 0-1: routed gate/up rows, then every poll
      for (int part = b; part < n_gu; part += nwg) {
        gu_load(sh.sel[part / a.nGUs], part % a.nGUs);
        gu_dots();
        gu_publish(part);
      }
      const int t = tid;    // 0 .. 127
      bool ok = poll_shared<128>(lds_x, rsh, I, ep, a.spin_ticks, t);
      ok &= poll_images<BITS, 128>(lds_ap, 1, rimg, I, 1, k, ep, a.spin_ticks, t);
      if (!ok) sh.fail = 1;
      lds_barrier();   // images polled
      CHAIN_MARK(5, 0);   // first images in LDS
      image_from_f32<BITS, 128>(lds_ap, lds_x, I, t);
      lds_barrier();   // shared image built
      lds_barrier();                   // the holders' part sums in sh.part[2..3]
      // the next layer's first loads, ahead of the polls (they complete in
      // order: the first poll returns when these have arrived)
      first_loads(ch.layer[min(l + 1, ch.n - 1)]);
      if (!poll_parts()) sh.fail = 1;
      CHAIN_MARK(7, 0);   // every part polled
      lds_barrier();   // every part's h and sum in LDS
      // the sum of squares in the one-token kernel's order: parts t, t + 128,
      // ... per thread, then across the waves' lanes, then wave 0 + wave 1
      const float* lds_ss = reinterpret_cast<const float*>(lds_xp);
      float p = 0.f;
      for (int d = t; d < a.nD; d += 128) p += lds_ss[d];
      p = sum_lanes(p, kWave);
      if (lane == kWave - 1) sh.part[wave] = p;
      lds_barrier();   // phase D polled
      lds_barrier();   // next x complete
      CHAIN_MARK(8, 0);   // next x complete
    }
  }
  if (b == 0 && tid_x() == 64 * 3) st_agent(epoch_word, (int)((ep_base + (uint32_t)ch.n) & 0x7FFFFFFFu));
}

}  // namespace fmoe
