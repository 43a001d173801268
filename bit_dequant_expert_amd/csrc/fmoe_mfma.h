// fmoe_mfma.h -- the experts of a batch on the matrix cores (4-bit codes).
//
// An expert that receives tokens of a batch is applied as a matrix product
// Y[tokens x N] = X[tokens x K] * deq(W)^T with v_mfma_f32_16x16x32_f16
// instead of one matrix-vector product per token.  The activations enter as
// fp16 scaled by one power of two per vector (x = sc x', max|x'| in
// [2^13, 2^14)); the weights as fp16 w = q s + b, made in registers from the
// codes: the magic-number form 1024 + q of the GEMV (one v_and_or_b32 per
// pair), minus 1024 in one packed add (exact), then one packed fma with the
// group's scale and bias ([WAS] "2. FMA-optimierte Dequantisierungs-Kernel":
// the dequantisation as a single fused multiply-add) rounded once to fp16.
// Products accumulate in fp32; y = sc * sum w x'.  For codes q and bf16 s
// and b the fp16 weight is exact whenever q s + b has at most 11 significant
// bits (b = -z s with a small integer z does), else it is rounded once.
//
// Work split: one wave owns 16 weight rows of one expert over the whole K
// (no reduction across waves); the 4 waves of a workgroup take 4 adjacent row
// tiles of the same expert (down: kMoeDnTiles such groups of 64 rows, each
// wave one tile of each, sharing its activation words).  Tokens go in passes of 16 (one MFMA tile).
// K runs in blocks of 128: lane group l / 16 takes 32 consecutive codes (16
// bytes) of its row, one 16-byte load, and feeds them to 4 MFMA steps; the
// activation words follow the same k order.  Codes (and the gate/up
// activation words of passes with many tokens) stream through a register
// ring of blocks; the scales of the workgroup's rows and the other
// activation images sit in LDS.  Gate/up workgroups are smaller (64 /
// kMoeGuSplit rows, kMoeGuSplit waves splitting K per 16-row tile), so that
// the last of the many workgroups a layer needs leave fewer compute units idle.
#pragma once

#include <type_traits>

#include "fmoe_fused.h"

namespace fmoe {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Activation image of a K-vector for the matrix cores: word w (elements
// 8w..8w+7) is 16 bytes holding the fp16 pairs (x'[8w+i], x'[8w+4+i]),
// i = 0..3, the order in which the nibble masks take a 32-bit code word
// apart; x' = x / sc with sc a power of two that puts max|x'| in
// [2^13, 2^14).  Per group of G elements: the sum of the fp16 x' values
// (written when sums is not null).  One wave converts src[0..K) into
// dst[0..K/8) and sums[0..K/G) and returns sc (dst and sums may be global or
// LDS); K <= 512 MAXW.
// The loads of image_row: MAXW words per lane (K <= 512 MAXW), clamped.
template <int MAXW>
__device__ __forceinline__ void image_load(const float* src, int K, float4 (&lo)[MAXW],
                                           float4 (&hi)[MAXW]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int NW = K / 8;
  const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int j = 0; j < MAXW; ++j) {
    const int w = min(j * kWave + lane, NW - 1);
    lo[j] = s4[2 * w];
    hi[j] = s4[2 * w + 1];
  }
}

// The rest of image_row, from the loaded words: the max, the scale, the
// conversion and the stores; returns sc.
template <int G, int MAXW>
__device__ __forceinline__ float image_finish(const float4 (&lo)[MAXW], const float4 (&hi)[MAXW],
                                              int K, uint4* dst, float* sums) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int WPG = G / 8;   // words per group
  const int NW = K / 8;
  uint32_t m = 0;   // max |x| as bits (non-negative floats order like their bits)
#pragma unroll
  for (int j = 0; j < MAXW; ++j) {
    const float v = fmaxf(fmaxf(fmaxf(fabsf(lo[j].x), fabsf(lo[j].y)), fmaxf(fabsf(lo[j].z), fabsf(lo[j].w))),
                          fmaxf(fmaxf(fabsf(hi[j].x), fabsf(hi[j].y)), fmaxf(fabsf(hi[j].z), fabsf(hi[j].w))));
    m = max(m, __float_as_uint(v));
  }
  m = wave_max_u32(m);
  const float mx = __uint_as_float(m);
  int sh = 0;
  if (mx > 0.f && mx <= 3.402823466e38f) {
    int ex;
    frexpf(mx, &ex);        // mx = f * 2^ex, f in [0.5, 1)
    sh = ex - 14;           // max|x'| in [2^13, 2^14)
  }
#pragma unroll
  for (int j = 0; j < MAXW; ++j) {
    const int w = j * kWave + lane;
    if (j * kWave < NW) {   // uniform
      const float xv[8] = {lo[j].x, lo[j].y, lo[j].z, lo[j].w, hi[j].x, hi[j].y, hi[j].z, hi[j].w};
      _Float16 h[8];
      float s2 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        h[e] = (_Float16)ldexpf(xv[e], -sh);
        s2 += (float)h[e];
      }
      uint32_t p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p[i] = (uint32_t)__builtin_bit_cast(uint16_t, h[i]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h[4 + i]) << 16);
      if (w < NW) dst[w] = make_uint4(p[0], p[1], p[2], p[3]);
      // The words of a group sit in WPG consecutive lanes (WPG divides 64).
      if (sums) {
        s2 = sum_lanes(s2, WPG);
        if (w < NW && lane % WPG == WPG - 1) sums[w / WPG] = s2;
      }
    }
  }
  return ldexpf(1.f, sh);
}

template <int G, int MAXW>
__device__ __forceinline__ float image_row(const float* src, int K, uint4* dst, float* sums) {
  float4 lo[MAXW], hi[MAXW];
  image_load<MAXW>(src, K, lo, hi);
  return image_finish<G, MAXW>(lo, hi, K, dst, sums);
}

// Weights of one 32-bit code word (8 codes, in the nibble-mask order) as the
// B operand's 8 halves: q exactly (1024 + q minus 1024), then q s + b.
__device__ __forceinline__ f16x8 weights_f16x8(uint32_t w, f16x2 s2, f16x2 b2) {
  const uint32_t mg = magic_v();
  const f16x2 off = {(_Float16)1024.f, (_Float16)1024.f};
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 q = __builtin_bit_cast(f16x2, ((w >> (4 * i)) & 0x000F000Fu) | mg) - off;
    p[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
  }
  return __builtin_bit_cast(f16x8, make_uint4(p[0], p[1], p[2], p[3]));
}

// LDS of k_moe_mfma: scales and biases of the workgroup's RW rows
// ([NM][2][RW] rows of NG*SB bytes, padded by 4), then the images of the
// pass's inputs that are read from LDS ([kMoeLdsTokens or 16][K/8 + 1] words),
// an area that gate/up reuses for the sums of its waves' K shares.
__host__ __device__ inline int moe_scl_row(int K, int G, int SB) { return (K / G) * SB + 4; }
__host__ __device__ inline size_t moe_mfma_lds(int mode, int H, int I, int G, int SB) {
  const int nm = mode == 0 ? 2 : 1, K = mode == 0 ? H : I;
  const int rw = mode == 0 ? kMoeGuRows : kMoeDnRows;
  const size_t scl = ((size_t)nm * 2 * rw * moe_scl_row(K, G, SB) + 15) / 16 * 16;
  const size_t img = (size_t)(mode == 0 ? kMoeLdsTokens : 16) * (K / 8 + 1) * 16;
  const size_t red =
      mode == 0 ? (size_t)(kThreads / kWave / kMoeGuSplit) * (kMoeGuSplit - 1) * nm * kWave * 16 : 0;
  return scl + (img > red ? img : red);
}

// Blocks of 128 k a wave keeps in flight.  A ring slot holds the lane's 16
// bytes of codes per matrix and, when the activation words come from global
// memory (gate/up passes of many tokens), those too (16 VGPRs).
#ifndef FMOE_MOE_PB_GU
#define FMOE_MOE_PB_GU 4    // gate/up, activation words from LDS
#endif
#ifndef FMOE_MOE_PB_REG
#define FMOE_MOE_PB_REG 2   // gate/up, activation words in the ring
#endif
#ifndef FMOE_MOE_PB_DN
#define FMOE_MOE_PB_DN 4    // down (K / 128 = 8 blocks: two whole rings)
#endif

// Workgroup (ai, rb): active expert ai (every expert with at least
// a.mfma_thr tokens).  MODE 0: rows RW rb .. RW rb + RW - 1 (RW = kMoeGuRows),
// wave w the tile of 16 rows RW rb + 16 (w / S) over its part w % S of the
// blocks of K (S = kMoeGuSplit), the S partial tiles added in wave order; gate
// and up (K = H) with SwiGLU into abuf; the activation words come from the
// token images in LDS when the pass has at most kMoeLdsTokens tokens, else
// from global memory through the register ring.  MODE 1 rows: 64 rb .. 64 rb
// + 63 (N % 64 == 0), wave w the tile of 16 rows 64 rb + 16 w, all of K
// (with kMoeDnTiles > 1: rows kMoeDnRows rb .., wave w the tiles 16 w + 64 j).  MODE 1: down (K = I) into yslot, the images of the pass's SwiGLU
// rows built in LDS first.  Lane l: B column (weight row) l % 16, A row
// (token) l % 16, k sub-block l / 16; D element i is token 4 (l / 16) + i,
// weight row l % 16.  Needs K % 128 == 0.
template <int G, int SB, int MODE>
__global__ __launch_bounds__(kThreads, MODE == 1 ? kMoeDnWgs : 4) void k_moe_mfma(MfmaArgs a) {
  constexpr int NM = MODE == 0 ? 2 : 1;   // matrices: gate and up, or down
  // Code streams (accumulators) of a wave: the two matrices, or the down tiles.
  constexpr int NA = MODE == 0 ? 2 : kMoeDnTiles;
  extern __shared__ __align__(16) uint4 lds4[];
  __shared__ float s_sc[16];
  __shared__ int s_ent[16];
  // Per row of the workgroup: the largest |scale| or |bias| of the row in its
  // matrices (gate and up, or down), as an fp32 bit pattern, gathered while the
  // scales are staged.  The row's scales and biases enter fp16 times a power of
  // two that puts that largest value in [2^10, 2^11) (so every dequantised fp16
  // weight stays below 2^15), and the fp32 result is multiplied back: fp16's
  // range does not limit the format's.
  __shared__ uint32_t s_rmax[MODE == 0 ? 64 : kMoeDnRows];
  // Gate/up: kMoeGuRows rows per workgroup, S waves per 16-row tile, each
  // over a part of K; down: 64 rows, a wave's 16 rows over the whole K.
  constexpr int S = MODE == 0 ? kMoeGuSplit : 1;
  constexpr int RW = MODE == 0 ? 64 / S : kMoeDnRows;   // rows per workgroup
  const int N = MODE == 0 ? a.I : a.H, K = MODE == 0 ? a.H : a.I;
  const int nrb = N / RW;
  const int ai = blockIdx.x / nrb, rb = blockIdx.x - ai * nrb;
  const ActView av{a.act, a.maxA};
  // The list header and this workgroup's entry in one round trip (ai < maxA:
  // the entry is inside the list even when it is not in use).
  const int nact = av.base[0], cnt = av.cnt()[ai];
  const int64_t e = av.e()[ai];
  const int eoff = av.off()[ai];
  if (ai >= nact || cnt < a.mfma_thr) return;
  const uint8_t* base = a.src.base + e * a.src.stride;
  const int tid = tid_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = wave / S, part = wave - tile * S;   // 16-row tile, part of K
  const int n = rb * RW + tile * 16 + (lane & 15);
  const int jg = lane >> 4, am = lane & 15;
  const int NG = K / G, NW = K / 8;
  // The wave's blocks of 128 k: [kb0, kb0 + NBK), its part of K (empty for
  // some waves when K has fewer than S blocks).
  const int kb0 = (part * (K / 128)) / S;
  const int NBK = ((part + 1) * (K / 128)) / S - kb0;
  const int SROW = moe_scl_row(K, G, SB);
  const int nl = tile * 16 + (lane & 15);   // row within the workgroup's
  const int om = MODE == 0 ? 0 : 6;
  static_assert(RW <= kThreads, "row maxima");
  if (tid < RW) s_rmax[tid] = 0u;   // ordered before the staging by the pass barriers
  // |v| of the scale words of one 4-byte word (fp32: one value; bf16: two,
  // as the fp32 bit patterns of their magnitudes), for an unsigned max.
  auto word_max = [](uint32_t w) -> uint32_t {
    if (SB == 4) return w & 0x7fffffffu;
    return max(w & 0x7fffu, (w >> 16) & 0x7fffu) << 16;
  };
  auto chunk_max = [&](uint4 v) -> uint32_t {
    return max(max(word_max(v.x), word_max(v.y)), max(word_max(v.z), word_max(v.w)));
  };
  uint8_t* s_scl = reinterpret_cast<uint8_t*>(lds4);
  uint4* s_img = reinterpret_cast<uint4*>(s_scl + ((size_t)NM * 2 * RW * SROW + 15) / 16 * 16);

  // Scales and biases of the workgroup's RW rows: contiguous in the slab, copied
  // into padded LDS rows.  When they fit in kSR 16-byte words per thread they
  // are loaded into registers first and stored later (scales_load,
  // scales_store), else copied in one loop (stage_scales).
  constexpr int kSR = MODE == 1 ? kMoeDnTiles : 1;
  const int rowb = NG * SB;
  const int sper = RW * rowb / 16, stot = 2 * NM * sper;
  // (Down only: gate/up has no registers to spare for it.)
  const bool sfast = MODE == 1 && rowb % 16 == 0 && stot <= kSR * kThreads;   // uniform
  uint4 sreg[kSR];
  auto scl_src = [&](int arr) {
    return base + a.src.off[om + 3 * (arr >> 1) + 1 + (arr & 1)] + (int64_t)rb * RW * rowb;
  };
  auto scales_load = [&]() {
#pragma unroll
    for (int j = 0; j < kSR; ++j) {
      const int i = min(j * kThreads + tid, stot - 1);
      const int arr = i / sper, k = i - arr * sper;
      sreg[j] = reinterpret_cast<const uint4*>(scl_src(arr))[k];
    }
  };
  auto scales_store = [&]() {
#pragma unroll
    for (int j = 0; j < kSR; ++j) {
      const int i = j * kThreads + tid;
      if (i < stot) {
        const int arr = i / sper, k = i - arr * sper;
        const int r = (k * 16) / rowb, c = k * 16 - r * rowb;
        uint32_t* d = reinterpret_cast<uint32_t*>(s_scl + (size_t)arr * RW * SROW + r * SROW + c);
        d[0] = sreg[j].x; d[1] = sreg[j].y; d[2] = sreg[j].z; d[3] = sreg[j].w;
        atomicMax(&s_rmax[r], chunk_max(sreg[j]));
      }
    }
  };
  auto stage_scales = [&]() {
#pragma unroll
    for (int arr = 0; arr < 2 * NM; ++arr) {
      const uint8_t* src = base + a.src.off[om + 3 * (arr >> 1) + 1 + (arr & 1)] +
                           (int64_t)rb * RW * rowb;
      uint8_t* dst = s_scl + (size_t)arr * RW * SROW;
      if (rowb % 16 == 0) {
        for (int i = tid; i < RW * rowb / 16; i += kThreads) {
          const uint4 v = reinterpret_cast<const uint4*>(src)[i];
          const int r = (i * 16) / rowb, c = (i * 16) - r * rowb;
          uint32_t* d = reinterpret_cast<uint32_t*>(dst + r * SROW + c);
          d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
          atomicMax(&s_rmax[r], chunk_max(v));
        }
      } else {
        for (int i = tid; i < RW * rowb / 4; i += kThreads) {
          const uint32_t v = reinterpret_cast<const uint32_t*>(src)[i];
          const int r = (i * 4) / rowb, c = (i * 4) - r * rowb;
          *reinterpret_cast<uint32_t*>(dst + r * SROW + c) = v;
          atomicMax(&s_rmax[r], word_max(v));
        }
      }
    }
  };
  // Addresses: the wave's first row as a wave-uniform base (SGPRs) and one
  // 32-bit offset per lane, so that a ring slot costs no address registers.
  const int64_t row0 = (int64_t)rb * RW + tile * 16;
  const uint8_t* qm[NA];
#pragma unroll
  for (int mi = 0; mi < NA; ++mi)
    qm[mi] = MODE == 0 ? uniform_gptr(base + a.src.off[3 * mi] + row0 * (K / 2) + kb0 * 64)
                       : uniform_gptr(base + a.src.off[om] + (row0 + 64 * mi) * (K / 2) + kb0 * 64);
  const uint32_t lq = (uint32_t)(lane & 15) * (uint32_t)(K / 2) + (uint32_t)jg * 16u;

  for (int c0 = 0; c0 < cnt; c0 += 16) {
    const int pc = min(16, cnt - c0);     // tokens in this pass
    __syncthreads();                      // the previous pass is done with LDS
    if (tid < 16) {
      const int p = av.entries()[eoff + c0 + min(tid, pc - 1)];
      s_ent[tid] = tid < pc ? p : -1;
      if (MODE == 0) s_sc[tid] = a.xsc[p / a.kp1];
    }
    __syncthreads();
    // A row of this lane: token am of the pass, or (idle rows, am >= pc) the
    // pass's last token again.  An output row of the product depends on its
    // own A row only, and idle rows are never stored, so they need no zeros.
    const int ar = min(am, pc - 1);

    f32x4 acc[NA];
#pragma unroll
    for (int mi = 0; mi < NA; ++mi) acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Row of the workgroup that code stream mi of this lane takes.
    auto srow = [&](int mi) { return MODE == 0 ? nl : nl + 64 * mi; };
    // The power of two of a weight row (see s_rmax): 2^-e into fp16.
    auto row_shift = [&](int r) {
      const float mx = __uint_as_float(s_rmax[r]);
      int ex = 0;
      frexpf(mx, &ex);   // mx in [2^(ex-1), 2^ex)
      return mx > 0.f ? min(max(ex - 11, -100), 100) : 0;
    };
    float rin[NA];

    auto run = [&](auto al_c) {
      constexpr bool AL = decltype(al_c)::value;          // activation words from LDS
      constexpr int PB = MODE == 1 ? FMOE_MOE_PB_DN : (AL ? FMOE_MOE_PB_GU : FMOE_MOE_PB_REG);
      constexpr int NXW = AL ? 1 : 4;
      const uint4* xrow = a.ximg + (int64_t)(MODE == 0 ? s_ent[ar] / a.kp1 : 0) * NW + kb0 * 16 + jg * 4;
      const uint4* lrow = s_img + ar * (NW + 1) + kb0 * 16 + jg * 4;
      uint4 rq[PB][NA], rx[PB][NXW];
      auto issue = [&](int u, int b) {
#pragma unroll
        for (int mi = 0; mi < NA; ++mi)
          rq[u][mi] = *reinterpret_cast<const uint4*>(uniform_gptr(qm[mi] + b * 64) + lq);
        if (!AL) {
#pragma unroll
          for (int s = 0; s < NXW; ++s) rx[u][s] = xrow[b * 16 + s];
        }
      };
      auto compute = [&](int u, int b) {
        uint4 xw[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) xw[s] = AL ? lrow[b * 16 + s] : rx[u][s % NXW];
        const int gi = ((kb0 + b) * 128 + jg * 32) / G;
#pragma unroll
        for (int mi = 0; mi < NA; ++mi) {
          const int ms = MODE == 0 ? mi : 0;   // matrix of the stream
          const uint8_t* sr = s_scl + ((size_t)(2 * ms) * RW + srow(mi)) * SROW + gi * SB;
          const uint8_t* br = s_scl + ((size_t)(2 * ms + 1) * RW + srow(mi)) * SROW + gi * SB;
          const float sv = SB == 2 ? sb_value<2>(*reinterpret_cast<const uint16_t*>(sr))
                                   : *reinterpret_cast<const float*>(sr);
          const float bv = SB == 2 ? sb_value<2>(*reinterpret_cast<const uint16_t*>(br))
                                   : *reinterpret_cast<const float*>(br);
          const _Float16 sh = (_Float16)(sv * rin[mi]), bh = (_Float16)(bv * rin[mi]);
          const f16x2 s2 = {sh, sh}, b2 = {bh, bh};
          const uint32_t cw[4] = {rq[u][mi].x, rq[u][mi].y, rq[u][mi].z, rq[u][mi].w};
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(f16x8, xw[s]), weights_f16x8(cw[s], s2, b2), acc[mi], 0, 0, 0);
        }
      };
      // LDS set-up: the staging loads go out first (scales on the first pass,
      // the inputs), then the first ring of code loads, then the LDS stores,
      // each of which waits for its own loads only (one in-order counter);
      // the code latency overlaps the set-up.
      constexpr int IMW = kMfmaMaxI / 512;   // down: words per lane of an input row
      constexpr int kXS = 4;                 // gate/up: image words per thread
      const bool stage_s = c0 == 0;
      if (stage_s && sfast) scales_load();
      float4 ilo[IMW], ihi[IMW];
      uint4 xs[kXS];
      const bool xfast = false;   // gate/up: no registers to spare (copied after the ring)
      if (MODE == 1) {
        image_load<IMW>(a.abuf + (int64_t)s_ent[min(wave, pc - 1)] * a.I, a.I, ilo, ihi);
      } else if (xfast) {
#pragma unroll
        for (int j = 0; j < kXS; ++j) {
          const int i = min(j * kThreads + tid, pc * NW - 1), m = i / NW, w = i - m * NW;
          xs[j] = a.ximg[(int64_t)(s_ent[m] / a.kp1) * NW + w];
        }
      }
#pragma unroll
      for (int u = 0; u < PB; ++u) issue(u, max(0, min(u, NBK - 1)));
      if (stage_s && sfast) scales_store();
      else if (stage_s) stage_scales();
      if (MODE == 1) {
        if (wave < pc) {
          const float sc = image_finish<G, IMW>(ilo, ihi, a.I, s_img + wave * (NW + 1), nullptr);
          if (lane == 0) s_sc[wave] = sc;
        }
        for (int r = wave + kThreads / kWave; r < pc; r += kThreads / kWave) {
          const float sc = image_row<G, IMW>(a.abuf + (int64_t)s_ent[r] * a.I, a.I,
                                             s_img + r * (NW + 1), nullptr);
          if (lane == 0) s_sc[r] = sc;
        }
      } else if (xfast) {
#pragma unroll
        for (int j = 0; j < kXS; ++j) {
          const int i = j * kThreads + tid, m = i / NW, w = i - m * NW;
          if (i < pc * NW) s_img[m * (NW + 1) + w] = xs[j];
        }
      } else if (AL) {
        for (int i = tid; i < pc * NW; i += kThreads) {
          const int m = i / NW, w = i - m * NW;
          s_img[m * (NW + 1) + w] = a.ximg[(int64_t)(s_ent[m] / a.kp1) * NW + w];
        }
      }
      __syncthreads();
#pragma unroll
      for (int mi = 0; mi < NA; ++mi) rin[mi] = ldexpf(1.f, -row_shift(srow(mi)));
      // Whole rings without branches while a whole next ring follows (the
      // load waits stay exact); then the ring in flight is computed while the
      // r blocks after it, if any, are requested, and those last.  No block
      // is requested twice.
      int bb = 0;
      for (; bb + 2 * PB <= NBK; bb += PB) {
#pragma unroll
        for (int u = 0; u < PB; ++u) {
          compute(u, bb + u);
          issue(u, bb + u + PB);
        }
      }
      const int r = NBK - bb - PB;   // < 0 when the whole K is one short ring
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        if (bb + u < NBK) compute(u, bb + u);
        if (u < r) issue(u, bb + PB + u);
      }
#pragma unroll
      for (int u = 0; u < PB; ++u)
        if (u < r) compute(u, bb + PB + u);
    };
    if (MODE == 1 || pc <= kMoeLdsTokens) run(std::true_type{});
    else run(std::false_type{});

    if constexpr (S > 1) {
      // The parts of K of a tile are added in part order through LDS (the
      // image area, free once every wave is past its products); the part-0
      // wave keeps the sums and stores.
      f32x4* s_red = reinterpret_cast<f32x4*>(s_img);
      __syncthreads();
      if (part > 0) {
#pragma unroll
        for (int mi = 0; mi < NA; ++mi)
          s_red[((tile * (S - 1) + part - 1) * NA + mi) * kWave + lane] = acc[mi];
      }
      __syncthreads();
      if (part > 0) continue;
#pragma unroll
      for (int j = 1; j < S; ++j)
#pragma unroll
        for (int mi = 0; mi < NA; ++mi) {
          const f32x4 v = s_red[((tile * (S - 1) + j - 1) * NA + mi) * kWave + lane];
          acc[mi] = f32x4{acc[mi][0] + v[0], acc[mi][1] + v[1], acc[mi][2] + v[2], acc[mi][3] + v[3]};
        }
    }

    float rout[NA];
#pragma unroll
    for (int mi = 0; mi < NA; ++mi) rout[mi] = ldexpf(1.f, row_shift(srow(mi)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * jg + i;
      if (m < pc) {
        const int p = s_ent[m];
        if constexpr (MODE == 0) {
          const float sc = s_sc[m] * rout[0];
          a.abuf[(int64_t)p * a.I + n] = silu(acc[0][i] * sc) * (acc[1][i] * sc);
        } else {
#pragma unroll
          for (int mi = 0; mi < NA; ++mi)
            a.yslot[(int64_t)p * a.H + n + 64 * mi] = acc[mi][i] * (s_sc[m] * rout[mi]);
        }
      }
    }
  }
}

}  // namespace fmoe
