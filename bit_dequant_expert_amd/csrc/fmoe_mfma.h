// fmoe_mfma.h -- experts that receive many tokens of a batch, on the matrix
// cores (4-bit codes).
//
// When a batch routes at least kMfmaTokens tokens to one expert, the expert
// is applied as a matrix product instead of one matrix-vector product per
// token: Y[tokens x N] = X[tokens x K] * deq(W)^T with v_mfma_f32_16x16x32_f16.
// The codes enter the matrix core as exact fp16 integers (the magic-number
// form 1024 + q of the GEMV, one v_and_or_b32 per pair, minus 1024 in one
// packed add: the fp32 accumulator then holds sum q x' without a large offset
// to cancel), the activations as fp16 scaled by one power of two per vector.
// Per group of G codes the accumulator is scaled by the group's scale, and the
// bias enters through the group sum of the activations, as [WAS] "2.
// FMA-optimierte Dequantisierungs-Kernel" takes the bias out of the inner loop:
//   sum_{k in g} (q s + b) x = sc (s sum q x' + b sum x'),   x = sc x'.
// Both sums run over the same fp16-rounded x': with the bias near -s times
// the middle code, the rounding errors of x' then enter through the centred
// weight (q - z) s instead of through q s, which is several times larger.
// The products are exact and accumulate in fp32; the only rounding beyond the
// GEMV path's is x' in fp16.
#pragma once

#include "fmoe_fused.h"

namespace fmoe {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaMT = 2;   // 16-token tiles per pass: 32 tokens share each weight load
constexpr int kMfmaPF = 4;   // groups whose loads are issued together (per wave)

// Activation image of a K-vector for the matrix cores: word w (elements
// 8w..8w+7) is 16 bytes holding the fp16 pairs (x'[8w+i], x'[8w+4+i]),
// i = 0..3, the order in which the nibble masks take a 32-bit code word
// apart; x' = x / sc with sc a power of two that puts max|x'| in
// [2^13, 2^14).  Per group of G elements: the sum of the fp16 x' values.

// One vector per workgroup.  mode 0: token blockIdx.x of x (gate/up input);
// mode 1: the blockIdx.x-th entry of the experts on this path, in the order
// of the path's list (down input, from abuf).
template <int G>
__global__ __launch_bounds__(kThreads) void k_mimg_prep(MfmaArgs a, int mode) {
  __shared__ uint32_t s_max[kThreads / kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int idx = -1, K;
  const float* src;
  uint4* img;
  float* sc;
  float* sums;
  if (mode == 0) {
    if ((int)blockIdx.x >= a.T) return;
    idx = blockIdx.x;
    K = a.H;
    src = a.x + (int64_t)idx * a.H;
    img = a.ximg; sc = a.xsc; sums = a.xsum;
  } else {
    const ActView av{a.act, a.maxA};
    const int nm = av.base[1];
    int b = blockIdx.x;
    for (int j = 0; j < nm; ++j) {
      const int i = av.mfma()[j], cnt = av.cnt()[i];
      if (b < cnt) {
        idx = av.entries()[av.off()[i] + b];
        break;
      }
      b -= cnt;
    }
    if (idx < 0) return;
    K = a.I;
    src = a.abuf + (int64_t)idx * a.I;
    img = a.aimg; sc = a.asc; sums = a.asum;
  }
  constexpr int WPG = G / 8;   // words per group
  const int NW = K / 8, NG = K / G;
  const float4* s4 = reinterpret_cast<const float4*>(src);
  uint32_t m = 0;   // max |x| as bits (non-negative floats order like their bits)
  for (int w = tid; w < NW; w += kThreads) {
    const float4 lo = s4[2 * w], hi = s4[2 * w + 1];
    const float v = fmaxf(fmaxf(fmaxf(fabsf(lo.x), fabsf(lo.y)), fmaxf(fabsf(lo.z), fabsf(lo.w))),
                          fmaxf(fmaxf(fabsf(hi.x), fabsf(hi.y)), fmaxf(fabsf(hi.z), fabsf(hi.w))));
    m = max(m, __float_as_uint(v));
  }
  m = wave_max_u32(m);
  if (lane == 0) s_max[wave] = m;
  __syncthreads();
  m = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  const float mx = __uint_as_float(m);
  int sh = 0;
  if (mx > 0.f && mx <= 3.402823466e38f) {
    int ex;
    frexpf(mx, &ex);        // mx = f * 2^ex, f in [0.5, 1)
    sh = ex - 14;           // max|x'| in [2^13, 2^14)
  }
  for (int w0 = 0; w0 < NW; w0 += kThreads) {
    const int w = w0 + tid;
    float s2 = 0.f;
    if (w < NW) {
      const float4 lo = s4[2 * w], hi = s4[2 * w + 1];
      const float xv[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      _Float16 h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xs = ldexpf(xv[e], -sh);
        h[e] = (_Float16)xs;
        s2 += (float)h[e];
      }
      uint32_t p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p[i] = (uint32_t)__builtin_bit_cast(uint16_t, h[i]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h[4 + i]) << 16);
      img[(int64_t)idx * NW + w] = make_uint4(p[0], p[1], p[2], p[3]);
    }
    // The words of a group sit in WPG consecutive lanes (WPG divides 64).
    s2 = sum_lanes(s2, WPG);
    if (w < NW && lane % WPG == WPG - 1) sums[(int64_t)idx * NG + w / WPG] = s2;
  }
  if (tid == 0) sc[idx] = ldexpf(1.f, sh);
}

// A code word as the B operand's 8 halves: the four pairs the masks
// 0x000F000F << 4i take out of it, OR 1024.0, minus 1024.0 (exact).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f16x8 codes_f16x8(uint32_t w) {
  const uint32_t mg = magic_v();
  const f16x2 off = {(_Float16)1024.f, (_Float16)1024.f};
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 v = __builtin_bit_cast(f16x2, ((w >> (4 * i)) & 0x000F000Fu) | mg) - off;
    p[i] = __builtin_bit_cast(uint32_t, v);
  }
  return __builtin_bit_cast(f16x8, make_uint4(p[0], p[1], p[2], p[3]));
}

// One workgroup: 16 output rows of one expert on this path, all of its
// tokens (in passes of 16 * kMfmaMT); the 4 waves split the K groups and add
// their tiles through LDS.  MODE 0: gate and up (K = H) with SwiGLU into abuf;
// MODE 1: down (K = I) into yslot.  Lane l holds B column (row n) l % 16 and
// code words of lane group l / 16; A row (token) l % 16; D rows 4 (l / 16) + i.
template <int G, int SB, int MODE>
__global__ __launch_bounds__(kThreads) void k_expert_mfma(MfmaArgs a) {
  constexpr int NM = MODE == 0 ? 2 : 1;   // matrices: gate and up, or down
  constexpr int SPG = G / 32;             // code words per lane group per group (MFMA steps)
  __shared__ f32x4 s_tot[3][NM * kMfmaMT][64];
  __shared__ float s_sum[16 * kMfmaMT][kMfmaMaxGroups];
  __shared__ float s_sc[16 * kMfmaMT];
  __shared__ int s_ent[16 * kMfmaMT];
  const int N = MODE == 0 ? a.I : a.H, K = MODE == 0 ? a.H : a.I;
  const int ntile = N / 16;
  const int jm = blockIdx.x / ntile, rt = blockIdx.x - jm * ntile;
  const ActView av{a.act, a.maxA};
  if (jm >= av.base[1]) return;
  const int ai = av.mfma()[jm];
  const int64_t e = av.e()[ai];
  const int cnt = av.cnt()[ai], eoff = av.off()[ai];
  const uint8_t* base = a.src.base + e * a.src.stride;
  const int tid = tid_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = rt * 16 + (lane & 15), jg = lane >> 4;
  const int NG = K / G, RB = K / 2, NW = K / 8;
  const int g0 = wave * NG / 4, g1 = (wave + 1) * NG / 4;
  const int om = MODE == 0 ? 0 : 6;
  const uint8_t* qm[NM];
  const uint8_t* sm[NM];
  const uint8_t* bm[NM];
#pragma unroll
  for (int mi = 0; mi < NM; ++mi) {
    qm[mi] = base + a.src.off[om + 3 * mi] + (int64_t)n * RB + jg * SPG * 4;
    sm[mi] = base + a.src.off[om + 3 * mi + 1] + (int64_t)n * NG * SB;
    bm[mi] = base + a.src.off[om + 3 * mi + 2] + (int64_t)n * NG * SB;
  }
  const uint4* img = MODE == 0 ? a.ximg : a.aimg;
  const float* vsc = MODE == 0 ? a.xsc : a.asc;
  const float* vsum = MODE == 0 ? a.xsum : a.asum;

  for (int c0 = 0; c0 < cnt; c0 += 16 * kMfmaMT) {
    // The pass's vectors: entry ids, scales and group sums in LDS.
    __syncthreads();
    for (int r = tid; r < 16 * kMfmaMT; r += kThreads) {
      const int jt = min(c0 + r, cnt - 1);
      const int p = av.entries()[eoff + jt];
      const int v = MODE == 0 ? p / a.kp1 : p;
      s_ent[r] = c0 + r < cnt ? p : -1;
      s_sc[r] = vsc[v];
    }
    __syncthreads();
    for (int r = tid; r < 16 * kMfmaMT * NG; r += kThreads) {
      const int rv = r / NG, g = r - rv * NG;
      const int p = s_ent[rv];
      const int v = p < 0 ? 0 : (MODE == 0 ? p / a.kp1 : p);
      s_sum[rv][g] = p < 0 ? 0.f : vsum[(int64_t)v * NG + g];
    }
    // A rows of this lane (token tile mt, row lane % 16); idle rows read row 0.
    int64_t arow[kMfmaMT];
    bool aval[kMfmaMT];
#pragma unroll
    for (int mt = 0; mt < kMfmaMT; ++mt) {
      const int jt = c0 + 16 * mt + (lane & 15);
      aval[mt] = jt < cnt;
      const int p = av.entries()[eoff + min(jt, cnt - 1)];
      arow[mt] = (int64_t)(MODE == 0 ? p / a.kp1 : p) * NW;
    }
    __syncthreads();

    f32x4 tot[NM][kMfmaMT];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
      for (int mt = 0; mt < kMfmaMT; ++mt) tot[mi][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int gb = g0; gb < g1; gb += kMfmaPF) {
      // Loads of kMfmaPF groups first (clamped), then their products.
      uint32_t wq[kMfmaPF][NM][SPG];
      uint32_t ws[kMfmaPF][NM], wb[kMfmaPF][NM];
      uint4 av4[kMfmaPF][kMfmaMT][SPG];
#pragma unroll
      for (int u = 0; u < kMfmaPF; ++u) {
        const int g = min(gb + u, g1 - 1);
#pragma unroll
        for (int mi = 0; mi < NM; ++mi) {
          const uint8_t* qp = qm[mi] + g * (G / 2);
          if (SPG == 2) {
            const uint64_t v2 = ld_nt(reinterpret_cast<const uint64_t*>(qp));
            wq[u][mi][0] = (uint32_t)v2;
            wq[u][mi][SPG - 1] = (uint32_t)(v2 >> 32);
          } else {
            wq[u][mi][0] = ld_nt(reinterpret_cast<const uint32_t*>(qp));
          }
          if (SB == 2) {
            ws[u][mi] = ld_nt(reinterpret_cast<const uint16_t*>(sm[mi] + g * 2));
            wb[u][mi] = ld_nt(reinterpret_cast<const uint16_t*>(bm[mi] + g * 2));
          } else {
            ws[u][mi] = ld_nt(reinterpret_cast<const uint32_t*>(sm[mi] + g * 4));
            wb[u][mi] = ld_nt(reinterpret_cast<const uint32_t*>(bm[mi] + g * 4));
          }
        }
#pragma unroll
        for (int mt = 0; mt < kMfmaMT; ++mt)
#pragma unroll
          for (int s = 0; s < SPG; ++s)
            av4[u][mt][s] = img[arow[mt] + g * (G / 8) + jg * SPG + s];
      }
#pragma unroll
      for (int u = 0; u < kMfmaPF; ++u) {
        const int g = gb + u;
        if (g < g1) {   // uniform
#pragma unroll
          for (int mt = 0; mt < kMfmaMT; ++mt) {
            float s2[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) s2[i] = s_sum[16 * mt + 4 * jg + i][g];
#pragma unroll
            for (int mi = 0; mi < NM; ++mi) {
              f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s = 0; s < SPG; ++s) {
                const uint4 x4 = aval[mt] ? av4[u][mt][s] : make_uint4(0, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x4),
                                                             codes_f16x8(wq[u][mi][s]), acc, 0, 0, 0);
              }
              const float sc = sb_value<SB>(ws[u][mi]), bi = sb_value<SB>(wb[u][mi]);
#pragma unroll
              for (int i = 0; i < 4; ++i) tot[mi][mt][i] = fmaf(bi, s2[i], fmaf(sc, acc[i], tot[mi][mt][i]));
            }
          }
        }
      }
    }
    // Waves 1..3 hand their partial tiles to wave 0, which finishes the rows.
    if (wave > 0) {
#pragma unroll
      for (int mi = 0; mi < NM; ++mi)
#pragma unroll
        for (int mt = 0; mt < kMfmaMT; ++mt) s_tot[wave - 1][mi * kMfmaMT + mt][lane] = tot[mi][mt];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int mt = 0; mt < kMfmaMT; ++mt) {
        f32x4 y[NM];
#pragma unroll
        for (int mi = 0; mi < NM; ++mi) {
          y[mi] = tot[mi][mt];
#pragma unroll
          for (int w = 0; w < 3; ++w) y[mi] += s_tot[w][mi * kMfmaMT + mt][lane];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mt + 4 * jg + i;
          const int p = s_ent[r];
          if (p >= 0) {
            const float sc = s_sc[r];
            if (MODE == 0) {
              const float gs = y[0][i] * sc, us = y[NM - 1][i] * sc;
              a.abuf[(int64_t)p * a.I + n] = silu(gs) * us;
            } else {
              a.yslot[(int64_t)p * a.H + n] = y[0][i] * sc;
            }
          }
        }
      }
    }
  }
}

}  // namespace fmoe
