// fmoe_device.h -- device building blocks of the quantised MoE kernels (gfx950).
//
// Dequantised dot products.  A weight is w = q * s + b with an unsigned code q
// and a per-group scale s and bias b ("Was ist Flash-MoE?", section
// "2. FMA-optimierte Dequantisierungs-Kernel").  The pages fold scale and bias
// into the activation per element (fma(q, s*x, b*x)); here they are pulled out
// of each block instead, which costs nothing per element:
//     sum_k w_k x_k = s * sum_k q_k x_k + b * sum_k x_k      (over one block)
// and the inner sum runs on v_dot2_f32_f16 with the codes turned into fp16
// without a convert instruction: OR-ing a code into the mantissa of 1024.0
// (0x6400) gives the fp16 value 1024 + q * 2^p, where p is the bit position the
// code sits at inside its 16-bit half.  The activation slot paired with that
// code is pre-scaled by 2^-p, and the 1024 offset is removed once per block
// with a precomputed sum.  Per 4-bit weight this is 1/2 AND-OR, 1/8 shift and
// 1/2 dot2; per 2-bit weight 1/2 AND-OR, 1/16 shift and 1/2 dot2.
//
// Prepared activations ("xprep").  A vector of K fp32 values is stored once
// per use as
//   pairs : K/2 dwords, two fp16 each, in the order the unpack consumes them
//   consts: K/32 float4 {P, C, A, 0}, one per block of 32 elements
// where the block's values are x * 2^-sh rounded to fp16 (sh chosen from the
// block's largest magnitude so nothing overflows), P = 2^sh, C = 1024 * P *
// (sum of the fp16 slots) and A = P * (sum of the slots scaled back by 2^p).
// For a block with codes q and dot2 chain D:  sum q_k x'_k = P*D - C, and the
// block contributes s*(P*D - C) + b*A, where x'_k is x_k rounded to an
// 11-bit significand.  Values stay finite for |x| < 2^100.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmoe {

constexpr int kWave = 64;
constexpr uint32_t kMagic = 0x64006400u;  // fp16 pair (1024.0, 1024.0)

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c,
                                false);
}

// Code layout of one 16-byte segment of a packed row.
template <int BITS> struct QF;
template <> struct QF<4> {
  static constexpr int EPS = 32;  // elements per 16-byte segment
  static constexpr int PPS = 16;  // fp16 pairs per segment
  static constexpr int CPS = 1;   // 32-element blocks per segment
};
template <> struct QF<2> {
  static constexpr int EPS = 64;
  static constexpr int PPS = 32;
  static constexpr int CPS = 2;
};

// ------------------------------------------------------------ cross-workgroup
// Data handed from one workgroup to another inside a kernel is stored and
// loaded at agent scope (coherent across the XCDs' L2s); the hand-off is a
// vmcnt drain, a barrier and a relaxed agent-scope counter update.
template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_agent(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0): every load and store this wave issued has completed.
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ------------------------------------------------------------------ shuffles
__device__ __forceinline__ float sum_lanes(float v, int width) {
  for (int d = 1; d < width; d <<= 1) v += __shfl_xor(v, d);
  return v;
}
__device__ __forceinline__ double sum_lanes64(double v) {
  for (int d = 1; d < kWave; d <<= 1) v += __shfl_xor(v, d);
  return v;
}

// ------------------------------------------------------- activation prep
// Halfword slot and pre-scale exponent of element j of a prepared vector.
template <int BITS>
__device__ __forceinline__ void pair_slot(int j, int& half_idx, int& p) {
  if (BITS == 4) {
    const int seg = j >> 5, e = j & 31, d = e >> 3, r = e & 7, i = r & 3, hi = r >> 2;
    half_idx = ((seg * 16 + d * 4 + i) << 1) | hi;
    p = (i & 1) * 4;
  } else {
    const int seg = j >> 6, e = j & 63, d = e >> 4, r = e & 15, hi = r >> 3, i = r & 7;
    half_idx = ((seg * 32 + d * 8 + i) << 1) | hi;
    p = (i <= 4) ? 2 * i : 2 * (i - 5);
  }
}

// Prepare up to 8 blocks of 32 elements with one wave: lane L works on elements
// 4*(L&7) .. +3 of block (L>>3) of the wave's set.  Every lane of the wave must
// call this (cross-lane shuffles).  `blk` is the block index within the vector
// this lane group handles (or -1 for none), src points at the vector, dst at
// its prepared image (pairs then consts) and K is the vector length.
template <int BITS, bool AGENT>
__device__ __forceinline__ void prep_blocks(const float* src, uint8_t* dst, int K, int blk) {
  const int sub = threadIdx.x & 7;
  const bool ok = blk >= 0;
  float x[4] = {0.f, 0.f, 0.f, 0.f};
  if (ok) {
    const float* p = src + 32 * blk + 4 * sub;
    if (AGENT) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = ld_agent(p + e);
    } else {
      const float4 v = *reinterpret_cast<const float4*>(p);
      x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
  }
  float m = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  m = fmaxf(m, __shfl_xor(m, 4));
  int sh = 0;
  if (m > 0.f && m <= 3.402823466e38f) {
    int ex;
    frexpf(m, &ex);                       // m = f * 2^ex, f in [0.5, 1)
    sh = min(max(ex - 1 - 14, -100), 113);  // scaled block max in [2^14, 2^15)
  }
  uint16_t* halves = reinterpret_cast<uint16_t*>(dst);
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    int hidx, p;
    pair_slot<BITS>(32 * (ok ? blk : 0) + 4 * sub + e, hidx, p);
    const _Float16 h = (_Float16)ldexpf(x[e], -sh - p);
    if (ok) halves[hidx] = __builtin_bit_cast(uint16_t, h);
    const float hf = (float)h;
    s1 += hf;
    s2 += ldexpf(hf, p);
  }
  s1 += __shfl_xor(s1, 1);
  s1 += __shfl_xor(s1, 2);
  s1 += __shfl_xor(s1, 4);
  s2 += __shfl_xor(s2, 1);
  s2 += __shfl_xor(s2, 2);
  s2 += __shfl_xor(s2, 4);
  if (ok && sub == 0) {
    float4* consts = reinterpret_cast<float4*>(dst + 2 * (int64_t)K);
    consts[blk] = make_float4(ldexpf(1.f, sh), ldexpf(s1, 10 + sh), ldexpf(s2, sh), 0.f);
  }
}

// --------------------------------------------------------- segment products
// D = sum over the segment's codes of (1024 + q*2^p) * slot, one value per
// 32-element block (one for 4-bit, two for 2-bit).
template <int BITS>
__device__ __forceinline__ void seg_dot(const uint4& w, const uint32_t* xp, float* d);

template <>
__device__ __forceinline__ void seg_dot<4>(const uint4& w, const uint32_t* xp, float* d) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v0 = v[i], v1 = v0 >> 8;
    a = dot2((v0 & 0x000F000Fu) | kMagic, xp[4 * i + 0], a);
    b = dot2((v0 & 0x00F000F0u) | kMagic, xp[4 * i + 1], b);
    a = dot2((v1 & 0x000F000Fu) | kMagic, xp[4 * i + 2], a);
    b = dot2((v1 & 0x00F000F0u) | kMagic, xp[4 * i + 3], b);
  }
  d[0] = a + b;
}

template <>
__device__ __forceinline__ void seg_dot<2>(const uint4& w, const uint32_t* xp, float* d) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
  float acc[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v0 = v[i], v1 = v0 >> 10;
    float a = acc[i >> 1];
#pragma unroll
    for (int j = 0; j < 5; ++j) a = dot2((v0 & (0x00030003u << (2 * j))) | kMagic, xp[8 * i + j], a);
#pragma unroll
    for (int j = 0; j < 3; ++j)
      a = dot2((v1 & (0x00030003u << (2 * j))) | kMagic, xp[8 * i + 5 + j], a);
    acc[i >> 1] = a;
  }
  d[0] = acc[0];
  d[1] = acc[1];
}

// ------------------------------------------------------------- row tiles
// Row geometry of a packed matrix as seen by one wave.  S = 16-byte segments
// per row; LPR = lanes per row = min(S, 64); RPI = rows per wave iteration.
struct RowGeo {
  int S, LPR, RPI, lane_row, lane_seg;
  __device__ __forceinline__ RowGeo(int K, int bits) {
    S = K * bits / 128;
    LPR = S < kWave ? S : kWave;
    RPI = kWave / LPR;
    const int lane = threadIdx.x & (kWave - 1);
    lane_row = lane / LPR;
    lane_seg = lane % LPR;
  }
  __device__ __forceinline__ int seg(int j) const { return j * LPR + lane_seg; }
};

// Packed codes, scales and biases of the NS segments one lane reads from one row.
template <int BITS, int G, int SB, int NS>
struct Tile {
  static constexpr int GPS = (BITS == 2 && G == 32) ? 2 : 1;  // groups per segment
  uint4 q[NS];
  uint32_t s[NS][GPS], b[NS][GPS];  // raw stored bits (bf16 in the low half)

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      q[j] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int g = 0; g < GPS; ++g) { s[j][g] = 0; b[j][g] = 0; }
    }
  }

  // Row n of a matrix with K columns: codes at q0, scales at s0, biases at b0.
  __device__ __forceinline__ void load(const uint8_t* q0, const uint8_t* s0, const uint8_t* b0,
                                       int K, int64_t n, const RowGeo& geo) {
    const int64_t rb = (int64_t)K * BITS / 8;
    const int64_t ng = K / G;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int sg = geo.seg(j);
      q[j] = *reinterpret_cast<const uint4*>(q0 + n * rb + (int64_t)sg * 16);
      const int64_t gi = n * ng + (int64_t)sg * QF<BITS>::EPS / G;
      if (SB == 2) {
        if (GPS == 1) {
          s[j][0] = *reinterpret_cast<const uint16_t*>(s0 + 2 * gi);
          b[j][0] = *reinterpret_cast<const uint16_t*>(b0 + 2 * gi);
        } else {
          const uint32_t sv = *reinterpret_cast<const uint32_t*>(s0 + 2 * gi);
          const uint32_t bv = *reinterpret_cast<const uint32_t*>(b0 + 2 * gi);
          s[j][0] = sv & 0xFFFFu; s[j][GPS - 1] = sv >> 16;
          b[j][0] = bv & 0xFFFFu; b[j][GPS - 1] = bv >> 16;
        }
      } else {
#pragma unroll
        for (int g = 0; g < GPS; ++g) {
          s[j][g] = *reinterpret_cast<const uint32_t*>(s0 + 4 * (gi + g));
          b[j][g] = *reinterpret_cast<const uint32_t*>(b0 + 4 * (gi + g));
        }
      }
    }
  }
};

template <int SB>
__device__ __forceinline__ float sb_value(uint32_t raw) {
  return SB == 2 ? __uint_as_float(raw << 16) : __uint_as_float(raw);
}

// Prepared activations for the NS segments one lane works on.
template <int BITS, int NS>
struct XRegs {
  static constexpr int PPS = QF<BITS>::PPS, CPS = QF<BITS>::CPS;
  uint32_t p[NS][PPS];
  float P[NS][CPS], C[NS][CPS], A[NS][CPS];

  // src: prepared image of a K-vector (LDS or global).
  __device__ __forceinline__ void load(const uint8_t* src, int K, const RowGeo& geo) {
    const uint4* pr = reinterpret_cast<const uint4*>(src);
    const float4* cs = reinterpret_cast<const float4*>(src + 2 * (int64_t)K);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int sg = geo.seg(j);
#pragma unroll
      for (int v = 0; v < PPS / 4; ++v) {
        const uint4 u = pr[sg * (PPS / 4) + v];
        p[j][4 * v + 0] = u.x; p[j][4 * v + 1] = u.y;
        p[j][4 * v + 2] = u.z; p[j][4 * v + 3] = u.w;
      }
#pragma unroll
      for (int c = 0; c < CPS; ++c) {
        const float4 k4 = cs[sg * CPS + c];
        P[j][c] = k4.x; C[j][c] = k4.y; A[j][c] = k4.z;
      }
    }
  }
};

// This lane's share of sum_k deq(W)[n,k] * x_k for the row held in t.
template <int BITS, int G, int SB, int NS>
__device__ __forceinline__ float tile_dot(const Tile<BITS, G, SB, NS>& t, const XRegs<BITS, NS>& x) {
  constexpr int CPS = QF<BITS>::CPS, GPS = Tile<BITS, G, SB, NS>::GPS;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    float d[CPS];
    seg_dot<BITS>(t.q[j], x.p[j], d);
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      const int g = (GPS == 2) ? c : 0;
      const float s = sb_value<SB>(t.s[j][g]), b = sb_value<SB>(t.b[j][g]);
      const float u = fmaf(d[c], x.P[j][c], -x.C[j][c]);
      acc = fmaf(s, u, acc);
      acc = fmaf(b, x.A[j][c], acc);
    }
  }
  return acc;
}

__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

}  // namespace fmoe
