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
// kMagic in a VGPR: (codes & mask) | magic then takes one v_and_or_b32 (the
// mask in an SGPR) instead of an and and an or with two literals.
__device__ __forceinline__ uint32_t magic_v() {
  uint32_t m = kMagic;
  asm volatile("" : "+v"(m));
  return m;
}

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
// Weights are read once per layer: nontemporal loads keep them from evicting
// the kernel's code and the small hot data (activations, counters) from L2.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ld_nt(const float4* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) {
  return __builtin_nontemporal_load(p);
}

// tid_x() behind an empty asm: values derived from it are computed where
// they are used.  Persistent loops need this: otherwise the optimiser hoists
// every lane-dependent address and index of every path in front of the loop
// and keeps them all live in VGPRs across it.
__device__ __forceinline__ int tid_x() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load and store of the wave (its release fence
// covers all address spaces, and on this architecture one counter tracks
// loads and stores alike), which would stall weight loads issued well ahead
// of their use.  Global data handed to other waves or workgroups is published
// with an explicit vm_drain() first.
// The acquire side covers every address space (it costs no wait), so no
// later global access is moved above the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// s_waitcnt vmcnt(0): every load and store this wave issued has completed.
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ------------------------------------------------------------------ shuffles
// Cross-lane sums on DPP row operations (no LDS round trip).  After
// sum_lanes(v, width) the group total of each aligned group of `width` lanes
// (a power of two) is in the group's LAST lane; for width <= 16 every lane of
// the group holds it.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within 16 lanes
constexpr int kDppBcast15 = 0x142;     // lane 15 of row r -> row r+1
constexpr int kDppBcast31 = 0x143;     // lane 31 -> rows 2 and 3

__device__ __forceinline__ float sum_lanes(float v, int width) {
  if (width >= 2) v += dpp_f<kDppXor1>(v);
  if (width >= 4) v += dpp_f<kDppXor2>(v);
  if (width >= 8) v += dpp_f<kDppHalfMirror>(v);
  if (width >= 16) v += dpp_f<kDppMirror>(v);
  if (width >= 32) v += dpp_f<kDppBcast15, 0xA>(v);
  if (width >= 64) v += dpp_f<kDppBcast31, 0xC>(v);
  return v;
}
// Sum over the whole wave, returned in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                       __builtin_bit_cast(int, sum_lanes(v, kWave)), kWave - 1));
}
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  return fmaxf(v, dpp_f<kDppHalfMirror>(v));
}
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  return v + dpp_f<kDppHalfMirror>(v);
}
// fp64 sum over the wave on DPP row operations; the total lands in lane 63.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xF, true);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double sum_lanes_f64(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  v += dpp_f64<kDppBcast15, 0xA>(v);
  v += dpp_f64<kDppBcast31, 0xC>(v);
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

// LDS copies of prepared images are chunk-transposed: with S segments per
// row and C = PPS/4 16-byte chunks of slots per segment, chunk v of segment
// sg sits at chunk index v*S + sg, and constant chunk c of segment sg (CC per
// segment) at S*C + c*S + sg.  A wave then reads consecutive 16-byte chunks
// in consecutive lanes (no bank conflicts) where the linear layout (used in
// global memory) puts lanes 64 bytes apart.
template <int BITS, int CC>
__device__ __forceinline__ int lds_chunk(int g, int S) {
  constexpr int C = QF<BITS>::PPS / 4;
  if (g < S * C) {
    const int sg = g / C, v = g - sg * C;
    return v * S + sg;
  }
  const int h = g - S * C, sg = h / CC, c = h - sg * CC;
  return S * C + c * S + sg;
}

// Prepare blocks of 32 elements with one wave: lane L works on elements
// 4*(L&7) .. +3 of block `blk` (the same for the 8 lanes of a group, or -1 for
// none), whose values it already holds in x.  Every lane of the wave must call
// this (cross-lane operations).  dst is the prepared image of a K-vector
// (pairs, then consts), linear (global) or chunk-transposed (LDS_T, an LDS
// copy).  AGENT: other workgroups will read the image.
template <int BITS, bool AGENT, bool LDS_T = false>
__device__ __forceinline__ void prep_x4(const float4& xv, uint8_t* dst, int K, int blk) {
  const int sub = tid_x() & 7;
  const bool ok = blk >= 0;
  const float x[4] = {xv.x, xv.y, xv.z, xv.w};
  const float m = max8(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
  int sh = 0;
  if (m > 0.f && m <= 3.402823466e38f) {
    int ex;
    frexpf(m, &ex);                         // m = f * 2^ex, f in [0.5, 1)
    sh = min(max(ex - 1 - 14, -100), 113);  // scaled block max in [2^14, 2^15)
  }
  uint16_t* halves = reinterpret_cast<uint16_t*>(dst);
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    int hidx, p;
    pair_slot<BITS>(32 * (ok ? blk : 0) + 4 * sub + e, hidx, p);
    if (LDS_T) {
      const int dw = hidx >> 1, S = K * BITS / 128;
      hidx = (((lds_chunk<BITS, QF<BITS>::CPS>(dw >> 2, S)) << 2 | (dw & 3)) << 1) | (hidx & 1);
    }
    const _Float16 h = (_Float16)ldexpf(x[e], -sh - p);
    if (ok) {
      if (AGENT) st_agent(halves + hidx, __builtin_bit_cast(uint16_t, h));
      else halves[hidx] = __builtin_bit_cast(uint16_t, h);
    }
    const float hf = (float)h;
    s1 += hf;
    s2 += ldexpf(hf, p);
  }
  s1 = sum8(s1);
  s2 = sum8(s2);
  if (ok && sub == 0) {
    constexpr int CPS = QF<BITS>::CPS;
    const int S = K * BITS / 128;
    float* c = LDS_T ? reinterpret_cast<float*>(dst) +
                           4 * lds_chunk<BITS, CPS>(S * (QF<BITS>::PPS / 4) + blk, S)
                     : reinterpret_cast<float*>(dst + 2 * (int64_t)K) + 4 * blk;
    const float P = ldexpf(1.f, sh), C = ldexpf(s1, 10 + sh), A = ldexpf(s2, sh);
    if (AGENT) {
      st_agent(c + 0, P); st_agent(c + 1, C); st_agent(c + 2, A); st_agent(c + 3, 0.f);
    } else {
      *reinterpret_cast<float4*>(c) = make_float4(P, C, A, 0.f);
    }
  }
}

// The 4 values of block blk (>= 0) this lane prepares.
template <bool AGENT>
__device__ __forceinline__ float4 prep_load(const float* src, int blk) {
  const float* p = src + 32 * blk + 4 * (tid_x() & 7);
  if (AGENT) {
    const uint64_t lo = ld_agent(reinterpret_cast<const uint64_t*>(p));
    const uint64_t hi = ld_agent(reinterpret_cast<const uint64_t*>(p) + 1);
    return make_float4(__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                       __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32)));
  }
  return *reinterpret_cast<const float4*>(p);
}

// One wave-call prepares block blk (see prep_x4; -1: none), loading it first
// (block 0 is read in place of none, so the load is never predicated).
template <int BITS, bool AGENT>
__device__ __forceinline__ void prep_blocks(const float* src, uint8_t* dst, int K, int blk) {
  prep_x4<BITS, false>(prep_load<AGENT>(src, blk < 0 ? 0 : blk), dst, K, blk);
}

// The whole workgroup (NT threads) prepares nvec K-vectors (vector v at
// src + v*K, its chunk-transposed image at dst + v*xprep_bytes(K), in LDS);
// the loads of up to
// 8 passes are issued before any block is processed.  AGENT: the vectors were
// written by other workgroups of this launch.
template <int BITS, int NT, bool AGENT>
__device__ __forceinline__ void prep_vectors(const float* src, uint8_t* dst, int K, int nvec) {
  constexpr int kPer = NT / 8;   // blocks per pass
  constexpr int kBatch = 8;      // passes whose loads are issued together
  const int bpv = K / 32, nblk = bpv * nvec;
  const int64_t xb = 2 * (int64_t)K + (int64_t)(K / 32) * 16;
  for (int p0 = 0; p0 * kPer < nblk; p0 += kBatch) {
    float4 xv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int gb0 = (p0 + j) * kPer + (tid_x() >> 3);
      const int gb = gb0 < nblk ? gb0 : nblk - 1;   // clamped, never predicated
      const int v = gb / bpv;
      xv[j] = prep_load<AGENT>(src + (int64_t)v * K, gb - v * bpv);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if ((p0 + j) * kPer < nblk) {   // uniform over the workgroup
        const int gb = (p0 + j) * kPer + (tid_x() >> 3);
        const int v = gb < nblk ? gb / bpv : 0;
        prep_x4<BITS, false, true>(xv[j], dst + v * xb, K, gb < nblk ? gb - v * bpv : -1);
      }
    }
  }
}

template <int BITS, int NT, bool AGENT = false>
__device__ __forceinline__ void prep_vector(const float* src, uint8_t* dst, int K) {
  prep_vectors<BITS, NT, AGENT>(src, dst, K, 1);
}

// Copy n16 16-byte words into LDS with the workgroup; each thread issues its
// loads in batches of 4 before storing, so the round trips overlap.  Loads
// past the end read the last word (never a predicated load: predicated loads
// with their data used at once serialise on a wait each); only stores are
// predicated.  n16 >= 1.
__device__ __forceinline__ void copy_to_lds(uint4* dst, const uint4* src, int n16, int nthreads) {
  const int tid = tid_x();
  for (int base = 0; base < n16; base += 4 * nthreads) {
    uint4 t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + j * nthreads + tid;
      t[j] = src[i < n16 ? i : n16 - 1];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + j * nthreads + tid;
      if (i < n16) dst[i] = t[j];
    }
  }
}

// Same for data another workgroup of this launch wrote (agent-scope loads).
__device__ __forceinline__ void copy_to_lds_agent(uint64_t* dst, const uint64_t* src, int n8,
                                                  int nthreads) {
  const int tid = tid_x();
  for (int base = 0; base < n8; base += 8 * nthreads) {
    uint64_t t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * nthreads + tid;
      t[j] = ld_agent(src + (i < n8 ? i : n8 - 1));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * nthreads + tid;
      if (i < n8) dst[i] = t[j];
    }
  }
}

// A linear prepared image (K-vector, BITS-bit consumer, CC constant chunks per
// segment: QF<BITS>::CPS for xprep, 4 for word-blocked images) copied into LDS
// chunk-transposed; loads in batches of 4 (clamped), stores placed.
template <int BITS, int CC>
__device__ __forceinline__ void copy_image_to_lds(uint4* dst, const uint4* src, int K,
                                                  int nthreads) {
  const int S = K * BITS / 128;
  const int n16 = S * (QF<BITS>::PPS / 4 + CC);
  const int tid = tid_x();
  for (int base = 0; base < n16; base += 4 * nthreads) {
    uint4 t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + j * nthreads + tid;
      t[j] = src[i < n16 ? i : n16 - 1];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + j * nthreads + tid;
      if (i < n16) dst[lds_chunk<BITS, CC>(i, S)] = t[j];
    }
  }
}

// nimg word-blocked images (contiguous in global, written by other workgroups
// of this launch: agent-scope loads) copied into LDS chunk-transposed, image
// after image.  Every load is issued before any is stored: MAXIMG images of at
// most PER*NT 8-byte words each.  Only the pass count is a branch (uniform);
// image and word indices are clamped, so a lane past the end re-copies the
// last word to its own place.
template <int BITS, int NT, int MAXIMG, int PER>
__device__ __forceinline__ void copy_wimgs_to_lds_agent(uint64_t* dst, const uint64_t* src,
                                                        int K, int nimg) {
  const int S = K * BITS / 128;
  const int n8 = (2 * K + (K / (32 / BITS)) * 16) / 8;   // 8-byte words per image
  const int tid = tid_x();
  uint64_t t[MAXIMG][PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (j * NT < n8) {
      const int i = min(j * NT + tid, n8 - 1);
#pragma unroll
      for (int im = 0; im < MAXIMG; ++im)
        t[im][j] = ld_agent(src + (int64_t)min(im, nimg - 1) * n8 + i);
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (j * NT < n8) {
      const int i = min(j * NT + tid, n8 - 1);
      const int o = 2 * lds_chunk<BITS, 4>(i >> 1, S) + (i & 1);
#pragma unroll
      for (int im = 0; im < MAXIMG; ++im) dst[(int64_t)min(im, nimg - 1) * n8 + o] = t[im][j];
    }
  }
}

// --------------------------------------------------------- segment products
// D = sum over the segment's codes of (1024 + q*2^p) * slot, one value per
// 32-element block (one for 4-bit, two for 2-bit).
template <int BITS>
__device__ __forceinline__ void seg_dot(const uint4& w, const uint32_t* xp, float* d);

template <>
__device__ __forceinline__ void seg_dot<4>(const uint4& w, const uint32_t* xp, float* d) {
  const uint32_t mg = magic_v();
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v0 = v[i], v1 = v0 >> 8;
    a = dot2((v0 & 0x000F000Fu) | mg, xp[4 * i + 0], a);
    b = dot2((v0 & 0x00F000F0u) | mg, xp[4 * i + 1], b);
    a = dot2((v1 & 0x000F000Fu) | mg, xp[4 * i + 2], a);
    b = dot2((v1 & 0x00F000F0u) | mg, xp[4 * i + 3], b);
  }
  d[0] = a + b;
}

template <>
__device__ __forceinline__ void seg_dot<2>(const uint4& w, const uint32_t* xp, float* d) {
  const uint32_t mg = magic_v();
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
  float acc[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v0 = v[i], v1 = v0 >> 10;
    float a = acc[i >> 1];
#pragma unroll
    for (int j = 0; j < 5; ++j) a = dot2((v0 & (0x00030003u << (2 * j))) | mg, xp[8 * i + j], a);
#pragma unroll
    for (int j = 0; j < 3; ++j)
      a = dot2((v1 & (0x00030003u << (2 * j))) | mg, xp[8 * i + 5 + j], a);
    acc[i >> 1] = a;
  }
  d[0] = acc[0];
  d[1] = acc[1];
}

// ------------------------------------------------------------- row tiles
// Values the caller guarantees to be equal in every active lane, moved to
// SGPRs (a pointer keeps its global address space).
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ const uint8_t* uniform_gptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)uniform_i64((int64_t)reinterpret_cast<uint64_t>(p));
  return (const uint8_t*)((const __attribute__((address_space(1))) uint8_t*)v);
}

// Row geometry of a packed matrix as seen by one wave.  S = 16-byte segments
// per row; LPR = lanes per row = min(S, 64); RPI = rows per wave iteration.
struct RowGeo {
  int S, LPR, RPI, lane_row, lane_seg;
  __device__ __forceinline__ RowGeo(int K, int bits) {
    S = K * bits / 128;
    LPR = S < kWave ? S : kWave;
    RPI = kWave / LPR;
    const int lane = tid_x() & (kWave - 1);
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
  // n = (a row index that is the same in every lane) + geo.lane_row, and the
  // three pointers are the same in every lane: the row bases then live in
  // SGPRs and each load takes a 32-bit per-lane offset (no 64-bit VGPR
  // address per load).
  __device__ __forceinline__ void load(const uint8_t* q0, const uint8_t* s0, const uint8_t* b0,
                                       int K, int64_t n, const RowGeo& geo) {
    const int rb = K * BITS / 8;
    const int ng = K / G;
    const int64_t nu = uniform_i64(n - geo.lane_row);
    const uint8_t* qr = uniform_gptr(q0 + nu * rb);
    const uint8_t* sr = uniform_gptr(s0 + nu * ng * SB);
    const uint8_t* br = uniform_gptr(b0 + nu * ng * SB);
    const uint32_t lr = (uint32_t)geo.lane_row;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const uint32_t sg = (uint32_t)geo.seg(j);
      q[j] = ld_nt(reinterpret_cast<const uint4*>(qr + (lr * (uint32_t)rb + sg * 16u)));
      const uint32_t go = SB * (lr * (uint32_t)ng + sg * (uint32_t)QF<BITS>::EPS / (uint32_t)G);
      if (SB == 2) {
        if (GPS == 1) {
          s[j][0] = ld_nt(reinterpret_cast<const uint16_t*>(sr + go));
          b[j][0] = ld_nt(reinterpret_cast<const uint16_t*>(br + go));
        } else {
          const uint32_t sv = ld_nt(reinterpret_cast<const uint32_t*>(sr + go));
          const uint32_t bv = ld_nt(reinterpret_cast<const uint32_t*>(br + go));
          s[j][0] = sv & 0xFFFFu; s[j][GPS - 1] = sv >> 16;
          b[j][0] = bv & 0xFFFFu; b[j][GPS - 1] = bv >> 16;
        }
      } else {
#pragma unroll
        for (int g = 0; g < GPS; ++g) {
          s[j][g] = ld_nt(reinterpret_cast<const uint32_t*>(sr + go + 4u * g));
          b[j][g] = ld_nt(reinterpret_cast<const uint32_t*>(br + go + 4u * g));
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

  // src: chunk-transposed LDS copy of the prepared image of a K-vector.
  __device__ __forceinline__ void load(const uint8_t* src, int K, const RowGeo& geo) {
    const int S = geo.S;
    const uint4* pr = reinterpret_cast<const uint4*>(src);
    const float4* cs = reinterpret_cast<const float4*>(src) + S * (PPS / 4);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int sg = geo.seg(j);
#pragma unroll
      for (int v = 0; v < PPS / 4; ++v) {
        const uint4 u = pr[v * S + sg];
        p[j][4 * v + 0] = u.x; p[j][4 * v + 1] = u.y;
        p[j][4 * v + 2] = u.z; p[j][4 * v + 3] = u.w;
      }
#pragma unroll
      for (int c = 0; c < CPS; ++c) {
        const float4 k4 = cs[c * S + sg];
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

// ------------------------------------------------ word-blocked activations
// The same prepared form with one power-of-two scale per 32-bit code word
// (W = 32/BITS elements: 8 for 4-bit codes, 16 for 2-bit), so that a producer
// of W consecutive values can publish its block on its own.  A block's fp16
// slots are contiguous (W/2 pair dwords at dword index block*W/2) and its
// constants are the float4 {P, C, A, 0} at byte 2*K + 16*block.
//
// One lane per element: lanes L .. L+W-1 (L a multiple of W) hold the W
// values of block `blk` (element j = blk*W + lane%W); every lane of the wave
// calls this (cross-lane sums); `live` selects the lanes that hold a value.
// The image is written with agent-scope stores (read by other workgroups).
template <int BITS>
__device__ __forceinline__ void wimg_publish(float x, bool live, uint8_t* img, int K, int j) {
  constexpr int W = 32 / BITS;
  const float ax = live ? fabsf(x) : 0.f;
  float m = fmaxf(ax, dpp_f<kDppXor1>(ax));
  m = fmaxf(m, dpp_f<kDppXor2>(m));
  m = fmaxf(m, dpp_f<kDppHalfMirror>(m));
  if (W == 16) m = fmaxf(m, dpp_f<kDppMirror>(m));
  int sh = 0;
  if (m > 0.f && m <= 3.402823466e38f) {
    int ex;
    frexpf(m, &ex);                         // m = f * 2^ex, f in [0.5, 1)
    sh = min(max(ex - 1 - 14, -100), 113);  // scaled block max in [2^14, 2^15)
  }
  int hidx, p;
  pair_slot<BITS>(j, hidx, p);
  const _Float16 h = (_Float16)ldexpf(live ? x : 0.f, -sh - p);
  if (live) st_agent(reinterpret_cast<uint16_t*>(img) + hidx, __builtin_bit_cast(uint16_t, h));
  const float hf = (float)h;
  float s1 = hf, s2 = ldexpf(hf, p);
  s1 += dpp_f<kDppXor1>(s1);  s2 += dpp_f<kDppXor1>(s2);
  s1 += dpp_f<kDppXor2>(s1);  s2 += dpp_f<kDppXor2>(s2);
  s1 += dpp_f<kDppHalfMirror>(s1);  s2 += dpp_f<kDppHalfMirror>(s2);
  if (W == 16) { s1 += dpp_f<kDppMirror>(s1); s2 += dpp_f<kDppMirror>(s2); }
  if (live && j % W == 0) {
    float* c = reinterpret_cast<float*>(img + 2 * (int64_t)K) + 4 * (j / W);
    st_agent(c + 0, ldexpf(1.f, sh));
    st_agent(c + 1, ldexpf(s1, 10 + sh));
    st_agent(c + 2, ldexpf(s2, sh));
    st_agent(c + 3, 0.f);
  }
}

// D_w = sum over code word w's elements of (1024 + q*2^p) * slot, for the 4
// words of a 16-byte segment.
template <int BITS>
__device__ __forceinline__ void seg_dot_words(const uint4& w, const uint32_t* xp, float* d);

template <>
__device__ __forceinline__ void seg_dot_words<4>(const uint4& w, const uint32_t* xp, float* d) {
  const uint32_t mg = magic_v();
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v0 = v[i], v1 = v0 >> 8;
    float a = dot2((v0 & 0x000F000Fu) | mg, xp[4 * i + 0], 0.f);
    a = dot2((v0 & 0x00F000F0u) | mg, xp[4 * i + 1], a);
    a = dot2((v1 & 0x000F000Fu) | mg, xp[4 * i + 2], a);
    d[i] = dot2((v1 & 0x00F000F0u) | mg, xp[4 * i + 3], a);
  }
}

template <>
__device__ __forceinline__ void seg_dot_words<2>(const uint4& w, const uint32_t* xp, float* d) {
  const uint32_t mg = magic_v();
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v0 = v[i], v1 = v0 >> 10;
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < 5; ++j) a = dot2((v0 & (0x00030003u << (2 * j))) | mg, xp[8 * i + j], a);
#pragma unroll
    for (int j = 0; j < 3; ++j)
      a = dot2((v1 & (0x00030003u << (2 * j))) | mg, xp[8 * i + 5 + j], a);
    d[i] = a;
  }
}

// A word-blocked image's slots and constants for one lane's segment (one
// segment per lane: the down rows of the layer have at most 64 segments).
template <int BITS>
struct XRegsW {
  static constexpr int PPS = QF<BITS>::PPS;
  uint32_t p[PPS];
  float P[4], C[4], A[4];

  // src: chunk-transposed LDS copy of a word-blocked image.
  __device__ __forceinline__ void load(const uint8_t* src, int K, const RowGeo& geo) {
    const int S = geo.S;
    const uint4* pr = reinterpret_cast<const uint4*>(src);
    const float4* cs = reinterpret_cast<const float4*>(src) + S * (PPS / 4);
    const int sg = geo.seg(0);
#pragma unroll
    for (int v = 0; v < PPS / 4; ++v) {
      const uint4 u = pr[v * S + sg];
      p[4 * v + 0] = u.x; p[4 * v + 1] = u.y; p[4 * v + 2] = u.z; p[4 * v + 3] = u.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 k4 = cs[i * S + sg];
      P[i] = k4.x; C[i] = k4.y; A[i] = k4.z;
    }
  }
};

// This lane's share of sum_k deq(W)[n,k] * x_k for a one-segment row tile
// against a word-blocked image.
template <int BITS, int G, int SB>
__device__ __forceinline__ float tile_dot_w(const Tile<BITS, G, SB, 1>& t, const XRegsW<BITS>& x) {
  constexpr int GPS = Tile<BITS, G, SB, 1>::GPS;   // groups per segment
  float d[4];
  seg_dot_words<BITS>(t.q[0], x.p, d);
  float acc = 0.f;
#pragma unroll
  for (int g = 0; g < GPS; ++g) {
    float u = 0.f, as = 0.f;
#pragma unroll
    for (int i = g * 4 / GPS; i < (g + 1) * 4 / GPS; ++i) {
      u += fmaf(d[i], x.P[i], -x.C[i]);
      as += x.A[i];
    }
    acc = fmaf(sb_value<SB>(t.s[0][g]), u, acc);
    acc = fmaf(sb_value<SB>(t.b[0][g]), as, acc);
  }
  return acc;
}

// A one-segment 4-bit row tile whose codes are already fp16 pairs
// (1024 + q, magic-number form): a later product with a word-blocked image
// is dot2s only.  Made while the tile would otherwise sit idle in registers.
template <int G, int SB>
struct TileDq4 {
  static constexpr int GPS = Tile<4, G, SB, 1>::GPS;
  uint32_t h[16];
  uint32_t s[GPS], b[GPS];
  __device__ __forceinline__ void from(const Tile<4, G, SB, 1>& t) {
    const uint32_t mg = magic_v();
    const uint32_t v[4] = {t.q[0].x, t.q[0].y, t.q[0].z, t.q[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t v0 = v[i], v1 = v0 >> 8;
      h[4 * i + 0] = (v0 & 0x000F000Fu) | mg;
      h[4 * i + 1] = (v0 & 0x00F000F0u) | mg;
      h[4 * i + 2] = (v1 & 0x000F000Fu) | mg;
      h[4 * i + 3] = (v1 & 0x00F000F0u) | mg;
    }
    // Pin the pairs here: the compiler would otherwise recompute them at their
    // use, after the wait this conversion is meant to fill.
#pragma unroll
    for (int k = 0; k < 16; ++k) asm volatile("" : "+v"(h[k]));
#pragma unroll
    for (int g = 0; g < GPS; ++g) {
      s[g] = t.s[0][g];
      b[g] = t.b[0][g];
    }
  }
};

// tile_dot_w for a tile in fp16-pair form (same sums, same order).
template <int G, int SB>
__device__ __forceinline__ float tile_dot_w(const TileDq4<G, SB>& t, const XRegsW<4>& x) {
  constexpr int GPS = TileDq4<G, SB>::GPS;
  float d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = dot2(t.h[4 * i + 0], x.p[4 * i + 0], 0.f);
    a = dot2(t.h[4 * i + 1], x.p[4 * i + 1], a);
    a = dot2(t.h[4 * i + 2], x.p[4 * i + 2], a);
    d[i] = dot2(t.h[4 * i + 3], x.p[4 * i + 3], a);
  }
  float acc = 0.f;
#pragma unroll
  for (int g = 0; g < GPS; ++g) {
    float u = 0.f, as = 0.f;
#pragma unroll
    for (int i = g * 4 / GPS; i < (g + 1) * 4 / GPS; ++i) {
      u += fmaf(d[i], x.P[i], -x.C[i]);
      as += x.A[i];
    }
    acc = fmaf(sb_value<SB>(t.s[g]), u, acc);
    acc = fmaf(sb_value<SB>(t.b[g]), as, acc);
  }
  return acc;
}

}  // namespace fmoe
