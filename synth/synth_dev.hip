// synth_dev.hip -- device-side generator of synthetic expert slabs.
//
// Input generation only (no part of the MoE layer's arithmetic).  Implements
// the same definition as synth/__init__.py: SplitMix64 (Steele, Lea and Flood,
// OOPSLA 2014) used as a counter hash, word i of the stream keyed K being
// mix(K + (i+1) * 0x9E3779B97F4A7C15).  Packed code sections are the raw
// little-endian words; scales are lo + (hi - lo) * u in fp32 with every
// operation rounded separately, u = (word >> 40) * 2^-24; bf16 storage rounds
// to nearest-even; bias = bias_mult * (stored scale), rounded the same way.
// Padding between sections is written as zero, so a generated slab is
// byte-identical to the host's.
#include <hip/hip_runtime.h>
#include <stdint.h>

// Every fp32 operation of the scale rule is rounded on its own, as on the
// host: no multiply-add contraction anywhere in this file.
#pragma clang fp contract(off)

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t word(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * kGolden);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

struct Spec {
  int64_t off[9];
  int64_t qbytes[3];
  int64_t nsb[3];  // number of scale (= bias) entries per matrix
  int64_t slab_bytes;
  int sbytes;
  float lo, rng, bias_mult;
};

__device__ __forceinline__ void scale_bias(const Spec& sp, uint64_t w, float* s_out,
                                           float* b_out, uint32_t* s16, uint32_t* b16) {
  float u = __fmul_rn((float)(uint32_t)(w >> 40), 5.9604644775390625e-08f);  // 2^-24
  float s32 = __fadd_rn(sp.lo, __fmul_rn(sp.rng, u));
  if (sp.sbytes == 2) {
    uint32_t sb = bf16_rne(s32);
    float sw = __uint_as_float(sb << 16);
    uint32_t bb = bf16_rne(__fmul_rn(sw, sp.bias_mult));
    *s16 = sb;
    *b16 = bb;
  } else {
    *s_out = s32;
    *b_out = __fmul_rn(s32, sp.bias_mult);
  }
}

// One thread per 8-byte word of the slab range.
__global__ void fill_kernel(uint8_t* base, int64_t stride, int64_t first, int64_t count,
                            uint64_t seed, int32_t layer, Spec sp) {
  const int64_t words_per_slab = sp.slab_bytes / 8;
  const int64_t total = words_per_slab * count;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t si = t / words_per_slab;
    const int64_t byte = (t - si * words_per_slab) * 8;
    const uint64_t slab_id = (uint64_t)(first + si);
    uint64_t out = 0;
    for (int m = 0; m < 3; ++m) {
      const int64_t qo = sp.off[3 * m], so = sp.off[3 * m + 1], bo = sp.off[3 * m + 2];
      const int64_t sl = sp.nsb[m] * sp.sbytes;
      uint64_t kl = word(seed, (uint64_t)layer);
      uint64_t ks = word(kl, slab_id);
      if (byte >= qo && byte < qo + sp.qbytes[m]) {
        uint64_t key = word(ks, (uint64_t)(2 * m + 1));
        out = word(key, (uint64_t)((byte - qo) / 8));
      } else if ((byte >= so && byte < so + sl) || (byte >= bo && byte < bo + sl)) {
        const bool is_bias = byte >= bo;
        const int64_t rel = byte - (is_bias ? bo : so);
        uint64_t key = word(ks, (uint64_t)(2 * m + 2));
        const int per = 8 / sp.sbytes;
        for (int j = 0; j < per; ++j) {
          const int64_t e = rel / sp.sbytes + j;
          if (e >= sp.nsb[m]) break;
          float sf = 0.f, bf = 0.f;
          uint32_t s16 = 0, b16 = 0;
          scale_bias(sp, word(key, (uint64_t)e), &sf, &bf, &s16, &b16);
          if (sp.sbytes == 2) {
            out |= (uint64_t)(is_bias ? b16 : s16) << (16 * j);
          } else {
            out |= (uint64_t)__float_as_uint(is_bias ? bf : sf) << (32 * j);
          }
        }
      }
    }
    *reinterpret_cast<uint64_t*>(base + si * stride + byte) = out;
  }
}

int64_t round256(int64_t v) { return (v + 255) / 256 * 256; }

}  // namespace

extern "C" int synth_fill_slabs(void* base, int64_t stride, int64_t first, int64_t count,
                                uint64_t seed, int32_t layer, int32_t H, int32_t I,
                                int32_t bits, int32_t group, int32_t sbytes, float lo,
                                float hi, float bias_mult, void* stream) {
  Spec sp{};
  const int64_t rows[3] = {I, I, H}, cols[3] = {H, H, I};
  int64_t pos = 0;
  for (int m = 0; m < 3; ++m) {
    sp.qbytes[m] = rows[m] * cols[m] * bits / 8;
    sp.nsb[m] = rows[m] * (cols[m] / group);
    sp.off[3 * m] = pos;
    pos = round256(pos + sp.qbytes[m]);
    sp.off[3 * m + 1] = pos;
    pos = round256(pos + sp.nsb[m] * sbytes);
    sp.off[3 * m + 2] = pos;
    pos = round256(pos + sp.nsb[m] * sbytes);
  }
  sp.slab_bytes = pos;
  sp.sbytes = sbytes;
  sp.lo = lo;
  {
    volatile float vh = hi, vl = lo;  // hi - lo rounded once in fp32, as on the host
    sp.rng = vh - vl;
  }
  sp.bias_mult = bias_mult;
  if (stride < pos || stride % 8 != 0 || count <= 0) return -1;
  const int64_t total = pos / 8 * count;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)base, stride, first, count, seed, layer, sp);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}
