// fmoe_attention.hip -- decode attention of one new token over a bf16 KV cache,
// with the query's rotary embedding applied on the fly.
//
// [WAS] "3. Handoptimierte Metal Compute-Shader" lists GPU-side RoPE with the
// query de-interleaved and batched attention for the full-attention layers;
// the layer list names the products Q K^T, softmax and scores V.  Per sequence
// b and query head h (KV head h / G, G = NQ / NKV query heads per KV head):
//   q' = RoPE(q, len_b - 1)   (pairs (q[2i], q[2i+1]) rotated into (q'[i], q'[i + D/2]))
//   s_t = q' . K_t / sqrt(D),  p = softmax(s),  o = sum_t p_t V_t   (t < len_b)
//
// The cache dominates the bytes: 2 D bytes per position and KV head for K and
// for V.  A workgroup takes one KV head of one sequence and a chunk of 256
// positions, for all G <= 16 query heads that read that KV head, so the cache is
// read once per step:
//   - Q K^T is a [16 x D] x [D x 16] product per tile of 16 positions, on the
//     matrix cores (v_mfma_f32_16x16x32_bf16): the cache rows are the B operand
//     as stored (16 bytes per lane along D); the rotated query enters as two
//     bf16 halves (hi + lo, 16 significant bits) so that its rounding stays
//     below 2^-16 while K is exact;
//   - the chunk's softmax runs in LDS (max and sum per head);
//   - P V on the vector ALUs: a thread owns one column of V and accumulates
//     the G heads' weighted sums, the probabilities broadcast from LDS;
//   - the chunk's (max, sum, unnormalised output) go to the workspace, and a
//     second kernel merges the chunks of each head (flash-decoding split).
#include <math.h>

#include "fmoe_device.h"
#include "fmoe_internal.h"

namespace fmoe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
constexpr int kAtThreads = 256;
constexpr int kAtChunk = 128;     // positions per workgroup: 4 waves x kAtTiles tiles x 16
constexpr int kAtTiles = kAtChunk / 64;
constexpr int kAtHeads = 16;      // query heads per KV head (MFMA rows)

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;   // finite inputs
}
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Workspace: the rotated query of each (sequence, KV head) as matrix-core A
// operands ([B * NKV][D / 32][hi, lo][64 lanes] uint4), then per (sequence,
// KV head, chunk) the chunk's max and sum per head and its unnormalised output
// [16][D].
__host__ __device__ inline size_t at_part_floats(int D) { return 2 * kAtHeads + (size_t)kAtHeads * D; }
__host__ __device__ inline size_t at_qa_bytes(int B, int NKV, int D) {
  return ((size_t)B * NKV * (D / 32) * 2 * 64 * 16 + 255) / 256 * 256;
}

// One workgroup per (sequence, KV head): the rotation at position len - 1
// (angles in fp64, one pair per thread), then the rotated query heads of that
// KV head scaled by 1/sqrt(D) (zero rows past G), split into bf16 halves in
// the A-operand lane layout -- lane l holds head l % 16, d = 32 s + 8 (l / 16)
// + j -- each wave building k-steps s = wave, wave + 4, ...  q'[d] for d < D/2
// rotates pair (2d, 2d+1) into its first element, for d >= D/2 pair
// (2(d - D/2), ...) into its second.
template <int D>
__global__ __launch_bounds__(kAtThreads) void k_attn_qprep(AttnArgs p) {
  constexpr int KS = D / 32;
  __shared__ float2 s_cs[D / 2];
  const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
  const int bk = blockIdx.x, b = bk / p.NKV, kvh = bk - b * p.NKV;
  const int len = min(max(p.lens[b], 0), p.cap);
  for (int i = tid; i < D / 2; i += kAtThreads) {
    const double th = (double)max(len - 1, 0) * pow((double)p.base, -2.0 * (double)i / (double)D);
    double sn, cs;
    sincos(th, &sn, &cs);
    s_cs[i] = make_float2((float)cs, (float)sn);
  }
  __syncthreads();
  const int G = p.NQ / p.NKV, m = lane & 15, g = lane >> 4;
  const float scale = 1.f / sqrtf((float)D);
  const float* qh = p.q + ((size_t)b * p.NQ + (size_t)kvh * G + min(m, G - 1)) * D;
  uint4* qa = reinterpret_cast<uint4*>(p.ws) + (size_t)bk * KS * 2 * kWave;
  for (int s = wave; s < KS; s += kAtThreads / kWave) {
    uint32_t hw[8], lw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = 32 * s + 8 * g + j;
      const int i = d < D / 2 ? d : d - D / 2;
      const float2 xv = *reinterpret_cast<const float2*>(qh + 2 * i);
      const float2 r = s_cs[i];
      float v = d < D / 2 ? xv.x * r.x - xv.y * r.y : xv.x * r.y + xv.y * r.x;
      v = m < G ? v * scale : 0.f;
      hw[j] = bf16_bits_rne(v);
      lw[j] = bf16_bits_rne(v - bf16_to_f32(hw[j]));
    }
    qa[(s * 2 + 0) * kWave + lane] =
        make_uint4(hw[0] | hw[1] << 16, hw[2] | hw[3] << 16, hw[4] | hw[5] << 16, hw[6] | hw[7] << 16);
    qa[(s * 2 + 1) * kWave + lane] =
        make_uint4(lw[0] | lw[1] << 16, lw[2] | lw[3] << 16, lw[4] | lw[5] << 16, lw[6] | lw[7] << 16);
  }
}

// Workgroup (b * NKV + kvh) * nch + c.
template <int D>
__global__ __launch_bounds__(kAtThreads, 4) void k_attn_chunk(AttnArgs p) {
  constexpr int KS = D / 32;                  // MFMA k-steps over D
  constexpr int CG = D / 4;                   // P V column groups (4 columns each)
  constexpr int PG = kAtThreads / CG;         // P V position groups
  constexpr int PU = 8;                       // P V positions loaded ahead per thread
  __shared__ __align__(16) float s_p[kAtChunk][kAtHeads];   // scores, then probabilities
  __shared__ __align__(16) float s_red[kAtHeads][D];        // P V sums of one position group
  const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
  const int nch = (p.cap + kAtChunk - 1) / kAtChunk;
  const int c = blockIdx.x % nch;
  const int bk = blockIdx.x / nch;            // b * NKV + kvh
  const int b = bk / p.NKV, kvh = bk - b * p.NKV;
  const int len = min(max(p.lens[b], 0), p.cap);   // in bounds whatever the lengths hold
  const int p0 = c * kAtChunk;
  if (p0 >= len) return;                      // chunk past the sequence: the merge skips it
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(p.ws) + at_qa_bytes(p.B, p.NKV, D)) +
                ((size_t)bk * nch + c) * at_part_floats(D);
  const uint16_t* kbase = p.kc + (size_t)bk * p.cap * D;
  const uint16_t* vbase = p.vc + (size_t)bk * p.cap * D;

  // MFMA lanes: A operand row (query head) m = lane % 16, k sub-block g =
  // lane / 16 (d = 32 s + 8 g + j); B operand column: position lane % 16 of a
  // tile of 16, the same d.  The wave's first tile of cache rows is requested
  // before anything else (it does not depend on the query).
  const int m = lane & 15, g = lane >> 4;
  auto k_tile = [&](uint4 (&kv)[KS], int t) {
    const int pos = min(p0 + wave * 16 * kAtTiles + t * 16 + m, len - 1);   // rows past the end: the last row
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kv[s] = *reinterpret_cast<const uint4*>(kbase + (size_t)pos * D + 32 * s + 8 * g);
  };
  uint4 kv[KS];
  k_tile(kv, 0);

  // ---- this lane's A operands: the rotated query, prepared by k_attn_qprep
  const uint4* qa = reinterpret_cast<const uint4*>(p.ws) + (size_t)bk * KS * 2 * kWave;
  uint4 qhi[KS], qlo[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qhi[s] = qa[(s * 2 + 0) * kWave + lane];
    qlo[s] = qa[(s * 2 + 1) * kWave + lane];
  }

  // ---- Q K^T: the wave's 4 tiles, the next tile's rows in flight during the
  // current tile's products.
#pragma unroll
  for (int t = 0; t < kAtTiles; ++t) {
    uint4 kn[KS];
    if (t + 1 < kAtTiles) k_tile(kn, t + 1);
    f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qhi[s]),
                                                    __builtin_bit_cast(bf16x8, kv[s]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qlo[s]),
                                                    __builtin_bit_cast(bf16x8, kv[s]), acc, 0, 0, 0);
    }
    // D element i: head 4 g + i, position m of the tile
    const int pl = wave * 16 * kAtTiles + t * 16 + m;
#pragma unroll
    for (int i = 0; i < 4; ++i) s_p[pl][4 * g + i] = p0 + pl < len ? acc[i] : -INFINITY;
    if (t + 1 < kAtTiles) {
#pragma unroll
      for (int s = 0; s < KS; ++s) kv[s] = kn[s];
    }
  }
  __syncthreads();

  // ---- the first rows of V this thread sums are requested now (they do not
  // depend on the softmax)
  const int cg = tid % CG, pg = tid / CG;
  const int nvalid = min(kAtChunk, len - p0);
  auto v_rows = [&](uint2 (&vr)[PU], int j0) {
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const int j = min(j0 + u * PG, nvalid - 1);
      vr[u] = *reinterpret_cast<const uint2*>(vbase + (size_t)(p0 + j) * D + 4 * cg);
    }
  };
  uint2 vr[PU];
  v_rows(vr, pg);

  // ---- the chunk's softmax per head: 16 threads per head, kAtChunk / 16
  // positions each
  {
    constexpr int SP = kAtChunk / 16;
    const int h = tid >> 4, j0 = tid & 15;
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < SP; ++k) mx = fmaxf(mx, s_p[j0 + 16 * k][h]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < SP; ++k) {
      const float sc = s_p[j0 + 16 * k][h];
      const float e = sc == -INFINITY ? 0.f : expf(sc - mx);
      s_p[j0 + 16 * k][h] = e;
      sum += e;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o);
    if (j0 == 0) {
      part[h] = mx;
      part[kAtHeads + h] = sum;
    }
  }
  __syncthreads();

  // ---- P V: thread (column group cg: columns 4 cg .. 4 cg + 3, position group
  // pg: positions pg, pg + PG, ...), the next PU rows of V in flight while the
  // current PU are summed.
  float o[kAtHeads][4];
#pragma unroll
  for (int h = 0; h < kAtHeads; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) o[h][e] = 0.f;
  for (int j0 = pg; j0 < nvalid; j0 += PG * PU) {
    uint2 vn[PU];
    if (j0 + PG * PU < nvalid) v_rows(vn, j0 + PG * PU);   // the next batch in flight
#pragma unroll
    for (int u = 0; u < PU; ++u) {
      const int j = j0 + u * PG;
      if (j < nvalid) {
        const float v0 = bf16_to_f32(vr[u].x & 0xFFFFu), v1 = bf16_to_f32(vr[u].x >> 16);
        const float v2 = bf16_to_f32(vr[u].y & 0xFFFFu), v3 = bf16_to_f32(vr[u].y >> 16);
        const float4* pr = reinterpret_cast<const float4*>(&s_p[j][0]);
#pragma unroll
        for (int q4 = 0; q4 < kAtHeads / 4; ++q4) {
          const float4 pv = pr[q4];
          const float pw[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
          for (int hh = 0; hh < 4; ++hh) {
            float* oh = o[4 * q4 + hh];
            oh[0] = fmaf(pw[hh], v0, oh[0]);
            oh[1] = fmaf(pw[hh], v1, oh[1]);
            oh[2] = fmaf(pw[hh], v2, oh[2]);
            oh[3] = fmaf(pw[hh], v3, oh[3]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < PU; ++u) vr[u] = vn[u];
  }
  // position groups summed through LDS in group order; group 0 stores
  for (int r = 1; r < PG; ++r) {
    if (pg == r) {
#pragma unroll
      for (int h = 0; h < kAtHeads; ++h)
        *reinterpret_cast<float4*>(&s_red[h][4 * cg]) = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
    }
    __syncthreads();
    if (pg == 0) {
#pragma unroll
      for (int h = 0; h < kAtHeads; ++h) {
        const float4 v = *reinterpret_cast<const float4*>(&s_red[h][4 * cg]);
        o[h][0] += v.x; o[h][1] += v.y; o[h][2] += v.z; o[h][3] += v.w;
      }
    }
    __syncthreads();
  }
  if (pg == 0) {
    float* out = part + 2 * kAtHeads;
#pragma unroll
    for (int h = 0; h < kAtHeads; ++h)
      *reinterpret_cast<float4*>(out + (size_t)h * D + 4 * cg) =
          make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
  }
}

// One workgroup per (sequence, query head): merge the chunks.  The chunks'
// maxima, weights exp(m_c - M) and weighted sums go through LDS (one chunk per
// thread); each thread then sums its column over the chunks with the loads of
// 16 chunks in flight.
template <int D>
__global__ __launch_bounds__(kAtThreads) void k_attn_merge(AttnArgs p) {
  __shared__ float s_w[kAtThreads];
  __shared__ float s_r[kAtThreads / kWave];
  const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / p.NQ, h = blockIdx.x - b * p.NQ;
  const int G = p.NQ / p.NKV, kvh = h / G, m = h - kvh * G;
  const int nch = (p.cap + kAtChunk - 1) / kAtChunk;
  const int len = min(max(p.lens[b], 0), p.cap);
  const int nc = (len + kAtChunk - 1) / kAtChunk;   // 0 for an empty sequence: NaN output
  const float* base = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(p.ws) +
                                                    at_qa_bytes(p.B, p.NKV, D)) +
                      ((size_t)b * p.NKV + kvh) * nch * at_part_floats(D);
  // M: the maximum over every chunk
  float mx = -INFINITY;
  for (int c = tid; c < nc; c += kAtThreads) mx = fmaxf(mx, base[(size_t)c * at_part_floats(D) + m]);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) s_r[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_r[0], s_r[1]), fmaxf(s_r[2], s_r[3]));
  __syncthreads();
  float acc = 0.f, z = 0.f;
  for (int c0 = 0; c0 < nc; c0 += kAtThreads) {
    const int n = min(kAtThreads, nc - c0);
    float zw = 0.f;
    if (tid < n) {
      const float* pc = base + (size_t)(c0 + tid) * at_part_floats(D);
      const float w = expf(pc[m] - M);
      s_w[tid] = w;
      zw = w * pc[kAtHeads + m];
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) zw += __shfl_xor(zw, o);
    if (lane == 0) s_r[wave] = zw;
    __syncthreads();
    z += ((s_r[0] + s_r[1]) + s_r[2]) + s_r[3];
    if (tid < D) {
      const float* col = base + 2 * kAtHeads + (size_t)m * D + tid;
      int c = 0;
      for (; c + 16 <= n; c += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = col[(size_t)(c0 + c + u) * at_part_floats(D)];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc = fmaf(s_w[c + u], v[u], acc);
      }
      for (; c < n; ++c) acc = fmaf(s_w[c], col[(size_t)(c0 + c) * at_part_floats(D)], acc);
    }
    __syncthreads();
  }
  if (tid < D) p.out[((size_t)b * p.NQ + h) * D + tid] = acc / z;
}

template <int D>
hipError_t launch_d(const AttnArgs& p, hipStream_t st) {
  const int nch = (p.cap + kAtChunk - 1) / kAtChunk;
  const int64_t grid = (int64_t)p.B * p.NKV * nch;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attn_qprep<D>, dim3((unsigned)(p.B * p.NKV)), dim3(kAtThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_chunk<D>, dim3((unsigned)grid), dim3(kAtThreads), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_merge<D>, dim3((unsigned)(p.B * p.NQ)), dim3(kAtThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

bool attention_supported(int NQ, int NKV, int D) {
  return (D == 64 || D == 128 || D == 256) && NKV > 0 && NQ > 0 && NQ % NKV == 0 &&
         NQ / NKV <= kAtHeads;
}

size_t attention_ws_bytes(int B, int NKV, int D, int cap) {
  const size_t nch = ((size_t)cap + kAtChunk - 1) / kAtChunk;
  return at_qa_bytes(B, NKV, D) + (size_t)B * NKV * nch * at_part_floats(D) * sizeof(float);
}

hipError_t launch_attention(const AttnArgs& p, hipStream_t st) {
  if (!attention_supported(p.NQ, p.NKV, p.D)) return hipErrorNotSupported;
  if (p.B == 0) return hipSuccess;
  switch (p.D) {
    case 64: return launch_d<64>(p, st);
    case 128: return launch_d<128>(p, st);
    default: return launch_d<256>(p, st);
  }
}

}  // namespace fmoe
