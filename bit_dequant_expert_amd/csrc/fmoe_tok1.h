// fmoe_tok1.h -- the one-token MoE layer in one launch, with self-checking
// hand-off records.
//
// [HADA] "Deferred GPU Expert Compute" describes combine, norm and residual
// handed straight to the next layer with no host round trip, and [WAS]
// "3. Handoptimierte Metal Compute-Shader" fuses each step of the layer into a
// kernel.  On MI355X a one-token layer moves ~44 MB in a few microseconds, so
// it is bound by its chain of dependent memory round trips, not by bytes.  The
// mathematics imposes three grid-wide dependencies: every routed expert
// depends on all E logits (top-k), every down row on all I SwiGLU outputs of
// every active expert, every output on the sum of h^2 over the whole vector
// (RMSNorm).  Each of them is one round trip here:
//
//   A producer stores its result as 16-byte records whose last word is a check
//   word: the call's epoch xor a mix of the record's data words xor a salt.  A
//   consumer loads the records it needs with device-coherent loads and accepts
//   them when every check word matches; otherwise it sleeps briefly and loads
//   the failing records again.  A record left by an earlier call carries
//   another epoch and never passes, and one read half-written fails its mix.
//   The poll is the load of the data: no arrival counters, no drain of the
//   producer's stores ahead of a flag.
//
// Every wave's loads and stores complete in issue order, so the waves of a
// workgroup have fixed roles that keep each wave's queue free of what it does
// not wait for: wave 3 stores every record (a wave that polls never waits for
// its own stores), waves 0 and 1 poll, and waves 2 and 3 hold the down rows
// (their loads never sit in front of a poll).
//
// Workgroup b (all workgroups resident; the launcher checks occupancy):
//   phase A  all waves load x and a quarter of router row b; wave 3 also
//            loads the shared expert's gate and up rows n = 2b, 2b + 1.  x is
//            staged in LDS in fp32; the fp64 logit of row b, with a partial
//            dot product of the shared-gate row over x[b*H/E, (b+1)*H/E), goes
//            out as a record; then x is prepared as fp16 pairs for the gate/up
//            rows
//   phase B  wave 0 polls the E logit records and takes the top-k (one wave,
//            lower index on ties) and the shared gate, while wave 3 computes
//            the two shared SwiGLU values and publishes them; all waves load and
//            compute routed gate/up part b (expert slot b / (I/gu_rows)),
//            published as prepared fp16 blocks; waves 2-3 load the selected
//            experts' down rows right behind their gate/up rows
//   phase C  waves 0-1 poll the routed blocks and the shared SwiGLU values into
//            LDS images; waves 2-3 compute the down rows' dot products,
//            weighted by the routing weights and the shared gate, plus the
//            residual: h for the part's rows, and the part's sum of h^2
//   phase D  waves 0-1 poll every part's sum of h^2 and sum them in a fixed
//            order (the same bits in every workgroup); waves 2-3 write y
// Workgroup 0 finally stores the epoch, after its phase-D poll has seen every
// part's record (so every workgroup has read the epoch already).
//
// Every wait is bounded by a wall-clock limit.  A workgroup whose wait gives up
// sets the workspace's timeout word, publishes NaN in its later records and
// writes NaN outputs, so a call whose wait gave up cannot leave output that
// looks valid.
#pragma once

#include "fmoe_fused.h"

namespace fmoe {

// ------------------------------------------------------------- records
// Device-coherent 16-byte loads and stores of records through a raw buffer
// resource (out-of-range offsets read zeros instead of faulting).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kCpolDevice = 16;   // sc1: coherent at device scope (across XCDs)
__device__ __forceinline__ rsrc_t rec_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t rec_ld(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCpolDevice);
}
__device__ __forceinline__ void rec_st(rsrc_t r, uint32_t off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kCpolDevice);
}
__device__ __forceinline__ uint32_t rotl32(uint32_t v, int s) { return (v << s) | (v >> (32 - s)); }
// Check word of a record with data words d0, d1, d2.
__device__ __forceinline__ uint32_t rec_check(uint32_t ep, uint32_t d0, uint32_t d1, uint32_t d2,
                                              uint32_t salt) {
  return ep ^ salt ^ d0 ^ rotl32(d1, 7) ^ rotl32(d2, 19);
}
__device__ __forceinline__ bool rec_ok(const u32x4_t& r, uint32_t ep, uint32_t salt) {
  return rec_check(ep, r[0], r[1], r[2], salt) == r[3];
}
constexpr uint32_t kSaltLogit = 0x3C6EF372u;
constexpr uint32_t kSaltImg = 0xA54FF53Au;
constexpr uint32_t kSaltPart = 0x510E527Fu;
constexpr uint32_t kSaltShared = 0x1F83D9ABu;
// Records indexed by position carry the position in their salt.
__device__ __forceinline__ uint32_t pos_salt(uint32_t base, int i) {
  return base ^ ((uint32_t)i * 0x9E3779B1u);
}

// The record area's layout (kTok1*Off, kTok1AreaBytes) is in fmoe_fused_args.h.

// A routed SwiGLU block: the W = 32/BITS values of one code word of the down
// rows, prepared as in wimg_publish (fp16 slots with one power-of-two scale,
// and the block constants C and A).  Payload words: W/2 pair dwords, C, A;
// three per record; the last record's check word carries the scale exponent in
// its low byte (the check is compared on the upper 24 bits there).
template <int BITS>
struct ImgBlk {
  static constexpr int W = 32 / BITS;
  static constexpr int NPAY = W / 2 + 2;
  static constexpr int NCH = (NPAY + 2) / 3;   // 16-byte records per block
  static constexpr int BYTES = NCH * 16;
};

__device__ __forceinline__ uint64_t now_ticks() { return wall_clock64(); }

// Phase trace of the FMOE_TRACE build: one thread of each workgroup stamps the
// 100 MHz wall clock at phase boundaries (events listed at their marks).
#ifdef FMOE_TRACE
#define TOK1_MARK_W(ev, w)                                                             \
  do {                                                                                 \
    if (tid_x() == 64 * (w) && a.trace) a.trace[blockIdx.x * kTok1TraceEvents + (ev)] = wall_clock64(); \
  } while (0)
#else
#define TOK1_MARK_W(ev, w) do {} while (0)
#endif
#define TOK1_MARK(ev) TOK1_MARK_W(ev, 0)

// Shared state of one workgroup.
struct Tok1Shared {
  int sel[16];
  float coef[17];     // shared gate, then the routing weights
  int fail;
  double rp[kFusedWaves];
  double gp[kFusedWaves];
  float act[kWave];
  float part[kFusedWaves];
  uint32_t pay[2][16];  // block payload assembly (two blocks per part at most; word 15: exponent)
};

// --------------------------------------------------------------- helpers
// Publishes the SwiGLU block(s) of a gate/up part from one wave: lanes
// 0 .. nrows-1 hold the part's values (rows n0 ..); block n0/W + i goes to
// record (slot, block).  NaN payloads if the workgroup's inputs were invalid.
template <int BITS>
__device__ __forceinline__ void publish_blocks(float v, int nrows, int n0, int slot, int I,
                                               const rsrc_t& rimg, uint32_t ep, bool poison,
                                               Tok1Shared& sh) {
  using B = ImgBlk<BITS>;
  constexpr int W = B::W;
  const int lane = tid_x() & 63;
  const bool live = lane < nrows;
  const float x = poison ? __builtin_nanf("") : v;
  // block max -> scale exponent (groups of W lanes)
  const float ax = live ? fabsf(x) : 0.f;
  float m = fmaxf(ax, dpp_f<kDppXor1>(ax));
  m = fmaxf(m, dpp_f<kDppXor2>(m));
  m = fmaxf(m, dpp_f<kDppHalfMirror>(m));
  if (W == 16) m = fmaxf(m, dpp_f<kDppMirror>(m));
  int s = 0;
  if (m > 0.f && m <= 3.402823466e38f) {
    int ex;
    frexpf(m, &ex);
    s = min(max(ex - 1 - 14, -100), 113);   // scaled block max in [2^14, 2^15)
  }
  int hidx, p;
  pair_slot<BITS>(n0 + lane, hidx, p);      // half index within the whole image
  const _Float16 h = (_Float16)ldexpf(live ? x : 0.f, -s - p);
  const float hf = (float)h;
  float s1 = hf, s2 = ldexpf(hf, p);
  s1 += dpp_f<kDppXor1>(s1);  s2 += dpp_f<kDppXor1>(s2);
  s1 += dpp_f<kDppXor2>(s1);  s2 += dpp_f<kDppXor2>(s2);
  s1 += dpp_f<kDppHalfMirror>(s1);  s2 += dpp_f<kDppHalfMirror>(s2);
  if (W == 16) { s1 += dpp_f<kDppMirror>(s1); s2 += dpp_f<kDppMirror>(s2); }
  // The block's halves into the payload scratch (dword (hidx/2) mod W/2).
  const int bi = lane / W;                   // block of this part (0 or 1)
  uint16_t* halves = reinterpret_cast<uint16_t*>(&sh.pay[bi & 1][0]);
  if (live) halves[hidx % W] = __builtin_bit_cast(uint16_t, h);
  if (live && lane % W == 0) {
    sh.pay[bi & 1][W / 2] = __float_as_uint(ldexpf(s1, 10 + s));
    sh.pay[bi & 1][W / 2 + 1] = __float_as_uint(ldexpf(s2, s));
    sh.pay[bi & 1][15] = (uint32_t)((s + 128) & 0xFF);   // the scale exponent
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  // Lane c < nblk*NCH writes record c % NCH of block c / NCH.
  const int nblk = nrows / W;
  const int c = lane % B::NCH, blk = lane / B::NCH;
  if (blk < nblk) {
    const uint32_t* pw = &sh.pay[blk & 1][0];
    const uint32_t d0 = 3 * c < B::NPAY ? pw[3 * c] : 0u;
    const uint32_t d1 = 3 * c + 1 < B::NPAY ? pw[3 * c + 1] : 0u;
    const uint32_t d2 = 3 * c + 2 < B::NPAY ? pw[3 * c + 2] : 0u;
    uint32_t chk = rec_check(ep, d0, d1, d2, kSaltImg + c);
    if (c == B::NCH - 1) chk = (chk & 0xFFFFFF00u) | pw[15];
    const int gblk = n0 / W + blk;
    const uint32_t off = (uint32_t)((slot * (I / W) + gblk) * B::BYTES + c * 16);
    rec_st(rimg, off, u32x4_t{d0, d1, d2, chk});
  }
}

// Polls the routed SwiGLU blocks of slots [s0, s0 + ns) into word-blocked,
// chunk-transposed LDS images (as XRegsW reads them), image i at lds_ap +
// (lds_first + i) * ib.  Called by NT threads (thread index t); each wave
// retries only its own failing blocks.  Returns false if the wait gave up.
template <int BITS, int NT>
__device__ __forceinline__ bool poll_images(uint8_t* lds_ap, int lds_first, const rsrc_t& rimg,
                                            int I, int s0, int ns, uint32_t ep, uint64_t limit,
                                            int t) {
  using B = ImgBlk<BITS>;
  constexpr int W = B::W, PPS = QF<BITS>::PPS;
  const int S = I * BITS / 128;
  const int nb = I / W;                       // blocks per image
  const int total = ns * nb;
  const int64_t ib = wimg_bytes(I, BITS);
  // One block per thread a pass: polls in small rounds finish sooner than one
  // round over every block (a poll's cost grows with the records it reads).
  constexpr int kPer = 1;                     // blocks per thread per pass
  bool ok_all = true;
  for (int base = 0; base < total; base += kPer * NT) {
    bool done[kPer];
    u32x4_t r[kPer][B::NCH];
#pragma unroll
    for (int j = 0; j < kPer; ++j) done[j] = base + j * NT + t >= total;
    const uint64_t t0 = now_ticks();
    for (;;) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int g = min(base + j * NT + t, total - 1);
        const int sl = g / nb, blk = g - sl * nb;
        const uint32_t off = (uint32_t)(((s0 + sl) * nb + blk) * B::BYTES);
        if (!done[j]) {
#pragma unroll
          for (int c = 0; c < B::NCH; ++c) r[j][c] = rec_ld(rimg, off + 16 * c);
        }
      }
      bool pending = false;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (done[j]) continue;
        bool ok = true;
#pragma unroll
        for (int c = 0; c < B::NCH; ++c) {
          const uint32_t chk = rec_check(ep, r[j][c][0], r[j][c][1], r[j][c][2], kSaltImg + c);
          ok &= c == B::NCH - 1 ? ((chk ^ r[j][c][3]) & 0xFFFFFF00u) == 0 : chk == r[j][c][3];
        }
        if (!ok) { pending = true; continue; }
        done[j] = true;
        const int g = base + j * NT + t;
        const int sl = g / nb, blk = g - sl * nb;
        uint32_t pw[B::NCH * 3];
#pragma unroll
        for (int c = 0; c < B::NCH; ++c) {
          pw[3 * c] = r[j][c][0]; pw[3 * c + 1] = r[j][c][1]; pw[3 * c + 2] = r[j][c][2];
        }
        const int sh = (int)(r[j][B::NCH - 1][3] & 0xFFu) - 128;
        uint8_t* img = lds_ap + (lds_first + sl) * ib;
        // pair chunks of this block, then its constants {P, C, A, 0}
#pragma unroll
        for (int v = 0; v < W / 8; ++v) {
          const int lin = blk * (W / 8) + v;
          reinterpret_cast<uint4*>(img)[lds_chunk<BITS, 4>(lin, S)] =
              make_uint4(pw[4 * v], pw[4 * v + 1], pw[4 * v + 2], pw[4 * v + 3]);
        }
        reinterpret_cast<float4*>(img)[lds_chunk<BITS, 4>(S * (PPS / 4) + blk, S)] =
            make_float4(ldexpf(1.f, sh), __uint_as_float(pw[W / 2]),
                        __uint_as_float(pw[W / 2 + 1]), 0.f);
      }
      if (!__any(pending)) break;
      if (now_ticks() - t0 > limit) { ok_all = false; break; }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return ok_all;
}

// Polls the shared expert's I/2 SwiGLU records (two fp32 values each) into an
// fp32 staging area of LDS.  NT threads, thread index t.
template <int NT>
__device__ __forceinline__ bool poll_shared(float* stage, const rsrc_t& rsh, int I, uint32_t ep,
                                            uint64_t limit, int t) {
  constexpr int kPer = 1;
  const int n = I / 2;
  bool ok_all = true;
  for (int base = 0; base < n; base += kPer * NT) {
    bool done[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) done[j] = base + j * NT + t >= n;
    const uint64_t t0 = now_ticks();
    for (;;) {
      u32x4_t r[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = min(base + j * NT + t, n - 1);
        if (!done[j]) r[j] = rec_ld(rsh, (uint32_t)(16 * i));
      }
      bool pending = false;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (done[j]) continue;
        const int i = base + j * NT + t;
        if (!rec_ok(r[j], ep, pos_salt(kSaltShared, i))) { pending = true; continue; }
        done[j] = true;
        reinterpret_cast<float2*>(stage)[i] = make_float2(__uint_as_float(r[j][0]),
                                                          __uint_as_float(r[j][1]));
      }
      if (!__any(pending)) break;
      if (now_ticks() - t0 > limit) { ok_all = false; break; }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return ok_all;
}

// Builds the word-blocked, chunk-transposed LDS image of I fp32 values (the
// same form wimg_publish publishes): one thread per block of W values.
template <int BITS, int NT>
__device__ __forceinline__ void image_from_f32(uint8_t* img, const float* stage, int I, int t) {
  constexpr int W = 32 / BITS, PPS = QF<BITS>::PPS;
  const int S = I * BITS / 128;
  const int nb = I / W;
  for (int blk = t; blk < nb; blk += NT) {
    float v[W];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < W; ++j) {
      v[j] = stage[blk * W + j];
      m = fmaxf(m, fabsf(v[j]));
    }
    int s = 0;
    if (m > 0.f && m <= 3.402823466e38f) {
      int ex;
      frexpf(m, &ex);
      s = min(max(ex - 1 - 14, -100), 113);   // scaled block max in [2^14, 2^15)
    }
    uint32_t pairs[W / 2];
#pragma unroll
    for (int j = 0; j < W / 2; ++j) pairs[j] = 0u;
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int j = 0; j < W; ++j) {
      int hidx, p;
      pair_slot<BITS>(blk * W + j, hidx, p);
      const _Float16 h = (_Float16)ldexpf(v[j], -s - p);
      const int q = hidx % W;
      pairs[q >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, h) << (16 * (q & 1));
      const float hf = (float)h;
      s1 += hf;
      s2 += ldexpf(hf, p);
    }
#pragma unroll
    for (int v8 = 0; v8 < W / 8; ++v8)
      reinterpret_cast<uint4*>(img)[lds_chunk<BITS, 4>(blk * (W / 8) + v8, S)] =
          make_uint4(pairs[4 * v8], pairs[4 * v8 + 1], pairs[4 * v8 + 2], pairs[4 * v8 + 3]);
    reinterpret_cast<float4*>(img)[lds_chunk<BITS, 4>(S * (PPS / 4) + blk, S)] =
        make_float4(ldexpf(1.f, s), ldexpf(s1, 10 + s), ldexpf(s2, s), 0.f);
  }
}

// The top-k of the E logit records by one wave (lane l holds records l + 64 v),
// lower index on ties; weights = softmax over the selected logits.  Each
// record also carries a partial dot product of the shared-gate row; their sum
// (per lane in record order, then across the wave: the same order in every
// workgroup) gives the shared gate sigmoid(wsg . x) in sh.coef[0].  Returns
// false if the wait for the records gave up (the selection is then made from
// whatever the records hold, still a valid set of indices).
template <int VW>
__device__ __forceinline__ bool topk_wave(const rsrc_t& rlog, int E, int k, uint32_t ep,
                                          uint64_t limit, Tok1Shared& sh) {
  const int lane = tid_x() & 63;
  uint64_t key[VW];
  float gp[VW];
  bool done[VW];
#pragma unroll
  for (int v = 0; v < VW; ++v) {
    done[v] = lane + 64 * v >= E;
    key[v] = 0ull;
    gp[v] = 0.f;
  }
  bool ok_all = true;
  const uint64_t t0 = now_ticks();
  for (;;) {
    u32x4_t r[VW];
#pragma unroll
    for (int v = 0; v < VW; ++v) {
      const int e = min(lane + 64 * v, E - 1);
      if (!done[v]) r[v] = rec_ld(rlog, (uint32_t)(16 * e));
    }
    bool pending = false;
#pragma unroll
    for (int v = 0; v < VW; ++v) {
      if (done[v]) continue;
      const int e = lane + 64 * v;
      if (!rec_ok(r[v], ep, pos_salt(kSaltLogit, e))) {
        pending = true;
        continue;
      }
      done[v] = true;
      key[v] = order_key(__longlong_as_double((long long)(((uint64_t)r[v][1] << 32) | r[v][0])));
      gp[v] = __uint_as_float(r[v][2]);
    }
    if (!__any(pending)) break;
    if (now_ticks() - t0 > limit) { ok_all = false; break; }
    __builtin_amdgcn_s_sleep(1);
  }
  double gsum = 0.0;
#pragma unroll
  for (int v = 0; v < VW; ++v) gsum += (double)gp[v];
  gsum = sum_lanes_f64(gsum);
  const double gl = readlane_f64(gsum, kWave - 1);
  // k rounds of a wave maximum: high halves first, full keys among ties, then
  // the lowest index among equal keys.
  __builtin_assume(k >= 1);
  __builtin_assume(k <= 16);
  double l0 = 0.0;
  float ex_own = 0.f;
  int rank_own = -1;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
    int bv = 0;
#pragma unroll
    for (int v = 0; v < VW; ++v)
      if (key[v] > best) { best = key[v]; bv = v; }
    const uint32_t hi = (uint32_t)(best >> 32);
    const uint32_t mh = wave_max_u32(hi);
    uint64_t ball = __ballot(hi == mh);
    if (__popcll(ball) != 1) {
      const uint32_t ml = wave_max_u32(hi == mh ? (uint32_t)best : 0u);
      ball = __ballot(best == (((uint64_t)mh << 32) | ml));
      if (__popcll(ball) != 1) {   // equal keys: the lowest index wins
        const uint32_t cand = best == (((uint64_t)mh << 32) | ml) ? (uint32_t)(lane + 64 * bv)
                                                                    : 0xFFFFFFFFu;
        const uint32_t mi = ~wave_max_u32(~cand);
        ball = __ballot(cand == mi);
      }
    }
    const int L = __ffsll((unsigned long long)ball) - 1;
    const int we = __builtin_amdgcn_readlane(lane + 64 * bv, L);
    const uint64_t wk = ((uint64_t)mh << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)best, L);
#pragma unroll
    for (int v = 0; v < VW; ++v)
      if (lane == L && v == bv) key[v] = 0ull;
    const double lv = key_value(wk);
    if (r == 0) l0 = lv;
    if (lane == r) {
      rank_own = we;
      ex_own = expf((float)(lv - l0));
    }
  }
  const float z = wave_sum(lane < k ? ex_own : 0.f);
  if (lane < k) {
    sh.sel[lane] = rank_own;
    sh.coef[1 + lane] = ex_own / z;
  }
  if (lane == 0) sh.coef[0] = 1.f / (1.f + expf(-(float)gl));
  return ok_all;
}

// A held tile behind an empty asm: the unpack of its codes stays where the
// tile is used (the compiler would otherwise unpack every held tile at once,
// ahead of the first use, and run out of registers).
template <int BITS, int G, int SB>
__device__ __forceinline__ void pin_tile(Tile<BITS, G, SB, 1>& t) {
  asm volatile("" : "+v"(t.q[0].x), "+v"(t.q[0].y), "+v"(t.q[0].z), "+v"(t.q[0].w));
}

// ------------------------------------------------------------------ kernel
template <int BITS, int G, int SB, int NSH, int VW>
__global__ __launch_bounds__(kThreads, 2) void k_layer1t(const float* __restrict__ x_in,
                                                         const float* __restrict__ wr_in,
                                                         uint8_t* area_in,
                                                         const float* __restrict__ wsg_in,
                                                         const uint8_t* __restrict__ slabs_in,
                                                         Tok1Args a) {
  // The five pointers the first loads need come as separate parameters (the
  // hardware preloads leading parameters into scalar registers at launch);
  // they equal a.x, a.Wr, a.area, a.wsg and a.slabs.
  a.x = x_in;
  a.Wr = wr_in;
  a.area = area_in;
  a.wsg = wsg_in;
  a.slabs = slabs_in;
  // LDS: [x fp32 | x prepared | images (kFusedMaxSlots)]; the shared SwiGLU
  // values are staged in the x fp32 area once the router no longer needs it.
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ Tok1Shared sh;
  using TileH = Tile<BITS, G, SB, NSH>;
  using TileI = Tile<BITS, G, SB, 1>;
  constexpr int kUG = fused_ug(NSH);
  constexpr int kQ = 8 * NSH / BITS;    // float4 of x per thread, and of a router quarter row per lane
  constexpr int W = 32 / BITS;
  constexpr int kUD = 2;                // down row iterations of each of waves 2-3
  const int tid = tid_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool poller = wave < 2, holder = wave >= 2, writer_wave = wave == 3;
  const int b = blockIdx.x, nwg = gridDim.x;
  const int H = a.H, I = a.I, E = a.E, k = a.k, kp1 = k + 1;
  float* lds_x = reinterpret_cast<float*>(lds);
  uint8_t* lds_xp = lds + (int64_t)H * 4;
  uint8_t* lds_ap = lds_xp + xprep_bytes(H);
  const int64_t ib = wimg_bytes(I, BITS);
  const RowGeo geoH(H, BITS), geoI(I, BITS);
  const rsrc_t rlog = rec_rsrc(a.area + kTok1LogitOff, (uint32_t)(16 * E));
  const rsrc_t rsh = rec_rsrc(a.area + kTok1SharedOff, (uint32_t)(16 * (I / 2)));
  const rsrc_t rpart = rec_rsrc(a.area + kTok1PartOff, (uint32_t)(16 * a.nD));
  const rsrc_t rimg = rec_rsrc(a.area + kTok1ImgOff,
                               (uint32_t)(kp1 * (I / W) * ImgBlk<BITS>::BYTES));
  int* epoch_word = reinterpret_cast<int*>(a.area);
  if (tid == 0) sh.fail = 0;
  TOK1_MARK(0);   // entry

  // ---------------------------------------------------------------- phase A
  // Every load here is issued on every path (indices clamped), so that each
  // wait below counts exactly the loads issued after the one it waits for.
  float4 xq[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) xq[q] = reinterpret_cast<const float4*>(a.x)[q * kThreads + tid];
  const int ep_raw = ld_agent(epoch_word);
  auto router_load = [&](float4 (&wv)[kQ], int e) {
    const float4* row = reinterpret_cast<const float4*>(a.Wr + (int64_t)e * H);
    const int q0 = wave * (H / 16) + lane;
#pragma unroll
    for (int q = 0; q < kQ; ++q) wv[q] = ld_nt(row + q0 + q * 64);
  };
  auto gate_slice = [&](int e, int& lo, int& hi) {
    lo = (int)((int64_t)e * H / E);
    hi = (int)((int64_t)(e + 1) * H / E);
  };
  float4 wv[kQ];
  router_load(wv, min(b, E - 1));
  int glo, ghi;
  gate_slice(min(b, E - 1), glo, ghi);
  const float wsg_v = a.wsg[min(glo + tid, H - 1)];   // used where glo + tid < ghi
  // The shared expert's rows 2 sp and 2 sp + 1 (gate and up of each), for
  // shared pairs sp = b, b + nwg, ..., are wave 3's alone: it computes both
  // SwiGLU values and publishes them with no workgroup barrier, while wave 0
  // polls the logits.
  const int n_sp = I / 2;
  TileH ts[2][2];   // wave 3: [row 2 sp + r][gate, up]
  auto shared_load = [&](int sp) {
    const uint8_t* base = a.slabs + (int64_t)E * a.stride;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int m = 0; m < 2; ++m)
        ts[r][m].load(base + a.off[3 * m], base + a.off[3 * m + 1], base + a.off[3 * m + 2], H,
                      2 * sp + r, geoH);
  };
  if (writer_wave) shared_load(min(b, n_sp - 1));
  TOK1_MARK(14);   // phase A loads issued
  // Down rows of part b held by waves 2-3: rows b*d_rows + (w-2)*kUD*RPI +
  // u*RPI + lane_row (u < kUD).
  const bool has_d = b < a.nD;
  int drow[kUD];
#pragma unroll
  for (int u = 0; u < kUD; ++u)
    drow[u] = (has_d ? b : 0) * a.d_rows + (holder ? wave - 2 : 0) * kUD * geoI.RPI +
              u * geoI.RPI + geoI.lane_row;
  auto down_tile = [&](TileI& t, int64_t e, int u) {
    const uint8_t* base = a.slabs + e * a.stride;
    t.load(base + a.off[6], base + a.off[7], base + a.off[8], I, drow[u], geoI);
  };
  TileI td[kFusedMaxSlots][kUD];

  // x to LDS in fp32 for the router first; its fp16 preparation for the
  // gate/up rows follows the logit (it is not on the routing's path).
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    reinterpret_cast<float4*>(lds_x)[q * kThreads + tid] = xq[q];
    if (q == 0) TOK1_MARK(15);   // x (first quarter) in registers
  }
  lds_barrier();
  TOK1_MARK(1);   // x staged (fp32)

  uint32_t ep = (uint32_t)__builtin_amdgcn_readfirstlane(ep_raw) + 1u;
  ep &= 0x7FFFFFFFu;
  if (ep == 0) ep = 1;
  // Router rows b, b + nwg, ... below E; row e also carries the partial
  // shared-gate dot over x[e*H/E, (e+1)*H/E).
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
      for (int j = lo + kThreads + tid; j < hi; j += kThreads)   // long slices (few experts)
        gacc = fma((double)a.wsg[j], (double)lds_x[j], gacc);
    } else {
      for (int j = lo + tid; j < hi; j += kThreads) gacc = fma((double)a.wsg[j], (double)lds_x[j], gacc);
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
      const double l = ((sh.rp[0] + sh.rp[1]) + sh.rp[2]) + sh.rp[3];
      const float gsl = (float)(((sh.gp[0] + sh.gp[1]) + sh.gp[2]) + sh.gp[3]);
      const uint64_t bits = (uint64_t)__double_as_longlong(l);
      const uint32_t w0 = (uint32_t)bits, w1 = (uint32_t)(bits >> 32), w2 = __float_as_uint(gsl);
      rec_st(rlog, (uint32_t)(16 * e),
             u32x4_t{w0, w1, w2, rec_check(ep, w0, w1, w2, pos_salt(kSaltLogit, e))});
    }
    lds_barrier();   // sh.rp is reused
  }
  TOK1_MARK(2);   // logit records stored

#pragma unroll
  for (int q = 0; q < kQ; ++q) prep_x4<BITS, false, true>(xq[q], lds_xp, H, q * (kThreads / 8) + tid / 8);
  lds_barrier();   // x prepared

  // ---------------------------------------------------------------- phase B
  // Wave 0 polls the logits and takes the top-k; wave 3 meanwhile computes
  // the shared expert's SwiGLU of rows 2 sp, 2 sp + 1 (one record each pair).
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
    TOK1_MARK_W(3, 3);   // shared SwiGLU published
  }
  lds_barrier();
  TOK1_MARK(4);   // top-k known
  if (b == 0 && tid < k) {
    if (a.idx_out) a.idx_out[tid] = sh.sel[tid];
    if (a.w_out) a.w_out[tid] = sh.coef[1 + tid];
  }
  // Routed gate/up parts b, b + nwg, ... (expert slot part / nGUs).  From
  // here on the two roles run on branches of their own (the same sequence of
  // barriers on both), so that neither role's registers are live in the other
  // role's code.
  const int n_gu = k * a.nGUs;
  TileH tg[kUG], tu[kUG];
  auto gu_load = [&](int64_t e, int part) {
    const uint8_t* base = a.slabs + e * a.stride;
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
  auto gu_publish = [&](int part) {   // two barriers
    lds_barrier();
    if (writer_wave)
      publish_blocks<BITS>(sh.act[lane < a.gu_rows ? lane : 0], a.gu_rows,
                           (part % a.nGUs) * a.gu_rows, 1 + part / a.nGUs, I, rimg, ep,
                           sh.fail != 0, sh);
    lds_barrier();   // sh.act and sh.pay are reused
  };

  if (holder) {
    // ---- waves 2-3: routed gate/up rows, then the down rows they hold
    float rv[kUD], gv[kUD];
    for (int part = b; part < n_gu; part += nwg) {
      gu_load(sh.sel[part / a.nGUs], part % a.nGUs);
      gu_dots();
      TOK1_MARK_W(12, 3);   // wave 3: gate/up dot products done
      gu_publish(part);
    }
    TOK1_MARK_W(5, 3);   // routed SwiGLU published
    if (!has_d) return;   // workgroup-uniform
    // The down rows of every active expert (slot 0: the shared one), in
    // flight while the pollers wait for the images.
#pragma unroll
    for (int sl = 0; sl < kFusedMaxSlots; ++sl)
#pragma unroll
      for (int u = 0; u < kUD; ++u)
        down_tile(td[sl][u], sl == 0 ? (int64_t)E : (int64_t)sh.sel[min(sl, k) - 1], u);
#pragma unroll
    for (int u = 0; u < kUD; ++u) {
      rv[u] = a.resid[drow[u]];
      gv[u] = a.gamma[drow[u]];
    }
    TOK1_MARK_W(13, 3);   // wave 3: down rows requested

    // ---- phase C: the down rows against the images the pollers bring in
    float acc[kUD];
#pragma unroll
    for (int u = 0; u < kUD; ++u) acc[u] = 0.f;
    for (int s0 = 0; s0 < kp1; s0 += kFusedMaxSlots) {
      const int ns = min(kFusedMaxSlots, kp1 - s0);
      lds_barrier();                 // images polled
      if (s0 == 0) lds_barrier();    // shared image built
      float pacc[kUD];
#pragma unroll
      for (int u = 0; u < kUD; ++u) pacc[u] = 0.f;
      if (s0 == 0) {
#pragma unroll
        for (int sl = 0; sl < kFusedMaxSlots; ++sl) {
          if (sl < ns) {
            XRegsW<BITS> xw;
            xw.load(lds_ap + sl * ib, I, geoI);
            const float c = sh.coef[sl];
#pragma unroll
            for (int u = 0; u < kUD; ++u) {
              pin_tile(td[sl][u]);
              pacc[u] = fmaf(c, tile_dot_w(td[sl][u], xw), pacc[u]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);   // one expert's activations in registers at a time
        }
      } else {
        // later batches (k + 1 > 5): their tiles are loaded now
        TileI tl[kFusedMaxSlots][kUD];
#pragma unroll
        for (int sl = 0; sl < kFusedMaxSlots; ++sl)
#pragma unroll
          for (int u = 0; u < kUD; ++u) down_tile(tl[sl][u], sh.sel[min(s0 + sl, kp1 - 1) - 1], u);
#pragma unroll
        for (int sl = 0; sl < kFusedMaxSlots; ++sl) {
          if (sl < ns) {
            XRegsW<BITS> xw;
            xw.load(lds_ap + sl * ib, I, geoI);
            const float c = sh.coef[s0 + sl];
#pragma unroll
            for (int u = 0; u < kUD; ++u) {
              pin_tile(tl[sl][u]);
              pacc[u] = fmaf(c, tile_dot_w(tl[sl][u], xw), pacc[u]);
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kUD; ++u) acc[u] += sum_lanes(pacc[u], geoI.LPR);
      lds_barrier();   // lds_ap is reused by the next batch
    }
    const bool writer = geoI.lane_seg == geoI.LPR - 1;
    const bool bad = sh.fail != 0;
    float hval[kUD];
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < kUD; ++u) {
      hval[u] = bad ? __builtin_nanf("") : rv[u] + acc[u];
      // x may alias h_out: every read of x happened in phase A, before this
      // workgroup's logit and shared records, and every write of h_out here
      // follows the poll of every logit (top-k) and every shared record.
      if (writer) {
        a.h_out[drow[u]] = hval[u];
        if (a.moe_out) a.moe_out[drow[u]] = bad ? hval[u] : acc[u];
        ss = fmaf(hval[u], hval[u], ss);
      }
    }
    ss = sum_lanes(ss, kWave);
    if (lane == kWave - 1) sh.part[wave] = ss;
    lds_barrier();
    if (writer_wave && lane == 0 && b != a.stall_part) {
      const float tot = sh.part[2] + sh.part[3];
      const uint32_t tb = __float_as_uint(tot);
      rec_st(rpart, (uint32_t)(16 * b),
             u32x4_t{tb, 0u, 0u, rec_check(ep, tb, 0u, 0u, pos_salt(kSaltPart, b))});
    }
    TOK1_MARK_W(7, 3);   // sum of squares published
    lds_barrier();       // every part's sum in (the pollers' phase D)
    const float tot = sh.part[0] + sh.part[1];
    const float inv = 1.f / sqrtf(tot / (float)H + a.eps);
    const bool bad2 = sh.fail != 0;
#pragma unroll
    for (int u = 0; u < kUD; ++u)
      if (writer) a.y_out[drow[u]] = bad2 ? __builtin_nanf("") : gv[u] * hval[u] * inv;
    if (bad2 && writer_wave && lane == 0) st_agent(a.timeout, 1);
    if (b == 0 && writer_wave && lane == 0) st_agent(epoch_word, (int)ep);
    TOK1_MARK_W(9, 3);   // exit
  } else {
    // ---- waves 0-1: routed gate/up rows, then every poll
    for (int part = b; part < n_gu; part += nwg) {
      gu_load(sh.sel[part / a.nGUs], part % a.nGUs);
      gu_dots();
      TOK1_MARK(11);        // wave 0: gate/up dot products done
      gu_publish(part);
    }
    if (!has_d) return;   // workgroup-uniform
    const int t = tid;    // 0 .. 127
    for (int s0 = 0; s0 < kp1; s0 += kFusedMaxSlots) {
      const int ns = min(kFusedMaxSlots, kp1 - s0);
      bool ok = true;
      if (s0 == 0) {
        // the shared expert's values (image slot 0 is built from them below)
        ok &= poll_shared<128>(lds_x, rsh, I, ep, a.spin_ticks, t);
        ok &= poll_images<BITS, 128>(lds_ap, 1, rimg, I, 1, ns - 1, ep, a.spin_ticks, t);
      } else {
        ok &= poll_images<BITS, 128>(lds_ap, 0, rimg, I, s0, ns, ep, a.spin_ticks, t);
      }
      if (!ok) sh.fail = 1;
      lds_barrier();                 // images polled
      if (s0 == 0) {
        image_from_f32<BITS, 128>(lds_ap, lds_x, I, t);
        lds_barrier();               // shared image built
        TOK1_MARK(6);                // first images in LDS
      }
      lds_barrier();                 // batch computed
    }
    lds_barrier();                   // the holders' sums of squares in sh.part[2..3]
    // ---- phase D: every part's sum of h^2, in a fixed order
    constexpr int J = kTok1MaxParts / 128;
    float pv[J];
    bool done[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      done[j] = j * 128 + t >= a.nD;
      pv[j] = 0.f;
    }
    const uint64_t t0 = now_ticks();
    bool ok_all = true;
    // each wave polls its own parts, two a thread per pass (small poll rounds
    // finish sooner; one a pass adds a round trip more than it saves)
    constexpr int JP = 2;
#pragma unroll
    for (int j0 = 0; j0 < J; j0 += JP) {
      for (;;) {
        u32x4_t r[JP];
#pragma unroll
        for (int jj = 0; jj < JP; ++jj) {
          const int j = j0 + jj, d = min(j * 128 + t, a.nD - 1);
          if (j < J && !done[j]) r[jj] = rec_ld(rpart, (uint32_t)(16 * d));
        }
        bool pending = false;
#pragma unroll
        for (int jj = 0; jj < JP; ++jj) {
          const int j = j0 + jj;
          if (j >= J || done[j]) continue;
          const int d = j * 128 + t;
          if (!rec_ok(r[jj], ep, pos_salt(kSaltPart, d))) { pending = true; continue; }
          done[j] = true;
          pv[j] = __uint_as_float(r[jj][0]);
        }
        if (!__any(pending)) break;
        if (now_ticks() - t0 > a.spin_ticks) { ok_all = false; break; }
        __builtin_amdgcn_s_sleep(1);
      }
      if (!ok_all) break;
    }
    float p = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) p += pv[j];   // parts j*128 + t, in order of j
    p = sum_lanes(p, kWave);
    if (lane == kWave - 1) sh.part[wave] = p;
    if (!ok_all) sh.fail = 1;
    TOK1_MARK(8);   // every sum in
    lds_barrier();
  }
}

}  // namespace fmoe
