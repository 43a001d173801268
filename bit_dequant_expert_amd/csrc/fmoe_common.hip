// fmoe_common.hip -- launchers of the format-independent kernels and the
// dispatch of format-templated launches to their translation units.
#include <mutex>

#include "fmoe_mfma.h"
#include "fmoe_route.h"

namespace fmoe {

// ================================================= combine + norm (tokens)
// One workgroup per token.  [WAS] section 3, "MoE-Kombination + Residual +
// Sigmoid-Gating", and the two-phase RMSNorm: h = r + sum_i w_i y_i + g y_s
// (routed slots in selection order, then the shared one), y = gamma h / rms(h).
// Each thread keeps its float4s of h in registers between the two phases; the
// slot loads are issued four slots at a time ahead of their use.  1024 threads
// a token: a CU has every float4 of a 4096-wide row in flight at once.
constexpr int kCombThreads = 1024;
__global__ __launch_bounds__(kCombThreads) void k_combine_norm(CombineArgs a) {
  constexpr int NT = kCombThreads;
  constexpr int MAXJ = 2;   // H <= 2 * 4 * NT
  __shared__ float s_part[NT / kWave];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nf = a.H / 4;
  const int64_t row = (int64_t)t * a.H;
  const float4* ys = reinterpret_cast<const float4*>(a.yslot + (int64_t)t * a.kp1 * a.H);
  float4 acc[MAXJ], rv[MAXJ], gm[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int f = j * NT + tid;
    const int fc = f < nf ? f : 0;
    acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    rv[j] = reinterpret_cast<const float4*>(a.resid + row)[fc];
    gm[j] = reinterpret_cast<const float4*>(a.gamma)[fc];
  }
  for (int i0 = 0; i0 < a.kp1; i0 += 4) {
    float4 v[4][MAXJ];
    float c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + q < a.kp1 ? i0 + q : a.k;
      c[q] = i < a.k ? a.w_ws[(int64_t)t * a.k + i] : a.g_ws[t];
      if (i0 + q >= a.kp1) c[q] = 0.f;
#pragma unroll
      for (int j = 0; j < MAXJ; ++j) {
        const int f = j * NT + tid;
        v[q][j] = ys[(int64_t)i * nf + (f < nf ? f : 0)];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (i0 + q < a.kp1) {
#pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
          acc[j].x = fmaf(c[q], v[q][j].x, acc[j].x);
          acc[j].y = fmaf(c[q], v[q][j].y, acc[j].y);
          acc[j].z = fmaf(c[q], v[q][j].z, acc[j].z);
          acc[j].w = fmaf(c[q], v[q][j].w, acc[j].w);
        }
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int f = j * NT + tid;
    if (f < nf) {
      const float4 h = make_float4(rv[j].x + acc[j].x, rv[j].y + acc[j].y, rv[j].z + acc[j].z,
                                   rv[j].w + acc[j].w);
      rv[j] = h;
      reinterpret_cast<float4*>(a.h_out + row)[f] = h;
      if (a.moe_out) reinterpret_cast<float4*>(a.moe_out + row)[f] = acc[j];
      ss = fmaf(h.x, h.x, ss);
      ss = fmaf(h.y, h.y, ss);
      ss = fmaf(h.z, h.z, ss);
      ss = fmaf(h.w, h.w, ss);
    }
  }
  ss = sum_lanes(ss, kWave);
  if (lane == kWave - 1) s_part[wave] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < NT / kWave; ++w) tot += s_part[w];
  const float inv = 1.f / sqrtf(tot / (float)a.H + a.eps);
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int f = j * NT + tid;
    if (f < nf)
      reinterpret_cast<float4*>(a.y_out + row)[f] =
          make_float4(gm[j].x * rv[j].x * inv, gm[j].y * rv[j].y * inv, gm[j].z * rv[j].z * inv,
                      gm[j].w * rv[j].w * inv);
  }
}


namespace {

hipError_t run_variant(const VCall& c) {
  if (c.f.bits == 4 && c.f.group == 32) return run_variant_4_32(c);
  if (c.f.bits == 4 && c.f.group == 64) return run_variant_4_64(c);
  if (c.f.bits == 2 && c.f.group == 32) return run_variant_2_32(c);
  if (c.f.bits == 2 && c.f.group == 64) return run_variant_2_64(c);
  return hipErrorInvalidValue;
}

VCall make_call(VCall::Kind kind, QFmt f, int ns, int grid, hipStream_t st) {
  VCall c{};
  c.kind = kind;
  c.f = f;
  c.ns = ns;
  c.grid = grid;
  c.st = st;
  return c;
}

}  // namespace

hipError_t launch_gemv(QFmt f, const uint8_t* q, const uint8_t* s, const uint8_t* b, int N,
                       int K, const float* x, float* y, hipStream_t st) {
  VCall c = make_call(VCall::GEMV, f, segs_per_lane(K, f.bits), 0, st);
  c.q = q; c.s = s; c.b = b; c.N = N; c.K = K; c.x = x; c.y = y;
  return run_variant(c);
}

hipError_t launch_gemv_swiglu(QFmt f, const uint8_t* gq, const uint8_t* gs, const uint8_t* gb,
                              const uint8_t* uq, const uint8_t* us, const uint8_t* ub, int N,
                              int K, const float* x, float* a, hipStream_t st) {
  VCall c = make_call(VCall::GEMV_SWIGLU, f, segs_per_lane(K, f.bits), 0, st);
  c.q = gq; c.s = gs; c.b = gb; c.q2 = uq; c.s2 = us; c.b2 = ub;
  c.N = N; c.K = K; c.x = x; c.y = a;
  return run_variant(c);
}

hipError_t launch_gateup(QFmt f, const GUArgs& a, int grid, hipStream_t st) {
  VCall c = make_call(VCall::GATEUP, f, segs_per_lane(a.H, f.bits), grid, st);
  c.gu = &a;
  return run_variant(c);
}

hipError_t launch_down_combine(QFmt f, const DArgs& a, hipStream_t st) {
  VCall c = make_call(VCall::DOWN_COMBINE, f, segs_per_lane(a.I, f.bits), a.nrb, st);
  c.d = &a;
  return run_variant(c);
}

hipError_t launch_down_slots(QFmt f, const DArgs& a, int grid, hipStream_t st) {
  VCall c = make_call(VCall::DOWN_SLOTS, f, segs_per_lane(a.I, f.bits), grid, st);
  c.d = &a;
  return run_variant(c);
}

bool mfma_supported(int H, int I, int bits, int group) {
  return bits == 4 && H % 128 == 0 && H % kMoeDnRows == 0 && I % 128 == 0 && I <= kMfmaMaxI && H <= kMfmaMaxH &&
         H / group <= kMfmaMaxGroups && I / group <= kMfmaMaxGroups && H / group >= 4 &&
         I / group >= 4;
}

hipError_t launch_moe_mfma(QFmt f, const MfmaArgs& a, int mode, hipStream_t st) {
  const int N = mode == 0 ? a.I : a.H;
  const int grid = a.maxA * (N / (mode == 0 ? kMoeGuRows : kMoeDnRows));
  if (grid <= 0) return hipSuccess;
  VCall c = make_call(VCall::EXPERT_MFMA, f, 1, grid, st);
  c.mf = &a;
  c.mode = mode;
  return run_variant(c);
}

bool fused1_supported(int H, int I, int E, int bits) {
  const int sh = H * bits / 128, si = I * bits / 128;
  if (!((sh == 64 || sh == 128) && (si == 16 || si == 32 || si == 64) && E <= 2048 &&
        H <= 8192 && H % 16 == 0 && I % fused_gu_rows(H, bits) == 0 &&
        fused_gu_rows(H, bits) % (32 / bits) == 0 && H % fused_d_rows(I, bits) == 0 &&
        wimg_bytes(I, bits) <= (int64_t)kFusedImgPer * kThreads * 8))
    return false;
  const int dr = fused_d_rows(I, bits);
  return (H + dr - 1) / dr <= kFusedMaxNormParts;
}

size_t wait_timeout_offset() { return (size_t)kTimeoutLine * kLine * sizeof(int); }

hipError_t launch_expert1(QFmt f, Expert1Args a, hipStream_t st) {
  const int H = a.H, I = a.I, bits = f.bits;
  const int sh = H * bits / 128, si = I * bits / 128;
  const int gr = fused_gu_rows(H, bits), dr = fused_d_rows(I, bits);
  if (!((sh == 64 || sh == 128) && (si == 16 || si == 32 || si == 64) && I % gr == 0 &&
        gr % (32 / bits) == 0 && gr <= kWave && H % dr == 0 &&
        wimg_bytes(I, bits) <= (int64_t)kFusedImgPer * kThreads * 8))
    return hipErrorNotSupported;
  a.gu_rows = gr;
  a.d_rows = dr;
  a.nGU = I / gr;
  a.nD = H / dr;
  const int grid = a.nGU > a.nD ? a.nGU : a.nD;
  if (grid < kSubs) return hipErrorNotSupported;   // the epoch needs every sub-counter in use
  const size_t lds = expert1_lds_bytes(H, I, bits);
  const int ns = segs_per_lane(H, bits);
  int occ = 0;
  if (bits == 4 && f.group == 32) occ = expert1_occupancy_4_32(f.sb, ns, lds);
  if (bits == 4 && f.group == 64) occ = expert1_occupancy_4_64(f.sb, ns, lds);
  if (bits == 2 && f.group == 32) occ = expert1_occupancy_2_32(f.sb, ns, lds);
  if (bits == 2 && f.group == 64) occ = expert1_occupancy_2_64(f.sb, ns, lds);
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n_cu < 1)
      n_cu = 1;
  }
  // Every workgroup waits for all the others' arrivals: all must be resident.
  if (grid > occ * n_cu) return hipErrorNotSupported;
  VCall c = make_call(VCall::EXPERT1, f, ns, grid, st);
  c.ex = &a;
  c.lds = lds;
  return run_variant(c);
}

namespace {

// The shape checks and part geometry of the one-token kernels (a.gu_rows,
// a.d_rows, a.nGUs, a.nD); hipErrorNotSupported outside what they handle.
hipError_t tok1_geometry(QFmt f, Tok1Args& a) {
  const int H = a.H, I = a.I, E = a.E, k = a.k, bits = f.bits;
  const int sh = H * bits / 128, si = I * bits / 128, W = 32 / bits;
  if (!((sh == 64 || sh == 128) && (si == 16 || si == 32 || si == 64))) return hipErrorNotSupported;
  if (E > kTok1MaxE || k + 1 > kTok1MaxSlots || H % 16 != 0 || I > H || I % 2 != 0)
    return hipErrorNotSupported;
  if (I > (bits == 4 ? kTok1MaxI4 : kTok1MaxI2)) return hipErrorNotSupported;
  const int gr = fused_gu_rows(H, bits);
  const int dr = 2 * 2 * rows_per_iter(I, bits);   // waves 2-3, two row iterations each
  if (I % gr != 0 || gr % W != 0 || gr / W > 2 || gr > kWave || H % dr != 0)
    return hipErrorNotSupported;
  a.gu_rows = gr;
  a.d_rows = dr;
  a.nGUs = I / gr;
  a.nD = H / dr;
  if (a.nD > kTok1MaxParts) return hipErrorNotSupported;
  return hipSuccess;
}

int tok1_n_cu() {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n_cu = 0;
  }
  return n_cu;
}

}  // namespace

// The one-token layer with self-checking records (fmoe_tok1.h).  Shapes:
// hidden rows of 64 or 128 segments, intermediate rows of 16, 32 or 64
// segments with I <= H, E <= 2048, k + 1 <= 17 slots, at most 1024 down parts.
// Grid: max(routed gate/up parts, down parts, shared row pairs), capped at the
// resident workgroups (routed parts and shared pairs past the grid loop).
// Every workgroup must hold a router row or a shared row pair (b < E or
// b < I/2): both are published after the workgroup's last read of x and
// polled by every workgroup before its first write of h_out, which may alias x.
hipError_t launch_tok1(QFmt f, const Tok1Args& a_in, hipStream_t st) {
  Tok1Args a = a_in;
  hipError_t ge = tok1_geometry(f, a);
  if (ge != hipSuccess) return ge;
  const int H = a.H, I = a.I, E = a.E, k = a.k, bits = f.bits;
  const int n_gu = k * a.nGUs, n_sp = I / 2;
  int want = n_gu > a.nD ? n_gu : a.nD;
  if (n_sp > want) want = n_sp;
  const size_t lds = fused_lds_bytes(H, I, bits);
  const int ns = segs_per_lane(H, bits);
  int occ = 0;
  if (bits == 4 && f.group == 32) occ = tok1_occupancy_4_32(f.sb, ns, E, lds);
  if (bits == 4 && f.group == 64) occ = tok1_occupancy_4_64(f.sb, ns, E, lds);
  if (bits == 2 && f.group == 32) occ = tok1_occupancy_2_32(f.sb, ns, E, lds);
  if (bits == 2 && f.group == 64) occ = tok1_occupancy_2_64(f.sb, ns, E, lds);
  const int cap = occ * tok1_n_cu();
  const int grid = want < cap ? want : cap;
  if (grid < 1 || a.nD > grid) return hipErrorNotSupported;
  if (grid > (E > n_sp ? E : n_sp)) return hipErrorNotSupported;
  VCall c = make_call(VCall::TOK1, f, ns, grid, st);
  c.t1 = &a;
  c.lds = lds;
  return run_variant(c);
}

// The chained one-token kernel (fmoe_chain.h): the shapes of the one-token
// kernel with E <= 512 and k + 1 <= kFusedMaxSlots, one workgroup per down
// part (grid = nD, all resident), every workgroup holding a router row or a
// shared row pair (nD <= max(E, I/2)), at most kTok1MaxPartRecs part records
// and kTok1MaxChain layers.
hipError_t launch_chain1(QFmt f, const Tok1Args& a_in, const Tok1Chain& ch, hipStream_t st) {
  Tok1Args a = a_in;
  hipError_t ge = tok1_geometry(f, a);
  if (ge != hipSuccess) return ge;
  if (ch.n < 1 || ch.n > kTok1MaxChain) return hipErrorInvalidValue;
  const int H = a.H, I = a.I, E = a.E, bits = f.bits;
  if (E > 512) return hipErrorNotSupported;   // one wave's top-k of 8 keys per lane
  if (a.k + 1 > kFusedMaxSlots) return hipErrorNotSupported;   // phase C in one batch
  const int R = (a.d_rows + 3) / 3;
  if (a.d_rows > 16 || (int64_t)R * a.nD > kTok1MaxPartRecs) return hipErrorNotSupported;
  if (H / 4 % 128 != 0) return hipErrorNotSupported;   // the next x: float4 per holder thread
  const int n_sp = I / 2;
  if (a.nD > (E > n_sp ? E : n_sp)) return hipErrorNotSupported;
  // Dynamic LDS of at least a third of the CU's: two workgroups a CU at most,
  // so that the grid spreads evenly over the CUs (the kernel's registers
  // would admit three on some CUs and leave others with one).
  size_t lds = fused_lds_bytes(H, I, bits);
  if (lds < (size_t)kLdsPerCu / 3 + 1024) lds = (size_t)kLdsPerCu / 3 + 1024;
  const int ns = segs_per_lane(H, bits);
  int occ = 0;
  if (bits == 4 && f.group == 32) occ = chain1_occupancy_4_32(f.sb, ns, E, lds);
  if (bits == 4 && f.group == 64) occ = chain1_occupancy_4_64(f.sb, ns, E, lds);
  if (bits == 2 && f.group == 32) occ = chain1_occupancy_2_32(f.sb, ns, E, lds);
  if (bits == 2 && f.group == 64) occ = chain1_occupancy_2_64(f.sb, ns, E, lds);
  if (a.nD > occ * tok1_n_cu()) return hipErrorNotSupported;
  VCall c = make_call(VCall::CHAIN1, f, ns, a.nD, st);
  c.t1 = &a;
  c.ch = &ch;
  c.lds = lds;
  return run_variant(c);
}

hipError_t launch_fused1(QFmt f, const FusedArgs& a, hipStream_t st) {
  if (!fused1_supported(a.H, a.I, a.E, f.bits)) return hipErrorNotSupported;
  const size_t lds = fused_lds_bytes(a.H, a.I, f.bits);
  const int ns = segs_per_lane(a.H, f.bits);
  int occ = 1;
  if (f.bits == 4 && f.group == 32) occ = fused_occupancy_4_32(f.sb, ns, a.E, lds);
  if (f.bits == 4 && f.group == 64) occ = fused_occupancy_4_64(f.sb, ns, a.E, lds);
  if (f.bits == 2 && f.group == 32) occ = fused_occupancy_2_32(f.sb, ns, a.E, lds);
  if (f.bits == 2 && f.group == 64) occ = fused_occupancy_2_64(f.sb, ns, a.E, lds);
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n_cu < 1)
      n_cu = 256;
  }
  // Router rows go to the first min(grid, E) items (rows f, f + nRr, ... below
  // E, and the shared-expert gate row E to item E mod nRr), so every one of
  // them is the first item of a running workgroup.
  FusedArgs b = a;
  const int g = occ * n_cu;
  const int grid = g < a.nF ? g : a.nF;
  b.nRr = grid < a.E ? grid : a.E;
  VCall c = make_call(VCall::FUSED1, f, ns, grid, st);
  c.fu = &b;
  c.lds = lds;
  return run_variant(c);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  const int nlog = ((a.rows + 15) / 16) * ((a.T + 31) / 32) * a.ksplit;
  const int nx = (a.ximg || a.gl) ? a.T : 0;   // per token (first): its image and gate logit
  hipLaunchKernelGGL(k_route_logits, dim3(nlog + a.n_prep_wgs + nx), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lg = (size_t)a.rows * 8;
  // grouping: token masks (T <= 64), selections, three per-expert arrays
  const size_t gr =
      a.act ? (a.T <= 64 ? (size_t)a.E * 8 : 0) + ((size_t)a.T * a.k + 3 * (size_t)a.E) * 4 : 0;
  const size_t lds = lg > gr ? lg : gr;
  const int v_need = (a.E + 63) / 64;
#define FMOE_RS(V)                                                                   \
  if (v_need <= V) {                                                                 \
    hipLaunchKernelGGL((k_route_select<V>), dim3(a.T), dim3(kThreads), lds, st, a);  \
    return hipGetLastError();                                                        \
  }
  FMOE_RS(1) FMOE_RS(2) FMOE_RS(4) FMOE_RS(8) FMOE_RS(16) FMOE_RS(32)
#undef FMOE_RS
  return hipErrorInvalidValue;
}

hipError_t launch_combine_norm(const CombineArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_combine_norm, dim3(a.T), dim3(kCombThreads), 0, st, a);
  return hipGetLastError();
}

// ===================================================== static scratch
// The workspace of the allocation-free layer call: a file-scope device array
// that every GPU the library runs on holds until the process ends.  In host
// code `scratch` names a host-side stand-in; its device address, which differs
// per GPU, is taken once per device below and only that address is handed to
// kernels and memory calls.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch(hipStream_t st, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // Set-up on the first call on this device: the address, then one clear
    // (the layer's counters rest at zero between calls), ordered ahead of the
    // call's kernels on its stream.  Outside graph capture only, so that no
    // memory-set node is ever recorded.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(st, &cs)) != hipSuccess) return e;
    if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    if ((e = hipMemsetAsync(p, 0, kStaticScratchBytes, st)) != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace fmoe
