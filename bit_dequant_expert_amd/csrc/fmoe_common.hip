// fmoe_common.hip -- launchers of the format-independent kernels and the
// dispatch of format-templated launches to their translation units.
#include "fmoe_mfma.h"

namespace fmoe {

// ================================================= combine + norm (tokens)
__global__ __launch_bounds__(kThreads) void k_combine_norm(CombineArgs a) {
  __shared__ float s_part[kThreads / kWave];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = (int64_t)t * a.H;
  float ss = 0.f;
  for (int m = tid; m < a.H; m += kThreads) {
    float moe = 0.f;
    for (int i = 0; i < a.k; ++i)
      moe = fmaf(a.w_ws[(int64_t)t * a.k + i], a.yslot[((int64_t)t * a.kp1 + i) * a.H + m], moe);
    moe = fmaf(a.g_ws[t], a.yslot[((int64_t)t * a.kp1 + a.k) * a.H + m], moe);
    const float h = a.resid[row + m] + moe;
    a.h_out[row + m] = h;
    if (a.moe_out) a.moe_out[row + m] = moe;
    ss = fmaf(h, h, ss);
  }
  ss = sum_lanes(ss, kWave);
  if (lane == kWave - 1) s_part[wave] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < kThreads / kWave; ++w) tot += s_part[w];
  const float inv = 1.f / sqrtf(tot / (float)a.H + a.eps);
  for (int m = tid; m < a.H; m += kThreads) a.y_out[row + m] = a.gamma[m] * a.h_out[row + m] * inv;
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
  return bits == 4 && H % 64 == 0 && I % 64 == 0 && H / group <= kMfmaMaxGroups &&
         I / group <= kMfmaMaxGroups && H / group >= 4 && I / group >= 4;
}

hipError_t launch_mimg_prep(QFmt f, const MfmaArgs& a, int mode, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  VCall c = make_call(VCall::MIMG_PREP, f, 1, grid, st);
  c.mf = &a;
  c.mode = mode;
  return run_variant(c);
}

hipError_t launch_expert_mfma(QFmt f, const MfmaArgs& a, int mode, int grid, hipStream_t st) {
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

hipError_t launch_route(const RouteArgs& a, size_t lds_bytes, hipStream_t st) {
  const int nj_need = (a.H + 255) / 256, v_need = (a.E + 63) / 64;
  const int grid = a.n_router_wgs + a.n_prep_wgs;
#define FMOE_RT(NJ, V)                                                                  \
  if (nj_need <= NJ && v_need <= V) {                                                  \
    hipLaunchKernelGGL((k_route<NJ, V>), dim3(grid), dim3(kThreads), lds_bytes, st, a); \
    return hipGetLastError();                                                          \
  }
#define FMOE_RV(NJ) FMOE_RT(NJ, 1) FMOE_RT(NJ, 2) FMOE_RT(NJ, 4) FMOE_RT(NJ, 8) FMOE_RT(NJ, 16) FMOE_RT(NJ, 32)
  FMOE_RV(1) FMOE_RV(2) FMOE_RV(4) FMOE_RV(8) FMOE_RV(16) FMOE_RV(32)
#undef FMOE_RV
#undef FMOE_RT
  return hipErrorInvalidValue;
}

hipError_t launch_ffn_prep(int bits, const float* x, int H, uint8_t* xprep, int32_t* act, int maxA,
                           hipStream_t st) {
  const int grid = (H / 32 + kThreads / 8 - 1) / (kThreads / 8);
  if (bits == 4)
    hipLaunchKernelGGL(k_ffn_prep<4>, dim3(grid), dim3(kThreads), 0, st, x, H, xprep, act, maxA);
  else
    hipLaunchKernelGGL(k_ffn_prep<2>, dim3(grid), dim3(kThreads), 0, st, x, H, xprep, act, maxA);
  return hipGetLastError();
}

hipError_t launch_combine_norm(const CombineArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_combine_norm, dim3(a.T), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace fmoe
