// fmoe_deltanet.hip -- one decode step of the Gated DeltaNet state update.
//
// [WAS] "4. Accelerate BLAS fuer Gated DeltaNet-Schichten": the state matrix
// of each of the 64 heads of a linear-attention layer is updated with a scale,
// a matrix-vector product and a rank-1 update.  Per (sequence, head), with
// state S [dk x dv], key k and query q [dk], value v [dv], decay a, strength b:
//   S <- a S;  u = S^T k;  S <- S + b k (v - u)^T;  o = S^T q.
// The four steps read and write the whole state four times as written; here
// they are one pass over it.  Column j of the result depends only on column j
// of the old state, through two of its dot products:
//   u_j = a (S^T k)_j,   d_j = b (v_j - u_j),
//   S'_ij = a S_ij + k_i d_j,   o_j = a (S^T q)_j + (k . q) d_j,
// so a workgroup loads a block of 32 columns of one head's state, reduces both
// dot products over the rows, and writes the block back: 2 dk dv fp32 bytes
// of HBM traffic per head and step (read once, written once), the bound of
// the step.
#include "fmoe_device.h"
#include "fmoe_internal.h"

namespace fmoe {

namespace {

typedef float f32v4 __attribute__((ext_vector_type(4)));
constexpr int kDnThreads = 256;
constexpr int kDnCols = 32;      // columns per workgroup: 8 lanes x float4

// Workgroup (bh, cb): head bh = b * NH + h, columns 32 cb .. 32 cb + 31.
// Thread t: float4 column quad c = t % 8, rows t / 8 + 32 r (r < DK / 32).
template <int DK>
__global__ __launch_bounds__(kDnThreads) void k_deltanet_step(DeltaNetArgs p) {
  constexpr int R = DK / 32;
  __shared__ float s_red[kDnThreads / kWave][8][9];
  const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
  const int ncb = p.dv / kDnCols;
  const int64_t bh = blockIdx.x / ncb;
  const int cb = blockIdx.x - (int)bh * ncb;
  const int c = tid & 7, rb = tid >> 3;
  const int col = cb * kDnCols + 4 * c;
  float* S = p.state + bh * (int64_t)DK * p.dv;
  const float* kh = p.k + bh * DK;
  const float* qh = p.q + bh * DK;

  f32v4 s[R];
  float kr[R], qr[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    s[r] = __builtin_nontemporal_load(
        reinterpret_cast<const f32v4*>(S + (int64_t)(rb + 32 * r) * p.dv + col));
#pragma unroll
  for (int r = 0; r < R; ++r) {
    kr[r] = kh[rb + 32 * r];
    qr[r] = qh[rb + 32 * r];
  }
  const float a = p.decay[bh], beta = p.beta[bh];
  const float4 vv = *reinterpret_cast<const float4*>(p.v + bh * p.dv + col);

  // Partial dot products over this thread's rows: S^T k and S^T q for its
  // four columns, and k . q.
  float acc[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) acc[i] = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    acc[0] = fmaf(s[r].x, kr[r], acc[0]);
    acc[1] = fmaf(s[r].y, kr[r], acc[1]);
    acc[2] = fmaf(s[r].z, kr[r], acc[2]);
    acc[3] = fmaf(s[r].w, kr[r], acc[3]);
    acc[4] = fmaf(s[r].x, qr[r], acc[4]);
    acc[5] = fmaf(s[r].y, qr[r], acc[5]);
    acc[6] = fmaf(s[r].z, qr[r], acc[6]);
    acc[7] = fmaf(s[r].w, qr[r], acc[7]);
    acc[8] = fmaf(kr[r], qr[r], acc[8]);
  }
  // Over the 8 row groups of the wave (lanes c, c + 8, ..., c + 56) ...
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    float v = acc[i];
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    acc[i] = v;
  }
  if (lane < 8) {
#pragma unroll
    for (int i = 0; i < 9; ++i) s_red[wave][lane][i] = acc[i];
  }
  __syncthreads();
  // ... then over the 4 waves, in wave order (the same sums in every thread).
  float tot[9];
#pragma unroll
  for (int i = 0; i < 9; ++i)
    tot[i] = ((s_red[0][c][i] + s_red[1][c][i]) + s_red[2][c][i]) + s_red[3][c][i];
  // k . q: every column quad reduced the same row products; take quad 0's.
  const float kq = ((s_red[0][0][8] + s_red[1][0][8]) + s_red[2][0][8]) + s_red[3][0][8];

  const float d0 = beta * (vv.x - a * tot[0]), d1 = beta * (vv.y - a * tot[1]);
  const float d2 = beta * (vv.z - a * tot[2]), d3 = beta * (vv.w - a * tot[3]);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    f32v4 o;
    o.x = fmaf(a, s[r].x, kr[r] * d0);
    o.y = fmaf(a, s[r].y, kr[r] * d1);
    o.z = fmaf(a, s[r].z, kr[r] * d2);
    o.w = fmaf(a, s[r].w, kr[r] * d3);
    __builtin_nontemporal_store(o, reinterpret_cast<f32v4*>(S + (int64_t)(rb + 32 * r) * p.dv + col));
  }
  if (rb == 0) {
    float4 o;
    o.x = fmaf(a, tot[4], kq * d0);
    o.y = fmaf(a, tot[5], kq * d1);
    o.z = fmaf(a, tot[6], kq * d2);
    o.w = fmaf(a, tot[7], kq * d3);
    *reinterpret_cast<float4*>(p.out + bh * p.dv + col) = o;
  }
}

}  // namespace

bool deltanet_supported(int dk, int dv) {
  return (dk == 32 || dk == 64 || dk == 128 || dk == 256) && dv >= kDnCols && dv % kDnCols == 0;
}

hipError_t launch_deltanet(const DeltaNetArgs& p, hipStream_t st) {
  if (!deltanet_supported(p.dk, p.dv)) return hipErrorNotSupported;
  const int64_t grid = (int64_t)p.B * p.NH * (p.dv / kDnCols);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  switch (p.dk) {
    case 32: hipLaunchKernelGGL(k_deltanet_step<32>, dim3((unsigned)grid), dim3(kDnThreads), 0, st, p); break;
    case 64: hipLaunchKernelGGL(k_deltanet_step<64>, dim3((unsigned)grid), dim3(kDnThreads), 0, st, p); break;
    case 128: hipLaunchKernelGGL(k_deltanet_step<128>, dim3((unsigned)grid), dim3(kDnThreads), 0, st, p); break;
    default: hipLaunchKernelGGL(k_deltanet_step<256>, dim3((unsigned)grid), dim3(kDnThreads), 0, st, p); break;
  }
  return hipGetLastError();
}

}  // namespace fmoe
