// fmoe_internal.h -- kernel argument blocks and launchers shared by the C ABI
// (fmoe_api.cpp) and the kernels (fmoe_kernels.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmoe {

struct QFmt {
  int bits;   // 2 or 4
  int group;  // 32 or 64
  int sb;     // bytes per scale/bias: 4 (fp32) or 2 (bf16)
};

// Where an expert's nine sections live: expert e's section j is at
// base + e * stride + off[j].  A slab array uses base = slabs; a single
// expert given by loose pointers uses base = 0, stride = 0, off = addresses.
struct ExpertSrc {
  const uint8_t* base;
  int64_t stride;
  int64_t off[9];
};

// Active-expert list written by the routing kernel, read by the expert kernels:
//   act[0] = number of active experts, act[1] = number of them on the MFMA path,
//   then act_e[maxA], act_off[maxA], act_cnt[maxA], mfma[maxA], entries[T*(k+1)].
// Entry p = t*(k+1) + slot names token t's slot (slot k = the shared expert).
// Batches list the shared expert first (index 0, entries T*k ..), then the
// routed experts in expert order with their entries in token order.
struct ActView {
  const int32_t* base;
  int maxA;
  __host__ __device__ const int32_t* e() const { return base + 2; }
  __host__ __device__ const int32_t* off() const { return base + 2 + maxA; }
  __host__ __device__ const int32_t* cnt() const { return base + 2 + 2 * maxA; }
  __host__ __device__ const int32_t* mfma() const { return base + 2 + 3 * maxA; }
  __host__ __device__ const int32_t* entries() const { return base + 2 + 4 * maxA; }
};

struct RouteArgs {
  const float* Wr;
  const float* wsg;        // shared-gate vector or null
  double* gl;              // [T] its logits wsg . x (written by k_route_logits) or null
  const float* x;          // [T, H]
  int T, H, E, k, rows;    // rows of the logit product (= E)
  int ksplit;              // slices of the hidden dim (route_ksplit)
  double* part;            // [ksplit, T, rows] partial logits
  int32_t* sel_ws;         // [T, k] selections handed to the grouping, or null
  float* logits_out;       // [T, E] or null
  int32_t* idx_out;        // [T, k] or null
  float* w_out;            // [T, k] or null
  float* w_ws;             // [T, k] or null (internal copy for the combine)
  float* g_ws;             // [T] or null
  int* counter;            // self-resetting completion counter
  int32_t* act;            // active list (layer mode) or null
  int maxA, kp1, mfma_thr;
  uint8_t* xprep;          // per-token prepared activations or null
  int bits;
  int n_prep_wgs;
  uint4* ximg;             // per-token matrix-core images [T][H/8] or null
  float* xsc;              // their scales [T]
  int* ccnt;               // gate/up completion counters, cleared by the prep workgroups
  int n_ccnt;
  uint64_t* trace;         // phase stamps (FMOE_TRACE builds only): kRouteTraceSel per
                           // select workgroup, then kRouteTraceLog per logit workgroup
};
constexpr int kRouteTraceSel = 8, kRouteTraceLog = 4;

// Slices of the hidden dim for the router's matrix product: enough
// workgroups (16 rows x 32 tokens x slice) to cover the chip, at most 8.
constexpr int kRouteMaxSplit = 8;
inline int route_ksplit(int T, int rows) {
  const int tiles = ((rows + 15) / 16) * ((T + 31) / 32);
  int ks = (256 + tiles - 1) / tiles;
  return ks < 1 ? 1 : (ks > kRouteMaxSplit ? kRouteMaxSplit : ks);
}

struct GUArgs {
  ExpertSrc src;
  const int32_t* act;
  int maxA, kp1, H, I;
  const uint8_t* xprep;    // per token, xprep_bytes(H) each
  float* abuf;             // per entry, I floats
  uint8_t* aprep;          // per entry, xprep_bytes(I)
  int* ccnt;               // per entry, I/32 counters
  int nrb, U, mfma_thr;
};

struct DArgs {
  ExpertSrc src;
  const int32_t* act;
  int maxA, kp1, k, H, I;
  const uint8_t* aprep;
  const float* w_ws;
  const float* g_ws;
  const float* resid;
  float* h_out;
  float* y_out;
  float* moe_out;
  const float* gamma;
  float eps;
  float* yslot;            // per-entry outputs (slot mode)
  float* partials;         // per workgroup sum of squares (combine mode)
  int* ncnt;               // self-resetting counter (combine mode)
  int nrb, U, mfma_thr;
  int nbatch;              // active slots staged in LDS at once (combine mode)
};

struct CombineArgs {
  int T, H, k, kp1;
  const float* yslot;
  const float* w_ws;
  const float* g_ws;
  const float* resid;
  float* h_out;
  float* y_out;
  float* moe_out;
  const float* gamma;
  float eps;
};

struct FusedArgs;

// Experts with many tokens on the matrix cores (4-bit): activation images
// (fp16 words, one power-of-two scale per vector, scaled group sums) of the
// tokens' x and of those experts' SwiGLU outputs, and where results go.
constexpr int kMfmaTokens = 1;        // an expert with at least this many tokens takes the path
constexpr int kLdsPerCu = 160 * 1024;  // LDS of one gfx950 compute unit
constexpr int kMfmaMaxGroups = 128;   // K / G the path admits
constexpr int kMfmaMaxI = 2048;       // down input images of a 16-token pass held in LDS
constexpr int kMfmaMaxH = 8192;       // gate/up input images built in one pass of registers
#ifndef FMOE_MOE_GU_SPLIT
#define FMOE_MOE_GU_SPLIT 2
#endif
// Gate/up matrix-core workgroups: kMoeGuSplit waves share each 16-row tile,
// each taking a part of K, so a workgroup covers kMoeGuRows rows.
constexpr int kMoeGuSplit = FMOE_MOE_GU_SPLIT;
constexpr int kMoeGuRows = 64 / kMoeGuSplit;
constexpr int kMoeLdsTokens = 2;      // gate/up passes with at most this many tokens read A from LDS
#ifndef FMOE_MOE_DN_TILES
#define FMOE_MOE_DN_TILES 2
#endif
#ifndef FMOE_MOE_DN_WGS
#define FMOE_MOE_DN_WGS 3
#endif
// Down matrix-core workgroups: each wave takes kMoeDnTiles 16-row tiles, 64
// rows apart, so a workgroup covers kMoeDnRows rows; kMoeDnWgs workgroups a CU.
constexpr int kMoeDnTiles = FMOE_MOE_DN_TILES;
constexpr int kMoeDnRows = 64 * kMoeDnTiles;
constexpr int kMoeDnWgs = FMOE_MOE_DN_WGS;
struct MfmaArgs {
  ExpertSrc src;
  const int32_t* act;
  int maxA, kp1, T, H, I;
  int mfma_thr;        // experts with fewer tokens are left to the GEMV kernels
  const float* x;      // [T][H] layer input
  uint4* ximg;         // [T][H/8]
  float* xsc;          // [T]
  float* xsum;         // [T][H/G]
  float* abuf;         // [T*kp1][I] SwiGLU outputs
  float* yslot;        // [T*kp1][H] down outputs
};

// Bytes of the prepared image of a K-vector: K/2 fp16 pairs + K/32 float4.
__host__ __device__ constexpr int64_t xprep_bytes(int64_t K) { return 2 * K + (K / 32) * 16; }
// Word-blocked prepared image (the down projection's input inside the one-
// launch layer): pairs as in xprep, then one float4 {P, C, A, 0} per block of
// one 32-bit code word (32/bits elements).
__host__ __device__ constexpr int64_t wimg_bytes(int64_t K, int bits) {
  return 2 * K + (K / (32 / bits)) * 16;
}

inline int segs_per_lane(int K, int bits) {  // NS: 16-byte segments one lane reads per row
  const int S = K * bits / 128;
  return S >= 64 ? S / 64 : 1;
}

// One launch of a format-templated kernel; run_variant_<bits>_<group> (one
// translation unit per pair, compiled in parallel) instantiates the kernels.
struct VCall {
  enum Kind { GEMV, GEMV_SWIGLU, GATEUP, DOWN_COMBINE, DOWN_SLOTS, EXPERT_MFMA, FUSED1, EXPERT1,
              TOK1, CHAIN1 } kind;
  QFmt f;
  int ns;
  int grid;
  hipStream_t st;
  const uint8_t *q, *s, *b;
  const uint8_t *q2, *s2, *b2;   // GEMV_SWIGLU: the up matrix (q, s, b: gate)
  int N, K;
  const float* x;
  float* y;
  const struct GUArgs* gu;
  const struct DArgs* d;
  const struct MfmaArgs* mf;
  int mode;
  const struct FusedArgs* fu;
  const struct Expert1Args* ex;
  const struct Tok1Args* t1;
  const struct Tok1Chain* ch;   // CHAIN1: the layers (t1: the shared arguments)
  size_t lds;
};
hipError_t run_variant_4_32(const VCall& c);
hipError_t run_variant_4_64(const VCall& c);
hipError_t run_variant_2_32(const VCall& c);
hipError_t run_variant_2_64(const VCall& c);
int fused_occupancy_4_32(int sb, int ns, int E, size_t lds);
int fused_occupancy_4_64(int sb, int ns, int E, size_t lds);
int fused_occupancy_2_32(int sb, int ns, int E, size_t lds);
int fused_occupancy_2_64(int sb, int ns, int E, size_t lds);
int tok1_occupancy_4_32(int sb, int ns, int E, size_t lds);
int tok1_occupancy_4_64(int sb, int ns, int E, size_t lds);
int tok1_occupancy_2_32(int sb, int ns, int E, size_t lds);
int tok1_occupancy_2_64(int sb, int ns, int E, size_t lds);
int chain1_occupancy_4_32(int sb, int ns, int E, size_t lds);
int chain1_occupancy_4_64(int sb, int ns, int E, size_t lds);
int chain1_occupancy_2_32(int sb, int ns, int E, size_t lds);
int chain1_occupancy_2_64(int sb, int ns, int E, size_t lds);
int expert1_occupancy_4_32(int sb, int ns, size_t lds);
int expert1_occupancy_4_64(int sb, int ns, size_t lds);
int expert1_occupancy_2_32(int sb, int ns, size_t lds);
int expert1_occupancy_2_64(int sb, int ns, size_t lds);

hipError_t launch_gemv(QFmt f, const uint8_t* q, const uint8_t* s, const uint8_t* b, int N,
                       int K, const float* x, float* y, hipStream_t st);
// a[n] = silu(gate . x)[n] * (up . x)[n] for one expert's [N x K] gate and up.
hipError_t launch_gemv_swiglu(QFmt f, const uint8_t* gq, const uint8_t* gs, const uint8_t* gb,
                              const uint8_t* uq, const uint8_t* us, const uint8_t* ub, int N,
                              int K, const float* x, float* a, hipStream_t st);
hipError_t launch_route(const RouteArgs& a, hipStream_t st);
hipError_t launch_gateup(QFmt f, const GUArgs& a, int grid, hipStream_t st);
hipError_t launch_down_combine(QFmt f, const DArgs& a, hipStream_t st);
hipError_t launch_down_slots(QFmt f, const DArgs& a, int grid, hipStream_t st);
hipError_t launch_combine_norm(const CombineArgs& a, hipStream_t st);
// mode 0: gate/up (x images, then SwiGLU into abuf); mode 1: down (images of
// the path's abuf entries, then yslot).  The prep is one launch per mode.
bool mfma_supported(int H, int I, int bits, int group);
hipError_t launch_moe_mfma(QFmt f, const MfmaArgs& a, int mode, hipStream_t st);
// One-token layer in one persistent launch; returns hipErrorNotSupported when
// the row geometry is outside what the fused kernel is instantiated for.
hipError_t launch_fused1(QFmt f, const FusedArgs& a, hipStream_t st);
hipError_t launch_tok1(QFmt f, const struct Tok1Args& a, hipStream_t st);
// One token through ch.n layers of one shape in one persistent launch
// (fmoe_chain.h); a.h_out, a.y_out hold ch.n rows of H, a.idx_out, a.w_out
// ch.n rows of k.  hipErrorNotSupported where the shape or the resident
// workgroups do not admit it.
hipError_t launch_chain1(QFmt f, const struct Tok1Args& a, const struct Tok1Chain& ch,
                         hipStream_t st);
// The single-expert FFN in one launch; hipErrorNotSupported when the shape
// or the resident workgroups do not admit it (the caller then uses two).
hipError_t launch_expert1(QFmt f, Expert1Args a, hipStream_t st);
// Workspace of the allocation-free layer call: a static device array of
// kStaticScratchBytes per GPU.  static_scratch returns this device's address
// of it; the first call on a device takes the address and clears the array on
// `st` (hipErrorStreamCaptureUnsupported if `st` is capturing then).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
hipError_t static_scratch(hipStream_t st, void** ptr);
// One Gated DeltaNet decode step (fmoe_deltanet.hip): B sequences x NH heads,
// state [B][NH][dk][dv] updated in place, out [B][NH][dv].
struct DeltaNetArgs {
  const float *q, *k, *v, *decay, *beta;
  float* state;
  float* out;
  int B, NH, dk, dv;
};
bool deltanet_supported(int dk, int dv);
hipError_t launch_deltanet(const DeltaNetArgs& p, hipStream_t st);
// Decode attention over a bf16 KV cache (fmoe_attention.hip).
struct AttnArgs {
  const float* q;          // [B][NQ][D], rotation pairs interleaved
  const uint16_t* kc;      // [B][NKV][cap][D] bf16 bits, keys rotated (half-split order)
  const uint16_t* vc;      // [B][NKV][cap][D] bf16 bits
  const int32_t* lens;     // [B] positions in use (the new token's is lens - 1)
  float* out;              // [B][NQ][D]
  float* ws;               // attention_ws_bytes
  int B, NQ, NKV, D, cap;
  float base;              // rotary base
};
bool attention_supported(int NQ, int NKV, int D);
size_t attention_ws_bytes(int B, int NKV, int D, int cap);
hipError_t launch_attention(const AttnArgs& p, hipStream_t st);
// Host-tier expert streaming (fmoe_stream.hip).
struct FetchArgs {
  const int32_t* idx;      // [n_idx] experts to fetch (device)
  int n_idx;
  int shared;              // one more expert fetched with them, or -1
  const uint8_t* host;     // device address of the pinned host slabs
  uint8_t* dev;            // HBM slabs
  int64_t slab_bytes, stride;
  int32_t* tags;           // [n_slots] tag of what each HBM slot holds
  int n_slots;
  int tag;
  int* n_copied;           // optional: incremented once per slab copied
};
hipError_t launch_fetch(const FetchArgs& a, hipStream_t st);
// Byte offset of the counter block's wait-timeout word.
size_t wait_timeout_offset();
bool fused1_supported(int H, int I, int E, int bits);

// Row-block sizing shared by host and launchers.  RPI = rows one wave covers
// per iteration (64 lanes / lanes per row); each wave of the expert kernels
// runs U = 2 iterations when RPI <= 2, else 1, so a 4-wave workgroup covers
// 8 rows (long rows), 16 rows, or 4*RPI rows (short rows).
inline int rows_per_iter(int K, int bits) {
  const int S = K * bits / 128;
  return S >= 64 ? 1 : 64 / S;
}
inline int iters_per_wave(int K, int bits) { return rows_per_iter(K, bits) <= 2 ? 2 : 1; }
inline int rows_per_wg(int K, int bits) { return 4 * rows_per_iter(K, bits) * iters_per_wave(K, bits); }

}  // namespace fmoe
