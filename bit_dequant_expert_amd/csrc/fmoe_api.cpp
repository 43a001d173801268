// fmoe_api.cpp -- the C ABI of libfmoe.so (declared in include/fmoe.h).
//
// Host side only: validates every argument before anything is enqueued, carves
// the caller's workspace, picks launch shapes and enqueues the kernels of
// fmoe_kernels.hip on the caller's stream.  Nothing here allocates, copies or
// synchronises.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <algorithm>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fmoe.h"
#include "fmoe_internal.h"
#include "fmoe_fused_args.h"

namespace {

using fmoe::QFmt;

thread_local char g_err[512] = "";

fmoe_status fail(fmoe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

fmoe_status hip_fail(hipError_t e, const char* what) {
  return fail(FMOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

constexpr int kMaxE = 2048;       // experts held in registers by the top-k wave
constexpr int kMaxH = 8192;       // router row held in registers
constexpr int kMaxK = 16;
constexpr int kMaxSel = 8192;     // T * k selections grouped in LDS
constexpr int kMfmaThreshold = INT_MAX;  // experts with >= this many tokens use MFMA

fmoe_status check_fmt(const fmoe_qformat* f, QFmt* out) {
  if (!f) return fail(FMOE_ERR_NULL, "fmt is NULL");
  if (f->bits != 2 && f->bits != 4)
    return fail(FMOE_ERR_UNSUPPORTED, "bits=%d (supported: 2, 4)", f->bits);
  if (f->group != 32 && f->group != 64)
    return fail(FMOE_ERR_UNSUPPORTED, "group=%d (supported: 32, 64)", f->group);
  if (f->sdtype != FMOE_F32 && f->sdtype != FMOE_BF16)
    return fail(FMOE_ERR_UNSUPPORTED, "sdtype=%d (supported: FMOE_F32, FMOE_BF16)", f->sdtype);
  out->bits = f->bits;
  out->group = f->group;
  out->sb = f->sdtype == FMOE_BF16 ? 2 : 4;
  return FMOE_OK;
}

// Shape rules for a row of K codes; min_segs > 1 for the expert paths.
fmoe_status check_k(int K, const QFmt& f, int min_segs, const char* name) {
  if (K <= 0) return fail(FMOE_ERR_SHAPE, "%s: k=%d must be positive", name, K);
  if (K % f.group != 0)
    return fail(FMOE_ERR_SHAPE, "%s: k=%d is not a multiple of group %d", name, K, f.group);
  if (((int64_t)K * f.bits) % 128 != 0)
    return fail(FMOE_ERR_SHAPE, "%s: k*bits/8 = %lld is not a multiple of 16", name,
                (long long)K * f.bits / 8);
  const int S = (int)((int64_t)K * f.bits / 128);
  const bool ok = (S < 64 && 64 % S == 0) || S == 64 || S == 128 || S == 256;
  if (!ok)
    return fail(FMOE_ERR_UNSUPPORTED,
                "%s: k=%d gives %d 16-byte segments per row (supported: divisors of 64, "
                "or 64/128/256)", name, K, S);
  if (S < min_segs)
    return fail(FMOE_ERR_UNSUPPORTED, "%s: k=%d is too short (need k*bits >= %d)", name, K,
                128 * min_segs);
  return FMOE_OK;
}

fmoe_status check_qmat(const fmoe_qmat* W, const QFmt& f, int n, int k, int min_segs,
                       const char* name) {
  if (!W) return fail(FMOE_ERR_NULL, "%s is NULL", name);
  if (!W->q || !W->scale || !W->bias)
    return fail(FMOE_ERR_NULL, "%s: q/scale/bias must not be NULL", name);
  if (!aligned(W->q, 16) || !aligned(W->scale, 16) || !aligned(W->bias, 16))
    return fail(FMOE_ERR_ALIGN, "%s: q/scale/bias must be 16-byte aligned", name);
  if (W->n <= 0) return fail(FMOE_ERR_SHAPE, "%s: n=%d must be positive", name, W->n);
  if ((n >= 0 && W->n != n) || (k >= 0 && W->k != k))
    return fail(FMOE_ERR_SHAPE, "%s: shape %dx%d, expected %dx%d", name, W->n, W->k, n, k);
  return check_k(W->k, f, min_segs, name);
}

fmoe_status check_vec(const void* p, const char* name) {
  if (!p) return fail(FMOE_ERR_NULL, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(FMOE_ERR_ALIGN, "%s must be 16-byte aligned", name);
  return FMOE_OK;
}

int64_t slab_layout(int H, int I, const QFmt& f, int64_t off[9]) {
  const int64_t rows[3] = {I, I, H}, cols[3] = {H, H, I};
  int64_t pos = 0;
  for (int m = 0; m < 3; ++m) {
    const int64_t qb = rows[m] * cols[m] * f.bits / 8;
    const int64_t sb = rows[m] * (cols[m] / f.group) * f.sb;
    off[3 * m] = pos;
    pos = (int64_t)align256((size_t)(pos + qb));
    off[3 * m + 1] = pos;
    pos = (int64_t)align256((size_t)(pos + sb));
    off[3 * m + 2] = pos;
    pos = (int64_t)align256((size_t)(pos + sb));
  }
  return pos;
}

// ------------------------------------------------------------- workspace
struct LayerWs {
  size_t ctr, lg64, sel, w, g, gl, act, xprep, abuf, ccnt, aprep, yslot, gh, part, dlist;
  size_t ximg, xsc, xsum, total;
  int maxA, nrb_gu, nrb_d;
};

size_t act_ints(int maxA, int T, int kp1) { return 2 + 4 * (size_t)maxA + (size_t)T * kp1; }

LayerWs layer_ws(int T, int H, int I, int E, int k, int bits) {
  LayerWs w{};
  const int kp1 = k + 1;
  const int64_t sel = (int64_t)T * k;
  w.maxA = (int)((sel < E ? sel : E) + 1);
  w.nrb_gu = (I + fmoe::rows_per_wg(H, bits) - 1) / fmoe::rows_per_wg(H, bits);
  w.nrb_d = (H + fmoe::rows_per_wg(I, bits) - 1) / fmoe::rows_per_wg(I, bits);
  const size_t ent = (size_t)T * kp1;
  size_t pos = 0;
  w.ctr = pos; pos += fmoe::kWsReserved;   // counters (the one-launch path's block)
  // Router logits: [T, E+1] for the one-launch path, partial sums per slice
  // [ksplit, T, E] for the multi-launch path (ksplit >= 1).
  const size_t lg_n = (size_t)fmoe::route_ksplit(T, E) * T * E;
  w.lg64 = pos; pos = align256(pos + (lg_n > (size_t)T * (E + 1) ? lg_n : (size_t)T * (E + 1)) * 8);
  w.sel = pos; pos = align256(pos + (size_t)T * k * 4);
  w.w = pos; pos = align256(pos + (size_t)T * k * 4);
  w.g = pos; pos = align256(pos + (size_t)T * 4);
  w.gl = pos; pos = align256(pos + (size_t)T * 8);
  w.act = pos; pos = align256(pos + act_ints(w.maxA, T, kp1) * 4);
  w.xprep = pos; pos = align256(pos + (size_t)T * fmoe::xprep_bytes(H));
  w.abuf = pos; pos = align256(pos + ent * I * 4);
  w.ccnt = pos; pos = align256(pos + ent * (I / 32) * 4);
  w.aprep = pos; pos = align256(pos + ent * fmoe::xprep_bytes(I));
  w.yslot = pos; pos = align256(pos + (T > 1 ? ent * H * 4 : 0));
  w.gh = pos; pos = align256(pos + (T == 1 ? (size_t)H * 4 : 0));
  const int nd_fused = (H + fmoe::fused_d_rows(I, bits) - 1) / fmoe::fused_d_rows(I, bits);
  w.part = pos; pos = align256(pos + (size_t)(nd_fused > w.nrb_d ? nd_fused : w.nrb_d) * 4);
  w.dlist = pos; pos = align256(pos + (T == 1 ? (size_t)nd_fused * 4 : 0));
  // Matrix-core path (batches): activation images of the tokens, with their
  // scales and group sums (group 32: the larger).
  const size_t mt = T > 1 ? (size_t)T : 0;
  w.ximg = pos; pos = align256(pos + mt * (size_t)H * 2);
  w.xsc = pos; pos = align256(pos + mt * 4);
  w.xsum = pos; pos = align256(pos + mt * (size_t)(H / 32) * 4);
  w.total = pos;
  return w;
}

struct FfnWs {
  size_t ctr, abuf, total;
};

FfnWs ffn_ws(int H, int I) {
  (void)H;
  FfnWs w{};
  size_t pos = 0;
  w.ctr = pos; pos += fmoe::kWsReserved;   // same reserved head as every layout
  w.abuf = pos; pos = align256(pos + (size_t)I * 4);   // SwiGLU output (fp32 or its image)
  w.total = pos;
  return w;
}

size_t route_ws(int T, int E) {
  return fmoe::kWsReserved + align256((size_t)fmoe::route_ksplit(T, E) * T * E * 8);
}

// Kernel-path selection (include/fmoe.h, fmoe_paths): read from the
// environment once when the library is loaded, changed only by fmoe_set_paths.
fmoe_paths g_paths = {0, 0, fmoe::kMfmaTokens, 0, 0, 0, 0};
#ifdef FMOE_TRACE
void* g_trace = nullptr;
#endif

bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v && v[0] == '1';
}

struct PathsFromEnv {
  PathsFromEnv() {
    g_paths.no_fused = env_flag("FMOE_NO_FUSED");
    g_paths.no_mfma = env_flag("FMOE_NO_MFMA");
    const char* v = getenv("FMOE_MFMA_MIN_TOKENS");
    const int n = v ? atoi(v) : 0;
    g_paths.mfma_min_tokens = n >= 1 ? n : fmoe::kMfmaTokens;
    g_paths.debug_sync = env_flag("FMOE_DEBUG_SYNC");
    g_paths.t1_counters = env_flag("FMOE_T1_COUNTERS");
    const char* w = getenv("FMOE_WAIT_LIMIT_US");
    const int us = w ? atoi(w) : 0;
    g_paths.wait_limit_us = us > 0 ? us : 0;
  }
} g_paths_from_env;

bool mfma_disabled() { return g_paths.no_mfma != 0; }
int mfma_min_tokens() { return g_paths.mfma_min_tokens; }
bool fused_disabled() { return g_paths.no_fused != 0; }
bool expert1_enabled() { return !fused_disabled(); }

// With debug_sync set, an entry point that enqueued its kernels waits for them
// and reports a fault or launch failure as FMOE_ERR_HIP.
fmoe_status finish(fmoe_status st, void* stream, const char* what) {
  if (st != FMOE_OK || !g_paths.debug_sync) return st;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  return FMOE_OK;
}

fmoe_status check_router(int T, int H, int E, int k) {
  if (T < 0) return fail(FMOE_ERR_SHAPE, "T=%d must be >= 0", T);
  if (H <= 0 || H % 4 != 0) return fail(FMOE_ERR_SHAPE, "H=%d must be a positive multiple of 4", H);
  if (H > kMaxH) return fail(FMOE_ERR_UNSUPPORTED, "H=%d exceeds %d", H, kMaxH);
  if (E <= 0) return fail(FMOE_ERR_SHAPE, "E=%d must be positive", E);
  if (E > kMaxE) return fail(FMOE_ERR_UNSUPPORTED, "E=%d exceeds %d", E, kMaxE);
  if (k < 1 || k > E) return fail(FMOE_ERR_SHAPE, "k=%d must be in [1, E=%d]", k, E);
  if (k > kMaxK) return fail(FMOE_ERR_UNSUPPORTED, "k=%d exceeds %d", k, kMaxK);
  if ((int64_t)T * k > kMaxSel)
    return fail(FMOE_ERR_UNSUPPORTED, "T*k=%lld exceeds %d", (long long)T * k, kMaxSel);
  return FMOE_OK;
}

}  // namespace

extern "C" {

int32_t fmoe_abi_version(void) { return FMOE_ABI_VERSION; }

#ifdef FMOE_TRACE
// Trace build only (not part of the interface): device buffer of
// kTok1TraceEvents 64-bit stamps per workgroup of the one-token kernel.
void fmoe_trace_set(void* dev_buf) { g_trace = dev_buf; }
#endif

void fmoe_get_paths(fmoe_paths* p) {
  if (p) *p = g_paths;
}

fmoe_status fmoe_set_paths(const fmoe_paths* p) {
  if (!p) return fail(FMOE_ERR_NULL, "paths is NULL");
  if (p->mfma_min_tokens < 1)
    return fail(FMOE_ERR_SHAPE, "mfma_min_tokens=%d must be >= 1", p->mfma_min_tokens);
  if (p->wait_limit_us < 0 || p->test_stall_part < 0)
    return fail(FMOE_ERR_SHAPE, "wait_limit_us and test_stall_part must be >= 0");
  g_paths = *p;
  return FMOE_OK;
}

const char* fmoe_last_error(void) { return g_err; }

size_t fmoe_wait_timeout_offset(void) { return fmoe::wait_timeout_offset(); }

int64_t fmoe_slab_layout(int32_t hidden, int32_t inter, const fmoe_qformat* fmt, int64_t off[9]) {
  QFmt f;
  if (check_fmt(fmt, &f) != FMOE_OK) return -1;
  if (!off) { fail(FMOE_ERR_NULL, "off is NULL"); return -1; }
  if (hidden <= 0 || inter <= 0 || hidden % f.group || inter % f.group) {
    fail(FMOE_ERR_SHAPE, "hidden=%d / inter=%d must be positive multiples of group %d", hidden,
         inter, f.group);
    return -1;
  }
  return slab_layout(hidden, inter, f, off);
}

size_t fmoe_route_workspace_size(int32_t T, int32_t E) {
  if (T < 0 || E <= 0) return 0;
  return route_ws(T, E);
}

static fmoe_status fmoe_route_topk_impl(const float* router_w, const float* x, int32_t T, int32_t H, int32_t E,
                            int32_t k, int32_t* idx, float* w, float* logits_out, void* ws,
                            size_t ws_bytes, void* stream) {
  fmoe_status st = check_router(T, H, E, k);
  if (st != FMOE_OK) return st;
  if ((st = check_vec(router_w, "router_w")) != FMOE_OK) return st;
  if ((st = check_vec(x, "x")) != FMOE_OK) return st;
  if (!idx || !w) return fail(FMOE_ERR_NULL, "idx and w must not be NULL");
  if (T == 0) return FMOE_OK;
  if (!ws) return fail(FMOE_ERR_WORKSPACE, "ws is NULL");
  if (!aligned(ws, 256)) return fail(FMOE_ERR_ALIGN, "ws must be 256-byte aligned");
  if (ws_bytes < route_ws(T, E))
    return fail(FMOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, route_ws(T, E));
  uint8_t* wsb = (uint8_t*)ws;
  fmoe::RouteArgs a{};
  a.Wr = router_w;
  a.wsg = nullptr;
  a.x = x;
  a.T = T; a.H = H; a.E = E; a.k = k; a.rows = E;
  a.ksplit = fmoe::route_ksplit(T, E);
  a.part = (double*)(wsb + fmoe::kWsReserved);
  a.sel_ws = nullptr;
  a.logits_out = logits_out;
  a.idx_out = idx;
  a.w_out = w;
  a.counter = (int*)wsb;
  a.kp1 = k + 1;
  a.mfma_thr = kMfmaThreshold;
  a.n_prep_wgs = 0;
  hipError_t e = fmoe::launch_route(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "route kernel");
  return FMOE_OK;
}

static fmoe_status fmoe_dequant_gemv_impl(const fmoe_qmat* W, const fmoe_qformat* fmt, const float* x,
                              float* y, void* stream) {
  QFmt f;
  fmoe_status st = check_fmt(fmt, &f);
  if (st != FMOE_OK) return st;
  if ((st = check_qmat(W, f, -1, -1, 1, "W")) != FMOE_OK) return st;
  if ((st = check_vec(x, "x")) != FMOE_OK) return st;
  if ((st = check_vec(y, "y")) != FMOE_OK) return st;
  if (overlap(x, (size_t)W->k * 4, y, (size_t)W->n * 4)) return fail(FMOE_ERR_SHAPE, "y overlaps x");
  hipError_t e = fmoe::launch_gemv(f, (const uint8_t*)W->q, (const uint8_t*)W->scale,
                                   (const uint8_t*)W->bias, W->n, W->k, x, y, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "gemv kernel");
  return FMOE_OK;
}

size_t fmoe_expert_ffn_workspace_size(const fmoe_expert* e, const fmoe_qformat* fmt) {
  if (!e || !fmt) return 0;
  return ffn_ws(e->gate.k, e->gate.n).total;
}

static fmoe_status fmoe_expert_ffn_impl(const fmoe_expert* e, const fmoe_qformat* fmt, const float* x,
                            float* y, void* ws, size_t ws_bytes, void* stream) {
  QFmt f;
  fmoe_status st = check_fmt(fmt, &f);
  if (st != FMOE_OK) return st;
  if (!e) return fail(FMOE_ERR_NULL, "expert is NULL");
  const int H = e->gate.k, I = e->gate.n;
  if ((st = check_qmat(&e->gate, f, -1, -1, 4, "gate")) != FMOE_OK) return st;
  if ((st = check_qmat(&e->up, f, I, H, 4, "up")) != FMOE_OK) return st;
  if ((st = check_qmat(&e->down, f, H, I, 4, "down")) != FMOE_OK) return st;
  if ((st = check_vec(x, "x")) != FMOE_OK) return st;
  if ((st = check_vec(y, "y")) != FMOE_OK) return st;
  if (overlap(x, (size_t)H * 4, y, (size_t)H * 4)) return fail(FMOE_ERR_SHAPE, "y overlaps x");
  const FfnWs L = ffn_ws(H, I);
  if (!ws) return fail(FMOE_ERR_WORKSPACE, "ws is NULL");
  if (!aligned(ws, 256)) return fail(FMOE_ERR_ALIGN, "ws must be 256-byte aligned");
  if (ws_bytes < L.total) return fail(FMOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, L.total);
  uint8_t* wsb = (uint8_t*)ws;
  hipStream_t s = (hipStream_t)stream;

  // One launch when the shape and the resident workgroups admit it (the
  // SwiGLU image in abuf); else two: gate and up with SwiGLU into the
  // workspace, then down.
  float* abuf = (float*)(wsb + L.abuf);
  fmoe::Expert1Args ea{};
  ea.gq = (const uint8_t*)e->gate.q; ea.gs = (const uint8_t*)e->gate.scale; ea.gb = (const uint8_t*)e->gate.bias;
  ea.uq = (const uint8_t*)e->up.q; ea.us = (const uint8_t*)e->up.scale; ea.ub = (const uint8_t*)e->up.bias;
  ea.dq = (const uint8_t*)e->down.q; ea.ds = (const uint8_t*)e->down.scale; ea.db = (const uint8_t*)e->down.bias;
  ea.x = x; ea.y = y; ea.img = (uint8_t*)abuf; ea.ctr = (int*)(wsb + L.ctr); ea.H = H; ea.I = I;
  hipError_t he = expert1_enabled() ? fmoe::launch_expert1(f, ea, s) : hipErrorNotSupported;
  if (he == hipSuccess) return FMOE_OK;
  if (he != hipErrorNotSupported) return hip_fail(he, "expert kernel");
  he = fmoe::launch_gemv_swiglu(
      f, (const uint8_t*)e->gate.q, (const uint8_t*)e->gate.scale, (const uint8_t*)e->gate.bias,
      (const uint8_t*)e->up.q, (const uint8_t*)e->up.scale, (const uint8_t*)e->up.bias, I, H, x,
      abuf, s);
  if (he != hipSuccess) return hip_fail(he, "gate/up kernel");
  he = fmoe::launch_gemv(f, (const uint8_t*)e->down.q, (const uint8_t*)e->down.scale,
                         (const uint8_t*)e->down.bias, H, I, abuf, y, s);
  if (he != hipSuccess) return hip_fail(he, "down kernel");
  return FMOE_OK;
}

size_t fmoe_workspace_size(const fmoe_layer* L, int32_t T) {
  if (!L || T < 0 || L->n_experts <= 0 || L->top_k <= 0 || L->fmt.bits <= 0) return 0;
  return layer_ws(T, L->hidden, L->inter, L->n_experts, L->top_k, L->fmt.bits).total;
}

// Host-side validation of a layer call's arguments (everything but the
// workspace); FMOE_OK when the call may proceed.
static fmoe_status layer_args_check(const fmoe_layer* L, int32_t T, const float* x,
                                    const float* residual, const float* h_out, const float* y_out,
                                    const float* moe_out) {
  if (!L) return fail(FMOE_ERR_NULL, "layer is NULL");
  QFmt f;
  fmoe_status st = check_fmt(&L->fmt, &f);
  if (st != FMOE_OK) return st;
  const int H = L->hidden, I = L->inter, E = L->n_experts, k = L->top_k;
  if ((st = check_router(T, H, E, k)) != FMOE_OK) return st;
  if ((st = check_k(H, f, 4, "hidden")) != FMOE_OK) return st;
  if ((st = check_k(I, f, 4, "inter")) != FMOE_OK) return st;
  if ((st = check_vec(L->router_w, "router_w")) != FMOE_OK) return st;
  if ((st = check_vec(L->shared_gate_w, "shared_gate_w")) != FMOE_OK) return st;
  if ((st = check_vec(L->norm_w, "norm_w")) != FMOE_OK) return st;
  if (!L->slabs) return fail(FMOE_ERR_NULL, "slabs is NULL");
  if (!aligned(L->slabs, 256)) return fail(FMOE_ERR_ALIGN, "slabs must be 256-byte aligned");
  int64_t off[9];
  const int64_t slab = slab_layout(H, I, f, off);
  if (L->slab_stride % 256 != 0)
    return fail(FMOE_ERR_ALIGN, "slab_stride=%lld is not a multiple of 256", (long long)L->slab_stride);
  if (L->slab_stride < slab)
    return fail(FMOE_ERR_SHAPE, "slab_stride=%lld < slab size %lld", (long long)L->slab_stride,
                (long long)slab);
  if (!(L->norm_eps >= 0.f)) return fail(FMOE_ERR_SHAPE, "norm_eps must be >= 0");
  if ((st = check_vec(x, "x")) != FMOE_OK) return st;
  if ((st = check_vec(residual, "residual")) != FMOE_OK) return st;
  if ((st = check_vec(h_out, "h_out")) != FMOE_OK) return st;
  if ((st = check_vec(y_out, "y_out")) != FMOE_OK) return st;
  if (moe_out && !aligned(moe_out, 16)) return fail(FMOE_ERR_ALIGN, "moe_out must be 16-byte aligned");
  if (T == 0) return FMOE_OK;
  const size_t vb = (size_t)T * H * 4;
  if (residual != x && overlap(residual, vb, x, vb))
    return fail(FMOE_ERR_SHAPE, "residual partially overlaps x");
  if (h_out != residual && (overlap(h_out, vb, residual, vb) || overlap(h_out, vb, x, vb)))
    return fail(FMOE_ERR_SHAPE, "h_out overlaps x/residual without being residual");
  if (overlap(y_out, vb, x, vb) || overlap(y_out, vb, residual, vb) || overlap(y_out, vb, h_out, vb))
    return fail(FMOE_ERR_SHAPE, "y_out overlaps x, residual or h_out");
  if (moe_out && (overlap(moe_out, vb, x, vb) || overlap(moe_out, vb, residual, vb) ||
                  overlap(moe_out, vb, h_out, vb) || overlap(moe_out, vb, y_out, vb)))
    return fail(FMOE_ERR_SHAPE, "moe_out overlaps another vector");
  return FMOE_OK;
}

// The arguments of the one-token kernels that come from the layer and the
// workspace (the vectors are the caller's to set).
static fmoe::Tok1Args tok1_args(const fmoe_layer* L, const int64_t off[9], uint8_t* wsb) {
  fmoe::Tok1Args ta{};
  ta.slabs = (const uint8_t*)L->slabs;
  ta.stride = L->slab_stride;
  for (int i = 0; i < 9; ++i) ta.off[i] = off[i];
  ta.Wr = L->router_w; ta.wsg = L->shared_gate_w; ta.gamma = L->norm_w;
  ta.eps = L->norm_eps;
  ta.H = L->hidden; ta.I = L->inter; ta.E = L->n_experts; ta.k = L->top_k;
  ta.area = wsb + fmoe::kFusedCtrBytes;
  ta.timeout = (int*)(wsb + fmoe::wait_timeout_offset());
  const uint64_t lim_us = g_paths.wait_limit_us > 0 ? (uint64_t)g_paths.wait_limit_us : 200000u;
  ta.spin_ticks = lim_us * 100u;   // the wall clock runs at 100 MHz
  ta.stall_part = g_paths.test_stall_part > 0 ? g_paths.test_stall_part - 1 : -1;
  return ta;
}

static fmoe_status fmoe_moe_layer_forward_impl(const fmoe_layer* L, int32_t T, const float* x,
                                   const float* residual, float* h_out, float* y_out,
                                   int32_t* idx_out, float* w_out, float* moe_out, void* ws,
                                   size_t ws_bytes, void* stream) {
  fmoe_status st = layer_args_check(L, T, x, residual, h_out, y_out, moe_out);
  if (st != FMOE_OK || T == 0) return st;
  QFmt f;
  check_fmt(&L->fmt, &f);
  const int H = L->hidden, I = L->inter, E = L->n_experts, k = L->top_k;
  int64_t off[9];
  slab_layout(H, I, f, off);
  const LayerWs W = layer_ws(T, H, I, E, k, f.bits);
  if (!ws) return fail(FMOE_ERR_WORKSPACE, "ws is NULL");
  if (!aligned(ws, 256)) return fail(FMOE_ERR_ALIGN, "ws must be 256-byte aligned");
  if (ws_bytes < W.total) return fail(FMOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, W.total);

  uint8_t* wsb = (uint8_t*)ws;
  hipStream_t s = (hipStream_t)stream;
  const int kp1 = k + 1;
  int32_t* act = (int32_t*)(wsb + W.act);
  int* ctr = (int*)(wsb + W.ctr);

  fmoe::ExpertSrc src{};
  src.base = (const uint8_t*)L->slabs;
  src.stride = L->slab_stride;
  memcpy(src.off, off, sizeof off);

  if (T == 1 && !fused_disabled() && !g_paths.t1_counters) {
    fmoe::Tok1Args ta = tok1_args(L, off, wsb);
    ta.x = x; ta.resid = residual;
    ta.h_out = h_out; ta.y_out = y_out; ta.moe_out = moe_out;
    ta.w_out = w_out; ta.idx_out = idx_out;
#ifdef FMOE_TRACE
    ta.trace = (uint64_t*)g_trace;
#endif
    hipError_t te = fmoe::launch_tok1(f, ta, s);
    if (te == hipSuccess) return FMOE_OK;
    if (te != hipErrorNotSupported) return hip_fail(te, "one-token layer kernel");
  }
  if (T == 1 && fmoe::fused1_supported(H, I, E, f.bits) && !fused_disabled()) {
    fmoe::FusedArgs fa{};
    fa.src = src;
    fa.Wr = L->router_w; fa.wsg = L->shared_gate_w; fa.x = x; fa.resid = residual;
    fa.gamma = L->norm_w; fa.h_out = h_out; fa.y_out = y_out; fa.moe_out = moe_out;
    fa.w_out = w_out; fa.idx_out = idx_out; fa.eps = L->norm_eps;
    fa.H = H; fa.I = I; fa.E = E; fa.k = k;
    fa.lg64 = (double*)(wsb + W.lg64);
    fa.abuf = (float*)(wsb + W.abuf);
    fa.gh = (float*)(wsb + W.gh);
    fa.partials = (float*)(wsb + W.part);
    fa.dlist = (int*)(wsb + W.dlist);
    fa.ctr = ctr;
    fa.gu_rows = fmoe::fused_gu_rows(H, f.bits);
    fa.nGUs = I / fa.gu_rows;
    fa.d_rows = fmoe::fused_d_rows(I, f.bits);
    fa.nD = (H + fa.d_rows - 1) / fa.d_rows;
    fa.nF = k * fa.nGUs > fa.nD ? k * fa.nGUs : fa.nD;
    hipError_t fe = fmoe::launch_fused1(f, fa, s);
    if (fe == hipSuccess) return FMOE_OK;
    if (fe != hipErrorNotSupported) return hip_fail(fe, "fused layer kernel");
  }

  // Experts of a batch take the matrix cores (4-bit); experts with fewer than
  // mfma_thr tokens (none at the default threshold) take the GEMV kernels.
  const bool use_mfma = T > 1 && fmoe::mfma_supported(H, I, f.bits, f.group) && !mfma_disabled();
  const int mfma_thr = use_mfma ? mfma_min_tokens() : kMfmaThreshold;
  const bool use_gemv = !use_mfma || mfma_thr > 1;

  fmoe::RouteArgs ra{};
  ra.Wr = L->router_w; ra.wsg = L->shared_gate_w; ra.x = x;
  // The router rows only (512 rows are 32 whole tiles of the logit product);
  // the shared gate's dot product is taken by a wave of its own.
  ra.T = T; ra.H = H; ra.E = E; ra.k = k; ra.rows = E;
  ra.ksplit = fmoe::route_ksplit(T, E);
  ra.part = (double*)(wsb + W.lg64);
  ra.sel_ws = (int32_t*)(wsb + W.sel);
  ra.idx_out = idx_out; ra.w_out = w_out;
  ra.w_ws = (float*)(wsb + W.w); ra.g_ws = (float*)(wsb + W.g); ra.gl = (double*)(wsb + W.gl);
  ra.counter = ctr + 0;
  ra.act = act; ra.maxA = W.maxA; ra.kp1 = kp1; ra.mfma_thr = mfma_thr;
  ra.xprep = use_gemv ? wsb + W.xprep : nullptr; ra.bits = f.bits;
  ra.n_prep_wgs = use_gemv ? (int)(((int64_t)T * (H / 32) + 31) / 32) : 0;
  if (use_gemv) {
    ra.ccnt = (int*)(wsb + W.ccnt);
    ra.n_ccnt = (int)((size_t)T * kp1 * (I / 32));
  }
  if (use_mfma) {   // the tokens' matrix-core images, in the same launch
    ra.ximg = (uint4*)(wsb + W.ximg);
    ra.xsc = (float*)(wsb + W.xsc);
  }
#ifdef FMOE_TRACE
  ra.trace = (uint64_t*)g_trace;
#endif
  hipError_t he = fmoe::launch_route(ra, s);
  if (he != hipSuccess) return hip_fail(he, "route kernel");

  if (use_gemv) {
    fmoe::GUArgs g{};
    g.src = src; g.act = act; g.maxA = W.maxA; g.kp1 = kp1; g.H = H; g.I = I;
    g.xprep = wsb + W.xprep; g.abuf = (float*)(wsb + W.abuf); g.aprep = wsb + W.aprep;
    g.ccnt = (int*)(wsb + W.ccnt);
    g.nrb = W.nrb_gu; g.U = fmoe::iters_per_wave(H, f.bits); g.mfma_thr = mfma_thr;
    he = fmoe::launch_gateup(f, g, W.maxA * W.nrb_gu, s);
    if (he != hipSuccess) return hip_fail(he, "gate/up kernel");
  }

  fmoe::MfmaArgs m{};
  if (use_mfma) {
    m.src = src; m.act = act; m.maxA = W.maxA; m.kp1 = kp1; m.T = T; m.H = H; m.I = I;
    m.mfma_thr = mfma_thr;
    m.x = x;
    m.ximg = (uint4*)(wsb + W.ximg); m.xsc = (float*)(wsb + W.xsc); m.xsum = (float*)(wsb + W.xsum);
    m.abuf = (float*)(wsb + W.abuf); m.yslot = (float*)(wsb + W.yslot);
    if ((he = fmoe::launch_moe_mfma(f, m, 0, s)) != hipSuccess)
      return hip_fail(he, "gate/up matrix-core kernel");
  }

  fmoe::DArgs d{};
  d.src = src; d.act = act; d.maxA = W.maxA; d.kp1 = kp1; d.k = k; d.H = H; d.I = I;
  d.aprep = wsb + W.aprep; d.w_ws = (const float*)(wsb + W.w); d.g_ws = (const float*)(wsb + W.g);
  d.resid = residual; d.h_out = h_out; d.y_out = y_out; d.moe_out = moe_out;
  d.gamma = L->norm_w; d.eps = L->norm_eps;
  d.nrb = W.nrb_d; d.U = fmoe::iters_per_wave(I, f.bits); d.mfma_thr = mfma_thr;
  if (T == 1) {
    d.partials = (float*)(wsb + W.part);
    d.ncnt = ctr + 1;
    const int64_t ab = fmoe::xprep_bytes(I);
    int nb = (int)(49152 / ab);
    nb = nb < 1 ? 1 : nb;
    nb = nb > 8 ? 8 : nb;
    d.nbatch = nb < kp1 ? nb : kp1;
    he = fmoe::launch_down_combine(f, d, s);
    if (he != hipSuccess) return hip_fail(he, "down/combine kernel");
  } else {
    d.yslot = (float*)(wsb + W.yslot);
    if (use_gemv) {
      he = fmoe::launch_down_slots(f, d, W.maxA * W.nrb_d, s);
      if (he != hipSuccess) return hip_fail(he, "down kernel");
    }
    if (use_mfma) {
      if ((he = fmoe::launch_moe_mfma(f, m, 1, s)) != hipSuccess)
        return hip_fail(he, "down matrix-core kernel");
    }
    fmoe::CombineArgs c{};
    c.T = T; c.H = H; c.k = k; c.kp1 = kp1;
    c.yslot = d.yslot; c.w_ws = d.w_ws; c.g_ws = d.g_ws; c.resid = residual;
    c.h_out = h_out; c.y_out = y_out; c.moe_out = moe_out; c.gamma = L->norm_w; c.eps = L->norm_eps;
    he = fmoe::launch_combine_norm(c, s);
    if (he != hipSuccess) return hip_fail(he, "combine kernel");
  }
  return FMOE_OK;
}

fmoe_status fmoe_route_topk(const float* router_w, const float* x, int32_t T, int32_t H, int32_t E,
                            int32_t k, int32_t* idx, float* w, float* logits_out, void* ws,
                            size_t ws_bytes, void* stream) {
  return finish(fmoe_route_topk_impl(router_w, x, T, H, E, k, idx, w, logits_out, ws, ws_bytes,
                                     stream), stream, "route kernel (debug sync)");
}

fmoe_status fmoe_dequant_gemv(const fmoe_qmat* W, const fmoe_qformat* fmt, const float* x,
                              float* y, void* stream) {
  return finish(fmoe_dequant_gemv_impl(W, fmt, x, y, stream), stream, "gemv (debug sync)");
}

fmoe_status fmoe_expert_ffn(const fmoe_expert* e, const fmoe_qformat* fmt, const float* x,
                            float* y, void* ws, size_t ws_bytes, void* stream) {
  return finish(fmoe_expert_ffn_impl(e, fmt, x, y, ws, ws_bytes, stream), stream,
                "expert FFN (debug sync)");
}

fmoe_status fmoe_moe_layer_forward(const fmoe_layer* L, int32_t T, const float* x,
                                   const float* residual, float* h_out, float* y_out,
                                   int32_t* idx_out, float* w_out, float* moe_out, void* ws,
                                   size_t ws_bytes, void* stream) {
  return finish(fmoe_moe_layer_forward_impl(L, T, x, residual, h_out, y_out, idx_out, w_out,
                                            moe_out, ws, ws_bytes, stream),
                stream, "layer (debug sync)");
}

// Layers of one stack call must agree in everything but their weights.
static bool same_shape(const fmoe_layer& a, const fmoe_layer& b) {
  return a.hidden == b.hidden && a.inter == b.inter && a.n_experts == b.n_experts &&
         a.top_k == b.top_k && a.fmt.bits == b.fmt.bits && a.fmt.group == b.fmt.group &&
         a.fmt.sdtype == b.fmt.sdtype && a.slab_stride == b.slab_stride &&
         a.norm_eps == b.norm_eps;
}

static fmoe_status fmoe_moe_stack_forward_impl(const fmoe_layer* layers, int32_t n_layers,
                                               int32_t T, const float* x, const float* residual,
                                               float* h_out, float* y_out, int32_t* idx_out,
                                               float* w_out, void* ws, size_t ws_bytes,
                                               void* stream) {
  if (!layers) return fail(FMOE_ERR_NULL, "layers is NULL");
  if (n_layers < 0) return fail(FMOE_ERR_SHAPE, "n_layers=%d must be >= 0", n_layers);
  if (n_layers == 0) return FMOE_OK;
  for (int l = 0; l < n_layers; ++l) {
    if (!same_shape(layers[l], layers[0]))
      return fail(FMOE_ERR_SHAPE, "layer %d differs from layer 0 in shape, format, stride or eps", l);
    fmoe_status st = layer_args_check(&layers[l], T, x, residual, h_out, y_out, nullptr);
    if (st != FMOE_OK) return st;
  }
  if (T == 0) return FMOE_OK;
  const fmoe_layer* L = &layers[0];
  const int H = L->hidden, k = L->top_k;
  const size_t vb = (size_t)T * H * 4, ob = vb * (size_t)n_layers;
  if (residual != x && overlap(residual, vb, x, vb))
    return fail(FMOE_ERR_SHAPE, "residual partially overlaps x");
  if (overlap(h_out, ob, x, vb) || overlap(h_out, ob, residual, vb) ||
      overlap(y_out, ob, x, vb) || overlap(y_out, ob, residual, vb) || overlap(y_out, ob, h_out, ob))
    return fail(FMOE_ERR_SHAPE, "h_out and y_out must not overlap x, residual or each other");
  const size_t ib = (size_t)T * k * 4 * (size_t)n_layers;
  if (idx_out && w_out && overlap(idx_out, ib, w_out, ib))
    return fail(FMOE_ERR_SHAPE, "idx_out overlaps w_out");
  QFmt f;
  check_fmt(&L->fmt, &f);
  const LayerWs W = layer_ws(T, H, L->inter, L->n_experts, k, f.bits);
  if (!ws) return fail(FMOE_ERR_WORKSPACE, "ws is NULL");
  if (!aligned(ws, 256)) return fail(FMOE_ERR_ALIGN, "ws must be 256-byte aligned");
  if (ws_bytes < W.total) return fail(FMOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, W.total);
  uint8_t* wsb = (uint8_t*)ws;
  hipStream_t s = (hipStream_t)stream;

  if (T == 1 && !fused_disabled() && !g_paths.t1_counters) {
    // one launch per fmoe::kTok1MaxChain layers
    int64_t off[9];
    slab_layout(H, L->inter, f, off);
    int done = 0;
    while (done < n_layers) {
      const int n = n_layers - done < fmoe::kTok1MaxChain ? n_layers - done : fmoe::kTok1MaxChain;
      fmoe::Tok1Args ta = tok1_args(L, off, wsb);
      ta.x = done == 0 ? x : y_out + (size_t)(done - 1) * H;
      ta.resid = done == 0 ? residual : h_out + (size_t)(done - 1) * H;
      ta.h_out = h_out + (size_t)done * H;
      ta.y_out = y_out + (size_t)done * H;
      ta.idx_out = idx_out ? idx_out + (size_t)done * k : nullptr;
      ta.w_out = w_out ? w_out + (size_t)done * k : nullptr;
#ifdef FMOE_TRACE
      ta.trace = (uint64_t*)g_trace;
#endif
      fmoe::Tok1Chain ch{};
      ch.n = n;
      for (int l = 0; l < n; ++l) {
        const fmoe_layer& Ll = layers[done + l];
        ch.layer[l] = fmoe::Tok1ChainLayer{Ll.router_w, Ll.shared_gate_w, Ll.norm_w,
                                           (const uint8_t*)Ll.slabs};
      }
      hipError_t te = fmoe::launch_chain1(f, ta, ch, s);
      if (te == hipErrorNotSupported && done == 0) break;   // the shape: per-layer calls
      if (te != hipSuccess) return hip_fail(te, "chained one-token kernel");
      done += n;
    }
    if (done == n_layers) return FMOE_OK;
  }
  for (int l = 0; l < n_layers; ++l) {
    const size_t o = (size_t)l * T * H, oi = (size_t)l * T * k;
    fmoe_status st = fmoe_moe_layer_forward_impl(
        &layers[l], T, l == 0 ? x : y_out + o - (size_t)T * H,
        l == 0 ? residual : h_out + o - (size_t)T * H, h_out + o, y_out + o,
        idx_out ? idx_out + oi : nullptr, w_out ? w_out + oi : nullptr, nullptr, ws, ws_bytes,
        stream);
    if (st != FMOE_OK) return st;
  }
  return FMOE_OK;
}

fmoe_status fmoe_moe_stack_forward(const fmoe_layer* layers, int32_t n_layers, int32_t T,
                                   const float* x, const float* residual, float* h_out,
                                   float* y_out, int32_t* idx_out, float* w_out, void* ws,
                                   size_t ws_bytes, void* stream) {
  return finish(fmoe_moe_stack_forward_impl(layers, n_layers, T, x, residual, h_out, y_out,
                                            idx_out, w_out, ws, ws_bytes, stream),
                stream, "stack (debug sync)");
}

static fmoe_status fmoe_deltanet_step_impl(const float* q, const float* k, const float* v,
                                           const float* decay, const float* beta, float* state,
                                           float* out, int32_t batch, int32_t heads, int32_t dk,
                                           int32_t dv, void* stream) {
  if (batch < 0 || heads < 0) return fail(FMOE_ERR_SHAPE, "batch=%d and heads=%d must be >= 0", batch, heads);
  if (!fmoe::deltanet_supported(dk, dv))
    return fail(FMOE_ERR_UNSUPPORTED, "dk=%d must be 32, 64, 128 or 256 and dv=%d a positive "
                "multiple of 32", dk, dv);
  const size_t nbh = (size_t)batch * heads;
  if (nbh == 0) return FMOE_OK;   // nothing to read or write
  fmoe_status st;
  if ((st = check_vec(q, "q")) != FMOE_OK) return st;
  if ((st = check_vec(k, "k")) != FMOE_OK) return st;
  if ((st = check_vec(v, "v")) != FMOE_OK) return st;
  if ((st = check_vec(state, "state")) != FMOE_OK) return st;
  if ((st = check_vec(out, "out")) != FMOE_OK) return st;
  if (!decay) return fail(FMOE_ERR_NULL, "decay is NULL");
  if (!beta) return fail(FMOE_ERR_NULL, "beta is NULL");
  const size_t sb = nbh * dk * dv * 4, ob = nbh * dv * 4;
  if (overlap(out, ob, state, sb) || overlap(out, ob, q, nbh * dk * 4) ||
      overlap(out, ob, k, nbh * dk * 4) || overlap(out, ob, v, ob))
    return fail(FMOE_ERR_SHAPE, "out overlaps the state or an input");
  if (overlap(state, sb, q, nbh * dk * 4) || overlap(state, sb, k, nbh * dk * 4) ||
      overlap(state, sb, v, ob) || overlap(state, sb, decay, nbh * 4) ||
      overlap(state, sb, beta, nbh * 4))
    return fail(FMOE_ERR_SHAPE, "state overlaps an input");
  fmoe::DeltaNetArgs p{q, k, v, decay, beta, state, out, batch, heads, dk, dv};
  const hipError_t e = fmoe::launch_deltanet(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "deltanet kernel");
  return FMOE_OK;
}

fmoe_status fmoe_deltanet_step(const float* q, const float* k, const float* v, const float* decay,
                               const float* beta, float* state, float* out, int32_t batch,
                               int32_t heads, int32_t dk, int32_t dv, void* stream) {
  return finish(fmoe_deltanet_step_impl(q, k, v, decay, beta, state, out, batch, heads, dk, dv,
                                        stream),
                stream, "deltanet (debug sync)");
}

size_t fmoe_attention_workspace_size(int32_t batch, int32_t n_kv_heads, int32_t head_dim,
                                     int32_t cap) {
  if (batch < 0 || n_kv_heads <= 0 || head_dim <= 0 || cap < 0) return 0;
  return fmoe::attention_ws_bytes(batch, n_kv_heads, head_dim, cap);
}

static fmoe_status fmoe_attention_decode_impl(const float* q, const uint16_t* k_cache,
                                              const uint16_t* v_cache, const int32_t* lens,
                                              int32_t batch, int32_t n_q_heads,
                                              int32_t n_kv_heads, int32_t head_dim, int32_t cap,
                                              float rope_base, float* out, void* ws,
                                              size_t ws_bytes, void* stream) {
  if (batch < 0 || cap < 1) return fail(FMOE_ERR_SHAPE, "batch=%d must be >= 0 and cap=%d >= 1", batch, cap);
  if (!fmoe::attention_supported(n_q_heads, n_kv_heads, head_dim))
    return fail(FMOE_ERR_UNSUPPORTED, "head_dim=%d must be 64, 128 or 256 and n_q_heads=%d a "
                "multiple of n_kv_heads=%d by at most 16", head_dim, n_q_heads, n_kv_heads);
  if (!(rope_base > 1.f)) return fail(FMOE_ERR_SHAPE, "rope_base must be > 1");
  if (batch == 0) return FMOE_OK;
  fmoe_status st;
  if ((st = check_vec(q, "q")) != FMOE_OK) return st;
  if ((st = check_vec(k_cache, "k_cache")) != FMOE_OK) return st;
  if ((st = check_vec(v_cache, "v_cache")) != FMOE_OK) return st;
  if ((st = check_vec(out, "out")) != FMOE_OK) return st;
  if (!lens) return fail(FMOE_ERR_NULL, "lens is NULL");
  const size_t ob = (size_t)batch * n_q_heads * head_dim * 4;
  const size_t cb = (size_t)batch * n_kv_heads * cap * head_dim * 2;
  if (overlap(out, ob, q, ob) || overlap(out, ob, k_cache, cb) || overlap(out, ob, v_cache, cb))
    return fail(FMOE_ERR_SHAPE, "out overlaps an input");
  const size_t need = fmoe::attention_ws_bytes(batch, n_kv_heads, head_dim, cap);
  if (!ws) return fail(FMOE_ERR_WORKSPACE, "ws is NULL");
  if (!aligned(ws, 256)) return fail(FMOE_ERR_ALIGN, "ws must be 256-byte aligned");
  if (ws_bytes < need) return fail(FMOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu", ws_bytes, need);
  if (overlap(ws, need, out, ob)) return fail(FMOE_ERR_SHAPE, "ws overlaps out");
  fmoe::AttnArgs p{q, k_cache, v_cache, lens, out, (float*)ws, batch, n_q_heads, n_kv_heads,
                   head_dim, cap, rope_base};
  const hipError_t e = fmoe::launch_attention(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernels");
  return FMOE_OK;
}

fmoe_status fmoe_attention_decode(const float* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                  const int32_t* lens, int32_t batch, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim, int32_t cap,
                                  float rope_base, float* out, void* ws, size_t ws_bytes,
                                  void* stream) {
  return finish(fmoe_attention_decode_impl(q, k_cache, v_cache, lens, batch, n_q_heads,
                                           n_kv_heads, head_dim, cap, rope_base, out, ws,
                                           ws_bytes, stream),
                stream, "attention (debug sync)");
}

static fmoe_status fmoe_fetch_experts_impl(const int32_t* idx, int32_t n_idx, int32_t shared,
                                           const void* host_slabs, int64_t slab_bytes,
                                           int64_t slab_stride, void* dev_slabs, int32_t* tags,
                                           int32_t n_slots, int32_t tag, int32_t* n_copied,
                                           void* stream) {
  if (n_idx < 0 || n_idx > kMaxSel) return fail(FMOE_ERR_SHAPE, "n_idx=%d must be in [0, %d]", n_idx, kMaxSel);
  if (n_slots <= 0) return fail(FMOE_ERR_SHAPE, "n_slots=%d must be positive", n_slots);
  if (shared < -1 || shared >= n_slots) return fail(FMOE_ERR_SHAPE, "shared=%d must be -1 or a slot", shared);
  if (slab_bytes <= 0 || slab_bytes % 16 != 0)
    return fail(FMOE_ERR_SHAPE, "slab_bytes=%lld must be a positive multiple of 16", (long long)slab_bytes);
  if (slab_stride < slab_bytes || slab_stride % 16 != 0)
    return fail(FMOE_ERR_SHAPE, "slab_stride=%lld must be a multiple of 16 and >= slab_bytes", (long long)slab_stride);
  if (n_idx == 0 && shared < 0) return FMOE_OK;
  if (n_idx > 0 && !idx) return fail(FMOE_ERR_NULL, "idx is NULL");
  if (!host_slabs) return fail(FMOE_ERR_NULL, "host_slabs is NULL");
  if (!dev_slabs) return fail(FMOE_ERR_NULL, "dev_slabs is NULL");
  if (!tags) return fail(FMOE_ERR_NULL, "tags is NULL");
  if (!aligned(host_slabs, 16) || !aligned(dev_slabs, 16))
    return fail(FMOE_ERR_ALIGN, "host_slabs and dev_slabs must be 16-byte aligned");
  const size_t span = (size_t)(n_slots - 1) * (size_t)slab_stride + (size_t)slab_bytes;
  if (overlap(host_slabs, span, dev_slabs, span)) return fail(FMOE_ERR_SHAPE, "host_slabs overlaps dev_slabs");
  // The host tier must be pinned host memory the GPU can read: anything else is
  // rejected here instead of faulting in the kernel.
  hipPointerAttribute_t attr;
  hipError_t he = hipPointerGetAttributes(&attr, host_slabs);
  if (he != hipSuccess || attr.type != hipMemoryTypeHost || !attr.devicePointer) {
    (void)hipGetLastError();
    return fail(FMOE_ERR_UNSUPPORTED, "host_slabs is not pinned host memory mapped for the GPU");
  }
  fmoe::FetchArgs a{idx, n_idx, shared, (const uint8_t*)attr.devicePointer, (uint8_t*)dev_slabs,
                    slab_bytes, slab_stride, tags, n_slots, tag, n_copied};
  he = fmoe::launch_fetch(a, (hipStream_t)stream);
  if (he != hipSuccess) return hip_fail(he, "fetch kernels");
  return FMOE_OK;
}

fmoe_status fmoe_fetch_experts(const int32_t* idx, int32_t n_idx, int32_t shared,
                               const void* host_slabs, int64_t slab_bytes, int64_t slab_stride,
                               void* dev_slabs, int32_t* tags, int32_t n_slots, int32_t tag,
                               int32_t* n_copied, void* stream) {
  return finish(fmoe_fetch_experts_impl(idx, n_idx, shared, host_slabs, slab_bytes, slab_stride,
                                        dev_slabs, tags, n_slots, tag, n_copied, stream),
                stream, "fetch (debug sync)");
}

fmoe_status fmoe_moe_layer_forward_noalloc(const fmoe_layer* L, int32_t T, const float* x,
                                           const float* residual, float* h_out, float* y_out,
                                           int32_t* idx_out, float* w_out, float* moe_out,
                                           void* stream) {
  static_assert(fmoe::kStaticScratchBytes == FMOE_STATIC_SCRATCH_BYTES, "scratch size");
  fmoe_status st = layer_args_check(L, T, x, residual, h_out, y_out, moe_out);
  if (st != FMOE_OK || T == 0) return st;
  const size_t need = fmoe_workspace_size(L, T);
  if (need > fmoe::kStaticScratchBytes)
    return fail(FMOE_ERR_WORKSPACE,
                "T=%d needs %zu bytes of workspace; the static scratch holds %zu "
                "(use fmoe_moe_layer_forward with a workspace)",
                (int)T, need, fmoe::kStaticScratchBytes);
  void* ws = nullptr;
  const hipError_t e = fmoe::static_scratch((hipStream_t)stream, &ws);
  if (e == hipErrorStreamCaptureUnsupported)
    return fail(FMOE_ERR_HIP, "the first call on a device clears the static scratch and "
                              "must not be under graph capture");
  if (e != hipSuccess) return hip_fail(e, "static scratch set-up");
  return finish(fmoe_moe_layer_forward_impl(L, T, x, residual, h_out, y_out, idx_out, w_out,
                                            moe_out, ws, fmoe::kStaticScratchBytes, stream),
                stream, "layer (debug sync)");
}

}  // extern "C"
