"""ctypes front end of the CPU oracle (oracle/fmoe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
CPU-baseline leg of bench.py.  The product package never imports this module.

All results come back as float64 numpy arrays (the oracle computes in fp64);
inputs are passed as they are stored (uint8 packed codes, fp32 or bf16-bit
uint16 scales, fp32 vectors).
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        san = os.environ.get("FMOE_SANITIZER_BUILD") == "1"
        path = _build.SAN_LIB if san else _build.LIB
        if not os.path.exists(path):
            _build.build(sanitize=san)
        L = C.CDLL(path)
        P = C.c_void_p
        i32, i64, dbl = C.c_int, C.c_int64, C.c_double

        class Fmt(C.Structure):
            _fields_ = [("bits", C.c_int32), ("group", C.c_int32), ("sbytes", C.c_int32)]

        L.Fmt = Fmt
        L.or_code.argtypes = [P, i32, i64]
        L.or_code.restype = i32
        L.or_sb.argtypes = [P, i32, i64]
        L.or_sb.restype = dbl
        L.or_slab_layout.argtypes = [i32, i32, Fmt, P]
        L.or_slab_layout.restype = i64
        for name in ("or_gemv", "or_gemv_fma_form", "or_gemv_groupsum"):
            getattr(L, name).argtypes = [P, P, P, Fmt, i32, i32, P, P]
            getattr(L, name).restype = None
        L.or_dequant.argtypes = [P, P, P, Fmt, i32, i32, P]
        L.or_dequant.restype = None
        L.or_gemv_naive_f32.argtypes = [P, P, P, Fmt, i32, i32, P, P]
        L.or_gemv_naive_f32.restype = None
        L.or_gemv_dense.argtypes = [P, i32, i32, P, P]
        L.or_gemv_dense.restype = None
        L.or_route.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P]
        L.or_route.restype = i32
        L.or_topk_kpass.argtypes = [P, i32, i32, P]
        L.or_topk_kpass.restype = None
        L.or_silu.argtypes = [dbl]
        L.or_silu.restype = dbl
        L.or_expert_ffn.argtypes = [P, i32, i32, Fmt, P, P]
        L.or_expert_ffn.restype = None
        L.or_rmsnorm.argtypes = [P, P, i32, dbl, P]
        L.or_rmsnorm.restype = None
        L.or_moe_token.argtypes = [P, P, i32, P, i32, i32, Fmt, P, P, dbl, P, P, P, P, P, P]
        L.or_moe_token.restype = None
        L.or_layer_forward.argtypes = [P, P, i64, P, P, dbl, i32, i32, i32, i32, Fmt, i32,
                                       P, P, P, P, P, P, P, P, P, P, P]
        L.or_layer_forward.restype = i32
        L.or_deltanet_step.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, P, P]
        L.or_deltanet_step.restype = None
        L.or_rope_deinterleave.argtypes = [P, i32, i32, dbl, P]
        L.or_rope_deinterleave.restype = None
        L.or_attention_decode.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, dbl, P]
        L.or_attention_decode.restype = None
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def fmt(bits, group, sbytes):
    return lib().Fmt(bits, group, sbytes)


def _sdt(sbytes):
    return np.uint16 if sbytes == 2 else np.float32


def code(row, bits, k):
    row = _c(row, np.uint8)
    return lib().or_code(_p(row), bits, k)


def slab_layout(H, I, bits, group, sbytes):
    off = np.zeros(9, np.int64)
    size = lib().or_slab_layout(H, I, fmt(bits, group, sbytes), _p(off))
    return off, int(size)


def dequant(q, s, b, bits, group, sbytes, N, K):
    q, s, b = _c(q, np.uint8), _c(s, _sdt(sbytes)), _c(b, _sdt(sbytes))
    W = np.empty((N, K), np.float64)
    lib().or_dequant(_p(q), _p(s), _p(b), fmt(bits, group, sbytes), N, K, _p(W))
    return W


def _gemv(name, q, s, b, bits, group, sbytes, N, K, x):
    q, s, b = _c(q, np.uint8), _c(s, _sdt(sbytes)), _c(b, _sdt(sbytes))
    x = _c(x, np.float64)
    y = np.empty(N, np.float64)
    getattr(lib(), name)(_p(q), _p(s), _p(b), fmt(bits, group, sbytes), N, K, _p(x), _p(y))
    return y


def gemv(q, s, b, bits, group, sbytes, N, K, x):
    """Quantised GEMV by definition (dequantise, then dense fp64 product)."""
    return _gemv("or_gemv", q, s, b, bits, group, sbytes, N, K, x)


def gemv_fma_form(q, s, b, bits, group, sbytes, N, K, x):
    return _gemv("or_gemv_fma_form", q, s, b, bits, group, sbytes, N, K, x)


def gemv_groupsum(q, s, b, bits, group, sbytes, N, K, x):
    return _gemv("or_gemv_groupsum", q, s, b, bits, group, sbytes, N, K, x)


def gemv_naive_f32(q, s, b, bits, group, sbytes, N, K, x):
    q, s, b = _c(q, np.uint8), _c(s, _sdt(sbytes)), _c(b, _sdt(sbytes))
    x = _c(x, np.float32)
    y = np.empty(N, np.float32)
    lib().or_gemv_naive_f32(_p(q), _p(s), _p(b), fmt(bits, group, sbytes), N, K, _p(x), _p(y))
    return y


def gemv_dense(W, x):
    W = _c(W, np.float64)
    x = _c(x, np.float64)
    N, K = W.shape
    y = np.empty(N, np.float64)
    lib().or_gemv_dense(_p(W), N, K, _p(x), _p(y))
    return y


def route(Wr, x, k):
    """Returns (idx [T,k] int32, w [T,k], logits [T,E], gap [T], status)."""
    Wr = _c(Wr, np.float32)
    x = _c(np.atleast_2d(x), np.float32)
    E, H = Wr.shape
    T = x.shape[0]
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lg = np.empty((T, E), np.float64)
    gap = np.empty(T, np.float64)
    st = lib().or_route(_p(Wr), _p(x), T, H, E, k, _p(idx), _p(w), _p(lg), _p(gap))
    return idx, w, lg, gap, st


def topk_kpass(logits, k):
    logits = _c(logits, np.float64)
    idx = np.empty(k, np.int32)
    lib().or_topk_kpass(_p(logits), logits.shape[0], k, _p(idx))
    return idx


def silu(z):
    return lib().or_silu(float(z))


def expert_ffn(slab, H, I, bits, group, sbytes, x):
    slab = _c(slab, np.uint8)
    x = _c(x, np.float64)
    y = np.empty(H, np.float64)
    lib().or_expert_ffn(_p(slab), H, I, fmt(bits, group, sbytes), _p(x), _p(y))
    return y


def rmsnorm(h, gamma, eps):
    h = _c(h, np.float64)
    gamma = _c(gamma, np.float32)
    y = np.empty_like(h)
    lib().or_rmsnorm(_p(h), _p(gamma), h.shape[0], float(eps), _p(y))
    return y


def moe_token(routed_slabs, w, shared_slab, H, I, bits, group, sbytes,
              wsg, gamma, eps, x, r):
    """One token given its routing; routed_slabs is a list of uint8 arrays."""
    k = len(routed_slabs)
    rs = [_c(s, np.uint8) for s in routed_slabs]
    ptrs = (C.c_void_p * max(k, 1))(*[s.ctypes.data for s in rs])
    w = _c(w, np.float64)
    shared_slab = _c(shared_slab, np.uint8)
    wsg, gamma = _c(wsg, np.float32), _c(gamma, np.float32)
    x, r = _c(x, np.float32), _c(r, np.float32)
    g = C.c_double(0.0)
    moe = np.empty(H, np.float64)
    h = np.empty(H, np.float64)
    y = np.empty(H, np.float64)
    lib().or_moe_token(C.cast(ptrs, C.c_void_p), _p(w), k, _p(shared_slab), H, I,
                       fmt(bits, group, sbytes), _p(wsg), _p(gamma), float(eps),
                       _p(x), _p(r), C.byref(g), _p(moe), _p(h), _p(y))
    return dict(g=g.value, moe=moe, h=h, y=y)


def layer_forward(Wr, slabs, slab_stride, wsg, gamma, eps, H, I, E, k,
                  bits, group, sbytes, x, r, forced_idx=None):
    """Whole layer for T tokens.  slabs: uint8 array of (E+1)*slab_stride bytes."""
    Wr = _c(Wr, np.float32)
    slabs = _c(slabs, np.uint8)
    wsg, gamma = _c(wsg, np.float32), _c(gamma, np.float32)
    x = _c(np.atleast_2d(x), np.float32)
    r = _c(np.atleast_2d(r), np.float32)
    T = x.shape[0]
    fi = None if forced_idx is None else _c(np.atleast_2d(forced_idx), np.int32)
    out = dict(idx=np.empty((T, k), np.int32), w=np.empty((T, k)), logits=np.empty((T, E)),
               gap=np.empty(T), g=np.empty(T), moe=np.empty((T, H)), h=np.empty((T, H)),
               y=np.empty((T, H)))
    st = lib().or_layer_forward(_p(Wr), _p(slabs), int(slab_stride), _p(wsg), _p(gamma),
                                float(eps), H, I, E, k, fmt(bits, group, sbytes), T,
                                _p(x), _p(r), _p(fi), _p(out["idx"]), _p(out["w"]),
                                _p(out["logits"]), _p(out["gap"]), _p(out["g"]),
                                _p(out["moe"]), _p(out["h"]), _p(out["y"]))
    out["status"] = st
    return out


# ------------------------------------------------- Gated DeltaNet, attention
def deltanet_step(q, k, v, a, beta, state):
    """One Gated DeltaNet decode step (fmoe_oracle_next.h).  q, k [B, NH, dk],
    v [B, NH, dv], a, beta [B, NH], state [B, NH, dk, dv] (all fp32).  Returns
    (new state, out) in fp64."""
    B, NH, dk, dv = state.shape
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    a, beta, state = _c(a, np.float32), _c(beta, np.float32), _c(state, np.float32)
    assert q.shape == (B, NH, dk) and k.shape == (B, NH, dk) and v.shape == (B, NH, dv)
    assert a.shape == (B, NH) and beta.shape == (B, NH)
    s_out = np.empty((B, NH, dk, dv), np.float64)
    out = np.empty((B, NH, dv), np.float64)
    lib().or_deltanet_step(_p(q), _p(k), _p(v), _p(a), _p(beta), _p(state), B, NH, dk, dv,
                           _p(s_out), _p(out))
    return s_out, out


def rope_deinterleave(x, pos, base=10000.0):
    x = _c(x, np.float32)
    y = np.empty(x.shape[0], np.float64)
    lib().or_rope_deinterleave(_p(x), x.shape[0], int(pos), float(base), _p(y))
    return y


def attention_decode(q, kc, vc, lens, base=10000.0):
    """Decode attention (fmoe_oracle_next.h): q [B, NQ, D] fp32 (interleaved
    pairs, unrotated), kc / vc [B, NKV, cap, D] bf16 bits (uint16), lens [B]
    (>= 1).  Returns out [B, NQ, D] fp64."""
    q = _c(q, np.float32)
    kc, vc = _c(kc, np.uint16), _c(vc, np.uint16)
    lens = _c(lens, np.int32)
    B, NQ, D = q.shape
    _, NKV, cap, _ = kc.shape
    assert kc.shape == vc.shape == (B, NKV, cap, D) and lens.shape == (B,)
    assert NQ % NKV == 0 and (lens >= 1).all() and (lens <= cap).all()
    out = np.empty((B, NQ, D), np.float64)
    lib().or_attention_decode(_p(q), _p(kc), _p(vc), _p(lens), B, NQ, NKV, D, cap, float(base),
                              _p(out))
    return out
