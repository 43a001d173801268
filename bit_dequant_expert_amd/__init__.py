"""Python binding of libfmoe.so: quantised MoE decode layer for AMD MI355X.

Argument marshalling only.  Every function here forwards to the C ABI of the
same name declared in include/fmoe.h; all arithmetic runs in the library's HIP
kernels.  Tensors are PyTorch device tensors (used only as device memory);
`stream` is a torch.cuda.Stream, a raw hipStream_t integer, or None for the
current stream.  A non-OK status raises FmoeError with the library's message.

The library must have been built (``python -m bit_dequant_expert_amd.build``
or ``__graft_entry__.build()``); importing the binding without it fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfmoe.so")
# The phase-trace build (same kernels, plus wall-clock stamps of the one-token
# kernel's phases); selected by use_trace_library() before the first call.
TRACE_LIB_PATH = os.path.join(PKG, "libfmoe_trace.so")
# The host-sanitizer build (host code with AddressSanitizer and UBSan, the same
# device code), for CPU runs with the sanitizer runtimes preloaded; selected
# by use_sanitizer_library() or FMOE_SANITIZER_BUILD=1 before the first call.
SAN_LIB_PATH = os.path.join(PKG, "libfmoe_san.so")
if os.environ.get("FMOE_SANITIZER_BUILD") == "1":
    LIB_PATH = SAN_LIB_PATH


def use_trace_library():
    """Load the phase-trace build instead of the plain one (before lib())."""
    global LIB_PATH
    if _lib is not None:
        raise RuntimeError("the library is already loaded")
    LIB_PATH = TRACE_LIB_PATH

def use_sanitizer_library():
    """Load the host-sanitizer build instead of the plain one (before lib())."""
    global LIB_PATH
    if _lib is not None:
        raise RuntimeError("the library is already loaded")
    LIB_PATH = SAN_LIB_PATH


FMOE_OK, FMOE_ERR_NULL, FMOE_ERR_SHAPE, FMOE_ERR_ALIGN = 0, 1, 2, 3
FMOE_ERR_UNSUPPORTED, FMOE_ERR_WORKSPACE, FMOE_ERR_HIP = 4, 5, 6
FMOE_F32, FMOE_BF16 = 0, 1

STATUS_NAMES = {0: "FMOE_OK", 1: "FMOE_ERR_NULL", 2: "FMOE_ERR_SHAPE", 3: "FMOE_ERR_ALIGN",
                4: "FMOE_ERR_UNSUPPORTED", 5: "FMOE_ERR_WORKSPACE", 6: "FMOE_ERR_HIP"}

# Every symbol include/fmoe.h declares.
ABI_SYMBOLS = ("fmoe_abi_version", "fmoe_last_error", "fmoe_slab_layout", "fmoe_route_topk",
               "fmoe_route_workspace_size", "fmoe_dequant_gemv", "fmoe_expert_ffn",
               "fmoe_expert_ffn_workspace_size", "fmoe_moe_layer_forward",
               "fmoe_workspace_size", "fmoe_wait_timeout_offset", "fmoe_get_paths",
               "fmoe_set_paths", "fmoe_moe_layer_forward_noalloc", "fmoe_deltanet_step",
               "fmoe_attention_decode", "fmoe_attention_workspace_size", "fmoe_fetch_experts",
               "fmoe_moe_stack_forward")


class FmoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class fmoe_qformat(C.Structure):
    _fields_ = [("bits", C.c_int32), ("group", C.c_int32), ("sdtype", C.c_int32)]


class fmoe_qmat(C.Structure):
    _fields_ = [("q", C.c_void_p), ("scale", C.c_void_p), ("bias", C.c_void_p),
                ("n", C.c_int32), ("k", C.c_int32)]


class fmoe_expert(C.Structure):
    _fields_ = [("gate", fmoe_qmat), ("up", fmoe_qmat), ("down", fmoe_qmat)]


class fmoe_layer(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("inter", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("fmt", fmoe_qformat), ("router_w", C.c_void_p),
                ("slabs", C.c_void_p), ("slab_stride", C.c_int64),
                ("shared_gate_w", C.c_void_p), ("norm_w", C.c_void_p),
                ("norm_eps", C.c_float)]


class fmoe_paths(C.Structure):
    _fields_ = [("no_fused", C.c_int32), ("no_mfma", C.c_int32), ("mfma_min_tokens", C.c_int32),
                ("debug_sync", C.c_int32), ("t1_counters", C.c_int32),
                ("wait_limit_us", C.c_int32), ("test_stall_part", C.c_int32)]


_lib = None


def lib() -> C.CDLL:
    """The loaded libfmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_dequant_expert_amd.build`")
        L = C.CDLL(LIB_PATH)
        P, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.fmoe_abi_version.argtypes, L.fmoe_abi_version.restype = [], i32
        L.fmoe_last_error.argtypes, L.fmoe_last_error.restype = [], C.c_char_p
        L.fmoe_wait_timeout_offset.argtypes, L.fmoe_wait_timeout_offset.restype = [], sz
        L.fmoe_get_paths.argtypes, L.fmoe_get_paths.restype = [C.POINTER(fmoe_paths)], None
        L.fmoe_set_paths.argtypes, L.fmoe_set_paths.restype = [C.POINTER(fmoe_paths)], C.c_int
        L.fmoe_slab_layout.argtypes = [i32, i32, C.POINTER(fmoe_qformat), C.POINTER(C.c_int64)]
        L.fmoe_slab_layout.restype = i64
        L.fmoe_route_topk.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P, sz, P]
        L.fmoe_route_topk.restype = C.c_int
        L.fmoe_route_workspace_size.argtypes, L.fmoe_route_workspace_size.restype = [i32, i32], sz
        L.fmoe_dequant_gemv.argtypes = [C.POINTER(fmoe_qmat), C.POINTER(fmoe_qformat), P, P, P]
        L.fmoe_dequant_gemv.restype = C.c_int
        L.fmoe_expert_ffn.argtypes = [C.POINTER(fmoe_expert), C.POINTER(fmoe_qformat), P, P, P,
                                      sz, P]
        L.fmoe_expert_ffn.restype = C.c_int
        L.fmoe_expert_ffn_workspace_size.argtypes = [C.POINTER(fmoe_expert),
                                                     C.POINTER(fmoe_qformat)]
        L.fmoe_expert_ffn_workspace_size.restype = sz
        L.fmoe_moe_layer_forward.argtypes = [C.POINTER(fmoe_layer), i32, P, P, P, P, P, P, P, P,
                                             sz, P]
        L.fmoe_moe_layer_forward.restype = C.c_int
        L.fmoe_moe_layer_forward_noalloc.argtypes = [C.POINTER(fmoe_layer), i32, P, P, P, P, P,
                                                     P, P, P]
        L.fmoe_moe_layer_forward_noalloc.restype = C.c_int
        L.fmoe_deltanet_step.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, P]
        L.fmoe_deltanet_step.restype = C.c_int
        L.fmoe_attention_decode.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, C.c_float, P,
                                            P, sz, P]
        L.fmoe_attention_decode.restype = C.c_int
        L.fmoe_attention_workspace_size.argtypes = [i32, i32, i32, i32]
        L.fmoe_attention_workspace_size.restype = sz
        L.fmoe_fetch_experts.argtypes = [P, i32, i32, P, i64, i64, P, P, i32, i32, P, P]
        L.fmoe_fetch_experts.restype = C.c_int
        L.fmoe_moe_stack_forward.argtypes = [C.POINTER(fmoe_layer), i32, i32, P, P, P, P, P, P,
                                             P, sz, P]
        L.fmoe_moe_stack_forward.restype = C.c_int
        L.fmoe_workspace_size.argtypes = [C.POINTER(fmoe_layer), i32]
        L.fmoe_workspace_size.restype = sz
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t):
    return t.numel() * t.element_size()


def _check(status: int):
    if status != FMOE_OK:
        raise FmoeError(status, lib().fmoe_last_error().decode())


def qformat(bits: int, group: int, bf16: bool) -> fmoe_qformat:
    return fmoe_qformat(bits, group, FMOE_BF16 if bf16 else FMOE_F32)


def qmat(q, scale, bias, n: int, k: int) -> fmoe_qmat:
    """Descriptor of one quantised matrix; keeps the tensors it points at alive."""
    m = fmoe_qmat(_ptr(q), _ptr(scale), _ptr(bias), n, k)
    m._refs = (q, scale, bias)
    return m


def fmoe_abi_version() -> int:
    return lib().fmoe_abi_version()


def fmoe_last_error() -> str:
    return lib().fmoe_last_error().decode()


def fmoe_wait_timeout_offset() -> int:
    return int(lib().fmoe_wait_timeout_offset())


def fmoe_get_paths() -> fmoe_paths:
    p = fmoe_paths()
    lib().fmoe_get_paths(C.byref(p))
    return p


def fmoe_set_paths(p: fmoe_paths):
    _check(lib().fmoe_set_paths(C.byref(p)))


class paths:
    """Context manager that changes the kernel-path selection (fmoe_paths
    fields as keywords) and restores the previous one on exit."""

    def __init__(self, **kw):
        self.kw = kw

    def __enter__(self):
        self.saved = fmoe_get_paths()
        p = fmoe_get_paths()
        for k, v in self.kw.items():
            setattr(p, k, int(v))
        fmoe_set_paths(p)
        return p

    def __exit__(self, *exc):
        fmoe_set_paths(self.saved)
        return False


def fmoe_slab_layout(hidden: int, inter: int, fmt: fmoe_qformat):
    off = (C.c_int64 * 9)()
    size = lib().fmoe_slab_layout(hidden, inter, C.byref(fmt), off)
    if size < 0:
        raise FmoeError(FMOE_ERR_SHAPE, fmoe_last_error())
    return list(off), int(size)


def fmoe_route_workspace_size(T: int, E: int) -> int:
    return lib().fmoe_route_workspace_size(T, E)


def fmoe_route_topk(router_w, x, k, idx, w, logits=None, ws=None, stream=None):
    """router_w [E,H] fp32, x [T,H] fp32 -> idx [T,k] int32, w [T,k] fp32 (in place)."""
    E, H = router_w.shape
    T = x.shape[0] if x.dim() == 2 else 1
    _check(lib().fmoe_route_topk(_ptr(router_w), _ptr(x), T, H, E, k, _ptr(idx), _ptr(w),
                                 _ptr(logits), _ptr(ws), 0 if ws is None else _nbytes(ws),
                                 _stream(stream)))


def fmoe_dequant_gemv(W: fmoe_qmat, fmt: fmoe_qformat, x, y, stream=None):
    _check(lib().fmoe_dequant_gemv(C.byref(W), C.byref(fmt), _ptr(x), _ptr(y), _stream(stream)))


def fmoe_expert_ffn_workspace_size(e: fmoe_expert, fmt: fmoe_qformat) -> int:
    return lib().fmoe_expert_ffn_workspace_size(C.byref(e), C.byref(fmt))


def fmoe_expert_ffn(e: fmoe_expert, fmt: fmoe_qformat, x, y, ws, stream=None):
    _check(lib().fmoe_expert_ffn(C.byref(e), C.byref(fmt), _ptr(x), _ptr(y), _ptr(ws),
                                 0 if ws is None else _nbytes(ws), _stream(stream)))


def fmoe_layer_desc(hidden, inter, n_experts, top_k, fmt, router_w, slabs, slab_stride,
                    shared_gate_w, norm_w, norm_eps=1e-6) -> fmoe_layer:
    L = fmoe_layer(hidden, inter, n_experts, top_k, fmt, _ptr(router_w), _ptr(slabs),
                   slab_stride, _ptr(shared_gate_w), _ptr(norm_w), norm_eps)
    L._refs = (router_w, slabs, shared_gate_w, norm_w)   # keep the buffers alive
    return L


def fmoe_workspace_size(L: fmoe_layer, T: int) -> int:
    return lib().fmoe_workspace_size(C.byref(L), T)


def fmoe_moe_layer_forward(L: fmoe_layer, T: int, x, residual, h_out, y_out, idx_out=None,
                           w_out=None, moe_out=None, ws=None, stream=None):
    _check(lib().fmoe_moe_layer_forward(
        C.byref(L), T, _ptr(x), _ptr(residual), _ptr(h_out), _ptr(y_out), _ptr(idx_out),
        _ptr(w_out), _ptr(moe_out), _ptr(ws), 0 if ws is None else _nbytes(ws),
        _stream(stream)))


def fmoe_moe_stack_forward(layers, T: int, x, residual, h_out, y_out, idx_out=None,
                           w_out=None, ws=None, stream=None):
    """layers: a sequence of fmoe_layer (or a ctypes array of them)."""
    arr = layers if isinstance(layers, C.Array) else (fmoe_layer * max(1, len(layers)))(*layers)
    _check(lib().fmoe_moe_stack_forward(
        arr, len(layers), T, _ptr(x), _ptr(residual), _ptr(h_out), _ptr(y_out), _ptr(idx_out),
        _ptr(w_out), _ptr(ws), 0 if ws is None else _nbytes(ws), _stream(stream)))


def fmoe_moe_layer_forward_noalloc(L: fmoe_layer, T: int, x, residual, h_out, y_out,
                                   idx_out=None, w_out=None, moe_out=None, stream=None):
    _check(lib().fmoe_moe_layer_forward_noalloc(
        C.byref(L), T, _ptr(x), _ptr(residual), _ptr(h_out), _ptr(y_out), _ptr(idx_out),
        _ptr(w_out), _ptr(moe_out), _stream(stream)))


STATIC_SCRATCH_BYTES = 16 << 20


def fmoe_fetch_experts(idx, n_idx, shared, host_slabs, slab_bytes, slab_stride, dev_slabs, tags,
                       n_slots, tag, n_copied=None, stream=None):
    _check(lib().fmoe_fetch_experts(_ptr(idx), n_idx, shared, _ptr(host_slabs), slab_bytes,
                                    slab_stride, _ptr(dev_slabs), _ptr(tags), n_slots, tag,
                                    _ptr(n_copied), _stream(stream)))


def fmoe_attention_workspace_size(batch, n_kv_heads, head_dim, cap) -> int:
    return lib().fmoe_attention_workspace_size(batch, n_kv_heads, head_dim, cap)


def fmoe_attention_decode(q, k_cache, v_cache, lens, out, ws, rope_base=10000.0, stream=None):
    """q [B, NQ, D] fp32, caches [B, NKV, cap, D] bf16 bits (int16/uint16 tensors),
    lens [B] int32 on the device, out [B, NQ, D]; shapes taken from q and the cache."""
    B, NQ, D = q.shape
    _, NKV, cap, _ = k_cache.shape
    _check(lib().fmoe_attention_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens), B, NQ,
                                       NKV, D, cap, float(rope_base), _ptr(out), _ptr(ws),
                                       0 if ws is None else _nbytes(ws), _stream(stream)))


def fmoe_deltanet_step(q, k, v, decay, beta, state, out, stream=None):
    """state [B, NH, dk, dv] is updated in place; shapes are taken from it."""
    B, NH, dk, dv = state.shape
    _check(lib().fmoe_deltanet_step(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(beta),
                                    _ptr(state), _ptr(out), B, NH, dk, dv, _stream(stream)))


_raw_fwd = None


def fmoe_moe_layer_forward_raw(Lp, T, x, residual, h_out, y_out, idx_out, w_out, moe_out,
                               ws, ws_bytes, stream) -> int:
    """Pointer-level call (the layer descriptor's address and raw device
    pointers as ints) for tight launch loops; returns the status."""
    global _raw_fwd
    if _raw_fwd is None:
        P = C.c_void_p
        proto = C.CFUNCTYPE(C.c_int, P, C.c_int32, P, P, P, P, P, P, P, P, C.c_size_t, P)
        _raw_fwd = proto(C.cast(lib().fmoe_moe_layer_forward, C.c_void_p).value)
    return _raw_fwd(Lp, T, x, residual, h_out, y_out, idx_out, w_out, moe_out, ws, ws_bytes,
                    stream)
