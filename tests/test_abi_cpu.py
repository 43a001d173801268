"""The C ABI library on the host: it loads, exports every symbol the header
declares, its host-side slab layout agrees with the oracle's, and invalid
arguments are rejected with the documented status before anything is
enqueued.  No GPU is touched: every call here fails validation, so no kernel
is launched."""
import ctypes as C
import os
import re

import pytest

import bit_dequant_expert_amd as fm
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Fake, suitably aligned device addresses: validation only inspects values.
A = 0x7F0000000000


def _declared_symbols():
    txt = open(os.path.join(ROOT, "include", "fmoe.h")).read()
    return sorted(set(re.findall(r"\b(fmoe_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = fm.lib()
    declared = _declared_symbols()
    assert declared == sorted(fm.ABI_SYMBOLS)
    for name in declared:
        assert getattr(L, name) is not None


def test_abi_version():
    assert fm.fmoe_abi_version() == 1


@pytest.mark.parametrize("H,I,bits,G,bf16", [(4096, 1024, 4, 64, True), (4096, 1024, 2, 64, True),
                                             (256, 128, 4, 32, False), (512, 256, 2, 32, False)])
def test_slab_layout_matches_oracle(H, I, bits, G, bf16):
    off, size = fm.fmoe_slab_layout(H, I, fm.qformat(bits, G, bf16))
    ooff, osize = oracle.slab_layout(H, I, bits, G, 2 if bf16 else 4)
    assert size == osize and off == list(ooff)


def test_slab_layout_rejects_bad_format():
    with pytest.raises(fm.FmoeError):
        fm.fmoe_slab_layout(4096, 1024, fm.qformat(3, 64, True))


def _gemv(W, fmt, x=A, y=A + 0x100000):
    return fm.lib().fmoe_dequant_gemv(C.byref(W), C.byref(fmt), x, y, None)


def test_gemv_validation():
    f = fm.qformat(4, 64, True)
    ok = fm.fmoe_qmat(A, A + 0x10000, A + 0x20000, 1024, 4096)
    assert _gemv(fm.fmoe_qmat(0, A, A, 8, 4096), f) == fm.FMOE_ERR_NULL
    assert _gemv(ok, f, x=0) == fm.FMOE_ERR_NULL
    assert _gemv(fm.fmoe_qmat(A + 4, A, A, 8, 4096), f) == fm.FMOE_ERR_ALIGN
    assert _gemv(ok, f, x=A + 8) == fm.FMOE_ERR_ALIGN
    assert _gemv(fm.fmoe_qmat(A, A, A, 8, 4000), f) == fm.FMOE_ERR_SHAPE        # k % group
    assert _gemv(fm.fmoe_qmat(A, A, A, 0, 4096), f) == fm.FMOE_ERR_SHAPE
    assert _gemv(ok, fm.qformat(3, 64, True)) == fm.FMOE_ERR_UNSUPPORTED
    assert _gemv(ok, fm.qformat(4, 128, True)) == fm.FMOE_ERR_UNSUPPORTED
    assert _gemv(fm.fmoe_qmat(A, A, A, 8, 64 * 96), f) == fm.FMOE_ERR_UNSUPPORTED  # 192 segs
    assert _gemv(ok, f, x=A, y=A + 64) == fm.FMOE_ERR_SHAPE                       # overlap
    assert "overlaps" in fm.fmoe_last_error()


def _route(T=1, H=4096, E=512, k=4, ws=A, ws_bytes=1 << 30, idx=A, w=A, x=A, Wr=A):
    return fm.lib().fmoe_route_topk(Wr, x, T, H, E, k, idx, w, None, ws, ws_bytes, None)


def test_route_validation():
    assert _route(k=0) == fm.FMOE_ERR_SHAPE
    assert _route(k=600) == fm.FMOE_ERR_SHAPE
    assert _route(k=17, E=64) == fm.FMOE_ERR_UNSUPPORTED
    assert _route(E=4096) == fm.FMOE_ERR_UNSUPPORTED
    assert _route(H=4097) == fm.FMOE_ERR_SHAPE
    assert _route(Wr=0) == fm.FMOE_ERR_NULL
    assert _route(x=A + 4) == fm.FMOE_ERR_ALIGN
    assert _route(idx=0) == fm.FMOE_ERR_NULL
    assert _route(ws=0) == fm.FMOE_ERR_WORKSPACE
    assert _route(ws_bytes=100) == fm.FMOE_ERR_WORKSPACE
    assert _route(ws=A + 16) == fm.FMOE_ERR_ALIGN
    assert _route(T=-1) == fm.FMOE_ERR_SHAPE


def _layer(**kw):
    p = dict(hidden=4096, inter=1024, n_experts=512, top_k=4, bits=4, group=64, bf16=True,
             stride=7077888, slabs=A, router=A, wsg=A, gamma=A, eps=1e-6)
    p.update(kw)
    return fm.fmoe_layer(p["hidden"], p["inter"], p["n_experts"], p["top_k"],
                         fm.qformat(p["bits"], p["group"], p["bf16"]), p["router"], p["slabs"],
                         p["stride"], p["wsg"], p["gamma"], p["eps"])


def _fwd(L, T=1, x=A, r=A, h=A + 0x400000, y=A + 0x800000, moe=None, ws=A + 0x1000000,
         ws_bytes=1 << 34):
    return fm.lib().fmoe_moe_layer_forward(C.byref(L), T, x, r, h, y, None, None, moe, ws,
                                           ws_bytes, None)


def test_layer_validation():
    assert _fwd(_layer(bits=3)) == fm.FMOE_ERR_UNSUPPORTED
    assert _fwd(_layer(top_k=0)) == fm.FMOE_ERR_SHAPE
    assert _fwd(_layer(top_k=513)) == fm.FMOE_ERR_SHAPE
    assert _fwd(_layer(slabs=0)) == fm.FMOE_ERR_NULL
    assert _fwd(_layer(slabs=A + 16)) == fm.FMOE_ERR_ALIGN
    assert _fwd(_layer(stride=7077888 + 16)) == fm.FMOE_ERR_ALIGN
    assert _fwd(_layer(stride=7077888 - 256)) == fm.FMOE_ERR_SHAPE
    assert _fwd(_layer(router=0)) == fm.FMOE_ERR_NULL
    assert _fwd(_layer(inter=1000)) == fm.FMOE_ERR_SHAPE
    assert _fwd(_layer(hidden=64, inter=64, stride=1 << 20)) == fm.FMOE_ERR_UNSUPPORTED
    assert _fwd(_layer(), ws_bytes=1000) == fm.FMOE_ERR_WORKSPACE
    assert _fwd(_layer(), ws=0) == fm.FMOE_ERR_WORKSPACE
    assert _fwd(_layer(), y=A) == fm.FMOE_ERR_SHAPE          # y overlaps x
    assert _fwd(_layer(), h=A + 64, r=A) == fm.FMOE_ERR_SHAPE  # partial overlap
    assert _fwd(_layer(), x=0) == fm.FMOE_ERR_NULL
    assert _fwd(_layer(), T=-2) == fm.FMOE_ERR_SHAPE
    assert _fwd(_layer(eps=-1.0)) == fm.FMOE_ERR_SHAPE
    assert fm.fmoe_last_error()


def test_layer_T0_is_noop():
    assert _fwd(_layer(), T=0) == fm.FMOE_OK


def test_workspace_sizes():
    L = _layer()
    w1 = fm.fmoe_workspace_size(L, 1)
    w32 = fm.fmoe_workspace_size(L, 32)
    assert 0 < w1 < w32 < (64 << 20)
    assert fm.fmoe_route_workspace_size(32, 512) >= 32 * 512 * 8
    e = fm.fmoe_expert(fm.fmoe_qmat(A, A, A, 1024, 4096), fm.fmoe_qmat(A, A, A, 1024, 4096),
                       fm.fmoe_qmat(A, A, A, 4096, 1024))
    assert fm.fmoe_expert_ffn_workspace_size(e, fm.qformat(4, 64, True)) > 0


def test_ffn_validation():
    f = fm.qformat(4, 64, True)
    good = fm.fmoe_qmat(A, A, A, 1024, 4096)
    down = fm.fmoe_qmat(A, A, A, 4096, 1024)
    bad_down = fm.fmoe_qmat(A, A, A, 4096, 512)
    e = fm.fmoe_expert(good, good, bad_down)
    rc = fm.lib().fmoe_expert_ffn(C.byref(e), C.byref(f), A, A + 0x100000, A, 1 << 30, None)
    assert rc == fm.FMOE_ERR_SHAPE
    e = fm.fmoe_expert(good, good, down)
    rc = fm.lib().fmoe_expert_ffn(C.byref(e), C.byref(f), A, A + 0x100000, A, 10, None)
    assert rc == fm.FMOE_ERR_WORKSPACE
