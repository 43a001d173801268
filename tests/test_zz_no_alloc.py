"""The allocation-free layer call (fmoe_moe_layer_forward_noalloc) against the
layer call with a caller-owned workspace, through the C ABI.

Bar (the parity bar of the layer): expert indices bit-exact, routing weights
within 1e-5, moe / h / y within relative L2 2e-3 per token.  Two calls in a
row share the static scratch, the second with fewer tokens than the first;
both calls are compared.  The one-token case is also checked against the
oracle, and replayed from a HIP graph.
"""
import numpy as np
import pytest
import torch

import bit_dequant_expert_amd as fm
import synth
from qtest_util import rel_l2
from test_gpu_parity import GpuLayer, check_layer, dev, note

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _outputs(cfg, T):
    return dict(h=torch.empty(T, cfg.H, device="cuda"), y=torch.empty(T, cfg.H, device="cuda"),
                moe=torch.empty(T, cfg.H, device="cuda"),
                idx=torch.empty(T, cfg.k, dtype=torch.int32, device="cuda"),
                w=torch.empty(T, cfg.k, device="cuda"))


def _noalloc(gl, x, r):
    T = x.shape[0]
    out = _outputs(gl.cfg, T)
    fm.fmoe_moe_layer_forward_noalloc(gl.L, T, x, r, out["h"], out["y"], out["idx"], out["w"],
                                      out["moe"])
    return out


def _host(out):
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _same_bar(a, b):
    T = a["y"].shape[0]
    assert np.array_equal(a["idx"], b["idx"])
    assert np.allclose(a["w"], b["w"], rtol=0, atol=1e-5)
    for t in range(T):
        for name in ("moe", "h", "y"):
            err = rel_l2(a[name][t], b[name][t])
            assert err <= TOL, (t, name, err)
        assert np.isfinite(a["y"][t]).all(), t


@pytest.mark.parametrize("cfg_name,T1,T2", [("tiny", 9, 2), ("layer4", 4, 1)])
def test_noalloc_matches_workspace_call(cfg_name, T1, T2):
    cfg = synth.CONFIGS[cfg_name]
    note(f"noalloc {cfg_name} T={T1} then T={T2}")
    gl = GpuLayer(cfg, random_gamma=cfg_name == "tiny")
    x = synth.activations(cfg, T1, pool=T1)
    r = synth.normal(cfg.seed, 2, 77, (T1, cfg.H))
    xd, rd = dev(x), dev(r)
    # Both calls enqueued back to back on one stream (the second overwrites
    # what the first left in the scratch), then read.
    a1 = _noalloc(gl, xd, rd)
    a2 = _noalloc(gl, xd[:T2], rd[:T2])
    got1, got2 = _host(a1), _host(a2)
    ref1 = gl.forward(x, r)
    ref2 = gl.forward(x[:T2], r[:T2])
    _same_bar(got1, ref1)
    _same_bar(got2, ref2)
    if T2 == 1:
        check_layer(gl, x[:1], r[:1], got2, [0])


def test_noalloc_graph_replays():
    # After the first (uncaptured) call on the device, the call can be
    # captured; every replay matches the eager call.
    cfg = synth.CONFIGS["tiny"]
    note("noalloc graph replay")
    gl = GpuLayer(cfg)
    n = 3
    x = dev(synth.activations(cfg, n, pool=n))
    h = torch.empty(n, cfg.H, device="cuda")
    y = torch.empty(n, cfg.H, device="cuda")
    for t in range(n):
        fm.fmoe_moe_layer_forward_noalloc(gl.L, 1, x[t], x[t], h[t], y[t])
    torch.cuda.synchronize()
    h_ref, y_ref = h.clone(), y.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for t in range(n):
            fm.fmoe_moe_layer_forward_noalloc(gl.L, 1, x[t], x[t], h[t], y[t],
                                              stream=torch.cuda.current_stream())
    for rep in range(3):
        h.zero_()
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, h_ref) and torch.equal(y, y_ref), rep
        _ = (x * 2).sum().item()


def test_noalloc_rejects_oversize():
    cfg = synth.CONFIGS["tiny"]
    gl = GpuLayer(cfg)
    T = next(t for t in range(1, 1 << 16)
             if fm.fmoe_workspace_size(gl.L, t) > fm.STATIC_SCRATCH_BYTES)
    x = torch.zeros(T, cfg.H, device="cuda")
    h = torch.empty(T, cfg.H, device="cuda")
    y = torch.empty(T, cfg.H, device="cuda")
    with pytest.raises(fm.FmoeError) as ei:
        fm.fmoe_moe_layer_forward_noalloc(gl.L, T, x, x, h, y)
    assert ei.value.status == fm.FMOE_ERR_WORKSPACE
