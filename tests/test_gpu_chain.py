"""GPU parity of fmoe_moe_stack_forward: layers chained on the device.

At one token the stack runs up to 64 layers in one launch of the chained
one-token kernel.  It adds the sums of squares in the one-token kernel's order
and builds each next input as the one-token kernel builds y, so its outputs
must equal, bit for bit, one fmoe_moe_layer_forward call per layer fed the
previous layer's y and h; those per-layer calls are checked against the oracle
here as well (teacher-forced on the GPU's own layer inputs).
"""
import numpy as np
import pytest
import torch

import bit_dequant_expert_amd as fm
import synth
from test_gpu_parity import MID, MID2, GpuLayer, _wait_timeouts, check_layer, dev, note

pytestmark = pytest.mark.gpu


def run_stack(layers, x, r, ws, stream=None):
    cfg = layers[0].cfg
    n, T = len(layers), x.shape[0]
    out = dict(h=torch.full((n, T, cfg.H), -1.0, device="cuda"),
               y=torch.full((n, T, cfg.H), -1.0, device="cuda"),
               idx=torch.full((n, T, cfg.k), -1, dtype=torch.int32, device="cuda"),
               w=torch.full((n, T, cfg.k), -1.0, device="cuda"))
    fm.fmoe_moe_stack_forward([gl.L for gl in layers], T, x, r, out["h"], out["y"], out["idx"],
                              out["w"], ws, stream=stream)
    return out


def run_layers(layers, x, r, ws):
    """One layer call per layer (x <- y, r <- h); the per-layer outputs and the
    inputs each layer saw, on the host."""
    cfg = layers[0].cfg
    T = x.shape[0]
    outs = []
    for gl in layers:
        o = dict(h=torch.empty(T, cfg.H, device="cuda"), y=torch.empty(T, cfg.H, device="cuda"),
                 moe=torch.empty(T, cfg.H, device="cuda"),
                 idx=torch.empty(T, cfg.k, dtype=torch.int32, device="cuda"),
                 w=torch.empty(T, cfg.k, device="cuda"))
        fm.fmoe_moe_layer_forward(gl.L, T, x, r, o["h"], o["y"], o["idx"], o["w"], o["moe"], ws)
        o["x_in"], o["r_in"] = x, r
        outs.append(o)
        x, r = o["y"], o["h"]
    torch.cuda.synchronize()
    return outs


def assert_same(stack, outs):
    for l, o in enumerate(outs):
        for name in ("h", "y", "idx", "w"):
            assert torch.equal(stack[name][l], o[name]), (l, name)


def oracle_check(gl, o, tokens=(0,)):
    got = {k: o[k].cpu().numpy() for k in ("h", "y", "moe", "idx", "w")}
    return check_layer(gl, o["x_in"].cpu().numpy(), o["r_in"].cpu().numpy(), got, list(tokens))


@pytest.fixture(scope="module")
def layers4():
    note("generate 4 layer4 layers on device")
    return [GpuLayer(synth.CONFIGS["layer4"], layer=20 + l, random_gamma=(l % 2 == 1))
            for l in range(4)]


def test_stack_one_launch_matches_layer_calls(layers4):
    cfg = layers4[0].cfg
    ws = torch.zeros(fm.fmoe_workspace_size(layers4[0].L, 1), dtype=torch.uint8, device="cuda")
    x = dev(synth.activations(cfg, 3, pool=21))
    r = dev(synth.normal(cfg.seed, 0, 61, (3, cfg.H)))
    for t in range(3):
        note(f"layer4 stack of 4, token {t}")
        st = run_stack(layers4, x[t:t + 1], r[t:t + 1], ws)
        outs = run_layers(layers4, x[t:t + 1], r[t:t + 1], ws)
        assert _wait_timeouts(ws) == 0
        assert_same(st, outs)
        excluded = sum(oracle_check(gl, o) for gl, o in zip(layers4, outs))
        assert excluded <= 1


def test_stack_residual_aliases_x(layers4):
    cfg = layers4[0].cfg
    note("layer4 stack, residual = x")
    ws = torch.zeros(fm.fmoe_workspace_size(layers4[0].L, 1), dtype=torch.uint8, device="cuda")
    x = dev(synth.activations(cfg, 1, pool=22))
    st = run_stack(layers4[:2], x, x, ws)
    outs = run_layers(layers4[:2], x, x, ws)
    assert_same(st, outs)


def test_stack_over_64_layers(layers4):
    # 70 layers (the four layers in turn) take two launches, 64 + 6; the
    # second starts from the first one's last y and h.
    cfg = layers4[0].cfg
    note("layer4 stack of 70")
    ws = torch.zeros(fm.fmoe_workspace_size(layers4[0].L, 1), dtype=torch.uint8, device="cuda")
    seq = [layers4[l % 4] for l in range(70)]
    x = dev(synth.activations(cfg, 1, pool=23))
    st = run_stack(seq, x, x, ws)
    outs = run_layers(seq, x, x, ws)
    assert _wait_timeouts(ws) == 0
    assert_same(st, outs)
    assert np.isfinite(st["y"].cpu().numpy()).all()


@pytest.mark.parametrize("n", [1, 65])
def test_stack_one_and_65_layers(layers4, n):
    # A chain of one layer (one launch that is also the last layer), and 65
    # layers (a launch of 64 and a launch of 1).
    cfg = layers4[0].cfg
    note(f"layer4 stack of {n}")
    ws = torch.zeros(fm.fmoe_workspace_size(layers4[0].L, 1), dtype=torch.uint8, device="cuda")
    seq = [layers4[(3 * l) % 4] for l in range(n)]
    x = dev(synth.activations(cfg, 1, pool=28))
    r = dev(synth.normal(cfg.seed, 0, 63, (1, cfg.H)))
    st = run_stack(seq, x, r, ws)
    outs = run_layers(seq, x, r, ws)
    assert _wait_timeouts(ws) == 0
    assert_same(st, outs)


def test_stack_calls_interleaved_on_one_workspace(layers4):
    # Stack calls and single-layer calls in turn on one workspace, 40 times:
    # every call a new epoch of the shared records; each reproduces its first
    # result bit for bit.
    cfg = layers4[0].cfg
    note("layer4 stack / layer calls interleaved")
    ws = torch.zeros(fm.fmoe_workspace_size(layers4[0].L, 1), dtype=torch.uint8, device="cuda")
    x = dev(synth.activations(cfg, 2, pool=24))
    ref_st = [run_stack(layers4, x[j:j + 1], x[j:j + 1], ws) for j in range(2)]
    ref_l = [run_layers(layers4[:1], x[j:j + 1], x[j:j + 1], ws)[0] for j in range(2)]
    for i in range(40):
        j = i % 2
        st = run_stack(layers4, x[j:j + 1], x[j:j + 1], ws)
        o = run_layers(layers4[:1], x[j:j + 1], x[j:j + 1], ws)[0]
        assert torch.equal(st["y"], ref_st[j]["y"]) and torch.equal(st["h"], ref_st[j]["h"]), i
        assert torch.equal(o["y"], ref_l[j]["y"]), i
    assert _wait_timeouts(ws) == 0


@pytest.mark.parametrize("name", ["mid4", "layer2", "mid2"])
def test_stack_other_shapes(name):
    # 16 rows a down part (mid4 and the full-size 2-bit layer2: six records a
    # part); mid2 (top-6 of 96, 2-bit) runs one layer call after another.
    cfg = {"mid4": MID, "mid2": MID2, "layer2": synth.CONFIGS["layer2"]}[name]
    note(f"stack of 3, {cfg.name}")
    layers = [GpuLayer(cfg, layer=l, random_gamma=True) for l in range(3)]
    ws = torch.zeros(fm.fmoe_workspace_size(layers[0].L, 1), dtype=torch.uint8, device="cuda")
    x = dev(synth.activations(cfg, 2, pool=3))
    r = dev(synth.normal(cfg.seed, 0, 62, (2, cfg.H)))
    for t in range(2):
        st = run_stack(layers, x[t:t + 1], r[t:t + 1], ws)
        outs = run_layers(layers, x[t:t + 1], r[t:t + 1], ws)
        assert _wait_timeouts(ws) == 0
        assert_same(st, outs)
        for gl, o in zip(layers, outs):
            oracle_check(gl, o)


@pytest.mark.parametrize("T", [1, 4])
def test_stack_layer_by_layer_shapes(T):
    # Shapes outside the chained kernel (the tiny layer at one token) and
    # batches run one layer call after another through the same entry point.
    cfg = synth.CONFIGS["tiny"]
    note(f"tiny stack of 3, T={T}")
    layers = [GpuLayer(cfg, layer=l) for l in range(3)]
    ws = torch.zeros(fm.fmoe_workspace_size(layers[0].L, T), dtype=torch.uint8, device="cuda")
    x = dev(synth.activations(cfg, T, pool=5))
    st = run_stack(layers, x, x, ws)
    outs = run_layers(layers, x, x, ws)
    assert_same(st, outs)
    for gl, o in zip(layers, outs):
        oracle_check(gl, o, range(T))


def test_stack_batch32_layer_by_layer(layers4):
    # A batch through the stack entry point: the batched path, one layer call
    # after another, equal to the caller's own chain of layer calls.
    cfg = layers4[0].cfg
    note("layer4 stack of 2, T=32")
    T = 32
    ws = torch.zeros(fm.fmoe_workspace_size(layers4[0].L, T), dtype=torch.uint8, device="cuda")
    x = dev(synth.activations(cfg, T, pool=27))
    st = run_stack(layers4[:2], x, x, ws)
    outs = run_layers(layers4[:2], x, x, ws)
    assert _wait_timeouts(ws) == 0
    assert_same(st, outs)
    excluded = oracle_check(layers4[1], outs[1], (0, 31))
    assert excluded <= 1


def test_stack_wait_gives_up_loud(layers4):
    # Forced from the host: down part 0 never publishes (fmoe_paths.test_stall_part)
    # and waits are bounded at 2 ms.  Every layer's outputs are NaN, the timeout
    # word is set, and the next call on the workspace is valid again.
    cfg = layers4[0].cfg
    note("layer4 stack, forced wait timeout")
    ws = torch.zeros(fm.fmoe_workspace_size(layers4[0].L, 1), dtype=torch.uint8, device="cuda")
    x = dev(synth.activations(cfg, 1, pool=25))
    with fm.paths(wait_limit_us=2000, test_stall_part=1):
        st = run_stack(layers4[:3], x, x, ws)
        torch.cuda.synchronize()
    assert _wait_timeouts(ws) == 1
    assert torch.isnan(st["y"]).all()
    off = fm.fmoe_wait_timeout_offset()
    ws[off:off + 4].zero_()
    st = run_stack(layers4[:3], x, x, ws)
    outs = run_layers(layers4[:3], x, x, ws)
    assert _wait_timeouts(ws) == 0
    assert_same(st, outs)


def test_stack_graph_replays_match_eager(layers4):
    # A stack call captured in a HIP graph: every replay, with eager work and
    # synchronisation between replays, reproduces the eager result.
    cfg = layers4[0].cfg
    note("layer4 stack, graph replay")
    ws = torch.zeros(fm.fmoe_workspace_size(layers4[0].L, 1), dtype=torch.uint8, device="cuda")
    x = dev(synth.activations(cfg, 1, pool=26))
    ref = run_stack(layers4, x, x, ws)
    torch.cuda.synchronize()
    out = {k: torch.empty_like(v) for k, v in ref.items()}
    arr = [gl.L for gl in layers4]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fm.fmoe_moe_stack_forward(arr, 1, x, x, out["h"], out["y"], out["idx"], out["w"], ws,
                                  stream=torch.cuda.current_stream())
    for rep in range(4):
        for v in out.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(out[k], ref[k]), (rep, k)
        _ = (x * 2).sum().item()
    assert _wait_timeouts(ws) == 0
