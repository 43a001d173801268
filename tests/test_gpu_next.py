"""GPU parity of the decode steps beside the MoE layer, through the C ABI,
against the CPU oracle: the Gated DeltaNet state update (fmoe_deltanet_step)
and decode attention with rotary embedding (fmoe_attention_decode).

DeltaNet bar: the step runs in fp32 with dot products over dk <= 256 terms; against the
fp64 oracle on the same fp32 inputs each head's output and new state must be
within relative L2 2e-5 (fp32 rounding of a dk-term sum is about
sqrt(dk) 2^-24 relative; the bar leaves a wide margin and still fails any
wrong term).
"""
import numpy as np
import pytest
import torch

import bit_dequant_expert_amd as fm
import oracle
from qtest_util import rel_l2

pytestmark = pytest.mark.gpu

DN_TOL = 2e-5


def note(msg):
    print(f"[case] {msg}", flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dn_inputs(rng, B, NH, dk, dv):
    """Decode-step inputs as a linear-attention layer produces them: unit-norm
    keys and queries, decay in (0.5, 1), write strength in (0, 1), a state of
    accumulated outer products."""
    def unit(x):
        return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)
    q = unit(rng.standard_normal((B, NH, dk)))
    k = unit(rng.standard_normal((B, NH, dk)))
    v = rng.standard_normal((B, NH, dv)).astype(np.float32)
    a = rng.uniform(0.5, 1.0, (B, NH)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (B, NH)).astype(np.float32)
    S = (rng.standard_normal((B, NH, dk, dv)) * 0.3).astype(np.float32)
    return q, k, v, a, beta, S


def run_dn(q, k, v, a, beta, S):
    st = dev(S)
    out = torch.empty(S.shape[0], S.shape[1], S.shape[3], device="cuda")
    fm.fmoe_deltanet_step(dev(q), dev(k), dev(v), dev(a), dev(beta), st, out)
    torch.cuda.synchronize()
    return st.cpu().numpy(), out.cpu().numpy()


def check_dn(got_s, got_o, ref_s, ref_o):
    B, NH = got_o.shape[:2]
    worst = 0.0
    for b in range(B):
        for h in range(NH):
            eo = rel_l2(got_o[b, h], ref_o[b, h])
            es = rel_l2(got_s[b, h], ref_s[b, h])
            worst = max(worst, eo, es)
            assert eo <= DN_TOL and es <= DN_TOL, (b, h, eo, es)
    return worst


@pytest.mark.parametrize("B,NH,dk,dv", [(1, 64, 128, 128), (2, 3, 32, 32), (3, 2, 64, 96),
                                        (1, 5, 256, 64), (2, 4, 128, 256), (1, 1, 256, 32)])
def test_deltanet_matches_oracle(B, NH, dk, dv):
    note(f"deltanet B={B} NH={NH} dk={dk} dv={dv}")
    rng = np.random.default_rng(B * 1000 + NH * 10 + dk + dv)
    q, k, v, a, beta, S = dn_inputs(rng, B, NH, dk, dv)
    gs, go = run_dn(q, k, v, a, beta, S)
    rs, ro = oracle.deltanet_step(q, k, v, a, beta, S)
    check_dn(gs, go, rs, ro)


def test_deltanet_chained_steps_teacher_forced():
    # Eight decode steps on one resident state; each step against the oracle
    # fed the GPU's own state before it.
    B, NH, dk, dv = 2, 64, 128, 128
    note("deltanet 8 chained steps")
    rng = np.random.default_rng(77)
    _, _, _, _, _, S0 = dn_inputs(rng, B, NH, dk, dv)
    st = dev(S0)
    out = torch.empty(B, NH, dv, device="cuda")
    for t in range(8):
        q, k, v, a, beta, _ = dn_inputs(rng, B, NH, dk, 32)
        v = rng.standard_normal((B, NH, dv)).astype(np.float32)
        before = st.cpu().numpy()
        fm.fmoe_deltanet_step(dev(q), dev(k), dev(v), dev(a), dev(beta), st, out)
        torch.cuda.synchronize()
        rs, ro = oracle.deltanet_step(q, k, v, a, beta, before)
        check_dn(st.cpu().numpy(), out.cpu().numpy(), rs, ro)


def test_deltanet_special_cases():
    # beta = 0 leaves a decayed state; a = 1, beta = 1 with a unit key makes
    # the state return v for that key (the delta rule's store).
    B, NH, dk, dv = 1, 8, 64, 64
    rng = np.random.default_rng(78)
    q, k, v, a, beta, S = dn_inputs(rng, B, NH, dk, dv)
    gs, _ = run_dn(q, k, v, a, np.zeros_like(beta), S)
    np.testing.assert_allclose(gs, a[..., None, None] * S, rtol=1e-6, atol=1e-7)
    gs, _ = run_dn(q, k, v, np.ones_like(a), np.ones_like(beta), S)
    for h in range(NH):
        kk = k[0, h].astype(np.float64)
        read = gs[0, h].astype(np.float64).T @ kk
        np.testing.assert_allclose(read, v[0, h], rtol=1e-4, atol=1e-5)


def test_deltanet_empty_is_noop():
    st = torch.zeros(0, 64, 128, 128, device="cuda")
    out = torch.zeros(0, 64, 128, device="cuda")
    z = torch.zeros(1, device="cuda")
    fm.fmoe_deltanet_step(z, z, z, z, z, st, out)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- attention
# Bar: the rotated query enters the matrix cores as two bf16 halves (16
# significant bits, relative rounding below 2^-16); scores, softmax and P V are
# fp32.  A score error of e moves the probabilities by about e relative, so each
# head's output must be within relative L2 1e-4 of the fp64 oracle (scores here
# are O(1): a wrong term, index or rotation is off by far more).
ATT_TOL = 1e-4


def bf16_bits(x):
    import synth
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def att_inputs(rng, B, NQ, NKV, D, cap, qscale=1.0):
    q = (rng.standard_normal((B, NQ, D)) * qscale).astype(np.float32)
    kc = bf16_bits(rng.standard_normal((B, NKV, cap, D)))
    vc = bf16_bits(rng.standard_normal((B, NKV, cap, D)))
    return q, kc, vc


def run_att(q, kc, vc, lens, base=10000.0):
    B, NQ, D = q.shape
    _, NKV, cap, _ = kc.shape
    out = torch.empty(B, NQ, D, device="cuda")
    ws = torch.empty(max(1, fm.fmoe_attention_workspace_size(B, NKV, D, cap)), dtype=torch.uint8,
                     device="cuda")
    kd = torch.from_numpy(kc.view(np.int16)).cuda()
    vd = torch.from_numpy(vc.view(np.int16)).cuda()
    ld = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    fm.fmoe_attention_decode(dev(q), kd, vd, ld, out, ws, rope_base=base)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_att(got, ref):
    worst = 0.0
    for b in range(got.shape[0]):
        for h in range(got.shape[1]):
            e = rel_l2(got[b, h], ref[b, h])
            worst = max(worst, e)
            assert e <= ATT_TOL, (b, h, e)
    return worst


@pytest.mark.parametrize("B,NQ,NKV,D,cap,lens", [
    (2, 32, 2, 256, 600, [600, 1]),          # 16 query heads per KV head, two chunks + a tail
    (3, 8, 8, 128, 300, [1, 257, 300]),      # one query head per KV head, ragged lengths
    (1, 16, 4, 64, 1000, [513]),             # head_dim 64, length just past two chunks
    (2, 12, 3, 128, 256, [256, 255]),        # 4 heads per KV head, one full chunk
])
def test_attention_matches_oracle(B, NQ, NKV, D, cap, lens):
    note(f"attention B={B} NQ={NQ} NKV={NKV} D={D} cap={cap} lens={lens}")
    rng = np.random.default_rng(B * 100 + NQ + D + cap)
    q, kc, vc = att_inputs(rng, B, NQ, NKV, D, cap)
    got = run_att(q, kc, vc, lens)
    ref = oracle.attention_decode(q, kc, vc, lens)
    check_att(got, ref)


def test_attention_long_context_and_peaked_scores():
    # Positions up to 8191 (rotation angles far past 2 pi) and a query scaled so
    # that each head's softmax is concentrated on a few positions.
    B, NQ, NKV, D, cap = 2, 32, 2, 256, 8192
    note("attention long context")
    rng = np.random.default_rng(91)
    q, kc, vc = att_inputs(rng, B, NQ, NKV, D, cap, qscale=4.0)
    lens = [8192, 5000]
    got = run_att(q, kc, vc, lens)
    ref = oracle.attention_decode(q, kc, vc, lens)
    check_att(got, ref)


def test_attention_rope_base_and_empty_batch():
    rng = np.random.default_rng(92)
    q, kc, vc = att_inputs(rng, 1, 4, 1, 64, 40)
    got = run_att(q, kc, vc, [37], base=1e6)
    ref = oracle.attention_decode(q, kc, vc, [37], base=1e6)
    check_att(got, ref)
    out = torch.empty(0, 4, 64, device="cuda")
    z = torch.zeros(1, device="cuda")
    zc = torch.zeros(0, 1, 40, 64, dtype=torch.int16, device="cuda")
    fm.fmoe_attention_decode(torch.empty(0, 4, 64, device="cuda"), zc, zc,
                             torch.zeros(1, dtype=torch.int32, device="cuda"), out, z)
    torch.cuda.synchronize()


# ------------------------------------------------------- expert streaming
def _pinned(nbytes):
    return torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)


def _fetch_setup(cfg, layer=0):
    """Host tier (pinned) holding the layer's slabs, an HBM tier filled with a
    marker byte, tags zero."""
    import synth
    sp = cfg.spec
    _, stride = sp.layout()
    host = _pinned(stride * (cfg.E + 1))
    dev_tmp = torch.empty(stride * (cfg.E + 1), dtype=torch.uint8, device="cuda")
    synth.fill_device_slabs(dev_tmp.data_ptr(), sp, cfg.seed, layer, 0, cfg.E + 1, stride)
    host.copy_(dev_tmp.cpu())
    del dev_tmp
    hbm = torch.full((stride * (cfg.E + 1),), 0xAB, dtype=torch.uint8, device="cuda")
    tags = torch.zeros(cfg.E + 1, dtype=torch.int32, device="cuda")
    ncp = torch.zeros(1, dtype=torch.int32, device="cuda")
    return host, hbm, tags, ncp, stride


def test_fetch_experts_routing_driven_cache():
    # Route 3 tokens on the device, fetch their experts and the shared one into
    # HBM, run the layer on the HBM tier and check it against the oracle; a
    # second fetch with the same tag copies nothing (cache hit), a new tag
    # copies again.
    import synth
    from test_gpu_parity import GpuLayer, check_layer
    cfg = synth.CONFIGS["tiny"]
    note("fetch tiny")
    host, hbm, tags, ncp, stride = _fetch_setup(cfg)
    gl = GpuLayer(cfg)                  # router, gates, norm (and its own slabs, unused here)
    T = 3
    x = synth.activations(cfg, T, pool=50)
    idx = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, cfg.k, device="cuda")
    ws = torch.zeros(fm.fmoe_route_workspace_size(T, cfg.E), dtype=torch.uint8, device="cuda")
    fm.fmoe_route_topk(gl.Wr_d, dev(x), cfg.k, idx, w, None, ws)
    fm.fmoe_fetch_experts(idx, T * cfg.k, cfg.E, host, stride, stride, hbm, tags, cfg.E + 1, 7,
                          ncp)
    torch.cuda.synchronize()
    sel = sorted(set(idx.cpu().numpy().ravel().tolist()) | {cfg.E})
    assert int(ncp.item()) == len(sel)
    hb = host.numpy().reshape(cfg.E + 1, stride).copy()
    db = hbm.cpu().numpy().reshape(cfg.E + 1, stride)
    tg = tags.cpu().numpy()
    for e in range(cfg.E + 1):
        if e in sel:
            assert np.array_equal(db[e], hb[e]) and tg[e] == 7, e
        else:
            assert (db[e] == 0xAB).all() and tg[e] == 0, e
    # the layer on the HBM tier
    L = fm.fmoe_layer_desc(cfg.H, cfg.I, cfg.E, cfg.k, gl.fmt, gl.Wr_d, hbm, stride, gl.wsg_d,
                           gl.g_d, cfg.eps)
    out = dict(h=torch.empty(T, cfg.H, device="cuda"), y=torch.empty(T, cfg.H, device="cuda"),
               moe=torch.empty(T, cfg.H, device="cuda"),
               idx=torch.empty(T, cfg.k, dtype=torch.int32, device="cuda"),
               w=torch.empty(T, cfg.k, device="cuda"))
    lws = torch.zeros(fm.fmoe_workspace_size(L, T), dtype=torch.uint8, device="cuda")
    xd = dev(x)
    fm.fmoe_moe_layer_forward(L, T, xd, xd, out["h"], out["y"], out["idx"], out["w"], out["moe"],
                              lws)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    assert np.array_equal(got["idx"], idx.cpu().numpy())
    check_layer(gl, x, x, got, list(range(T)))
    # same tag: a hit, even though the host tier changed meanwhile
    host[:] = 0x11
    fm.fmoe_fetch_experts(idx, T * cfg.k, cfg.E, host, stride, stride, hbm, tags, cfg.E + 1, 7,
                          ncp)
    torch.cuda.synchronize()
    assert int(ncp.item()) == len(sel)
    assert np.array_equal(hbm.cpu().numpy().reshape(cfg.E + 1, stride)[sel], hb[sel])
    # new tag: copied again
    fm.fmoe_fetch_experts(idx, T * cfg.k, -1, host, stride, stride, hbm, tags, cfg.E + 1, 8, ncp)
    torch.cuda.synchronize()
    routed = sorted(set(idx.cpu().numpy().ravel().tolist()))
    assert int(ncp.item()) == len(sel) + len(routed)
    db = hbm.cpu().numpy().reshape(cfg.E + 1, stride)
    for e in routed:
        assert (db[e] == 0x11).all() and tags[e].item() == 8
    assert np.array_equal(db[cfg.E], hb[cfg.E]) and tags[cfg.E].item() == 7


def test_fetch_experts_full_size_slabs():
    # Full-size 4-bit slabs (6.75 MiB, 108 pieces each), a list with repeats and
    # an out-of-range entry.
    import synth
    base = synth.CONFIGS["layer4"]
    cfg = synth.Config("fetch64", base.H, base.I, 64, 4, base.spec, base.seed)
    note("fetch full-size slabs")
    host, hbm, tags, ncp, stride = _fetch_setup(cfg, layer=2)
    lst = torch.tensor([5, 17, 5, 63, -3, 64, 17, 40], dtype=torch.int32, device="cuda")
    fm.fmoe_fetch_experts(lst, 8, 64, host, stride, stride, hbm, tags, cfg.E + 1, 3, ncp)
    torch.cuda.synchronize()
    want = [5, 17, 63, 64, 40]
    assert int(ncp.item()) == len(want)
    hb = host.numpy().reshape(cfg.E + 1, stride)
    db = hbm.cpu().numpy().reshape(cfg.E + 1, stride)
    for e in range(cfg.E + 1):
        if e in want:
            assert np.array_equal(db[e], hb[e]), e
        else:
            assert (db[e] == 0xAB).all(), e


def test_fetch_experts_rejects_unpinned_host_memory():
    host = np.zeros(1 << 16, np.uint8)             # pageable
    hbm = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    tags = torch.zeros(4, dtype=torch.int32, device="cuda")
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(fm.FmoeError) as ei:
        fm.fmoe_fetch_experts(idx, 1, -1, host.ctypes.data, 1 << 14, 1 << 14, hbm, tags, 4, 1)
    assert ei.value.status == fm.FMOE_ERR_UNSUPPORTED
