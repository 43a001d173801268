"""Pins of the CPU oracle to facts outside itself: brute force, closed forms,
special cases, round trips, invariants and the pages' printed sizes.  CPU only.

Each check is chosen so a plausible oracle mistake fails one of them: a wrong
bit order or group index (one-hot, round trip, brute force), a dropped bias or
scale (x = 1, s = 0, zero-weight cases), swapped gate/up/down (the asymmetric
closed-form FFN), a wrong combine sign or term (identical-experts layer),
wrong tie rule or ordering (full sort vs k-pass, identical rows), wrong
renormalisation (ln-weights closed form, E = k softmax).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import synth
from qtest_util import (FORMATS, build_slab, dequant, pack_codes, rand_qmat, rel_l2, store_sb,
                        unpack_codes, widen)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("bits", [4, 2])
def test_code_roundtrip(bits):
    rng = np.random.default_rng(1)
    K = 128
    raw = rng.integers(0, 256, size=(3, K * bits // 8), dtype=np.uint8)
    codes = unpack_codes(raw, bits, K)
    assert np.array_equal(pack_codes(codes, bits), raw)
    for n in range(3):
        got = [oracle.code(raw[n], bits, k) for k in range(K)]
        assert got == codes[n].tolist()


@pytest.mark.parametrize("bits,G,sb", FORMATS)
def test_gemv_brute_force(bits, G, sb):
    rng = np.random.default_rng(2)
    N, K = 24, 256
    codes, q, s, b = rand_qmat(rng, N, K, bits, G, sb)
    x = rng.standard_normal(K)
    W = dequant(codes, s, b, sb, G)
    ref = W @ x                       # library dgemv on an independently dequantised matrix
    got = oracle.gemv(q, s, b, bits, G, sb, N, K, x)
    assert rel_l2(got, ref) < 1e-13
    assert np.allclose(oracle.dequant(q, s, b, bits, G, sb, N, K), W, rtol=0, atol=0)


@pytest.mark.parametrize("bits,G,sb", FORMATS)
def test_fma_identity(bits, G, sb):
    rng = np.random.default_rng(3)
    N, K = 16, 512
    _, q, s, b = rand_qmat(rng, N, K, bits, G, sb)
    x = rng.standard_normal(K)
    ref = oracle.gemv(q, s, b, bits, G, sb, N, K, x)
    assert rel_l2(oracle.gemv_fma_form(q, s, b, bits, G, sb, N, K, x), ref) < 1e-13
    assert rel_l2(oracle.gemv_groupsum(q, s, b, bits, G, sb, N, K, x), ref) < 1e-13
    naive = oracle.gemv_naive_f32(q, s, b, bits, G, sb, N, K, x.astype(np.float32))
    assert rel_l2(naive, ref) < 1e-5


@pytest.mark.parametrize("bits,G,sb", FORMATS)
def test_gemv_one_hot_exact(bits, G, sb):
    rng = np.random.default_rng(4)
    N, K = 8, 128
    codes, q, s, b = rand_qmat(rng, N, K, bits, G, sb)
    for j in (0, 1, 7, 31, 32, 63, 64, 127):
        x = np.zeros(K)
        x[j] = 1.0
        got = oracle.gemv(q, s, b, bits, G, sb, N, K, x)
        g = j // G
        exp = codes[:, j].astype(np.float64) * widen(s, sb)[:, g] + widen(b, sb)[:, g]
        assert np.array_equal(got, exp), j


def test_gemv_zero_weights_exact():
    # 4-bit codes 8 with bias -8*scale dequantise to exactly zero.
    rng = np.random.default_rng(5)
    N, K, G = 16, 256, 64
    codes = np.full((N, K), 8, np.uint8)
    s32 = rng.uniform(0.001, 0.01, (N, K // G)).astype(np.float32)
    for sb in (4, 2):
        s = store_sb(s32, sb)
        b = store_sb(-8.0 * (synth.bf16_bits_to_f32(s) if sb == 2 else s), sb)
        y = oracle.gemv(pack_codes(codes, 4), s, b, 4, G, sb, N, K, rng.standard_normal(K))
        assert np.array_equal(y, np.zeros(N))


@pytest.mark.parametrize("bits,G,sb", FORMATS)
def test_gemv_ones_and_zero_scale(bits, G, sb):
    rng = np.random.default_rng(6)
    N, K = 8, 256
    codes, q, s, b = rand_qmat(rng, N, K, bits, G, sb)
    sw, bw = widen(s, sb), widen(b, sb)
    # x = 1: y_n = sum_g (s_g * (integer sum of codes) + G * b_g)
    y1 = oracle.gemv(q, s, b, bits, G, sb, N, K, np.ones(K))
    isum = codes.reshape(N, K // G, G).sum(axis=2).astype(np.float64)
    assert np.allclose(y1, (sw * isum + G * bw).sum(axis=1), rtol=1e-14, atol=0)
    # s = 0: y_n = sum_g b_g * (sum of x over the group)
    x = rng.standard_normal(K)
    z = np.zeros_like(s)
    y0 = oracle.gemv(q, z, b, bits, G, sb, N, K, x)
    xs = x.reshape(K // G, G).sum(axis=1)
    assert np.allclose(y0, bw @ xs, rtol=1e-13, atol=1e-15)


def _sorted_ref(logits, k):
    E = logits.shape[0]
    order = np.lexsort((np.arange(E), -logits))   # logit desc, index asc
    return order[:k]


def test_topk_full_sort_vs_kpass_and_lexsort():
    rng = np.random.default_rng(7)
    E, H, k, T = 64, 32, 6, 40
    Wr = rng.standard_normal((E, H)).astype(np.float32)
    Wr[10] = Wr[3]                # planted ties
    Wr[40] = Wr[3]
    Wr[11] = Wr[12]
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[0] = np.abs(x[0])
    idx, w, lg, gap, st = oracle.route(Wr, x, k)
    assert st == 0
    for t in range(T):
        assert idx[t].tolist() == _sorted_ref(lg[t], k).tolist()
        assert idx[t].tolist() == oracle.topk_kpass(lg[t], k).tolist()
    # logits are the fp64 dot products of the fp32 inputs
    assert np.allclose(lg, x.astype(np.float64) @ Wr.astype(np.float64).T, rtol=1e-12, atol=1e-12)


def test_route_invariants():
    rng = np.random.default_rng(8)
    E, H, k, T = 32, 64, 4, 20
    Wr = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    x = rng.standard_normal((T, H)).astype(np.float32)
    idx, w, lg, gap, st = oracle.route(Wr, x, k)
    assert st == 0
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0) and np.all(w > 0) and np.all(w <= 1)
    sel_l = np.take_along_axis(lg, idx, axis=1)
    assert np.allclose(gap, sel_l[:, -1] - np.sort(lg, axis=1)[:, -k - 1])
    # E == k: everything selected, weights are the full softmax
    idx2, w2, lg2, gap2, st = oracle.route(Wr[:4], x, 4)
    for t in range(T):
        sm = scipy.special.softmax(lg2[t])
        assert np.allclose(w2[t], sm[idx2[t]], rtol=1e-12)
        assert sorted(idx2[t].tolist()) == [0, 1, 2, 3]
        assert math.isinf(gap2[t])
    # identical router rows: lower index wins every tie, weights 1/k
    Wi = np.tile(Wr[:1], (E, 1))
    idx3, w3, _, _, _ = oracle.route(Wi, x, k)
    assert np.all(idx3 == np.arange(k)) and np.allclose(w3, 1.0 / k, rtol=1e-15)


def test_route_weights_closed_form():
    # logits ln 4, ln 3, ln 2, ln 1 for experts 5, 2, 7, 0; others far below:
    # renormalised weights 4/10, 3/10, 2/10, 1/10.
    E, H, k = 12, 8, 4
    c = np.full(E, -30.0)
    c[[5, 2, 7, 0]] = np.log([4.0, 3.0, 2.0, 1.0])
    Wr = np.zeros((E, H), np.float32)
    Wr[:, 0] = c
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    idx, w, lg, gap, st = oracle.route(Wr, x, k)
    assert idx[0].tolist() == [5, 2, 7, 0]
    assert np.allclose(w[0], [0.4, 0.3, 0.2, 0.1], rtol=1e-6)


def test_silu_special_values():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15
    assert abs(oracle.silu(60.0) - 60.0) < 1e-20 * 60 + 1e-24
    assert abs(oracle.silu(-60.0)) < 1e-23


def test_rmsnorm_closed_form():
    H, eps = 16, 1e-6
    g = np.linspace(0.5, 1.5, H).astype(np.float32)
    for c in (3.0, -0.25, 1e-4):
        y = oracle.rmsnorm(np.full(H, c), g, eps)
        assert np.allclose(y, g.astype(np.float64) * c / math.sqrt(c * c + eps), rtol=1e-14)
    h = np.zeros(H)
    h[0], h[1] = 3.0, 4.0
    y = oracle.rmsnorm(h, np.ones(H, np.float32), 0.0)
    assert np.allclose(y[:2], [3 / math.sqrt(25 / H), 4 / math.sqrt(25 / H)], rtol=1e-15)


def _const_mat(n, k, G, sb, bval):
    """Matrix with zero scales and constant bias bval: every weight equals bval."""
    q = np.zeros((n, k * 4 // 8), np.uint8)
    s = store_sb(np.zeros((n, k // G)), sb)
    b = store_sb(np.full((n, k // G), bval), sb)
    return q, s, b


@pytest.mark.parametrize("sb", [4, 2])
def test_ffn_closed_form(sb):
    # gate = c_g * H, up = c_u * H for x = 1; y = c_d * I * silu(gate) * up.
    H, I, G = 128, 64, 32
    cg, cu, cd = 0.0625, -0.5, 0.25      # exact in bf16
    spec = synth.QSpec(H, I, 4, G, sb, 0.001, 0.01, -8.0)
    slab = build_slab(spec, [_const_mat(I, H, G, sb, cg), _const_mat(I, H, G, sb, cu),
                             _const_mat(H, I, G, sb, cd)])
    y = oracle.expert_ffn(slab, H, I, 4, G, sb, np.ones(H))
    gate, up = cg * H, cu * H
    exp = cd * I * (gate / (1 + math.exp(-gate))) * up
    assert np.allclose(y, exp, rtol=1e-14)
    # swapping gate and up would give silu(up) * gate instead
    assert not np.isclose(exp, cd * I * (up / (1 + math.exp(-up))) * gate)


def test_ffn_zero_gate_gives_zero():
    rng = np.random.default_rng(9)
    H, I, G, sb = 128, 64, 32, 4
    spec = synth.QSpec(H, I, 4, G, sb, 0.001, 0.01, -8.0)
    s = rng.uniform(0.001, 0.01, (I, H // G)).astype(np.float32)
    gate = (pack_codes(np.full((I, H), 8, np.uint8), 4), s, -8.0 * s)
    _, uq, us, ub = rand_qmat(rng, I, H, 4, G, sb)
    _, dq, ds, db = rand_qmat(rng, H, I, 4, G, sb)
    slab = build_slab(spec, [gate, (uq, us, ub), (dq, ds, db)])
    y = oracle.expert_ffn(slab, H, I, 4, G, sb, rng.standard_normal(H))
    assert np.array_equal(y, np.zeros(H))


def _tiny_layer(rng, E=8, H=128, I=64, k=2):
    cfg = synth.Config("t", H, I, E, k, synth.QSpec(H, I, 4, 32, 4, 0.001, 0.01, -8.0), 77)
    off, size = cfg.spec.layout()
    slabs = synth.layer_slabs(cfg.spec, cfg.seed, 0, E + 1)
    Wr = (rng.standard_normal((E, H)) * 0.1).astype(np.float32)
    return cfg, size, slabs, Wr


def test_layer_identical_experts_combine():
    # All E+1 slabs identical and a zero shared-gate vector (g = 1/2): because
    # the routing weights sum to 1, moe = 1.5 * FFN(x).
    rng = np.random.default_rng(10)
    cfg, size, slabs, Wr = _tiny_layer(rng)
    one = slabs[:size]
    same = np.tile(one, cfg.E + 1)
    wsg = np.zeros(cfg.H, np.float32)
    gamma = rng.uniform(0.5, 1.5, cfg.H).astype(np.float32)
    x = rng.standard_normal((3, cfg.H)).astype(np.float32)
    r = rng.standard_normal((3, cfg.H)).astype(np.float32)
    out = oracle.layer_forward(Wr, same, size, wsg, gamma, 1e-6, cfg.H, cfg.I, cfg.E, cfg.k,
                               4, 32, 4, x, r)
    assert out["status"] == 0
    for t in range(3):
        f = oracle.expert_ffn(one, cfg.H, cfg.I, 4, 32, 4, x[t].astype(np.float64))
        assert np.allclose(out["moe"][t], 1.5 * f, rtol=1e-12, atol=1e-15)
        assert out["g"][t] == 0.5
        assert np.allclose(out["h"][t], r[t] + out["moe"][t], rtol=1e-15)
        h = out["h"][t]
        assert np.allclose(out["y"][t], gamma * h / np.sqrt(np.mean(h * h) + 1e-6), rtol=1e-13)


def test_layer_zero_experts():
    # Every expert dequantises to zero: moe = 0, h = r, y = RMSNorm(r).
    rng = np.random.default_rng(11)
    H, I, E, k, G = 128, 64, 6, 2, 32
    spec = synth.QSpec(H, I, 4, G, 4, 0.001, 0.01, -8.0)
    mats = []
    for n, kk in spec.mats():
        s = rng.uniform(0.001, 0.01, (n, kk // G)).astype(np.float32)
        mats.append((pack_codes(np.full((n, kk), 8, np.uint8), 4), s, -8.0 * s))
    one = build_slab(spec, mats)
    slabs = np.tile(one, E + 1)
    Wr = rng.standard_normal((E, H)).astype(np.float32)
    wsg = rng.standard_normal(H).astype(np.float32)
    gamma = np.ones(H, np.float32)
    x = rng.standard_normal((2, H)).astype(np.float32)
    out = oracle.layer_forward(Wr, slabs, one.size, wsg, gamma, 1e-6, H, I, E, k, 4, G, 4, x, x)
    assert np.array_equal(out["moe"], np.zeros((2, H)))
    assert np.array_equal(out["h"], x.astype(np.float64))
    for t in range(2):
        xt = x[t].astype(np.float64)
        assert np.allclose(out["y"][t], xt / np.sqrt(np.mean(xt * xt) + 1e-6), rtol=1e-14)


def test_layer_forced_routing():
    rng = np.random.default_rng(12)
    cfg, size, slabs, Wr = _tiny_layer(rng)
    wsg = (rng.standard_normal(cfg.H) * 0.1).astype(np.float32)
    gamma = np.ones(cfg.H, np.float32)
    x = rng.standard_normal((2, cfg.H)).astype(np.float32)
    free = oracle.layer_forward(Wr, slabs, size, wsg, gamma, 1e-6, cfg.H, cfg.I, cfg.E, cfg.k,
                                4, 32, 4, x, x)
    forced = oracle.layer_forward(Wr, slabs, size, wsg, gamma, 1e-6, cfg.H, cfg.I, cfg.E, cfg.k,
                                  4, 32, 4, x, x, forced_idx=free["idx"])
    assert np.array_equal(free["y"], forced["y"]) or rel_l2(free["y"], forced["y"]) < 1e-15
    other = np.array([[0, 1], [2, 3]], np.int32)
    f2 = oracle.layer_forward(Wr, slabs, size, wsg, gamma, 1e-6, cfg.H, cfg.I, cfg.E, cfg.k,
                              4, 32, 4, x, x, forced_idx=other)
    for t in range(2):
        sm = scipy.special.softmax(f2["logits"][t][other[t]])
        assert np.allclose(f2["w"][t], sm, rtol=1e-14)


def test_slab_layout_page_sizes():
    # One unit reading for every size the pages print: their "MB" and "GB" are
    # binary units (MiB, GiB).  The slab is the exact pin (6.75 MiB); the model
    # totals are the pages' rounded figures for 60 x 512 slabs plus the 5.5 GiB
    # of non-expert weights, and agree with this layout within 2%.
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    off, size4 = oracle.slab_layout(4096, 1024, 4, 64, 2)
    assert size4 == 7_077_888 == int(facts["expert_bytes_mb"]["value"] * 2 ** 20)
    assert list(off) == [0, 2097152, 2228224, 2359296, 4456448, 4587520, 4718592, 6815744,
                         6946816]
    L, E = facts["layers"]["value"], facts["experts_per_layer"]["value"]
    non_expert = facts["non_expert_bytes_gb"]["value"]
    _, size2 = oracle.slab_layout(4096, 1024, 2, 64, 2)
    assert size2 == 3_932_160 == int(3.75 * 2 ** 20)
    for size, key in ((size4, "model_bytes_4bit_gb"), (size2, "model_bytes_2bit_gb")):
        total_gib = size * E * L / 2 ** 30 + non_expert
        assert abs(total_gib / facts[key]["value"] - 1) < 0.02, (key, total_gib)
    _, size0 = oracle.slab_layout(256, 128, 4, 32, 4)
    assert size0 == 73_728


def _row_const_mat(n, k, G, sb, rowvals):
    """Zero scales and bias rowvals[r] in every group of row r: every weight of
    row r equals rowvals[r]."""
    q = np.zeros((n, k * 4 // 8), np.uint8)
    s = store_sb(np.zeros((n, k // G)), sb)
    b = store_sb(np.repeat(np.asarray(rowvals, np.float64)[:, None], k // G, axis=1), sb)
    return q, s, b


@pytest.mark.parametrize("sb", [4, 2])
def test_layer_combine_gate_and_pairing_closed_form(sb):
    # Closed form of the whole layer at x = 1 (length H = 128):
    #   every gate weight 1/128 and every up weight 1/256 -> gate = 1, up = 1/2,
    #   so every SwiGLU output is a0 = silu(1)/2 = 1/(2 (1 + e^-1));
    #   down row m of expert e is the constant d_e[m] -> FFN_e(x)[m] = I a0 d_e[m];
    #   router rows are constants making the logits ln 2, -3, ln 4, 0, -4, ln 3
    #   for experts 0..5, so with k = 4 the selection is (2, 5, 0, 3) with
    #   weights 0.4, 0.3, 0.2, 0.1; the shared-gate vector gives wsg . x = ln 3,
    #   so g = sigmoid(ln 3) = 3/4.
    # A flipped sigmoid (g = 1/4), a gate taken on the residual, or weights
    # paired with the wrong experts each change moe by far more than 1e-12.
    H, I, G, E, k = 128, 64, 32, 6, 4
    rng = np.random.default_rng(21)
    spec = synth.QSpec(H, I, 4, G, sb, 0.001, 0.01, -8.0)
    # down rows: small integers / 64, exact in bf16, distinct per expert and row
    d = rng.integers(-64, 65, size=(E + 1, H)).astype(np.float64) / 64.0
    slabs = []
    for e in range(E + 1):
        slabs.append(build_slab(spec, [_row_const_mat(I, H, G, sb, np.full(I, 1 / 128)),
                                       _row_const_mat(I, H, G, sb, np.full(I, 1 / 256)),
                                       _row_const_mat(H, I, G, sb, d[e])]))
    size = slabs[0].size
    target = np.array([math.log(2), -3.0, math.log(4), 0.0, -4.0, math.log(3)])
    Wr = np.repeat((target / H).astype(np.float32)[:, None], H, axis=1)
    wsg = np.full(H, np.float32(math.log(3) / H), np.float32)
    gamma = rng.uniform(0.5, 1.5, H).astype(np.float32)
    x = np.ones((1, H), np.float32)
    r = rng.standard_normal((1, H)).astype(np.float32)
    out = oracle.layer_forward(Wr, np.concatenate(slabs), size, wsg, gamma, 1e-6, H, I, E, k,
                               4, G, sb, x, r)
    assert out["status"] == 0
    assert out["idx"][0].tolist() == [2, 5, 0, 3]
    # the stored router values are fp32: the logits are H times them, exactly
    logit = H * Wr[:, 0].astype(np.float64)
    assert np.array_equal(out["logits"][0], logit)
    sel = logit[[2, 5, 0, 3]]
    w = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
    assert np.allclose(out["w"][0], w, rtol=1e-14)
    assert np.allclose(w, [0.4, 0.3, 0.2, 0.1], atol=1e-6)
    gl = H * np.float64(wsg[0])
    g = 1.0 / (1.0 + math.exp(-gl))
    assert abs(g - 0.75) < 1e-6 and abs(out["g"][0] - g) < 1e-15
    a0 = 1.0 / (2.0 * (1.0 + math.exp(-1.0)))
    moe = I * a0 * (sum(wi * d[e] for wi, e in zip(w, [2, 5, 0, 3])) + g * d[E])
    assert np.allclose(out["moe"][0], moe, rtol=1e-12, atol=1e-14)
    h = r[0].astype(np.float64) + moe
    assert np.allclose(out["h"][0], h, rtol=1e-12, atol=1e-12)
    yref = gamma.astype(np.float64) * h / math.sqrt(np.mean(h * h) + 1e-6)
    assert np.allclose(out["y"][0], yref, rtol=1e-12)
    # the alternatives this rules out differ from the oracle's result by far more
    wrong_g = I * a0 * (sum(wi * d[e] for wi, e in zip(w, [2, 5, 0, 3])) + (1 - g) * d[E])
    reversed_pairs = I * a0 * (sum(wi * d[e] for wi, e in zip(w, [3, 0, 5, 2])) + g * d[E])
    for alt in (wrong_g, reversed_pairs):
        assert rel_l2(alt, out["moe"][0]) > 1e-3


def test_layer_matches_separate_expert_calls():
    # Random distinct experts and random x, r: the layer's moe equals the
    # routing-weighted sum of separate single-expert FFNs of the selected slabs,
    # in the selection's order, plus sigmoid(wsg . x) times the shared FFN.
    rng = np.random.default_rng(22)
    cfg, size, slabs, Wr = _tiny_layer(rng, E=8, k=3)
    wsg = (rng.standard_normal(cfg.H) * 0.1).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, cfg.H).astype(np.float32)
    x = rng.standard_normal((2, cfg.H)).astype(np.float32)
    r = rng.standard_normal((2, cfg.H)).astype(np.float32)
    out = oracle.layer_forward(Wr, slabs, size, wsg, gamma, 1e-6, cfg.H, cfg.I, cfg.E, cfg.k,
                               4, 32, 4, x, r)
    for t in range(2):
        xt = x[t].astype(np.float64)
        f = {e: oracle.expert_ffn(slabs[e * size:(e + 1) * size], cfg.H, cfg.I, 4, 32, 4, xt)
             for e in range(cfg.E + 1)}
        gl = float(np.dot(wsg.astype(np.float64), xt))
        g = 1.0 / (1.0 + math.exp(-gl))
        moe = sum(out["w"][t][i] * f[int(e)] for i, e in enumerate(out["idx"][t])) \
            + g * f[cfg.E]
        assert abs(out["g"][t] - g) < 1e-15
        assert rel_l2(out["moe"][t], moe) < 1e-14
        # every expert's output differs, so any other pairing of weights and
        # experts would not match
        perm = out["idx"][t][::-1]
        alt = sum(out["w"][t][i] * f[int(e)] for i, e in enumerate(perm)) + g * f[cfg.E]
        assert rel_l2(alt, moe) > 1e-3


def test_layer_tiny_config_runs():
    cfg = synth.CONFIGS["tiny"]
    off, size = cfg.spec.layout()
    slabs = synth.layer_slabs(cfg.spec, cfg.seed, 0, cfg.E + 1)
    x = synth.activations(cfg, 4)
    out = oracle.layer_forward(synth.router(cfg, 0), slabs, size, synth.shared_gate(cfg, 0),
                               synth.gamma(cfg, 0), cfg.eps, cfg.H, cfg.I, cfg.E, cfg.k,
                               4, 32, 4, x, x)
    assert out["status"] == 0
    assert np.all(np.isfinite(out["y"])) and np.allclose(out["w"].sum(axis=1), 1.0)
