"""Pins of the oracle's Gated DeltaNet step and decode attention (CPU only).

Each check fixes the oracle to something other than itself: closed forms of
special cases, the defining invariant of the delta rule, the rotation
identities of the rotary embedding, and a library attention routine (torch's
scaled_dot_product_attention in fp64 on the CPU) on the same rotated inputs.
A plausible slip -- a transposed state, the decay applied after the read, a
sign or frequency error in the rotation, a wrong query-to-KV-head mapping, a
missing 1/sqrt(D) -- fails at least one of them.
"""
import numpy as np
import pytest

import oracle
import synth


def _rng(seed):
    return np.random.default_rng(seed)


def _dn_inputs(rng, B, NH, dk, dv, unit_k=False):
    q = rng.standard_normal((B, NH, dk)).astype(np.float32)
    k = rng.standard_normal((B, NH, dk)).astype(np.float32)
    if unit_k:
        k = (k / np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, NH, dv)).astype(np.float32)
    a = rng.uniform(0.5, 1.0, (B, NH)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (B, NH)).astype(np.float32)
    S = rng.standard_normal((B, NH, dk, dv)).astype(np.float32)
    return q, k, v, a, beta, S


# ----------------------------------------------------------- Gated DeltaNet
def test_deltanet_from_zero_state_is_outer_product():
    # S = 0: the read is 0, the write is beta k v^T, the output beta (k.q) v.
    q, k, v, a, beta, S = _dn_inputs(_rng(1), 2, 3, 8, 12)
    S[:] = 0
    S2, o = oracle.deltanet_step(q, k, v, a, beta, S)
    for b in range(2):
        for h in range(3):
            kk, qq, vv = (t[b, h].astype(np.float64) for t in (k, q, v))
            bt = float(beta[b, h])
            np.testing.assert_allclose(S2[b, h], bt * np.outer(kk, vv), rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(o[b, h], bt * float(kk @ qq) * vv, rtol=1e-12, atol=1e-13)


def test_deltanet_no_write_is_decayed_read():
    # beta = 0: the state is only decayed and the output is the decayed
    # state's read for q (a plain matrix product).
    q, k, v, a, beta, S = _dn_inputs(_rng(2), 1, 4, 16, 8)
    beta[:] = 0
    S2, o = oracle.deltanet_step(q, k, v, a, beta, S)
    for h in range(4):
        Sd = float(a[0, h]) * S[0, h].astype(np.float64)
        np.testing.assert_allclose(S2[0, h], Sd, rtol=1e-15)
        np.testing.assert_allclose(o[0, h], Sd.T @ q[0, h].astype(np.float64), rtol=1e-11,
                                   atol=1e-12)


@pytest.mark.parametrize("dk,dv", [(8, 12), (12, 8), (16, 16)])
def test_deltanet_full_write_stores_value_at_key(dk, dv):
    # The delta rule's defining property: with beta = 1 and a unit key, the
    # updated state returns exactly v for that key, whatever the decay and
    # the old state (non-square shapes catch a transposed state).
    q, k, v, a, beta, S = _dn_inputs(_rng(3 + dk), 2, 2, dk, dv, unit_k=True)
    beta[:] = 1
    S2, _ = oracle.deltanet_step(q, k, v, a, beta, S)
    for b in range(2):
        for h in range(2):
            kk = k[b, h].astype(np.float64)
            # the key as stored is unit length to fp32 rounding: correct the
            # read by the key's own norm (S2^T k = v |k|^2 + a S^T k (1 - |k|^2))
            n2 = float(kk @ kk)
            exp = v[b, h].astype(np.float64) * n2 + float(a[b, h]) * (S[b, h].astype(np.float64).T @ kk) * (1 - n2)
            np.testing.assert_allclose(S2[b, h].T @ kk, exp, rtol=1e-10, atol=1e-10)


def test_deltanet_partial_write_moves_read_toward_value():
    # beta in (0, 1), unit key: the new read is (1 - beta) times the decayed
    # old read plus beta times v.
    q, k, v, a, beta, S = _dn_inputs(_rng(9), 1, 3, 10, 6, unit_k=True)
    S2, _ = oracle.deltanet_step(q, k, v, a, beta, S)
    for h in range(3):
        kk = k[0, h].astype(np.float64)
        n2 = float(kk @ kk)
        old = float(a[0, h]) * (S[0, h].astype(np.float64).T @ kk)
        bt = float(beta[0, h])
        exp = old + bt * n2 * (v[0, h] - old)
        np.testing.assert_allclose(S2[0, h].T @ kk, exp, rtol=1e-9, atol=1e-9)


def test_deltanet_heads_and_sequences_independent():
    q, k, v, a, beta, S = _dn_inputs(_rng(5), 3, 4, 8, 8)
    S2, o = oracle.deltanet_step(q, k, v, a, beta, S)
    for b, h in ((0, 0), (2, 3), (1, 2)):
        s1, o1 = oracle.deltanet_step(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                      v[b:b + 1, h:h + 1], a[b:b + 1, h:h + 1],
                                      beta[b:b + 1, h:h + 1], S[b:b + 1, h:h + 1])
        np.testing.assert_array_equal(s1[0, 0], S2[b, h])
        np.testing.assert_array_equal(o1[0, 0], o[b, h])


# -------------------------------------------------------------------- RoPE
def test_rope_position_zero_only_deinterleaves():
    x = _rng(6).standard_normal(16).astype(np.float32)
    y = oracle.rope_deinterleave(x, 0)
    np.testing.assert_array_equal(y, np.concatenate([x[0::2], x[1::2]]).astype(np.float64))


@pytest.mark.parametrize("pos", [1, 3, 1000, 70000])
def test_rope_explicit_angles(pos):
    # D = 4, base 10000: pair 0 turns by pos, pair 1 by pos / 100.
    y = oracle.rope_deinterleave(np.array([1, 0, 0, 0], np.float32), pos)
    np.testing.assert_allclose(y, [np.cos(pos), 0, np.sin(pos), 0], atol=1e-12)
    y = oracle.rope_deinterleave(np.array([0, 0, 1, 0], np.float32), pos)
    np.testing.assert_allclose(y, [0, np.cos(pos / 100), 0, np.sin(pos / 100)], atol=1e-12)
    y = oracle.rope_deinterleave(np.array([0, 0, 0, 1], np.float32), pos)
    np.testing.assert_allclose(y, [0, -np.sin(pos / 100), 0, np.cos(pos / 100)], atol=1e-12)


def test_rope_relative_position_and_norm():
    # Rotations preserve each pair's norm, and a dot product of a rotated
    # query and key depends only on the difference of their positions.
    rng = _rng(7)
    D = 64
    q = rng.standard_normal(D).astype(np.float32)
    k = rng.standard_normal(D).astype(np.float32)
    for p, s in ((5, 2), (100, 37), (4000, 3999)):
        qp, ks = oracle.rope_deinterleave(q, p), oracle.rope_deinterleave(k, s)
        qd, k0 = oracle.rope_deinterleave(q, p - s), oracle.rope_deinterleave(k, 0)
        assert abs(qp @ ks - qd @ k0) <= 1e-9 * np.linalg.norm(q) * np.linalg.norm(k)
        np.testing.assert_allclose(np.hypot(qp[:D // 2], qp[D // 2:]),
                                   np.hypot(q[0::2].astype(np.float64), q[1::2].astype(np.float64)),
                                   rtol=1e-12)


# --------------------------------------------------------------- attention
def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def _att_inputs(rng, B, NQ, NKV, D, cap, lens):
    q = rng.standard_normal((B, NQ, D)).astype(np.float32)
    kc = _bf16(rng.standard_normal((B, NKV, cap, D)))
    vc = _bf16(rng.standard_normal((B, NKV, cap, D)))
    return q, kc, vc, np.asarray(lens, np.int32)


def test_attention_single_entry_returns_value():
    rng = _rng(10)
    q, kc, vc, lens = _att_inputs(rng, 2, 4, 2, 16, 5, [1, 1])
    out = oracle.attention_decode(q, kc, vc, lens)
    V = synth.bf16_bits_to_f32(vc).astype(np.float64)
    for b in range(2):
        for h in range(4):
            np.testing.assert_allclose(out[b, h], V[b, h // 2, 0], rtol=1e-15)


def test_attention_zero_query_averages_values():
    rng = _rng(11)
    q, kc, vc, lens = _att_inputs(rng, 1, 2, 1, 8, 9, [7])
    q[:] = 0
    out = oracle.attention_decode(q, kc, vc, lens)
    V = synth.bf16_bits_to_f32(vc).astype(np.float64)
    np.testing.assert_allclose(out[0, 0], V[0, 0, :7].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_attention_query_head_groups():
    # Query head h reads KV head h // (NQ / NKV): values constant per KV head.
    rng = _rng(12)
    q, kc, vc, lens = _att_inputs(rng, 1, 8, 4, 8, 3, [3])
    for g in range(4):
        vc[0, g] = _bf16(np.full((3, 8), g + 1.0))
    out = oracle.attention_decode(q, kc, vc, lens)
    for h in range(8):
        np.testing.assert_allclose(out[0, h], np.full(8, h // 2 + 1.0), rtol=1e-14)


@pytest.mark.parametrize("lens", [[1, 5, 33], [64, 2, 17]])
def test_attention_matches_library_attention(lens):
    # The library routine on the same rotated query and cache (fp64, CPU).
    torch = pytest.importorskip("torch")
    rng = _rng(13 + lens[0])
    B, NQ, NKV, D, cap = 3, 8, 2, 32, 64
    q, kc, vc, lens = _att_inputs(rng, B, NQ, NKV, D, cap, lens)
    out = oracle.attention_decode(q, kc, vc, lens)
    K = synth.bf16_bits_to_f32(kc).astype(np.float64)
    V = synth.bf16_bits_to_f32(vc).astype(np.float64)
    F = torch.nn.functional
    for b in range(B):
        L = int(lens[b])
        qr = np.stack([oracle.rope_deinterleave(q[b, h], L - 1) for h in range(NQ)])
        Kh = np.repeat(K[b, :, :L], NQ // NKV, axis=0)      # [NQ, L, D]
        Vh = np.repeat(V[b, :, :L], NQ // NKV, axis=0)
        ref = F.scaled_dot_product_attention(torch.from_numpy(qr[:, None, :]),
                                              torch.from_numpy(Kh), torch.from_numpy(Vh))
        np.testing.assert_allclose(out[b], ref[:, 0, :].numpy(), rtol=1e-10, atol=1e-12)
