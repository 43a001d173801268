"""The seeded input generator (host side): published SplitMix64 outputs,
bf16 rounding table, scale/bias rules and slab layout.  CPU only."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_vector():
    v = json.load(open(os.path.join(GOLDEN, "splitmix64_vectors.json")))
    exp = [int(s) for s in v["outputs"]]
    assert synth.stream(v["seed"], 5).tolist() == exp
    assert [synth.word(v["seed"], i) for i in range(5)] == exp


def test_stream_offsets_consistent():
    k = synth.derive_key(5, 1, 2, 3)
    full = synth.stream(k, 40)
    assert np.array_equal(full[17:], synth.stream(k, 23, start=17))


# (fp32 input, expected bf16 bits): nearest, ties to even, signed zero,
# subnormals, overflow to infinity.
BF16_TABLE = [
    (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
    (1.0 + 2.0 ** -8, 0x3F80),            # tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),
    (1.0 + 2.0 ** -9, 0x3F80),
    (2.0 ** -149, 0x0000),                # smallest subnormal rounds to +0
    (2.0 ** -126, 0x0080),
    (3.3895313892515355e38, 0x7F7F),      # largest finite bf16
    (3.4028234663852886e38, 0x7F80),      # largest fp32 rounds up to +inf
    (0.1, 0x3DCD), (0.01, 0x3C24), (0.001, 0x3A83),
]


@pytest.mark.parametrize("f,bits", BF16_TABLE)
def test_bf16_rne_table(f, bits):
    assert int(synth.f32_to_bf16_bits(np.array([f], np.float32))[0]) == bits


def test_scale_rules():
    cfg = synth.CONFIGS["layer4"]
    q, s, b = synth.matrix(cfg.spec, cfg.seed, 0, 3, 0)
    assert q.shape == (1024, 2048) and s.shape == (1024, 64) and s.dtype == np.uint16
    sf = synth.bf16_bits_to_f32(s)
    assert sf.min() >= 0.001 * (1 - 2 ** -8) and sf.max() <= 0.01 * (1 + 2 ** -8)
    assert np.array_equal(synth.bf16_bits_to_f32(b), -8 * sf)   # exact for powers of two
    c2 = synth.CONFIGS["layer2"]
    _, s2, b2 = synth.matrix(c2.spec, c2.seed, 0, 0, 2)
    sf2 = synth.bf16_bits_to_f32(s2)
    assert sf2.min() >= 0.002 * (1 - 2 ** -8) and sf2.max() <= 0.02 * (1 + 2 ** -8)
    exp = synth.f32_to_bf16_bits((sf2 * np.float32(-1.5)).astype(np.float32))
    assert np.array_equal(b2, exp)
    ct = synth.CONFIGS["tiny"]
    _, s0, b0 = synth.matrix(ct.spec, ct.seed, 0, 0, 0)
    assert s0.dtype == np.float32 and np.array_equal(b0, -8 * s0)


def test_codes_uniform():
    q = synth.stream(synth.derive_key(1, 0, 0, 1), 1 << 16).view(np.uint8)
    lo, hi = q & 15, q >> 4
    for nib in (lo, hi):
        counts = np.bincount(nib, minlength=16)
        assert np.all(np.abs(counts / counts.mean() - 1) < 0.05)


@pytest.mark.parametrize("name", ["tiny", "layer4", "layer2"])
def test_slab_layout_matches_oracle(name):
    sp = synth.CONFIGS[name].spec
    off, size = sp.layout()
    ooff, osize = oracle.slab_layout(sp.H, sp.I, sp.bits, sp.group, sp.sbytes)
    assert size == osize and list(off) == list(ooff)


def test_slab_bytes_place_sections():
    cfg = synth.CONFIGS["tiny"]
    sp = cfg.spec
    off, size = sp.layout()
    sl = synth.slab(sp, cfg.seed, 0, 5)
    for m in range(3):
        q, s, b = synth.matrix(sp, cfg.seed, 0, 5, m)
        assert np.array_equal(sl[off[3 * m]:off[3 * m] + q.size], q.ravel())
        sv = s.ravel().view(np.uint8)
        assert np.array_equal(sl[off[3 * m + 1]:off[3 * m + 1] + sv.size], sv)
