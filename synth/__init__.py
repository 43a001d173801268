"""Seeded synthetic inputs for the quantized MoE layer (host side).

This module is the one piece that both the GPU path's tests/benchmark and the
CPU oracle draw their inputs from.  It holds none of the layer's arithmetic:
it only produces packed codes, per-group scales and biases, expert slabs and
normal-distributed vectors, deterministically from a seed.

Packed codes and scales come from SplitMix64 used as a counter hash (the
generator of Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014; finaliser constants as published there and in
Vigna's reference splitmix64.c).  Word i of a stream with key K is
mix(K + (i+1) * 0x9E3779B97F4A7C15), i.e. the i-th output of a SplitMix64
generator seeded with K.  The same definition is implemented on the device in
synth/synth_dev.hip, so a 200+ GB expert set can be generated in HBM and any
slab of it regenerated bit-identically on the host.

Scale rule (both sides, fp32 with every operation rounded separately):
    u = (word >> 40) * 2**-24           (exact)
    s = lo + (hi - lo) * u              (hi - lo rounded once, product once, sum once)
    bf16 storage rounds s to nearest-even; the bias is bias_mult * (stored s),
    computed in fp32 and rounded the same way.
Normals (router weights, shared-gate vector, activations, test gammas) are
generated on the host only, with numpy's PCG64 from a seed sequence.
"""
from __future__ import annotations

import dataclasses
import os

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK = (1 << 64) - 1

# tensor tags inside one expert slab: matrix m in (gate, up, down)
TAG_Q = (1, 3, 5)
TAG_S = (2, 4, 6)


def _mix_int(z: int) -> int:
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def word(key: int, i: int) -> int:
    """Word i of the stream keyed by `key` (Python ints, exact)."""
    return _mix_int((key + (i + 1) * 0x9E3779B97F4A7C15) & _MASK)


def derive_key(seed: int, layer: int, slab: int, tag: int) -> int:
    k = word(seed & _MASK, layer)
    k = word(k, slab)
    return word(k, tag)


def stream(key: int, n: int, start: int = 0) -> np.ndarray:
    """Words start .. start+n-1 of the stream keyed by `key` (uint64 array)."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(key) + i * GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the 16 stored bits.
    Finite inputs only (NaN is not produced by this generator)."""
    b = np.ascontiguousarray(f, np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return (r & np.uint64(0xFFFF)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class QSpec:
    """Shape and value recipe of one expert (gate/up [I x H], down [H x I])."""
    H: int
    I: int
    bits: int
    group: int
    sbytes: int          # 4 = fp32 scale/bias, 2 = bf16
    lo: float            # scale ~ U(lo, hi)
    hi: float
    bias_mult: float     # bias = bias_mult * scale

    def mats(self):
        return ((self.I, self.H), (self.I, self.H), (self.H, self.I))

    def layout(self):
        """Section offsets (9) and slab size; 256-byte aligned sections in the
        order gate.q gate.s gate.b up.q up.s up.b down.q down.s down.b."""
        off, pos = [], 0
        r256 = lambda v: (v + 255) // 256 * 256
        for n, k in self.mats():
            qb = n * k * self.bits // 8
            sb = n * (k // self.group) * self.sbytes
            off.append(pos); pos = r256(pos + qb)
            off.append(pos); pos = r256(pos + sb)
            off.append(pos); pos = r256(pos + sb)
        return off, pos


def scales_and_bias(spec: QSpec, key: int, n: int):
    """The first n (scale, bias) pairs of a scale stream, as stored."""
    u = (stream(key, n) >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)
    lo, hi = np.float32(spec.lo), np.float32(spec.hi)
    rng = np.float32(hi - lo)
    s32 = (lo + (rng * u).astype(np.float32)).astype(np.float32)
    bm = np.float32(spec.bias_mult)
    if spec.sbytes == 2:
        s = f32_to_bf16_bits(s32)
        b = f32_to_bf16_bits((bf16_bits_to_f32(s) * bm).astype(np.float32))
        return s, b
    return s32, (s32 * bm).astype(np.float32)


def matrix(spec: QSpec, seed: int, layer: int, slab: int, m: int):
    """(q bytes [n, k*bits/8], scale [n, k/G], bias [n, k/G]) of matrix m."""
    n, k = spec.mats()[m]
    rb = k * spec.bits // 8
    q = stream(derive_key(seed, layer, slab, TAG_Q[m]), n * rb // 8).view(np.uint8).reshape(n, rb)
    s, b = scales_and_bias(spec, derive_key(seed, layer, slab, TAG_S[m]), n * (k // spec.group))
    return q, s.reshape(n, -1), b.reshape(n, -1)


def slab(spec: QSpec, seed: int, layer: int, slab_id: int) -> np.ndarray:
    """All bytes of one expert slab (padding is zero)."""
    off, size = spec.layout()
    out = np.zeros(size, np.uint8)
    for m in range(3):
        q, s, b = matrix(spec, seed, layer, slab_id, m)
        out[off[3 * m]:off[3 * m] + q.size] = q.reshape(-1)
        sv, bv = s.reshape(-1).view(np.uint8), b.reshape(-1).view(np.uint8)
        out[off[3 * m + 1]:off[3 * m + 1] + sv.size] = sv
        out[off[3 * m + 2]:off[3 * m + 2] + bv.size] = bv
    return out


def layer_slabs(spec: QSpec, seed: int, layer: int, n_slabs: int) -> np.ndarray:
    """Slabs 0 .. n_slabs-1 of one layer, back to back (host; small sizes)."""
    return np.concatenate([slab(spec, seed, layer, e) for e in range(n_slabs)])


def normal(seed: int, layer: int, tag: int, shape, std: float = 1.0) -> np.ndarray:
    """fp32 N(0, std^2) array, host only."""
    g = np.random.default_rng(np.random.SeedSequence([seed, layer, tag]))
    return (g.standard_normal(size=shape) * std).astype(np.float32)


def uniform(seed: int, layer: int, tag: int, shape, lo: float, hi: float) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence([seed, layer, tag]))
    return g.uniform(lo, hi, size=shape).astype(np.float32)


# host tags for the normal-distributed tensors
TAG_ROUTER, TAG_WSG, TAG_X, TAG_GAMMA = 101, 102, 103, 104


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    H: int
    I: int
    E: int
    k: int
    spec: QSpec
    seed: int
    layers: int = 1
    T: int = 1
    eps: float = 1e-6


def _spec4(H, I, group, sbytes):
    return QSpec(H, I, 4, group, sbytes, 0.001, 0.01, -8.0)


CONFIGS = {
    # tiny layer: H256, 16 experts, I128, top-2 + shared, 4-bit g32 fp32 scales
    "tiny": Config("tiny", 256, 128, 16, 2, _spec4(256, 128, 32, 4), 1000),
    # one expert, 4-bit g64 bf16 (gate/up 1024x4096, down 4096x1024)
    "expert": Config("expert", 4096, 1024, 0, 0, _spec4(4096, 1024, 64, 2), 1001),
    # full layer at hidden 4096 / 512 experts / I 1024, top-4 + shared, 4-bit
    "layer4": Config("layer4", 4096, 1024, 512, 4, _spec4(4096, 1024, 64, 2), 1002),
    # same layer with 2-bit codes, scale U(0.002, 0.02), bias -1.5 * scale
    "layer2": Config("layer2", 4096, 1024, 512, 4,
                     QSpec(4096, 1024, 2, 64, 2, 0.002, 0.02, -1.5), 1003),
    # 60 stacked 4-bit layers, 32 tokens
    "stack": Config("stack", 4096, 1024, 512, 4, _spec4(4096, 1024, 64, 2), 1004,
                    layers=60, T=32),
}


def router(cfg: Config, layer: int) -> np.ndarray:
    return normal(cfg.seed, layer, TAG_ROUTER, (cfg.E, cfg.H), 0.02)


def shared_gate(cfg: Config, layer: int) -> np.ndarray:
    return normal(cfg.seed, layer, TAG_WSG, (cfg.H,), 0.02)


def activations(cfg: Config, n: int, pool: int = 0) -> np.ndarray:
    return normal(cfg.seed, 10_000 + pool, TAG_X, (n, cfg.H), 1.0)


def gamma(cfg: Config, layer: int, random: bool = False) -> np.ndarray:
    if random:
        return uniform(cfg.seed, layer, TAG_GAMMA, (cfg.H,), 0.5, 1.5)
    return np.ones(cfg.H, np.float32)


# ---------------------------------------------------------------- device side
_dev = None
HERE = os.path.dirname(os.path.abspath(__file__))
DEV_LIB = os.path.join(HERE, "libfmoe_synth.so")


def device_lib():
    """ctypes handle of the device generator (synth/synth_dev.hip)."""
    global _dev
    if _dev is None:
        import ctypes as C
        if not os.path.exists(DEV_LIB):
            raise RuntimeError("synth device generator not built: run __graft_entry__.build()")
        L = C.CDLL(DEV_LIB)
        L.synth_fill_slabs.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int64,
                                       C.c_uint64, C.c_int32, C.c_int32, C.c_int32,
                                       C.c_int32, C.c_int32, C.c_int32, C.c_float,
                                       C.c_float, C.c_float, C.c_void_p]
        L.synth_fill_slabs.restype = C.c_int
        _dev = L
    return _dev


def fill_device_slabs(ptr: int, spec: QSpec, seed: int, layer: int, first: int,
                      count: int, stride: int, stream: int = 0) -> None:
    """Write slabs first .. first+count-1 of `layer` at device address ptr
    (slab i at ptr + (i - first) * stride).  Enqueued on `stream`."""
    rc = device_lib().synth_fill_slabs(ptr, stride, first, count, seed, layer, spec.H,
                                       spec.I, spec.bits, spec.group, spec.sbytes,
                                       spec.lo, spec.hi, spec.bias_mult, stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_slabs failed with HIP error {rc}")
