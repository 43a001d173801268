"""Test-side helpers written independently of the oracle and of the library:
a numpy packer/unpacker for the LSB-first code layout, a numpy dequantiser and
random quantised matrices.  Used to pin the oracle (brute force, round trips).
"""
import numpy as np

import synth


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes [N, K] in 0..2^bits-1 -> packed bytes [N, K*bits/8], element j of a
    byte at bits [bits*j, bits*j + bits)."""
    N, K = codes.shape
    per = 8 // bits
    c = codes.astype(np.uint16).reshape(N, K // per, per)
    out = np.zeros((N, K // per), np.uint16)
    for j in range(per):
        out |= c[:, :, j] << np.uint16(bits * j)
    return out.astype(np.uint8)


def unpack_codes(q: np.ndarray, bits: int, K: int) -> np.ndarray:
    N = q.shape[0]
    per = 8 // bits
    q = q.reshape(N, K // per).astype(np.uint16)
    out = np.empty((N, K // per, per), np.uint8)
    for j in range(per):
        out[:, :, j] = (q >> np.uint16(bits * j)) & np.uint16((1 << bits) - 1)
    return out.reshape(N, K)


def widen(sb: np.ndarray, sbytes: int) -> np.ndarray:
    if sbytes == 2:
        return synth.bf16_bits_to_f32(sb).astype(np.float64)
    return np.asarray(sb, np.float32).astype(np.float64)


def dequant(codes, s, b, sbytes, G) -> np.ndarray:
    sw = np.repeat(widen(s, sbytes), G, axis=1)
    bw = np.repeat(widen(b, sbytes), G, axis=1)
    return codes.astype(np.float64) * sw + bw


def store_sb(v: np.ndarray, sbytes: int) -> np.ndarray:
    v = np.asarray(v, np.float32)
    return synth.f32_to_bf16_bits(v) if sbytes == 2 else v


def rand_qmat(rng, N, K, bits, G, sbytes, lo=0.001, hi=0.01, bias_range=0.05):
    codes = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    s = store_sb(rng.uniform(lo, hi, size=(N, K // G)), sbytes)
    b = store_sb(rng.uniform(-bias_range, bias_range, size=(N, K // G)), sbytes)
    return codes, pack_codes(codes, bits), s, b


def rel_l2(a, ref) -> float:
    a = np.asarray(a, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    n = np.linalg.norm(ref)
    d = np.linalg.norm(a - ref)
    return d if n == 0 else d / n


FORMATS = [(b, g, s) for b in (4, 2) for g in (32, 64) for s in (4, 2)]


def build_slab(spec_like, mats):
    """Assemble an expert slab from (q, s, b) for gate, up, down following the
    canonical layout (256-byte aligned sections), independent of the oracle."""
    off, size = spec_like.layout()
    out = np.zeros(size, np.uint8)
    for m, (q, s, b) in enumerate(mats):
        for j, arr in enumerate((q, s, b)):
            raw = np.ascontiguousarray(arr).view(np.uint8).ravel()
            out[off[3 * m + j]:off[3 * m + j] + raw.size] = raw
    return out
