"""GPU parity of the decode steps beside the MoE layer, through the C ABI,
against the CPU oracle: the Gated DeltaNet state update (fmoe_deltanet_step).

Bar: the step runs in fp32 with dot products over dk <= 256 terms; against the
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
