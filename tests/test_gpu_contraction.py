"""GPU parity of the projective contraction certificate (sinkhorn_attn_contraction_certificate and
its dustbin_block form) against the fp64 oracle's block_diameters (pinned in
test_oracle_contraction.py).  Which block pairs are active is an integer decision: it must match
exactly.  Delta and kappa on active pairs: max-abs 1e-4 (Delta combines four fp32 scores, each
within about 1e-5 of the fp64 value for these inputs, and bf16 inputs are rounded once, the same
values on both sides).  The long workload is checked on sampled row blocks, whose diameters depend
only on their own rows and columns."""

import numpy as np
import pytest
import torch

import oracle
from entropic_ot_attention_amd.workloads import LONG_L262K, DUSTBIN_L4096, Workload, make_inputs
from tests.gpu_common import as64, say

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _gpu(x, W, eps, block, dustbin=False):
    from entropic_ot_attention_amd import binding as B
    dev = torch.device("cuda:0")
    d, k, dm = B.contraction_certificate(x["Q"].to(dev), x["K"].to(dev), W, eps, block, dustbin)
    torch.cuda.synchronize()
    return d.cpu().double().numpy(), k.cpu().double().numpy(), dm.cpu().double().numpy()


def _check(got_d, got_k, got_max, ref_d, label):
    ref_k = oracle.contraction_coefficients(ref_d)
    assert got_d.shape == ref_d.shape, (label, got_d.shape, ref_d.shape)
    act = ref_d >= 0
    np.testing.assert_array_equal(got_d >= 0, act, err_msg=f"{label}: active pattern")
    np.testing.assert_array_equal(got_d[~act], -1.0)
    np.testing.assert_array_equal(got_k[~act], -1.0)
    err = float(np.abs(got_d[act] - ref_d[act]).max()) if act.any() else 0.0
    errk = float(np.abs(got_k[act] - ref_k[act]).max()) if act.any() else 0.0
    say(f"{label}: {int(act.sum())} active block pairs, Delta max-abs {err:.2e}, kappa {errk:.2e}")
    assert err <= TOL and errk <= TOL, (label, err, errk)
    if got_max is not None:
        want = ref_d.max() if act.any() else -1.0
        assert abs(got_max - want) <= TOL, (label, got_max, want)


CASES = [
    # name, bh, L, W, eps, dtype, block, dustbin
    ("L300_W40_B16_f32", 2, 300, 40, 1.0, "f32", 16, False),
    ("L517_W256_B16_bf16", 2, 517, 256, 0.8, "bf16", 16, False),
    ("L700_W300_B32_f32", 1, 700, 300, 1.0, "f32", 32, False),
    ("L900_W600_B64_f32", 1, 900, 600, 1.3, "f32", 64, False),
    ("L1000_W512_B128_bf16", 1, 1000, 512, 1.0, "bf16", 128, False),
    ("L33_W0_B16_f32", 1, 33, 0, 1.0, "f32", 16, False),
    ("L40_W2000_B16_dense", 1, 40, 2000, 1.0, "f32", 16, False),
    ("dustbin_L200p1_B32", 2, 200, 64, 1.0, "f32", 32, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_diameters_match_the_oracle(case):
    name, bh, L, W, eps, dt, block, dustbin = case
    w = Workload("case", 1, bh, L, 64, W, 1, 2, eps, dt, 500 + L, dustbin=dustbin)
    x = make_inputs(w, with_cotangent=False)
    say(f"[gpu] contraction {name}")
    got_d, got_k, got_max = _gpu(x, W, eps, block, dustbin)
    for b in range(bh):
        ref = oracle.block_diameters(as64(x["Q"][b]), as64(x["K"][b]),
                                     oracle.BandProblem(W=W, T=1, R=2, eps=eps), block, dustbin)
        _check(got_d[b], got_k[b], got_max[b], ref, f"{name} head {b}")


def test_dustbin_L4096_heads0_block16():
    """The dustbin_block workload (4 heads, 4096 + 1 tokens, dense support): every block pair is
    active; head 0 in full."""
    w = DUSTBIN_L4096
    x = make_inputs(w, with_cotangent=False)
    say("[gpu] contraction dustbin_block_L4096p1 B=16")
    got_d, got_k, got_max = _gpu(x, w.W, w.eps, 16, dustbin=True)
    ref = oracle.block_diameters(as64(x["Q"][0]), as64(x["K"][0]),
                                 oracle.BandProblem(W=w.W, T=1, R=2, eps=w.eps), 16, True)
    _check(got_d[0], got_k[0], got_max[0], ref, "dustbin L4096 head 0")


def test_long_L262144_sampled_row_blocks():
    """The long workload (4 heads, L = 262144, W = 256, bf16) at B = 16: sampled row blocks of
    every head against the oracle on the tokens those blocks touch."""
    w = LONG_L262K
    x = make_inputs(w, with_cotangent=False)
    B_ = 16
    say("[gpu] contraction seq1x4_L262144 B=16 sampled row blocks")
    got_d, got_k, got_max = _gpu(x, w.W, w.eps, B_)
    h = w.W // 2
    nb, m = oracle.block_layout(w.L, h, B_)
    r = np.random.default_rng(7)
    for b in range(w.bh):
        rows = sorted(set([0, 1, nb - 1, nb - 2] + list(r.integers(0, nb, 6))))
        for rb in rows:
            lo = max(rb - m, 0)
            hi = min(rb + m + 1, nb)
            t0, t1 = lo * B_, min(hi * B_, w.L)
            ref = oracle.block_diameters(as64(x["Q"][b, t0:t1]), as64(x["K"][b, t0:t1]),
                                         oracle.BandProblem(W=w.W, T=1, R=2, eps=w.eps), B_)
            mloc = (ref.shape[1] - 1) // 2
            want = np.full(2 * m + 1, -1.0)
            for o in range(-m, m + 1):
                if abs(o) <= mloc and 0 <= rb - lo + o < ref.shape[0]:
                    want[o + m] = ref[rb - lo, o + mloc]
            _check(got_d[b, rb], got_k[b, rb], None, want, f"long head {b} row block {rb}")
        act = got_d[b] >= 0
        assert abs(got_max[b] - got_d[b][act].max()) <= 0.0
