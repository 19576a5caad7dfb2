"""GPU parity of full backpropagation through the base and of the a posteriori bias certificate
(sinkhorn_attn_tail_remainder) against the fp64 oracle (vjp_full, tail_remainder), both pinned in
test_oracle_tail.py.  Full backpropagation runs the general adjoint at depth T + R, beyond the
register-held modifier depths, so these cases also cover the run-time-depth passes."""

import numpy as np
import pytest
import torch

import oracle
from entropic_ot_attention_amd.workloads import TINY_L512, Workload, make_inputs
from tests.gpu_common import as64, compare, say

pytestmark = pytest.mark.gpu

F32, BF16 = "f32", "bf16"


def _inputs(bh, L, W, T, R, eps, dtype, seed, qk_scale=1.0):
    w = Workload("case", 1, bh, L, 64, W, T, R, eps, dtype, seed)
    x = make_inputs(w)
    if qk_scale != 1.0:
        x = dict(x, Q=(x["Q"].float() * qk_scale).to(x["Q"].dtype),
                 K=(x["K"].float() * qk_scale).to(x["K"].dtype))
    return w, x


@pytest.mark.parametrize("case", [
    ("L300_W40_T5_R2_f32", 2, 300, 40, 5, 2, 1.0, F32),
    ("L500_W200_T6_R1_bf16", 2, 500, 200, 6, 1, 1.0, BF16),
    ("L200_W1000_T4_R2_dense_f32", 1, 200, 1000, 4, 2, 0.8, F32),
    ("L260_W64_T3_R0_f32", 2, 260, 64, 3, 0, 1.0, F32),
], ids=lambda c: c[0])
def test_full_backprop_gradients(case):
    """grad_full = the adjoint at depth T + R with no stopped base (T' = 0)."""
    name, bh, L, W, T, R, eps, dt = case
    w, x = _inputs(bh, L, W, T, R, eps, dt, seed=400 + L)
    say(f"[gpu] full backprop {name}")
    from entropic_ot_attention_amd import binding as B
    dev = torch.device("cuda:0")
    Qd, Kd, Vd, dOd = (x[k].to(dev) for k in ("Q", "K", "V", "dO"))
    O, duals = B.forward(Qd, Kd, Vd, W, 0, T + R, eps)
    dQ, dK, dV = B.vjp(Qd, Kd, Vd, duals, dOd, W, 0, T + R, eps)
    torch.cuda.synchronize()
    got = {k: v.float().cpu().double().numpy() for k, v in dict(O=O, dQ=dQ, dK=dK, dV=dV).items()}
    ref = {k: [] for k in ("O", "dQ", "dK", "dV")}
    for b in range(bh):
        Q, K, V, dO = (as64(x[k][b]) for k in ("Q", "K", "V", "dO"))
        p = oracle.BandProblem(W=W, T=T, R=R, eps=eps)
        dQ, dK, dV = oracle.vjp_full(Q, K, V, dO, p)
        O, _ = oracle.forward(Q, K, V, p)
        for k, v in (("O", O), ("dQ", dQ), ("dK", dK), ("dV", dV)):
            ref[k].append(v)
    compare(got, ref, w.torch_dtype, name)


def _certificate(x, W, T, R, eps):
    from entropic_ot_attention_amd import binding as B
    dev = torch.device("cuda:0")
    Q, K, V, dO = (x[k].to(dev) for k in ("Q", "K", "V", "dO"))
    return B.tail_remainder(Q, K, V, dO, W, T, R, eps)


def _oracle_certificate(x, W, T, R, eps):
    tot = {"rem_dQ2": 0.0, "full_dQ2": 0.0, "rem_dK2": 0.0, "full_dK2": 0.0}
    for b in range(x["Q"].shape[0]):
        r = oracle.tail_remainder(*(as64(x[k][b]) for k in ("Q", "K", "V", "dO")),
                                  oracle.BandProblem(W=W, T=T, R=R, eps=eps))
        for k in tot:
            tot[k] += r[k]
    tot["eta"] = float(np.sqrt((tot["rem_dQ2"] + tot["rem_dK2"]) / (tot["full_dQ2"] + tot["full_dK2"])))
    return tot


# The certified remainder eta_R = ||grad_full - grad_R|| / ||grad_full|| is formed from two fp32
# gradients.  Full backpropagation runs 2 (T + R) reduction sweeps, each adding about one unit of
# fp32 rounding (2^-24) relative to the gradient's norm, so the difference of the two gradients
# carries an absolute error of about 2 (T + R) 2^-24 in eta units whatever eta is (measured:
# up to 7e-7 at T + R = 18, where eta_3 ~ 1e-7 is below it).  Comparisons allow 1e-3 relative
# plus that floor.
ETA_REL = 1e-3


def _eta_close(g, o, T, R):
    return abs(g - o) <= ETA_REL * o + 2 * (T + R) * 2.0 ** -24


@pytest.mark.parametrize("R", [0, 1, 2, 4])
def test_certificate_matches_oracle(R):
    """Full-gradient norms to fp32 rounding; the certified remainder eta_R to 1e-3 relative
    (plus the fp32 floor of the two gradients it subtracts)."""
    W, T, eps = 40, 5, 1.0
    w, x = _inputs(2, 300, W, T, R, eps, F32, seed=410)
    say(f"[gpu] certificate L300 W40 T5 R={R}")
    g = _certificate(x, W, T, R, eps)
    o = _oracle_certificate(x, W, T, R, eps)
    say(f"eta gpu {g['eta']:.9e} oracle {o['eta']:.9e} diff {abs(g['eta'] - o['eta']):.2e}")
    for k in ("full_dQ2", "full_dK2"):
        assert abs(g[k] - o[k]) <= 1e-5 * o[k], (k, g[k], o[k])
    assert _eta_close(g["eta"], o["eta"], T, R), (g["eta"], o["eta"])


@pytest.mark.parametrize("qk_scale,expect_R", [(0.5, 2), (0.56, 3)])
def test_certificate_resolves_tau_from_either_side(qk_scale, expect_R):
    """Dense low-contrast problems whose eta_2 lies within a factor 2 of tau = 1e-5: below it
    (8.0e-6, scores scaled by 0.5, R = 2 certified) and above it (1.67e-5, scaled by 0.56, so
    R = 3 is the smallest certified depth).  The GPU selects the oracle's depth and matches
    every eta_R on the way."""
    from entropic_ot_attention_amd import binding as B
    W, T, eps = 128, 15, 1.0
    w, x = _inputs(1, 64, W, T, 2, eps, F32, seed=420, qk_scale=qk_scale)
    say(f"[gpu] certificate near tau, qk scale {qk_scale}")
    dev = torch.device("cuda:0")
    Q, K, V, dO = (x[k].to(dev) for k in ("Q", "K", "V", "dO"))
    R, etas = B.select_tail_depth(Q, K, V, dO, W, T, eps, tau=1e-5, R_max=4)
    Ro, etas_o = oracle.select_tail_depth(*(as64(x[k][0]) for k in ("Q", "K", "V", "dO")),
                                          W, T, eps, tau=1e-5, R_max=4)
    say(f"gpu R={R} etas={etas}  oracle R={Ro} etas={etas_o}")
    assert Ro == expect_R and 0.5e-5 <= etas_o[2] <= 2e-5
    assert R == Ro and sorted(etas) == sorted(etas_o)
    say(f"eta_2 gpu - oracle = {etas[2] - etas_o[2]:.2e} (tau - eta_2 = {1e-5 - etas_o[2]:.2e})")
    for k in etas:
        assert _eta_close(etas[k], etas_o[k], T, k), (k, etas[k], etas_o[k])


def test_certificate_selects_r2_on_a_contracting_problem():
    """Dense support, low-contrast scores: the remainder falls by about three decades per tail
    step and R = 2 is the smallest depth certified at tau = 1e-5 on the GPU, as in the oracle
    (and as the pages report for their problems)."""
    from entropic_ot_attention_amd import binding as B
    W, T, eps = 128, 15, 1.0
    w, x = _inputs(1, 64, W, T, 2, eps, F32, seed=420, qk_scale=0.3)
    say("[gpu] certificate depth selection, dense low-contrast L64")
    dev = torch.device("cuda:0")
    Q, K, V, dO = (x[k].to(dev) for k in ("Q", "K", "V", "dO"))
    R, etas = B.select_tail_depth(Q, K, V, dO, W, T, eps, tau=1e-5, R_max=4)
    Ro, etas_o = oracle.select_tail_depth(*(as64(x[k][0]) for k in ("Q", "K", "V", "dO")),
                                          W, T, eps, tau=1e-5, R_max=4)
    say(f"gpu R={R} etas={etas}  oracle R={Ro} etas={etas_o}")
    assert R == Ro == 2 and sorted(etas) == sorted(etas_o) == [0, 1, 2]
    for k in etas:
        assert _eta_close(etas[k], etas_o[k], T, k), (k, etas[k], etas_o[k])


def test_tiny_workload_certificate():
    """The tiny workload (L = 512, W = 64, T = 15, fp32) at R = 2: the banded support contracts
    slowly, so the certified remainder stays near 1e-2."""
    w = TINY_L512
    x = make_inputs(w)
    say("[gpu] certificate tiny L512")
    g = _certificate(x, w.W, w.T, 2, w.eps)
    o = _oracle_certificate(x, w.W, w.T, 2, w.eps)
    say(f"tiny eta gpu {g['eta']:.6e} oracle {o['eta']:.6e}")
    assert _eta_close(g["eta"], o["eta"], w.T, 2), (g["eta"], o["eta"])
