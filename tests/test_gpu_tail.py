"""GPU parity of the general tail depth (R = 0, 1, 3, 4): forward duals and output, and the exact
one-reference adjoint with 2 R + 2 passes (R = 0: the base plan with both duals stopped, dV, dQ
and dK with the score cotangent P g), against the fp64 oracle's general-depth orbit form
(itself pinned to dense autograd, finite differences and the step form in test_oracle_tail.py).
Small cases compare every element over narrow, wide and dense supports, both dtypes; the heads8
workload at R = 4 is checked on sampled rows."""

import numpy as np
import pytest
import torch

from entropic_ot_attention_amd.workloads import HEADS8_L32K, Workload, make_inputs
from tests.gpu_common import as64, compare, gpu_run, oracle_head, say

pytestmark = pytest.mark.gpu

F32, BF16 = "f32", "bf16"

CASES = [
    # name, bh, L, W, T, eps, dtype, R
    ("R1_L300_W40", 2, 300, 40, 5, 1.0, F32, 1),
    ("R1_L17_W0", 2, 17, 0, 2, 1.0, F32, 1),
    ("R3_L500_W128", 2, 500, 128, 4, 1.0, F32, 3),
    ("R3_L1000_W256_bf16", 2, 1000, 256, 5, 1.0, BF16, 3),
    ("R4_L700_W64_bf16", 2, 700, 64, 6, 1.0, BF16, 4),
    ("R4_L900_W600_eps07_wide", 1, 900, 600, 3, 0.7, F32, 4),
    ("R4_L260_W1000_dense", 1, 260, 1000, 2, 1.0, F32, 4),
    ("R0_L300_W40", 2, 300, 40, 5, 1.0, F32, 0),
    ("R0_L600_W256_bf16", 2, 600, 256, 4, 1.0, BF16, 0),
    ("R0_L900_W600_wide", 1, 900, 600, 3, 0.8, F32, 0),
    ("R0_L20_W0_T1", 1, 20, 0, 1, 1.0, F32, 0),
    # streaming general passes: shorter than one block, one block plus one token, the diagonal
    # band in bf16, and many segments (level partials across segment boundaries)
    ("R4_L1_W64_bf16", 2, 1, 64, 3, 1.0, BF16, 4),
    ("R3_L129_W32_bf16", 2, 129, 32, 4, 1.0, BF16, 3),
    ("R4_L97_W0_bf16", 1, 97, 0, 2, 1.0, BF16, 4),
    ("R3_L6000_W96_f32_segments", 3, 6000, 96, 5, 0.9, F32, 3),
    ("R1_L4500_W256_bf16_segments", 2, 4500, 256, 6, 1.0, BF16, 1),
]


def _inputs(bh, L, W, T, eps, dtype, seed, R, dustbin=False):
    w = Workload("case", 1, bh, L, 64, W, T, R, eps, dtype, seed, dustbin=dustbin)
    return w, make_inputs(w)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_general_tail_depth_elementwise(case):
    name, bh, L, W, T, eps, dt, R = case
    w, x = _inputs(bh, L, W, T, eps, dt, 300 + [c[0] for c in CASES].index(name), R)
    say(f"[gpu] tail {name} R={R} bh={bh} L={L} W={W} T={T} dtype={dt}")
    got = gpu_run(x["Q"], x["K"], x["V"], x["dO"], W, T, R, eps)
    ref = {k: [] for k in ("O", "duals", "dQ", "dK", "dV")}
    for b in range(bh):
        r = oracle_head(*(as64(x[k][b]) for k in ("Q", "K", "V", "dO")), W, T, R, eps)
        for k in ref:
            ref[k].append(r[k])
    compare(got, ref, w.torch_dtype, name)


@pytest.mark.parametrize("R", [3, 0])
def test_dustbin_block_general_tail_depth(R):
    """The dustbin-block entry points at R = 3 and 0: the same general adjoint on the augmented
    (dense) support, gradients for every row including the dustbin token."""
    w, x = _inputs(2, 200, 64, 4, 1.0, F32, 330, R, dustbin=True)
    say(f"[gpu] dustbin tail R={R} L=200+1")
    got = gpu_run(x["Q"], x["K"], x["V"], x["dO"], 64, 4, R, 1.0, dustbin=True)
    ref = {k: [] for k in ("O", "duals", "dQ", "dK", "dV")}
    for b in range(2):
        r = oracle_head(*(as64(x[k][b]) for k in ("Q", "K", "V", "dO")), 64, 4, R, 1.0,
                        dustbin=True)
        for k in ref:
            ref[k].append(r[k])
    compare(got, ref, torch.float32, f"dustbin R={R}")


def test_direct_four_needs_r2():
    from entropic_ot_attention_amd import binding as B
    w, x = _inputs(1, 64, 16, 1, 1.0, F32, 340, 3)
    say("[gpu] direct-four rejected at R=3")
    dev = torch.device("cuda:0")
    Q, K, V, dO = (x[k].to(dev) for k in ("Q", "K", "V", "dO"))
    O, duals = B.forward(Q, K, V, 16, 1, 3, 1.0)
    with pytest.raises(RuntimeError, match="R == 2"):
        B.vjp(Q, K, V, duals, dO, 16, 1, 3, 1.0, schedule="direct_four")


def test_heads8_L32768_R4_sampled_rows():
    """The heads8 workload (8 heads, L = 32768, W = 256, T = 20, bf16) with a four-step tail,
    checked on sampled rows computed exactly on their dependency windows."""
    import oracle
    base = HEADS8_L32K
    w = Workload("heads8_R4", base.batch, base.heads, base.L, base.d, base.W, base.T, 4,
                 base.eps, base.dtype, base.seed)
    x = make_inputs(w)
    say("[gpu] heads8 L32768 R=4")
    got = gpu_run(x["Q"], x["K"], x["V"], x["dO"], w.W, w.T, 4, w.eps)
    p = oracle.BandProblem(W=w.W, T=w.T, R=4, eps=w.eps)
    rows = {0: [0, w.L - 1], 3: [w.L // 2], 6: [int(np.random.default_rng(5).integers(0, w.L))]}
    ref = {k: [] for k in ("O", "dQ", "dK", "dV")}
    sub = {k: [] for k in ref}
    for b, rr in rows.items():
        r = oracle.sampled_rows(*(as64(x[k][b]) for k in ("Q", "K", "V", "dO")), p, rr)
        for k in ref:
            ref[k].append(r[k])
            sub[k].append(got[k][b][rr])
    compare({k: np.concatenate(v) for k, v in sub.items()},
            {k: np.concatenate(v) for k, v in ref.items()}, w.torch_dtype, "heads8 R=4 sampled")
