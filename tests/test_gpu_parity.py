"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs.

Small cases compare every element and span several tiles, ragged tails, W = 0, a band
wider than the sequence, T = 0, L = 1 and a non-unit epsilon.  The named workloads run at
their full sizes in the launch configuration the benchmark times and are compared on every
element, with both adjoint schedules: the long sequences are cut into contiguous row ranges
that the oracle evaluates exactly on windows of the tokens that can influence them
(oracle.row_range), in parallel threads."""

import numpy as np
import pytest
import torch

from entropic_ot_attention_amd.workloads import (BATCH_L2048, DUSTBIN_L4096, HEADS8_L32K,
                                                 LONG_L262K, TINY_L512, Workload, make_inputs)
import oracle
from tests.gpu_common import (as64, compare, for_schedule, gpu_run, gpu_run_schedules,
                              oracle_every_row, oracle_head, parallel, say)

pytestmark = pytest.mark.gpu

F32, BF16 = "f32", "bf16"

SMALL = [
    # name, bh, L, W, T, eps, dtype
    ("L1_W4", 2, 1, 4, 2, 1.0, F32),
    ("L17_W0", 3, 17, 0, 3, 1.0, F32),
    ("L100_W300_band_wider_than_sequence", 2, 100, 300, 4, 1.0, F32),
    ("L333_W50_eps07", 2, 333, 50, 4, 0.7, F32),
    ("L97_W18_T0", 2, 97, 18, 0, 1.0, F32),
    ("L200_W64_T15", 1, 200, 64, 15, 1.0, F32),
    ("L1000_W256_T5", 2, 1000, 256, 5, 1.0, F32),
    ("L65_W30_eps025", 1, 65, 30, 6, 0.25, F32),
    ("L333_W50_bf16", 2, 333, 50, 4, 1.0, BF16),
    ("L1000_W256_T5_bf16", 2, 1000, 256, 5, 1.0, BF16),
    ("L31_W8_bf16", 3, 31, 8, 2, 1.0, BF16),
    ("L300_W80_bf16", 2, 300, 80, 4, 1.0, BF16),
    ("L400_W500_split_path", 2, 400, 500, 3, 1.0, F32),
    # interior blocks of every register-resident band class (h = 16 H16) on both dtypes
    ("L700_W64_bf16", 2, 700, 64, 6, 1.0, BF16),
    ("L900_W128_bf16", 2, 900, 128, 6, 1.0, BF16),
    ("L1500_W256_eps05_bf16", 1, 1500, 256, 4, 0.5, BF16),
    ("L600_W128_T4", 2, 600, 128, 4, 1.0, F32),
    # the widest register-resident class (25 tiles, h up to 192): interior blocks (h = 192,
    # bf16) and a half-width below the class's halo (h = 160, fp32)
    ("L1400_W384_bf16", 1, 1400, 384, 4, 1.0, BF16),
    ("L900_W320_T3", 1, 900, 320, 3, 1.0, F32),
    # wide engine: register-strip fused step (windows up to 8 x 33 tiles) and window-split passes
    ("L900_W600_bf16_wide", 2, 900, 600, 5, 1.0, BF16),
    ("L700_W2000_dense", 1, 700, 2000, 4, 1.0, F32),
    ("L1300_W700_eps05_wide", 1, 1300, 700, 3, 0.5, F32),
    # fp32 wide step on three-plane operands with a last row tile of one row (L = 16 k + 1)
    ("L1009_W700_wide_single_row_tile", 1, 1009, 700, 3, 1.0, F32),
]


def _inputs(bh, L, W, T, eps, dtype, seed, dustbin=False):
    w = Workload("case", 1, bh, L, 64, W, T, 2, eps, dtype, seed, dustbin=dustbin)
    return w, make_inputs(w)


@pytest.mark.parametrize("schedule", ["one_reference", "direct_four"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases_elementwise(case, schedule):
    name, bh, L, W, T, eps, dt = case
    w, x = _inputs(bh, L, W, T, eps, dt, seed=100 + [c[0] for c in SMALL].index(name))
    say(f"[gpu] small case {name} schedule={schedule} bh={bh} L={L} W={W} T={T} dtype={dt}")
    got = gpu_run(x["Q"], x["K"], x["V"], x["dO"], W, T, 2, eps, schedule)
    ref = {k: [] for k in ("O", "duals", "dQ", "dK", "dV")}
    for b in range(bh):
        r = oracle_head(*(as64(x[k][b]) for k in ("Q", "K", "V", "dO")), W, T, 2, eps, schedule)
        for k in ref:
            ref[k].append(r[k])
    compare(got, ref, w.torch_dtype, f"{name}/{schedule}")


def test_tiny_epsilon_exact_column_fallback():
    """epsilon = 0.01: scores span about +-360 nats, so after the first row update some column
    masses fall below 2^-60 and the fused step finishes those columns by an exact
    log-sum-exp.  fp32 rounding of scores of magnitude |S|max moves exponents by
    about |S|max 2^-24, so outputs, gradients and duals are held to 64 |S|max 2^-24 (relative l2
    for O, dQ, dK, dV; absolute for the duals, whose magnitude is about |S|max)."""
    import oracle
    w, x = _inputs(1, 120, 40, 3, 0.01, F32, seed=7)
    say("[gpu] tiny epsilon column fallback")
    got = gpu_run(x["Q"], x["K"], x["V"], x["dO"], 40, 3, 2, 0.01)
    Q, K, V, dO = (as64(x[k][0]) for k in ("Q", "K", "V", "dO"))
    ref = oracle_head(Q, K, V, dO, 40, 3, 2, 0.01)
    S = oracle.band_scores(Q, K, 20, 0.01)
    smax = float(np.abs(S[np.isfinite(S)]).max())
    tol = 64 * smax * 2.0 ** -24
    for name in ("O", "dQ", "dK", "dV"):
        g, r = got[name][0], ref[name]
        rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        assert np.all(np.isfinite(g)) and rel <= tol, (name, rel, tol)
    err = float(np.abs(got["duals"][0] - ref["duals"]).max())
    say(f"tiny epsilon: |S|max={smax:.1f} tol={tol:.2e} duals maxabs={err:.2e}")
    assert err <= tol, (err, tol)


def test_tiny_epsilon_wide_exact_column_fallback():
    """The same epsilon = 0.01 regime on a dense support (W > 2 L): the wide step's column finish
    takes the exact log-sum-exp for columns whose mass falls below 2^-60; tolerances as in the
    banded case."""
    import oracle
    w, x = _inputs(1, 150, 400, 3, 0.01, F32, seed=8)
    say("[gpu] tiny epsilon wide column fallback")
    got = gpu_run(x["Q"], x["K"], x["V"], x["dO"], 400, 3, 2, 0.01)
    Q, K, V, dO = (as64(x[k][0]) for k in ("Q", "K", "V", "dO"))
    ref = oracle_head(Q, K, V, dO, 400, 3, 2, 0.01)
    S = oracle.band_scores(Q, K, 150, 0.01)
    smax = float(np.abs(S[np.isfinite(S)]).max())
    tol = 64 * smax * 2.0 ** -24
    for name in ("O", "dQ", "dK", "dV"):
        g, r = got[name][0], ref[name]
        rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        assert np.all(np.isfinite(g)) and rel <= tol, (name, rel, tol)
    err = float(np.abs(got["duals"][0] - ref["duals"]).max())
    say(f"tiny epsilon wide: |S|max={smax:.1f} tol={tol:.2e} duals maxabs={err:.2e}")
    assert err <= tol, (err, tol)


@pytest.mark.parametrize("R", [2, 0])
def test_split_half_steps_beyond_register_window(R):
    """A window of 271 tiles (L = 4400, h = 2150) is wider than the wide step holds in registers
    (8 waves x 33 tiles): the forward runs separate row and column half-steps (R = 0: the base
    pair u^(0), v^(0) saved after the last base step)."""
    w, x = _inputs(1, 4400, 4300, 1, 1.0, F32, seed=9)
    say(f"[gpu] split half-steps L=4400 W=4300 T=1 R={R}")
    got = gpu_run(x["Q"], x["K"], x["V"], x["dO"], 4300, 1, R)
    ref = {k: [v] for k, v in oracle_head(*(as64(x[k][0]) for k in ("Q", "K", "V", "dO")),
                                          4300, 1, R, 1.0).items()}
    compare(got, ref, torch.float32, f"split L4400 W4300 R={R}")


@pytest.mark.parametrize("R", [0, 1, 3, 4])
def test_forward_general_tail_depth(R):
    w, x = _inputs(2, 150, 40, 5, 1.0, F32, seed=77 + R)
    say(f"[gpu] forward R={R}")
    got = gpu_run(x["Q"], x["K"], x["V"], x["dO"], 40, 5, R)
    ref = {"O": [], "duals": []}
    for b in range(2):
        r = oracle_head(*(as64(x[k][b]) for k in ("Q", "K", "V", "dO")), 40, 5, R)
        ref["O"].append(r["O"])
        ref["duals"].append(r["duals"])
    compare(got, ref, torch.float32, f"forward R={R}")


@pytest.mark.parametrize("R,W,dtype", [(2, 128, BF16), (3, 128, BF16), (0, 96, BF16),
                                       (4, 600, F32), (1, 64, F32)])
def test_repeat_runs_are_bitwise_identical(R, W, dtype):
    """Every reduction runs in a fixed order (no atomics on the forward or VJP paths), so two runs
    give the same bits: the R = 2 passes, the general-depth streaming passes (R = 0, 1, 3) and the
    wide passes (W = 600)."""
    w, x = _inputs(2, 700, W, 6, 1.0, dtype, seed=5)
    say(f"[gpu] determinism L=700 W={W} R={R} {dtype}")
    a = gpu_run(x["Q"], x["K"], x["V"], x["dO"], W, 6, R)
    b = gpu_run(x["Q"], x["K"], x["V"], x["dO"], W, 6, R)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_certificates_are_bitwise_repeatable():
    """The bias certificate's fp64 norm sums and the contraction certificate's diameters and
    per-problem maxima repeat bit for bit."""
    from entropic_ot_attention_amd import binding as B
    w, x = _inputs(2, 500, 64, 5, 1.0, F32, seed=6)
    dev = torch.device("cuda:0")
    Q, K, V, dO = (x[k].to(dev) for k in ("Q", "K", "V", "dO"))
    say("[gpu] determinism of the certificates")
    r1 = B.tail_remainder(Q, K, V, dO, 64, 5, 2, 1.0)
    r2 = B.tail_remainder(Q, K, V, dO, 64, 5, 2, 1.0)
    assert r1 == r2
    c1 = B.contraction_certificate(Q, K, 64, 1.0, 16)
    c2 = B.contraction_certificate(Q, K, 64, 1.0, 16)
    for u, v in zip(c1, c2):
        assert torch.equal(u, v)


BOTH = ("one_reference", "direct_four")


def _full_oracle(w, x, heads, schedules=BOTH):
    """The oracle on whole heads (one forward, each schedule's VJP), heads in parallel."""
    args = {b: tuple(as64(x[k][b]) for k in ("Q", "K", "V", "dO")) for b in heads}

    def one(b):
        r = {s: oracle_head(*args[b], w.W, w.T, w.R, w.eps, s, dustbin=w.dustbin)
             for s in schedules}
        return r

    per_head = parallel(one, list(heads), w.name)
    ref = {}
    for s in schedules:
        ref[s] = {k: [r[s][k] for r in per_head] for k in ("O", "duals", "dQ", "dK", "dV")}
    return ref


def test_tiny_L512_full():
    """Every element of the tiny workload, both adjoint schedules."""
    w = TINY_L512
    x = make_inputs(w)
    say(f"[gpu] {w.name}")
    got = gpu_run_schedules(x["Q"], x["K"], x["V"], x["dO"], w.W, w.T, w.R, w.eps)
    ref = _full_oracle(w, x, range(w.bh))
    for s in BOTH:
        compare(for_schedule(got, s), ref[s], w.torch_dtype, f"{w.name}/{s}")


def test_batch4x8_L2048_full():
    """Every element of all 32 problems of the batch workload, both adjoint schedules."""
    w = BATCH_L2048
    x = make_inputs(w)
    say(f"[gpu] {w.name}")
    got = gpu_run_schedules(x["Q"], x["K"], x["V"], x["dO"], w.W, w.T, w.R, w.eps)
    ref = _full_oracle(w, x, range(w.bh))
    for s in BOTH:
        compare(for_schedule(got, s), ref[s], w.torch_dtype, f"{w.name}/{s}")


@pytest.mark.timeout(600)
def test_dustbin_block_L4096_all_heads():
    """Every element of all four dustbin_block problems (4097 tokens, dense support), both
    adjoint schedules through sinkhorn_attn_dustbin_block_vjp."""
    w = DUSTBIN_L4096
    x = make_inputs(w)
    say(f"[gpu] {w.name} all heads, both schedules")
    got = gpu_run_schedules(x["Q"], x["K"], x["V"], x["dO"], w.W, w.T, w.R, w.eps, dustbin=True)
    ref = _full_oracle(w, x, range(w.bh))
    for s in BOTH:
        compare(for_schedule(got, s), ref[s], w.torch_dtype, f"{w.name}/{s}")


def _every_row(w, chunk):
    x = make_inputs(w)
    say(f"[gpu] {w.name}: forward + both VJPs")
    got = gpu_run_schedules(x["Q"], x["K"], x["V"], x["dO"], w.W, w.T, w.R, w.eps)
    prob = oracle.BandProblem(W=w.W, T=w.T, R=w.R, eps=w.eps)
    ref = oracle_every_row(x, range(w.bh), prob, BOTH, w.name, chunk=chunk)
    for s in BOTH:
        compare(for_schedule(got, s), {"O": ref["O"], "duals": ref["duals"], **ref[s]},
                w.torch_dtype, f"{w.name}/{s} (every row)")


@pytest.mark.timeout(600)
def test_heads8_L32768_every_row():
    """Every element of all 8 heads at L = 32768 (T = 20): O, the saved duals and both
    schedules' dQ, dK, dV against the oracle, each head evaluated whole."""
    _every_row(HEADS8_L32K, chunk=32768)


@pytest.mark.timeout(900)
def test_long_L262144_every_row():
    """Every element of all 4 heads at L = 262144 (1,048,576 rows, the launch geometry the
    benchmark times): O, the saved duals and both schedules' dQ, dK, dV against the oracle.
    Each head is cut into ranges of 65536 rows, each evaluated exactly on its own window
    (oracle.row_range), so every segment seam of every kernel is covered, and both ends."""
    _every_row(LONG_L262K, chunk=65536)


@pytest.mark.parametrize("L,W,T,R,dtype", [(1000, 256, 4, 2, BF16), (333, 50, 3, 0, F32),
                                           (777, 128, 2, 1, BF16), (1000, 200, 3, 2, F32),
                                           (1000, 352, 3, 2, BF16), (700, 600, 3, 2, F32)])
def test_workspace_contents_do_not_matter(L, W, T, R, dtype):
    """The forward and VJP read no workspace location they have not written in the same call:
    a workspace filled with NaN bit patterns gives the same results, bit for bit, as a zeroed
    one (ragged L, several segments, R = 0, 1, 2; the fused step feeding the wide output pass,
    fp32 W = 200 and bf16 W = 352; the wide step, W = 600), for the VJP with and without the
    forward's output."""
    from entropic_ot_attention_amd import binding as B
    say(f"[gpu] workspace contents L={L} W={W} T={T} R={R} {dtype}")
    w, x = _inputs(2, L, W, T, 1.0, dtype, seed=31)
    dev = torch.device("cuda:0")
    Q, K, V, dO = (x[k].to(dev) for k in ("Q", "K", "V", "dO"))
    prob = B.make_problem(2, L, 64, W, T, R, 1.0, w.torch_dtype)
    outs = []
    for fill in (0, 255):
        ws_f = B.workspace_for(prob, B.SKA_OP_FWD, dev)
        ws_v = B.workspace_for(prob, B.SKA_OP_VJP, dev)
        ws_f.fill_(fill)
        ws_v.fill_(fill)
        O = torch.empty_like(Q)
        duals = torch.empty(2, B.n_duals(R), L, dtype=torch.float32, device=dev)
        B.sinkhorn_attn_fwd(prob, Q, K, V, O, duals, ws_f)
        res = [O, duals]
        for given_o in (None, O):
            dQ, dK, dV = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
            ws_v.fill_(fill)
            B.sinkhorn_attn_vjp(prob, Q, K, V, duals, dO, dQ, dK, dV, B.SCHEDULES["one_reference"],
                                ws_v, O=given_o)
            res += [dQ, dK, dV]
        torch.cuda.synchronize()
        outs.append([t.clone() for t in res])
    for a, b in zip(*outs):
        assert torch.isfinite(a.float()).all()
        assert torch.equal(a, b)
