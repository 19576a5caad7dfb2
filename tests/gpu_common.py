"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI binding and the
fp64 oracle on the same seeded inputs, and compare at the tolerance of the inputs' dtype
(fp32: max-abs 1e-4 on O, dQ, dK, dV; bf16: relative l2 1e-2)."""

from __future__ import annotations

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import oracle

TOL_F32_MAXABS = 1e-4
TOL_BF16_RELL2 = 1e-2
# The duals are fp32 on both sides of the bf16 path (scores from the same rounded inputs),
# so they are held to an absolute bar as well.
TOL_DUALS_F32 = 1e-4
TOL_DUALS_BF16 = 1e-3
# A relative bar is meaningless against a reference that is exactly zero: at W = 0 or L = 1 each
# row's plan holds one entry, the plan is the identity whatever the scores, and the exact dQ and
# dK are zero.  There bf16 gradients are held to an absolute bound.  The bf16 passes form the
# modifier as a split-bf16 product, within about 2^-16 of its terms (|g| ~ 10), and given the
# forward's output they take the row sum of P g as dO . O in fp32 instead of the matrix-core g
# (a difference of a few fp32 roundings of |g|), so dS keeps a residual near 1e-4 at most;
# 1e-3 bounds it with room.  (fp32 keeps max-abs 1e-4, which an exact zero does not change.)
ZERO_GRAD_MAXABS = 1e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_run(Q, K, V, dO, W, T, R=2, eps=1.0, schedule="one_reference", dustbin=False):
    from entropic_ot_attention_amd import binding as B
    dev = torch.device("cuda:0")
    Qd, Kd, Vd, dOd = (x.to(dev) for x in (Q, K, V, dO))
    O, duals = B.forward(Qd, Kd, Vd, W, T, R, eps, dustbin=dustbin)
    out = dict(O=O, duals=duals)
    if R <= 4:
        # the VJP given the forward's output (as the autograd wrapper calls it), and without it
        dQ, dK, dV = B.vjp(Qd, Kd, Vd, duals, dOd, W, T, R, eps, schedule=schedule, dustbin=dustbin,
                           O=O)
        out.update(dQ=dQ, dK=dK, dV=dV)
        dQ, dK, dV = B.vjp(Qd, Kd, Vd, duals, dOd, W, T, R, eps, schedule=schedule, dustbin=dustbin)
        out.update(dQ_noO=dQ, dK_noO=dK, dV_noO=dV)
    torch.cuda.synchronize()
    return {k: v.float().cpu().double().numpy() for k, v in out.items()}


def gpu_run_schedules(Q, K, V, dO, W, T, R=2, eps=1.0,
                      schedules=("one_reference", "direct_four"), dustbin=False):
    """One forward and, per schedule, the VJP through the C ABI given the forward's output O and
    without it; returns {"O", "duals", schedule: {"dQ", "dK", "dV", and
    "dQ_noO", "dK_noO", "dV_noO"}} as fp64 numpy arrays [bh, ...]."""
    from entropic_ot_attention_amd import binding as B
    dev = torch.device("cuda:0")
    Qd, Kd, Vd, dOd = (x.to(dev) for x in (Q, K, V, dO))
    O, duals = B.forward(Qd, Kd, Vd, W, T, R, eps, dustbin=dustbin)
    host = lambda t: t.float().cpu().double().numpy()
    out = {"O": host(O), "duals": host(duals)}
    for s in schedules:
        dQ, dK, dV = B.vjp(Qd, Kd, Vd, duals, dOd, W, T, R, eps, schedule=s, dustbin=dustbin, O=O)
        torch.cuda.synchronize()
        out[s] = {"dQ": host(dQ), "dK": host(dK), "dV": host(dV)}
        dQ, dK, dV = B.vjp(Qd, Kd, Vd, duals, dOd, W, T, R, eps, schedule=s, dustbin=dustbin)
        torch.cuda.synchronize()
        out[s].update(dQ_noO=host(dQ), dK_noO=host(dK), dV_noO=host(dV))
    torch.cuda.synchronize()
    return out


def for_schedule(res: dict, schedule: str) -> dict:
    """The flat {"O", "duals", "dQ", "dK", "dV"} view of one schedule's results."""
    return {"O": res["O"], "duals": res["duals"], **res[schedule]}


def oracle_head(Q, K, V, dO, W, T, R=2, eps=1.0, schedule="one_reference", dustbin=False):
    """Q..dO: one head as fp64 numpy arrays."""
    p = oracle.BandProblem(W=W, T=T, R=R, eps=eps)
    if dustbin:
        O, duals = oracle.dustbin_block_forward(Q, K, V, p)
        out = dict(O=O, duals=duals)
        if R <= 4:
            dQ, dK, dV = oracle.dustbin_block_vjp(Q, K, V, dO, duals, p, schedule=schedule)
            out.update(dQ=dQ, dK=dK, dV=dV)
        return out
    O, duals = oracle.forward(Q, K, V, p)
    out = dict(O=O, duals=duals)
    if R == 2:
        fn = oracle.vjp_one_reference if schedule == "one_reference" else oracle.vjp_direct_four
    elif R <= 4:
        fn = oracle.vjp_tail_one_reference     # general tail depth (one-reference schedule)
    else:
        fn = None
    if fn is not None:
        dQ, dK, dV = fn(Q, K, V, dO, duals, p)
        out.update(dQ=dQ, dK=dK, dV=dV)
    return out


def as64(x: torch.Tensor) -> np.ndarray:
    return x.float().double().numpy()


def compare(got: dict, ref: dict, dtype: torch.dtype, label: str, heads=None):
    """got: arrays [bh, ...]; ref: dict of lists per head (or arrays with leading head axis).
    Gradients the VJP gave without the forward's output (keys "<name>_noO") are held to the
    same bar against the same reference."""
    report = {}
    names = [n for n in ("O", "dQ", "dK", "dV", "duals") if n in ref]
    names += [n + "_noO" for n in ("dQ", "dK", "dV") if n in ref and n + "_noO" in got]
    for name in names:
        g = got[name] if heads is None else got[name][heads]
        r = np.asarray(ref[name.replace("_noO", "")])
        assert g.shape == r.shape, (name, g.shape, r.shape)
        assert np.all(np.isfinite(g)), f"{label}: non-finite values in {name}"
        err = float(np.abs(g - r).max())
        rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
        report[name] = (err, rel)
        if name == "duals":
            tol = TOL_DUALS_F32 if dtype == torch.float32 else TOL_DUALS_BF16
            assert err <= tol, f"{label}: duals max-abs {err:.3e} > {tol}"
        elif dtype == torch.float32:
            assert err <= TOL_F32_MAXABS, f"{label}: {name} max-abs {err:.3e} > {TOL_F32_MAXABS}"
        elif float(np.abs(r).max()) == 0.0:
            assert err <= ZERO_GRAD_MAXABS, f"{label}: {name} max-abs {err:.2e} against an exact zero"
        else:
            assert rel <= TOL_BF16_RELL2, f"{label}: {name} rel-l2 {rel:.3e} > {TOL_BF16_RELL2}"
    say(f"{label}: " + ", ".join(f"{k} maxabs={v[0]:.2e} rell2={v[1]:.2e}" for k, v in report.items()))
    return report


def oracle_workers() -> int:
    """Threads for the oracle: the host cores this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def parallel(fn, items, label: str):
    """fn over items on oracle_workers() threads, each numpy call single-threaded (numpy
    releases the interpreter lock inside its array loops); results in item order."""
    t0 = time.time()
    done = [0]

    def run(item):
        r = fn(item)
        done[0] += 1
        say(f"  {label}: {done[0]}/{len(items)} oracle tasks done ({time.time() - t0:.1f} s)")
        return r

    with threadpool_limits(1), ThreadPoolExecutor(min(oracle_workers(), len(items))) as ex:
        return list(ex.map(run, items))


def oracle_ranges(x: dict, tasks, prob, schedules, label: str):
    """oracle.row_range for each task (head, start, stop) on the seeded inputs x, in parallel."""
    heads = sorted({t[0] for t in tasks})
    arrs = {b: tuple(as64(x[k][b]) for k in ("Q", "K", "V", "dO")) for b in heads}
    return parallel(lambda t: oracle.row_range(*arrs[t[0]], prob, t[1], t[2], schedules),
                    list(tasks), label)


def oracle_every_row(x: dict, heads, prob, schedules, label: str, chunk: int = 65536):
    """Every row of the given heads from the oracle, each head cut into contiguous ranges of at
    most `chunk` rows evaluated on their own windows (exact: oracle.row_range).  Returns
    {"O": [nh, L, d], "duals": [nh, n_d, L], schedule: {"dQ", "dK", "dV": [nh, L, d]}}."""
    L = x["Q"].shape[1]
    tasks = [(b, a, min(L, a + chunk)) for b in heads for a in range(0, L, chunk)]
    parts = oracle_ranges(x, tasks, prob, schedules, label)
    out = {"O": [], "duals": []}
    for s in schedules:
        out[s] = {"dQ": [], "dK": [], "dV": []}
    for b in heads:
        mine = [p for t, p in zip(tasks, parts) if t[0] == b]
        out["O"].append(np.concatenate([p["O"] for p in mine]))
        out["duals"].append(np.concatenate([p["duals"] for p in mine], axis=1))
        for s in schedules:
            for k in ("dQ", "dK", "dV"):
                out[s][k].append(np.concatenate([p[s][k] for p in mine]))
    return out
