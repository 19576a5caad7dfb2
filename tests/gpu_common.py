"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI binding and the
fp64 oracle on the same seeded inputs, and compare at the tolerance of the inputs' dtype
(fp32: max-abs 1e-4 on O, dQ, dK, dV; bf16: relative l2 1e-2)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

TOL_F32_MAXABS = 1e-4
TOL_BF16_RELL2 = 1e-2
# The duals are fp32 on both sides of the bf16 path (scores from the same rounded inputs),
# so they are held to an absolute bar as well.
TOL_DUALS_F32 = 1e-4
TOL_DUALS_BF16 = 1e-3


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
        dQ, dK, dV = B.vjp(Qd, Kd, Vd, duals, dOd, W, T, R, eps, schedule=schedule, dustbin=dustbin)
        out.update(dQ=dQ, dK=dK, dV=dV)
    torch.cuda.synchronize()
    return {k: v.float().cpu().double().numpy() for k, v in out.items()}


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
    """got: arrays [bh, ...]; ref: dict of lists per head (or arrays with leading head axis)."""
    report = {}
    for name in ("O", "dQ", "dK", "dV", "duals"):
        if name not in ref:
            continue
        g = got[name] if heads is None else got[name][heads]
        r = np.asarray(ref[name])
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
        else:
            assert rel <= TOL_BF16_RELL2, f"{label}: {name} rel-l2 {rel:.3e} > {TOL_BF16_RELL2}"
    say(f"{label}: " + ", ".join(f"{k} maxabs={v[0]:.2e} rell2={v[1]:.2e}" for k, v in report.items()))
    return report
