"""GPU checks of the library's launch timing (ska_timing_*): counts per kernel family, reset on
enable, nothing counted while disabled, and launches left pending by an earlier enable dropped
when timing is enabled again."""

import pytest
import torch

from entropic_ot_attention_amd import binding as B
from entropic_ot_attention_amd.workloads import Workload, make_inputs
from tests.gpu_common import say

pytestmark = pytest.mark.gpu


def _run_once(T=3, R=2, L=700, W=128):
    w = Workload("timing", 1, 2, L, 64, W, T, R, 1.0, "bf16", 11)
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    Q, K, V, dO = (x[k].to(dev) for k in ("Q", "K", "V", "dO"))
    O, duals = B.forward(Q, K, V, W, T, R, 1.0)
    B.vjp(Q, K, V, duals, dO, W, T, R, 1.0)
    torch.cuda.synchronize()


def test_launch_counts_and_reset():
    say("[gpu] timing: counts, reset, disabled")
    T, R = 3, 2
    _run_once(T, R)                        # build and warm up outside any timed region
    B.ska_timing_enable(True)
    _run_once(T, R)
    ms, n = B.ska_timing_read(B.TIMED_STEP)
    assert n == T + R and ms > 0.0         # one fused step launch per Sinkhorn step
    ms_out, n_out = B.ska_timing_read(B.TIMED_OUT)
    assert n_out == 1 and ms_out > 0.0
    _, n_vjp = B.ska_timing_read(B.TIMED_VJP)
    assert n_vjp == 4                      # the four streaming VJP passes at R = 2
    B.ska_timing_enable(False)
    _run_once(T, R)                        # not counted
    assert B.ska_timing_read(B.TIMED_STEP)[1] == T + R
    B.ska_timing_enable(True)              # reset
    assert B.ska_timing_read(B.TIMED_STEP) == (0.0, 0)
    B.ska_timing_enable(False)


def test_reenable_drops_pending_launches():
    say("[gpu] timing: re-enable drops pending launches")
    _run_once()
    B.ska_timing_enable(True)
    _run_once()                            # pending until read
    B.ska_timing_enable(True)              # drops them
    assert B.ska_timing_read(B.TIMED_STEP) == (0.0, 0)
    _run_once(T=4, R=1)
    assert B.ska_timing_read(B.TIMED_STEP)[1] == 5
    B.ska_timing_enable(False)
