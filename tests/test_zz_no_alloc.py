"""The forward entry point that allocates nothing (sinkhorn_attn_fwd_noalloc, workspace in the
library's static device array) against sinkhorn_attn_fwd with a caller workspace, through the
C ABI: two calls in a row on the same GPU, the second on a smaller problem (the array then holds
the first call's contents), on the fused band path and on the wide path.  Both entry points run
the same kernels on the same inputs, so O and the saved duals must agree bit for bit."""

import pytest
import torch

from entropic_ot_attention_amd.workloads import Workload, make_inputs
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

CALLS = [
    # name, bh, L, W, T, R, dtype: the second call is smaller than the first
    ("fused_bf16_L3000_W256", 2, 3000, 256, 4, 2, "bf16"),
    ("wide_f32_L700_W600", 1, 700, 600, 3, 2, "f32"),
]


def _run_both(bh, L, W, T, R, dtype, seed):
    from entropic_ot_attention_amd import binding as B
    w = Workload("noalloc", 1, bh, L, 64, W, T, R, 1.0, dtype, seed)
    x = make_inputs(w, with_cotangent=False)
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("Q", "K", "V"))
    prob = B.make_problem(bh, L, 64, W, T, R, 1.0, w.torch_dtype)
    ws = B.workspace_for(prob, B.SKA_OP_FWD, dev)
    O_ref = torch.empty_like(Q)
    d_ref = torch.empty(bh, B.n_duals(R), L, dtype=torch.float32, device=dev)
    B.sinkhorn_attn_fwd(prob, Q, K, V, O_ref, d_ref, ws)
    O = torch.full_like(Q, float("nan"))
    d = torch.full_like(d_ref, float("nan"))
    B.sinkhorn_attn_fwd_noalloc(prob, Q, K, V, O, d)
    torch.cuda.synchronize()
    return (O_ref, d_ref), (O, d)


def test_noalloc_forward_matches_workspace_forward_on_consecutive_calls():
    for n, (name, bh, L, W, T, R, dt) in enumerate(CALLS):
        say(f"[gpu] noalloc forward call {n + 1}: {name} bh={bh} L={L} W={W} T={T} R={R} {dt}")
        (O_ref, d_ref), (O, d) = _run_both(bh, L, W, T, R, dt, seed=40 + n)
        assert torch.isfinite(O.float()).all() and torch.isfinite(d).all()
        assert torch.equal(O, O_ref), name
        assert torch.equal(d, d_ref), name


def test_noalloc_forward_rejects_problems_beyond_the_static_scratch():
    from entropic_ot_attention_amd import binding as B
    prob = B.make_problem(8, 262144, 64, 256, 15, 2, 1.0, torch.bfloat16)
    assert B.ska_workspace_bytes(prob, B.SKA_OP_FWD) > (32 << 20)
    dev = torch.device("cuda:0")
    t = torch.empty(16, dtype=torch.bfloat16, device=dev)
    with pytest.raises(B.SinkhornAttnError) as e:
        B.sinkhorn_attn_fwd_noalloc(prob, t, t, t, t, t.float())
    assert "static scratch" in str(e.value)
