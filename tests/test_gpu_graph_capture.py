"""HIP graph capture of the library's calls: the forward that allocates nothing
(sinkhorn_attn_fwd_noalloc, whose scratch address the eager call looks up before any capture),
and the forward and VJP with caller workspaces.  Each is captured once and replayed several
times with eager work and synchronisation between the replays; every replay gives the eager
calls' results bit for bit."""

import pytest
import torch

from entropic_ot_attention_amd.workloads import Workload, make_inputs
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

# name, bh, L, W, T, R, dtype: the fused step (bf16, and fp32 at R = 0), the wide path
CASES = [
    ("fused_bf16_L3000_W256", 2, 3000, 256, 4, 2, "bf16"),
    ("fused_f32_L900_W128_R0", 2, 900, 128, 3, 0, "f32"),
    ("wide_f32_L700_W600", 1, 700, 600, 3, 2, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_captured_forward_replays_match_the_eager_call(case):
    from entropic_ot_attention_amd import binding as B
    name, bh, L, W, T, R, dt = case
    say(f"[gpu] graph capture: {name}")
    w = Workload("graph", 1, bh, L, 64, W, T, R, 1.0, dt, 50)
    x = make_inputs(w, with_cotangent=False)
    dev = torch.device("cuda:0")
    Q, K, V = (x[k].to(dev) for k in ("Q", "K", "V"))
    prob = B.make_problem(bh, L, 64, W, T, R, 1.0, w.torch_dtype)
    O = torch.empty_like(Q)
    d = torch.empty(bh, B.n_duals(R), L, dtype=torch.float32, device=dev)
    B.sinkhorn_attn_fwd_noalloc(prob, Q, K, V, O, d)
    torch.cuda.synchronize()
    O_ref, d_ref = O.clone(), d.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.sinkhorn_attn_fwd_noalloc(prob, Q, K, V, O, d)
    torch.cuda.synchronize()
    for i in range(4):
        O.fill_(float("nan"))               # eager work between the replays
        d.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(O, O_ref), f"{name}: O after replay {i}"
        assert torch.equal(d, d_ref), f"{name}: duals after replay {i}"


# name, bh, L, W, T, R, dtype, schedule: the streaming passes (both schedules) and the wide passes
STEP_CASES = [
    ("stream_bf16_one_reference", 2, 1000, 256, 4, 2, "bf16", "one_reference"),
    ("stream_f32_direct_four", 2, 700, 64, 3, 2, "f32", "direct_four"),
    ("wide_f32_one_reference", 1, 700, 600, 3, 2, "f32", "one_reference"),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_captured_forward_and_vjp_replay_match_the_eager_calls(case):
    """sinkhorn_attn_fwd and sinkhorn_attn_vjp with caller workspaces and outputs allocated before
    the capture: the whole training-step kernel sequence as one graph."""
    from entropic_ot_attention_amd import binding as B
    name, bh, L, W, T, R, dt, sched = case
    say(f"[gpu] graph capture fwd + vjp: {name}")
    w = Workload("graph", 1, bh, L, 64, W, T, R, 1.0, dt, 51)
    x = make_inputs(w)
    dev = torch.device("cuda:0")
    Q, K, V, dO = (x[k].to(dev) for k in ("Q", "K", "V", "dO"))
    prob = B.make_problem(bh, L, 64, W, T, R, 1.0, w.torch_dtype)
    ws_f = B.workspace_for(prob, B.SKA_OP_FWD, dev)
    ws_v = B.workspace_for(prob, B.SKA_OP_VJP, dev)
    O = torch.empty_like(Q)
    d = torch.empty(bh, B.n_duals(R), L, dtype=torch.float32, device=dev)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
    sch = B.SCHEDULES[sched]
    outs = (O, d, dQ, dK, dV)

    def step():
        B.sinkhorn_attn_fwd(prob, Q, K, V, O, d, ws_f)
        B.sinkhorn_attn_vjp(prob, Q, K, V, d, dO, dQ, dK, dV, sch, ws_v, O=O)

    step()
    torch.cuda.synchronize()
    ref = tuple(t.clone() for t in outs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        for t in outs:                      # eager work between the replays
            t.fill_(float("nan"))
        ws_f.fill_(255)                     # every fp32 word of the workspaces a NaN
        ws_v.fill_(255)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for nm, a, b in zip(("O", "duals", "dQ", "dK", "dV"), ref, outs):
            assert torch.equal(a, b), f"{name}: {nm} after replay {i}"
