"""GPU checks that every launch of a call goes to the stream the caller gives: the forward and the
VJP run on side streams (default priority) give the same results, bit for bit, as on the current
stream, also with two problems in flight at once on two streams, each with its own workspace."""

import pytest
import torch

from entropic_ot_attention_amd import binding as B
from entropic_ot_attention_amd.workloads import Workload, make_inputs
from tests.gpu_common import say

pytestmark = pytest.mark.gpu

# name, L, W, T, R, dtype, dustbin, schedule: the fused step with the streaming passes (bf16 and
# fp32, both schedules), the wide engine, the dense dustbin and the general-depth passes
CASES = [
    ("fused_bf16", 1000, 256, 5, 2, "bf16", False, "one_reference"),
    ("fused_f32_direct_four", 700, 64, 4, 2, "f32", False, "direct_four"),
    ("wide_f32", 900, 600, 3, 2, "f32", False, "one_reference"),
    ("dustbin_f32", 300, 64, 3, 2, "f32", True, "one_reference"),
    ("general_depth_bf16", 600, 128, 3, 3, "bf16", False, "one_reference"),
]


def _inputs(case, seed):
    name, L, W, T, R, dtype, dustbin, _ = case
    x = make_inputs(Workload(name, 1, 2, L, 64, W, T, R, 1.0, dtype, seed, dustbin=dustbin))
    dev = torch.device("cuda:0")
    return tuple(x[k].to(dev) for k in ("Q", "K", "V", "dO"))


def _run(case, tensors, stream=None):
    _, _, W, T, R, _, dustbin, schedule = case
    Q, K, V, dO = tensors
    O, duals = B.forward(Q, K, V, W, T, R, 1.0, dustbin=dustbin, stream=stream)
    dQ, dK, dV = B.vjp(Q, K, V, duals, dO, W, T, R, 1.0, schedule=schedule, dustbin=dustbin,
                       stream=stream)
    return (O, duals, dQ, dK, dV)


def _same(ref, got, what):
    for name, a, b in zip(("O", "duals", "dQ", "dK", "dV"), ref, got):
        assert torch.equal(a, b), f"{what}: {name} differs from the current-stream result"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_side_stream_matches_current_stream(case):
    say(f"[gpu] streams: {case[0]} on a side stream")
    tensors = _inputs(case, 21)
    ref = _run(case, tensors)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # allocations and launches on the side stream
        got = _run(case, tensors)
    side.synchronize()
    _same(ref, got, case[0])
    # the stream passed as an argument while another one is current: the binding allocates on
    # the current stream, so the side stream waits for it, and the current one for the results
    side2 = torch.cuda.Stream()
    side2.wait_stream(torch.cuda.current_stream())
    got2 = _run(case, tensors, stream=side2)
    torch.cuda.current_stream().wait_stream(side2)
    torch.cuda.synchronize()
    _same(ref, got2, case[0] + " (explicit stream)")


def test_two_problems_in_flight_on_two_streams():
    say("[gpu] streams: two problems at once")
    a_case, b_case = CASES[0], CASES[2]
    ta, tb = _inputs(a_case, 31), _inputs(b_case, 32)
    ref_a, ref_b = _run(a_case, ta), _run(b_case, tb)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(sa):
        got_a = _run(a_case, ta)
    with torch.cuda.stream(sb):
        got_b = _run(b_case, tb)
    sa.synchronize()
    sb.synchronize()
    _same(ref_a, got_a, a_case[0] + " beside " + b_case[0])
    _same(ref_b, got_b, b_case[0] + " beside " + a_case[0])


def test_two_host_threads_on_two_streams():
    """Two host threads call the library at once, each on its own stream (the binding releases
    the interpreter lock during the calls): the results match the single-thread ones."""
    import threading
    say("[gpu] streams: two host threads")
    cases = [CASES[0], CASES[1]]
    tensors = [_inputs(c, 41 + i) for i, c in enumerate(cases)]
    refs = [_run(c, t) for c, t in zip(cases, tensors)]
    torch.cuda.synchronize()
    got = [None, None]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.default_stream())
            with torch.cuda.stream(s):
                for _ in range(3):
                    got[i] = _run(cases[i], tensors[i])
            s.synchronize()
        except Exception as e:      # reported below, in the test's own thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    for c, r, g in zip(cases, refs, got):
        _same(r, g, c[0] + " (two host threads)")
