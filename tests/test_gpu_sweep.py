"""A seeded sweep of random configurations through the C ABI against the fp64 oracle: token counts
from 1 to 2000 (ragged against every tile and block size), even band widths from 0 to 600
(streaming, register-resident and wide engines), T from 0 to 6, tail depths R = 0..4, epsilon
0.5..2, bf16 and fp32, both adjoint schedules at R = 2, and the dustbin augmentation; then a few
mid-size problems (3000-12000 tokens, up to three heads: many segments and seams) and calls of
16-160 short problems.  Every element is compared at the tolerances of the other parity tests.

At W = 0 each row's plan holds a single entry: the plan is the identity whatever the scores, so
the exact dQ and dK are zero; compare holds bf16 gradients against an exact zero to an absolute
bound (ZERO_GRAD_MAXABS)."""

import random

import pytest

from entropic_ot_attention_amd.workloads import Workload, make_inputs
from tests.gpu_common import compare, for_schedule, gpu_run_schedules, oracle_head, parallel, say

pytestmark = pytest.mark.gpu


def _configs(seed=3, n=48):
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        dt = rng.choice(["bf16", "f32"])
        dustbin = rng.random() < 0.15
        if dustbin:
            dt = "f32"
        L = rng.choice([rng.randint(1, 80), rng.randint(60, 700), rng.randint(600, 2000)])
        W = 2 * rng.choice([0, rng.randint(1, 32), rng.randint(32, 150), rng.randint(150, 300)])
        if dustbin:
            L = min(L, 600)
        R = rng.choice([0, 1, 2, 2, 2, 3, 4])
        T = rng.randint(1 if R == 0 else 0, 6)
        eps = rng.choice([0.5, 1.0, 2.0])
        bh = rng.choice([1, 2])
        out.append((bh, L, W, T, R, eps, dt, dustbin, rng.randint(0, 10**6)))
    return out


def _mid_configs(seed=5, n=3):
    """Mid-size problems: many segments per head at varied segment lengths and seams."""
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        L = rng.randint(3000, 12000)
        W = 2 * rng.randint(16, 200)
        dt = rng.choice(["bf16", "f32"])
        out.append((rng.choice([1, 2, 3]), L, W, rng.randint(1, 3), rng.choice([0, 2, 2, 3]),
                    rng.choice([0.5, 1.0, 2.0]), dt, False, rng.randint(0, 10**6)))
    return out


def _many_head_configs(seed=13, n=3):
    """Many short problems in one call (one segment each)."""
    rng = random.Random(seed)
    return [(rng.choice([16, 64, 160]), rng.randint(1, 300), 2 * rng.randint(0, 150),
             rng.randint(1, 4), rng.choice([0, 2, 3]), rng.choice([0.5, 1.0, 2.0]),
             rng.choice(["bf16", "f32"]), False, rng.randint(0, 10**6)) for _ in range(n)]


CONFIGS = _configs() + _mid_configs() + _many_head_configs()


def _id(c):
    bh, L, W, T, R, eps, dt, dustbin, _ = c
    return f"bh{bh}_L{L}_W{W}_T{T}_R{R}_eps{eps}_{dt}" + ("_dustbin" if dustbin else "")


@pytest.mark.parametrize("cfg", CONFIGS, ids=[_id(c) for c in CONFIGS])
def test_random_configuration_matches_the_oracle(cfg):
    bh, L, W, T, R, eps, dt, dustbin, seed = cfg
    label = "[gpu] sweep " + _id(cfg)
    say(label)
    w = Workload("sweep", 1, bh, L, 64, W, T, R, eps, dt, seed, dustbin=dustbin)
    x = make_inputs(w)
    schedules = ("one_reference", "direct_four") if R == 2 else ("one_reference",)
    got = gpu_run_schedules(x["Q"], x["K"], x["V"], x["dO"], W, T, R, eps, schedules=schedules,
                            dustbin=dustbin)
    heads = [tuple(x[k][b].double().numpy() for k in ("Q", "K", "V", "dO")) for b in range(bh)]
    for s in schedules:
        refs = parallel(lambda h: oracle_head(*h, W, T, R, eps, s, dustbin=dustbin), heads, label)
        ref = {k: [r[k] for r in refs] for k in refs[0]}
        compare(for_schedule(got, s), ref, w.torch_dtype, f"{label} {s}")
