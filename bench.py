"""Benchmark: forward + exact R=2 VJP of banded balanced Sinkhorn attention on one MI355X.

One step = sinkhorn_attn_fwd followed by sinkhorn_attn_vjp (one-reference schedule, given the
forward's output as the autograd wrapper passes it) on the
seeded synthetic workload "seq1x4_L262144_W256_bf16" (one sequence, 4 heads, L = 262144
tokens, d = 64, band W = 256, T = 15 base steps, R = 2, bf16 inputs, fp32 duals).  Inputs are
resident in HBM before the timed region.  The metric is tokens of the sequence per second:
L / (t_fwd + t_vjp) for all heads together; the median step is reported beside the mean.

Prints ONE JSON line.  Besides the throughput it reports, for the dominant kernel (the fused
balanced Sinkhorn step, T + R launches per step), its average launch time measured with HIP
events on its own stream during the last timed step (per-launch events add GPU idle time, so
they are kept out of the other timed steps) and the achieved fraction of its binding roofline:
its minimal VALU work (bf16; its floor lies above the HBM floor of reading Q and K once) or its
matrix-core work (fp32), with the HBM and matrix-core fractions, the measured HBM bytes per
launch and the SQ-counter busy fractions of the committed rocprofv3 records (when they describe
the current source) beside it, and the same fractions for the output pass, the VJP passes and
the whole step.  The fp64 CPU oracle runs on the same workload first, one process per head.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# VALU roofline of MI355X from unit counts and clock: the fp32 vector peak of 157.3 TFLOP/s is
# 256 CUs x 4 SIMDs x 32 fma lanes per cycle x 2 flops x 2.4 GHz, i.e. a wave64 fp32 instruction
# every 2 cycles per SIMD: 78.6e12 lane-operations per second.  Unpacked instructions reach it
# (measured with the shader clock: 2.5 cycles per wave64 fma with two or more waves per SIMD, 5
# with one).  v_exp_f32 issues at a quarter of that rate (8.5-10 cycles measured), so one
# exponential takes 4 issue slots.
VALU_LANE_OPS_PER_S = 256 * 4 * 32 * 2.4e9
EXP_SLOTS = 4
# Minimal VALU work of one fused balanced Sinkhorn step per band entry: form the exponent with the
# row shift already in the matrix-core accumulator (1 fma), exponentiate (1 exp = 4 slots),
# accumulate the row sum (1 add) and the column sum of the normalised plan (1 fma): 7 issue slots.
SLOTS_PER_ENTRY_STEP = 3 + EXP_SLOTS
# Issue time on a SIMD: matrix-core products and vector instructions of one SIMD do not overlap
# (measured: a wave of bf16 products beside a wave of fmas takes the sum of their times), so the
# step's SIMD floor adds its products' cycles (two bf16 16x16x32 products of 16 cycles per 16 x 16
# tile) and its VALU cycles (2 per issue slot of a wave64 instruction).
N_SIMD = 256 * 4
CLOCK_HZ = 2.4e9
BF16_MFMA_CYCLES = 16
VALU_SLOT_CYCLES = 2
HBM_PEAK_GBS = 8000.0
# O(L) fp32 vectors one step reads and writes per token and head: previous column duals, previous
# row duals, column partials in; row duals, column duals, column partials out
STEP_VECTOR_BYTES_PER_TOKEN = 6 * 4
MFMA_BF16_PEAK_TFLOPS = 2500.0      # dense
MFMA_F32_PEAK_TFLOPS = 157.3
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_sinkhorn_step_kernel.json")


def band_entries(L: int, h: int) -> int:
    """|{(i, j): 0 <= i, j < L, |i - j| <= h}|."""
    h = min(h, L - 1) if L > 0 else 0
    return L * (2 * h + 1) - h * (h + 1)


def traffic_per_launch(workload: str):
    """HBM bytes per step-kernel launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    record, or None when there is none, it was taken on another workload, or the kernel source
    changed since it was taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
        from entropic_ot_attention_amd.profiling import source_sha
        if rec.get("source_sha256") != source_sha() or rec.get("workload") != workload:
            return None
        return round(float(rec["bytes_per_launch"]))
    except (OSError, ValueError, KeyError):
        return None


STEP_COUNTER_RECORD = os.path.join(ROOT, "profiles", "counters_sinkhorn_step_kernel.json")


def step_counters(workload: str):
    """Unit busy fractions of the step kernel from the committed rocprofv3 SQ-counter record, or
    None when there is none, it is of another workload, or the kernel changed since."""
    try:
        with open(STEP_COUNTER_RECORD) as f:
            rec = json.load(f)
        from entropic_ot_attention_amd.profiling import source_sha
        if rec.get("source_sha256") != source_sha() or rec.get("workload") != workload:
            return None
        return {k: rec[k] for k in ("valu_busy", "mfma_busy", "lds_busy", "valu_insts_per_wave",
                                    "trans_insts_per_wave", "waves", "record")}
    except (OSError, ValueError, KeyError):
        return None


# matrix-core flops per band entry of the R = 2 VJP given the forward's output, in units of d:
# pass 1 score + dV contraction (4), pass 2 score (2), pass 3 score + g + two dQ contractions (8),
# pass 4 score + g + dK contraction (6)
VJP_R2_FLOPS_PER_ENTRY_D = 20


def family_rooflines(w, rows, nnz, elt, schedule, step_launch_ms, out_launch_ms, vjp_ms, step_ms):
    """Algorithmic work and achieved fractions of each kernel family of one forward + VJP, from
    their HIP-event times: one Sinkhorn step launch, the output pass, the R = 2 VJP passes
    (the four streaming passes, given the forward's output: dV and dv2 = V . dV; du2 from dO . O
    with the dv1 column partials; du1 and dQ; dK) and the whole step.  Bytes are each family's
    compulsory tensor traffic (every pass streams the tensors it reads once and writes its outputs
    once); flops are matrix-core flops per band entry with the scores (and value scores g)
    recomputed in every pass that needs them: 4 d, 2 d, 8 d and 6 d, 20 d in all; exponentials
    per band entry: 1 per step and output pass, 1 per VJP pass (one-reference) or 1 + 2 + 4 + 4
    (direct-four)."""
    d, bh = w.d, w.bh
    tens = bh * rows * d * elt                       # bytes of one [bh, tokens, d] tensor
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    exp_peak = VALU_LANE_OPS_PER_S / EXP_SLOTS / 1e12

    def fr(ms, byts, flops, exps, extra=None):
        t = ms / 1e3
        r = {"ms": round(ms, 4), "bytes": int(byts), "flops": int(flops), "exps": int(exps),
             "hbm_GB_per_s": round(byts / t / 1e9, 1), "hbm_frac": round(byts / t / 1e9 / HBM_PEAK_GBS, 4),
             "mfma_TFLOP_per_s": round(flops / t / 1e12, 1), "mfma_peak": mfma_peak,
             "mfma_frac": round(flops / t / 1e12 / mfma_peak, 4),
             "exp_T_per_s": round(exps / t / 1e12, 3), "exp_frac": round(exps / t / 1e12 / exp_peak, 4)}
        if extra:
            r.update(extra)
        return r

    n_steps = w.T + w.R
    step = fr(step_launch_ms, 2 * tens, 2 * d * nnz, nnz,
              {"bytes_with_vectors": 2 * tens + STEP_VECTOR_BYTES_PER_TOKEN * bh * rows,
               "valu_T_per_s": round(SLOTS_PER_ENTRY_STEP * nnz / (step_launch_ms / 1e3) / 1e12, 3),
               "valu_frac": round(SLOTS_PER_ENTRY_STEP * nnz / (step_launch_ms / 1e3)
                                  / VALU_LANE_OPS_PER_S, 4),
               "per": "one launch (one full Sinkhorn step)"})
    out = fr(out_launch_ms, 4 * tens, 4 * d * nnz, nnz, {"per": "one launch: O = P V"})
    res = {"step": step, "output": out}
    if w.R == 2:
        vexp = (1 + 2 + 4 + 4) if schedule == "direct_four" else 4
        vjp = fr(vjp_ms, 19 * tens, VJP_R2_FLOPS_PER_ENTRY_D * d * nnz, vexp * nnz,
                 {"per": "one VJP given O: 4 passes reading 4 tensors each, writing dQ, dK, dV"})
        res["vjp"] = vjp
        whole_exps = (n_steps + 1 + vexp) * nnz
        res["whole_step"] = fr(step_ms, n_steps * 2 * tens + 4 * tens + 19 * tens,
                               (n_steps * 2 + 4 + VJP_R2_FLOPS_PER_ENTRY_D) * d * nnz, whole_exps,
                               {"per": f"forward ({n_steps} steps, output) + VJP"})
    return res


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # a fresh GPU takes a few tens of steps to reach steady clocks: the first 10 timed steps
    # after 3 warm-up steps ran ~4% slower than the next ones
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="seq1x4_L262144_W256_bf16")
    ap.add_argument("--schedule", default="one_reference", choices=["one_reference", "direct_four"])
    ap.add_argument("--tail-depth", type=int, default=0,
                    help="run the named workload with this tail depth R (1..4) instead of its own")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None,
                    help="tokens per head in the oracle's CPU baseline (default: all of them; the "
                         "certificate, contraction and training modes: a bounded sample)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="one device copy of this many MiB before warmup (counter calibration)")
    ap.add_argument("--certificate", action="store_true",
                    help="time the a posteriori bias certificate eta_R (fp32 inputs) for "
                         "R = 0..--r-max on the workload instead of the forward + VJP step")
    ap.add_argument("--r-max", type=int, default=4)
    ap.add_argument("--contraction", action="store_true",
                    help="time the projective contraction certificate of the workload's active "
                         "blocks instead of the forward + VJP step")
    ap.add_argument("--block", type=int, default=16)
    ap.add_argument("--train", action="store_true",
                    help="time the synthetic masked-reconstruction training step (projections, "
                         "the attention layer, loss, SGD) instead of the attention op alone")
    ap.add_argument("--train-workload", default="train_b8_L1024_D1280_W256_T15_bf16")
    ap.add_argument("--tau", type=float, default=1e-5)
    return ap.parse_args()


def warm_up(run, warmup: int, instrumented: int = 1) -> None:
    """`warmup` untimed calls; the library's per-launch timing is on during the last
    `instrumented` of them, so the HIP events that the timed region's instrumented calls use
    exist before that region starts."""
    import torch
    from entropic_ot_attention_amd import binding as B
    for i in range(warmup):
        if i == max(0, warmup - instrumented):
            B.ska_timing_enable(True)
        run()
    torch.cuda.synchronize()
    B.ska_timing_enable(False)


def timed_region(run, steps: int, stream, instrumented: int = 1):
    """Time `steps` calls run(i) between two HIP events on `stream`, synchronised on both sides.
    The library's per-launch HIP events (for the roofline's launch average) are on only during
    the last `instrumented` calls: each event pair leaves the GPU idle for a few microseconds
    between launches, which would otherwise be charged to every timed step.
    Returns (ms per call, host wall seconds, number of instrumented calls)."""
    import torch
    from entropic_ot_attention_amd import binding as B
    n_inst = max(1, min(instrumented, steps))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        if i == steps - n_inst:
            B.ska_timing_enable(True)
        run(i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / steps, time.perf_counter() - t0, n_inst


def tail_pass_flops_per_entry(R: int, d: int) -> int:
    """Matrix-core flops per band entry of the one-reference adjoint at tail depth R >= 1, with
    one score recompute per sweep over the band: dV and dv^(R) = V . dV (score and the dV
    contraction, 4 d), du^(R) (score and value scores g = dO . V, 4 d), one sweep per level
    a = R-1 .. 1 that both reduces its row sums and emits the next level's column partials
    (score, 2 d each), dQ (score, g and the contraction, 6 d) and dK (the same, 6 d):
    (18 + 2 R) d.  The streaming passes run exactly this (without the forward's output, as the
    certificate runs them); the wide engine's passes, with two sweeps per level, do more."""
    return (18 + 2 * R) * d


def contraction_main(args):
    """Projective contraction certificate on the GPU: the diameters and Birkhoff-Hopf coefficients
    of every active block pair of the workload, timed over --steps calls; the roofline is the
    certificate kernel's VALU work (B (B - 1) / 2 row pairs x B columns x 2 operations per active
    block pair: a subtraction, and half of a 3-input maximum and of a 3-input minimum) against the
    MI355X VALU peak, with its HBM floor (Q and K read once) beside it.
    The oracle's block_diameters runs beside it on a sample."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from entropic_ot_attention_amd import binding as B
    from entropic_ot_attention_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    blk = args.block
    dev = torch.device("cuda:0")
    x = make_inputs(w, with_cotangent=False)
    Q, K = x["Q"].to(dev), x["K"].to(dev)
    rows = w.tokens
    prob = B.make_problem(w.bh, w.L, w.d, w.W, 1, 2, w.eps, w.torch_dtype)
    op = B.SKA_OP_DUSTBIN_BLOCK_CONTRACTION if w.dustbin else B.SKA_OP_CONTRACTION
    nb, m = B.ska_contraction_layout(prob, op, blk)
    delta = torch.empty(w.bh, nb, 2 * m + 1, dtype=torch.float32, device=dev)
    kappa = torch.empty_like(delta)
    dmax = torch.empty(w.bh, dtype=torch.float32, device=dev)
    fn = (B.sinkhorn_attn_dustbin_block_contraction_certificate if w.dustbin
          else B.sinkhorn_attn_contraction_certificate)
    stream = torch.cuda.current_stream()
    warm_up(lambda: fn(prob, blk, Q, K, delta, kappa, dmax, stream), args.warmup, instrumented=3)
    call_ms, _, _ = timed_region(lambda i: fn(prob, blk, Q, K, delta, kappa, dmax, stream),
                                 args.steps, stream, instrumented=3)
    k_ms, k_n = B.ska_timing_read(B.TIMED_CERT)
    B.ska_timing_enable(False)
    d = delta.cpu().double().numpy()
    act = d >= 0
    # VALU work per active block pair: nr (nr - 1) / 2 row pairs x nc columns x 2 operations
    sizes = np.minimum(blk, rows - blk * np.arange(nb))
    o = np.arange(-m, m + 1)
    nr = sizes[:, None]
    cb = np.arange(nb)[:, None] + o[None, :]
    nc = np.where((cb >= 0) & (cb < nb), sizes[np.clip(cb, 0, nb - 1)], 0)
    ops = float((act * (2.0 * nr * (nr - 1) / 2 * nc)[None]).sum())
    launch_s = k_ms / max(k_n, 1) / 1e3
    elt = 2 if w.dtype == "bf16" else 4
    hbm_bytes = 2 * w.bh * rows * w.d * elt + 2 * delta.numel() * 4
    achieved = ops / launch_s / 1e12
    peak = VALU_LANE_OPS_PER_S / 1e12
    kap = np.tanh(d[act] / 4)
    out = {
        "metric": f"projective contraction certificate tokens/s at L={w.L} W={w.W} d={w.d}, "
                  f"block {blk}; % of VALU roofline",
        "value": round(w.batch * w.L / (call_ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(call_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) Q/K)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "L": w.L, "d": w.d,
                   "W": w.W, "epsilon": w.eps, "block": blk},
        "certificate": {"active_block_pairs": int(act.sum()),
                        "delta_max": float(d[act].max()) if act.any() else None,
                        "delta_median": float(np.median(d[act])) if act.any() else None,
                        "kappa_max": float(kap.max()) if act.any() else None,
                        "kappa_median": float(np.median(kap)) if act.any() else None},
        "roofline": {
            "bound": "alu",
            "kernel": f"contraction_kernel<{w.dtype}, {blk}>",
            "achieved": round(achieved, 3),
            "peak": round(peak, 3),
            "unit": "T VALU lane-ops/s",
            "frac": round(achieved / peak, 4),
            "traffic": None,
            "avg_launch_us": round(launch_s * 1e6, 2),
            "launches_timed": k_n,
            "algorithmic_work": f"{ops:.4g} lane-ops (2 per row pair and column of each active "
                                f"block pair)",
            "hbm_floor_us": round(hbm_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        n = min(args.cpu_sample_tokens or 262144, rows)
        n -= n % blk if n > blk else 0
        Qh, Kh = (x[k][0, :n].double().numpy() for k in ("Q", "K"))
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.block_diameters(Qh, Kh, oracle.BandProblem(W=w.W, T=1, R=2, eps=w.eps), blk,
                                   w.dustbin)
            dt = time.perf_counter() - t0
        out["cpu_baseline"] = {
            "value": round(n / (w.bh * dt), 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"head 0 of {w.bh}, tokens 0..{n - 1}, block diameters in fp64 numpy, "
                      f"{dt:.2f} s; tokens/s = tokens / ({w.bh} heads x time)"}
    print(json.dumps(out), flush=True)


def train_main(args):
    """Synthetic training step: masked-reconstruction loss through Q/K/V projections, the
    library's attention forward and tail VJP, and an output projection, then an SGD update, on one
    fixed seeded batch.  value = examples per second.  The roofline is that of the library's
    dominant kernel in the step (the fused Sinkhorn step, as for the attention op); the breakdown
    splits the step between the attention kernels and the rest (GEMMs, loss, update).  The
    oracle's step runs beside it on one example."""
    import torch
    from threadpoolctl import threadpool_limits

    from entropic_ot_attention_amd import binding as B
    from entropic_ot_attention_amd.training import ReconstructionModel, sgd_step
    from entropic_ot_attention_amd.workloads import TRAIN_WORKLOADS, make_training_batch

    w = TRAIN_WORKLOADS[args.train_workload]
    dev = torch.device("cuda:0")
    X, mask, weights = make_training_batch(w)
    Xd, md = X.to(dev), mask.to(dev)
    model = ReconstructionModel([x.to(dev) for x in weights], w.heads, w.W, w.T, w.R, w.eps,
                                w.torch_dtype)
    warm_up(lambda: sgd_step(model, Xd, md, w.lr), args.warmup)
    stream = torch.cuda.current_stream()
    losses = []
    step_ms, _, n_inst = timed_region(lambda i: losses.append(sgd_step(model, Xd, md, w.lr)[0]),
                                      args.steps, stream)
    kstep_ms, kstep_n = B.ska_timing_read(B.TIMED_STEP)
    kout_ms, _ = B.ska_timing_read(B.TIMED_OUT)
    kvjp_ms, _ = B.ska_timing_read(B.TIMED_VJP)
    B.ska_timing_enable(False)
    attn_ms = (kstep_ms + kout_ms + kvjp_ms) / n_inst     # per instrumented step
    bh, rows = w.batch * w.heads, w.L
    avg_launch_s = (kstep_ms / max(kstep_n, 1)) / 1e3
    elt = 2 if w.compute == "bf16" else 4
    alg_bytes = bh * rows * (2 * 64 * elt + STEP_VECTOR_BYTES_PER_TOKEN)
    hbm_gbs = alg_bytes / avg_launch_s / 1e9
    gemm_flops = 9 * 2 * w.batch * w.L * w.D * w.D     # 4 forward and 5 backward projections
    out = {
        "metric": f"synthetic reconstruction training step examples/s at batch {w.batch}, "
                  f"L={w.L}, D={w.D} ({w.heads} heads), W={w.W}",
        "value": round(w.batch / (step_ms / 1e3), 2),
        "unit": "examples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.compute == "bf16" else "f32",
        "data": "synthetic (seeded AR(1) embeddings, Bernoulli token mask)",
        "config": {"workload": w.name, "batch": w.batch, "L": w.L, "D": w.D, "heads": w.heads,
                   "W": w.W, "T": w.T, "R": w.R, "epsilon": w.eps, "masked": w.masked,
                   "lr": w.lr, "optimizer": "sgd"},
        "breakdown": {"attention_kernels_ms": round(attn_ms, 4),
                      "step_kernels_ms": round(kstep_ms / n_inst, 4),
                      "out_kernel_ms": round(kout_ms / n_inst, 4),
                      "vjp_kernels_ms": round(kvjp_ms / n_inst, 4),
                      "rest_ms": round(step_ms - attn_ms, 4),
                      "projection_gemm_tflops_if_rest": round(gemm_flops / max(step_ms - attn_ms, 1e-9) / 1e9, 1),
                      "loss_first": float(losses[0]), "loss_last": float(losses[-1])},
        "roofline": {
            "bound": "hbm",
            "kernel": "sinkhorn_step_kernel (fused balanced Sinkhorn step)",
            "achieved": round(hbm_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
            "traffic": None,
            "avg_launch_us": round(avg_launch_s * 1e6, 2),
            "launches_timed": kstep_n,
            "algorithmic_bytes": alg_bytes,
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        cfg = oracle.TrainConfig(heads=w.heads, W=w.W, T=w.T, R=w.R, eps=w.eps, lr=w.lr)
        params = tuple(x.double().numpy() for x in weights)
        nex = min(6, w.batch)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.reconstruction_step(params, X[:nex].double().numpy(), mask[:nex].double().numpy(),
                                       cfg)
            dt = time.perf_counter() - t0
        out["cpu_baseline"] = {
            "value": round(nex / dt, 4), "unit": "examples/s", "cores": 1, "kind": "oracle",
            "sample": f"examples 0..{nex - 1} of {w.batch} (all {w.heads} heads, L = {w.L}), one "
                      f"fp64 step (projections, attention forward and one-reference VJP, loss, "
                      f"SGD) in numpy, {dt:.2f} s"}
    print(json.dumps(out), flush=True)


def certificate_main(args):
    """A posteriori bias certificate on the GPU: for R = 0..r_max, eta_R of the workload's
    inputs in fp32 (each call runs the forward and VJP at (T, R) and full backpropagation, the
    adjoint at depth T + R, then the fixed-order norm reductions), the smallest R with
    eta_R <= tau, and the matrix-core roofline of full backpropagation at depth T + 2, its
    dominant part.  The oracle's certificate runs beside it on head 0."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from entropic_ot_attention_amd import binding as B
    from entropic_ot_attention_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    if w.dustbin:
        raise SystemExit("the certificate runs on the banded entry points (no dustbin workload)")
    w = w.with_(dtype="f32")               # remainders are resolved in fp32 only
    dev = torch.device("cuda:0")
    x = make_inputs(w)
    Q, K, V, dO = (x[k].to(dev) for k in ("Q", "K", "V", "dO"))
    L, rows = w.L, w.tokens
    stream = torch.cuda.current_stream()
    sums = torch.zeros(4, dtype=torch.float64, device=dev)
    per_r = {}
    selected = None
    for R in range(0, args.r_max + 1):
        if R == 0 and w.T == 0:
            continue
        prob = B.make_problem(w.bh, L, w.d, w.W, w.T, R, w.eps, torch.float32)
        ws = B.workspace_for(prob, B.SKA_OP_TAIL_REMAINDER, dev)
        for _ in range(args.warmup):
            B.sinkhorn_attn_tail_remainder(prob, Q, K, V, dO, sums, ws, stream)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(args.steps):
            B.sinkhorn_attn_tail_remainder(prob, Q, K, V, dO, sums, ws, stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / args.steps
        rq, fq, rk, fk = (float(v) for v in sums.cpu())
        eta = ((rq + rk) / (fq + fk)) ** 0.5 if fq + fk > 0 else 0.0
        per_r[R] = {"eta": eta, "ms": round(ms, 4)}
        if selected is None and eta <= args.tau:
            selected = R
        del ws

    # full backpropagation at depth T + 2 alone, timed call by call (two events around the calls:
    # per-launch events around each of its 2 (T + 2) + 2 passes would add their own GPU time)
    Rf = w.T + 2
    pf = B.make_problem(w.bh, L, w.d, w.W, 0, Rf, w.eps, torch.float32)
    wsf = B.workspace_for(pf, B.SKA_OP_VJP, dev)
    O = torch.empty_like(Q)
    duals = torch.empty(w.bh, B.n_duals(Rf), rows, dtype=torch.float32, device=dev)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
    B.sinkhorn_attn_fwd(pf, Q, K, V, O, duals, B.workspace_for(pf, B.SKA_OP_FWD, dev))
    for _ in range(args.warmup):
        B.sinkhorn_attn_vjp(pf, Q, K, V, duals, dO, dQ, dK, dV, B.SCHEDULES["one_reference"], wsf)
    torch.cuda.synchronize()
    evf = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    evf[0].record(stream)
    for _ in range(args.steps):
        B.sinkhorn_attn_vjp(pf, Q, K, V, duals, dO, dQ, dK, dV, B.SCHEDULES["one_reference"], wsf)
    evf[1].record(stream)
    torch.cuda.synchronize()
    nnz = band_entries(rows, min(w.W // 2, rows)) * w.bh
    vjp_s = evf[0].elapsed_time(evf[1]) / args.steps / 1e3
    flops = tail_pass_flops_per_entry(Rf, w.d) * nnz
    tflops = flops / vjp_s / 1e12
    roofline = {
        "bound": "mfma",
        "kernel": f"VJP passes of full backpropagation = the adjoint at depth T + 2 = {Rf} "
                  f"(whole VJP calls timed, small preparation kernels included)",
        "achieved": round(tflops, 2),
        "peak": MFMA_F32_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(tflops / MFMA_F32_PEAK_TFLOPS, 4),
        "traffic": None,
        "vjp_call_us": round(vjp_s * 1e6, 2),
        "calls_timed": args.steps,
        "algorithmic_flops": flops,
        "algorithmic_work": f"(18 + 2 x {Rf}) x {w.d} flops x {nnz} band entries per VJP",
    }
    out = {
        "metric": f"bias certificate eta_R tokens/s at L={L} W={w.W} d={w.d} T={w.T}, R=2; "
                  f"% of MFMA roofline of full backpropagation",
        "value": round(w.batch * L / (per_r[2]["ms"] / 1e3), 1) if 2 in per_r else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": per_r.get(2, {}).get("ms"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V/dO)",
        "config": {"workload": w.name + " (certified in fp32)", "batch": w.batch,
                   "heads": w.heads, "L": L, "d": w.d, "W": w.W, "T": w.T, "epsilon": w.eps,
                   "tau": args.tau},
        "certificate": {"eta": {str(R): v["eta"] for R, v in per_r.items()},
                        "ms": {str(R): v["ms"] for R, v in per_r.items()},
                        "selected_R": selected},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        import oracle
        n = min(args.cpu_sample_tokens or 32768, rows)
        Qh, Kh, Vh, dOh = (x[k][0, :n].double().numpy() for k in ("Q", "K", "V", "dO"))
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            ro = oracle.tail_remainder(Qh, Kh, Vh, dOh,
                                       oracle.BandProblem(W=w.W, T=w.T, R=2, eps=w.eps))
            dt = time.perf_counter() - t0
        g = B.tail_remainder(*(t[0:1, :n].contiguous() for t in (Q, K, V, dO)), w.W, w.T, 2, w.eps)
        out["cpu_baseline"] = {
            "value": round(n / (w.bh * dt), 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"head 0 of {w.bh}, tokens 0..{n - 1}, R = 2 certificate (forward, tail "
                      f"VJP and full backpropagation) in fp64 numpy, {dt:.2f} s; eta_2 oracle "
                      f"{ro['eta']:.6e}, GPU on the same sample {g['eta']:.6e}"}
    print(json.dumps(out), flush=True)


def _oracle_head_worker(job):
    """One head of the workload through the fp64 oracle (forward + one-reference VJP), in its
    own process, numpy single-threaded.  Returns (head, compute start, compute end, peak RSS MB);
    the inputs are drawn from the workload's seed before the clock starts."""
    import resource

    from threadpoolctl import threadpool_limits

    import oracle
    from entropic_ot_attention_amd.workloads import WORKLOADS, make_inputs

    name, R, head, n = job
    w = WORKLOADS[name].with_(R=R)
    x = make_inputs(w)
    Q, K, V, dO = (x[k][head, :n].float().double().numpy() for k in ("Q", "K", "V", "dO"))
    del x
    p = oracle.BandProblem(W=w.W, T=w.T, R=w.R, eps=w.eps)
    with threadpool_limits(limits=1):
        t0 = time.time()
        O, duals = oracle.forward(Q, K, V, p)
        if w.R == 2:
            oracle.vjp_one_reference(Q, K, V, dO, duals, p)
        else:
            oracle.vjp_tail_one_reference(Q, K, V, dO, duals, p)
        t1 = time.time()
    return head, t0, t1, resource.getrusage(resource.RUSAGE_SELF).ru_maxrss / 1024.0


def cpu_baseline(w, tokens_per_head=None):
    """fp64 oracle (as it stands) on the workload's own inputs: one process per (batch, head)
    problem, all running at once on the host's cores, each computing the forward and the
    one-reference VJP of its problem's first `tokens_per_head` tokens (default: all of them).
    tokens/s = tokens of the sequence per head / wall time from the first process's start to the
    last one's end.  Runs before the GPU is touched (its processes are started fresh)."""
    import multiprocessing as mp

    if w.dustbin:
        raise SystemExit("the CPU baseline runs on the banded workloads")
    n = min(tokens_per_head or w.tokens, w.tokens)
    avail = len(os.sched_getaffinity(0))
    procs = min(w.bh, avail)
    jobs = [(w.name, w.R, b, n) for b in range(w.bh)]
    ctx = mp.get_context("spawn")
    t0 = time.time()
    with ctx.Pool(processes=procs) as pool:
        res = pool.map(_oracle_head_worker, jobs, chunksize=1)
    total = time.time() - t0
    wall = max(r[2] for r in res) - min(r[1] for r in res)
    per_head = [r[2] - r[1] for r in res]
    whole = "all" if n == w.tokens else f"the first {n}"
    return {"value": round(w.batch * n / wall, 1), "unit": "tokens/s", "cores": procs,
            "kind": "oracle",
            "sample": f"{whole} tokens of each of the {w.bh} heads, one process per head "
                      f"({procs} at once), fwd + one-reference VJP in fp64 numpy (one thread "
                      f"each); wall {wall:.2f} s from the first start to the last end "
                      f"(per head {min(per_head):.2f}-{max(per_head):.2f} s); tokens/s = "
                      f"{n} tokens / wall",
            "wall_s": round(wall, 2), "wall_with_input_generation_s": round(total, 2),
            "host_cores_available": avail,
            "peak_rss_mb_per_process": round(max(r[3] for r in res), 1)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (every (batch, "
              "head) problem is independent, and sharding over them is a design note only). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.certificate:
        certificate_main(args)
        return
    if args.contraction:
        contraction_main(args)
        return
    if args.train:
        train_main(args)
        return

    from entropic_ot_attention_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    if args.tail_depth:
        w = w.with_(R=args.tail_depth)
    # the oracle's processes run first, before this process touches the GPU
    cpu = None
    if not args.no_cpu_baseline and not w.dustbin:
        cpu = cpu_baseline(w, args.cpu_sample_tokens)

    import torch

    from entropic_ot_attention_amd import binding as B

    dev = torch.device("cuda:0")
    x = make_inputs(w)
    Q, K, V, dO = (x[k].to(dev) for k in ("Q", "K", "V", "dO"))
    L = w.L
    rows = w.tokens
    prob = B.make_problem(w.bh, L, w.d, w.W, w.T, w.R, w.eps, w.torch_dtype)
    fwd_op = B.SKA_OP_DUSTBIN_BLOCK_FWD if w.dustbin else B.SKA_OP_FWD
    vjp_op = B.SKA_OP_DUSTBIN_BLOCK_VJP if w.dustbin else B.SKA_OP_VJP
    ws = B.workspace_for(prob, max(fwd_op, vjp_op), dev)
    ws_f = B.workspace_for(prob, fwd_op, dev)
    O = torch.empty_like(Q)
    duals = torch.empty(w.bh, B.n_duals(w.R), rows, dtype=torch.float32, device=dev)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
    sched = B.SCHEDULES[args.schedule]
    fwd = B.sinkhorn_attn_dustbin_block_fwd if w.dustbin else B.sinkhorn_attn_fwd
    vjp = B.sinkhorn_attn_dustbin_block_vjp if w.dustbin else B.sinkhorn_attn_vjp
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fwd(prob, Q, K, V, O, duals, ws_f)
        if ev is not None:
            ev[1].record(stream)
        # the VJP given the forward's output, as the autograd wrapper calls it
        vjp(prob, Q, K, V, duals, dO, dQ, dK, dV, sched, ws, O=O)
        if ev is not None:
            ev[2].record(stream)

    if args.calibration_copy_mib > 0:
        # one elementwise kernel that reads and writes exactly this many bytes; the source is
        # evicted from the last-level cache first (a fill of another buffer of the same size),
        # so every byte it reads comes from HBM
        n = args.calibration_copy_mib << 18
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        evict = torch.empty_like(src)
        evict.fill_(2.0)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst, evict

    warm_up(lambda: step(), args.warmup)

    # the timed region, with one event at every step boundary (for the median step)
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]

    def timed_step(i):
        bounds[i].record(stream)
        step()
        if i == args.steps - 1:
            bounds[args.steps].record(stream)

    step_ms, wall, n_inst = timed_region(timed_step, args.steps, stream)
    per_step = sorted(bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps))
    median_ms = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    kstep_ms, kstep_n = B.ska_timing_read(B.TIMED_STEP)
    kout_ms, kout_n = B.ska_timing_read(B.TIMED_OUT)
    kvjp_ms, kvjp_n = B.ska_timing_read(B.TIMED_VJP)
    B.ska_timing_enable(False)
    # forward / VJP split, after the timed region: the same steps with an event between the halves
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    vjp_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps

    tokens_per_step = w.batch * L
    value = tokens_per_step / (step_ms / 1e3)
    h = min(w.W // 2, rows) if not w.dustbin else rows
    nnz = band_entries(rows, h) * w.bh                         # band entries per launch
    avg_launch_s = (kstep_ms / max(kstep_n, 1)) / 1e3
    elt = 2 if w.dtype == "bf16" else 4
    fam = family_rooflines(w, rows, nnz, elt, args.schedule, avg_launch_s * 1e3,
                           kout_ms / max(kout_n, 1), kvjp_ms / n_inst, step_ms)
    traffic = traffic_per_launch(w.name)
    step_fam = fam["step"]
    valu_peak = VALU_LANE_OPS_PER_S / 1e12
    if w.dtype == "bf16":
        # The step's floors per launch: Q and K read once (the per-pass byte count of the method's
        # cost model) at 8 TB/s, its minimal VALU work (7 issue slots per band entry) at the fp32
        # vector peak, and its matrix-core flops at the bf16 peak.  The HBM floor is the highest,
        # so the line reports "hbm".  Beside it: the VALU and MFMA fractions, the SIMD issue floor
        # (products and vector instructions add on a SIMD), and the SQ counters' busy fractions,
        # which name the VALU as the busiest unit in practice.
        simd_cycles = nnz * (2 * BF16_MFMA_CYCLES / 256 + SLOTS_PER_ENTRY_STEP * VALU_SLOT_CYCLES / 64)
        simd_floor_s = simd_cycles / (N_SIMD * CLOCK_HZ)
        roofline = {
            "bound": "hbm",
            "kernel": "sinkhorn_step_kernel (fused balanced Sinkhorn step)",
            "achieved": step_fam["hbm_GB_per_s"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": step_fam["hbm_frac"],
            "traffic": traffic,
            "avg_launch_us": round(avg_launch_s * 1e6, 2),
            "launches_timed": kstep_n,
            "algorithmic_work": f"{w.bh * rows} token rows x 2 x {w.d} x {elt} B (Q and K read "
                                f"once) = {step_fam['bytes']} B per launch",
            "valu": {"achieved": step_fam["valu_T_per_s"], "peak": round(valu_peak, 3),
                     "unit": "T VALU lane-slots/s", "frac": step_fam["valu_frac"],
                     "work": f"{SLOTS_PER_ENTRY_STEP} issue slots (fma, exp = {EXP_SLOTS}, add, "
                             f"fma) x {nnz} band entries per launch"},
            "simd_issue": {"floor_us": round(simd_floor_s * 1e6, 2),
                           "frac": round(simd_floor_s / avg_launch_s, 4),
                           "work": f"per band entry {2 * BF16_MFMA_CYCLES}/256 product cycles + "
                                   f"{SLOTS_PER_ENTRY_STEP} x {VALU_SLOT_CYCLES}/64 VALU cycles, "
                                   f"over {N_SIMD} SIMDs at {CLOCK_HZ / 1e9:g} GHz"},
            "hbm_with_vectors": {
                "achieved": round(step_fam["bytes_with_vectors"] / avg_launch_s / 1e9, 1),
                "frac": round(step_fam["bytes_with_vectors"] / avg_launch_s / 1e9 / HBM_PEAK_GBS, 4),
                "algorithmic_bytes": step_fam["bytes_with_vectors"],
                "work": f"plus {STEP_VECTOR_BYTES_PER_TOKEN} B of O(L) fp32 vectors per token"},
            "mfma": {"achieved": step_fam["mfma_TFLOP_per_s"], "peak": step_fam["mfma_peak"],
                     "unit": "TFLOP/s", "frac": step_fam["mfma_frac"]},
            "binding_unit_counters": step_counters(w.name),
            "families": fam,
        }
        if traffic is not None:
            roofline["traffic_gbs"] = round(traffic / avg_launch_s / 1e9, 1)
    else:
        # fp32 workloads: the fp32 matrix cores bind (every pass recomputes its scores at 157 TF)
        roofline = {
            "bound": "mfma",
            "kernel": "Sinkhorn step kernel (fused balanced Sinkhorn step)",
            "achieved": step_fam["mfma_TFLOP_per_s"],
            "peak": step_fam["mfma_peak"],
            "unit": "TFLOP/s",
            "frac": step_fam["mfma_frac"],
            "traffic": traffic,
            "avg_launch_us": round(avg_launch_s * 1e6, 2),
            "launches_timed": kstep_n,
            "algorithmic_work": f"2 x {w.d} flops x {nnz} band entries per launch",
            "families": fam,
        }
    out = {
        "metric": f"fwd+R={w.R} VJP tokens/s at L={L} W={w.W} d={w.d}; % of MFMA/HBM roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "median_ms_per_step": round(median_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V/dO)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "L": L, "d": w.d,
                   "W": w.W, "T": w.T, "R": w.R, "epsilon": w.eps, "schedule": args.schedule},
        "breakdown": {"fwd_ms": round(fwd_ms, 4), "vjp_ms": round(vjp_ms, 4),
                      "wall_s": round(wall, 3),
                      "step_kernels_ms": round(kstep_ms / n_inst, 4),
                      "out_kernel_ms": round(kout_ms / n_inst, 4),
                      "vjp_kernels_ms": round(kvjp_ms / n_inst, 4),
                      "instrumented_steps": n_inst},
        "roofline": roofline,
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
