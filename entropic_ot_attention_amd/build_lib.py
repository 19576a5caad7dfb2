"""Compile libsinkhorn_attn.so for gfx950 with hipcc (in-tree, into entropic_ot_attention_amd/_lib).

Each source is compiled to its own object in parallel (no relocatable device code: every kernel
is launched from the translation unit that defines it), then the objects are linked."""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libsinkhorn_attn.so")
OBJ_DIR = os.path.join(LIB_DIR, "obj")
PROBE_PATH = os.path.join(LIB_DIR, "issue_probe")
SOURCES = ["ska_kernels.hip", "ska_fused.hip", "ska_vjp_stream.hip", "ska_wide.hip",
           "ska_contraction.hip", "ska_noalloc.hip", "ska_geometry.cpp",
           "ska_capi.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep hipcc from forming packed fp32 instructions (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs (no copies out of the accumulation registers)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]
# per-source additions: the streaming VJP passes and the wide engine schedule for instruction-level
# parallelism (their dK/dV pass and wide passes ran 1-6% faster with it); the fused step keeps the
# default scheduler, under which it ran 2% faster
SOURCE_FLAGS = {
    "ska_vjp_stream.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "ska_wide.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    return r.returncode, err


def compile_cmd(src: str, obj: str) -> list:
    return [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-I", os.path.join(ROOT, "include"),
            "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    if jobs is None:
        jobs = min(len(SOURCES), max(1, len(os.sched_getaffinity(0))), 16)
    objs = [os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [compile_cmd(s, o) for s, o in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for src, (rc, err) in zip(SOURCES, results):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    rc, err = _run(link)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB_PATH)
    # the issue-cost probe behind the VALU and issue rooflines (a standalone program)
    probe = [hipcc(), *HIPCC_FLAGS, os.path.join(CSRC, "issue_probe.hip"), "-o", PROBE_PATH]
    if verbose:
        print(" ".join(probe), flush=True)
    rc, err = _run(probe)
    if rc != 0:
        raise RuntimeError(f"hipcc failed on issue_probe.hip ({rc}):\n{err}")
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
