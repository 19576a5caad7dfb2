"""ctypes binding of libsinkhorn_attn.so (argument marshalling only).

Every computation runs in the HIP library; this module checks tensor shapes, dtypes
and devices, allocates outputs and workspaces with torch when asked, and passes raw
device pointers and torch's current HIP stream to the C entry points, which keep the
names of include/sinkhorn_attn.h.  Importing it raises if the library is not built.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libsinkhorn_attn.so")

SKA_F32, SKA_BF16 = 0, 1
SKA_ONE_REFERENCE, SKA_DIRECT_FOUR = 0, 1
SKA_OP_FWD, SKA_OP_VJP, SKA_OP_DUSTBIN_BLOCK_FWD, SKA_OP_DUSTBIN_BLOCK_VJP = 0, 1, 2, 3
SKA_OP_TAIL_REMAINDER = 4
SKA_OP_CONTRACTION, SKA_OP_DUSTBIN_BLOCK_CONTRACTION = 5, 6
SKA_OK = 0
TIMED_STEP, TIMED_OUT, TIMED_VJP, TIMED_CERT = 0, 1, 2, 3

SCHEDULES = {"one_reference": SKA_ONE_REFERENCE, "direct_four": SKA_DIRECT_FOUR}

# every entry point the header declares
EXPORTS = (
    "ska_workspace_bytes", "sinkhorn_attn_fwd", "sinkhorn_attn_fwd_noalloc", "sinkhorn_attn_vjp",
    "sinkhorn_attn_dustbin_block_fwd", "sinkhorn_attn_dustbin_block_vjp",
    "sinkhorn_attn_tail_remainder", "ska_contraction_layout",
    "sinkhorn_attn_contraction_certificate", "sinkhorn_attn_dustbin_block_contraction_certificate",
    "ska_status_string", "ska_last_error", "ska_timing_enable", "ska_timing_read",
)


class SkaProblem(ctypes.Structure):
    _fields_ = [("bh", ctypes.c_int64), ("L", ctypes.c_int64), ("d", ctypes.c_int64),
                ("W", ctypes.c_int64), ("T", ctypes.c_int32), ("R", ctypes.c_int32),
                ("epsilon", ctypes.c_float), ("dtype", ctypes.c_int32)]


class SinkhornAttnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(SkaProblem)
    vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.ska_workspace_bytes.argtypes = [P, st, ctypes.POINTER(sz)]
    lib.sinkhorn_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sinkhorn_attn_dustbin_block_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sinkhorn_attn_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.sinkhorn_attn_vjp.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, st, vp, sz, vp]
    lib.sinkhorn_attn_dustbin_block_vjp.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, st, vp, sz,
                                                    vp]
    lib.sinkhorn_attn_tail_remainder.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    i32 = ctypes.c_int32
    lib.ska_contraction_layout.argtypes = [P, st, i32, ctypes.POINTER(ctypes.c_int64),
                                           ctypes.POINTER(i32)]
    lib.sinkhorn_attn_contraction_certificate.argtypes = [P, i32, vp, vp, vp, vp, vp, vp]
    lib.sinkhorn_attn_dustbin_block_contraction_certificate.argtypes = [P, i32, vp, vp, vp, vp, vp, vp]
    for name in ("ska_workspace_bytes", "sinkhorn_attn_fwd", "sinkhorn_attn_fwd_noalloc",
                 "sinkhorn_attn_dustbin_block_fwd",
                 "sinkhorn_attn_vjp", "sinkhorn_attn_dustbin_block_vjp",
                 "sinkhorn_attn_tail_remainder", "ska_contraction_layout",
                 "sinkhorn_attn_contraction_certificate",
                 "sinkhorn_attn_dustbin_block_contraction_certificate",
                 "ska_timing_enable", "ska_timing_read"):
        getattr(lib, name).restype = ctypes.c_int
    lib.ska_status_string.argtypes = [ctypes.c_int]
    lib.ska_status_string.restype = ctypes.c_char_p
    lib.ska_last_error.argtypes = []
    lib.ska_last_error.restype = ctypes.c_char_p
    lib.ska_timing_enable.argtypes = [ctypes.c_int]
    lib.ska_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64)]
    return lib


lib = _load()


def _check(status: int, where: str):
    if status != SKA_OK:
        raise SinkhornAttnError(status, where, lib.ska_last_error().decode() or
                                lib.ska_status_string(status).decode())


def ska_status_string(status: int) -> str:
    return lib.ska_status_string(status).decode()


def ska_last_error() -> str:
    return lib.ska_last_error().decode()


def make_problem(bh: int, L: int, d: int, W: int, T: int, R: int, epsilon: float,
                 dtype: torch.dtype) -> SkaProblem:
    code = {torch.float32: SKA_F32, torch.bfloat16: SKA_BF16}.get(dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {dtype}")
    return SkaProblem(bh, L, d, W, T, R, float(epsilon), code)


def ska_workspace_bytes(problem: SkaProblem, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.ska_workspace_bytes(ctypes.byref(problem), op, ctypes.byref(n)), "ska_workspace_bytes")
    return n.value


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: torch.Tensor | None, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _ws(workspace: torch.Tensor | None):
    if workspace is None:
        return None, 0
    return _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()


def sinkhorn_attn_fwd(problem, Q, K, V, O, duals, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check(lib.sinkhorn_attn_fwd(ctypes.byref(problem), _ptr(Q, "Q"), _ptr(K, "K"), _ptr(V, "V"),
                                 _ptr(O, "O"), _ptr(duals, "duals"), ws, nb, _stream(stream)),
           "sinkhorn_attn_fwd")


def sinkhorn_attn_fwd_noalloc(problem, Q, K, V, O, duals, stream=None):
    _check(lib.sinkhorn_attn_fwd_noalloc(ctypes.byref(problem), _ptr(Q, "Q"), _ptr(K, "K"),
                                         _ptr(V, "V"), _ptr(O, "O"), _ptr(duals, "duals"),
                                         _stream(stream)),
           "sinkhorn_attn_fwd_noalloc")


def sinkhorn_attn_dustbin_block_fwd(problem, Q, K, V, O, duals, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check(lib.sinkhorn_attn_dustbin_block_fwd(ctypes.byref(problem), _ptr(Q, "Q"), _ptr(K, "K"),
                                               _ptr(V, "V"), _ptr(O, "O"), _ptr(duals, "duals"),
                                               ws, nb, _stream(stream)),
           "sinkhorn_attn_dustbin_block_fwd")


def sinkhorn_attn_vjp(problem, Q, K, V, duals, dO, dQ, dK, dV, schedule, workspace, stream=None,
                      O=None):
    """O (optional): the forward's output for the same inputs and duals."""
    ws, nb = _ws(workspace)
    _check(lib.sinkhorn_attn_vjp(ctypes.byref(problem), _ptr(Q, "Q"), _ptr(K, "K"), _ptr(V, "V"),
                                 _ptr(duals, "duals"), _ptr(dO, "dO"), _ptr(O, "O"), _ptr(dQ, "dQ"),
                                 _ptr(dK, "dK"), _ptr(dV, "dV"), schedule, ws, nb, _stream(stream)),
           "sinkhorn_attn_vjp")


def sinkhorn_attn_dustbin_block_vjp(problem, Q, K, V, duals, dO, dQ, dK, dV, schedule, workspace,
                                    stream=None, O=None):
    """O (optional): the forward's output for the same inputs and duals."""
    ws, nb = _ws(workspace)
    _check(lib.sinkhorn_attn_dustbin_block_vjp(ctypes.byref(problem), _ptr(Q, "Q"), _ptr(K, "K"),
                                               _ptr(V, "V"), _ptr(duals, "duals"), _ptr(dO, "dO"),
                                               _ptr(O, "O"), _ptr(dQ, "dQ"), _ptr(dK, "dK"),
                                               _ptr(dV, "dV"), schedule, ws, nb, _stream(stream)),
           "sinkhorn_attn_dustbin_block_vjp")


def sinkhorn_attn_tail_remainder(problem, Q, K, V, dO, sums, workspace, stream=None):
    ws, nb = _ws(workspace)
    _check(lib.sinkhorn_attn_tail_remainder(ctypes.byref(problem), _ptr(Q, "Q"), _ptr(K, "K"),
                                            _ptr(V, "V"), _ptr(dO, "dO"), _ptr(sums, "sums"),
                                            ws, nb, _stream(stream)),
           "sinkhorn_attn_tail_remainder")


def ska_contraction_layout(problem, op: int, block: int):
    """(nb, m) of the contraction certificate's [bh][nb][2 m + 1] outputs."""
    nb = ctypes.c_int64(0)
    m = ctypes.c_int32(0)
    _check(lib.ska_contraction_layout(ctypes.byref(problem), op, block, ctypes.byref(nb),
                                      ctypes.byref(m)), "ska_contraction_layout")
    return nb.value, m.value


def sinkhorn_attn_contraction_certificate(problem, block, Q, K, delta, kappa=None, delta_max=None,
                                          stream=None):
    _check(lib.sinkhorn_attn_contraction_certificate(
        ctypes.byref(problem), block, _ptr(Q, "Q"), _ptr(K, "K"), _ptr(delta, "delta"),
        _ptr(kappa, "kappa"), _ptr(delta_max, "delta_max"), _stream(stream)),
        "sinkhorn_attn_contraction_certificate")


def sinkhorn_attn_dustbin_block_contraction_certificate(problem, block, Q, K, delta, kappa=None,
                                                        delta_max=None, stream=None):
    _check(lib.sinkhorn_attn_dustbin_block_contraction_certificate(
        ctypes.byref(problem), block, _ptr(Q, "Q"), _ptr(K, "K"), _ptr(delta, "delta"),
        _ptr(kappa, "kappa"), _ptr(delta_max, "delta_max"), _stream(stream)),
        "sinkhorn_attn_dustbin_block_contraction_certificate")


def ska_timing_enable(on: bool):
    _check(lib.ska_timing_enable(1 if on else 0), "ska_timing_enable")


def ska_timing_read(kernel: int):
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(lib.ska_timing_read(kernel, ctypes.byref(ms), ctypes.byref(n)), "ska_timing_read")
    return ms.value, n.value


# ------------------------------------------------------------------------------------------
# allocation conveniences (torch allocates; the library computes)
# ------------------------------------------------------------------------------------------

def _shape_check(Q, K, V, dustbin):
    if Q.dim() != 3 or Q.shape != K.shape or Q.shape != V.shape:
        raise ValueError("Q, K, V must share the shape [bh, tokens, d]")
    if Q.dtype != K.dtype or Q.dtype != V.dtype:
        raise ValueError("Q, K, V must share one dtype")
    bh, rows, d = Q.shape
    L = rows - 1 if dustbin else rows
    if L < 0:
        raise ValueError("dustbin inputs need the dustbin row")
    return bh, rows, d, L


def workspace_for(problem: SkaProblem, op: int, device) -> torch.Tensor:
    nb = ska_workspace_bytes(problem, op)
    return torch.empty(max(nb, 16), dtype=torch.uint8, device=device)


def n_duals(R: int) -> int:
    """Saved dual rows per problem: v0, u1, v1, .., uR, vR (2R + 1), or u0, v0 when R = 0."""
    return 2 if R == 0 else 2 * R + 1


def forward(Q, K, V, W: int, T: int, R: int = 2, epsilon: float = 1.0, dustbin: bool = False,
            workspace: torch.Tensor | None = None, stream=None):
    """O and duals [bh, n_duals(R), tokens] (fp32, natural-log units)."""
    bh, rows, d, L = _shape_check(Q, K, V, dustbin)
    prob = make_problem(bh, L, d, W, T, R, epsilon, Q.dtype)
    op = SKA_OP_DUSTBIN_BLOCK_FWD if dustbin else SKA_OP_FWD
    if workspace is None:
        workspace = workspace_for(prob, op, Q.device)
    O = torch.empty_like(Q)
    duals = torch.empty(bh, n_duals(R), rows, dtype=torch.float32, device=Q.device)
    fn = sinkhorn_attn_dustbin_block_fwd if dustbin else sinkhorn_attn_fwd
    fn(prob, Q, K, V, O, duals, workspace, stream)
    return O, duals


def vjp(Q, K, V, duals, dO, W: int, T: int, R: int = 2, epsilon: float = 1.0,
        schedule: str = "one_reference", dustbin: bool = False,
        workspace: torch.Tensor | None = None, stream=None, O: torch.Tensor | None = None):
    """dQ, dK, dV for cotangent dO given the forward's duals (and optionally its output O, from
    which the R = 2 passes take the row cotangent sums)."""
    bh, rows, d, L = _shape_check(Q, K, V, dustbin)
    if dO.shape != Q.shape or dO.dtype != Q.dtype:
        raise ValueError("dO must match Q in shape and dtype")
    if O is not None and (O.shape != Q.shape or O.dtype != Q.dtype):
        raise ValueError("O must match Q in shape and dtype")
    if duals.shape != (bh, n_duals(R), rows) or duals.dtype != torch.float32:
        raise ValueError("duals must be fp32 [bh, n_duals(R), tokens]")
    prob = make_problem(bh, L, d, W, T, R, epsilon, Q.dtype)
    op = SKA_OP_DUSTBIN_BLOCK_VJP if dustbin else SKA_OP_VJP
    if workspace is None:
        workspace = workspace_for(prob, op, Q.device)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
    fn = sinkhorn_attn_dustbin_block_vjp if dustbin else sinkhorn_attn_vjp
    fn(prob, Q, K, V, duals, dO, dQ, dK, dV, SCHEDULES[schedule], workspace, stream, O=O)
    return dQ, dK, dV


def tail_remainder(Q, K, V, dO, W: int, T: int, R: int = 2, epsilon: float = 1.0,
                   workspace: torch.Tensor | None = None, stream=None) -> dict:
    """A posteriori bias certificate: squared norms of the gradient remainder dropped by the
    stopped base at tail depth R and of the full (all T + R steps) gradient, summed over all
    problems, as computed by sinkhorn_attn_tail_remainder; eta_R is their relative l2 ratio
    over dQ and dK."""
    bh, rows, d, L = _shape_check(Q, K, V, False)
    if dO.shape != Q.shape or dO.dtype != Q.dtype:
        raise ValueError("dO must match Q in shape and dtype")
    prob = make_problem(bh, L, d, W, T, R, epsilon, Q.dtype)
    if workspace is None:
        workspace = workspace_for(prob, SKA_OP_TAIL_REMAINDER, Q.device)
    sums = torch.zeros(4, dtype=torch.float64, device=Q.device)
    sinkhorn_attn_tail_remainder(prob, Q, K, V, dO, sums, workspace, stream)
    rq, fq, rk, fk = (float(x) for x in sums.cpu())
    return {"rem_dQ2": rq, "full_dQ2": fq, "rem_dK2": rk, "full_dK2": fk,
            "eta": ((rq + rk) / (fq + fk)) ** 0.5 if fq + fk > 0 else 0.0}


def select_tail_depth(Q, K, V, dO, W: int, T: int, epsilon: float = 1.0, tau: float = 1e-5,
                      R_max: int = 4, R_min: int = 0) -> tuple:
    """The smallest tail depth R in R_min..R_max whose certified remainder eta_R is at most tau
    (None if none is), and every eta_R computed on the way."""
    etas = {}
    for R in range(R_min, R_max + 1):
        etas[R] = tail_remainder(Q, K, V, dO, W, T, R, epsilon)["eta"]
        if etas[R] <= tau:
            return R, etas
    return None, etas


def contraction_certificate(Q, K, W: int, epsilon: float = 1.0, block: int = 16,
                            dustbin: bool = False, stream=None):
    """Projective diameters Delta and Birkhoff-Hopf coefficients kappa of every active block pair,
    fp32 [bh, nb, 2 m + 1] (-1 where a block pair is not active), and the largest Delta per
    problem [bh].  Q, K: [bh, tokens, d] (dustbin: the dustbin token as the last row)."""
    if Q.dim() != 3 or Q.shape != K.shape or Q.dtype != K.dtype:
        raise ValueError("Q and K must share one shape [bh, tokens, d] and dtype")
    bh, rows, d = Q.shape
    L = rows - 1 if dustbin else rows
    if L < 0:
        raise ValueError("dustbin inputs need the dustbin row")
    prob = make_problem(bh, L, d, W, 1, 2, epsilon, Q.dtype)      # T and R do not enter
    op = SKA_OP_DUSTBIN_BLOCK_CONTRACTION if dustbin else SKA_OP_CONTRACTION
    nb, m = ska_contraction_layout(prob, op, block)
    delta = torch.empty(bh, nb, 2 * m + 1, dtype=torch.float32, device=Q.device)
    kappa = torch.empty_like(delta)
    delta_max = torch.empty(bh, dtype=torch.float32, device=Q.device)
    fn = (sinkhorn_attn_dustbin_block_contraction_certificate if dustbin
          else sinkhorn_attn_contraction_certificate)
    fn(prob, block, Q, K, delta, kappa, delta_max, stream)
    return delta, kappa, delta_max
