"""Host-only checks of the C ABI (no GPU needed): the library loads, exports every entry
point include/sinkhorn_attn.h declares, the ctypes struct matches the C layout, and
argument errors come back as status codes before anything is enqueued."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from entropic_ot_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkhorn_attn.h")

FAKE = 0x10000  # 16-byte aligned non-null address; never dereferenced on error paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s+(\w+)\s*\(", text, flags=re.M))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"sinkhorn_attn_fwd", "sinkhorn_attn_vjp", "sinkhorn_attn_dustbin_block_fwd",
            "sinkhorn_attn_dustbin_block_vjp"} <= names
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = names - exported
    assert not missing, f"declared but not exported: {missing}"
    assert names == set(B.EXPORTS)


def test_problem_struct_layout_matches_c():
    src = r"""
    #include <stddef.h>
    #include <stdio.h>
    #include "sinkhorn_attn.h"
    int main(void) {
      printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(ska_problem),
             offsetof(ska_problem, bh), offsetof(ska_problem, L), offsetof(ska_problem, d),
             offsetof(ska_problem, W), offsetof(ska_problem, T), offsetof(ska_problem, R),
             offsetof(ska_problem, epsilon), offsetof(ska_problem, dtype));
      return 0;
    }
    """
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", c, "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                              check=True).stdout.split()]
    P = B.SkaProblem
    want = [ctypes.sizeof(P)] + [getattr(P, f).offset for f, _ in P._fields_]
    assert got == want


def _prob(**kw):
    base = dict(bh=2, L=100, d=64, W=16, T=3, R=2, epsilon=1.0, dtype=B.SKA_F32)
    base.update(kw)
    return B.SkaProblem(**base)


def _ws_bytes(prob, op):
    n = ctypes.c_size_t(0)
    st = B.lib.ska_workspace_bytes(ctypes.byref(prob), op, ctypes.byref(n))
    return st, n.value


def _fused_fwd_bytes(bh, L, W):
    """Forward workspace of the register-resident path: 4 dual vectors [bh][Lpad] and two
    column-partial buffers [bh][nseg][64 seg_len + 32 H16]; segments of seg_len 64-row blocks
    sized for about 768 workgroups, at least H16 / 2 blocks (H16 = even halo tile count)."""
    Lpad = -(-L // 64) * 64
    h = min(W // 2, L)
    h16 = -(-h // 16)
    H16 = next(c for c in (2, 4, 8, 12) if h16 <= c)
    nblk = -(-L // 64)
    sl = min(max(-(-bh * nblk // 768), (H16 + 1) // 2, 1), nblk)
    nseg = -(-nblk // sl)
    pst = 64 * sl + 32 * H16
    return (4 * bh * Lpad + 2 * bh * nseg * pst) * 4


def _wide_fwd_bytes(bh, Lr, h, fp32=True):
    """Forward workspace of bands wider than the register-resident step: 2 dual vectors
    [bh][Lpad] plus, while a row tile's window (at most min(ceil(Lr / 16), (2 h + 15) // 16 + 2)
    tiles) fits 8 waves x 33 register tiles, one partial row of 16 x window floats per 16-token
    row tile, rounded up to 64 floats, and for fp32 Q and K as three bf16 planes (192 bf16 = 96
    floats per row each); wider windows (split half-steps) need only the duals."""
    Lpad = -(-Lr // 64) * 64
    ntw = min(-(-Lr // 16), (2 * h + 15) // 16 + 2)
    part = bh * -(-Lr // 16) * 16 * ntw if -(-ntw // 8) <= 33 else 0
    part = -(-part // 64) * 64
    planes = 2 * bh * Lr * 96 if part and fp32 else 0
    return (2 * bh * Lpad + part + planes) * 4


def _vjp_bytes(bh, L, W, bf16=False):
    """VJP workspace: 14 vectors [bh][Lpad], plus dv1 column partials [bh][nseg][pstride] when
    the streaming passes cover the band (bf16: h <= 128 with 8-wave / 128-token blocks; fp32:
    h <= 64 with 4-wave / 64-token blocks)."""
    Lpad = -(-L // 64) * 64
    base = 14 * bh * Lpad
    h = min(W // 2, L)
    h16 = -(-h // 16)
    H16 = next((c for c in (2, 4, 8) if h16 <= c), 0)   # 0: chunked passes, no partials
    if H16 == 0 or (not bf16 and H16 > 4):
        return base * 4
    nw = 8 if bf16 else 4
    br = 16 * nw
    nblk = -(-L // br)
    sl = min(max(-(-bh * nblk // 256), -(-(32 * H16) // br), 1), nblk)
    nseg = -(-nblk // sl)
    return (base + bh * nseg * (br * sl + 32 * H16)) * 4


def test_workspace_sizes():
    for L, Lpad in ((1, 64), (64, 64), (65, 128), (1000, 1024)):
        st, n = _ws_bytes(_prob(L=L, bh=3), B.SKA_OP_FWD)
        assert st == 0 and n == _fused_fwd_bytes(3, L, 16)
        st, n = _ws_bytes(_prob(L=L, bh=3), B.SKA_OP_VJP)
        assert st == 0 and n == _vjp_bytes(3, L, 16)
        st, n = _ws_bytes(_prob(L=L, bh=3, W=500), B.SKA_OP_VJP)     # h = min(W/2, L)
        assert st == 0 and n == _vjp_bytes(3, L, 500)
    st, n = _ws_bytes(_prob(L=262144, bh=4, W=256, dtype=B.SKA_BF16), B.SKA_OP_VJP)
    assert st == 0 and n == _vjp_bytes(4, 262144, 256, bf16=True)
    assert n < 20 * 4 * 262144 * 4          # O(L): under 20 floats per token and head
    st, n = _ws_bytes(_prob(L=262144, bh=4, W=256), B.SKA_OP_FWD)
    assert st == 0 and n == _fused_fwd_bytes(4, 262144, 256)
    assert n < 8 * 4 * 262144 * 4           # O(L): under 8 floats per token and head
    # wider bands: the wide step's per-row-tile column partials, or only the duals once the
    # window outgrows the registers
    st, n = _ws_bytes(_prob(L=2000, bh=2, W=1000), B.SKA_OP_FWD)
    assert st == 0 and n == _wide_fwd_bytes(2, 2000, 500) == (2 * 2 * 2048 + 260032 + 2 * 2 * 2000 * 96) * 4
    st, n = _ws_bytes(_prob(L=2000, bh=2, W=1000, dtype=B.SKA_BF16), B.SKA_OP_FWD)
    assert st == 0 and n == _wide_fwd_bytes(2, 2000, 500, fp32=False) == (2 * 2 * 2048 + 260032) * 4
    st, n = _ws_bytes(_prob(L=4096, bh=4), B.SKA_OP_DUSTBIN_BLOCK_FWD)   # 4097 rows, dense
    assert st == 0 and n == _wide_fwd_bytes(4, 4097, 4096) == (2 * 4 * 4160 + 4 * 257 * 16 * 257 + 2 * 4 * 4097 * 96) * 4
    st, n = _ws_bytes(_prob(L=10000, bh=2, W=20000), B.SKA_OP_FWD)      # 625-tile windows
    assert st == 0 and n == _wide_fwd_bytes(2, 10000, 10000) == 2 * 2 * 10048 * 4
    st, n = _ws_bytes(_prob(L=0), B.SKA_OP_VJP)
    assert st == 0 and n == 0
    # bands the streaming passes do not cover need only the vectors, whatever the dtype
    assert (_ws_bytes(_prob(L=2000, W=4000), B.SKA_OP_VJP)
            == _ws_bytes(_prob(L=2000, W=4000, dtype=B.SKA_BF16), B.SKA_OP_VJP))


@pytest.mark.parametrize("kw,op,status", [
    (dict(d=32), B.SKA_OP_FWD, -2),
    (dict(d=128), B.SKA_OP_VJP, -2),
    (dict(W=7), B.SKA_OP_FWD, -1),
    (dict(W=-2), B.SKA_OP_FWD, -1),
    (dict(T=-1), B.SKA_OP_FWD, -1),
    (dict(R=-1), B.SKA_OP_FWD, -1),
    (dict(R=0, T=0), B.SKA_OP_FWD, -1),
    (dict(R=0, T=0), B.SKA_OP_TAIL_REMAINDER, -1),
    (dict(R=300), B.SKA_OP_VJP, -2),
    (dict(R=257), B.SKA_OP_DUSTBIN_BLOCK_VJP, -2),
    (dict(epsilon=0.0), B.SKA_OP_FWD, -1),
    (dict(epsilon=float("nan")), B.SKA_OP_VJP, -1),
    (dict(dtype=7), B.SKA_OP_FWD, -1),
    (dict(bh=-1), B.SKA_OP_FWD, -1),
    (dict(bh=70000), B.SKA_OP_FWD, -2),
    (dict(L=-1), B.SKA_OP_FWD, -1),
    (dict(L=(1 << 30) + 1), B.SKA_OP_FWD, -2),
    (dict(L=1 << 30), B.SKA_OP_DUSTBIN_BLOCK_FWD, -2),     # L + 1 tokens with the dustbin
    (dict(T=250, R=7), B.SKA_OP_TAIL_REMAINDER, -2),        # adjoint depth T + R > 256
    (dict(epsilon=float("inf")), B.SKA_OP_FWD, -1),
    (dict(W=-1), B.SKA_OP_VJP, -1),
])
def test_invalid_problems_are_rejected(kw, op, status):
    st, _ = _ws_bytes(_prob(**kw), op)
    assert st == status
    assert B.ska_last_error() != ""


def test_entry_points_reject_bad_arguments_before_launch():
    prob = _prob()
    _, need = _ws_bytes(prob, B.SKA_OP_FWD)
    V = ctypes.c_void_p
    f = B.lib.sinkhorn_attn_fwd
    # NULL problem
    assert f(None, V(FAKE), V(FAKE), V(FAKE), V(FAKE), V(FAKE), V(FAKE), need, None) == -1
    # NULL and misaligned tensors
    assert f(ctypes.byref(prob), None, V(FAKE), V(FAKE), V(FAKE), V(FAKE), V(FAKE), need, None) == -1
    assert f(ctypes.byref(prob), V(FAKE + 4), V(FAKE), V(FAKE), V(FAKE), V(FAKE), V(FAKE), need, None) == -1
    assert "aligned" in B.ska_last_error()
    # workspace missing or short
    assert f(ctypes.byref(prob), V(FAKE), V(FAKE), V(FAKE), V(FAKE), V(FAKE), None, need, None) == -3
    assert f(ctypes.byref(prob), V(FAKE), V(FAKE), V(FAKE), V(FAKE), V(FAKE), V(FAKE), need - 4, None) == -3
    g = B.lib.sinkhorn_attn_vjp
    _, needv = _ws_bytes(prob, B.SKA_OP_VJP)
    args = [V(FAKE)] * 9
    assert g(ctypes.byref(prob), *args, 5, V(FAKE), needv, None) == -1      # unknown schedule
    prob3 = _prob(R=3)
    _, need3 = _ws_bytes(prob3, B.SKA_OP_VJP)
    assert g(ctypes.byref(prob3), *args, 1, V(FAKE), need3, None) == -2     # direct-four needs R = 2
    assert "R == 2" in B.ska_last_error()
    assert g(ctypes.byref(prob), *args, 0, V(FAKE), needv - 1, None) == -3
    assert g(ctypes.byref(prob), *(args[:6] + [None] + args[7:]), 0, V(FAKE), needv, None) == -1
    # O (optional) may be NULL, but not misaligned
    assert g(ctypes.byref(prob), *(args[:5] + [V(FAKE + 4)] + args[6:]), 0, V(FAKE), needv,
             None) == -1
    assert "O is not 16-byte aligned" in B.ska_last_error()


def _stream_partials(bh, L, nw, nt):
    """Floats of one column-partial buffer of the streaming passes: nseg segments of seg_len
    blocks of 16 nw tokens per problem, each segment row 16 nw seg_len + 16 (nt - 1) long, with
    about one workgroup per compute unit (256) and a segment spanning at least twice the halo."""
    br = 16 * nw
    nblk = -(-L // br)
    seg_len = max(-(-(bh * nblk) // 256), -(-(16 * (nt - 1)) // br), 1)
    seg_len = min(seg_len, nblk)
    nseg = -(-nblk // seg_len)
    return bh * nseg * (16 * nw * seg_len + 16 * (nt - 1))


@pytest.mark.parametrize("R", [0, 1, 3, 4])
def test_general_tail_depth_workspace(R):
    """VJP of a tail depth other than 2: 3 + 4 R vectors [bh][Lpad] (u^(R), v^(R), R row and
    R + 1 column orbit factors, R + R scaled cotangents); bands the streaming passes cover
    (fp32 h <= 64, bf16 h <= 128) add two column-partial buffers for the level passes; the
    dustbin entry point (dense support, wide passes) sizes its L + 1 rows with the vectors
    alone."""
    st, n = _ws_bytes(_prob(R=R, L=1000, bh=3, W=16), B.SKA_OP_VJP)            # fp32, h = 8
    assert st == 0 and n == ((3 + 4 * R) * 3 * 1024 + 2 * _stream_partials(3, 1000, 4, 5)) * 4
    st, n = _ws_bytes(_prob(R=R, L=1000, bh=3, W=256, dtype=B.SKA_BF16), B.SKA_OP_VJP)  # h = 128
    assert st == 0 and n == ((3 + 4 * R) * 3 * 1024 + 2 * _stream_partials(3, 1000, 8, 17)) * 4
    st, n = _ws_bytes(_prob(R=R, L=1000, bh=3, W=600, dtype=B.SKA_BF16), B.SKA_OP_VJP)  # wide
    assert st == 0 and n == (3 + 4 * R) * 3 * 1024 * 4
    st, n = _ws_bytes(_prob(R=R, L=4096, bh=4), B.SKA_OP_DUSTBIN_BLOCK_VJP)
    assert st == 0 and n == (3 + 4 * R) * 4 * 4160 * 4


def test_tail_remainder_workspace_and_checks():
    """The certificate's workspace holds O and two gradient sets [bh][L][d] (input dtype), both
    dual sets (2R + 1 and 2(T + R) + 1 vectors), 256 x 2 doubles of block sums and the largest
    inner forward/VJP workspace, each piece rounded to 256 bytes; T + R above 256 is rejected."""
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for dtype, esz in ((B.SKA_F32, 4), (B.SKA_BF16, 2)):
        prob = _prob(L=1000, bh=3, W=16, T=5, R=2, dtype=dtype)
        st, n = _ws_bytes(prob, B.SKA_OP_TAIL_REMAINDER)
        inner = max(_ws_bytes(prob, B.SKA_OP_FWD)[1], _ws_bytes(prob, B.SKA_OP_VJP)[1],
                    _ws_bytes(_prob(L=1000, bh=3, W=16, T=0, R=7, dtype=dtype), B.SKA_OP_FWD)[1],
                    _ws_bytes(_prob(L=1000, bh=3, W=16, T=0, R=7, dtype=dtype), B.SKA_OP_VJP)[1])
        want = (7 * up(3 * 1000 * 64 * esz) + up(5 * 3 * 1000 * 4) + up(15 * 3 * 1000 * 4)
                + up(512 * 8) + up(inner))
        assert st == 0 and n == want
    # R = 0: the base pair (u^(0), v^(0)) beside the 2 T + 1 duals of full backpropagation
    prob0 = _prob(L=1000, bh=3, W=16, T=5, R=0)
    st, n = _ws_bytes(prob0, B.SKA_OP_TAIL_REMAINDER)
    inner = max(_ws_bytes(prob0, B.SKA_OP_FWD)[1], _ws_bytes(prob0, B.SKA_OP_VJP)[1],
                _ws_bytes(_prob(L=1000, bh=3, W=16, T=0, R=5), B.SKA_OP_FWD)[1],
                _ws_bytes(_prob(L=1000, bh=3, W=16, T=0, R=5), B.SKA_OP_VJP)[1])
    assert st == 0 and n == (7 * up(3 * 1000 * 64 * 4) + up(2 * 3 * 1000 * 4) + up(11 * 3 * 1000 * 4)
                             + up(512 * 8) + up(inner))
    st, _ = _ws_bytes(_prob(T=250, R=7), B.SKA_OP_TAIL_REMAINDER)
    assert st == -2 and "T + R" in B.ska_last_error()
    prob = _prob()
    _, need = _ws_bytes(prob, B.SKA_OP_TAIL_REMAINDER)
    V = ctypes.c_void_p
    f = B.lib.sinkhorn_attn_tail_remainder
    assert f(ctypes.byref(prob), V(FAKE), V(FAKE), V(FAKE), V(FAKE), None, V(FAKE), need, None) == -1
    assert f(ctypes.byref(prob), V(FAKE), V(FAKE), V(FAKE), V(FAKE), V(FAKE + 4), V(FAKE), need, None) == -1
    assert f(ctypes.byref(prob), V(FAKE), V(FAKE), V(FAKE), V(FAKE), V(FAKE), V(FAKE), need - 8, None) == -3


def test_empty_problems_enqueue_nothing():
    for kw in (dict(bh=0), dict(L=0)):
        prob = _prob(**kw)
        assert B.lib.sinkhorn_attn_fwd(ctypes.byref(prob), None, None, None, None, None, None, 0,
                                       None) == 0
        assert B.lib.sinkhorn_attn_vjp(ctypes.byref(prob), None, None, None, None, None, None,
                                       None, None, None, 0, None, 0, None) == 0
    prob = _prob(bh=0)
    assert B.lib.sinkhorn_attn_dustbin_block_fwd(ctypes.byref(prob), None, None, None, None, None,
                                                 None, 0, None) == 0


def test_status_strings():
    assert B.ska_status_string(0) == "ok"
    assert B.ska_status_string(-3) == "workspace too small"
    assert B.ska_status_string(42) == "unknown status"


def test_contraction_layout_and_checks():
    """The certificate's [bh][nb][2 m + 1] layout: nb = ceil(Lr / block), m = min(h // block,
    nb - 1), the same as the oracle's block_layout; the dustbin entry point counts L + 1 tokens on
    the dense support; bad blocks and null outputs are rejected before any launch."""
    import oracle
    for L, W, blk in ((100, 16, 16), (1000, 256, 16), (1000, 256, 64), (37, 0, 16), (5000, 4000, 128)):
        nb, m = B.ska_contraction_layout(_prob(L=L, W=W), B.SKA_OP_CONTRACTION, blk)
        assert (nb, m) == oracle.block_layout(L, min(W // 2, L), blk)
    nb, m = B.ska_contraction_layout(_prob(L=4096, W=256), B.SKA_OP_DUSTBIN_BLOCK_CONTRACTION, 16)
    assert (nb, m) == (257, 256) == oracle.block_layout(4097, 4096, 16)
    for bad in (0, 8, 48, 256):
        with pytest.raises(B.SinkhornAttnError):
            B.ska_contraction_layout(_prob(), B.SKA_OP_CONTRACTION, bad)
    with pytest.raises(B.SinkhornAttnError):
        B.ska_contraction_layout(_prob(), B.SKA_OP_FWD, 16)
    st, n = _ws_bytes(_prob(), B.SKA_OP_CONTRACTION)
    assert st == 0 and n == 0
    prob = _prob()
    V = ctypes.c_void_p
    f = B.lib.sinkhorn_attn_contraction_certificate
    assert f(ctypes.byref(prob), 16, V(FAKE), V(FAKE), None, None, None, None) == -1
    assert f(ctypes.byref(prob), 16, V(FAKE), V(FAKE + 4), V(FAKE), None, None, None) == -1
    assert f(ctypes.byref(prob), 24, V(FAKE), V(FAKE), V(FAKE), None, None, None) == -1
    assert f(ctypes.byref(prob), 16, V(FAKE), V(FAKE), V(FAKE + 2), None, None, None) == -1
    empty = _prob(bh=0)
    assert f(ctypes.byref(empty), 16, None, None, None, None, None, None) == 0


def test_noalloc_forward_checks_arguments_and_size_on_the_host():
    """sinkhorn_attn_fwd_noalloc rejects a malformed problem, and one whose forward workspace is
    larger than its static array (32 MiB), before it touches a device; 4 problems of 262144
    tokens at W = 256 fit, 8 do not."""
    vp = ctypes.c_void_p(FAKE)
    big = _prob(bh=8, L=262144, W=256, T=15, dtype=B.SKA_BF16)
    st, n = _ws_bytes(big, B.SKA_OP_FWD)
    assert st == 0 and n > (32 << 20)
    assert B.lib.sinkhorn_attn_fwd_noalloc(ctypes.byref(big), vp, vp, vp, vp, vp, None) == -2
    assert "static scratch" in B.ska_last_error()
    st, n = _ws_bytes(_prob(bh=4, L=262144, W=256, T=15, dtype=B.SKA_BF16), B.SKA_OP_FWD)
    assert st == 0 and n <= (32 << 20)
    assert B.lib.sinkhorn_attn_fwd_noalloc(ctypes.byref(_prob(W=15)), vp, vp, vp, vp, vp, None) == -1
    assert B.lib.sinkhorn_attn_fwd_noalloc(None, vp, vp, vp, vp, vp, None) == -1


def test_last_error_is_per_thread():
    """Two host threads, each failing with its own argument error at the same time, read back the
    detail of their own last error (the ABI keeps ska_last_error() per thread)."""
    import threading
    barrier = threading.Barrier(2, timeout=30)
    bad = []

    def worker(kw, expect):
        try:
            for _ in range(100):
                n = ctypes.c_size_t(0)
                st = B.lib.ska_workspace_bytes(ctypes.byref(_prob(**kw)), B.SKA_OP_FWD,
                                               ctypes.byref(n))
                barrier.wait()      # both threads have recorded an error before either reads
                got = B.ska_last_error()
                barrier.wait()
                if st >= 0 or expect not in got:
                    bad.append((kw, st, got))
        except threading.BrokenBarrierError:
            bad.append("barrier timed out")

    threads = [threading.Thread(target=worker, args=(dict(d=32), "head dimension")),
               threading.Thread(target=worker, args=(dict(L=-1), "L must be"))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(60)
    assert not any(t.is_alive() for t in threads)
    assert not bad, bad[:3]
