"""The C-ABI library: it loads, exports every function its header declares,
and rejects bad arguments on the host, before any GPU work (runs without a GPU)."""
import ctypes
import os
import re

import pytest

from io_aware_exact_06_amd import attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(attn_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(attn.EXPORTS)
    L = attn.lib()
    for n in names:
        assert hasattr(L, n), n


def test_cstep_library_exports_the_same_functions():
    """libattn_cstep.so (the hand-scheduled loops compiled out, for the bitwise
    GPU comparison) is the same C ABI."""
    L = attn.open_library(attn.CSTEP_LIB_PATH)
    for n in declared_functions():
        assert hasattr(L, n), n


def test_missing_library_raises_instead_of_falling_back(monkeypatch, tmp_path):
    """Without the built library every entry point fails loudly: there is no
    other path that could compute attention."""
    monkeypatch.setattr(attn, "LIB_PATH", str(tmp_path / "libattn.so"))
    monkeypatch.setattr(attn, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        attn.lib()
    with pytest.raises(RuntimeError, match="missing"):
        attn.attn_status_string(0)
    with pytest.raises(RuntimeError, match="missing"):
        attn.attn_fwd(0, 0, 0, 0, 0, 1, 1, 4, 64, 0, 0.125, attn.ATTN_F16, 0)


def test_status_strings():
    for s in range(9):
        assert attn.attn_status_string(s) and attn.attn_status_string(s) != "unknown status"
    assert attn.attn_status_string(99) == "unknown status"


# Fake device addresses: validation never dereferences them.
A = 0x10000000
SZ = 1 * 2 * 64 * 64 * 2  # bytes of a [1,2,64,64] 16-bit tensor


def fwd(q=A, k=A + 0x100000, v=A + 0x200000, o=A + 0x300000, lse=A + 0x400000, B=1, H=2, N=64, d=64,
        causal=0, scale=0.125, dtype=1):
    return attn.attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, None)


def bwd(ws_bytes=None, ws=A + 0x900000, **kw):
    a = dict(q=A, k=A + 0x100000, v=A + 0x200000, o=A + 0x300000, dout=A + 0x400000, lse=A + 0x500000,
             dq=A + 0x600000, dk=A + 0x700000, dv=A + 0x800000, B=1, H=2, N=64, d=64, causal=0,
             scale=0.125, dtype=1)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = attn.attn_bwd_workspace_bytes(a["B"], a["H"], a["N"], a["d"])
    return attn.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                         a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"], a["dtype"], ws, ws_bytes,
                         None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), 1), (dict(o=0), 1), (dict(lse=0), 1),
    (dict(N=-1), 2), (dict(B=-3), 2),
    (dict(d=96), 3), (dict(d=32), 3), (dict(dtype=2), 3), (dict(causal=2), 3),
    (dict(scale=float("nan")), 3), (dict(scale=float("inf")), 3), (dict(scale=-float("inf")), 3),
    (dict(q=A + 8), 4), (dict(o=A + 0x300002), 4), (dict(lse=A + 0x400002), 4),
    (dict(o=A + 0x100), 5), (dict(lse=A + 0x300000 + SZ - 4), 5), (dict(o=A + 0x200000), 5),
    (dict(B=1 << 30, H=1 << 30, N=1 << 20), 2),
])
def test_fwd_rejects(kw, status):
    assert fwd(**kw) == status


def test_any_finite_scale_is_accepted():
    """Negative and zero scales pass validation (an empty problem returns
    right after the checks, so nothing is launched)."""
    for s in (-1.0, -0.125, -0.0, 0.0, 1e30, -1e30):
        assert fwd(q=0, k=0, v=0, o=0, lse=0, N=0, scale=s) == 0
        assert bwd(q=0, k=0, v=0, o=0, dout=0, lse=0, dq=0, dk=0, dv=0, ws=0, ws_bytes=0, N=0, scale=s) == 0
        assert fwd_varlen(q=0, k=0, v=0, o=0, lse=0, tq=0, scale=s) == 0


def test_fwd_empty_problem_is_a_no_op():
    # nothing is enqueued and the pointers are not examined
    assert fwd(q=0, k=0, v=0, o=0, lse=0, N=0) == 0
    assert fwd(q=0, k=0, v=0, o=0, lse=0, B=0) == 0


def test_bwd_workspace_bytes():
    B, H, N, d = 2, 3, 100, 128
    n = attn.attn_bwd_workspace_bytes(B, H, N, d)
    assert n >= B * H * N * 4 and n % 256 == 0
    assert attn.attn_bwd_workspace_bytes(0, 3, 100, 128) == 0
    assert attn.attn_bwd_workspace_bytes(-1, 3, 100, 128) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("kw,status", [
    (dict(dout=0), 1), (dict(dv=0), 1), (dict(ws=0), 6),
    (dict(ws_bytes=100), 6), (dict(d=80), 3),
    (dict(dq=A + 4), 4), (dict(ws=A + 0x900008), 4),
    (dict(dq=A + 0x400000), 5), (dict(dk=A + 0x600000), 5), (dict(dv=A + 0x500000), 5),
    (dict(ws=A + 0x800000), 6), (dict(ws=A + 0x100000), 6),
])
def test_bwd_rejects(kw, status):
    assert bwd(**kw) == status


def test_bwd_empty_problem_is_a_no_op():
    assert bwd(q=0, k=0, v=0, o=0, dout=0, lse=0, dq=0, dk=0, dv=0, ws=0, ws_bytes=0, N=0) == 0


def fwd_varlen(q=A, k=A + 0x100000, v=A + 0x200000, o=A + 0x300000, lse=A + 0x400000, cu_q=A + 0x500000,
               cu_k=A + 0x500100, batch=2, H=2, tq=64, tk=80, max_q=40, d=64, causal=0, wl=-1, wr=-1,
               scale=0.125, dtype=1):
    return attn.attn_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, batch, H, tq, tk, max_q, d, causal, wl, wr, scale,
                                dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(cu_q=0), 1), (dict(q=0), 1), (dict(k=0), 1), (dict(lse=0), 1),
    (dict(batch=-1), 2), (dict(tq=-5), 2), (dict(max_q=-1), 2),
    (dict(d=48), 3), (dict(wl=-2), 3), (dict(wr=-3), 3), (dict(causal=3), 3), (dict(scale=float("nan")), 3),
    (dict(tq=1 << 29, tk=(1 << 29) + 1), 2),
    (dict(cu_k=A + 0x500102), 4), (dict(o=A + 0x300008), 4),
    (dict(o=A + 0x100010), 5), (dict(lse=A + 0x500000 - 8), 5), (dict(o=A + 0x500000 - 16), 5),
])
def test_fwd_varlen_rejects(kw, status):
    assert fwd_varlen(**kw) == status


def test_fwd_varlen_empty_calls_are_no_ops():
    assert fwd_varlen(q=0, k=0, v=0, o=0, lse=0, tq=0) == 0
    assert fwd_varlen(q=0, k=0, v=0, o=0, lse=0, max_q=0) == 0
    assert fwd_varlen(q=0, k=0, v=0, o=0, lse=0, cu_q=0, cu_k=0, batch=0) == 0


def test_bwd_varlen_workspace_and_rejects():
    n = attn.attn_bwd_varlen_workspace_bytes(3, 1000)
    assert n >= 3 * 1000 * 4 and n % 256 == 0
    assert attn.attn_bwd_varlen_workspace_bytes(0, 1000) == 0
    args = dict(q=A, k=A + 0x100000, v=A + 0x200000, o=A + 0x300000, dout=A + 0x400000, lse=A + 0x500000,
                dq=A + 0x600000, dk=A + 0x700000, dv=A + 0x800000, cu_q=A + 0x900000, cu_k=A + 0x900100,
                batch=2, H=2, tq=64, tk=80, max_q=40, max_k=50, d=64, causal=1, wl=-1, wr=-1, scale=0.1,
                dtype=0, ws=A + 0xA00000, ws_bytes=attn.attn_bwd_varlen_workspace_bytes(2, 64))

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return attn.attn_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"],
                                    a["dv"], a["cu_q"], a["cu_k"], a["batch"], a["H"], a["tq"], a["tk"],
                                    a["max_q"], a["max_k"], a["d"], a["causal"], a["wl"], a["wr"], a["scale"],
                                    a["dtype"], a["ws"], a["ws_bytes"], None)
    assert call(dq=0) == 1
    assert call(ws=0) == 6
    assert call(ws_bytes=16) == 6
    assert call(dk=A + 0x100000) == 5
    assert call(ws=A + 0x900000) == 6
    assert call(max_k=-1) == 2
    assert call(q=0, k=0, v=0, o=0, dout=0, lse=0, dq=0, dk=0, dv=0, tq=0, tk=0) == 0


def test_fwd_unfused_validation():
    B, H, N, d = 1, 2, 64, 64
    need = attn.attn_fwd_unfused_workspace_bytes(B, H, N)
    assert need >= B * H * N * N * 6 and need % 256 == 0
    assert attn.attn_fwd_unfused_workspace_bytes(1, 1 << 17, 4) == ctypes.c_size_t(-1).value
    base = dict(q=A, k=A + 0x100000, v=A + 0x200000, o=A + 0x300000, lse=A + 0x400000, ws=A + 0x500000)

    def call(ws_bytes=need, **kw):
        a = dict(base)
        a.update(kw)
        return attn.attn_fwd_unfused(a["q"], a["k"], a["v"], a["o"], a["lse"], B, H, N, d, 1, 0.125, 1, a["ws"],
                                     ws_bytes, None)
    assert call(ws=0) == 6
    assert call(ws_bytes=need - 1) == 6
    assert call(ws=A + 0x500004) == 4
    assert call(o=A + 0x200000) == 5
    assert call(ws=A + 0x300000) == 6


def test_blocksparse_validation():
    B, H, N, d = 1, 2, 300, 64          # nb = 3 blocks of 128
    nb = 3
    q, k, v, o, lse, bm = A, A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000, A + 0x500000
    f = lambda **kw: attn.attn_fwd_blocksparse(kw.get("q", q), k, v, kw.get("o", o), lse, B, H, kw.get("N", N), d,
                                               kw.get("bm", bm), kw.get("mh", 1), 1, 0.125, 1, None)
    assert f(bm=None) == 1                  # a block mask is required
    assert f(mh=3) == 2 and f(mh=0) == 2    # mask_heads must be 1, H or B*H
    assert f(o=bm - 16) == 5                # the output overlaps the mask ([1, 3, 3] bytes)
    assert f(N=0, bm=None) == 0             # empty problems do nothing
    assert f(mh=2, o=bm + 16) == 5          # [2, 3, 3] bytes reach the output at byte 16
    assert f(mh=1, q=0) == 1
    ws = A + 0x600000
    need = attn.attn_bwd_workspace_bytes(B, H, N, d)
    g = lambda **kw: attn.attn_bwd_blocksparse(q, k, v, o, A + 0x700000, lse, kw.get("dq", A + 0x800000),
                                               A + 0x900000, A + 0xa00000, B, H, N, d, kw.get("bm", bm),
                                               kw.get("mh", 2), 0, 0.125, 1, ws, need, None)
    assert g(bm=None) == 1 and g(mh=5) == 2
    assert g(dq=bm - 16) == 5               # a gradient overlaps the mask


def test_bench_traffic_gate():
    """bench.py reports the stored HBM traffic only for the kernel code it was
    measured on (comments aside)."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    digest = bench.kernel_code_digest()
    saved = dict(bench.TRAFFIC)
    try:
        bench.TRAFFIC["sha256"] = digest
        assert bench.measured_traffic("fwd") == saved["fwd"]
        bench.TRAFFIC["sha256"] = "0" * 64
        assert bench.measured_traffic("fwd") is None and bench.measured_traffic("bwd") is None
    finally:
        bench.TRAFFIC.update(saved)


def bwd_noalloc(**kw):
    a = dict(q=A, k=A + 0x100000, v=A + 0x200000, o=A + 0x300000, dout=A + 0x400000, lse=A + 0x500000,
             dq=A + 0x600000, dk=A + 0x700000, dv=A + 0x800000, B=1, H=2, N=64, d=64, causal=0,
             scale=0.125, dtype=1)
    a.update(kw)
    return attn.attn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                                 a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dout=0), 1), (dict(dv=0), 1), (dict(d=80), 3), (dict(scale=float("nan")), 3),
    (dict(dq=A + 4), 4), (dict(dq=A + 0x400000), 5), (dict(dk=A + 0x600000), 5),
    (dict(B=1, H=1, N=attn.NOALLOC_MAX_ROWS + 1), 8),
    (dict(B=2, H=8, N=attn.NOALLOC_MAX_ROWS // 16 + 1), 8),
])
def test_bwd_noalloc_rejects(kw, status):
    """Host checks of the allocation-free backward, the size limit of its fixed
    scratch included, all before any HIP call."""
    assert bwd_noalloc(**kw) == status


def test_bwd_noalloc_empty_problem_is_a_no_op():
    assert bwd_noalloc(q=0, k=0, v=0, o=0, dout=0, lse=0, dq=0, dk=0, dv=0, N=0) == 0
