"""The hand-scheduled loops against the C++ steps they replace, bitwise.

libattn.so runs the unmasked tiles of the forward (d = 128), the dQ kernel
(d = 64, 128) and the dK/dV kernel (d = 128) through inline-assembly loops
that issue the C++ steps' arithmetic in the same order; libattn_cstep.so is
the same sources built with the loops compiled out.  Both run on the same
inputs, and O, lse, dQ, dK and dV must be identical bit for bit: causal and
not, both 16-bit types, ragged lengths, grids above and below 256 work
groups, walks of one tile and of many, and packed sequences with sliding
windows (walks that start at odd tiles).
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

from io_aware_exact_06_amd import attn
from io_aware_exact_06_amd.inputs import default_scale, make_inputs

pytestmark = pytest.mark.gpu

LIBS = {}


def libs():
    if not LIBS:
        LIBS["loop"] = attn.lib()
        LIBS["cstep"] = attn.open_library(attn.CSTEP_LIB_PATH)
    return LIBS["loop"], LIBS["cstep"]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_dense(L, q, k, v, do, causal, scale, dtype):
    B, H, N, d = q.shape
    st = torch.cuda.current_stream().cuda_stream
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=q.device, dtype=torch.float32)
    assert L.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                      int(causal), scale, dtype, st) == 0
    wsb = L.attn_bwd_workspace_bytes(B, H, N, d)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    g = [torch.empty_like(q) for _ in range(3)]
    assert L.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                      g[0].data_ptr(), g[1].data_ptr(), g[2].data_ptr(), B, H, N, d, int(causal), scale, dtype,
                      ws.data_ptr(), wsb, st) == 0
    torch.cuda.synchronize()
    return [o, lse] + g


def same(label, a, b):
    names = ("O", "lse", "dQ", "dK", "dV")
    diff = [n for n, x, y in zip(names, a, b) if not torch.equal(x, y)]
    say("%s: %s" % (label, "bitwise equal" if not diff else "differ in " + ", ".join(diff)))
    assert not diff, (label, diff)


@pytest.mark.parametrize("B,H,N,d,dtype,causal", [
    (2, 20, 1024, 128, "bf16", True),    # > 256 groups: the forward's loop path
    (2, 20, 1024, 128, "f16", False),
    (3, 24, 777, 128, "bf16", False),    # ragged
    (1, 4, 1500, 128, "f16", True),      # <= 256 groups: the forward's key split (no loop), both backward walks
    (2, 2, 320, 128, "bf16", False),     # short walks
    (1, 3, 128, 128, "f16", False),      # a one-tile dQ walk
    (2, 16, 1024, 64, "f16", True),      # d = 64: the dQ walk only
    (1, 3, 777, 64, "bf16", False),
])
def test_loops_match_cstep(B, H, N, d, dtype, causal):
    loop, cstep = libs()
    inp = make_inputs(B, H, N, d, dtype, seed=N + 3 * H + d + causal, with_dout=True)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "dout"))
    dt = attn.ATTN_BF16 if dtype == "bf16" else attn.ATTN_F16
    scale = default_scale(d)
    a = run_dense(loop, q, k, v, do, causal, scale, dt)
    b = run_dense(cstep, q, k, v, do, causal, scale, dt)
    same("B%d H%d N%d d%d %s causal=%d" % (B, H, N, d, dtype, causal), a, b)


def run_varlen(L, q, k, v, do, cu, maxlen, scale, window, dtype):
    T, H, d = q.shape[1], q.shape[0], q.shape[2]
    st = torch.cuda.current_stream().cuda_stream
    batch = cu.numel() - 1
    o = torch.empty_like(q)
    lse = torch.empty(H, T, device=q.device, dtype=torch.float32)
    assert L.attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             cu.data_ptr(), cu.data_ptr(), batch, H, T, T, maxlen, d, 0,
                             window[0], window[1], scale, dtype, st) == 0
    wsb = L.attn_bwd_varlen_workspace_bytes(H, T)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=q.device)
    g = [torch.empty_like(q) for _ in range(3)]
    assert L.attn_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                             lse.data_ptr(), g[0].data_ptr(), g[1].data_ptr(), g[2].data_ptr(), cu.data_ptr(),
                             cu.data_ptr(), batch, H, T, T, maxlen, maxlen, d, 0, window[0], window[1], scale,
                             dtype, ws.data_ptr(), wsb, st) == 0
    torch.cuda.synchronize()
    return [o, lse] + g


@pytest.mark.parametrize("window,d", [((400, 0), 128), ((700, 300), 128), ((500, 200), 64)])
def test_loops_match_cstep_windows(window, d):
    loop, cstep = libs()
    lq = [2048, 1500, 2048]
    H, dtype = 16, "bf16"
    a = make_inputs(1, H, sum(lq), d, dtype, seed=sum(window) + d, with_dout=True)
    q, k, v, do = (a[n][0].cuda() for n in ("q", "k", "v", "dout"))
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)).cuda()
    scale = default_scale(d)
    ra = run_varlen(loop, q, k, v, do, cu, max(lq), scale, window, attn.ATTN_BF16)
    rb = run_varlen(cstep, q, k, v, do, cu, max(lq), scale, window, attn.ATTN_BF16)
    same("window %s d%d" % (window, d), ra, rb)
