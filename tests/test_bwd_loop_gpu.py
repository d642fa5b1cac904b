"""The backward's hand-scheduled walks (the dK/dV kernel's over unmasked query
tiles at d = 128, the dQ kernel's over unmasked key tiles at d = 64 and 128), against the
fp64 oracle: whole-tensor rel-L2 of dQ, dK, dV (the backward acceptance
measure) on shapes whose walks enter the loops at each ring-buffer phase (three
in the dK/dV walk, two K/V buffers in the dQ walk), run them for one tile or
many, and leave them before a ragged last tile; plus packed sequences with
sliding windows (walks starting at odd tiles), and determinism."""
import sys

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_06_amd import attn
from io_aware_exact_06_amd.inputs import default_scale, make_inputs
from tests.tolerance import GRAD_TOL, rel_l2

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("B,H,N,d,dtype,causal", [
    (1, 4, 1024, 128, "bf16", True),
    (2, 3, 1024, 128, "f16", False),
    (1, 2, 777, 128, "bf16", False),    # ragged: the last tiles go through the C++ tile
    (1, 3, 1500, 128, "f16", True),
    (2, 2, 320, 128, "bf16", False),    # walks of five tiles: the loop runs one or two
    (1, 2, 2048, 128, "bf16", True),
    (1, 3, 128, 128, "f16", False),     # two key tiles: the dQ walk runs a single tile
    (2, 2, 200, 128, "bf16", False),    # the dQ walk runs two tiles, a ragged one follows
    # d = 64: the dQ walk only (the dK/dV kernel keeps its C++ tile there)
    (1, 3, 1024, 64, "f16", True),
    (2, 2, 777, 64, "bf16", False),
    (1, 2, 128, 64, "bf16", False),
    (2, 3, 1500, 64, "f16", True),
])
def test_bwd_loop_dense(B, H, N, d, dtype, causal):
    label = "bwd loops B%d H%d N%d d%d %s causal=%d" % (B, H, N, d, dtype, causal)
    say(label)
    inp = make_inputs(B, H, N, d, dtype, seed=N + 7 * H + causal, with_dout=True)
    scale = default_scale(d)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "dout"))
    o, lse = attn.fwd(q, k, v, causal, scale)
    dq, dk, dv = attn.bwd(q, k, v, o, do, lse, causal, scale)
    torch.cuda.synchronize()
    r = lambda t: t.double().numpy().reshape(B * H, N, d)  # noqa: E731
    rq, rk, rv = oracle.bwd(r(inp["q"]), r(inp["k"]), r(inp["v"]), r(inp["dout"]), causal, scale)
    errs = [rel_l2(a.float().cpu().numpy().reshape(B * H, N, d), ref) for a, ref in ((dq, rq), (dk, rk), (dv, rv))]
    say("  rel-L2 dq %.3g dk %.3g dv %.3g" % tuple(errs))
    assert max(errs) <= GRAD_TOL, (label, errs)


@pytest.mark.parametrize("window,d", [((300, 0), 128), ((500, 200), 128), ((500, 200), 64)])
def test_bwd_loop_windows(window, d):
    lq = [1200, 700, 1600]
    H, dtype = 2, "bf16"
    tq = sum(lq)
    a = make_inputs(1, H, tq, d, dtype, seed=sum(window) + 5, with_dout=True)
    q, k, v, do = a["q"][0], a["k"][0], a["v"][0], a["dout"][0]
    cu = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    scale = default_scale(d)
    tcu = torch.from_numpy(cu).cuda()
    gq, gk, gv, gdo = (t.cuda() for t in (q, k, v, do))
    o, lse = attn.fwd_varlen(gq, gk, gv, tcu, tcu, max(lq), False, scale, window)
    dq, dk, dv = attn.bwd_varlen(gq, gk, gv, o, gdo, lse, tcu, tcu, max(lq), max(lq), False, scale, window)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(),
                                   cu, cu, False, scale, window)
    errs = [rel_l2(x.float().cpu().numpy(), ref) for x, ref in ((dq, rq), (dk, rk), (dv, rv))]
    say("window %s: rel-L2 dq %.3g dk %.3g dv %.3g" % ((window,) + tuple(errs)))
    assert max(errs) <= GRAD_TOL, errs


def test_bwd_loop_deterministic():
    inp = make_inputs(1, 4, 1024, 128, "bf16", seed=21, with_dout=True)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "dout"))
    o, lse = attn.fwd(q, k, v, True, 0.09)
    g1 = attn.bwd(q, k, v, o, do, lse, True, 0.09)
    g2 = attn.bwd(q, k, v, o, do, lse, True, 0.09)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))
