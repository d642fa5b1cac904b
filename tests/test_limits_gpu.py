"""Size limits on the GPU: very long sequences (N = 131072 at d = 64: 1024 query
tiles of one head, 2048 key tiles per causal row; N = 65536 at d = 128) and
very many tiny heads (4096 heads of 3 rows), against the fp64 oracle.  For the
long sequences the forward and dQ are checked on sampled rows the oracle
computes one by one; dK and dV through
identities exact at any size (sum_j dK_j = 0 because every row of dS sums to
zero; sum_j dV_j = sum_i dO_i because every row of P sums to one)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_06_amd import attn
from io_aware_exact_06_amd.inputs import default_scale, make_inputs
from tests.tolerance import GRAD_TOL, lse_report, o_report, rel_l2

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("N,d", [(131072, 64), (65536, 128)])
def test_long_sequence(N, d):
    """d = 128 runs the forward loop and both backward walks over runs of up to
    1024 tiles; d = 64 the dQ walk and the C++ steps."""
    B, H, dtype = 1, 1, "bf16"
    say("long sequence N=%d d=%d %s causal" % (N, d, dtype))
    inp = make_inputs(B, H, N, d, dtype, seed=131 + d, with_dout=True)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "dout"))
    scale = default_scale(d)
    o, lse = attn.fwd(q, k, v, True, scale)
    dq, dk, dv = attn.bwd(q, k, v, o, do, lse, True, scale)
    torch.cuda.synchronize()
    rows = np.array(sorted(set([0, 1, 127, 128, N // 2 - 1, N // 2, N - 2, N - 1] +
                               list(np.random.default_rng(3).choice(N, 24, replace=False)))))
    Q, K, V, dO = (inp[n][0].double().numpy() for n in ("q", "k", "v", "dout"))
    ro, rl = oracle.fwd(Q[:, rows], K, V, True, scale, qpos=rows)
    rep = o_report(o[0].float().cpu().numpy()[:, rows], ro, dtype)
    lrep = lse_report(lse[0].cpu().numpy()[:, rows], rl)
    assert rep["ok"], rep
    assert lrep["ok"], lrep
    # dq of the sampled rows: the oracle needs only their statistics (no key rows requested)
    rdq, _, _ = oracle.bwd(Q, K, V, dO, True, scale, rows=rows, keys=[])
    e_dq = rel_l2(dq[0].float().cpu().numpy()[:, rows], rdq)
    # identities over all keys, in fp64 on the host
    gdk = dk[0, 0].double().cpu().numpy()
    gdv = dv[0, 0].double().cpu().numpy()
    sdk = np.abs(gdk.sum(0)).max() / np.abs(gdk).sum(0).max()
    sdv = rel_l2(gdv.sum(0), dO[0].sum(0))
    say("  O max_abs %.3g lse %.3g dq %.3g | sum dK %.3g, sum dV vs sum dO %.3g" % (
        rep["max_abs"], lrep["max_floored_rel"], e_dq, sdk, sdv))
    assert e_dq <= GRAD_TOL
    assert sdk <= 1e-2 and sdv <= 1e-2


def test_many_tiny_heads():
    B, H, N, d, dtype = 64, 64, 3, 128, "f16"
    say("many heads B%d H%d N%d" % (B, H, N))
    inp = make_inputs(B, H, N, d, dtype, seed=64, with_dout=True)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "dout"))
    scale = default_scale(d)
    o, lse = attn.fwd(q, k, v, False, scale)
    dq, dk, dv = attn.bwd(q, k, v, o, do, lse, False, scale)
    torch.cuda.synchronize()
    hd = lambda t: t.double().numpy().reshape(B * H, N, d)
    ro, rl = oracle.fwd(hd(inp["q"]), hd(inp["k"]), hd(inp["v"]), False, scale)
    rep = o_report(o.float().cpu().numpy().reshape(B * H, N, d), ro, dtype)
    lrep = lse_report(lse.cpu().numpy().reshape(B * H, N), rl)
    assert rep["ok"] and lrep["ok"], (rep, lrep)
    rq, rk, rv = oracle.bwd(hd(inp["q"]), hd(inp["k"]), hd(inp["v"]), hd(inp["dout"]), False, scale)
    errs = [rel_l2(a.float().cpu().numpy().reshape(B * H, N, d), r) for a, r in ((dq, rq), (dk, rk), (dv, rv))]
    say("  O max_abs %.3g lse %.3g grads %.3g %.3g %.3g" % (rep["max_abs"], lrep["max_floored_rel"], *errs))
    assert max(errs) <= GRAD_TOL
