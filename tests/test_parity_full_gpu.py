"""Whole-tensor parity of the five problem configurations against the fp64 oracle.

Every element of O and lse, of every row of every head, is compared for all
five configurations.  For the two configurations with a backward pass, the
relative L2 error is taken per tensor over all elements of dQ, dK and dV.

Acceptance (tests/tolerance.py):
- O: |O_gpu - O_ref| <= tol + ulp(O_ref)/2, with tol 2e-3 for fp16 and 1e-2 for bf16;
- lse: |err| / max(1, |lse_ref|) <= 1e-4;
- gradients: relative L2 <= 1e-2.

The raw O max-abs, the count of elements where half an ulp of O_ref is
already at least tol, and the floored and unfloored lse errors are reported
as well.  With ATTN_PARITY_REPORT=<path> set, the module writes these figures
as a markdown table to <path> when it finishes.
"""
import os
import sys
import time

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_06_amd import attn
from io_aware_exact_06_amd.inputs import WORKLOADS, default_scale, workload_inputs
from tests.tolerance import GRAD_TOL, LSE_TOL, O_TOL, lse_report, o_report, rel_l2

pytestmark = pytest.mark.gpu

REPORT = {}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def heads(t):
    B, H, N, d = t.shape
    return t.double().numpy().reshape(B * H, N, d)


@pytest.fixture(scope="module", autouse=True)
def report_file():
    yield
    path = os.environ.get("ATTN_PARITY_REPORT")
    if not path or not REPORT:
        return
    lines = [
        "# Parity of the five configurations against the fp64 oracle (every element)",
        "",
        "Command: `ATTN_PARITY_REPORT=%s python -u -m pytest tests/test_parity_full_gpu.py -v` "
        "(one GPU; the oracle runs on %d host threads)." % (path, oracle.num_threads()),
        "",
        "Forward: O and lse of every row of every head.  `O max-abs` is the raw largest |O_gpu - O_ref|; "
        "`O worst excess` is the largest |O_gpu - O_ref| - (tol + ulp(O_ref)/2), which must be <= 0; "
        "`#half-ulp >= tol` counts the elements whose rounding to the storage type alone may reach the "
        "bare tolerance.  lse errors: floored |err| / max(1, |lse_ref|) (acceptance <= %g) and the plain "
        "relative |err| / |lse_ref|." % LSE_TOL,
        "",
        "| configuration | O elements | O tol | O max-abs | O worst excess | #half-ulp >= tol | "
        "lse floored rel | lse rel | oracle s |",
        "|---|---|---|---|---|---|---|---|---|",
    ]
    for w in WORKLOADS:
        r = REPORT.get((w.name, "fwd"))
        if r:
            lines.append("| %s | %d | %g | %.3g | %.3g | %d | %.3g | %.3g | %.1f |" % (
                w.name, r["n"], O_TOL[w.dtype], r["max_abs"], r["worst_excess"], r["n_halfulp_ge_tol"],
                r["max_floored_rel"], r["max_rel"], r["oracle_s"]))
    lines += ["", "Backward: relative L2 error per tensor over all elements (acceptance <= %g)." % GRAD_TOL, "",
              "| configuration | elements per tensor | dQ rel-L2 | dK rel-L2 | dV rel-L2 | oracle s |",
              "|---|---|---|---|---|---|"]
    for w in WORKLOADS:
        r = REPORT.get((w.name, "bwd"))
        if r:
            lines.append("| %s | %d | %.3g | %.3g | %.3g | %.1f |" % (
                w.name, r["n"], r["dq"], r["dk"], r["dv"], r["oracle_s"]))
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_fwd_every_element(idx):
    w = WORKLOADS[idx]
    say("full forward parity: %s" % w.name)
    inp = workload_inputs(idx)
    scale = default_scale(w.d)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o, lse = attn.fwd(q, k, v, w.causal, scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().reshape(-1, w.N, w.d)
    lse = lse.cpu().numpy().reshape(-1, w.N)
    del q, k, v
    t0 = time.perf_counter()
    ro, rl = oracle.fwd(heads(inp["q"]), heads(inp["k"]), heads(inp["v"]), w.causal, scale)
    t_or = time.perf_counter() - t0
    rep_o, rep_l = o_report(o, ro, w.dtype), lse_report(lse, rl)
    REPORT[(w.name, "fwd")] = dict(rep_o, **rep_l, n=o.size, oracle_s=t_or)
    say("  O max_abs=%.3g worst_excess=%.3g half-ulp>=tol: %d | lse floored=%.3g rel=%.3g | oracle %.1f s" % (
        rep_o["max_abs"], rep_o["worst_excess"], rep_o["n_halfulp_ge_tol"], rep_l["max_floored_rel"],
        rep_l["max_rel"], t_or))
    assert rep_o["ok"], rep_o
    assert rep_l["ok"], rep_l


@pytest.mark.parametrize("idx", [3, 4])
def test_bwd_every_element(idx):
    w = WORKLOADS[idx]
    say("full backward parity: %s" % w.name)
    inp = workload_inputs(idx)
    scale = default_scale(w.d)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "dout"))
    o, lse = attn.fwd(q, k, v, w.causal, scale)
    dq, dk, dv = attn.bwd(q, k, v, o, do, lse, w.causal, scale)
    torch.cuda.synchronize()
    g = [t.float().cpu().numpy().reshape(-1, w.N, w.d) for t in (dq, dk, dv)]
    del q, k, v, do, o, lse, dq, dk, dv
    t0 = time.perf_counter()
    ref = oracle.bwd(heads(inp["q"]), heads(inp["k"]), heads(inp["v"]), heads(inp["dout"]), w.causal, scale)
    t_or = time.perf_counter() - t0
    errs = [rel_l2(a, r) for a, r in zip(g, ref)]
    REPORT[(w.name, "bwd")] = dict(dq=errs[0], dk=errs[1], dv=errs[2], n=g[0].size, oracle_s=t_or)
    say("  rel-L2 dq %.3g dk %.3g dv %.3g | oracle %.1f s" % (*errs, t_or))
    assert max(errs) <= GRAD_TOL, errs
