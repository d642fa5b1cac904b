"""The unfused three-pass baseline on the GPU: same results as the oracle (and
as the fused forward, within the same tolerance)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_06_amd import attn
from io_aware_exact_06_amd.inputs import default_scale, make_inputs
from tests.tolerance import lse_report, o_report

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,N,d,dtype,causal", [
    (1, 2, 256, 64, "f16", False), (2, 1, 300, 128, "bf16", True), (1, 1, 77, 64, "bf16", False),
    (1, 2, 513, 128, "f16", True), (1, 1, 1, 64, "f16", True), (1, 1, 130, 128, "bf16", False),
])
def test_unfused_matches_oracle(B, H, N, d, dtype, causal):
    print("unfused B%d H%d N%d d%d %s causal=%d" % (B, H, N, d, dtype, causal), flush=True)
    inp = make_inputs(B, H, N, d, dtype, seed=N + 17 * d)
    scale = default_scale(d)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o, lse = attn.fwd_unfused(q, k, v, causal, scale)
    of, lf = attn.fwd(q, k, v, causal, scale)
    torch.cuda.synchronize()
    h = lambda t: t.double().numpy().reshape(B * H, N, d)
    ro, rl = oracle.fwd(h(inp["q"]), h(inp["k"]), h(inp["v"]), causal, scale)
    for oo, ll, name in ((o, lse, "unfused"), (of, lf, "fused")):
        r1 = o_report(oo.float().cpu().numpy().reshape(B * H, N, d), ro, dtype)
        r2 = lse_report(ll.cpu().numpy().reshape(B * H, N), rl)
        print("  %s: O max_abs %.3g lse %.3g" % (name, r1["max_abs"], r2["max_floored_rel"]), flush=True)
        assert r1["ok"] and r2["ok"], (name, r1, r2)
