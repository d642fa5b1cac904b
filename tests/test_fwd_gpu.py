"""Forward parity on the GPU: the HIP kernel through the C ABI against the fp64 oracle.

Small shapes are compared element by element in full (several tiles and a
ragged tail); the five workloads at their full sizes are compared on
sampled rows that the oracle computes one by one, plus closed forms that hold
at any size (V = 1 gives O = 1; Q = 0 gives the mean, or prefix mean, of V
and lse = ln(number of visible keys)).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_06_amd import attn
from io_aware_exact_06_amd.inputs import WORKLOADS, default_scale, make_inputs, workload_inputs
from tests.tolerance import lse_report, o_report

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_fwd(inp, causal, scale):
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o, lse = attn.fwd(q, k, v, causal, scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def heads(t):
    B, H, N, d = t.shape
    return t.double().numpy().reshape(B * H, N, d)


def oracle_fwd(inp, causal, scale, head_idx=None, rows=None):
    q, k, v = heads(inp["q"]), heads(inp["k"]), heads(inp["v"])
    if head_idx is not None:
        q, k, v = q[head_idx], k[head_idx], v[head_idx]
    if rows is not None:
        return oracle.fwd(q[:, rows], k, v, causal, scale, qpos=rows)
    return oracle.fwd(q, k, v, causal, scale)


def check(o, lse, ro, rl, dtype, label):
    rep_o, rep_l = o_report(o, ro, dtype), lse_report(lse, rl)
    say("%s: O max_abs=%.3g excess=%.3g | lse floored_rel=%.3g rel=%.3g" % (
        label, rep_o["max_abs"], rep_o["worst_excess"], rep_l["max_floored_rel"], rep_l["max_rel"]))
    assert rep_o["ok"], (label, rep_o)
    assert rep_l["ok"], (label, rep_l)


SMALL = [
    # B, H, N, d, dtype, causal
    (1, 2, 64, 128, "bf16", False),
    (1, 3, 300, 128, "bf16", True),
    (2, 2, 1, 64, "f16", True),
    (1, 1, 33, 128, "f16", False),
    (1, 2, 129, 64, "bf16", True),
    (2, 1, 191, 64, "f16", True),
    (1, 2, 1000, 128, "f16", True),
    (1, 2, 517, 64, "bf16", False),
    # more than 256 work groups of 128 rows: the path without the key split
    (4, 64, 200, 128, "bf16", True),
    (2, 80, 517, 64, "f16", False),
]


@pytest.mark.parametrize("B,H,N,d,dtype,causal", SMALL)
def test_fwd_small_full(B, H, N, d, dtype, causal):
    label = "small B%d H%d N%d d%d %s causal=%d" % (B, H, N, d, dtype, causal)
    say(label)
    inp = make_inputs(B, H, N, d, dtype, seed=N * 7 + d + causal)
    scale = default_scale(d)
    o, lse = gpu_fwd(inp, causal, scale)
    ro, rl = oracle_fwd(inp, causal, scale)
    check(o.reshape(B * H, N, d), lse.reshape(B * H, N), ro, rl, dtype, label)


@pytest.mark.parametrize("idx", [0, 1])
def test_fwd_workload_full(idx):
    w = WORKLOADS[idx]
    say("workload %s (full compare)" % w.name)
    inp = workload_inputs(idx)
    scale = default_scale(w.d)
    o, lse = gpu_fwd(inp, w.causal, scale)
    ro, rl = oracle_fwd(inp, w.causal, scale)
    check(o.reshape(-1, w.N, w.d), lse.reshape(-1, w.N), ro, rl, w.dtype, w.name)


def sample_rows(N, rng, extra=48):
    fixed = [0, 1, 2, 63, 64, 127, 128, 129, N // 2, N - 2, N - 1]
    rows = set(r for r in fixed if 0 <= r < N)
    rows.update(int(x) for x in rng.choice(N, size=min(extra, N), replace=False))
    return np.array(sorted(rows))


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_fwd_workload_sampled(idx):
    w = WORKLOADS[idx]
    say("workload %s (sampled rows)" % w.name)
    inp = workload_inputs(idx)
    scale = default_scale(w.d)
    o, lse = gpu_fwd(inp, w.causal, scale)
    o = o.reshape(-1, w.N, w.d)
    lse = lse.reshape(-1, w.N)
    rng = np.random.default_rng(idx)
    BH = w.B * w.H
    hsel = sorted(set([0, BH - 1] + [int(x) for x in rng.choice(BH, size=min(4, BH), replace=False)]))
    rows = sample_rows(w.N, rng)
    ro, rl = oracle_fwd(inp, w.causal, scale, head_idx=hsel, rows=rows)
    check(o[hsel][:, rows], lse[hsel][:, rows], ro, rl, w.dtype, w.name)


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_fwd_closed_forms_full_size(idx):
    """V = 1 -> O = 1;  Q = 0 -> O = mean (prefix mean if causal) of V, lse = ln(#visible keys)."""
    w = WORKLOADS[idx]
    say("closed forms at full size: %s" % w.name)
    inp = workload_inputs(idx)
    scale = default_scale(w.d)
    ones = dict(inp, v=torch.ones_like(inp["v"]))
    o, _ = gpu_fwd(ones, w.causal, scale)
    rep = o_report(o, np.ones_like(o), w.dtype)
    say("  V=1: max_abs=%.3g" % rep["max_abs"])
    assert rep["ok"], rep
    zq = dict(inp, q=torch.zeros_like(inp["q"]))
    o, lse = gpu_fwd(zq, w.causal, scale)
    v = inp["v"].double()
    if w.causal:
        ref = (torch.cumsum(v, dim=2) / torch.arange(1, w.N + 1, dtype=torch.float64)[:, None]).numpy()
        rl = np.broadcast_to(np.log(np.arange(1, w.N + 1)), lse.shape)
    else:
        ref = np.broadcast_to(v.mean(dim=2, keepdim=True).numpy(), o.shape)
        rl = np.full(lse.shape, math.log(w.N))
    rep_o, rep_l = o_report(o, ref, w.dtype), lse_report(lse, rl)
    say("  Q=0: O max_abs=%.3g lse floored_rel=%.3g" % (rep_o["max_abs"], rep_l["max_floored_rel"]))
    assert rep_o["ok"], rep_o
    assert rep_l["ok"], rep_l


def test_fwd_deterministic():
    say("determinism")
    inp = make_inputs(1, 4, 777, 128, "bf16", seed=5)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o1, l1 = attn.fwd(q, k, v, True, 0.1)
    o2, l2 = attn.fwd(q, k, v, True, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_large_and_zero_scale():
    """scale = 0 gives uniform weights; a large scale concentrates them (large logits)."""
    say("scale extremes")
    inp = make_inputs(1, 2, 200, 64, "f16", seed=9)
    for scale, causal in ((0.0, False), (0.0, True), (1.0, True), (1.0, False)):
        o, lse = gpu_fwd(inp, causal, scale)
        ro, rl = oracle_fwd(inp, causal, scale)
        check(o.reshape(2, 200, 64), lse.reshape(2, 200), ro, rl, "f16", "scale=%g causal=%d" % (scale, causal))
