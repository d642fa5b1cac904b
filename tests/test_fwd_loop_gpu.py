"""The forward's hand-scheduled loop over unmasked key tiles (d = 128, grids of
more than 256 work groups, so the path without the key split), against the
fp64 oracle element by element.

The loop branches out of line to raise the running maximum and to rescale the
partial output; random inputs raise it only on the first tile, so two cases
build logits whose row maximum keeps growing by more than 2^8 (in exp2 units)
from tile to tile, or jumps at a few keys inside long runs.  Sliding windows
make runs that start at odd tiles and runs of a single tile.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from io_aware_exact_06_amd import attn
from io_aware_exact_06_amd.inputs import default_scale, make_inputs
from tests.tolerance import lse_report, o_report

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_and_check(q, k, v, causal, scale, dtype, label):
    """q, k, v: [B, H, N, 128] CPU tensors of the 16-bit dtype."""
    B, H, N, d = q.shape
    o, lse = attn.fwd(q.cuda(), k.cuda(), v.cuda(), causal, scale)
    torch.cuda.synchronize()
    qd, kd, vd = (t.double().numpy().reshape(B * H, N, d) for t in (q, k, v))
    ro, rl = oracle.fwd(qd, kd, vd, causal, scale)
    rep_o = o_report(o.float().cpu().numpy().reshape(B * H, N, d), ro, dtype)
    rep_l = lse_report(lse.cpu().numpy().reshape(B * H, N), rl)
    say("%s: O max_abs=%.3g excess=%.3g | lse floored_rel=%.3g" % (
        label, rep_o["max_abs"], rep_o["worst_excess"], rep_l["max_floored_rel"]))
    assert rep_o["ok"], (label, rep_o)
    assert rep_l["ok"], (label, rep_l)


@pytest.mark.parametrize("B,H,N,dtype,causal", [
    (2, 20, 1024, "bf16", True),
    (2, 20, 1024, "f16", False),
    (2, 20, 1024, "f16", True),
    (3, 24, 777, "bf16", False),   # ragged: the last tiles go through the C++ step
    (1, 40, 700, "f16", True),
])
def test_loop_random(B, H, N, dtype, causal):
    inp = make_inputs(B, H, N, 128, dtype, seed=N + H + causal)
    run_and_check(inp["q"], inp["k"], inp["v"], causal, default_scale(128), dtype,
                  "loop B%d H%d N%d %s causal=%d" % (B, H, N, dtype, causal))


def growing_logits(H, N, dtype, spikes, seed):
    """Q, K whose logits rise with the key index: q_i = (a_i, small noise),
    k_j = (b_j, small noise).  With spikes=False, b_j = j / 2 (every 64-key tile
    raises the maximum by about 16 in exp2 units at scale 1/sqrt(128) for
    a_i near 4); with spikes=True, b_j is noise except at a few keys."""
    g = torch.Generator().manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    q = 0.05 * torch.randn(1, H, N, 128, generator=g)
    k = 0.05 * torch.randn(1, H, N, 128, generator=g)
    q[..., 0] = 1.0 + 3.0 * torch.rand(1, H, N, generator=g)
    j = torch.arange(N, dtype=torch.float32)
    if spikes:
        b = 0.3 * torch.randn(N, generator=g)
        for i, pos in enumerate((200, 520, 700, 901)):
            if pos < N:
                b[pos] = 60.0 * (i + 1)
    else:
        b = j / 2.0
    k[..., 0] = b
    v = torch.randn(1, H, N, 128, generator=g)
    return q.to(tdt), k.to(tdt), v.to(tdt)


@pytest.mark.parametrize("spikes", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_loop_growing_maximum(spikes, causal):
    dtype = "bf16" if spikes else "f16"
    q, k, v = growing_logits(40, 1024, dtype, spikes, seed=11 + spikes + 2 * causal)
    run_and_check(q, k, v, causal, default_scale(128), dtype,
                  "growing maximum spikes=%d causal=%d" % (spikes, causal))


@pytest.mark.parametrize("window", [(400, 0), (700, 300), (130, 70)])
def test_loop_sliding_window(window):
    lq = [2048, 1500, 2048]
    H, d, dtype = 16, 128, "bf16"
    tq = sum(lq)
    a = make_inputs(1, H, tq, d, dtype, seed=sum(window) + 1)
    q, k, v = a["q"][0], a["k"][0], a["v"][0]
    cu = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    scale = default_scale(d)
    tcu = torch.from_numpy(cu).cuda()
    o, lse = attn.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), tcu, tcu, max(lq), False, scale, window)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd_varlen(q.double().numpy(), k.double().numpy(), v.double().numpy(), cu, cu, False, scale,
                               window)
    rep_o = o_report(o.float().cpu().numpy(), ro, dtype)
    rep_l = lse_report(lse.cpu().numpy(), rl)
    say("window %s: O max_abs=%.3g | lse floored_rel=%.3g" % (window, rep_o["max_abs"], rep_l["max_floored_rel"]))
    assert rep_o["ok"], rep_o
    assert rep_l["ok"], rep_l


def test_loop_deterministic():
    inp = make_inputs(2, 20, 1024, 128, "bf16", seed=3)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    o1, l1 = attn.fwd(q, k, v, True, 0.09)
    o2, l2 = attn.fwd(q, k, v, True, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
