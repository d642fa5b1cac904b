"""The library's entry points captured in a HIP graph and replayed.

A forward and a backward step (dense d = 128, causal, a grid large enough for
the hand-scheduled loops) is captured once with every output and the
workspace allocated beforehand, then replayed three times, each time on new
input values copied into the captured buffers.  Eager calls and
synchronisations run between the replays, and each replay must reproduce the
eager results on the same inputs bit for bit.  The backward is captured both
through attn_bwd (caller workspace) and attn_bwd_noalloc (the library's fixed
scratch, the entry point meant for callers that cannot allocate).
"""
import sys

import pytest
import torch

from io_aware_exact_06_amd import attn
from io_aware_exact_06_amd.inputs import default_scale, make_inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("noalloc", [False, True])
def test_capture_and_replay(noalloc):
    B, H, N, d, dtype, causal = 2, 20, 1024, 128, "bf16", True
    scale = default_scale(d)
    dev = torch.device("cuda:0")
    inp = [make_inputs(B, H, N, d, dtype, seed=500 + 10 * r + noalloc, with_dout=True) for r in range(4)]
    q, k, v, do = (inp[0][n].to(dev) for n in ("q", "k", "v", "dout"))
    o, lse = torch.empty_like(q), torch.empty(B, H, N, device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(max(attn.attn_bwd_workspace_bytes(B, H, N, d), 1), dtype=torch.uint8, device=dev)

    def step():
        attn.fwd(q, k, v, causal, scale, o=o, lse=lse)
        if noalloc:
            attn.bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, causal, scale)
        else:
            attn.bwd(q, k, v, o, do, lse, causal, scale, dq=dq, dk=dk, dv=dv, workspace=ws)

    def eager(x):
        qq, kk, vv, dd = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
        oo, ll = attn.fwd(qq, kk, vv, causal, scale)
        g = attn.bwd(qq, kk, vv, oo, dd, ll, causal, scale)
        return [oo, ll] + list(g)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(1, 4):
        for name, t in (("q", q), ("k", k), ("v", v), ("dout", do)):
            t.copy_(inp[r][name].to(dev))
        ref = eager(inp[r])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o, lse, dq, dk, dv]
        diff = [n for n, a, b in zip(("O", "lse", "dQ", "dK", "dV"), got, ref) if not torch.equal(a, b)]
        say("replay %d (noalloc=%d): %s" % (r, noalloc, "bitwise equal to eager" if not diff else "differs in " + ", ".join(diff)))
        assert not diff, (r, diff)
