"""attn_bwd_noalloc (the backward whose D terms live in the library's fixed
device scratch) against attn_bwd (caller workspace), through the C ABI.

Two calls in a row, the second with a smaller problem, so the second runs on
a scratch that still holds the first call's values; both must equal attn_bwd
bit for bit (same kernels, same D).  Also at the largest size the scratch
takes, and with a negative scale."""
import sys

import pytest
import torch

from io_aware_exact_06_amd import attn
from io_aware_exact_06_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_both(B, H, N, d, dtype, causal, scale, seed):
    inp = make_inputs(B, H, N, d, dtype, seed=seed, with_dout=True)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "dout"))
    o, lse = attn.fwd(q, k, v, causal, scale)
    ref = attn.bwd(q, k, v, o, do, lse, causal, scale)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    st = attn.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                               lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal,
                               scale, attn.ATTN_BF16 if dtype == "bf16" else attn.ATTN_F16,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, attn.attn_status_string(st)
    torch.cuda.synchronize()
    return ref, (dq, dk, dv)


@pytest.mark.parametrize("first,second", [
    ((1, 4, 1000, 128, "bf16", True, 0.0884, 1), (1, 2, 300, 128, "bf16", True, 0.0884, 2)),
    ((2, 2, 777, 64, "f16", False, 0.125, 3), (1, 1, 65, 64, "f16", True, -0.125, 4)),
])
def test_noalloc_matches_workspace_call(first, second):
    for case in (first, second):
        say("noalloc vs workspace: B%d H%d N%d d%d %s causal=%d scale=%g" % case[:7])
        ref, got = run_both(*case)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a, b), name


def test_noalloc_at_its_size_limit():
    """B*H*N = 1048576 rows: the whole scratch is used."""
    case = (1, 16, attn.NOALLOC_MAX_ROWS // 16, 64, "bf16", True, 0.125, 5)
    say("noalloc at the limit: B%d H%d N%d d%d %s causal=%d scale=%g" % case[:7])
    ref, got = run_both(*case)
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a, b), name


def test_noalloc_too_large_is_refused():
    B, H, N, d = 1, 1, attn.NOALLOC_MAX_ROWS + 1, 64
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(B, H, N, dtype=torch.float32, device="cuda")
    with pytest.raises(attn.AttnError, match="TOO_LARGE"):
        attn.bwd_noalloc(q, q, q, q, q, lse, torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
