"""The torch helpers of the binding check every tensor argument (device, dtype,
shape, contiguity, offsets) and raise ValueError before any call into the
library, so no host pointer or short buffer ever reaches a kernel.

The CPU cases need no GPU; the others build the mismatched tensors on the GPU
and are marked gpu (nothing is launched in them)."""
import numpy as np
import pytest
import torch

from io_aware_exact_06_amd import attn


def test_cpu_tensors_are_refused():
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        attn.fwd(q, q, q, False, 0.125)
    with pytest.raises(ValueError, match="GPU"):
        attn.bwd(q, q, q, q, q, torch.zeros(1, 2, 64), False, 0.125)
    cu = torch.tensor([0, 64], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        attn.fwd_varlen(q[0], q[0], q[0], cu, cu, 64)
    with pytest.raises(ValueError, match="GPU"):
        attn.fwd_blocksparse(q, q, q, np.ones((1, 1), np.uint8))
    with pytest.raises(ValueError, match="GPU"):
        attn.fwd_unfused(q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        attn.fwd("not a tensor", q, q)


@pytest.mark.gpu
def test_dense_mismatches_raise():
    dev = torch.device("cuda")
    B, H, N, d = 1, 2, 64, 64
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(B, H, N, dtype=torch.float32, device=dev)
    bad = {
        "k on cpu": dict(k=q.cpu()),
        "k wrong dtype": dict(k=q.half()),
        "k wrong shape": dict(k=q[:, :, :32]),
        "v not contiguous": dict(v=q.transpose(2, 3).contiguous().transpose(2, 3)),
        "o wrong dtype": dict(o=torch.empty_like(q, dtype=torch.float16)),
        "o on cpu": dict(o=q.cpu()),
        "o wrong shape": dict(o=q[:, :1].contiguous()),
        "lse on cpu": dict(lse=lse.cpu()),
        "lse wrong dtype": dict(lse=lse.double()),
        "lse wrong shape": dict(lse=lse[:, :, :10].contiguous()),
    }
    for label, kw in bad.items():
        a = dict(q=q, k=q, v=q, o=None, lse=None)
        a.update(kw)
        with pytest.raises(ValueError):
            attn.fwd(a["q"], a["k"], a["v"], False, 0.125, o=a["o"], lse=a["lse"])
    with pytest.raises(ValueError):
        attn.fwd(q.float(), q.float(), q.float())
    bad_b = {
        "lse on cpu": dict(lse=lse.cpu()),
        "lse short": dict(lse=lse[:, :, :10].contiguous()),
        "dout wrong dtype": dict(dout=q.half()),
        "o on cpu": dict(o=q.cpu()),
        "dq wrong shape": dict(dq=q[:, :, :32].contiguous()),
        "dk on cpu": dict(dk=q.cpu()),
        "dv wrong dtype": dict(dv=q.half()),
        "workspace short": dict(workspace=torch.empty(16, dtype=torch.uint8, device=dev)),
        "workspace on cpu": dict(workspace=torch.empty(1 << 12, dtype=torch.uint8)),
    }
    for label, kw in bad_b.items():
        a = dict(q=q, k=q, v=q, o=q, dout=q, lse=lse, dq=None, dk=None, dv=None, workspace=None)
        a.update(kw)
        with pytest.raises(ValueError):
            attn.bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], False, 0.125, dq=a["dq"], dk=a["dk"],
                     dv=a["dv"], workspace=a["workspace"])
    # a workspace of another element type counts its bytes, not its elements
    ws = torch.empty(attn.attn_bwd_workspace_bytes(B, H, N, d) // 4, dtype=torch.float32, device=dev)
    attn.bwd(q, q, q, q, q, lse, False, 0.125, workspace=ws)
    torch.cuda.synchronize()


@pytest.mark.gpu
def test_packed_mismatches_raise():
    dev = torch.device("cuda")
    H, tq, tk, d = 2, 100, 120, 128
    q = torch.zeros(H, tq, d, dtype=torch.float16, device=dev)
    k = torch.zeros(H, tk, d, dtype=torch.float16, device=dev)
    cu_q = torch.tensor([0, 40, tq], dtype=torch.int32, device=dev)
    cu_k = torch.tensor([0, 50, tk], dtype=torch.int32, device=dev)
    lse = torch.zeros(H, tq, dtype=torch.float32, device=dev)
    fwd_bad = [
        dict(cu_k=cu_k[:2].contiguous()),          # batch + 1 offsets expected
        dict(cu_q=cu_q.long()),
        dict(cu_k=cu_k.cpu()),
        dict(k=k[:1].contiguous()),
        dict(v=k.bfloat16()),
        dict(o=q[:, :50].contiguous()),
        dict(lse=lse.cpu()),
    ]
    for kw in fwd_bad:
        a = dict(q=q, k=k, v=k, cu_q=cu_q, cu_k=cu_k, o=None, lse=None)
        a.update(kw)
        with pytest.raises(ValueError):
            attn.fwd_varlen(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], 60, True, 0.1, o=a["o"], lse=a["lse"])
    bwd_bad = [
        dict(cu_k=cu_k[:2].contiguous()),
        dict(cu_k=cu_k.float()),
        dict(cu_k=cu_k.cpu()),
        dict(o=q[:, :50].contiguous()),
        dict(dout=q.cpu()),
        dict(lse=lse[:, :10].contiguous()),
        dict(dq=k),
        dict(dk=q),
        dict(dv=k.cpu()),
        dict(workspace=torch.empty(8, dtype=torch.uint8, device=dev)),
    ]
    for kw in bwd_bad:
        a = dict(q=q, k=k, v=k, o=q, dout=q, lse=lse, cu_q=cu_q, cu_k=cu_k, dq=None, dk=None, dv=None,
                 workspace=None)
        a.update(kw)
        with pytest.raises(ValueError):
            attn.bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["cu_q"], a["cu_k"], 60, 70,
                            True, 0.1, dq=a["dq"], dk=a["dk"], dv=a["dv"], workspace=a["workspace"])


@pytest.mark.gpu
def test_blocksparse_and_unfused_mismatches_raise():
    dev = torch.device("cuda")
    B, H, N, d = 1, 2, 200, 64
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(B, H, N, dtype=torch.float32, device=dev)
    mask = np.ones((2, 2), np.uint8)
    with pytest.raises(ValueError):
        attn.fwd_blocksparse(q, q, q, mask, o=q.cpu())
    with pytest.raises(ValueError):
        attn.fwd_blocksparse(q, q, q, mask, lse=lse.half())
    with pytest.raises(ValueError):
        attn.fwd_blocksparse(q, q, q, np.ones((3, 3), np.uint8))
    with pytest.raises(ValueError):
        attn.bwd_blocksparse(q, q, q, q, q, lse.cpu(), mask)
    with pytest.raises(ValueError):
        attn.bwd_blocksparse(q, q, q, q, q, lse, mask, dk=q[:, :1].contiguous())
    with pytest.raises(ValueError):
        attn.fwd_unfused(q, q, q, lse=lse.cpu())
    with pytest.raises(ValueError):
        attn.fwd_unfused(q, q, q, workspace=torch.empty(64, dtype=torch.uint8, device=dev))
