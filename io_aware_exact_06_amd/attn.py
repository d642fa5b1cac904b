"""ctypes binding of the C ABI in include/attn.h (argument marshalling only).

``attn_fwd``, ``attn_bwd``, ``attn_bwd_workspace_bytes`` and
``attn_status_string`` call the C functions of the same names with raw
integers (device pointers, sizes, a hipStream_t).  ``fwd`` and ``bwd`` are
conveniences for torch tensors: they allocate the outputs (and the backward
workspace) with torch and pass ``data_ptr()`` values and the current stream.
Every step of the computation runs in the HIP library; if the library is not
built, the first call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")
# libattn.so with the hand-scheduled loops compiled out (tests compare the two bitwise)
CSTEP_LIB_PATH = os.path.join(HERE, "libattn_cstep.so")

ATTN_F16, ATTN_BF16 = 0, 1
STATUS = {
    0: "ATTN_OK", 1: "ATTN_E_NULL", 2: "ATTN_E_SHAPE", 3: "ATTN_E_UNSUPPORTED",
    4: "ATTN_E_ALIGN", 5: "ATTN_E_ALIAS", 6: "ATTN_E_WORKSPACE", 7: "ATTN_E_HIP", 8: "ATTN_E_TOO_LARGE",
}
NOALLOC_MAX_ROWS = 1048576  # ATTN_NOALLOC_MAX_ROWS
EXPORTS = ("attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_status_string",
           "attn_fwd_varlen", "attn_bwd_varlen", "attn_bwd_varlen_workspace_bytes",
           "attn_fwd_unfused", "attn_fwd_unfused_workspace_bytes",
           "attn_fwd_blocksparse", "attn_bwd_blocksparse", "attn_bwd_noalloc")
MASK_BLOCK = 128  # ATTN_MASK_BLOCK

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, msg))
        self.status = status


def lib() -> ctypes.CDLL:
    """Open libattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = open_library(LIB_PATH)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """Open a build of the library (libattn.so or libattn_cstep.so) and declare
    the C signatures.  Raises if it has not been built."""
    if not os.path.exists(path):
        raise RuntimeError("HIP library %s is missing: build it first "
                           "(python -m io_aware_exact_06_amd.build)" % path)
    L = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_fwd.restype = i
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    L.attn_bwd.restype = i
    L.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_bwd_noalloc.restype = i
    L.attn_status_string.argtypes = [i]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, vp]
    L.attn_fwd_varlen.restype = i
    L.attn_bwd_varlen_workspace_bytes.argtypes = [i, i]
    L.attn_bwd_varlen_workspace_bytes.restype = sz
    L.attn_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i,
                                  f, i, vp, sz, vp]
    L.attn_bwd_varlen.restype = i
    L.attn_fwd_unfused_workspace_bytes.argtypes = [i, i, i]
    L.attn_fwd_unfused_workspace_bytes.restype = sz
    L.attn_fwd_unfused.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    L.attn_fwd_unfused.restype = i
    L.attn_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, vp, i, i, f, i, vp]
    L.attn_fwd_blocksparse.restype = i
    L.attn_bwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, i, i, f, i, vp, sz,
                                       vp]
    L.attn_bwd_blocksparse.restype = i
    return L


# ---- the C functions, same names, raw arguments --------------------------------

def attn_status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, stream) -> int:
    return lib().attn_fwd(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), dtype, stream)


def attn_bwd_workspace_bytes(B, H, N, d) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, H, N, d))


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, scale, dtype,
             workspace, workspace_bytes, stream) -> int:
    return lib().attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, int(causal),
                          float(scale), dtype, workspace, workspace_bytes, stream)


def attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, scale, dtype, stream) -> int:
    return lib().attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, int(causal), float(scale),
                                  dtype, stream)


def attn_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, batch, H, total_q, total_k, max_q, d, causal,
                    window_left, window_right, scale, dtype, stream) -> int:
    return lib().attn_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, batch, H, total_q, total_k, max_q, d,
                                 int(causal), window_left, window_right, float(scale), dtype, stream)


def attn_bwd_varlen_workspace_bytes(H, total_q) -> int:
    return int(lib().attn_bwd_varlen_workspace_bytes(H, total_q))


def attn_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, cu_q, cu_k, batch, H, total_q, total_k, max_q, max_k,
                    d, causal, window_left, window_right, scale, dtype, workspace, workspace_bytes,
                    stream) -> int:
    return lib().attn_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, cu_q, cu_k, batch, H, total_q, total_k,
                                 max_q, max_k, d, int(causal), window_left, window_right, float(scale), dtype,
                                 workspace, workspace_bytes, stream)


def attn_fwd_blocksparse(q, k, v, o, lse, B, H, N, d, block_mask, mask_heads, causal, scale, dtype,
                         stream) -> int:
    return lib().attn_fwd_blocksparse(q, k, v, o, lse, B, H, N, d, block_mask, mask_heads, int(causal),
                                      float(scale), dtype, stream)


def attn_bwd_blocksparse(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, block_mask, mask_heads, causal, scale,
                         dtype, workspace, workspace_bytes, stream) -> int:
    return lib().attn_bwd_blocksparse(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, block_mask, mask_heads,
                                      int(causal), float(scale), dtype, workspace, workspace_bytes, stream)


def _check(status: int):
    if status != 0:
        raise AttnError(status, attn_status_string(status))


# ---- torch conveniences ---------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_F16
    raise ValueError("q/k/v must be float16 or bfloat16, got %s" % t.dtype)


def _stream_handle(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _on_gpu(q):
    import torch
    if not isinstance(q, torch.Tensor) or q.device.type != "cuda":
        raise ValueError("q must be a tensor on a GPU device")


def _need(t, name, shape, dtype, device):
    """Raise ValueError unless t is a contiguous `dtype` tensor of `shape` on `device`."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _workspace(ws, need, device):
    """Workspace bytes of a caller-supplied contiguous device tensor (any dtype), or a new one."""
    import torch
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % device)
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError("workspace holds %d bytes, %d needed" % (nbytes, need))
    return ws, nbytes


def _shape(q, *others):
    _on_gpu(q)
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    for i, t in enumerate(others):
        _need(t, "input %d" % (i + 1), q.shape, q.dtype, q.device)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    return tuple(int(x) for x in q.shape)


def fwd(q, k, v, causal: bool = False, scale: float | None = None, o=None, lse=None):
    """O, lse = attention(q, k, v) on q's device and current stream."""
    import torch
    B, H, N, d = _shape(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _need(o, "o", q.shape, q.dtype, q.device)
    _need(lse, "lse", (B, H, N), torch.float32, q.device)
    _check(attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    B, H, N, d, causal, scale, _dtype_code(q), _stream_handle(q.device)))
    return o, lse


def bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
        dq=None, dk=None, dv=None, workspace=None):
    """dq, dk, dv of attention by recomputation, on q's device and current stream."""
    import torch
    B, H, N, d = _shape(q, k, v, o, dout)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _need(lse, "lse", (B, H, N), torch.float32, q.device)
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, name, q.shape, q.dtype, q.device)
    workspace, ws_bytes = _workspace(workspace, attn_bwd_workspace_bytes(B, H, N, d), q.device)
    _check(attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                    causal, scale, _dtype_code(q), workspace.data_ptr(), ws_bytes,
                    _stream_handle(q.device)))
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, causal: bool = False, scale: float | None = None):
    """bwd into caller-owned dq, dk, dv with no workspace: the library's fixed
    device scratch holds D (B*H*N <= NOALLOC_MAX_ROWS).  Nothing is allocated."""
    import torch
    B, H, N, d = _shape(q, k, v, o, dout)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _need(lse, "lse", (B, H, N), torch.float32, q.device)
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, name, q.shape, q.dtype, q.device)
    _check(attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal,
                            scale, _dtype_code(q), _stream_handle(q.device)))
    return dq, dk, dv


def _packed(q, k, v):
    _on_gpu(q)
    if q.dim() != 3 or not hasattr(k, "dim") or k.dim() != 3:
        raise ValueError("packed tensors are [H, total, d]")
    H, tq, d = (int(x) for x in q.shape)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _need(k, "k", (H, int(k.shape[1]), d), q.dtype, q.device)
    _need(v, "v", k.shape, q.dtype, q.device)
    return H, tq, int(k.shape[1]), d


def _cu(cu, device, name="cu_seqlens"):
    """Number of sequences described by a cumulative-offset tensor (batch + 1 int32 values)."""
    import torch
    if not (isinstance(cu, torch.Tensor) and cu.dtype == torch.int32 and cu.device == device
            and cu.dim() == 1 and cu.numel() >= 1 and cu.is_contiguous()):
        raise ValueError("%s must be a contiguous 1-D int32 tensor of batch + 1 offsets on %s" % (name, device))
    return int(cu.numel()) - 1


def fwd_varlen(q, k, v, cu_q, cu_k, max_seqlen_q: int, causal: bool = False, scale: float | None = None,
               window=(-1, -1), o=None, lse=None):
    """Packed variable-length forward: q [H, total_q, d], k, v [H, total_k, d]."""
    import torch
    H, tq, tk, d = _packed(q, k, v)
    batch = _cu(cu_q, q.device, "cu_seqlens_q")
    if _cu(cu_k, q.device, "cu_seqlens_k") != batch:
        raise ValueError("cu_seqlens_q and cu_seqlens_k describe different batch sizes")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((H, tq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "o", q.shape, q.dtype, q.device)
    _need(lse, "lse", (H, tq), torch.float32, q.device)
    _check(attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           cu_q.data_ptr(), cu_k.data_ptr(), batch, H, tq, tk, int(max_seqlen_q), d, causal,
                           int(window[0]), int(window[1]), scale, _dtype_code(q), _stream_handle(q.device)))
    return o, lse


def bwd_varlen(q, k, v, o, dout, lse, cu_q, cu_k, max_seqlen_q: int, max_seqlen_k: int, causal: bool = False,
               scale: float | None = None, window=(-1, -1), dq=None, dk=None, dv=None, workspace=None):
    """Backward of fwd_varlen: returns dq [H, total_q, d], dk, dv [H, total_k, d]."""
    import torch
    H, tq, tk, d = _packed(q, k, v)
    batch = _cu(cu_q, q.device, "cu_seqlens_q")
    if _cu(cu_k, q.device, "cu_seqlens_k") != batch:
        raise ValueError("cu_seqlens_q and cu_seqlens_k describe different batch sizes")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, name in ((o, "o"), (dout, "dout"), (dq, "dq")):
        _need(t, name, q.shape, q.dtype, q.device)
    for t, name in ((dk, "dk"), (dv, "dv")):
        _need(t, name, k.shape, q.dtype, q.device)
    _need(lse, "lse", (H, tq), torch.float32, q.device)
    workspace, ws_bytes = _workspace(workspace, attn_bwd_varlen_workspace_bytes(H, tq), q.device)
    _check(attn_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                           lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_q.data_ptr(),
                           cu_k.data_ptr(), batch, H, tq, tk, int(max_seqlen_q), int(max_seqlen_k), d, causal,
                           int(window[0]), int(window[1]), scale, _dtype_code(q), workspace.data_ptr(),
                           ws_bytes, _stream_handle(q.device)))
    return dq, dk, dv


def attn_fwd_unfused_workspace_bytes(B, H, N) -> int:
    return int(lib().attn_fwd_unfused_workspace_bytes(B, H, N))


def attn_fwd_unfused(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, workspace, workspace_bytes,
                     stream) -> int:
    return lib().attn_fwd_unfused(q, k, v, o, lse, B, H, N, d, int(causal), float(scale), dtype, workspace,
                                  workspace_bytes, stream)


def fwd_unfused(q, k, v, causal: bool = False, scale: float | None = None, o=None, lse=None, workspace=None):
    """The standard three-pass forward (S and P through device memory); same outputs as fwd."""
    import torch
    B, H, N, d = _shape(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "o", q.shape, q.dtype, q.device)
    _need(lse, "lse", (B, H, N), torch.float32, q.device)
    need = attn_fwd_unfused_workspace_bytes(B, H, N)
    if need == ctypes.c_size_t(-1).value:
        raise ValueError("the unfused baseline takes B*H <= 65535 and N <= 2^24")
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    _check(attn_fwd_unfused(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                            causal, scale, _dtype_code(q), workspace.data_ptr(), ws_bytes,
                            _stream_handle(q.device)))
    return o, lse


def _block_mask(block_mask, B, H, N, device):
    """Device uint8 copy of a [nb, nb], [H, nb, nb] or [B*H, nb, nb] block mask; returns (tensor, mask_heads)."""
    import torch
    nb = (N + MASK_BLOCK - 1) // MASK_BLOCK
    m = torch.as_tensor(block_mask)
    if m.dim() == 2:
        m = m.unsqueeze(0)
    if m.dim() != 3 or m.shape[1:] != (nb, nb) or m.shape[0] not in (1, H, B * H):
        raise ValueError("block mask must be [nb, nb], [H, nb, nb] or [B*H, nb, nb] with nb = %d" % nb)
    m = (m != 0).to(device=device, dtype=torch.uint8).contiguous()
    return m, int(m.shape[0])


def fwd_blocksparse(q, k, v, block_mask, causal: bool = False, scale: float | None = None, o=None, lse=None):
    """O, lse of attention restricted to the active 128 x 128 blocks of block_mask."""
    import torch
    B, H, N, d = _shape(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    m, mh = _block_mask(block_mask, B, H, N, q.device)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _need(o, "o", q.shape, q.dtype, q.device)
    _need(lse, "lse", (B, H, N), torch.float32, q.device)
    _check(attn_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                B, H, N, d, m.data_ptr(), mh, causal, scale, _dtype_code(q),
                                _stream_handle(q.device)))
    return o, lse


def bwd_blocksparse(q, k, v, o, dout, lse, block_mask, causal: bool = False, scale: float | None = None,
                    dq=None, dk=None, dv=None, workspace=None):
    """dq, dk, dv of block-sparse attention (same mask as the forward)."""
    import torch
    B, H, N, d = _shape(q, k, v, o, dout)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    m, mh = _block_mask(block_mask, B, H, N, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _need(lse, "lse", (B, H, N), torch.float32, q.device)
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, name, q.shape, q.dtype, q.device)
    workspace, ws_bytes = _workspace(workspace, attn_bwd_workspace_bytes(B, H, N, d), q.device)
    _check(attn_bwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d,
                                m.data_ptr(), mh, causal, scale, _dtype_code(q), workspace.data_ptr(),
                                ws_bytes, _stream_handle(q.device)))
    return dq, dk, dv
