"""Acceptance checks of GPU results against the fp64 oracle.

* O:   element-wise |O_gpu - O_ref| <= tol + ulp(O_ref)/2, tol = 2e-3 (fp16) or
       1e-2 (bf16).  The half-ulp term is the rounding of the exact result to
       the storage dtype, which alone can exceed the bare bound where |O| is
       large (bf16 half-ulp is 0.0156 in [4, 8)).
* lse: |lse_gpu - lse_ref| / max(1, |lse_ref|) <= 1e-4.
* dQ, dK, dV: relative L2 error ||x - x_ref|| / ||x_ref|| <= 1e-2 per tensor.
"""
import numpy as np

O_TOL = {"f16": 2e-3, "bf16": 1e-2}
LSE_TOL = 1e-4
GRAD_TOL = 1e-2
_MANT = {"f16": 10, "bf16": 7}
_EMIN = {"f16": -14, "bf16": -126}


def half_ulp(x, dtype: str):
    """Half the spacing of `dtype` values around |x| (subnormals included)."""
    ax = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(ax, 1e-300)))
    e = np.maximum(e, _EMIN[dtype])
    return np.ldexp(1.0, (e - _MANT[dtype] - 1).astype(np.int64))


def o_report(o_gpu, o_ref, dtype: str) -> dict:
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    err = np.abs(o_gpu - o_ref)
    bound = O_TOL[dtype] + half_ulp(o_ref, dtype)
    finite = bool(np.isfinite(o_gpu).all())
    return {
        "max_abs": float(err.max()) if err.size else 0.0,
        "worst_excess": float((err - bound).max()) if err.size else -1.0,
        "n_halfulp_ge_tol": int((half_ulp(o_ref, dtype) >= O_TOL[dtype]).sum()),
        "ok": finite and (err.size == 0 or bool((err <= bound).all())),
    }


def lse_report(l_gpu, l_ref) -> dict:
    l_gpu = np.asarray(l_gpu, np.float64)
    l_ref = np.asarray(l_ref, np.float64)
    err = np.abs(l_gpu - l_ref)
    floored = err / np.maximum(1.0, np.abs(l_ref))
    rel = err / np.maximum(np.abs(l_ref), 1e-300)
    return {
        "max_floored_rel": float(floored.max()) if err.size else 0.0,
        "max_rel": float(rel.max()) if err.size else 0.0,
        "ok": bool(np.isfinite(l_gpu).all()) and (err.size == 0 or float(floored.max()) <= LSE_TOL),
    }


def rel_l2(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if not np.isfinite(x).all():
        return float("inf")
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))
