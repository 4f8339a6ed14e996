"""Comparison rules between a GPU result and the fp64 oracle -- TEST INFRASTRUCTURE.

Tolerances for bf16 outputs of attention and merge: max |gpu - oracle| <= 8e-3
and cosine similarity >= 0.99999 over the compared set; LSE: max abs error
<= 1e-3.  The pages' own check of their sequence-parallel attention against
full attention reached 0.004 max error and cosine > 0.99999 in bf16
("feat: support Ascend NPU backend ... #274", verification table), which these
bounds sit next to.

Prologue outputs reach |z| ~ 7, where one bf16 rounding alone can exceed
8e-3 (half an ulp is 1.56e-2 at |z| in [4, 8)).  For them each element must
satisfy |gpu - oracle| <= max(8e-3, ulp_bf16(oracle)), plus the cosine bound.
"""
from __future__ import annotations

import numpy as np

ATOL = 8e-3
COS_MIN = 0.99999
LSE_ATOL = 1e-3


def cosine(a, b) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0.0 and nb == 0.0:
        return 1.0
    if na == 0.0 or nb == 0.0:
        return 0.0
    return float(np.dot(a, b) / (na * nb))


def ulp_bf16(x) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.exp2(e - 7)


def attn_report(out, ref, lse=None, ref_lse=None, bf16: bool = True) -> dict:
    """Attention / merge outputs.  The 8e-3 bound applies literally, except
    for bf16 outputs where |oracle| >= 4: there half a bf16 ulp is 1.56e-2 and
    no bf16 value can be within 8e-3, so those elements (counted in
    ``n_ulp_rule``) must be within max(8e-3, ulp_bf16(oracle))."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if out.shape != ref.shape:
        raise ValueError(f"shape {out.shape} vs {ref.shape}")
    err = np.abs(out - ref)
    big = (np.abs(ref) >= 4.0) if bf16 else np.zeros(ref.shape, dtype=bool)
    small_err = err[~big]
    r = {
        "max_abs": float(err.max()) if out.size else 0.0,
        "max_abs_below_4": float(small_err.max()) if small_err.size else 0.0,
        "n_ulp_rule": int(big.sum()),
        "cos": cosine(out, ref),
        "finite": bool(np.isfinite(out).all()),
    }
    ok = r["finite"] and r["max_abs_below_4"] <= ATOL and r["cos"] >= COS_MIN
    if big.any():
        ok = ok and bool((err[big] <= np.maximum(ATOL, ulp_bf16(ref[big]))).all())
    if lse is not None:
        lse = np.asarray(lse, dtype=np.float64)
        ref_lse = np.asarray(ref_lse, dtype=np.float64)
        r["lse_err"] = float(np.abs(lse - ref_lse).max()) if lse.size else 0.0
        ok = ok and bool(np.isfinite(lse).all()) and r["lse_err"] <= LSE_ATOL
    r["ok"] = bool(ok)
    return r


def prologue_report(out, ref) -> dict:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(out - ref)
    bound = np.maximum(ATOL, ulp_bf16(ref))
    r = {
        "max_abs": float(err.max()),
        "n_above_atol": int((err > ATOL).sum()),
        "max_err_over_bound": float((err / bound).max()),
        "cos": cosine(out, ref),
    }
    r["ok"] = bool(np.isfinite(out).all() and r["max_err_over_bound"] <= 1.0 and r["cos"] >= COS_MIN)
    return r


def assert_ok(report: dict, what: str = ""):
    assert report["ok"], f"{what} parity failed: {report}"
