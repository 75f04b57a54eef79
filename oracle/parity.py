"""Parity rule shared by the GPU tests, the smoke check and the benchmark
(test infrastructure, like the rest of this package).

Rule (per output element):  |O_gpu - O_ref| - ulp(|O_ref|)/2 <= tol, with
tol = 2e-3 for fp16 inputs and 1e-2 for bf16 inputs, O_ref the fp64 oracle.
The half-ulp term is the storage rounding of the exact result into the
output dtype, which no kernel that returns O in that dtype can avoid (at
|O| >= 4 the bf16 spacing is 2^-5, whose half alone exceeds 1e-2).  The raw
max |dO| is reported beside it.
LSE: |lse_gpu - lse_ref| <= 1e-4 * max(1, |lse_ref|).
Infinite values (lse = -inf for a row that sees no key) must match exactly;
such mismatches are counted separately because the differences they give
are not finite.
"""
import numpy as np

O_TOL = {"f16": 2e-3, "bf16": 1e-2}
LSE_RTOL = 1e-4
MANTISSA_BITS = {"f16": 10, "bf16": 7}
MIN_EXP = {"f16": -14, "bf16": -126}


def ulp(x, dtype):
    """Spacing of `dtype` in the binade holding |x| (subnormal spacing below it)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, MIN_EXP[dtype])
    return np.exp2(e - MANTISSA_BITS[dtype])


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype):
    """Return a dict of error statistics (no assertion)."""
    with np.errstate(invalid="ignore"):      # inf - inf where both sides are -inf
        return _compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype)


def _compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    d = np.abs(o_gpu - o_ref)
    net = d - 0.5 * ulp(o_ref, dtype)
    st = {
        "max_abs": float(np.nanmax(d)) if d.size else 0.0,
        "max_ulp_net": float(np.nanmax(net)) if d.size else 0.0,
        "nan": int(np.isnan(o_gpu).sum()),
        "o_tol": O_TOL[dtype],
    }
    if lse_gpu is not None and lse_ref is not None:
        lg = np.asarray(lse_gpu, dtype=np.float64)
        lr = np.asarray(lse_ref, dtype=np.float64)
        dl = np.abs(lg - lr)
        st["lse_max_abs"] = float(np.nanmax(dl)) if dl.size else 0.0
        st["lse_max_scaled"] = float(np.nanmax(dl / np.maximum(1.0, np.abs(lr)))) if dl.size else 0.0
        st["lse_nan"] = int(np.isnan(lg).sum())
        st["lse_inf_mismatch"] = int(((np.isinf(lg) | np.isinf(lr)) & (lg != lr)).sum())
    st["inf_mismatch"] = int(((np.isinf(o_gpu) | np.isinf(o_ref)) & (o_gpu != o_ref)).sum())
    return st


def ok(st):
    good = st["nan"] == 0 and st["inf_mismatch"] == 0 and st["max_ulp_net"] <= st["o_tol"]
    if "lse_max_scaled" in st:
        good = good and st["lse_nan"] == 0 and st["lse_inf_mismatch"] == 0 and \
            st["lse_max_scaled"] <= LSE_RTOL
    return good


def assert_parity(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    st = compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype)
    assert ok(st), "parity failed %s: %s" % (what, st)
    return st
