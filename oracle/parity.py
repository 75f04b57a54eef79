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

Gradients (dQ, dK, dV of the backward), per (batch, head) slice G of each:
  max_e (|G_gpu - G_ref| - ulp(|G_ref|)/2) <= 3 u max|G_ref|   and
  rms(G_gpu - G_ref) <= 2 u rms(G_ref),
with u the unit roundoff of the input dtype (2^-8 for bf16, 2^-11 for fp16).
Each gradient is a sum of products in which one factor (the recomputed
probability P or the score gradient dS) is rounded to the input dtype before
the fp32-accumulated product, a relative perturbation of at most u per term;
an fp32 emulation of that rounding on N(0,1) inputs gives a largest error of
about 1.25 u max|G| and an rms error of about 0.6 u rms(G).  A slice whose
reference is all zero has no magnitude to be relative to.  Its zeros come
either from visibility (no key seen: exactly zero on both sides) or from
cancellation (one visible key: dS = P (dP - D_i) with dP = D_i = dO . v in
exact arithmetic).  For the latter the caller passes `zero_tol`, an absolute
bound from cancellation_tolerances(): the two fp32 dot products of D exact
terms (dP on the matrix cores, D_i from dO and the stored O) differ by at
most 2 D 2^-24 sum_d |dO_d v_d|, and with dropout the stored O is
keep_scale * v rounded to the input dtype, which adds u keep_scale
sum_d |dO_d v_d|.  Without `zero_tol` the slice must be exactly zero.
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
        # the error over the entries where both sides are finite (rows that
        # see no key have lse = -inf on both sides; a one-sided infinity is
        # counted below as a mismatch, a NaN as a NaN)
        both = np.isfinite(lg) & np.isfinite(lr)
        dl = np.abs(lg - lr)[both]
        st["lse_max_abs"] = float(np.max(dl)) if dl.size else 0.0
        st["lse_max_scaled"] = float(np.max(dl / np.maximum(1.0, np.abs(lr[both])))) if dl.size else 0.0
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


GRAD_U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
GRAD_MAX_C = 3.0
GRAD_RMS_C = 2.0


def cancellation_tolerances(q, k, v, dout, scale, dtype, dropout_p=0.0):
    """Absolute bounds for gradient slices that cancel to zero (see the module
    text): {"dq", "dk", "dv"} from the inputs (CPU tensors or arrays
    [B, H, S, D]).  dV has no cancellation (its zero slices are exact)."""
    as64 = lambda t: np.abs(np.asarray(t.float().numpy() if hasattr(t, "float") else t, dtype=np.float64))
    qa, ka, va, ga = as64(q), as64(k), as64(v), as64(dout)
    D = qa.shape[-1]
    # largest sum_d |dO_id v_jd| over all query/key pairs of a head
    dot = float(np.max(np.matmul(ga, np.swapaxes(va, -1, -2)))) if ga.size and va.size else 0.0
    t = round(dropout_p * 65536.0)
    keep_scale = 65536.0 / (65536.0 - t)
    rel = 2.0 * D * 2.0 ** -24 + (GRAD_U[dtype] if t else 0.0)
    ds = rel * keep_scale * dot          # bound on |dS| for a row with one visible key (P <= 1)
    return {"dq": scale * ds * float(np.max(ka)), "dk": scale * ds * float(np.max(qa)), "dv": 0.0}


def compare_grad(g_gpu, g_ref, dtype, zero_tol=None):
    """Error statistics of one gradient tensor [..., rows, D], per leading slice."""
    g_gpu = np.asarray(g_gpu, dtype=np.float64)
    g_ref = np.asarray(g_ref, dtype=np.float64)
    lead = g_ref.shape[:-2] if g_ref.ndim > 2 else ()
    gg = g_gpu.reshape((-1,) + g_gpu.shape[-2:]) if lead else g_gpu[None]
    gr = g_ref.reshape((-1,) + g_ref.shape[-2:]) if lead else g_ref[None]
    u = GRAD_U[dtype]
    worst_max, worst_rms = 0.0, 0.0
    nan = int(np.isnan(gg).sum()) + int(np.isinf(gg).sum())
    zero_bad = 0
    for a, r in zip(gg, gr):
        d = np.abs(a - r)
        m = float(np.max(np.abs(r))) if r.size else 0.0
        rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
        if m == 0.0:
            if not zero_tol:
                zero_bad += int(np.count_nonzero(a))
            else:
                zero_bad += int(np.count_nonzero(np.abs(a) > zero_tol))
            continue
        net = float(np.max(d - 0.5 * ulp(r, dtype)))
        worst_max = max(worst_max, net / (u * m))
        worst_rms = max(worst_rms, float(np.sqrt(np.mean(d * d))) / (u * rms))
    return {"max_in_u": worst_max, "rms_in_u": worst_rms, "nan_or_inf": nan,
            "nonzero_where_zero": zero_bad}


def grad_ok(st):
    return (st["nan_or_inf"] == 0 and st["nonzero_where_zero"] == 0
            and st["max_in_u"] <= GRAD_MAX_C and st["rms_in_u"] <= GRAD_RMS_C)


def assert_grad_parity(g_gpu, g_ref, dtype, what="", zero_tol=None):
    st = compare_grad(g_gpu, g_ref, dtype, zero_tol)
    assert grad_ok(st), "gradient parity failed %s: %s" % (what, st)
    return st


def operand_rounding_bounds(q, k, v, dout, o, lse, scale, causal, dtype, vis=None, zc=None):
    """Per-element absolute bounds on the gradients' error, for inputs whose
    gradients cancel far below the size of their terms (where the slice-wide
    rule above, calibrated on N(0,1) inputs and many visible keys per row,
    does not apply).  Same model: each product takes one factor rounded to
    the input dtype (dS for dQ and dK, P for dV; relative error u); the
    recomputed P carries the fp32 error of its score and of the stored lse,
        e_ij = (D + 2) 2^-24 scale sum_d |q_id k_jd| + 4 * 2^-24 max(1, |lse_i|);
    and D_i = dO_i . O_i is formed from the stored output, rounded to the
    dtype and carrying the forward's own rounding of P,
        dO_id = ulp(O_id)/2 + 2 u sum_j P_ij zc_ij |v_jd|,
        dD_i  = sum_d |dO_id| dO_id + (D + 2) 2^-24 sum_d |dO_id O_id|
    (dO_id here the error of O, beside the output gradient dO_id).  Both
    reach dS = P (zc dP - D_i), zc the dropout's keep-and-rescale factor
    (1 without dropout).  With
        w_ij = u |dS_ij| + e_ij P_ij |zc_ij dP_ij - D_i| + P_ij dD_i:
        dQ_id <= scale sum_j w_ij |k_jd|,   dK_jd <= scale sum_i w_ij |q_id|,
        dV_jd <= sum_i (u + e_ij) P_ij zc_ij |dO_id|.
    P, dP, D_i and dS are recomputed here in fp64 from the inputs and the
    oracle's O and lse.  vis: optional boolean [.., Sq, Sk] visibility (an
    explicit mask combined with the causal rule; when None, the
    bottom-right causal rule if `causal`); zc: optional [.., Sq, Sk] keep
    factors.  Inputs [B, H, S, D]; returns {"dq", "dk", "dv"} arrays shaped
    like the gradients."""
    as64 = lambda t: np.asarray(t.float().numpy() if hasattr(t, "float") else t, dtype=np.float64)
    qa, ka, va, ga = as64(q), as64(k), as64(v), as64(dout)
    oa = np.asarray(o, dtype=np.float64)
    la = np.asarray(lse, dtype=np.float64)
    Sq, Sk, D = qa.shape[-2], ka.shape[-2], qa.shape[-1]
    kt = np.swapaxes(ka, -1, -2)
    s = scale * np.matmul(qa, kt)
    if vis is None and causal:
        vis = np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] + (Sk - Sq)
    if vis is not None:
        s = np.where(vis, s, -np.inf)
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.where(np.isneginf(s), 0.0, np.exp(s - la[..., None]))
    p = np.nan_to_num(p, nan=0.0)
    z = 1.0 if zc is None else np.asarray(zc, dtype=np.float64)
    dp = np.matmul(ga, np.swapaxes(va, -1, -2))
    di = np.sum(p * z * dp, axis=-1, keepdims=True)
    ds = p * (z * dp - di)
    u = GRAD_U[dtype]
    e = (D + 2) * 2.0 ** -24 * scale * np.matmul(np.abs(qa), np.abs(kt)) + \
        4 * 2.0 ** -24 * np.maximum(1.0, np.abs(np.nan_to_num(la, neginf=0.0)))[..., None]
    o_err = 0.5 * ulp(oa, dtype) + 2.0 * u * np.matmul(p * z, np.abs(va))
    d_err = np.sum(np.abs(ga) * o_err, axis=-1, keepdims=True) + \
        (D + 2) * 2.0 ** -24 * np.sum(np.abs(ga * oa), axis=-1, keepdims=True)
    w = u * np.abs(ds) + e * p * np.abs(z * dp - di) + p * d_err
    return {"dq": scale * np.matmul(w, np.abs(ka)),
            "dk": scale * np.matmul(np.swapaxes(w, -1, -2), np.abs(qa)),
            "dv": np.matmul(np.swapaxes((u + e) * p * z, -1, -2), np.abs(ga))}


def assert_grad_within_bound(g_gpu, g_ref, bound, dtype, what=""):
    """|G_gpu - G_ref| <= 2 bound + 3 u max|G_ref| (per (batch, head) slice)
    plus half an output ulp, elementwise, and no NaN or infinity."""
    g = np.asarray(g_gpu, dtype=np.float64)
    r = np.asarray(g_ref, dtype=np.float64)
    b = np.asarray(bound, dtype=np.float64)
    assert np.isfinite(g).all(), "non-finite gradient %s" % what
    u = GRAD_U[dtype]
    m = np.max(np.abs(r), axis=(-2, -1), keepdims=True)
    excess = np.abs(g - r) - 0.5 * ulp(r, dtype) - (2.0 * b + GRAD_MAX_C * u * m)
    worst = float(np.max(excess))
    ratio = float(np.max(np.abs(g - r) / (2.0 * b + GRAD_MAX_C * u * m + 0.5 * ulp(r, dtype) + 1e-300)))
    assert worst <= 0.0, "gradient beyond its rounding bound %s: worst excess %.3e, ratio %.3f" % (what, worst, ratio)
    return {"ratio_to_bound": ratio}
