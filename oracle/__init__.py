"""fp64 CPU oracle for scaled dot-product attention (ctypes binding).

TEST INFRASTRUCTURE.  Only `tests/`, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library neither imports
nor links it, and it shares no code with the GPU path.

The C source (fa_oracle.c) computes the plain definition of attention --
full score row, two-pass softmax, weighted sum of V -- in fp64 from exactly
decoded fp16/bf16 inputs.  The definition is the scaled dot-product
attention formula of "FlashAttention-2 on Ascend NPU: how ops-transformer
reaches 3x" (2048ai.net, section 1), with the causal reading that key j is
visible to query i iff j <= i + (Sk - Sq).

The backward (attention_bwd, attention_bwd_rows) is the chain-rule
derivative of the same definition with the probability matrix materialised:
dV = P^T dO, dS = P * (dO V^T - rowsum(P * dO V^T)), dQ = scale dS K,
dK = scale dS^T Q.

attention_fwd_ext adds an explicit boolean mask and keep-and-rescale
dropout whose keep decisions come from Philox4x32-10 (philox4x32_10).

Inputs are numpy uint16 arrays holding the 16-bit patterns of the input
dtype, contiguous, shaped [B, H, S, D].
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16, BF16 = 0, 1
_DTYPES = {"f16": F16, "fp16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16,
           F16: F16, BF16: BF16}

_lib = None


def load(path: str = None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        _lib = _bind(ctypes.CDLL(_build.LIB))
    return _lib


def _bind(lib):
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.ora_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.ora_f16_to_f64.restype = ctypes.c_double
    lib.ora_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.ora_bf16_to_f64.restype = ctypes.c_double
    lib.ora_decode.argtypes = [u16p, f64p, ctypes.c_int64, ctypes.c_int]
    lib.ora_decode.restype = None
    lib.ora_max_threads.argtypes = []
    lib.ora_max_threads.restype = ctypes.c_int
    lib.ora_attention_fwd.argtypes = [u16p, u16p, u16p] + [ctypes.c_int] * 5 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, f64p, f64p, ctypes.c_int]
    lib.ora_attention_fwd.restype = ctypes.c_int
    lib.ora_attention_rows.argtypes = [u16p, u16p, u16p] + [ctypes.c_int] * 5 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, i64p, ctypes.c_int64, f64p, f64p,
        ctypes.c_int]
    lib.ora_attention_rows.restype = ctypes.c_int
    lib.ora_attention_bwd.argtypes = [u16p, u16p, u16p, u16p] + [ctypes.c_int] * 5 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, f64p, f64p, f64p, ctypes.c_int]
    lib.ora_attention_bwd.restype = ctypes.c_int
    lib.ora_attention_bwd_rows.argtypes = [u16p, u16p, u16p, u16p] + [ctypes.c_int] * 5 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, i64p, ctypes.c_int64, i64p, ctypes.c_int64,
        f64p, f64p, f64p, ctypes.c_int]
    lib.ora_attention_bwd_rows.restype = ctypes.c_int
    u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.ora_philox4x32_10.argtypes = [u32p, u32p, u32p]
    lib.ora_philox4x32_10.restype = None
    lib.ora_dropout_threshold.argtypes = [ctypes.c_float]
    lib.ora_dropout_threshold.restype = ctypes.c_int
    lib.ora_attention_fwd_ext.argtypes = [u16p, u16p, u16p] + [ctypes.c_int] * 5 + [
        ctypes.POINTER(ctypes.c_uint8), i64p, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint32,
        ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_int, i64p, ctypes.c_int64, f64p, f64p,
        ctypes.c_int]
    lib.ora_attention_fwd_ext.restype = ctypes.c_int
    lib.ora_attention_bwd_ext.argtypes = [u16p, u16p, u16p, u16p] + [ctypes.c_int] * 5 + [
        ctypes.POINTER(ctypes.c_uint8), i64p, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint32,
        ctypes.c_float, ctypes.c_int, ctypes.c_int64, ctypes.c_int, i64p, ctypes.c_int64, i64p, ctypes.c_int64,
        f64p, f64p, f64p, ctypes.c_int]
    lib.ora_attention_bwd_ext.restype = ctypes.c_int
    return lib


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are uint16 bit patterns, got %s" % a.dtype)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _f64p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def decode(bits, dtype, lib=None):
    """Exact fp64 values of an array of fp16/bf16 bit patterns."""
    lib = lib or load()
    a, p = _u16(bits)
    out = np.empty(a.shape, dtype=np.float64)
    lib.ora_decode(p, _f64p(out), a.size, _DTYPES[dtype])
    return out


def attention_fwd(q, k, v, *, scale, causal, dtype, nthreads=0, lib=None):
    """Full forward.  q: [B,H,Sq,D], k/v: [B,H,Sk,D] uint16 bit patterns.

    Returns (o [B,H,Sq,D] float64, lse [B,H,Sq] float64)."""
    lib = lib or load()
    q, qp = _u16(q)
    k, kp = _u16(k)
    v, vp = _u16(v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape != (B, H, Sk, D) or v.shape != k.shape:
        raise ValueError("shape mismatch q%s k%s v%s" % (q.shape, k.shape, v.shape))
    o = np.empty((B, H, Sq, D), dtype=np.float64)
    lse = np.empty((B, H, Sq), dtype=np.float64)
    rc = lib.ora_attention_fwd(qp, kp, vp, B, H, Sq, Sk, D, ctypes.c_float(scale),
                               int(bool(causal)), _DTYPES[dtype], _f64p(o), _f64p(lse),
                               int(nthreads))
    if rc != 0:
        raise RuntimeError("ora_attention_fwd failed with code %d" % rc)
    return o, lse


def attention_rows(q, k, v, rows, *, scale, causal, dtype, nthreads=0, lib=None):
    """Selected rows of the forward.  rows: flat ids (b*H + h)*Sq + i.

    Returns (o [n, D] float64, lse [n] float64)."""
    lib = lib or load()
    q, qp = _u16(q)
    k, kp = _u16(k)
    v, vp = _u16(v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((rows.size, D), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    rc = lib.ora_attention_rows(qp, kp, vp, B, H, Sq, Sk, D, ctypes.c_float(scale),
                                int(bool(causal)), _DTYPES[dtype],
                                rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                rows.size, _f64p(o), _f64p(lse), int(nthreads))
    if rc != 0:
        raise RuntimeError("ora_attention_rows failed with code %d" % rc)
    return o, lse


def attention_bwd(q, k, v, dout, *, scale, causal, dtype, nthreads=0, lib=None):
    """Full backward.  q, dout: [B,H,Sq,D], k/v: [B,H,Sk,D] uint16 bit patterns.

    Returns (dq [B,H,Sq,D], dk [B,H,Sk,D], dv [B,H,Sk,D]) float64: the
    gradients of sum(O * dout) with respect to q, k and v."""
    lib = lib or load()
    q, qp = _u16(q)
    k, kp = _u16(k)
    v, vp = _u16(v)
    dout, gp = _u16(dout)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape != (B, H, Sk, D) or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch q%s k%s v%s dout%s" % (q.shape, k.shape, v.shape, dout.shape))
    dq = np.empty((B, H, Sq, D), dtype=np.float64)
    dk = np.empty((B, H, Sk, D), dtype=np.float64)
    dv = np.empty((B, H, Sk, D), dtype=np.float64)
    rc = lib.ora_attention_bwd(qp, kp, vp, gp, B, H, Sq, Sk, D, ctypes.c_float(scale),
                               int(bool(causal)), _DTYPES[dtype], _f64p(dq), _f64p(dk), _f64p(dv),
                               int(nthreads))
    if rc != 0:
        raise RuntimeError("ora_attention_bwd failed with code %d" % rc)
    return dq, dk, dv


def attention_bwd_rows(q, k, v, dout, qrows, krows, *, scale, causal, dtype, nthreads=0, lib=None):
    """Selected rows of the backward.  qrows: flat query ids (b*H + h)*Sq + i
    (dQ rows); krows: flat key ids (b*H + h)*Sk + j (dK and dV rows).

    Returns (dq [nq, D], dk [nk, D], dv [nk, D]) float64."""
    lib = lib or load()
    q, qp = _u16(q)
    k, kp = _u16(k)
    v, vp = _u16(v)
    dout, gp = _u16(dout)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    qrows = np.ascontiguousarray(qrows, dtype=np.int64)
    krows = np.ascontiguousarray(krows, dtype=np.int64)
    dq = np.empty((qrows.size, D), dtype=np.float64)
    dk = np.empty((krows.size, D), dtype=np.float64)
    dv = np.empty((krows.size, D), dtype=np.float64)
    i64 = ctypes.POINTER(ctypes.c_int64)
    rc = lib.ora_attention_bwd_rows(qp, kp, vp, gp, B, H, Sq, Sk, D, ctypes.c_float(scale),
                                    int(bool(causal)), _DTYPES[dtype],
                                    qrows.ctypes.data_as(i64), qrows.size,
                                    krows.ctypes.data_as(i64), krows.size,
                                    _f64p(dq), _f64p(dk), _f64p(dv), int(nthreads))
    if rc != 0:
        raise RuntimeError("ora_attention_bwd_rows failed with code %d" % rc)
    return dq, dk, dv


def philox4x32_10(counter, key, lib=None):
    """One Philox4x32-10 block: four 32-bit counter words, two key words ->
    four 32-bit outputs."""
    lib = lib or load()
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xffffffff for x in counter])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xffffffff for x in key])
    out = (ctypes.c_uint32 * 4)()
    lib.ora_philox4x32_10(c, k, out)
    return [int(x) for x in out]


def dropout_threshold(p, lib=None):
    """t = round(p * 65536): a score is kept iff its 16-bit draw is >= t."""
    return (lib or load()).ora_dropout_threshold(ctypes.c_float(p))


def attention_fwd_ext(q, k, v, *, scale, causal, dtype, mask=None, mask_strides=None,
                      dropout_p=0.0, seed=0, offset=0, rows=None, causal_offset=None, nthreads=0, lib=None):
    """Forward with an explicit boolean mask (uint8, nonzero = keep, element
    strides (batch, head, row) in mask_strides, columns contiguous) and
    keep-and-rescale dropout.  rows: optional flat row ids.  causal_offset:
    the causal diagonal's offset c (key j visible to query i iff j <= i + c;
    None: c = Sk - Sq, bottom-right).

    Returns (o [B,H,Sq,D] or [n, D], lse [B,H,Sq] or [n]) float64."""
    lib = lib or load()
    q, qp = _u16(q)
    k, kp = _u16(k)
    v, vp = _u16(v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    mp, sp = None, None
    if mask is not None:
        mask = np.asarray(mask)
        if mask.dtype != np.uint8:
            raise TypeError("mask must be uint8")
        mask_strides = np.ascontiguousarray(mask_strides, dtype=np.int64)
        mp = mask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        sp = mask_strides.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        o = np.empty((rows.size, D), dtype=np.float64)
        lse = np.empty(rows.size, dtype=np.float64)
        rp, nr = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows.size
    else:
        o = np.empty((B, H, Sq, D), dtype=np.float64)
        lse = np.empty((B, H, Sq), dtype=np.float64)
        rp, nr = None, 0
    c = Sk - Sq if causal_offset is None else int(causal_offset)
    rc = lib.ora_attention_fwd_ext(qp, kp, vp, B, H, Sq, Sk, D, mp, sp, ctypes.c_float(dropout_p),
                                   ctypes.c_uint64(seed), ctypes.c_uint32(offset),
                                   ctypes.c_float(scale), int(bool(causal)), ctypes.c_int64(c), _DTYPES[dtype],
                                   rp, nr, _f64p(o), _f64p(lse), int(nthreads))
    if rc != 0:
        raise RuntimeError("ora_attention_fwd_ext failed with code %d" % rc)
    return o, lse


def attention_bwd_ext(q, k, v, dout, *, scale, causal, dtype, mask=None, mask_strides=None,
                      dropout_p=0.0, seed=0, offset=0, qrows=None, krows=None, causal_offset=None, nthreads=0,
                      lib=None):
    """Backward of attention_fwd_ext (gradients of sum(O * dout)).  qrows /
    krows: flat query / key row ids to return (all rows when None).
    causal_offset as for attention_fwd_ext.

    Returns (dq, dk, dv): [B,H,Sq,D], [B,H,Sk,D], [B,H,Sk,D] float64 when
    the rows are not given, else [nq, D], [nk, D], [nk, D]."""
    lib = lib or load()
    q, qp = _u16(q)
    k, kp = _u16(k)
    v, vp = _u16(v)
    dout, gp = _u16(dout)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    full = qrows is None and krows is None
    qrows = np.arange(B * H * Sq, dtype=np.int64) if qrows is None else np.ascontiguousarray(qrows, np.int64)
    krows = np.arange(B * H * Sk, dtype=np.int64) if krows is None else np.ascontiguousarray(krows, np.int64)
    mp, sp = None, None
    if mask is not None:
        mask = np.asarray(mask)
        if mask.dtype != np.uint8:
            raise TypeError("mask must be uint8")
        mask_strides = np.ascontiguousarray(mask_strides, dtype=np.int64)
        mp = mask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        sp = mask_strides.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    dq = np.empty((qrows.size, D), dtype=np.float64)
    dk = np.empty((krows.size, D), dtype=np.float64)
    dv = np.empty((krows.size, D), dtype=np.float64)
    i64 = ctypes.POINTER(ctypes.c_int64)
    c = Sk - Sq if causal_offset is None else int(causal_offset)
    rc = lib.ora_attention_bwd_ext(qp, kp, vp, gp, B, H, Sq, Sk, D, mp, sp, ctypes.c_float(dropout_p),
                                   ctypes.c_uint64(seed), ctypes.c_uint32(offset), ctypes.c_float(scale),
                                   int(bool(causal)), ctypes.c_int64(c), _DTYPES[dtype],
                                   qrows.ctypes.data_as(i64), qrows.size,
                                   krows.ctypes.data_as(i64), krows.size, _f64p(dq), _f64p(dk), _f64p(dv),
                                   int(nthreads))
    if rc != 0:
        raise RuntimeError("ora_attention_bwd_ext failed with code %d" % rc)
    if full:
        return dq.reshape(B, H, Sq, D), dk.reshape(B, H, Sk, D), dv.reshape(B, H, Sk, D)
    return dq, dk, dv


def max_threads(lib=None):
    return (lib or load()).ora_max_threads()
