"""Fused attention forward for AMD MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI in include/fa.h (libfa_hip.so, built from
csrc/ by build.py).  The functions named after the ABI entry points only
marshal arguments; every step of the computation runs in the HIP kernels.
PyTorch is used for device memory and streams only.

There is no fallback: if the HIP library is missing or cannot be loaded,
every call raises.
"""
import ctypes
import math
import os

__all__ = ["FaError", "fa_fwd", "fa_fwd_strided", "fa_fwd_plan", "fa_naive_fwd",
           "fa_naive_workspace_bytes", "fa_status_string", "fa_version", "forward",
           "naive_forward", "library_path", "F16", "BF16", "STATUS", "fa_bwd",
           "fa_bwd_workspace_bytes", "backward", "fa_fwd_ext", "forward_ext", "fa_bwd_ext",
           "backward_ext", "fa_bwd_strided", "fa_fwd_ext_strided", "fa_fwd_diag",
           "fa_fwd_diag_tile_slots", "DIAG_REVERSE_ORDER", "fa_clock_stamps", "clock_stamps",
           "clock_mhz", "fa_bwd_noalloc", "fa_bwd_noalloc_scratch_bytes"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfa_hip.so")

F16, BF16 = 0, 1
DIAG_REVERSE_ORDER = 1
STATUS = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED",
          4: "FA_ERR_ALIGN", 5: "FA_ERR_SCALE", 6: "FA_ERR_HIP", 7: "FA_ERR_ALIAS",
          8: "FA_ERR_STRIDE", 9: "FA_ERR_MASK_DROPOUT", 10: "FA_ERR_SCRATCH"}

_lib = None


class FaError(RuntimeError):
    def __init__(self, status, where="fa_fwd"):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, STATUS.get(status, status),
                                                 fa_status_string(status)))


def library_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("HIP library %s is not built; run tiled_attention_15_amd/build.py "
                          "(or __graft_entry__.build())" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    i64p = ctypes.POINTER(ctypes.c_int64)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.fa_fwd_plan.argtypes = [i, i, i, i, i, i, ip, ip, i64p, i64p]
    lib.fa_fwd_plan.restype = i
    lib.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i64p, i64p, i64p, i64p,
                                   f, i, i, vp]
    lib.fa_fwd_strided.restype = i
    lib.fa_naive_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, ctypes.c_int64, vp]
    lib.fa_naive_fwd.restype = i
    lib.fa_naive_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_naive_workspace_bytes.restype = ctypes.c_int64
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp,
                           ctypes.c_int64, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_int64
    lib.fa_fwd_ext.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, i64p, f, ctypes.c_uint64,
                               ctypes.c_uint32, f, i, i, vp]
    lib.fa_fwd_ext.restype = i
    lib.fa_bwd_ext.argtypes = [vp] * 9 + [i] * 5 + [vp, i64p, f, ctypes.c_uint64, ctypes.c_uint32, f, i, i,
                                                     vp, ctypes.c_int64, vp]
    lib.fa_bwd_ext.restype = i
    lib.fa_bwd_strided.argtypes = [vp] * 9 + [i] * 5 + [i64p, vp, i64p, f, ctypes.c_uint64, ctypes.c_uint32, f,
                                                         i, i, i, vp, ctypes.c_int64, vp]
    lib.fa_bwd_strided.restype = i
    lib.fa_fwd_ext_strided.argtypes = [vp] * 5 + [i] * 5 + [i64p, vp, i64p, f, ctypes.c_uint64, ctypes.c_uint32, f,
                                                             i, i, vp]
    lib.fa_fwd_ext_strided.restype = i
    lib.fa_fwd_causal_offset.argtypes = [vp] * 5 + [i] * 5 + [i64p, vp, i64p, f, ctypes.c_uint64, ctypes.c_uint32,
                                                               f, ctypes.c_int64, i, vp]
    lib.fa_fwd_causal_offset.restype = i
    lib.fa_bwd_causal_offset.argtypes = [vp] * 9 + [i] * 5 + [i64p, vp, i64p, f, ctypes.c_uint64, ctypes.c_uint32,
                                                               f, ctypes.c_int64, i, vp, ctypes.c_int64, vp]
    lib.fa_bwd_causal_offset.restype = i
    lib.fa_fwd_diag.argtypes = [vp] * 7 + [i] * 5 + [f, i, i, i, vp]
    lib.fa_fwd_diag.restype = i
    lib.fa_fwd_diag_tile_slots.argtypes = [i] * 5
    lib.fa_fwd_diag_tile_slots.restype = ctypes.c_int64
    lib.fa_clock_stamps.argtypes = [vp, i, vp]
    lib.fa_clock_stamps.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp] * 9 + [i] * 5 + [f, i, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc_scratch_bytes.argtypes = []
    lib.fa_bwd_noalloc_scratch_bytes.restype = ctypes.c_int64
    _lib = lib
    return lib


def _ptr(x):
    """A device address from an int, None or a tensor (its data_ptr)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr() or None


def _stream(s):
    """A hipStream_t from None, an int handle or a torch stream."""
    if s is None or isinstance(s, int):
        return s or None
    return s.cuda_stream or None


def fa_fwd(q, k, v, o, lse, B, H, S, D, scale, causal, dtype, stream):
    """The ABI call fa_fwd; pointers may be ints or tensors.  Returns the status."""
    return _load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(S),
                          int(D), ctypes.c_float(scale), int(bool(causal)), int(dtype),
                          _stream(stream))


def fa_fwd_diag(q, k, v, o, lse, o32, tile_counts, B, H, Sq, Sk, D, scale, causal, dtype, flags, stream):
    """The ABI call fa_fwd_diag (test-only diagnostic launch).  Returns the status."""
    return _load().fa_fwd_diag(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(o32), _ptr(tile_counts),
                               int(B), int(H), int(Sq), int(Sk), int(D), ctypes.c_float(scale),
                               int(bool(causal)), int(dtype), int(flags), _stream(stream))


def fa_fwd_diag_tile_slots(B, H, Sq, D, causal):
    return _load().fa_fwd_diag_tile_slots(int(B), int(H), int(Sq), int(D), int(bool(causal)))


def fa_clock_stamps(out, groups, stream):
    """The ABI call fa_clock_stamps.  Returns the status."""
    return _load().fa_clock_stamps(_ptr(out), int(groups), _stream(stream))


def clock_stamps(device=None, stream=None, groups=512):
    """Enqueue fa_clock_stamps on `stream` (default: torch's current stream)
    into a new int64 tensor [groups, 4]; read it after synchronising."""
    import torch
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    out = torch.empty((groups, 4), dtype=torch.int64, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    st = fa_clock_stamps(out, groups, stream)
    if st != 0:
        raise FaError(st, "fa_clock_stamps")
    return out


def clock_mhz(before, after):
    """Average shader clock per XCD between two clock_stamps() results (CPU
    or device tensors, read after the work between them has finished):
    {xcd: MHz}.  Uses, per XCD, the mean counters of its workgroups."""
    import numpy as np
    a = before.cpu().numpy().astype(np.float64)
    b = after.cpu().numpy().astype(np.float64)
    out = {}
    for x in sorted(set(a[:, 0].astype(int)) & set(b[:, 0].astype(int))):
        ra, rb = a[a[:, 0] == x], b[b[:, 0] == x]
        dt = rb[:, 1].mean() - ra[:, 1].mean()
        dr = rb[:, 2].mean() - ra[:, 2].mean()
        if dr > 0:
            out[int(x)] = dt / dr * 100.0
    return out


def _strides3(st):
    a = (ctypes.c_int64 * 3)(*[int(x) for x in st])
    return a


def fa_fwd_strided(q, k, v, o, lse, B, H, Sq, Sk, D, q_strides, k_strides, v_strides, o_strides,
                   scale, causal, dtype, stream):
    """The ABI call fa_fwd_strided; strides are 3-sequences of element strides
    (batch, head, row).  Returns the status."""
    return _load().fa_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                  int(Sq), int(Sk), int(D), _strides3(q_strides),
                                  _strides3(k_strides), _strides3(v_strides),
                                  _strides3(o_strides), ctypes.c_float(scale),
                                  int(bool(causal)), int(dtype), _stream(stream))


def fa_naive_fwd(q, k, v, o, lse, B, H, S, D, scale, causal, dtype, workspace, workspace_bytes,
                 stream):
    """The ABI call fa_naive_fwd (the unfused comparison path).  Returns the status."""
    return _load().fa_naive_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                int(S), int(D), ctypes.c_float(scale), int(bool(causal)),
                                int(dtype), _ptr(workspace), int(workspace_bytes),
                                _stream(stream))


def fa_naive_workspace_bytes(B, H, S, D):
    return _load().fa_naive_workspace_bytes(int(B), int(H), int(S), int(D))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Sq, Sk, D, scale, causal, dtype, deterministic,
           workspace, workspace_bytes, stream):
    """C ABI fa_bwd: gradients dq, dk, dv of the forward given dout
    (`deterministic` is passed through; the library ignores it)."""
    return _load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                          _ptr(dk), _ptr(dv), B, H, Sq, Sk, D, float(scale), int(bool(causal)),
                          int(dtype), int(bool(deterministic)), _ptr(workspace),
                          int(workspace_bytes), _stream(stream))


def fa_fwd_ext(q, k, v, o, lse, B, H, Sq, Sk, D, mask, mask_strides, dropout_p, seed, offset,
               scale, causal, dtype, stream):
    """C ABI fa_fwd_ext: the forward with an explicit boolean mask and/or dropout."""
    ms = None if mask_strides is None else _strides3(mask_strides)
    return _load().fa_fwd_ext(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Sq),
                              int(Sk), int(D), _ptr(mask), ms, ctypes.c_float(dropout_p),
                              ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
                              ctypes.c_uint32(int(offset) & 0xFFFFFFFF), ctypes.c_float(scale),
                              int(bool(causal)), int(dtype), _stream(stream))


def fa_fwd_ext_strided(q, k, v, o, lse, B, H, Sq, Sk, D, strides, mask, mask_strides, dropout_p, seed, offset,
                       scale, causal, dtype, stream):
    """C ABI fa_fwd_ext_strided: strides is a sequence of 12 element strides
    (batch, head, row of q, k, v, o)."""
    st = [int(x) for x in strides]
    if len(st) != 12:
        raise ValueError("fa: fa_fwd_ext_strided takes 12 strides")
    ms = None if mask_strides is None else _strides3(mask_strides)
    return _load().fa_fwd_ext_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Sq),
                                      int(Sk), int(D), (ctypes.c_int64 * 12)(*st), _ptr(mask), ms,
                                      ctypes.c_float(dropout_p), ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
                                      ctypes.c_uint32(int(offset) & 0xFFFFFFFF), ctypes.c_float(scale),
                                      int(bool(causal)), int(dtype), _stream(stream))


def fa_bwd_ext(q, k, v, o, dout, lse, dq, dk, dv, B, H, Sq, Sk, D, mask, mask_strides, dropout_p, seed,
               offset, scale, causal, dtype, workspace, workspace_bytes, stream):
    """C ABI fa_bwd_ext: gradients of the masked / dropout forward."""
    ms = None if mask_strides is None else _strides3(mask_strides)
    return _load().fa_bwd_ext(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                              _ptr(dk), _ptr(dv), int(B), int(H), int(Sq), int(Sk), int(D), _ptr(mask), ms,
                              ctypes.c_float(dropout_p), ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
                              ctypes.c_uint32(int(offset) & 0xFFFFFFFF), ctypes.c_float(scale),
                              int(bool(causal)), int(dtype), _ptr(workspace), int(workspace_bytes),
                              _stream(stream))


def fa_bwd_strided(q, k, v, o, dout, lse, dq, dk, dv, B, H, Sq, Sk, D, strides, mask, mask_strides,
                   dropout_p, seed, offset, scale, causal, dtype, deterministic, workspace, workspace_bytes,
                   stream):
    """C ABI fa_bwd_strided: strides is a sequence of 24 element strides
    (batch, head, row of q, k, v, o, dout, dq, dk, dv)."""
    st = [int(x) for x in strides]
    if len(st) != 24:
        raise ValueError("fa: fa_bwd_strided takes 24 strides")
    ms = None if mask_strides is None else _strides3(mask_strides)
    return _load().fa_bwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                  _ptr(dk), _ptr(dv), int(B), int(H), int(Sq), int(Sk), int(D),
                                  (ctypes.c_int64 * 24)(*st), _ptr(mask), ms, ctypes.c_float(dropout_p),
                                  ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
                                  ctypes.c_uint32(int(offset) & 0xFFFFFFFF), ctypes.c_float(scale),
                                  int(bool(causal)), int(dtype), int(bool(deterministic)), _ptr(workspace),
                                  int(workspace_bytes), _stream(stream))


def fa_fwd_causal_offset(q, k, v, o, lse, B, H, Sq, Sk, D, strides, mask, mask_strides, dropout_p, seed, offset,
                         scale, causal_offset, dtype, stream):
    """C ABI fa_fwd_causal_offset: fa_fwd_ext_strided under the causal rule
    with key j visible to query i iff j <= i + causal_offset."""
    st = [int(x) for x in strides]
    if len(st) != 12:
        raise ValueError("fa: fa_fwd_causal_offset takes 12 strides")
    ms = None if mask_strides is None else _strides3(mask_strides)
    return _load().fa_fwd_causal_offset(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Sq),
                                        int(Sk), int(D), (ctypes.c_int64 * 12)(*st), _ptr(mask), ms,
                                        ctypes.c_float(dropout_p), ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
                                        ctypes.c_uint32(int(offset) & 0xFFFFFFFF), ctypes.c_float(scale),
                                        ctypes.c_int64(int(causal_offset)), int(dtype), _stream(stream))


def fa_bwd_causal_offset(q, k, v, o, dout, lse, dq, dk, dv, B, H, Sq, Sk, D, strides, mask, mask_strides,
                         dropout_p, seed, offset, scale, causal_offset, dtype, workspace, workspace_bytes, stream):
    """C ABI fa_bwd_causal_offset: gradients of fa_fwd_causal_offset (24
    strides as for fa_bwd_strided)."""
    st = [int(x) for x in strides]
    if len(st) != 24:
        raise ValueError("fa: fa_bwd_causal_offset takes 24 strides")
    ms = None if mask_strides is None else _strides3(mask_strides)
    return _load().fa_bwd_causal_offset(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                        _ptr(dk), _ptr(dv), int(B), int(H), int(Sq), int(Sk), int(D),
                                        (ctypes.c_int64 * 24)(*st), _ptr(mask), ms, ctypes.c_float(dropout_p),
                                        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
                                        ctypes.c_uint32(int(offset) & 0xFFFFFFFF), ctypes.c_float(scale),
                                        ctypes.c_int64(int(causal_offset)), int(dtype), _ptr(workspace),
                                        int(workspace_bytes), _stream(stream))


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, Sq, Sk, D, scale, causal, dtype, stream):
    """C ABI fa_bwd_noalloc: the backward with the library's fixed
    scratch array as its workspace (no allocation)."""
    return _load().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                  _ptr(dk), _ptr(dv), int(B), int(H), int(Sq), int(Sk), int(D),
                                  ctypes.c_float(scale), int(bool(causal)), int(dtype), _stream(stream))


def fa_bwd_noalloc_scratch_bytes():
    return _load().fa_bwd_noalloc_scratch_bytes()


def fa_bwd_workspace_bytes(B, H, Sq, D, deterministic):
    return _load().fa_bwd_workspace_bytes(B, H, Sq, D, int(bool(deterministic)))


def fa_status_string(status):
    return _load().fa_status_string(int(status)).decode()


def fa_version():
    return _load().fa_version()


def fa_fwd_plan(B, H, S, D, causal, dtype):
    """The ABI call fa_fwd_plan: (block_q, block_kv, grid, tiles); raises on a bad shape."""
    bq, bkv = ctypes.c_int(), ctypes.c_int()
    grid, tiles = ctypes.c_int64(), ctypes.c_int64()
    st = _load().fa_fwd_plan(int(B), int(H), int(S), int(D), int(bool(causal)), int(dtype),
                             ctypes.byref(bq), ctypes.byref(bkv), ctypes.byref(grid),
                             ctypes.byref(tiles))
    if st != 0:
        raise FaError(st, "fa_fwd_plan")
    return bq.value, bkv.value, grid.value, tiles.value


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("fa: unsupported dtype %s (float16 or bfloat16)" % t.dtype)


def forward(q, k, v, causal=False, scale=None, return_lse=True, out=None, lse_out=None):
    """Attention forward on GPU tensors q [B, H, Sq, D], k and v [B, H, Sk, D].

    Any strides with a contiguous last dimension are accepted (for example a
    [B, S, H, D] tensor viewed as [B, H, S, D] with transpose(1, 2)).  Returns
    (o, lse): o [B, H, Sq, D] contiguous of q's dtype (or `out`, which may be
    strided) and lse float32 [B, H, Sq] (None when return_lse is False).
    causal: key j visible to query i iff j <= i + (Sk - Sq).  scale defaults
    to 1/sqrt(D).  Enqueued on the current torch stream; no synchronisation."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("fa: q, k, v must be 4-d [B, H, S, D]")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if tuple(k.shape) != (B, H, Sk, D) or tuple(v.shape) != (B, H, Sk, D):
        raise ValueError("fa: k and v must be [B, H, Sk, D] matching q [B, H, Sq, D]")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("fa: tensors must be on the GPU")
    if not (q.device == k.device == v.device):
        raise ValueError("fa: tensors must be on one device")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("fa: q, k, v must share one dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.stride(3) != 1 and D > 1:
            raise ValueError("fa: %s must have a contiguous last dimension" % name)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = out if out is not None else torch.empty((B, H, Sq, D), dtype=q.dtype, device=q.device)
    if tuple(o.shape) != (B, H, Sq, D) or o.dtype != q.dtype or o.stride(3) != 1:
        raise ValueError("fa: out must be [B, H, Sq, D] of q's dtype with a contiguous last dimension")
    lse = None
    if return_lse:
        lse = lse_out if lse_out is not None else torch.empty(
            (B, H, Sq), dtype=torch.float32, device=q.device)
        if tuple(lse.shape) != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("fa: lse_out must be contiguous float32 [B, H, Sq]")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
    st = fa_fwd_strided(q, k, v, o, lse, B, H, Sq, Sk, D, q.stride()[:3], k.stride()[:3],
                        v.stride()[:3], o.stride()[:3], scale, causal, _dtype_code(q), stream)
    if st != 0:
        raise FaError(st, "fa_fwd_strided")
    return o, lse


def naive_forward(q, k, v, causal=False, scale=None, workspace=None):
    """The unfused comparison path on contiguous [B, H, S, D] GPU tensors:
    scores and probabilities materialised in a workspace (allocated here with
    torch unless given as a uint8 tensor of at least fa_naive_workspace_bytes).
    Returns (o, lse)."""
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("fa: q, k, v must share one [B, H, S, D] shape")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("fa: the unfused path takes contiguous tensors")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("fa: q, k, v must share one dtype")
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = fa_naive_workspace_bytes(B, H, S, D)
    if need <= 0:
        raise FaError(2, "fa_naive_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
    st = fa_naive_fwd(q, k, v, o, lse, B, H, S, D, scale, causal, _dtype_code(q), workspace,
                      workspace.numel() * workspace.element_size(), stream)
    if st != 0:
        raise FaError(st, "fa_naive_fwd")
    return o, lse


def _bwd_call(q, k, v, o, lse, dout, causal, scale, mask, dropout_p, seed, offset, deterministic, workspace,
              grads, causal_offset=None):
    import torch
    if causal_offset is not None and not causal:
        raise ValueError("fa: causal_offset places the causal diagonal; it needs causal=True")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("fa: q/o/dout [B, H, Sq, D] and k/v [B, H, Sk, D] expected")
    if q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("fa: q and k must share batch, heads and head dimension")
    ts = (q, k, v, o, dout)
    if not all(t.is_cuda and t.device == q.device for t in ts + (lse,)):
        raise ValueError("fa: tensors must be on one GPU")
    if not all(t.dtype == q.dtype for t in ts) or lse.dtype != torch.float32:
        raise ValueError("fa: q, k, v, o, dout share one dtype; lse is float32")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if tuple(lse.shape) != (B, H, Sq) or not lse.is_contiguous():
        raise ValueError("fa: lse must be contiguous float32 [B, H, Sq]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    mask, mstrides = _mask_arg(mask, q, B, H, Sq, Sk)
    if grads is None:
        grads = tuple(t if t.stride(3) == 1 else torch.empty(t.shape, dtype=t.dtype, device=t.device)
                      for t in (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)))
    dq, dk, dv = grads
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if tuple(t.shape) != tuple(ref.shape) or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("fa: %s must match the shape and dtype of its input" % name)
    for t in ts + (dq, dk, dv):
        if t.stride(3) != 1 and D > 1:
            raise ValueError("fa: every tensor must have a contiguous last dimension")
    need = fa_bwd_workspace_bytes(B, H, Sq, D, deterministic)
    if need <= 0:
        raise FaError(2, "fa_bwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    strides = [s for t in ts + (dq, dk, dv) for s in t.stride()[:3]]
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
    if causal_offset is not None:
        st = fa_bwd_causal_offset(q, k, v, o, dout, lse, dq, dk, dv, B, H, Sq, Sk, D, strides, mask, mstrides,
                                  dropout_p, seed, offset, scale, causal_offset, _dtype_code(q), workspace,
                                  workspace.numel() * workspace.element_size(), stream)
        if st != 0:
            raise FaError(st, "fa_bwd_causal_offset")
        return dq, dk, dv
    st = fa_bwd_strided(q, k, v, o, dout, lse, dq, dk, dv, B, H, Sq, Sk, D, strides, mask, mstrides, dropout_p,
                        seed, offset, scale, causal, _dtype_code(q), deterministic, workspace,
                        workspace.numel() * workspace.element_size(), stream)
    if st != 0:
        raise FaError(st, "fa_bwd_strided")
    return dq, dk, dv


def backward(q, k, v, o, lse, dout, causal=False, scale=None, deterministic=True, workspace=None, grads=None):
    """Gradients (dq, dk, dv) of the forward on GPU tensors q, o, dout
    [B, H, Sq, D] and k, v [B, H, Sk, D], with o and lse from forward() on the
    same inputs.  Any strides with a contiguous last dimension are accepted
    (a [B, S, H, D] buffer viewed with transpose(1, 2), say).  The gradients
    are new tensors laid out like their inputs (torch.empty_like), or the
    given `grads` triple (any such strides).  The workspace (allocated here
    with torch unless given as a uint8 tensor of at least
    fa_bwd_workspace_bytes) holds the row dot products.  Results are
    bitwise reproducible; `deterministic` is kept for source compatibility
    and has no effect (there is no atomic dq mode)."""
    return _bwd_call(q, k, v, o, lse, dout, causal, scale, None, 0.0, 0, 0, deterministic, workspace, grads)


def _mask_arg(mask, q, B, H, Sq, Sk):
    """(mask view, byte strides) for the C ABI from a uint8/bool GPU tensor
    broadcastable to [B, H, Sq, Sk]: batch and head strides may be 0
    (broadcast); when the rows do not start on 4-byte boundaries, or the mask
    is broadcast over the query rows, it is copied once into a
    [.., Sq, Sk rounded up to 4] buffer."""
    import torch
    if mask is None:
        return None, None
    if mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    if mask.dtype != torch.uint8 or mask.device != q.device:
        raise ValueError("fa: mask must be a uint8/bool tensor on q's device")
    while mask.dim() < 4:
        mask = mask.unsqueeze(0)
    m = mask.expand(B, H, Sq, Sk)
    # the ABI takes rows that start on 4-byte boundaries, one row per query
    # (row stride >= Sk): a mask broadcast over the queries (a key-padding
    # mask [B, 1, 1, Sk], row stride 0) is copied too
    aligned = m.stride(3) == 1 and m.data_ptr() % 4 == 0 and all(st % 4 == 0 for st in m.stride()[:3]) and \
        m.stride(2) >= Sk
    if not aligned:
        lead = [B if mask.shape[0] != 1 else 1, H if mask.shape[1] != 1 else 1]
        ld = (Sk + 3) // 4 * 4
        padded = torch.zeros(lead + [Sq, ld], dtype=torch.uint8, device=q.device)
        padded[..., :Sk] = mask.expand(lead + [Sq, Sk])
        m = padded[..., :Sk].expand(B, H, Sq, Sk)
    return m, (m.stride(0), m.stride(1), m.stride(2))


def forward_ext(q, k, v, causal=False, scale=None, mask=None, dropout_p=0.0, seed=0, offset=0, out=None,
                causal_offset=None):
    """Forward with an explicit boolean mask and/or dropout on GPU tensors
    q [B, H, Sq, D] and k, v [B, H, Sk, D] with any strides whose last
    dimension is contiguous.  mask: a uint8 or bool GPU tensor broadcastable
    to [B, H, Sq, Sk] (nonzero keeps); rows that do not start on 4-byte
    boundaries are copied to an aligned buffer.  causal_offset (with
    causal=True): key j visible to query i iff j <= i + causal_offset (None:
    Sk - Sq, the bottom-right diagonal; 0: top-left; a block of a split
    sequence, queries from position qs and keys from ks: qs - ks).  Returns
    (o, lse): o contiguous (or `out`, which may be strided) and lse float32
    [B, H, Sq]."""
    import torch
    if causal_offset is not None and not causal:
        raise ValueError("fa: causal_offset places the causal diagonal; it needs causal=True")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("fa: q [B, H, Sq, D] and k, v [B, H, Sk, D] expected")
    if q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("fa: q and k must share batch, heads and head dimension")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("fa: tensors must be on one GPU")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("fa: q, k, v must share one dtype")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    o = out if out is not None else torch.empty((B, H, Sq, D), dtype=q.dtype, device=q.device)
    if tuple(o.shape) != (B, H, Sq, D) or o.dtype != q.dtype or o.device != q.device:
        raise ValueError("fa: out must be [B, H, Sq, D] of q's dtype")
    for t in (q, k, v, o):
        if t.stride(3) != 1 and D > 1:
            raise ValueError("fa: every tensor must have a contiguous last dimension")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    mask, mstrides = _mask_arg(mask, q, B, H, Sq, Sk)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    strides = [s for t in (q, k, v, o) for s in t.stride()[:3]]
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream().cuda_stream
    if causal_offset is not None:
        st = fa_fwd_causal_offset(q, k, v, o, lse, B, H, Sq, Sk, D, strides, mask, mstrides, dropout_p, seed,
                                  offset, scale, causal_offset, _dtype_code(q), stream)
        if st != 0:
            raise FaError(st, "fa_fwd_causal_offset")
        return o, lse
    st = fa_fwd_ext_strided(q, k, v, o, lse, B, H, Sq, Sk, D, strides, mask, mstrides, dropout_p, seed, offset,
                            scale, causal, _dtype_code(q), stream)
    if st != 0:
        raise FaError(st, "fa_fwd_ext_strided")
    return o, lse


def backward_ext(q, k, v, o, lse, dout, causal=False, scale=None, mask=None, dropout_p=0.0, seed=0, offset=0,
                 workspace=None, grads=None, causal_offset=None):
    """Gradients (dq, dk, dv) of forward_ext with the same mask, dropout_p,
    seed, offset and causal_offset (o and lse from that call); strides as
    for backward().  Bitwise reproducible like backward()."""
    return _bwd_call(q, k, v, o, lse, dout, causal, scale, mask, dropout_p, seed, offset, True, workspace, grads,
                     causal_offset)
