"""Seeded random shapes through every forward route, against the fp64 oracle.

Each case draws batch, heads, query and key lengths, head dimension, dtype,
causality, a mask (none, per head or shared) and a dropout probability from
a fixed generator, so the sweep reaches the tuned kernel's key-split,
masked and dropout instances and its pair split (D = 256), and strided
[B, S, H, D] views, with ragged lengths throughout.  Its small grids
(B*H <= 8) always take the key-split route at D <= 128; the unsplit 256-row
instance is checked on ragged shapes by test_parity_gpu.py.
25 further draws run the backward of the same routes (backward_ext) against
the oracle's full backward, and 18 draws on grids large enough for the
256-row instance (64-280 heads, 700-1536 rows; plain, masked, dropout,
strided) compare rows of every head, forward and backward.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import tiled_attention_15_amd as fa
from oracle_pins import _keep_matrix
from workloads import bits, make_inputs, softmax_scale

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def draw(i):
    rng = np.random.default_rng(9000 + i)
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 5))
    Sq = int(rng.choice([1, int(rng.integers(2, 129)), int(rng.integers(129, 700))]))
    Sk = Sq if rng.random() < 0.5 else int(rng.integers(1, 700))
    D = int(rng.choice([64, 128, 128, 256]))
    dtype = str(rng.choice(["f16", "bf16"]))
    causal = bool(rng.random() < 0.6)
    mask = str(rng.choice(["none", "none", "per_head", "shared"]))
    p = float(rng.choice([0.0, 0.0, 0.0, 0.2]))
    strided = bool(rng.random() < 0.3)
    return dict(B=B, H=H, Sq=Sq, Sk=Sk, D=D, dtype=dtype, causal=causal, mask=mask, p=p, strided=strided)


CASES = [draw(i) for i in range(32)]


@pytest.mark.parametrize("c", CASES, ids=["%d:%dx%dx%dx%dx%d%s%s_%s_p%g%s" % (
    i, c["B"], c["H"], c["Sq"], c["Sk"], c["D"], "c" if c["causal"] else "n", c["dtype"], c["mask"], c["p"],
    "_strided" if c["strided"] else "") for i, c in enumerate(CASES)])
def test_random_shape(c):
    print("case", c, flush=True)
    B, H, Sq, Sk, D, dtype = c["B"], c["H"], c["Sq"], c["Sk"], c["D"], c["dtype"]
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=9100 + Sq + 7 * Sk + D, Sk=Sk)
    q = q[:, :, :Sq].contiguous()
    rng = np.random.default_rng(9200 + Sq)
    if c["mask"] == "none":
        m, ms, mt = None, None, None
    else:
        mb, mh = (B, H) if c["mask"] == "per_head" else (1, 1)
        m = (rng.random((mb, mh, Sq, Sk)) < 0.8).astype(np.uint8)
        ms = (H * Sq * Sk if mb > 1 else 0, Sq * Sk if mh > 1 else 0, Sk)
        mt = torch.from_numpy(m).to(DEV)
        if c["mask"] == "shared":
            mt = mt[0, 0]
    args = [t.to(DEV) for t in (q, k, v)]
    if c["strided"]:
        args = [t.transpose(1, 2).contiguous().transpose(1, 2) for t in args]
    o, lse = fa.forward_ext(*args, causal=c["causal"], mask=mt, dropout_p=c["p"], seed=5, offset=1)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=c["causal"],
                                            dtype=dtype, mask=m, mask_strides=ms, dropout_p=c["p"], seed=5, offset=1)
    st = parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, "random %s" % (c,))
    print("  ", st, flush=True)


# draw 3040: one query over a masked 4-key range, whose gradients need the
# per-element bound (rows see too few keys for the slice-wide rule)
BWD_CASES = [draw(100 + i) for i in range(24)] + [draw(3040)]


@pytest.mark.parametrize("c", BWD_CASES, ids=["%d:%dx%dx%dx%dx%d%s%s_%s_p%g%s" % (
    i, c["B"], c["H"], c["Sq"], c["Sk"], c["D"], "c" if c["causal"] else "n", c["dtype"], c["mask"], c["p"],
    "_strided" if c["strided"] else "") for i, c in enumerate(BWD_CASES)])
def test_random_shape_backward(c):
    """The same draws through backward_ext (after forward_ext with the same
    mask and dropout): every gradient element against the oracle's backward,
    by the slice-wide rule, or where rows see too few keys for it, by the
    per-element bound of the operand rounding."""
    print("case backward", c, flush=True)
    B, H, Sq, Sk, D, dtype = c["B"], c["H"], c["Sq"], c["Sk"], c["D"], c["dtype"]
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=9300 + Sq + 7 * Sk + D, Sk=Sk)
    q = q[:, :, :Sq].contiguous()
    g, _, _ = make_inputs(B, H, Sq, D, dtype, seed=9400 + Sq + D)
    rng = np.random.default_rng(9500 + Sq)
    if c["mask"] == "none":
        m, ms, mt = None, None, None
    else:
        mb, mh = (B, H) if c["mask"] == "per_head" else (1, 1)
        m = (rng.random((mb, mh, Sq, Sk)) < 0.8).astype(np.uint8)
        ms = (H * Sq * Sk if mb > 1 else 0, Sq * Sk if mh > 1 else 0, Sk)
        mt = torch.from_numpy(m).to(DEV)
        if c["mask"] == "shared":
            mt = mt[0, 0]
    args = [t.to(DEV) for t in (q, k, v, g)]
    if c["strided"]:
        args = [t.transpose(1, 2).contiguous().transpose(1, 2) for t in args]
    kw = dict(causal=c["causal"], mask=mt, dropout_p=c["p"], seed=5, offset=1)
    o, lse = fa.forward_ext(*args[:3], **kw)
    grads = fa.backward_ext(*args[:3], o, lse, args[3], **kw)
    torch.cuda.synchronize()
    refs = oracle.attention_bwd_ext(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=c["causal"],
                                    dtype=dtype, mask=m, mask_strides=ms, dropout_p=c["p"], seed=5, offset=1)
    zs = parity.cancellation_tolerances(q, k, v, g, softmax_scale(D), dtype, dropout_p=c["p"])
    bnd = {}
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        st = parity.compare_grad(to64(got), ref, dtype, zs[name])
        if not parity.grad_ok(st):
            # Rows with very few visible keys (a short key range, a mask): the
            # error of D_i (from the stored O) is then one scalar per row times
            # a difference of two K rows, not an average of many independent
            # roundings, so each element is held to the operand-rounding bound.
            if not bnd:
                o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D),
                                                        causal=c["causal"], dtype=dtype, mask=m, mask_strides=ms,
                                                        dropout_p=c["p"], seed=5, offset=1)
                vis = np.ones((B, H, Sq, Sk), dtype=bool) if m is None else np.broadcast_to(m != 0, (B, H, Sq, Sk))
                if c["causal"]:
                    vis = vis & (np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] + (Sk - Sq))
                zc = _keep_matrix(B, H, Sq, Sk, 5, 1, c["p"]) if c["p"] > 0 else None
                bnd.update(parity.operand_rounding_bounds(q, k, v, g, o_ref, l_ref, softmax_scale(D), c["causal"],
                                                          dtype, vis=vis, zc=zc))
            st = dict(st, **parity.assert_grad_within_bound(to64(got), ref, bnd[name], dtype,
                                                            "%s random %s" % (name, c)))
        print("  ", name, st, flush=True)


def draw_big(i):
    """Grids large enough for the 256-row instance (B*H 64-280, 700-1536 rows)."""
    r = np.random.default_rng(7000 + i)
    B = int(r.integers(1, 3))
    H = int(r.integers(64, 141))
    Sq = int(r.integers(700, 1537))
    Sk = Sq if r.random() < 0.6 else int(r.integers(300, 1537))
    D = int(r.choice([64, 128, 128]))
    dtype = str(r.choice(["f16", "bf16"]))
    causal = bool(r.random() < 0.6)
    mask = str(r.choice(["none", "none", "shared"]))
    p = float(r.choice([0.0, 0.0, 0.15]))
    strided = bool(r.random() < 0.3)
    return dict(B=B, H=H, Sq=Sq, Sk=Sk, D=D, dtype=dtype, causal=causal, mask=mask, p=p, strided=strided)


BIG_CASES = [(i, False) for i in range(12)] + [(100 + i, True) for i in range(6)]


@pytest.mark.parametrize("case", BIG_CASES, ids=["big%d%s" % (i, "_bwd" if b else "") for i, b in BIG_CASES])
def test_random_big_grid(case):
    """Random draws on grids that take the 256-row instance (plain, masked,
    dropout, strided): six rows of every head (and the first and last rows)
    against the oracle; with the backward, those dQ rows and eight dK/dV rows
    of three heads."""
    i, bwd = case
    c = draw_big(i)
    print("case big", i, bwd, c, flush=True)
    B, H, Sq, Sk, D, dtype = c["B"], c["H"], c["Sq"], c["Sk"], c["D"], c["dtype"]
    assert fa.fa_fwd_plan(B, H, Sq, D, c["causal"], fa.BF16 if dtype == "bf16" else fa.F16)[0] == 256
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=7100 + i, Sk=Sk)
    q = q[:, :, :Sq].contiguous()
    g, _, _ = make_inputs(B, H, Sq, D, dtype, seed=7200 + i)
    r = np.random.default_rng(7300 + i)
    m = ms = mt = None
    if c["mask"] == "shared":
        m = (r.random((Sq, Sk)) < 0.85).astype(np.uint8)
        ms = (0, 0, Sk)
        mt = torch.from_numpy(m).to(DEV)
    args = [t.to(DEV) for t in (q, k, v, g)]
    if c["strided"]:
        args = [t.transpose(1, 2).contiguous().transpose(1, 2) for t in args]
    kw = dict(causal=c["causal"], mask=mt, dropout_p=c["p"], seed=9, offset=2)
    o, lse = fa.forward_ext(*args[:3], **kw)
    BH = B * H
    rows = np.unique(np.concatenate([h * Sq + r.choice(Sq, 6, replace=False) for h in range(BH)]
                                    + [np.array([0, Sq - 1, BH * Sq - 1])])).astype(np.int64)
    if not bwd:
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D),
                                                causal=c["causal"], dtype=dtype, mask=m, mask_strides=ms,
                                                dropout_p=c["p"], seed=9, offset=2, rows=rows)
        st = parity.assert_parity(to64(o).reshape(-1, D)[rows], to64(lse).reshape(-1)[rows], o_ref, l_ref, dtype,
                                  str(c))
        print("  ", rows.size, "rows", st, flush=True)
        return
    grads = fa.backward_ext(*args[:3], o, lse, args[3], **kw)
    torch.cuda.synchronize()
    heads = r.choice(BH, 3, replace=False)
    krows = np.unique(np.concatenate([h * Sk + r.choice(Sk, 8, replace=False) for h in heads])).astype(np.int64)
    rq, rk, rv = oracle.attention_bwd_ext(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D),
                                          causal=c["causal"], dtype=dtype, mask=m, mask_strides=ms,
                                          dropout_p=c["p"], seed=9, offset=2, qrows=rows, krows=krows)
    for nm, got, ref, rr in (("dq", grads[0], rq, rows), ("dk", grads[1], rk, krows), ("dv", grads[2], rv, krows)):
        sel = to64(got).reshape(-1, D)[rr]
        st = parity.assert_grad_parity(sel[None, None], ref[None, None], dtype, "%s %s" % (nm, c))
        print("  ", nm, rr.size, "rows", st, flush=True)
