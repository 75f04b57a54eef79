"""GPU parity of the backward with an explicit mask and dropout (fa_bwd_ext)
against the fp64 oracle's backward of the masked / dropout forward."""
import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import tiled_attention_15_amd as fa
from workloads import WORKLOADS, bits, make_inputs, softmax_scale, workload_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def to64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def grad_inputs(B, H, Sq, Sk, D, dtype, seed, q_mult=1.0):
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=seed, q_mult=q_mult, Sk=Sk)
    q = q[:, :, :Sq].contiguous()
    g, _, _ = make_inputs(B, H, Sq, D, dtype, seed=seed + 1000)
    return q, k, v, g


def make_mask(kind, B, H, Sq, Sk, seed):
    rng = np.random.default_rng(seed)
    if kind is None:
        return None, None
    ld = (Sk + 3) // 4 * 4
    if kind in ("per_head", "per_head_bytes"):
        m = np.zeros((B, H, Sq, ld), np.uint8)
        m[..., :Sk] = rng.random((B, H, Sq, Sk)) < 0.7
        m[0, 0, min(2, Sq - 1), :] = 0                  # a row with no visible key
        if kind == "per_head_bytes":                    # any nonzero byte keeps
            m *= rng.integers(1, 256, size=m.shape, dtype=np.uint8)
        return m, (H * Sq * ld, Sq * ld, ld)
    m = np.zeros((Sq, ld + 4), np.uint8)
    m[:, :Sk] = rng.random((Sq, Sk)) < 0.85
    return m, (0, 0, ld + 4)


def run(q, k, v, g, causal, dtype, mask, ms, p, seed, offset):
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    md = None if mask is None else torch.from_numpy(mask).to(DEV)
    code = fa.BF16 if dtype == "bf16" else fa.F16
    sc = softmax_scale(D)
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    assert fa.fa_fwd_ext(qd, kd, vd, o, lse, B, H, Sq, Sk, D, md, ms, p, seed, offset, sc, causal, code, None) == 0
    need = fa.fa_bwd_workspace_bytes(B, H, Sq, D, 1)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    st = fa.fa_bwd_ext(qd, kd, vd, o, gd, lse, dq, dk, dv, B, H, Sq, Sk, D, md, ms, p, seed, offset, sc, causal,
                       code, ws, need, None)
    assert st == 0, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return dq, dk, dv


CASES = [
    # (B, H, Sq, Sk, D, causal, dtype, mask kind, p)
    (1, 2, 64, 64, 64, False, "f16", "per_head", 0.0),
    (1, 2, 128, 128, 128, True, "bf16", None, 0.1),
    (2, 1, 200, 200, 64, True, "f16", "shared", 0.25),
    (1, 2, 257, 257, 128, True, "bf16", "per_head", 0.5),
    (1, 1, 100, 300, 128, True, "f16", "shared", 0.2),
    (1, 1, 300, 100, 64, True, "bf16", "per_head", 0.1),
    (2, 2, 130, 67, 128, False, "f16", None, 0.3),
    # mask only and dropout only on shapes with interior tiles (where the
    # bounds and causal tests are skipped) and ragged edges
    (1, 2, 190, 333, 128, True, "bf16", "per_head_bytes", 0.0),
    (2, 1, 129, 260, 128, False, "f16", "shared", 0.0),
    (1, 3, 260, 260, 64, False, "f16", None, 0.2),
    (1, 2, 333, 190, 64, True, "bf16", "shared", 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=["%dx%dx%dx%dx%d%s%s_%s_p%g" % (c[0], c[1], c[2], c[3], c[4],
                                                                          "c" if c[5] else "n", c[6], c[7], c[8])
                                             for c in CASES])
def test_bwd_ext_matches_oracle(case):
    B, H, Sq, Sk, D, causal, dtype, kind, p = case
    say("case bwd ext", case)
    q, k, v, g = grad_inputs(B, H, Sq, Sk, D, dtype, seed=3000 + Sq + 3 * Sk + D)
    mask, ms = make_mask(kind, B, H, Sq, Sk, seed=3100 + Sq)
    seed, offset = 0x5EED_0000_0001 + Sq, 11
    dq, dk, dv = run(q, k, v, g, causal, dtype, mask, ms, p, seed, offset)
    refs = oracle.attention_bwd_ext(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=causal,
                                    dtype=dtype, mask=mask, mask_strides=ms, dropout_p=p, seed=seed, offset=offset)
    zs = parity.cancellation_tolerances(q, k, v, g, softmax_scale(D), dtype, dropout_p=p)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        st = parity.assert_grad_parity(to64(got), ref, dtype, "%s %s" % (name, case), zero_tol=zs[name])
        say("  ", name, st)


def test_bwd_ext_without_mask_or_dropout_is_fa_bwd():
    q, k, v, g = grad_inputs(1, 3, 300, 300, 128, "bf16", seed=3200)
    a = run(q, k, v, g, True, "bf16", None, None, 0.0, 0, 0)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.forward_ext(qd, kd, vd, causal=True)
    b = fa.backward(qd, kd, vd, o, lse, gd, causal=True, deterministic=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_ext_medium_sampled_rows():
    """1x4x2048x128 bf16 causal with a shared mask and dropout 0.1: sampled dq
    rows and dk/dv rows of two heads against the oracle."""
    B, H, S, D = 1, 4, 2048, 128
    q, k, v, g = grad_inputs(B, H, S, S, D, "bf16", seed=3300)
    mask, ms = make_mask("shared", B, H, S, S, seed=3301)
    dq, dk, dv = run(q, k, v, g, True, "bf16", mask, ms, 0.1, 4242, 5)
    rng = np.random.default_rng(3302)
    qrows = np.sort(rng.choice(B * H * S, size=64, replace=False)).astype(np.int64)
    krows = np.sort(np.concatenate([h * S + rng.choice(S, size=24, replace=False) for h in (1, 3)])).astype(np.int64)
    rq, rk, rv = oracle.attention_bwd_ext(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=True,
                                          dtype="bf16", mask=mask, mask_strides=ms, dropout_p=0.1, seed=4242,
                                          offset=5, qrows=qrows, krows=krows)
    for nm, got, ref, rows in (("dq", dq, rq, qrows), ("dk", dk, rk, krows), ("dv", dv, rv, krows)):
        sel = to64(got).reshape(-1, D)[rows]
        say("  ", nm, parity.assert_grad_parity(sel[None, None], ref[None, None], "bf16", "medium " + nm))


def test_bwd_ext_headline_size_every_head():
    """The long causal workload (1x32x8192x128 bf16, Q x4) with one [S, S]
    mask shared by all heads (90% kept) and dropout 0.1, as the benchmark
    times it: gradients pre-filled with NaN and every element written and
    finite; 8 dQ rows of every head and 12 dK/dV rows (plus the first and last
    key) of four heads on different XCDs, against the oracle."""
    w = WORKLOADS["long_causal_1x32x8192x128_bf16_q4"]
    q, k, v = workload_inputs(w)
    g, _, _ = make_inputs(w.B, w.H, w.S, w.D, w.dtype, seed=w.seed + 1000)
    S, BH = w.S, w.B * w.H
    mask = (np.random.default_rng(3900).random((S, S)) < 0.9).astype(np.uint8)
    say("case bwd_ext headline size")
    kw = dict(causal=True, scale=w.scale, mask=torch.from_numpy(mask).to(DEV), dropout_p=0.1, seed=77, offset=9)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.forward_ext(qd, kd, vd, **kw)
    grads = tuple(torch.full_like(t, float("nan")) for t in (qd, kd, vd))
    fa.backward_ext(qd, kd, vd, o, lse, gd, grads=grads, **kw)
    torch.cuda.synchronize()
    for nm, t in zip(("dq", "dk", "dv"), grads):
        assert torch.isfinite(t).all().item(), "%s: an element is unwritten or not finite" % nm
    rng = np.random.default_rng(3901)
    qrows = np.unique(np.concatenate([h * S + rng.choice(S, size=8, replace=False) for h in range(BH)]))
    krows = np.unique(np.concatenate([h * S + np.concatenate([rng.choice(S, size=12, replace=False), [0, S - 1]])
                                      for h in (0, 9, 18, 27)]))
    rq, rk, rv = oracle.attention_bwd_ext(bits(q), bits(k), bits(v), bits(g), scale=w.scale, causal=True,
                                          dtype=w.dtype, mask=mask, mask_strides=(0, 0, S), dropout_p=0.1, seed=77,
                                          offset=9, qrows=qrows.astype(np.int64), krows=krows.astype(np.int64))
    for nm, got, ref, rows in (("dq", grads[0], rq, qrows), ("dk", grads[1], rk, krows), ("dv", grads[2], rv, krows)):
        sel = to64(got).reshape(-1, w.D)[rows]
        say("  ", nm, rows.size, "rows", parity.assert_grad_parity(sel[None, None], ref[None, None], w.dtype,
                                                                  "headline " + nm))
