"""GPU parity of the attention backward (fa_bwd, both dq modes) against the
fp64 oracle's backward: full gradients on small and ragged shapes, sampled
rows at workload sizes, determinism, and that every output element is
written."""
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


def gpu_grads(q, k, v, g, causal, deterministic=True, scale=None):
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, gd, causal=causal, scale=scale,
                             deterministic=deterministic)
    torch.cuda.synchronize()
    return dq, dk, dv


CASES = [
    # (B, H, Sq, Sk, D, causal, dtype, q_mult)
    (1, 2, 64, 64, 64, False, "f16", 1.0),
    (1, 2, 128, 128, 128, True, "bf16", 1.0),
    (2, 1, 200, 200, 64, True, "f16", 1.0),
    (1, 1, 1, 1, 64, False, "bf16", 1.0),
    (1, 1, 1, 1, 128, True, "f16", 1.0),
    (1, 2, 257, 257, 128, True, "bf16", 4.0),
    (1, 1, 100, 300, 128, True, "f16", 1.0),
    (1, 1, 300, 100, 64, True, "bf16", 1.0),
    (1, 2, 130, 67, 128, False, "f16", 1.0),
    (2, 2, 384, 384, 128, False, "bf16", 1.0),
    (1, 3, 129, 129, 64, True, "bf16", 4.0),
]


@pytest.mark.parametrize("case", CASES, ids=["x".join(map(str, c[:5])) + ("c" if c[5] else "n") + c[6]
                                             for c in CASES])
def test_bwd_matches_oracle(case):
    B, H, Sq, Sk, D, causal, dtype, q_mult = case
    say("case bwd", case)
    q, k, v, g = grad_inputs(B, H, Sq, Sk, D, dtype, seed=1500 + Sq + 7 * Sk + D, q_mult=q_mult)
    dq, dk, dv = gpu_grads(q, k, v, g, causal)
    rq, rk, rv = oracle.attention_bwd(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D),
                                      causal=causal, dtype=dtype)
    # bounds for slices that cancel to zero (one visible key)
    zs = parity.cancellation_tolerances(q, k, v, g, softmax_scale(D), dtype)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        st = parity.assert_grad_parity(to64(got), ref, dtype, "%s %s" % (name, case), zero_tol=zs[name])
        say("  ", name, st)


def test_bwd_is_bitwise_repeatable_whatever_the_flag():
    """Every backward is deterministic: repeated calls, with the flag set or
    not, give the same bits (there is no atomic dq mode)."""
    q, k, v, g = grad_inputs(1, 4, 700, 700, 128, "bf16", seed=1600)
    a = gpu_grads(q, k, v, g, True, True)
    for det in (True, False):
        b = gpu_grads(q, k, v, g, True, det)
        for name, x, y in zip(("dq", "dk", "dv"), a, b):
            assert torch.equal(x, y), (name, det)
    ref = oracle.attention_bwd(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(128),
                               causal=True, dtype="bf16")
    parity.assert_grad_parity(to64(a[0]), ref[0], "bf16", "dq")


def test_bwd_overwrites_stale_outputs_and_workspace():
    """Outputs and workspace pre-filled with NaN bit patterns are fully
    overwritten."""
    B, H, Sq, Sk, D = 1, 2, 190, 190, 64
    q, k, v, g = grad_inputs(B, H, Sq, Sk, D, "f16", seed=1700)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.forward(qd, kd, vd, causal=True)
    ref = oracle.attention_bwd(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D),
                               causal=True, dtype="f16")
    need = fa.fa_bwd_workspace_bytes(B, H, Sq, D, True)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    outs = [torch.full_like(t, float("nan")) for t in (qd, kd, vd)]
    st = fa.fa_bwd(qd, kd, vd, o, gd, lse, outs[0], outs[1], outs[2], B, H, Sq, Sk, D,
                   softmax_scale(D), True, 0, True, ws, need, None)
    assert st == 0
    torch.cuda.synchronize()
    for name, got, r in zip(("dq", "dk", "dv"), outs, ref):
        parity.assert_grad_parity(to64(got), r, "f16", name)


@pytest.mark.parametrize("name", ["gpt_causal_2x12x2048x64_f16", "llama_noncausal_1x32x2048x128_f16",
                                  "long_causal_1x32x8192x128_bf16_q4"])
def test_bwd_workload_sampled_rows(name):
    """At the workload sizes, sampled dq rows (any head) and dk/dv rows (of two
    heads: each needs a full pass over its head in the oracle)."""
    w = WORKLOADS[name]
    q, k, v = workload_inputs(w)
    g, _, _ = make_inputs(w.B, w.H, w.S, w.D, w.dtype, seed=w.seed + 1000)
    say("case bwd workload", name)
    rng = np.random.default_rng(11)
    BH = w.B * w.H
    qrows = np.sort(rng.choice(BH * w.S, size=96, replace=False)).astype(np.int64)
    heads = rng.choice(BH, size=2, replace=False)
    krows = np.sort(np.concatenate([h * w.S + rng.choice(w.S, size=24, replace=False) for h in heads]
                                   + [np.array([heads[0] * w.S, heads[0] * w.S + w.S - 1])]))
    krows = np.unique(krows).astype(np.int64)
    rq, rk, rv = oracle.attention_bwd_rows(bits(q), bits(k), bits(v), bits(g), qrows, krows,
                                           scale=w.scale, causal=w.causal, dtype=w.dtype)
    # the tolerance is relative to each gradient's magnitude over the sampled rows
    dq, dk, dv = gpu_grads(q, k, v, g, w.causal, scale=w.scale)
    for nm, got, ref, rows in (("dq", dq, rq, qrows), ("dk", dk, rk, krows), ("dv", dv, rv, krows)):
        sel = to64(got).reshape(-1, w.D)[rows]
        st = parity.assert_grad_parity(sel[None, None], ref[None, None], w.dtype, "%s %s" % (nm, name))
        say("  ", nm, st)
