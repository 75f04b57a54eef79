"""GPU parity of the attention backward (fa_bwd) against the fp64 oracle's
backward: full gradients on small and ragged shapes, rows of every head at
the workload sizes, determinism, and that every output element is
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


@pytest.mark.parametrize("name", [n for n in WORKLOADS if not n.startswith("tiny")])
def test_bwd_workload_every_head(name):
    """At the workload sizes, in the benchmark's launch configuration: the
    three gradients pre-filled with NaN and every element written and finite;
    12 dQ rows of every head (plus the first and last row of head 0) and 16
    dK/dV rows (plus the first and last key) of eight heads, one from each
    XCD's share when B*H is a multiple of 8 (each such head costs the oracle
    a full forward over it), against the oracle."""
    w = WORKLOADS[name]
    q, k, v = workload_inputs(w)
    g, _, _ = make_inputs(w.B, w.H, w.S, w.D, w.dtype, seed=w.seed + 1000)
    say("case bwd workload", name)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.forward(qd, kd, vd, causal=w.causal, scale=w.scale)
    grads = tuple(torch.full_like(t, float("nan")) for t in (qd, kd, vd))
    fa.backward(qd, kd, vd, o, lse, gd, causal=w.causal, scale=w.scale, grads=grads)
    torch.cuda.synchronize()
    for nm, t in zip(("dq", "dk", "dv"), grads):
        assert torch.isfinite(t).all().item(), "%s: an element is unwritten or not finite" % nm
    rng = np.random.default_rng(11)
    BH, S = w.B * w.H, w.S
    qrows = [h * S + rng.choice(S, size=12, replace=False) for h in range(BH)] + [np.array([0, S - 1])]
    qrows = np.unique(np.concatenate(qrows)).astype(np.int64)
    if BH % 8 == 0:
        hpx = BH // 8
        heads = [x * hpx + x % hpx for x in range(8)]
    else:
        heads = sorted(set(int(h) for h in rng.choice(BH, size=min(BH, 8), replace=False)))
    krows = [h * S + np.concatenate([rng.choice(S, size=16, replace=False), [0, S - 1]]) for h in heads]
    krows = np.unique(np.concatenate(krows)).astype(np.int64)
    rq, rk, rv = oracle.attention_bwd_rows(bits(q), bits(k), bits(v), bits(g), qrows, krows,
                                           scale=w.scale, causal=w.causal, dtype=w.dtype)
    # the tolerance is relative to each gradient's magnitude over the sampled rows
    for nm, got, ref, rows in (("dq", grads[0], rq, qrows), ("dk", grads[1], rk, krows),
                               ("dv", grads[2], rv, krows)):
        sel = to64(got).reshape(-1, w.D)[rows]
        st = parity.assert_grad_parity(sel[None, None], ref[None, None], w.dtype, "%s %s" % (nm, name))
        say("  ", nm, rows.size, "rows", st)


def test_concurrent_streams_and_threads_match_sequential():
    """Four host threads, each on its own stream (default priority), run the
    forward and the backward (plain, and with a mask and dropout) on their own
    inputs at the same time, several times over; every result equals, bit for
    bit, the same calls made one after another on the default stream.  The
    library keeps no state shared between calls besides read-only device
    properties."""
    import threading
    shapes = [(1, 4, 700, 128, "bf16", True), (2, 3, 333, 64, "f16", False),
              (1, 130, 300, 128, "f16", True), (1, 2, 1000, 256, "bf16", True)]
    say("case concurrent streams", len(shapes))
    ins = []
    for i, (B, H, S, D, dtype, causal) in enumerate(shapes):
        q, k, v, g = grad_inputs(B, H, S, S, D, dtype, seed=5600 + i)
        m = torch.from_numpy((np.random.default_rng(5650 + i).random((S, S)) < 0.85).astype(np.uint8)).to(DEV)
        ins.append(tuple(t.to(DEV) for t in (q, k, v, g)) + (m, causal))

    def work(qd, kd, vd, gd, m, causal):
        o, lse = fa.forward(qd, kd, vd, causal=causal)
        grads = fa.backward(qd, kd, vd, o, lse, gd, causal=causal)
        kw = dict(causal=causal, mask=m, dropout_p=0.1, seed=3, offset=1)
        oe, le = fa.forward_ext(qd, kd, vd, **kw)
        ge = fa.backward_ext(qd, kd, vd, oe, le, gd, **kw)
        return (o, lse) + tuple(grads) + (oe, le) + tuple(ge)

    ref = [work(*a) for a in ins]
    torch.cuda.synchronize()
    got = [None] * len(ins)
    errors = []

    def run(i, stream):
        try:
            with torch.cuda.stream(stream):
                for _ in range(3):
                    got[i] = work(*ins[i])
            stream.synchronize()
        except Exception as e:          # reported by the main thread
            errors.append(e)

    streams = [torch.cuda.Stream() for _ in ins]
    threads = [threading.Thread(target=run, args=(i, s)) for i, s in enumerate(streams)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(ref, got)):
        for j, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x, y), (shapes[i], j)
