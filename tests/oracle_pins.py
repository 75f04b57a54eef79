"""Pins for the fp64 CPU oracle: facts that the mathematics or the pages fix,
checked without trusting the oracle's own code.

Each pin takes a loaded oracle library and raises AssertionError when the
oracle disagrees with the fact.  The pins are run against the real oracle
(test_oracle.py) and against deliberately broken copies of it
(test_oracle_mutants.py), which must each fail at least one pin.

Independent routes used here:
  * input decoding goes through numpy/torch casts, never the oracle's decoder;
  * closed forms (Q = 0, causal row 0, constant V, key shift);
  * a 40-digit Python `decimal` evaluation of the definition without the
    max subtraction, on tiny shapes;
  * torch's scaled_dot_product_attention in fp64 on the CPU (the pages check
    their fused operator against exactly this routine: omica.com.cn learning
    path, "step three");
  * algebraic invariants (convexity, permutation, chunk merge).

The backward (gradients of sum(O * dO)) is pinned by torch autograd through
torch's fp64 scaled_dot_product_attention, by central differences of the
40-digit forward on tiny shapes, by closed forms (one key; Q = 0) and by
invariants (the key-shift symmetry gives sum_j dK_j = 0; rows of P sum to
one give sum_j dV_j = sum_i dO_i; the scores' bilinearity gives
sum_i q_i.dQ_i = sum_j k_j.dK_j).

The forward with an explicit mask and dropout is pinned by Philox4x32-10's
published known-answer vectors, by torch's fp64 scaled_dot_product_attention
with the same boolean mask, by the identity-V case (O = P) against a second
Philox written from its definition in this file, by the kept fraction, and
by reducing to the plain forward (no mask, p = 0; all-true mask; triangular
mask = causal flag) bit for bit.

The causal diagonal at an arbitrary offset c (key j visible to query i iff
j <= i + c) is pinned by a block decomposition: a causal sequence cut into
query and key chunks, each block computed with c = (query chunk start) -
(key chunk start) and the blocks merged by log-sum-exp, must give the full
causal attention of the plain forward (which the pins above fix); and, in
the forward and the backward, bit for bit by the equivalent explicit mask.
"""
from decimal import Decimal, getcontext
from fractions import Fraction
import json
import math
import os

import numpy as np
import torch

import oracle
from workloads import bits, make_inputs, softmax_scale


def _f64(t):
    """Exact fp64 values of a CPU fp16/bf16 tensor via torch's own cast."""
    return t.to(torch.float64).numpy()


def _run(lib, q, k, v, scale, causal, dtype):
    return oracle.attention_fwd(bits(q), bits(k), bits(v), scale=scale, causal=causal,
                                dtype=dtype, lib=lib)


def _visible(i, j, Sq, Sk, causal):
    return (not causal) or j <= i + (Sk - Sq)


def pin_decode_f16(lib):
    allbits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(allbits, "f16", lib=lib)
    ref = allbits.view(np.float16).astype(np.float64)
    assert np.array_equal(got, ref, equal_nan=True), "fp16 decode differs from numpy"
    assert np.array_equal(np.signbit(got), np.signbit(ref)), "fp16 decode sign differs"


def pin_decode_bf16(lib):
    allbits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(allbits, "bf16", lib=lib)
    ref = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).to(
        torch.float64).numpy()
    assert np.array_equal(got, ref, equal_nan=True), "bf16 decode differs from torch"
    assert np.array_equal(np.signbit(got), np.signbit(ref)), "bf16 decode sign differs"


def pin_q_zero(lib):
    """Q = 0: every visible score is 0, so O_i is the mean of the visible V rows
    and lse_i = ln(#visible)."""
    for dtype, (B, H, S, D) in (("f16", (1, 2, 37, 16)), ("bf16", (2, 1, 70, 8))):
        _, k, v = make_inputs(B, H, S, D, dtype, seed=11)
        q = torch.zeros(B, H, S, D, dtype=k.dtype)
        V = _f64(v)
        for causal in (False, True):
            o, lse = _run(lib, q, k, v, softmax_scale(D), causal, dtype)
            for i in range(S):
                n = i + 1 if causal else S
                exp_o = V[:, :, :n, :].mean(axis=2)
                assert np.allclose(o[:, :, i, :], exp_o, rtol=0, atol=1e-14), (dtype, causal, i)
                assert np.allclose(lse[:, :, i], math.log(n), rtol=0, atol=1e-14), (dtype, causal, i)


def pin_causal_row0(lib):
    """Causal row 0 sees key 0 only: O_0 = V_0 exactly, lse_0 = scale * q_0 . k_0."""
    for dtype, q_mult in (("f16", 1.0), ("bf16", 4.0)):
        B, H, S, D = 2, 3, 19, 64
        q, k, v = make_inputs(B, H, S, D, dtype, seed=12, q_mult=q_mult)
        scale = softmax_scale(D)
        o, lse = _run(lib, q, k, v, scale, True, dtype)
        assert np.array_equal(o[:, :, 0, :], _f64(v)[:, :, 0, :]), dtype
        Q, K = _f64(q), _f64(k)
        for b in range(B):
            for h in range(H):
                dot = sum(Fraction(float(a)) * Fraction(float(c)) for a, c in zip(Q[b, h, 0], K[b, h, 0]))
                want = float(Fraction(scale) * dot)
                assert abs(lse[b, h, 0] - want) <= 1e-14 * max(1.0, abs(want)), (dtype, b, h)


def pin_convexity(lib):
    """Each output row is a convex combination of the visible V rows."""
    B, H, S, D = 1, 2, 64, 32
    q, k, v = make_inputs(B, H, S, D, "f16", seed=13)
    V = _f64(v)
    for causal in (False, True):
        o, _ = _run(lib, q, k, v, softmax_scale(D), causal, "f16")
        for i in range(S):
            n = i + 1 if causal else S
            lo = V[:, :, :n, :].min(axis=2) - 1e-15
            hi = V[:, :, :n, :].max(axis=2) + 1e-15
            assert np.all(o[:, :, i, :] >= lo) and np.all(o[:, :, i, :] <= hi), (causal, i)


def _decimal_attention(Q, K, V, scale, causal):
    """The definition at 40 significant digits, without max subtraction."""
    getcontext().prec = 40
    Sq, D = Q.shape
    Sk = K.shape[0]
    sc = Decimal(scale)
    o = np.zeros((Sq, D))
    lse = np.zeros(Sq)
    for i in range(Sq):
        ws, num = [], [Decimal(0)] * D
        for j in range(Sk):
            if not _visible(i, j, Sq, Sk, causal):
                continue
            s = sc * sum(Decimal(float(Q[i, d])) * Decimal(float(K[j, d])) for d in range(D))
            w = s.exp()
            ws.append(w)
            for d in range(D):
                num[d] += w * Decimal(float(V[j, d]))
        tot = sum(ws)
        lse[i] = float(tot.ln())
        for d in range(D):
            o[i, d] = float(num[d] / tot)
    return o, lse


def pin_bruteforce_decimal(lib):
    cases = (("f16", 1, 5, 4, 1.0), ("f16", 2, 16, 8, 1.0), ("bf16", 1, 9, 3, 4.0),
             ("bf16", 1, 12, 8, 1.0))
    for dtype, H, S, D, q_mult in cases:
        q, k, v = make_inputs(1, H, S, D, dtype, seed=14 + S, q_mult=q_mult)
        scale = softmax_scale(D)
        Q, K, V = _f64(q), _f64(k), _f64(v)
        for causal in (False, True):
            o, lse = _run(lib, q, k, v, scale, causal, dtype)
            for h in range(H):
                eo, el = _decimal_attention(Q[0, h], K[0, h], V[0, h], scale, causal)
                assert np.all(np.abs(o[0, h] - eo) <= 1e-13 * np.maximum(1, np.abs(eo))), (dtype, S, causal)
                assert np.all(np.abs(lse[0, h] - el) <= 1e-13 * np.maximum(1, np.abs(el))), (dtype, S, causal)


def _sdpa(Q, K, V, scale, causal):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V), scale=scale,
        is_causal=causal).numpy()


def pin_sdpa_fp64(lib):
    for dtype, (B, H, S, D) in (("f16", (1, 2, 128, 64)), ("f16", (2, 3, 300, 32)),
                                ("bf16", (1, 2, 257, 128))):
        q, k, v = make_inputs(B, H, S, D, dtype, seed=15 + S)
        scale = softmax_scale(D)
        for causal in (False, True):
            o, _ = _run(lib, q, k, v, scale, causal, dtype)
            ref = _sdpa(_f64(q), _f64(k), _f64(v), scale, causal)
            assert np.max(np.abs(o - ref)) <= 1e-12, (dtype, S, causal, np.max(np.abs(o - ref)))
    # unequal query / key lengths, non-causal
    q, _, _ = make_inputs(1, 2, 50, 16, "f16", seed=16)
    _, k, v = make_inputs(1, 2, 77, 16, "f16", seed=17)
    o, _ = _run(lib, q, k, v, 0.25, False, "f16")
    ref = _sdpa(_f64(q), _f64(k), _f64(v), 0.25, False)
    assert np.max(np.abs(o - ref)) <= 1e-12


def pin_chunk_merge(lib):
    """Splitting the keys into chunks and merging the partial results by their
    log-sum-exp reproduces the one-shot result (the online-softmax identity)."""
    q, k, v = make_inputs(1, 2, 40, 32, "f16", seed=18, Sk=100)
    scale = softmax_scale(32)
    o, lse = _run(lib, q, k, v, scale, False, "f16")
    parts = []
    for a, b in ((0, 30), (30, 64), (64, 100)):
        parts.append(_run(lib, q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), scale,
                          False, "f16"))
    lse_m = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    o_m = sum(np.exp(p[1] - lse_m)[..., None] * p[0] for p in parts)
    assert np.max(np.abs(lse_m - lse)) <= 1e-12
    assert np.max(np.abs(o_m - o)) <= 1e-12


def pin_invariances(lib):
    B, H, S, D = 1, 2, 48, 16
    scale = softmax_scale(D)
    # joint permutation of key/value rows (non-causal) leaves O and lse unchanged
    q, k, v = make_inputs(B, H, S, D, "f16", seed=19)
    perm = torch.randperm(S, generator=torch.Generator().manual_seed(3))
    o1, l1 = _run(lib, q, k, v, scale, False, "f16")
    o2, l2 = _run(lib, q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), scale, False, "f16")
    assert np.max(np.abs(o1 - o2)) <= 1e-13 and np.max(np.abs(l1 - l2)) <= 1e-13
    # constant V rows give that constant
    cvec = torch.linspace(-3, 3, D).to(torch.float16)
    vc = cvec.expand(B, H, S, D).contiguous()
    for causal in (False, True):
        o, _ = _run(lib, q, k, vc, scale, causal, "f16")
        assert np.max(np.abs(o - _f64(cvec))) <= 1e-14, causal
    # adding u to every key shifts row i's scores by scale*q_i.u: O unchanged, lse shifted.
    # values on a 1/8 grid so q, k and k+u are exact in fp16
    g = torch.Generator().manual_seed(4)
    qg = (torch.randint(-16, 17, (B, H, S, D), generator=g) / 8.0).to(torch.float16)
    kg = (torch.randint(-16, 17, (B, H, S, D), generator=g) / 8.0).to(torch.float16)
    u = (torch.randint(-8, 9, (D,), generator=g) / 8.0)
    ku = (kg.to(torch.float32) + u).to(torch.float16)
    assert torch.equal(ku.to(torch.float32), kg.to(torch.float32) + u)
    for causal in (False, True):
        oa, la = _run(lib, qg, kg, v, scale, causal, "f16")
        ob, lb = _run(lib, qg, ku, v, scale, causal, "f16")
        shift = scale * (_f64(qg) @ u.double().numpy())
        assert np.max(np.abs(oa - ob)) <= 1e-12, causal
        assert np.max(np.abs(lb - la - shift)) <= 1e-12, causal


def pin_rows_match_full(lib):
    q, k, v = make_inputs(2, 3, 65, 32, "bf16", seed=20)
    scale = softmax_scale(32)
    for causal in (False, True):
        o, lse = _run(lib, q, k, v, scale, causal, "bf16")
        rows = np.array([0, 1, 64, 65, 130, 194, 2 * 3 * 65 - 1], dtype=np.int64)
        ro, rl = oracle.attention_rows(bits(q), bits(k), bits(v), rows, scale=scale,
                                       causal=causal, dtype="bf16", lib=lib)
        assert np.array_equal(ro, o.reshape(-1, 32)[rows])
        assert np.array_equal(rl, lse.reshape(-1)[rows])


def pin_unequal_causal_suffix(lib):
    """Causal attention of a query block against a longer key sequence is the
    tail of the square causal problem: with Sq < Sk, query row i plays the
    role of row i + (Sk - Sq) of the Sk x Sk problem (whose causal mask the
    pages fix: each position sees itself and earlier ones).  With Sq > Sk the
    first Sq - Sk rows see no key (O = 0, lse = -inf) and the rest are the
    square problem's rows."""
    D = 16
    scale = softmax_scale(D)
    for dtype, Sq, Sk in (("f16", 23, 57), ("bf16", 5, 64), ("f16", 57, 23)):
        qf, k, v = make_inputs(1, 2, max(Sq, Sk), D, dtype, seed=21 + Sq, Sk=Sk)
        o_sq, l_sq = _run(lib, qf[:, :, :Sk].contiguous(), k, v, scale, True, dtype)
        if Sq <= Sk:
            q = qf[:, :, Sk - Sq:Sk].contiguous()
            o, lse = _run(lib, q, k, v, scale, True, dtype)
            assert np.array_equal(o, o_sq[:, :, Sk - Sq:]), (dtype, Sq, Sk)
            assert np.array_equal(lse, l_sq[:, :, Sk - Sq:]), (dtype, Sq, Sk)
        else:
            q = torch.cat([qf[:, :, Sk:Sq], qf[:, :, :Sk]], dim=2).contiguous()
            o, lse = _run(lib, q, k, v, scale, True, dtype)
            n = Sq - Sk
            assert np.all(o[:, :, :n] == 0.0) and np.all(np.isneginf(lse[:, :, :n])), (dtype, Sq, Sk)
            assert np.array_equal(o[:, :, n:], o_sq) and np.array_equal(lse[:, :, n:], l_sq)
        # the last query row sees every key: it equals the non-causal result
        o_nc, l_nc = _run(lib, q, k, v, scale, False, dtype)
        assert np.array_equal(o[:, :, -1], o_nc[:, :, -1]) and np.array_equal(lse[:, :, -1], l_nc[:, :, -1])


def _run_bwd(lib, q, k, v, g, scale, causal, dtype):
    return oracle.attention_bwd(bits(q), bits(k), bits(v), bits(g), scale=scale, causal=causal,
                                dtype=dtype, lib=lib)


def _grad_inputs(B, H, Sq, Sk, D, dtype, seed, q_mult=1.0):
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=seed, q_mult=q_mult, Sk=Sk)
    q = q[:, :, :Sq].contiguous()
    g, _, _ = make_inputs(B, H, Sq, D, dtype, seed=seed + 1000)
    return q, k, v, g


def pin_bwd_autograd(lib):
    """torch autograd through torch's fp64 scaled_dot_product_attention (with a
    bottom-right boolean mask when causal) gives the same three gradients."""
    cases = (("f16", (1, 2, 64, 64, 32), False, 1.0), ("bf16", (2, 1, 45, 45, 16), True, 4.0),
             ("f16", (1, 2, 30, 71, 16), True, 1.0), ("bf16", (1, 1, 33, 20, 64), False, 1.0))
    for dtype, (B, H, Sq, Sk, D), causal, q_mult in cases:
        q, k, v, g = _grad_inputs(B, H, Sq, Sk, D, dtype, seed=30 + Sq, q_mult=q_mult)
        scale = softmax_scale(D)
        dq, dk, dv = _run_bwd(lib, q, k, v, g, scale, causal, dtype)
        Q, K, V = (torch.from_numpy(_f64(t)).requires_grad_() for t in (q, k, v))
        mask = None
        if causal:
            i = torch.arange(Sq)[:, None]
            j = torch.arange(Sk)[None, :]
            mask = j <= i + (Sk - Sq)
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
        (o * torch.from_numpy(_f64(g))).sum().backward()
        for name, got, ref in (("dq", dq, Q.grad), ("dk", dk, K.grad), ("dv", dv, V.grad)):
            ref = ref.numpy()
            err = np.max(np.abs(got - ref))
            assert err <= 1e-12 * max(1.0, np.max(np.abs(ref))), (name, dtype, Sq, Sk, causal, err)


def _decimal_loss(Q, K, V, G, scale, causal):
    """sum(O * G) of the definition at 40 digits (one head)."""
    o, _ = _decimal_attention(Q, K, V, scale, causal)
    return o, float(np.sum(o * G))


def pin_bwd_finite_difference(lib):
    """Central differences of the 40-digit forward: d/dx sum(O * dO) for single
    entries of q, k and v against the oracle's gradients."""
    getcontext().prec = 40
    for dtype, Sq, Sk, D, causal in (("f16", 3, 4, 3, False), ("bf16", 4, 4, 2, True),
                                     ("f16", 2, 5, 2, True)):
        q, k, v, g = _grad_inputs(1, 1, Sq, Sk, D, dtype, seed=40 + Sq + Sk)
        scale = softmax_scale(D)
        dq, dk, dv = _run_bwd(lib, q, k, v, g, scale, causal, dtype)
        Q, K, V, G = (_f64(t)[0, 0] for t in (q, k, v, g))
        sc = Decimal(scale)

        def loss(Qx, Kx, Vx):
            tot = Decimal(0)
            for i in range(Sq):
                ws, num = [], [Decimal(0)] * D
                for j in range(Sk):
                    if not _visible(i, j, Sq, Sk, causal):
                        continue
                    s = sc * sum(Qx[i][d] * Kx[j][d] for d in range(D))
                    w = s.exp()
                    ws.append(w)
                    for d in range(D):
                        num[d] += w * Vx[j][d]
                den = sum(ws)
                for d in range(D):
                    tot += num[d] / den * Decimal(float(G[i, d]))
            return tot

        dec = lambda A: [[Decimal(float(x)) for x in row] for row in A]
        h = Decimal("1e-12")
        for which, grad, rows in (("q", dq, Sq), ("k", dk, Sk), ("v", dv, Sk)):
            for r in range(rows):
                for d in range(D):
                    X = {"q": dec(Q), "k": dec(K), "v": dec(V)}
                    X[which][r][d] += h
                    up = loss(X["q"], X["k"], X["v"])
                    X[which][r][d] -= 2 * h
                    dn = loss(X["q"], X["k"], X["v"])
                    fd = float((up - dn) / (2 * h))
                    assert abs(grad[0, 0, r, d] - fd) <= 1e-12 * max(1.0, abs(fd)), \
                        (which, r, d, dtype, causal, grad[0, 0, r, d], fd)


def pin_bwd_closed_forms(lib):
    """One key: O_i = v_0 for every row that sees it (every row when
    non-causal; with the bottom-right causal mask only the last one), so dV_0
    is the sum of dO over those rows and dQ = dK = 0.
    Q = 0 (non-causal): P = 1/Sk, so dV_j = (1/Sk) sum_i dO_i and
    dQ_i = (scale/Sk) sum_j (dO_i . (v_j - mean v)) k_j."""
    for dtype in ("f16", "bf16"):
        q, k, v, g = _grad_inputs(2, 2, 13, 1, 16, dtype, seed=50)
        for causal in (False, True):
            dq, dk, dv = _run_bwd(lib, q, k, v, g, 0.25, causal, dtype)
            G = _f64(g)
            assert np.all(dq == 0.0) and np.all(dk == 0.0), (dtype, causal)
            want = G[:, :, -1] if causal else G.sum(axis=2)
            assert np.max(np.abs(dv[:, :, 0] - want)) <= 1e-13, (dtype, causal)
        q, k, v, g = _grad_inputs(1, 2, 20, 31, 8, dtype, seed=51)
        q = torch.zeros_like(q)
        scale = softmax_scale(8)
        dq, dk, dv = _run_bwd(lib, q, k, v, g, scale, False, dtype)
        K, V, G = _f64(k), _f64(v), _f64(g)
        Sk = K.shape[2]
        assert np.max(np.abs(dv - G.sum(axis=2, keepdims=True) / Sk)) <= 1e-13, dtype
        vc = V - V.mean(axis=2, keepdims=True)
        w = np.einsum("bhid,bhjd->bhij", G, vc)
        want = scale / Sk * np.einsum("bhij,bhjd->bhid", w, K)
        assert np.max(np.abs(dq - want)) <= 1e-13, dtype
        assert np.max(np.abs(dk)) == 0.0, dtype


def pin_bwd_invariants(lib):
    """sum_j dK_j = 0 (adding a vector to every key leaves O unchanged); rows of
    P sum to one, so sum_j dV_j = sum of dO over rows that see a key; the
    scores are bilinear in q and k, so sum_i q_i.dQ_i = sum_j k_j.dK_j; a row
    that sees no key has dQ = 0 and its dO reaches no gradient."""
    for dtype, (Sq, Sk), causal, q_mult in (("f16", (48, 48), False, 1.0), ("bf16", (48, 48), True, 4.0),
                                            ("f16", (29, 64), True, 1.0), ("bf16", (64, 29), True, 1.0)):
        q, k, v, g = _grad_inputs(1, 2, Sq, Sk, 16, dtype, seed=60 + Sq, q_mult=q_mult)
        scale = softmax_scale(16)
        dq, dk, dv = _run_bwd(lib, q, k, v, g, scale, causal, dtype)
        Q, K, G = _f64(q), _f64(k), _f64(g)
        big = max(1.0, np.max(np.abs(dk)))
        assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12 * big * Sk, (dtype, Sq, Sk, causal)
        seen = np.array([Sk > 0 and (not causal or i + (Sk - Sq) >= 0) for i in range(Sq)])
        assert np.max(np.abs(dv.sum(axis=2) - G[:, :, seen].sum(axis=2))) <= 1e-12 * Sq
        lhs = np.sum(Q * dq)
        rhs = np.sum(K * dk)
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, np.sum(np.abs(Q * dq))), (dtype, lhs, rhs)
        if not seen.all():
            assert np.all(dq[:, :, ~seen] == 0.0)
            g2 = g.clone()
            g2[:, :, torch.from_numpy(~seen)] = 0
            dq2, dk2, dv2 = _run_bwd(lib, q, k, v, g2, scale, causal, dtype)
            assert np.array_equal(dk2, dk) and np.array_equal(dv2, dv)


def pin_bwd_rows_match_full(lib):
    for dtype, (B, H, Sq, Sk), causal in (("bf16", (2, 3, 65, 65), True), ("f16", (1, 2, 40, 77), False),
                                          ("f16", (1, 2, 50, 30), True)):
        q, k, v, g = _grad_inputs(B, H, Sq, Sk, 32, dtype, seed=70 + Sq)
        scale = softmax_scale(32)
        dq, dk, dv = _run_bwd(lib, q, k, v, g, scale, causal, dtype)
        qr = np.array([0, 1, Sq - 1, Sq, (B * H * Sq) // 2 + 3, B * H * Sq - 1], dtype=np.int64)
        kr = np.array([0, Sk - 1, Sk + 2, B * H * Sk - 1, 5], dtype=np.int64)
        a, b, c = oracle.attention_bwd_rows(bits(q), bits(k), bits(v), bits(g), qr, kr, scale=scale,
                                            causal=causal, dtype=dtype, lib=lib)
        scl = max(1.0, np.max(np.abs(dk)), np.max(np.abs(dv)))
        assert np.max(np.abs(a - dq.reshape(-1, 32)[qr])) <= 1e-13 * scl, dtype
        assert np.max(np.abs(b - dk.reshape(-1, 32)[kr])) <= 1e-13 * scl, dtype
        assert np.max(np.abs(c - dv.reshape(-1, 32)[kr])) <= 1e-13 * scl, dtype


# --- explicit mask and dropout -------------------------------------------------

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pin_philox_kat(lib):
    """Philox4x32-10 against the known-answer vectors published with it."""
    kat = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for vec in kat["vectors"]:
        ctr = [int(x, 16) for x in vec["counter"]]
        key = [int(x, 16) for x in vec["key"]]
        want = [int(x, 16) for x in vec["out"]]
        assert oracle.philox4x32_10(ctr, key, lib=lib) == want, vec


def pin_dropout_threshold(lib):
    for p in (0.0, 0.1, 0.25, 0.5, 1.0 / 3.0, 0.9999):
        want = int(np.rint(np.float32(p) * np.float32(65536.0)))
        assert oracle.dropout_threshold(p, lib=lib) == want, p
    for p in (1.0, 1.5, -0.1, float("nan"), 0.99999999):
        assert oracle.dropout_threshold(p, lib=lib) == -1, p


def _philox_py(ctr, key):
    """Philox4x32-10 written again from its definition (Salmon et al. 2011),
    for the keep pattern check."""
    c0, c1, c2, c3 = ctr
    k0, k1 = key
    for r in range(10):
        if r:
            k0, k1 = (k0 + 0x9E3779B9) & 0xFFFFFFFF, (k1 + 0xBB67AE85) & 0xFFFFFFFF
        p0, p1 = 0xD2511F53 * c0, 0xCD9E8D57 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & 0xFFFFFFFF, p1 & 0xFFFFFFFF, \
            ((p0 >> 32) ^ c3 ^ k1) & 0xFFFFFFFF, p0 & 0xFFFFFFFF
    return c0, c1, c2, c3


def keep_pattern(Sq, Sk, bh, seed, offset, t):
    """keep[i, j] for one head: the 16-bit draw for key j is half j%2 of word
    (j%8)/2 of Philox4x32-10 at counter (j/8, i, bh, offset), key (seed low,
    seed high)."""
    keep = np.zeros((Sq, Sk), dtype=bool)
    for i in range(Sq):
        for jb in range((Sk + 7) // 8):
            out = _philox_py((jb, i, bh, offset), (seed & 0xFFFFFFFF, seed >> 32))
            for j in range(8 * jb, min(Sk, 8 * jb + 8)):
                r16 = (out[(j & 7) >> 1] >> (16 * (j & 1))) & 0xFFFF
                keep[i, j] = r16 >= t
    return keep


def _ext(lib, q, k, v, scale, causal, dtype, **kw):
    return oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=scale, causal=causal,
                                    dtype=dtype, lib=lib, **kw)


def pin_ext_plain_equals_forward(lib):
    """No mask and p = 0 is the forward itself, bit for bit; an all-true mask
    too; a bottom-right lower-triangular mask is the causal flag."""
    for dtype, (Sq, Sk) in (("f16", (40, 40)), ("bf16", (23, 57)), ("f16", (57, 23))):
        q, k, v = make_inputs(2, 2, max(Sq, Sk), 16, dtype, seed=80 + Sq, Sk=Sk)
        q = q[:, :, :Sq].contiguous()
        scale = softmax_scale(16)
        for causal in (False, True):
            o, lse = _run(lib, q, k, v, scale, causal, dtype)
            oe, le = _ext(lib, q, k, v, scale, causal, dtype)
            assert np.array_equal(o, oe) and np.array_equal(lse, le), (dtype, Sq, Sk, causal)
            ones = np.ones((Sq, Sk), np.uint8)
            om, lm = _ext(lib, q, k, v, scale, causal, dtype, mask=ones, mask_strides=(0, 0, Sk))
            assert np.array_equal(o, om) and np.array_equal(lse, lm)
        tri = np.array([[1 if j <= i + (Sk - Sq) else 0 for j in range(Sk)] for i in range(Sq)], np.uint8)
        oc, lc = _run(lib, q, k, v, scale, True, dtype)
        ot, lt = _ext(lib, q, k, v, scale, False, dtype, mask=tri, mask_strides=(0, 0, Sk))
        assert np.array_equal(oc, ot) and np.array_equal(lc, lt), (dtype, Sq, Sk)


def pin_ext_mask_sdpa(lib):
    """A random per-(batch, head) mask against torch's fp64 scaled dot-product
    attention with that boolean mask (True = attend); rows the mask hides
    completely give O = 0, lse = -inf."""
    B, H, Sq, Sk, D = 2, 3, 37, 45, 16
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, "bf16", seed=90, Sk=Sk)
    q = q[:, :, :Sq].contiguous()
    rng = np.random.default_rng(91)
    m = (rng.random((B, H, Sq, Sk)) < 0.6).astype(np.uint8)
    m[0, 1, 5, :] = 0
    m[1, 2, 0, :] = 0
    scale = softmax_scale(D)
    for causal in (False, True):
        o, lse = _ext(lib, q, k, v, scale, causal, "bf16", mask=m,
                      mask_strides=(H * Sq * Sk, Sq * Sk, Sk))
        allow = torch.from_numpy(m.astype(bool))
        if causal:
            i = torch.arange(Sq)[:, None]
            j = torch.arange(Sk)[None, :]
            allow = allow & (j <= i + (Sk - Sq))
        seen = allow.any(-1).numpy()
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(_f64(q)), torch.from_numpy(_f64(k)), torch.from_numpy(_f64(v)),
            attn_mask=allow, scale=scale).numpy()
        assert np.max(np.abs(o[seen] - ref[seen])) <= 1e-12, causal
        assert np.all(o[~seen] == 0.0) and np.all(np.isneginf(lse[~seen])), causal
        # a padded mask row (row stride > Sk) reads the same entries
        wide = np.zeros((B, H, Sq, Sk + 19), np.uint8)
        wide[..., :Sk] = m
        ow, lw = _ext(lib, q, k, v, scale, causal, "bf16", mask=wide,
                      mask_strides=(H * Sq * (Sk + 19), Sq * (Sk + 19), Sk + 19))
        assert np.array_equal(o, ow) and np.array_equal(lse, lw)


def pin_ext_dropout_pattern(lib):
    """With V = the identity (Sk = D), O_i is the probability row P_i itself;
    dropout must give P_ij * keep_ij * 65536 / (65536 - t) with keep from
    Philox4x32-10 at the documented counter, and lse unchanged."""
    Sq, Sk = 20, 32
    q, k, _ = make_inputs(1, 2, Sk, Sk, "f16", seed=95, Sk=Sk)
    q = q[:, :, :Sq].contiguous()
    v = torch.eye(Sk, dtype=torch.float16).expand(1, 2, Sk, Sk).contiguous()
    scale = softmax_scale(Sk)
    # a threshold equal to one draw: that score is kept (the comparison is >=)
    first = _philox_py((0, 0, 0, 11), (17, 0))[0] & 0xFFFF
    assert first > 0
    cases = ((0.25, 0x1234_5678_9ABC_DEF0, 7, False), (0.5, 3, 0, True), (first / 65536.0, 17, 11, False))
    for p, seed, offset, causal in cases:
        t = oracle.dropout_threshold(p, lib=lib)
        o0, l0 = _ext(lib, q, k, v, scale, causal, "f16")
        od, ld = _ext(lib, q, k, v, scale, causal, "f16", dropout_p=p, seed=seed, offset=offset)
        assert np.array_equal(l0, ld)
        for h in range(2):
            keep = keep_pattern(Sq, Sk, h, seed, offset, t)
            want = o0[0, h] * keep * (65536.0 / (65536.0 - t))
            assert np.max(np.abs(od[0, h] - want)) <= 1e-15, (p, h)


def pin_ext_dropout_rate(lib):
    """Over 64k scores the kept fraction is 1 - t/65536 within 5 sigma, and
    another offset gives another pattern."""
    S = 256
    q, k, _ = make_inputs(1, 1, S, S, "f16", seed=96)
    q = torch.zeros_like(q)                      # P = 1/S everywhere
    v = torch.eye(S, dtype=torch.float16)[None, None].contiguous()
    t = oracle.dropout_threshold(0.1, lib=lib)
    o1, _ = _ext(lib, q, k, v, 1.0, False, "f16", dropout_p=0.1, seed=42, offset=0)
    o2, _ = _ext(lib, q, k, v, 1.0, False, "f16", dropout_p=0.1, seed=42, offset=1)
    kept = o1 != 0
    pk = 1 - t / 65536.0
    sigma = math.sqrt(pk * (1 - pk) / kept.size)
    assert abs(kept.mean() - pk) <= 5 * sigma, kept.mean()
    assert np.allclose(o1[kept], 1.0 / S * 65536.0 / (65536.0 - t), rtol=1e-15, atol=0)
    assert (kept != (o2 != 0)).mean() > 0.1


def pin_ext_rows_match_full(lib):
    B, H, Sq, Sk, D = 2, 2, 50, 70, 32
    q, k, v = make_inputs(B, H, Sk, D, "bf16", seed=97, Sk=Sk)
    q = q[:, :, :Sq].contiguous()
    m = (np.random.default_rng(98).random((Sq, Sk)) < 0.8).astype(np.uint8)
    kw = dict(mask=m, mask_strides=(0, 0, Sk), dropout_p=0.2, seed=5, offset=9)
    o, lse = _ext(lib, q, k, v, softmax_scale(D), True, "bf16", **kw)
    rows = np.array([0, 3, Sq - 1, Sq, 2 * Sq + 7, B * H * Sq - 1], np.int64)
    ro, rl = _ext(lib, q, k, v, softmax_scale(D), True, "bf16", rows=rows, **kw)
    assert np.array_equal(ro, o.reshape(-1, D)[rows]) and np.array_equal(rl, lse.reshape(-1)[rows])


def _bwd_ext(lib, q, k, v, g, scale, causal, dtype, **kw):
    return oracle.attention_bwd_ext(bits(q), bits(k), bits(v), bits(g), scale=scale, causal=causal,
                                    dtype=dtype, lib=lib, **kw)


def pin_bwd_ext_plain_equals_bwd(lib):
    """No mask and p = 0: the backward of the plain forward."""
    for dtype, (Sq, Sk), causal in (("f16", (40, 40), True), ("bf16", (23, 57), False), ("f16", (57, 23), True)):
        q, k, v, g = _grad_inputs(1, 2, Sq, Sk, 16, dtype, seed=100 + Sq)
        a = _run_bwd(lib, q, k, v, g, softmax_scale(16), causal, dtype)
        b = _bwd_ext(lib, q, k, v, g, softmax_scale(16), causal, dtype)
        for x, y in zip(a, b):
            assert np.max(np.abs(x - y)) <= 1e-13 * max(1.0, np.max(np.abs(x))), (dtype, Sq, Sk)


def _keep_matrix(B, H, Sq, Sk, seed, offset, p):
    t = int(np.rint(np.float32(p) * np.float32(65536.0)))
    z = np.zeros((B, H, Sq, Sk))
    for bh in range(B * H):
        z[bh // H, bh % H] = keep_pattern(Sq, Sk, bh, seed, offset, t) * (65536.0 / (65536.0 - t))
    return z


def pin_bwd_ext_autograd(lib):
    """torch autograd in fp64 through softmax(masked scores) * Z * c @ V, with
    the keep matrix from the Philox written in this file: the oracle's
    gradients with a per-head mask and dropout."""
    for dtype, (B, H, Sq, Sk, D), causal, p in (("f16", (1, 2, 30, 41, 16), True, 0.25),
                                                ("bf16", (2, 1, 33, 33, 8), False, 0.5)):
        q, k, v, g = _grad_inputs(B, H, Sq, Sk, D, dtype, seed=110 + Sq)
        rng = np.random.default_rng(111 + Sq)
        m = (rng.random((B, H, Sq, Sk)) < 0.7).astype(np.uint8)
        m[0, 0, 2, :] = 0
        ms = (H * Sq * Sk, Sq * Sk, Sk)
        seed, offset = 0xABCDEF012345, 3
        scale = softmax_scale(D)
        dq, dk, dv = _bwd_ext(lib, q, k, v, g, scale, causal, dtype, mask=m, mask_strides=ms,
                              dropout_p=p, seed=seed, offset=offset)
        allow = torch.from_numpy(m.astype(bool))
        if causal:
            i = torch.arange(Sq)[:, None]
            j = torch.arange(Sk)[None, :]
            allow = allow & (j <= i + (Sk - Sq))
        Z = torch.from_numpy(_keep_matrix(B, H, Sq, Sk, seed, offset, p))
        Q, K, V = (torch.from_numpy(_f64(t)).requires_grad_() for t in (q, k, v))
        s = (scale * Q @ K.transpose(-1, -2)).masked_fill(~allow, float("-inf"))
        P = torch.softmax(s, dim=-1).nan_to_num(0.0)
        o = (P * Z) @ V
        (o * torch.from_numpy(_f64(g))).sum().backward()
        for name, got, ref in (("dq", dq, Q.grad), ("dk", dk, K.grad), ("dv", dv, V.grad)):
            ref = ref.numpy()
            err = np.max(np.abs(got - ref))
            assert err <= 1e-12 * max(1.0, np.max(np.abs(ref))), (name, dtype, err)
        assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12 * max(1.0, np.max(np.abs(dk))) * Sk


def pin_bwd_ext_finite_difference(lib):
    """Central differences of the 40-digit forward with a mask and dropout."""
    getcontext().prec = 40
    Sq, Sk, D, p = 3, 8, 2, 0.5
    q, k, v, g = _grad_inputs(1, 1, Sq, Sk, D, "f16", seed=120)
    m = np.array([[1, 1, 0, 1, 1, 1, 0, 1], [0, 1, 1, 1, 1, 0, 1, 1], [1, 0, 1, 1, 0, 1, 1, 1]], np.uint8)
    seed, offset = 77, 1
    scale = softmax_scale(D)
    dq, dk, dv = _bwd_ext(lib, q, k, v, g, scale, False, "f16", mask=m, mask_strides=(0, 0, Sk),
                          dropout_p=p, seed=seed, offset=offset)
    Z = _keep_matrix(1, 1, Sq, Sk, seed, offset, p)[0, 0]
    Q, K, V, G = (_f64(t)[0, 0] for t in (q, k, v, g))
    sc = Decimal(scale)

    def loss(Qx, Kx, Vx):
        tot = Decimal(0)
        for i in range(Sq):
            ws, num, den = [], [Decimal(0)] * D, Decimal(0)
            for j in range(Sk):
                if not m[i, j]:
                    continue
                w = (sc * sum(Qx[i][d] * Kx[j][d] for d in range(D))).exp()
                den += w
                for d in range(D):
                    num[d] += w * Decimal(float(Z[i, j])) * Vx[j][d]
            for d in range(D):
                tot += num[d] / den * Decimal(float(G[i, d]))
        return tot

    dec = lambda A: [[Decimal(float(x)) for x in row] for row in A]
    h = Decimal("1e-12")
    for which, grad, rows in (("q", dq, Sq), ("k", dk, Sk), ("v", dv, Sk)):
        for r in range(rows):
            for d in range(D):
                X = {"q": dec(Q), "k": dec(K), "v": dec(V)}
                X[which][r][d] += h
                up = loss(X["q"], X["k"], X["v"])
                X[which][r][d] -= 2 * h
                dn = loss(X["q"], X["k"], X["v"])
                fd = float((up - dn) / (2 * h))
                assert abs(grad[0, 0, r, d] - fd) <= 1e-12 * max(1.0, abs(fd)), (which, r, d, grad[0, 0, r, d], fd)


def pin_bwd_ext_rows_match_full(lib):
    B, H, Sq, Sk, D = 2, 2, 45, 60, 16
    q, k, v, g = _grad_inputs(B, H, Sq, Sk, D, "bf16", seed=130)
    m = (np.random.default_rng(131).random((Sq, Sk)) < 0.8).astype(np.uint8)
    kw = dict(mask=m, mask_strides=(0, 0, Sk), dropout_p=0.2, seed=9, offset=2)
    dq, dk, dv = _bwd_ext(lib, q, k, v, g, softmax_scale(D), True, "bf16", **kw)
    qr = np.array([0, 5, Sq - 1, 2 * Sq + 1, B * H * Sq - 1], np.int64)
    kr = np.array([0, Sk + 3, 3 * Sk - 1, B * H * Sk - 1], np.int64)
    a, b, c = _bwd_ext(lib, q, k, v, g, softmax_scale(D), True, "bf16", qrows=qr, krows=kr, **kw)
    scl = max(1.0, np.max(np.abs(dk)), np.max(np.abs(dv)), np.max(np.abs(dq)))
    assert np.max(np.abs(a - dq.reshape(-1, D)[qr])) <= 1e-13 * scl
    assert np.max(np.abs(b - dk.reshape(-1, D)[kr])) <= 1e-13 * scl
    assert np.max(np.abs(c - dv.reshape(-1, D)[kr])) <= 1e-13 * scl


def pin_causal_offset_blocks(lib):
    """A causal sequence of 90 tokens cut into chunks [0, 25), [25, 60),
    [60, 90) for queries and keys: block (a, b) computed with the diagonal at
    offset qs_a - ks_b (global position ks_b + j visible to qs_a + i iff
    ks_b + j <= qs_a + i), then merged over b by log-sum-exp, equals the
    one-shot causal forward on the whole sequence; blocks wholly in the
    future give O = 0 and lse = -inf."""
    S, D, dtype = 90, 16, "f16"
    q, k, v = make_inputs(2, 2, S, D, dtype, seed=140)
    scale = softmax_scale(D)
    o, lse = _run(lib, q, k, v, scale, True, dtype)
    cuts = ((0, 25), (25, 60), (60, 90))
    for qa, qb in cuts:
        parts = []
        for ka, kb in cuts:
            po, pl = _ext(lib, q[:, :, qa:qb].contiguous(), k[:, :, ka:kb].contiguous(),
                          v[:, :, ka:kb].contiguous(), scale, True, dtype, causal_offset=qa - ka)
            if ka > qb - 1:
                assert np.all(po == 0.0) and np.all(np.isneginf(pl)), (qa, ka)
            parts.append((po, pl))
        lse_m = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
        o_m = sum(np.where(np.isneginf(p[1]), 0.0, np.exp(p[1] - lse_m))[..., None] * p[0] for p in parts)
        assert np.max(np.abs(lse_m - lse[:, :, qa:qb])) <= 1e-12, (qa, qb)
        assert np.max(np.abs(o_m - o[:, :, qa:qb])) <= 1e-12, (qa, qb)


def pin_causal_offset_as_mask(lib):
    """The diagonal at offset c equals the explicit mask j <= i + c on a
    non-causal call, bit for bit, in the forward (with dropout) and the
    backward, for offsets that hide every key, some, the bottom-right and
    top-left diagonals, and none."""
    Sq, Sk, D, dtype = 21, 34, 16, "bf16"
    q, k, v, g = _grad_inputs(1, 2, Sq, Sk, D, dtype, seed=150)
    scale = softmax_scale(D)
    kw = dict(dropout_p=0.25, seed=31, offset=4)
    for c in (-Sq - 3, -5, 0, 4, Sk - Sq, Sk + 2):
        tri = np.array([[1 if j <= i + c else 0 for j in range(Sk)] for i in range(Sq)], np.uint8)
        ms = dict(mask=tri, mask_strides=(0, 0, Sk))
        oc, lc = _ext(lib, q, k, v, scale, True, dtype, causal_offset=c, **kw)
        om, lm = _ext(lib, q, k, v, scale, False, dtype, **ms, **kw)
        assert np.array_equal(oc, om) and np.array_equal(lc, lm), c
        a = _bwd_ext(lib, q, k, v, g, scale, True, dtype, causal_offset=c, **kw)
        b = _bwd_ext(lib, q, k, v, g, scale, False, dtype, **ms, **kw)
        for x, y in zip(a, b):
            assert np.array_equal(x, y), c
    # the default is the bottom-right diagonal
    oc, lc = _ext(lib, q, k, v, scale, True, dtype, causal_offset=Sk - Sq)
    od, ld = _ext(lib, q, k, v, scale, True, dtype)
    assert np.array_equal(oc, od) and np.array_equal(lc, ld)


ALL_PINS = [pin_decode_f16, pin_decode_bf16, pin_q_zero, pin_causal_row0, pin_convexity,
            pin_bruteforce_decimal, pin_sdpa_fp64, pin_chunk_merge, pin_invariances,
            pin_rows_match_full, pin_unequal_causal_suffix, pin_bwd_autograd,
            pin_bwd_finite_difference, pin_bwd_closed_forms, pin_bwd_invariants,
            pin_bwd_rows_match_full, pin_philox_kat, pin_dropout_threshold,
            pin_ext_plain_equals_forward, pin_ext_mask_sdpa, pin_ext_dropout_pattern,
            pin_ext_dropout_rate, pin_ext_rows_match_full, pin_bwd_ext_plain_equals_bwd,
            pin_bwd_ext_autograd, pin_bwd_ext_finite_difference, pin_bwd_ext_rows_match_full,
            pin_causal_offset_blocks, pin_causal_offset_as_mask]
