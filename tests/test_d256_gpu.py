"""GPU parity of head dimension 256 against the fp64 oracle: the forward
(the tuned kernel's pair split behind fa_fwd, fa_fwd_strided and
fa_fwd_ext at D = 256) and the backward (fa_bwd / fa_bwd_strided kernels at
D = 256, with a mask and dropout, on strided views)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import tiled_attention_15_amd as fa
from workloads import bits, make_inputs, softmax_scale

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
D = 256


def say(*a):
    print(*a, flush=True)


def to64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


@pytest.mark.parametrize("B,H,S,causal,dtype", [(1, 2, 64, False, "f16"), (1, 2, 257, True, "bf16"),
                                                (2, 1, 1, True, "f16"), (1, 3, 700, False, "bf16"),
                                                (2, 2, 333, True, "f16")])
def test_d256_forward_matches_oracle(B, H, S, causal, dtype):
    say("case d256", B, H, S, causal, dtype)
    q, k, v = make_inputs(B, H, S, D, dtype, seed=2500 + S)
    o, lse = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_fwd(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=causal,
                                        dtype=dtype)
    say("  ", parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, "d256 S%d" % S))


@pytest.mark.parametrize("Sq,Sk,causal", [(100, 300, True), (300, 100, True), (130, 67, False)])
def test_d256_strided_unequal_lengths(Sq, Sk, causal):
    """[B, S, H, D] tensors viewed as [B, H, S, D] (fa_fwd_strided), Sq != Sk."""
    B, H = 2, 3
    q, _, _ = make_inputs(B, H, Sq, D, "bf16", seed=2600 + Sq)
    _, k, v = make_inputs(B, H, Sk, D, "bf16", seed=2650 + Sk)
    qs = q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    ks = k.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    vs = v.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    say("case d256 strided", Sq, Sk, causal)
    o, lse = fa.forward(qs, ks, vs, causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_fwd(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=causal,
                                        dtype="bf16")
    say("  ", parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, "bf16", "d256 strided"))


def test_d256_mask_and_dropout():
    B, H, Sq, Sk = 1, 2, 190, 150
    q, _, _ = make_inputs(B, H, Sq, D, "f16", seed=2700)
    _, k, v = make_inputs(B, H, Sk, D, "f16", seed=2701)
    ld = (Sk + 3) // 4 * 4
    m = np.zeros((B, H, Sq, ld), np.uint8)
    m[..., :Sk] = np.random.default_rng(2702).random((B, H, Sq, Sk)) < 0.75
    ms = (H * Sq * ld, Sq * ld, ld)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    st = fa.fa_fwd_ext(qd, kd, vd, o, lse, B, H, Sq, Sk, D, torch.from_numpy(m).to(DEV), ms, 0.2, 99, 4,
                       softmax_scale(D), True, fa.F16, None)
    assert st == 0
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=True,
                                            dtype="f16", mask=m, mask_strides=ms, dropout_p=0.2, seed=99,
                                            offset=4)
    say("  ", parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, "f16", "d256 mask dropout"))


def _grad_inputs(B, H, Sq, Sk, dtype, seed):
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=seed, Sk=Sk)
    q = q[:, :, :Sq].contiguous()
    g, _, _ = make_inputs(B, H, Sq, D, dtype, seed=seed + 1000)
    return q, k, v, g


def _zero_scales(q, k, v, g, dtype="bf16", p=0.0):
    return parity.cancellation_tolerances(q, k, v, g, softmax_scale(D), dtype, dropout_p=p)


BWD_CASES = [
    # (B, H, Sq, Sk, causal, dtype)
    (1, 2, 64, 64, False, "f16"),
    (1, 2, 257, 257, True, "bf16"),
    (2, 1, 1, 1, True, "f16"),
    (1, 1, 100, 300, True, "bf16"),
    (1, 2, 300, 100, True, "f16"),
    (2, 2, 130, 67, False, "bf16"),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=["%dx%dx%dx%d%s%s" % (c[0], c[1], c[2], c[3], "c" if c[4] else "n",
                                                                      c[5]) for c in BWD_CASES])
def test_d256_backward_matches_oracle(case):
    B, H, Sq, Sk, causal, dtype = case
    say("case d256 bwd", case)
    q, k, v, g = _grad_inputs(B, H, Sq, Sk, dtype, seed=2800 + Sq + 3 * Sk)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.forward(qd, kd, vd, causal=causal)
    grads = fa.backward(qd, kd, vd, o, lse, gd, causal=causal)
    torch.cuda.synchronize()
    refs = oracle.attention_bwd(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=causal,
                                dtype=dtype)
    zs = _zero_scales(q, k, v, g, dtype)
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        say("  ", name, parity.assert_grad_parity(to64(got), ref, dtype, "d256 %s %s" % (name, case),
                                                  zero_tol=zs[name]))


def test_d256_backward_mask_dropout_strided():
    """Masked and dropout backward at D = 256 on [B, S, H, D] views: equal to
    the contiguous call bit for bit, and within the oracle's bound."""
    B, H, Sq, Sk, dtype = 1, 2, 150, 172, "bf16"
    say("case d256 bwd mask dropout", B, H, Sq, Sk, dtype)
    q, k, v, g = _grad_inputs(B, H, Sq, Sk, dtype, seed=2900)
    rng = np.random.default_rng(2901)
    mask = (rng.random((Sq, Sk)) < 0.8).astype(np.uint8)
    kw = dict(causal=True, mask=torch.from_numpy(mask).to(DEV), dropout_p=0.1, seed=21, offset=3)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.forward_ext(qd, kd, vd, **kw)
    ref = fa.backward_ext(qd, kd, vd, o, lse, gd, **kw)
    views = [t.transpose(1, 2).contiguous().transpose(1, 2) for t in (qd, kd, vd, o, gd)]
    got = fa.backward_ext(views[0], views[1], views[2], views[3], lse, views[4], **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name
    refs = oracle.attention_bwd_ext(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=True,
                                    dtype=dtype, mask=mask, mask_strides=(0, 0, Sk), dropout_p=0.1, seed=21,
                                    offset=3)
    zs = _zero_scales(q, k, v, g, dtype, 0.1)
    for name, a, r in zip(("dq", "dk", "dv"), got, refs):
        say("  ", name, parity.assert_grad_parity(to64(a), r, dtype, "d256 ext %s" % name, zero_tol=zs[name]))
