"""CPU checks of parity.operand_rounding_bounds, the per-element gradient
bound used for inputs whose gradients cancel far below their terms.

The backward's arithmetic model (one factor of each product rounded to the
input dtype, D_i from the output as stored) is emulated in fp64 with torch's rounding to fp16/bf16; its
gradients must lie within the bound of the fp64 oracle's, and two planted
mistakes in the emulation (dS without its D_i term; dV with every row's
probabilities taken from the next row) must not.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import parity
from workloads import bits, make_inputs, softmax_scale, torch_dtype


def rising_inputs(Sq, Sk, D, dtype, seed):
    q, k, v = make_inputs(1, 1, max(Sq, Sk), D, dtype, seed=seed, Sk=Sk, dist="uniform")
    q = q[:, :, :Sq].float() * 0.1
    k = k.float() * 0.1
    scale = softmax_scale(D)
    q[..., 0] = torch.from_numpy(1.0 + 0.25 * (np.arange(Sq) % 3)).float()
    k[..., 0] = torch.from_numpy(300.0 * np.arange(Sk) / (Sk - 1) / scale).float()
    g, _, _ = make_inputs(1, 1, Sq, D, dtype, seed=seed + 1, dist="uniform")
    td = torch_dtype(dtype)
    return q.to(td), k.to(td), v, g


def emulate(q, k, v, g, scale, causal, dtype, o, lse, mistake=None):
    """Gradients with P and dS rounded to `dtype` before their products and
    D_i formed from the output as stored (rounded to `dtype`)."""
    f = lambda t: t.double().numpy()
    qa, ka, va, ga = f(q), f(k), f(v), f(g)
    Sq, Sk = qa.shape[-2], ka.shape[-2]
    s = scale * qa @ np.swapaxes(ka, -1, -2)
    if causal:
        vis = np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] + (Sk - Sq)
        s = np.where(vis, s, -np.inf)
    p = np.exp(s - lse[..., None])
    dp = ga @ np.swapaxes(va, -1, -2)
    rnd = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch_dtype(dtype)).double().numpy()
    di = 0.0 if mistake == "no_di" else np.sum(ga * rnd(o), axis=-1, keepdims=True)
    ds = p * (dp - di)
    pr, dsr = rnd(p), rnd(ds)
    if mistake == "row_shift":
        pr = np.roll(pr, -1, axis=-2)
    dq = scale * dsr @ ka
    dk = scale * np.swapaxes(dsr, -1, -2) @ qa
    dv = np.swapaxes(pr, -1, -2) @ ga
    return {"dq": dq, "dk": dk, "dv": dv}


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_emulated_rounding_within_bound_and_mistakes_outside(dtype, causal):
    Sq, Sk, D = 96, 160, 32
    scale = softmax_scale(D)
    q, k, v, g = rising_inputs(Sq, Sk, D, dtype, seed=61 + causal)
    refs = dict(zip(("dq", "dk", "dv"), oracle.attention_bwd(bits(q), bits(k), bits(v), bits(g), scale=scale,
                                                              causal=causal, dtype=dtype)))
    o, lse = oracle.attention_fwd(bits(q), bits(k), bits(v), scale=scale, causal=causal, dtype=dtype)
    bnd = parity.operand_rounding_bounds(q, k, v, g, o, lse, scale, causal, dtype)
    for name in ("dq", "dk", "dv"):
        assert np.all(bnd[name] >= 0.0) and np.isfinite(bnd[name]).all()
    emu = emulate(q, k, v, g, scale, causal, dtype, o, lse)
    for name in ("dq", "dk", "dv"):
        parity.assert_grad_within_bound(emu[name], refs[name], bnd[name], dtype, "emulated " + name)
    # the slice-wide rule does reject these honest rounding errors of dQ
    assert not parity.grad_ok(parity.compare_grad(emu["dq"], refs["dq"], dtype))
    bad = emulate(q, k, v, g, scale, causal, dtype, o, lse, mistake="no_di")
    with pytest.raises(AssertionError):
        parity.assert_grad_within_bound(bad["dq"], refs["dq"], bnd["dq"], dtype, "no D_i")
    bad = emulate(q, k, v, g, scale, causal, dtype, o, lse, mistake="row_shift")
    with pytest.raises(AssertionError):
        parity.assert_grad_within_bound(bad["dv"], refs["dv"], bnd["dv"], dtype, "row shift")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bound_with_mask_and_dropout(dtype):
    """The same with an explicit mask and dropout (keep factors from the
    Philox pattern of the oracle pins): the emulation, with P Z c in the
    products, lies within the bound; dS formed without the keep factors
    does not."""
    from oracle_pins import _keep_matrix
    Sq, Sk, D, p, seed, offset = 40, 70, 32, 0.2, 21, 4
    scale = softmax_scale(D)
    q, k, v, g = rising_inputs(Sq, Sk, D, dtype, seed=71)
    m = (np.random.default_rng(72).random((1, 1, Sq, Sk)) < 0.7).astype(np.uint8)
    ms = (0, 0, Sk)
    refs = dict(zip(("dq", "dk", "dv"), oracle.attention_bwd_ext(
        bits(q), bits(k), bits(v), bits(g), scale=scale, causal=True, dtype=dtype, mask=m[0, 0], mask_strides=ms,
        dropout_p=p, seed=seed, offset=offset)))
    o, lse = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=scale, causal=True, dtype=dtype, mask=m[0, 0],
                                      mask_strides=ms, dropout_p=p, seed=seed, offset=offset)
    vis = (m != 0) & (np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] + (Sk - Sq))
    zc = _keep_matrix(1, 1, Sq, Sk, seed, offset, p)
    bnd = parity.operand_rounding_bounds(q, k, v, g, o, lse, scale, True, dtype, vis=vis, zc=zc)

    f = lambda t: t.double().numpy()
    qa, ka, va, ga = f(q), f(k), f(v), f(g)
    rnd = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch_dtype(dtype)).double().numpy()
    s = np.where(vis, scale * qa @ np.swapaxes(ka, -1, -2), -np.inf)
    pm = np.exp(s - lse[..., None])
    dp = ga @ np.swapaxes(va, -1, -2)
    di = np.sum(ga * rnd(o), axis=-1, keepdims=True)
    for name, ds in (("emulated", pm * (zc * dp - di)), ("no keep factor in dS", pm * (dp - di))):
        emu = {"dq": scale * rnd(ds) @ ka, "dk": scale * np.swapaxes(rnd(ds), -1, -2) @ qa,
               "dv": np.swapaxes(rnd(pm * zc), -1, -2) @ ga}
        if name == "emulated":
            for gname in ("dq", "dk", "dv"):
                parity.assert_grad_within_bound(emu[gname], refs[gname], bnd[gname], dtype, "emulated " + gname)
        else:
            with pytest.raises(AssertionError):
                parity.assert_grad_within_bound(emu["dq"], refs["dq"], bnd["dq"], dtype, name)
