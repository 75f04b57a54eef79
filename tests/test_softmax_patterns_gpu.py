"""GPU parity of the online softmax under score patterns that drive its
running maximum (FlashAttention-2, the forward's per-block max, rescale of
the partial output and of the row sum), against the fp64 oracle.

The scores are shaped through one head-dimension channel: q[i, 0] = c_i and
k[j, 0] = f(j) / scale, so row i's score for key j is c_i f(j) plus small
noise from the other channels.  Patterns of f over the key index:

  rising     f grows linearly to ~300 (natural-log units): the row maximum
             moves up on every tile, by more than the kernel's staleness
             bound (8 in log2 units) each time;
  falling    the reverse: the first tile holds the maximum, later tiles
             underflow to zero;
  spike      noise everywhere and one key near the end ~200 above the rest:
             a late rescale by a factor that underflows to zero;
  steps_in   a staircase rising 5 per 64-key tile (7.2 log2 units, inside
             the bound: the stale maximum is kept for a tile, then moved);
  steps_out  a staircase rising 12 per tile (17.3 log2 units: a rescale on
             every tile).

Each pattern runs on small grids (the key-split instance), on grids of more
than 256 blocks (the 256-row instance) and at D = 256, causal and not, f16
and bf16 (the masked and dropout instances on two of them); the backward
(which recomputes the probabilities from the saved lse) runs on the small
grids, each gradient element held to the bound of the operand rounding
(parity.operand_rounding_bounds).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import tiled_attention_15_amd as fa
from workloads import bits, make_inputs, softmax_scale, torch_dtype

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def to64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def profile(pattern, Sk):
    j = np.arange(Sk, dtype=np.float64)
    if pattern == "rising":
        return 300.0 * j / max(1, Sk - 1)
    if pattern == "falling":
        return 300.0 * (Sk - 1 - j) / max(1, Sk - 1)
    if pattern == "spike":
        f = np.zeros(Sk)
        f[max(0, Sk - 5)] = 200.0
        return f
    if pattern == "steps_in":
        return 5.0 * (j // 64)
    if pattern == "steps_out":
        return 12.0 * (j // 64)
    raise ValueError(pattern)


def shaped_inputs(B, H, Sq, Sk, D, dtype, pattern, seed):
    """q, k, v (CPU, dtype) with scores c_i f(j) + noise; c_i in {1, 1.25, 1.5}."""
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=seed, Sk=Sk, dist="uniform")
    q = q[:, :, :Sq].float() * 0.1
    k = k.float() * 0.1
    scale = softmax_scale(D)
    q[..., 0] = torch.from_numpy(1.0 + 0.25 * (np.arange(Sq) % 3)).float()
    k[..., 0] = torch.from_numpy(profile(pattern, Sk) / scale).float()
    td = torch_dtype(dtype)
    return q.to(td).contiguous(), k.to(td).contiguous(), v.contiguous()


PATTERNS = ["rising", "falling", "spike", "steps_in", "steps_out"]
SHAPES = [
    # (B, H, Sq, Sk, D, dtype, causal): two key-split grids, two 256-row-instance grids, D = 256
    (1, 2, 700, 700, 128, "bf16", True),
    (2, 1, 333, 900, 64, "f16", False),
    (1, 130, 333, 333, 128, "f16", True),
    (1, 136, 300, 420, 128, "bf16", False),
    (1, 2, 300, 500, 256, "bf16", True),     # D = 256: the pair split
]


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("shape", SHAPES, ids=["%dx%dx%dx%dx%d%s%s" % (s[0], s[1], s[2], s[3], s[4], s[5],
                                                                     "c" if s[6] else "n") for s in SHAPES])
def test_running_max_patterns(shape, pattern):
    B, H, Sq, Sk, D, dtype, causal = shape
    say("case softmax pattern", pattern, shape)
    q, k, v = shaped_inputs(B, H, Sq, Sk, D, dtype, pattern, seed=5100 + Sq + Sk + H)
    o = torch.full((B, H, Sq, D), float("nan"), dtype=q.dtype, device=DEV)
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=DEV)
    fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, out=o, lse_out=lse)
    torch.cuda.synchronize()
    og, lg = to64(o), to64(lse)
    assert not np.isnan(og).any() and not np.isnan(lg).any()
    BH = B * H
    if BH <= 2:
        rows = np.arange(BH * Sq, dtype=np.int64)
    else:
        # every row of two heads, 48 random rows of every other head
        rng = np.random.default_rng(Sq + Sk)
        rows = [h * Sq + np.arange(Sq) for h in (0, BH - 1)]
        rows += [h * Sq + rng.choice(Sq, 48, replace=False) for h in range(1, BH - 1)]
        rows = np.unique(np.concatenate(rows)).astype(np.int64)
    o_ref, l_ref = oracle.attention_rows(bits(q), bits(k), bits(v), rows, scale=softmax_scale(D), causal=causal,
                                         dtype=dtype)
    st = parity.assert_parity(og.reshape(-1, D)[rows], lg.reshape(-1)[rows], o_ref, l_ref, dtype,
                              "%s %s" % (pattern, shape))
    say("  ", rows.size, "rows", st)


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("shape", SHAPES[:2] + SHAPES[4:],
                         ids=["%dx%dx%dx%dx%d%s%s" % (s[0], s[1], s[2], s[3], s[4], s[5], "c" if s[6] else "n")
                              for s in SHAPES[:2] + SHAPES[4:]])
def test_running_max_patterns_backward(shape, pattern):
    B, H, Sq, Sk, D, dtype, causal = shape
    say("case softmax pattern backward", pattern, shape)
    q, k, v = shaped_inputs(B, H, Sq, Sk, D, dtype, pattern, seed=5200 + Sq + Sk + H)
    g, _, _ = make_inputs(B, H, Sq, D, dtype, seed=5300 + Sq, dist="uniform")
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.forward(qd, kd, vd, causal=causal)
    grads = fa.backward(qd, kd, vd, o, lse, gd, causal=causal)
    torch.cuda.synchronize()
    refs = oracle.attention_bwd(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=causal,
                                dtype=dtype)
    # These scores come from one large channel: the probable keys' k_j are
    # large and nearly equal, so dQ (and dK) cancel far below their terms and
    # the slice-wide rule does not apply; each element is held to the bound
    # of the backward's operand rounding instead.
    o_ref, l_ref = oracle.attention_fwd(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=causal,
                                        dtype=dtype)
    bnd = parity.operand_rounding_bounds(q, k, v, g, o_ref, l_ref, softmax_scale(D), causal, dtype)
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        st = parity.assert_grad_within_bound(to64(got), ref, bnd[name], dtype, "%s %s %s" % (name, pattern, shape))
        say("  ", name, st)


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("shape", [SHAPES[0], SHAPES[2]], ids=["1x2x700x700x128bf16c", "1x130x333x333x128f16c"])
def test_running_max_patterns_masked_dropout(shape, pattern):
    """The masked and dropout instances on the same profiles: a shared mask
    keeping 80% of the scores (-inf entries among the maxima) and dropout
    0.1 applied to the probabilities after the softmax."""
    B, H, Sq, Sk, D, dtype, causal = shape
    say("case softmax pattern masked/dropout", pattern, shape)
    q, k, v = shaped_inputs(B, H, Sq, Sk, D, dtype, pattern, seed=5400 + Sq + Sk + H)
    mask = (np.random.default_rng(5450 + Sq).random((Sq, Sk)) < 0.8).astype(np.uint8)
    kw = dict(causal=causal, mask=torch.from_numpy(mask).to(DEV), dropout_p=0.1, seed=17, offset=5)
    o, lse = fa.forward_ext(q.to(DEV), k.to(DEV), v.to(DEV), **kw)
    torch.cuda.synchronize()
    og, lg = to64(o), to64(lse)
    BH = B * H
    if BH <= 2:
        rows = np.arange(BH * Sq, dtype=np.int64)
    else:
        rng = np.random.default_rng(Sq + Sk + 1)
        rows = [h * Sq + np.arange(Sq) for h in (0, BH - 1)]
        rows += [h * Sq + rng.choice(Sq, 24, replace=False) for h in range(1, BH - 1)]
        rows = np.unique(np.concatenate(rows)).astype(np.int64)
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=causal,
                                            dtype=dtype, mask=mask, mask_strides=(0, 0, Sk), dropout_p=0.1,
                                            seed=17, offset=5, rows=rows)
    st = parity.assert_parity(og.reshape(-1, D)[rows], lg.reshape(-1)[rows], o_ref, l_ref, dtype,
                              "masked/dropout %s %s" % (pattern, shape))
    say("  ", rows.size, "rows", st)
