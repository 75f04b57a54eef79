"""GPU parity of the causal rule with the diagonal at an explicit offset
(fa_fwd_causal_offset, fa_bwd_causal_offset; key j visible to query i iff
j <= i + c) against the fp64 oracle: offsets that hide every key, some keys,
the top-left and bottom-right diagonals and none, on key-split, unsplit and
D = 256 grids, with a mask and dropout; the bottom-right offset bit-equal to
the plain causal call; and a causal sequence computed as blocks of a split
sequence (c = query chunk start - key chunk start) and merged by log-sum-exp
against the one-shot causal forward."""
import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import tiled_attention_15_amd as fa
from workloads import bits, make_inputs, softmax_scale

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def to64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def inputs(B, H, Sq, Sk, D, dtype, seed):
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=seed, Sk=Sk)
    g, _, _ = make_inputs(B, H, Sq, D, dtype, seed=seed + 1)
    return q[:, :, :Sq].contiguous(), k, v, g


def shared_mask(Sq, Sk, seed):
    ld = (Sk + 3) // 4 * 4
    m = np.zeros((Sq, ld), np.uint8)
    m[:, :Sk] = np.random.default_rng(seed).random((Sq, Sk)) < 0.8
    return m, (0, 0, ld)


# (B, H, Sq, Sk, D, dtype, mask, p, offsets); the 1x2 grids take the key
# split, 2x130x300 the unsplit 256-row instance, D = 256 the pair split
CASES = [
    (1, 2, 300, 200, 64, "f16", False, 0.0, (-305, -40, 0, 17)),
    (1, 2, 170, 420, 128, "bf16", True, 0.2, (0, 250, 425)),
    (2, 130, 300, 300, 64, "f16", False, 0.1, (-37, 0, 64)),
    (1, 2, 260, 190, 256, "bf16", True, 0.0, (-70, 0, 33)),
]


def _fwd(q, k, v, causal_offset, mask, ms, p, seed):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=DEV)
    st = [x for t in (qd, kd, vd, o) for x in t.stride()[:3]]
    md = None if mask is None else torch.from_numpy(mask).to(DEV)
    code = fa.BF16 if q.dtype == torch.bfloat16 else fa.F16
    rc = fa.fa_fwd_causal_offset(qd, kd, vd, o, lse, B, H, Sq, Sk, D, st, md, ms, p, seed, 3, softmax_scale(D),
                                 causal_offset, code, None)
    assert rc == 0, fa.fa_status_string(rc)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("case", CASES, ids=["%dx%dx%dx%dx%d%s%s_p%g" % (c[0], c[1], c[2], c[3], c[4], c[5],
                                                                        "_mask" if c[6] else "", c[7]) for c in CASES])
def test_forward_offsets_match_oracle(case):
    B, H, Sq, Sk, D, dtype, masked, p, offsets = case
    q, k, v, _ = inputs(B, H, Sq, Sk, D, dtype, seed=5000 + Sq + Sk + D)
    mask, ms = shared_mask(Sq, Sk, 5050 + Sq) if masked else (None, None)
    for c in offsets:
        say("case causal offset fwd", case[:8], "offset", c)
        o, lse = _fwd(q, k, v, c, mask, ms, p, 77)
        o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=True,
                                                dtype=dtype, mask=mask, mask_strides=ms, dropout_p=p, seed=77,
                                                offset=3, causal_offset=c)
        say("  ", parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, "offset %d %s" % (c, case[:8])))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_bottom_right_offset_is_the_causal_call(D):
    """causal_offset = Sk - Sq is the causal rule of fa_fwd_strided: the
    outputs are equal bit for bit (Sq < Sk and Sq > Sk)."""
    for Sq, Sk in ((300, 520), (520, 300)):
        q, k, v, _ = inputs(1, 4, Sq, Sk, D, "bf16", seed=5100 + D + Sq)
        qd, kd, vd = (t.to(DEV) for t in (q, k, v))
        o1, l1 = fa.forward_ext(qd, kd, vd, causal=True, causal_offset=Sk - Sq)
        o2, l2 = fa.forward(qd, kd, vd, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), (D, Sq, Sk)


def test_split_sequence_blocks_merge_to_the_causal_forward():
    """A causal sequence of 1000 tokens (4 heads, D = 128, bf16) cut into
    chunks [0, 300), [300, 640), [640, 1000): every (query chunk, key chunk)
    block computed with causal_offset = qs - ks, the blocks of a query chunk
    merged by log-sum-exp in fp64, against the oracle's one-shot causal
    forward (within the parity rule) and the GPU's (the merge only adds
    rounding)."""
    S, D, dtype = 1000, 128, "bf16"
    q, k, v, _ = inputs(1, 4, S, S, D, dtype, seed=5200)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o_full, l_full = fa.forward(qd, kd, vd, causal=True)
    o_ref, l_ref = oracle.attention_fwd(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=True, dtype=dtype)
    cuts = ((0, 300), (300, 640), (640, 1000))
    o_m = np.zeros((1, 4, S, D))
    l_m = np.zeros((1, 4, S))
    for qa, qb in cuts:
        parts = []
        for ka, kb in cuts:
            o_b, l_b = fa.forward_ext(qd[:, :, qa:qb], kd[:, :, ka:kb], vd[:, :, ka:kb], causal=True,
                                      causal_offset=qa - ka)
            torch.cuda.synchronize()
            o_b, l_b = to64(o_b), to64(l_b)
            if ka >= qb:
                assert np.all(o_b == 0.0) and np.all(np.isneginf(l_b)), (qa, ka)
            parts.append((o_b, l_b))
        lse = np.logaddexp.reduce(np.stack([p_[1] for p_ in parts]), axis=0)
        o_m[:, :, qa:qb] = sum(np.where(np.isneginf(p_[1]), 0.0, np.exp(p_[1] - lse))[..., None] * p_[0]
                               for p_ in parts)
        l_m[:, :, qa:qb] = lse
    say("  merged vs oracle", parity.assert_parity(o_m, l_m, o_ref, l_ref, dtype, "merged blocks"))
    assert np.max(np.abs(l_m - to64(l_full))) <= 1e-4
    assert np.max(np.abs(o_m - to64(o_full))) <= 2e-2


BWD_CASES = [
    (1, 2, 230, 150, 64, "f16", False, 0.0, (-100, 0, 40)),
    (1, 2, 190, 300, 128, "bf16", True, 0.2, (-200, 5, 310)),
    (1, 2, 130, 130, 256, "bf16", False, 0.1, (0, -20)),
    # plain D = 128: the 256-key dK/dV blocks, whose second half starts later
    (1, 2, 300, 420, 128, "bf16", False, 0.0, (-150, 0, 120, 400)),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=["%dx%dx%dx%dx%d%s%s_p%g" % (c[0], c[1], c[2], c[3], c[4], c[5],
                                                                            "_mask" if c[6] else "", c[7])
                                                 for c in BWD_CASES])
def test_backward_offsets_match_oracle(case):
    B, H, Sq, Sk, D, dtype, masked, p, offsets = case
    q, k, v, g = inputs(B, H, Sq, Sk, D, dtype, seed=5300 + Sq + Sk + D)
    mask, ms = shared_mask(Sq, Sk, 5350 + Sq) if masked else (None, None)
    md = None if mask is None else torch.from_numpy(mask[:, :Sk]).to(DEV)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    zs = parity.cancellation_tolerances(q, k, v, g, softmax_scale(D), dtype, dropout_p=p)
    for c in offsets:
        say("case causal offset bwd", case[:8], "offset", c)
        kw = dict(causal=True, mask=md, dropout_p=p, seed=21, offset=5, causal_offset=c)
        o, lse = fa.forward_ext(qd, kd, vd, **kw)
        grads = fa.backward_ext(qd, kd, vd, o, lse, gd, **kw)
        torch.cuda.synchronize()
        refs = oracle.attention_bwd_ext(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=True,
                                        dtype=dtype, mask=mask, mask_strides=ms, dropout_p=p, seed=21, offset=5,
                                        causal_offset=c)
        for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
            say("  ", name, parity.assert_grad_parity(to64(got), ref, dtype, "offset %d %s %s" % (c, name, case[:8]),
                                                      zero_tol=zs[name]))
