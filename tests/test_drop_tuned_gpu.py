"""GPU parity of the dropout instances of the tuned forward kernel
(fa_fwd_ext with dropout_p > 0): full outputs on grids large enough for the
unsplit 256-row instance (the small shapes of test_ext_gpu.py run the
key-split one), the exact keep pattern there, and the general kernel, which
serves row strides beyond the tuned kernel's 32-bit head offsets, drawing
the same keep pattern."""
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


def inputs(B, H, Sq, Sk, D, dtype, seed, q_mult=1.0):
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=seed, q_mult=q_mult, Sk=Sk)
    return q[:, :, :Sq].contiguous(), k, v


def code(dtype):
    return fa.BF16 if dtype == "bf16" else fa.F16


# (B, H, S, D, causal, dtype, mask, p): B*H*ceil(S/256) >= 256 query blocks,
# so neither the causal nor the non-causal grid takes the key split
UNSPLIT = [
    (1, 130, 300, 64, False, "f16", False, 0.1),
    (2, 65, 300, 128, True, "bf16", True, 0.2),
    (1, 256, 200, 128, False, "bf16", True, 0.5),
    (2, 128, 129, 64, True, "f16", False, 0.3),
]


@pytest.mark.parametrize("case", UNSPLIT, ids=["%dx%dx%dx%d%s%s%s_p%g" % (c[0], c[1], c[2], c[3], "c" if c[4] else "n",
                                                                         c[5], "_mask" if c[6] else "", c[7])
                                               for c in UNSPLIT])
def test_drop_unsplit_matches_oracle(case):
    B, H, S, D, causal, dtype, masked, p = case
    say("case drop unsplit", case)
    q, k, v = inputs(B, H, S, S, D, dtype, seed=4100 + S + D)
    mask, ms = None, None
    if masked:
        ld = (S + 3) // 4 * 4
        rng = np.random.default_rng(4150 + S)
        mask = np.zeros((S, ld), np.uint8)
        mask[:, :S] = rng.random((S, S)) < 0.8
        ms = (0, 0, ld)
    seed, offset = 0x1234_5678_9ABC + S, 7
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=DEV)
    md = None if mask is None else torch.from_numpy(mask).to(DEV)
    st = fa.fa_fwd_ext(qd, kd, vd, o, lse, B, H, S, S, D, md, ms, p, seed, offset, softmax_scale(D), causal,
                       code(dtype), None)
    assert st == 0, fa.fa_status_string(st)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=causal,
                                            dtype=dtype, mask=mask, mask_strides=ms, dropout_p=p, seed=seed,
                                            offset=offset)
    say("  ", parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, "drop unsplit %s" % (case,)))


@pytest.mark.parametrize("D,causal", [(64, False), (128, True)])
def test_drop_unsplit_keep_pattern_is_exact(D, causal):
    """V = the identity (Sk = D): the output row is the probability row times
    keep/(1-p), so the zero pattern is the keep pattern; on a grid of 256
    query blocks (the unsplit instance) it equals the oracle's element for
    element."""
    B, H, Sq, Sk, p = 2, 128, 96, D, 0.3
    q, k, _ = inputs(B, H, Sq, Sk, D, "f16", seed=4200 + D, q_mult=0.25)
    v = torch.eye(Sk, dtype=torch.float16).expand(B, H, Sk, D).contiguous()
    seed, offset = 987654321, 9
    o, _ = fa.forward_ext(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    o_ref, _ = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=causal,
                                        dtype="f16", dropout_p=p, seed=seed, offset=offset)
    got, want = to64(o) != 0, o_ref != 0
    assert np.array_equal(got, want), int((got != want).sum())
    say("   kept fraction", want.mean())


def test_general_kernel_beyond_tuned_reach_same_keep_pattern():
    """A row stride of 4,000,000 elements: a head padded to the tuned kernel's
    320 rows spans 2^31 bytes or more, so fa_fwd_ext_strided runs the general
    kernel (128-row blocks, 256 rows of reach).  With V = the identity its
    zero pattern equals the oracle's and the tuned kernel's on the same
    values in contiguous tensors, and both outputs match the oracle."""
    B, H, S, D, p, dtype = 1, 1, 100, 64, 0.25, "f16"
    r = 4_000_000
    q, k, _ = inputs(B, H, S, S, D, dtype, seed=4300, q_mult=0.25)
    v = torch.zeros(B, H, S, D, dtype=torch.float16)
    v[0, 0, :D, :] = torch.eye(D, dtype=torch.float16)
    n = (S - 1) * r + D
    say("case general kernel, row stride", r, "elements:", 4 * n * 2 / 2**30, "GiB")

    def strided(t):
        buf = torch.zeros(n, dtype=t.dtype, device=DEV)
        view = buf.as_strided((B, H, S, D), (S * r, S * r, r, 1))
        view.copy_(t.to(DEV))
        return buf, view

    bq, qs = strided(q)
    bk, ks = strided(k)
    bv, vs = strided(v)
    bo = torch.full((n,), float("nan"), dtype=torch.float16, device=DEV)
    os_ = bo.as_strided((B, H, S, D), (S * r, S * r, r, 1))
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    st = [S * r, S * r, r] * 4
    seed, offset = 55, 1
    assert fa.fa_fwd_ext_strided(qs, ks, vs, os_, lse, B, H, S, S, D, st, None, None, p, seed, offset,
                                 softmax_scale(D), False, fa.F16, None) == 0
    o_c, lse_c = fa.forward_ext(q.to(DEV), k.to(DEV), v.to(DEV), causal=False, dropout_p=p, seed=seed,
                                offset=offset)
    torch.cuda.synchronize()
    o_g = os_.to("cpu")
    del bq, bk, bv, bo
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=False,
                                            dtype=dtype, dropout_p=p, seed=seed, offset=offset)
    want = o_ref != 0
    assert np.array_equal(to64(o_g) != 0, want)
    assert np.array_equal(to64(o_c) != 0, want)
    parity.assert_parity(to64(o_g), to64(lse), o_ref, l_ref, dtype, "general kernel")
    parity.assert_parity(to64(o_c), to64(lse_c), o_ref, l_ref, dtype, "tuned kernel")
