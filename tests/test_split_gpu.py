"""GPU parity of the key-split instance of the tuned forward kernel.

At D = 64 and 128, for grids of 256-row blocks too small for the chip, the
forward runs 128-row blocks whose two wave groups share the rows and split
the K/V tiles (even / odd), merging their partial (O, m, l) through LDS at
the end.  Checked against the fp64 oracle on shapes with even
and odd tile counts (an odd count gives group 1 a fully masked padding tile),
unequal lengths, ragged rows and strided views.
"""
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
    return t.detach().float().cpu().numpy().astype(np.float64)


def inputs(B, H, Sq, Sk, D, dtype, seed):
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=seed, Sk=Sk)
    return q[:, :, :Sq].contiguous(), k, v


CASES = [
    # (B, H, Sq, Sk, causal, dtype, D)
    (1, 2, 256, 256, False, "f16", 64),      # the tiny workload's shape
    (1, 3, 192, 192, True, "bf16", 128),     # block 1: three tiles (odd)
    (2, 2, 129, 130, False, "f16", 128),     # three key tiles (odd), ragged rows
    (1, 1, 700, 190, True, "bf16", 128),
    (1, 2, 300, 777, True, "f16", 128),
    (1, 1, 1, 1, False, "bf16", 128),
    (1, 4, 1000, 1000, True, "bf16", 128),
    (1, 3, 192, 192, True, "bf16", 64),      # block 1: three tiles (odd)
    (2, 2, 129, 130, False, "f16", 64),      # three key tiles (odd), ragged rows
    (1, 1, 700, 190, True, "bf16", 64),      # Sq > Sk: leading rows see no key
    (1, 2, 300, 777, True, "f16", 64),       # Sq < Sk, bottom-right causal
    (1, 1, 1, 1, False, "f16", 64),
    (1, 4, 1000, 1000, True, "f16", 64),
]


@pytest.mark.parametrize("case", CASES, ids=["%dx%dx%dx%dx%d%s%s" % (c[0], c[1], c[2], c[3], c[6],
                                                                       "c" if c[4] else "n", c[5]) for c in CASES])
def test_split_matches_oracle(case):
    B, H, Sq, Sk, causal, dtype, D = case
    say("case split", case)
    assert fa.fa_fwd_plan(B, H, Sq, D, causal, fa.BF16 if dtype == "bf16" else fa.F16)[0] == 128
    q, k, v = inputs(B, H, Sq, Sk, D, dtype, seed=5000 + Sq + 3 * Sk)
    o, lse = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    o2, lse2 = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)            # fixed merge order: repeatable
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=causal,
                                            dtype=dtype)
    st = parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, "split %s" % (case,))
    say("  ", st)


@pytest.mark.parametrize("D", [64, 128])
def test_split_strided_views(D):
    """[B, S, H, D] views in and out: bit for bit the contiguous call."""
    B, H, Sq, Sk = 2, 3, 333, 400
    q, k, v = inputs(B, H, Sq, Sk, D, "bf16", seed=5100 + D)
    views = [t.to(DEV).transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v)]
    out = torch.empty((B, Sq, H, D), dtype=q.dtype, device=DEV).transpose(1, 2)
    o, lse = fa.forward(*views, causal=True, out=out)
    o_c, lse_c = fa.forward(*(t.to(DEV) for t in (q, k, v)), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_c) and torch.equal(lse, lse_c)
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=True,
                                            dtype="bf16")
    parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, "bf16", "split strided")


def test_split_gpt_workload_all_rows_of_two_heads():
    """The GPT-shaped workload (2x12x2048x64 f16 causal) runs split: every row
    of two heads (one per batch) against the oracle."""
    w = WORKLOADS["gpt_causal_2x12x2048x64_f16"]
    q, k, v = workload_inputs(w)
    o, lse = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    for b, h in ((0, 5), (1, 11)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref, l_ref = oracle.attention_fwd_ext(bits(q[sl].contiguous()), bits(k[sl].contiguous()),
                                                bits(v[sl].contiguous()), scale=w.scale, causal=True, dtype="f16")
        st = parity.assert_parity(to64(o[sl]), to64(lse[sl]), o_ref, l_ref, "f16", "gpt head %d,%d" % (b, h))
        say("  ", b, h, st)


def test_split_masked_gpt_workload_two_heads():
    """The GPT-shaped workload with one shared random mask (85% kept) runs the
    masked key-split instance: every row of two heads against the oracle."""
    w = WORKLOADS["gpt_causal_2x12x2048x64_f16"]
    q, k, v = workload_inputs(w)
    assert fa.fa_fwd_plan(w.B, w.H, w.S, w.D, True, fa.F16)[0] == 128
    rng = np.random.default_rng(5200)
    m = (rng.random((w.S, w.S)) < 0.85).astype(np.uint8)
    o, lse = fa.forward_ext(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, mask=torch.from_numpy(m).to(DEV))
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 7)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref, l_ref = oracle.attention_fwd_ext(bits(q[sl].contiguous()), bits(k[sl].contiguous()),
                                                bits(v[sl].contiguous()), scale=w.scale, causal=True, dtype="f16",
                                                mask=m, mask_strides=(0, 0, w.S))
        st = parity.assert_parity(to64(o[sl]), to64(lse[sl]), o_ref, l_ref, "f16", "masked gpt head %d,%d" % (b, h))
        say("  ", b, h, st)


def test_split_d128_two_full_heads():
    """1x16x2048x128 bf16 causal (128 blocks of 256 rows: the D = 128 key
    split): every row of heads 0 and 15 against the oracle."""
    B, H, S, D = 1, 16, 2048, 128
    assert fa.fa_fwd_plan(B, H, S, D, True, fa.BF16)[0] == 128
    q, k, v = inputs(B, H, S, S, D, "bf16", seed=5300)
    o, lse = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    for h in (0, 15):
        sl = (slice(0, 1), slice(h, h + 1))
        o_ref, l_ref = oracle.attention_fwd_ext(bits(q[sl].contiguous()), bits(k[sl].contiguous()),
                                                bits(v[sl].contiguous()), scale=softmax_scale(D), causal=True,
                                                dtype="bf16")
        st = parity.assert_parity(to64(o[sl]), to64(lse[sl]), o_ref, l_ref, "bf16", "d128 split head %d" % h)
        say("  ", h, st)
