"""GPU parity of the masked forward on the tuned kernel.

fa_fwd_ext / fa_fwd_ext_strided with a boolean mask and no dropout run the
tuned kernel's masked instance at D = 64, 128 and 256 (the mask bytes of each
lane's query row read one step ahead, hidden scores set to -inf before the
online softmax).  Checked here against the fp64 oracle's masked forward,
and bit for bit against the unmasked kernel where a mask changes nothing
(all ones) or restates the causal rule.
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


def inputs(B, H, Sq, Sk, D, dtype, seed, q_mult=1.0):
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=seed, q_mult=q_mult, Sk=Sk)
    return q[:, :, :Sq].contiguous(), k, v


def per_head_mask(B, H, Sq, Sk, seed, keep=0.7, pad=0):
    """[B, H, Sq, ld] uint8 with ld = Sk rounded up to 4 (+ pad), random
    keep pattern, one query row with no visible key and one 64-key range
    hidden from every row (a whole tile masked)."""
    rng = np.random.default_rng(seed)
    ld = (Sk + 3) // 4 * 4 + pad
    m = np.zeros((B, H, Sq, ld), np.uint8)
    m[..., :Sk] = rng.random((B, H, Sq, Sk)) < keep
    m[..., Sk:] = rng.integers(0, 2, size=(B, H, Sq, ld - Sk))      # padding: never read as keys
    m[0, 0, min(5, Sq - 1), :Sk] = 0
    if Sk > 128:
        m[0, -1, :, 64:128] = 0
    return m, (H * Sq * ld, Sq * ld, ld)


def run(q, k, v, causal, dtype, mask, ms):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    md = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask)).to(DEV)
    o = torch.full_like(qd, float("nan"))          # unwritten elements stay NaN
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=DEV)
    st = fa.fa_fwd_ext(qd, kd, vd, o, lse, B, H, Sq, Sk, D, md, ms, 0.0, 0, 0, softmax_scale(D), causal,
                       fa.BF16 if dtype == "bf16" else fa.F16, None)
    assert st == 0, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # (B, H, Sq, Sk, D, causal, dtype, shared mask, row padding)
    (1, 2, 64, 64, 64, False, "f16", False, 0),
    (1, 2, 600, 600, 128, True, "bf16", False, 0),       # three query blocks, ragged tail
    (2, 1, 513, 513, 64, True, "f16", True, 8),
    (1, 2, 300, 777, 128, True, "f16", False, 4),       # Sq < Sk, bottom-right causal
    (1, 1, 700, 190, 64, True, "bf16", False, 0),       # Sq > Sk: leading rows see no key
    (2, 2, 257, 131, 128, False, "bf16", True, 0),
    (1, 3, 1, 1, 128, False, "f16", False, 0),
    (1, 1, 45, 1029, 64, False, "bf16", False, 12),
    (1, 2, 300, 400, 256, True, "bf16", False, 4),      # D = 256: the pair split
    (2, 1, 257, 257, 256, False, "f16", True, 0),
]


@pytest.mark.parametrize("case", CASES, ids=["%dx%dx%dx%dx%d%s%s%s_pad%d" % (
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "n", c[6], "_shared" if c[7] else "", c[8]) for c in CASES])
def test_masked_matches_oracle(case):
    B, H, Sq, Sk, D, causal, dtype, shared, pad = case
    say("case masked tuned", case)
    q, k, v = inputs(B, H, Sq, Sk, D, dtype, seed=4000 + Sq + 7 * Sk + D)
    m, ms = per_head_mask(1 if shared else B, 1 if shared else H, Sq, Sk, seed=4100 + Sq, pad=pad)
    if shared:
        ms = (0, 0, ms[2])
    o, lse = run(q, k, v, causal, dtype, m, ms)
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=causal,
                                            dtype=dtype, mask=m, mask_strides=ms)
    st = parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, "masked tuned %s" % (case,))
    say("  ", st)


@pytest.mark.parametrize("D,dtype,causal", [(64, "f16", True), (128, "bf16", False), (128, "f16", True)])
def test_all_ones_mask_is_the_plain_forward(D, dtype, causal):
    """A mask that hides nothing leaves the arithmetic of every score
    unchanged: bit for bit the unmasked kernel's output and lse.  (The grid
    has at least 256 blocks of 256 rows, so the unmasked D = 64 call runs the
    same, unsplit, block layout.)"""
    B, H, Sq, Sk = 2, 64, 530, 530
    q, k, v = inputs(B, H, Sq, Sk, D, dtype, seed=4200 + D)
    ld = (Sk + 3) // 4 * 4 + 4
    ones = np.ones((Sq, ld), np.uint8)
    o, lse = run(q, k, v, causal, dtype, ones, (0, 0, ld))
    o_p, lse_p = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o_p)
    assert torch.equal(lse, lse_p)


@pytest.mark.parametrize("Sq,Sk", [(600, 600), (300, 700), (700, 300)])
def test_causal_rule_as_a_mask(Sq, Sk):
    """The causal rule written out as a mask (key j visible to query i iff
    j <= i + Sk - Sq) on a non-causal call: the tiles the causal call skips
    contribute exact zeros, so the two agree bit for bit.  (130 heads: enough
    256-row blocks that the causal call runs the unsplit block layout too.)"""
    D, dtype = 128, "bf16"
    q, k, v = inputs(1, 130, Sq, Sk, D, dtype, seed=4300 + Sq)
    i = np.arange(Sq)[:, None]
    j = np.arange(Sk)[None, :]
    ld = (Sk + 3) // 4 * 4
    m = np.zeros((Sq, ld), np.uint8)
    m[:, :Sk] = j <= i + (Sk - Sq)
    o, lse = run(q, k, v, False, dtype, m, (0, 0, ld))
    o_c, lse_c = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_c)
    assert torch.equal(lse, lse_c)


def test_masked_strided_views():
    """[B, S, H, D] views of q, k, v and the output with a per-head mask: bit
    for bit the contiguous call, and within the oracle's bound."""
    B, H, Sq, Sk, D, dtype = 2, 3, 400, 333, 128, "f16"
    q, k, v = inputs(B, H, Sq, Sk, D, dtype, seed=4400)
    m, ms = per_head_mask(B, H, Sq, Sk, seed=4401)
    md = torch.from_numpy(m).to(DEV)[..., :Sk]
    views = [t.to(DEV).transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v)]
    out = torch.empty((B, Sq, H, D), dtype=q.dtype, device=DEV).transpose(1, 2)
    o, lse = fa.forward_ext(*views, out=out, causal=True, mask=md)
    o_c, lse_c = fa.forward_ext(*(t.to(DEV) for t in (q, k, v)), causal=True, mask=md)
    torch.cuda.synchronize()
    assert torch.equal(o, o_c) and torch.equal(lse, lse_c)
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=True,
                                            dtype=dtype, mask=m, mask_strides=ms)
    parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, "masked strided")


def test_masked_workload_every_head():
    """The long causal workload (1x32x8192x128 bf16, Q x4) with one shared
    random mask (90% kept), launched as the benchmark does: every output
    element written, rows of every head against the oracle."""
    w = WORKLOADS["long_causal_1x32x8192x128_bf16_q4"]
    q, k, v = workload_inputs(w)
    S = w.S
    rng = np.random.default_rng(4500)
    mask = (rng.random((S, S)) < 0.9).astype(np.uint8)
    ms = (0, 0, S)
    say("case masked tuned workload", w.name)
    o, lse = run(q, k, v, w.causal, w.dtype, mask, ms)
    assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item(), "unwritten output"
    # 8 random rows of every head, and the first and last row of head 0
    rows = np.unique(np.concatenate([h * S + rng.choice(S, size=8, replace=False) for h in range(w.B * w.H)]
                                    + [np.array([0, S - 1])])).astype(np.int64)
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=w.scale, causal=w.causal,
                                            dtype=w.dtype, mask=mask, mask_strides=ms, rows=rows)
    st = parity.assert_parity(to64(o).reshape(-1, w.D)[rows], to64(lse).reshape(-1)[rows], o_ref, l_ref,
                              w.dtype, "masked workload rows")
    say("  ", st)
