"""GPU parity of the forward with an explicit boolean mask and dropout
(fa_fwd_ext) against the fp64 oracle: full outputs on small and ragged
shapes, the exact keep pattern of the dropout, and sampled rows at the long
causal workload's size."""
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


def inputs(B, H, Sq, Sk, D, dtype, seed, q_mult=1.0):
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=seed, q_mult=q_mult, Sk=Sk)
    return q[:, :, :Sq].contiguous(), k, v


def make_mask(kind, B, H, Sq, Sk, seed):
    """(mask uint8 numpy array laid out as stored, strides in bytes) or (None, None)."""
    rng = np.random.default_rng(seed)
    if kind is None:
        return None, None
    if kind == "per_head":                      # [B, H, Sq, Sk_pad], rows padded to a multiple of 4
        ld = (Sk + 3) // 4 * 4
        m = np.zeros((B, H, Sq, ld), np.uint8)
        m[..., :Sk] = rng.random((B, H, Sq, Sk)) < 0.7
        m[0, 0, min(3, Sq - 1), :] = 0           # one row with no visible key
        return m, (H * Sq * ld, Sq * ld, ld)
    if kind == "shared":                        # one [Sq, Sk_pad + 8] mask for every head
        ld = (Sk + 3) // 4 * 4 + 8
        m = np.zeros((Sq, ld), np.uint8)
        m[:, :Sk] = rng.random((Sq, Sk)) < 0.85
        return m, (0, 0, ld)
    raise ValueError(kind)


def run_ext(q, k, v, causal, dtype, mask, ms, p, seed, offset):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    md = None if mask is None else torch.from_numpy(mask).to(DEV)
    o = torch.full_like(qd, float("nan"))          # unwritten elements stay NaN
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=DEV)
    st = fa.fa_fwd_ext(qd, kd, vd, o, lse, B, H, Sq, Sk, D, md, ms, p, seed, offset,
                       softmax_scale(D), causal, fa.BF16 if dtype == "bf16" else fa.F16, None)
    assert st == 0, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # (B, H, Sq, Sk, D, causal, dtype, mask kind, dropout p)
    (1, 2, 64, 64, 64, False, "f16", "per_head", 0.0),
    (1, 2, 128, 128, 128, True, "bf16", None, 0.1),
    (2, 1, 200, 200, 64, True, "f16", "shared", 0.25),
    (1, 2, 257, 257, 128, True, "bf16", "per_head", 0.5),
    (1, 1, 100, 300, 128, True, "f16", "shared", 0.0),
    (1, 1, 300, 100, 64, True, "bf16", "per_head", 0.1),
    (2, 2, 130, 67, 128, False, "f16", None, 0.3),
    (1, 3, 1, 1, 64, False, "bf16", "per_head", 0.0),
    (1, 2, 77, 45, 64, False, "f16", None, 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=["%dx%dx%dx%dx%d%s%s_%s_p%g" % (c[0], c[1], c[2], c[3], c[4],
                                                                          "c" if c[5] else "n", c[6], c[7], c[8])
                                             for c in CASES])
def test_ext_matches_oracle(case):
    B, H, Sq, Sk, D, causal, dtype, kind, p = case
    say("case ext", case)
    q, k, v = inputs(B, H, Sq, Sk, D, dtype, seed=2000 + Sq + 3 * Sk + D)
    mask, ms = make_mask(kind, B, H, Sq, Sk, seed=2100 + Sq)
    seed, offset = 0xC0FFEE_0000_1234 + Sq, 5
    o, lse = run_ext(q, k, v, causal, dtype, mask, ms, p, seed, offset)
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D),
                                            causal=causal, dtype=dtype, mask=mask, mask_strides=ms,
                                            dropout_p=p, seed=seed, offset=offset)
    st = parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, "ext %s" % (case,))
    say("  ", st)


@pytest.mark.parametrize("D,p,causal", [(64, 0.1, False), (128, 0.5, True), (64, 0.3, True)])
def test_ext_keep_pattern_is_exact(D, p, causal):
    """With V = the identity (Sk = D) the output row is the probability row
    times keep/(1-p): the GPU's zero pattern must equal the oracle's, element
    for element (the keep decisions are integer comparisons on both sides)."""
    Sq, Sk = 96, D
    q, k, _ = inputs(2, 2, Sq, Sk, D, "f16", seed=2200 + D, q_mult=0.25)
    v = torch.eye(Sk, dtype=torch.float16).expand(2, 2, Sk, D).contiguous()
    seed, offset = 123456789, 3
    o, _ = run_ext(q, k, v, causal, "f16", None, None, p, seed, offset)
    o_ref, _ = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=causal,
                                        dtype="f16", dropout_p=p, seed=seed, offset=offset)
    got = to64(o) != 0
    want = o_ref != 0
    assert np.array_equal(got, want), int((got != want).sum())
    kept = want.sum() / max(1, (o_ref != 0).size)
    say("   kept fraction", kept)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_ext_plain_is_the_plain_forward(D):
    """No mask and p = 0: fa_fwd_ext runs the plain forward on the kernel
    fa_fwd_strided uses for that head dimension, so the two calls agree bit
    for bit (contiguous tensors and a [B, S, H, D] view, Sq != Sk)."""
    q, k, v = inputs(1, 4, 700, 520, D, "bf16", seed=2300 + D)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    qs, ks, vs = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (qd, kd, vd))
    for causal in (False, True):
        for args in ((qd, kd, vd), (qs, ks, vs)):
            o1, l1 = fa.forward_ext(*args, causal=causal)
            o2, l2 = fa.forward(*args, causal=causal)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2)
            assert torch.equal(l1, l2)


def test_ext_workload_every_head():
    """The long causal workload (1x32x8192x128 bf16, Q x4) with a shared random
    mask (90% kept) and dropout 0.1: every output element written, rows of
    every head against the oracle."""
    w = WORKLOADS["long_causal_1x32x8192x128_bf16_q4"]
    q, k, v = workload_inputs(w)
    S = w.S
    rng = np.random.default_rng(2400)
    mask = (rng.random((S, S)) < 0.9).astype(np.uint8)
    ms = (0, 0, S)
    say("case ext workload", w.name)
    o, lse = run_ext(q, k, v, w.causal, w.dtype, mask, ms, 0.1, 77, 0)
    assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item(), "unwritten output"
    # 8 random rows of every head, and the first and last row of head 0
    rows = np.unique(np.concatenate([h * S + rng.choice(S, size=8, replace=False) for h in range(w.B * w.H)]
                                    + [np.array([0, S - 1])])).astype(np.int64)
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=w.scale, causal=w.causal,
                                            dtype=w.dtype, mask=mask, mask_strides=ms, dropout_p=0.1,
                                            seed=77, offset=0, rows=rows)
    st = parity.assert_parity(to64(o).reshape(-1, w.D)[rows], to64(lse).reshape(-1)[rows], o_ref, l_ref,
                              w.dtype, "ext workload rows")
    say("  ", st)


def test_forward_ext_pads_unaligned_mask_rows():
    """A bool mask with rows of Sk = 45 bytes (not 4-byte aligned) goes through
    the binding (which copies it to aligned rows) and matches the oracle."""
    B, H, Sq, Sk, D = 1, 2, 50, 45, 64
    q, k, v = inputs(B, H, Sq, Sk, D, "f16", seed=2500)
    m = torch.rand(Sq, Sk, generator=torch.Generator().manual_seed(2501)) < 0.7
    o, lse = fa.forward_ext(q.to(DEV), k.to(DEV), v.to(DEV), causal=False, mask=m.to(DEV), dropout_p=0.2,
                            seed=3, offset=1)
    torch.cuda.synchronize()
    mu = m.numpy().astype(np.uint8)
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=False,
                                            dtype="f16", mask=mu, mask_strides=(0, 0, Sk), dropout_p=0.2, seed=3,
                                            offset=1)
    parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, "f16", "unaligned mask rows")


@pytest.mark.parametrize("p", [0.0, 0.1])
def test_forward_ext_key_padding_mask(p):
    """A key-padding mask [B, 1, 1, Sk] (broadcast over heads and query rows,
    a row stride of 0 after expansion) goes through the binding, forward and
    backward, and matches the oracle with the mask written out in full."""
    B, H, Sq, Sk, D, dtype = 2, 3, 150, 200, 128, "bf16"
    q, k, v = inputs(B, H, Sq, Sk, D, dtype, seed=2550)
    g, _, _ = make_inputs(B, H, Sq, D, dtype, seed=2551)
    keep = torch.ones(B, 1, 1, Sk, dtype=torch.bool)
    keep[0, ..., 170:] = False
    keep[1, ..., 30:60] = False
    kw = dict(causal=False, mask=keep.to(DEV), dropout_p=p, seed=5, offset=2)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.forward_ext(qd, kd, vd, **kw)
    grads = fa.backward_ext(qd, kd, vd, o, lse, gd, **kw)
    torch.cuda.synchronize()
    full = np.ascontiguousarray(keep.expand(B, H, Sq, Sk).numpy().astype(np.uint8))
    ms = (H * Sq * Sk, Sq * Sk, Sk)
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=False,
                                            dtype=dtype, mask=full, mask_strides=ms, dropout_p=p, seed=5, offset=2)
    say("key padding p=%g" % p, parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, "key padding"))
    refs = oracle.attention_bwd_ext(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=False,
                                    dtype=dtype, mask=full, mask_strides=ms, dropout_p=p, seed=5, offset=2)
    zs = parity.cancellation_tolerances(q, k, v, g, softmax_scale(D), dtype, dropout_p=p)
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        say("  ", name, parity.assert_grad_parity(to64(got), ref, dtype, "key padding %s" % name,
                                                  zero_tol=zs[name]))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_forward_ext_strided_views(D):
    """[B, S, H, D] views of q, k, v and of the output, with a mask and
    dropout: bit for bit the contiguous call's result (same kernel, other
    addresses), and within the oracle's bound."""
    B, H, Sq, Sk, dtype = 2, 3, 140, 196, "bf16"
    say("case ext strided", B, H, Sq, Sk, D)
    q, k, v = inputs(B, H, Sq, Sk, D, dtype, seed=2600 + D)
    mask, ms = make_mask("per_head", B, H, Sq, Sk, seed=2650 + D)
    md = torch.from_numpy(mask).to(DEV)[..., :Sk]
    kw = dict(causal=True, mask=md, dropout_p=0.2, seed=11, offset=2)
    views = [t.to(DEV).transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v)]
    out = torch.empty((B, Sq, H, D), dtype=q.dtype, device=DEV).transpose(1, 2)
    o, lse = fa.forward_ext(*views, out=out, **kw)
    assert o.data_ptr() == out.data_ptr()
    o_c, lse_c = fa.forward_ext(*(t.to(DEV) for t in (q, k, v)), **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_c) and torch.equal(lse, lse_c)
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=True,
                                            dtype=dtype, mask=mask, mask_strides=ms, dropout_p=0.2, seed=11,
                                            offset=2)
    parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, "ext strided D=%d" % D)


def test_forward_ext_packed_qkv_shared_mask():
    """q, k, v slices of one packed [B, S, 3, H, D] buffer, one [S, S] mask for
    every batch and head, dropout: against the oracle."""
    B, H, S, D, dtype = 1, 4, 230, 128, "f16"
    say("case ext packed qkv", B, H, S, D)
    q, k, v = inputs(B, H, S, S, D, dtype, seed=2700)
    packed = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).to(DEV)
    qv, kv, vv = (packed[:, :, i].transpose(1, 2) for i in range(3))
    m = (torch.rand(S, S, generator=torch.Generator().manual_seed(2701)) < 0.75)
    o, lse = fa.forward_ext(qv, kv, vv, causal=False, mask=m.to(DEV), dropout_p=0.1, seed=5, offset=0)
    torch.cuda.synchronize()
    ld = (S + 3) // 4 * 4
    mu = np.zeros((S, ld), np.uint8)
    mu[:, :S] = m.numpy()
    o_ref, l_ref = oracle.attention_fwd_ext(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=False,
                                            dtype=dtype, mask=mu, mask_strides=(0, 0, ld), dropout_p=0.1, seed=5,
                                            offset=0)
    parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, "ext packed qkv")
