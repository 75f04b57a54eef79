"""GPU parity of the backward on strided tensors (fa_bwd_strided through
backward() / backward_ext()): [B, S, H, D] views of every input and
gradient, a packed [B, S, 3, H, D] q/k/v buffer, K and V shared by all heads
(head stride 0).  Each case is checked against the fp64 oracle on contiguous
copies; the [B, S, H, D] result must also equal the contiguous call's bit
for bit (same arithmetic, other addresses)."""
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


def grad_inputs(B, H, Sq, Sk, D, dtype, seed):
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=seed, Sk=Sk)
    q = q[:, :, :Sq].contiguous()
    g, _, _ = make_inputs(B, H, Sq, D, dtype, seed=seed + 1000)
    return q, k, v, g


def bshd(t):
    """A [B, H, S, D] view of a [B, S, H, D] device buffer holding t."""
    return t.to(DEV).transpose(1, 2).contiguous().transpose(1, 2)


def bshd_empty(like):
    B, H, S, D = like.shape
    return torch.empty((B, S, H, D), dtype=like.dtype, device=DEV).transpose(1, 2)


def zero_scales(q, k, v, g, D, dtype="bf16", p=0.0):
    return parity.cancellation_tolerances(q, k, v, g, softmax_scale(D), dtype, dropout_p=p)


def check_oracle(grads, refs, dtype, what, zs):
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        st = parity.assert_grad_parity(to64(got), ref, dtype, "%s %s" % (name, what), zero_tol=zs[name])
        say("  ", name, st)


CASES = [
    # (B, H, Sq, Sk, D, causal, dtype)
    (2, 3, 150, 230, 64, True, "f16"),
    (1, 4, 257, 129, 128, False, "bf16"),
    (1, 2, 300, 300, 128, True, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=["x".join(map(str, c[:5])) + ("c" if c[5] else "n") + c[6]
                                             for c in CASES])
def test_bwd_bshd_views_match_oracle(case):
    """Every tensor (q, k, v, o, dout and the three gradients) a [B, S, H, D]
    view; o written by the forward through `out`."""
    B, H, Sq, Sk, D, causal, dtype = case
    say("case bwd strided bshd", case)
    q, k, v, g = grad_inputs(B, H, Sq, Sk, D, dtype, seed=3100 + Sq + Sk + D)
    qv, kv, vv, gv = (bshd(t) for t in (q, k, v, g))
    o = bshd_empty(qv)
    _, lse = fa.forward(qv, kv, vv, causal=causal, out=o)
    grads = (bshd_empty(qv), bshd_empty(kv), bshd_empty(vv))
    fa.backward(qv, kv, vv, o, lse, gv, causal=causal, grads=grads)
    torch.cuda.synchronize()
    refs = oracle.attention_bwd(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=causal,
                                dtype=dtype)
    check_oracle(grads, refs, dtype, case, zero_scales(q, k, v, g, D, dtype))
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    oc, lc = fa.forward(qd, kd, vd, causal=causal)
    ref = fa.backward(qd, kd, vd, oc, lc, gd, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(oc, o) and torch.equal(lc, lse)
    for name, a, b in zip(("dq", "dk", "dv"), grads, ref):
        assert torch.equal(a, b), name


def test_bwd_packed_qkv_input():
    """q, k, v as slices of one packed [B, S, 3, H, D] buffer (inputs may
    overlap each other); gradients in fresh tensors laid out like the inputs."""
    B, H, S, D, dtype = 2, 4, 333, 128, "bf16"
    say("case bwd packed qkv", B, H, S, D, dtype)
    q, k, v, g = grad_inputs(B, H, S, S, D, dtype, seed=3200)
    packed = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).to(DEV)   # [B, S, 3, H, D]
    qv, kv, vv = (packed[:, :, i].transpose(1, 2) for i in range(3))
    assert qv.stride() == (S * 3 * H * D, D, 3 * H * D, 1)
    o, lse = fa.forward(qv, kv, vv, causal=True)
    grads = fa.backward(qv, kv, vv, o, lse, g.to(DEV), causal=True, deterministic=True)
    torch.cuda.synchronize()
    refs = oracle.attention_bwd(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=True,
                                dtype=dtype)
    check_oracle(grads, refs, dtype, "packed qkv", zero_scales(q, k, v, g, D))


def test_bwd_kv_shared_by_heads():
    """K and V with head stride 0 (one K, V per batch for all heads): the
    gradients are those of the per-head copies (the caller sums dk, dv over
    heads for the shared tensor)."""
    B, H, Sq, Sk, D, dtype = 2, 4, 190, 250, 64, "f16"
    say("case bwd shared kv", B, H, Sq, Sk, D, dtype)
    _, k1, v1, _ = grad_inputs(B, 1, Sq, Sk, D, dtype, seed=3300)
    q, _, _, g = grad_inputs(B, H, Sq, Sk, D, dtype, seed=3301)
    kd, vd = k1.to(DEV).expand(B, H, Sk, D), v1.to(DEV).expand(B, H, Sk, D)
    assert kd.stride(1) == 0
    qd, gd = q.to(DEV), g.to(DEV)
    o, lse = fa.forward(qd, kd, vd, causal=True)
    grads = fa.backward(qd, kd, vd, o, lse, gd, causal=True)
    torch.cuda.synchronize()
    k, v = k1.expand(B, H, Sk, D).contiguous(), v1.expand(B, H, Sk, D).contiguous()
    refs = oracle.attention_bwd(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=True,
                                dtype=dtype)
    check_oracle(grads, refs, dtype, "shared kv", zero_scales(q, k, v, g, D))


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_ext_bshd_views_equal_contiguous(D):
    """Masked and dropout backward on [B, S, H, D] views: bit for bit the
    contiguous call's gradients, and within the oracle's bound."""
    B, H, Sq, Sk, dtype = 1, 3, 170, 140, "bf16"
    say("case bwd_ext strided", B, H, Sq, Sk, D, dtype)
    q, k, v, g = grad_inputs(B, H, Sq, Sk, D, dtype, seed=3400 + D)
    rng = np.random.default_rng(3450 + D)
    mask = (rng.random((B, H, Sq, Sk)) < 0.8).astype(np.uint8)
    md = torch.from_numpy(mask).to(DEV)
    kw = dict(causal=True, mask=md, dropout_p=0.15, seed=99, offset=4)
    qv, kv, vv, gv = (bshd(t) for t in (q, k, v, g))
    o, lse = fa.forward_ext(*(t.to(DEV) for t in (q, k, v)), **kw)
    ov = bshd(o)
    grads = (bshd_empty(qv), bshd_empty(kv), bshd_empty(vv))
    fa.backward_ext(qv, kv, vv, ov, lse, gv, grads=grads, **kw)
    ref = fa.backward_ext(*(t.to(DEV) for t in (q, k, v)), o, lse, g.to(DEV), **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), grads, ref):
        assert torch.equal(a, b), name
    refs = oracle.attention_bwd_ext(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=True,
                                    dtype=dtype, mask=mask, mask_strides=(H * Sq * Sk, Sq * Sk, Sk),
                                    dropout_p=0.15, seed=99, offset=4)
    check_oracle(grads, refs, dtype, "bwd_ext strided", zero_scales(q, k, v, g, D, dtype, 0.15))


def test_bwd_packed_gradients_are_rejected():
    """dq, dk, dv as slices of one packed buffer span the same bytes: the
    conservative aliasing rule refuses them (FA_ERR_ALIAS) before any launch."""
    B, H, S, D = 1, 2, 64, 64
    q, k, v, g = grad_inputs(B, H, S, S, D, "f16", seed=3500)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.forward(qd, kd, vd)
    dpacked = torch.empty((B, S, 3, H, D), dtype=torch.float16, device=DEV)
    grads = tuple(dpacked[:, :, i].transpose(1, 2) for i in range(3))
    with pytest.raises(fa.FaError) as e:
        fa.backward(qd, kd, vd, o, lse, gd, grads=grads)
    assert e.value.status == 7


def test_offsets_at_the_edge_of_the_32_bit_reach():
    """Row stride 2,790,000 elements, S = 256, D = 128: a head's rows span
    1.42e9 bytes, and the rows its tiles address past the sequence end (read
    as zero, never stored) reach 2.14e9 bytes, just under the 2^31-byte limit
    of the buffer offsets in the forward and in the backward (which rounds a
    head up to whole 128-key blocks plus one).  The forward, the backward and
    the masked/dropout backward equal the contiguous calls bit for bit and
    match the oracle."""
    B, H, S, D, dtype = 1, 1, 256, 128, "bf16"
    r = 2_790_000
    # inside both reaches, within 8192 elements of stride of the backward's
    assert (320 * r + D) * 2 < 2 ** 31 and (384 * r + D) * 2 < 2 ** 31 <= (384 * (r + 8192) + D) * 2
    say("case 32-bit reach, row stride", r)
    q, k, v, g = grad_inputs(B, H, S, S, D, dtype, seed=3600)
    n = (S - 1) * r + D
    bufs = []

    def wide(t=None, like=q):
        buf = torch.zeros(n, dtype=like.dtype, device=DEV)
        bufs.append(buf)
        view = buf.as_strided((B, H, S, D), (S * r, S * r, r, 1))
        if t is not None:
            view.copy_(t.to(DEV))
        return view

    qv, kv, vv, gv = (wide(t) for t in (q, k, v, g))
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))

    # forward and plain backward (causal)
    ov = wide()
    _, lse = fa.forward(qv, kv, vv, causal=True, out=ov)
    grads = (wide(), wide(), wide())
    fa.backward(qv, kv, vv, ov, lse, gv, causal=True, grads=grads)
    oc, lc = fa.forward(qd, kd, vd, causal=True)
    ref = fa.backward(qd, kd, vd, oc, lc, gd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(ov, oc) and torch.equal(lse, lc)
    for name, a, b in zip(("dq", "dk", "dv"), grads, ref):
        assert torch.equal(a, b), name
    o_ref, l_ref = oracle.attention_fwd(bits(q), bits(k), bits(v), scale=softmax_scale(D), causal=True, dtype=dtype)
    parity.assert_parity(to64(ov), to64(lse), o_ref, l_ref, dtype, "forward at the edge of the reach")
    refs = oracle.attention_bwd(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=True,
                                dtype=dtype)
    check_oracle(grads, refs, dtype, "backward at the edge of the reach", zero_scales(q, k, v, g, D, dtype))

    # masked/dropout backward (the other dK/dV kernel), non-causal
    rng = np.random.default_rng(3650)
    mask = (rng.random((S, S)) < 0.8).astype(np.uint8)
    md = torch.from_numpy(mask).to(DEV)
    kw = dict(causal=False, mask=md, dropout_p=0.1, seed=7, offset=3)
    oe, le = fa.forward_ext(qd, kd, vd, **kw)
    ov.copy_(oe)
    grads = (wide(), wide(), wide())
    fa.backward_ext(qv, kv, vv, ov, le, gv, grads=grads, **kw)
    ref = fa.backward_ext(qd, kd, vd, oe, le, gd, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), grads, ref):
        assert torch.equal(a, b), name
    refs = oracle.attention_bwd_ext(bits(q), bits(k), bits(v), bits(g), scale=softmax_scale(D), causal=False,
                                    dtype=dtype, mask=mask, mask_strides=(0, 0, S), dropout_p=0.1, seed=7,
                                    offset=3)
    check_oracle(grads, refs, dtype, "masked/dropout backward at the edge of the reach",
                 zero_scales(q, k, v, g, D, dtype, 0.1))
    del bufs
