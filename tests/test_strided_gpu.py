"""GPU parity of fa_fwd_strided: query and key sequences of different
lengths, strided layouts ([B, S, H, D] tensors, rows inside wider buffers,
K/V shared across heads) and strided outputs, against the fp64 oracle on
contiguous copies of the same inputs."""
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


def ref(q, k, v, causal, dtype):
    """Oracle on contiguous CPU copies."""
    D = q.shape[-1]
    return oracle.attention_fwd(bits(q.contiguous()), bits(k.contiguous()), bits(v.contiguous()),
                                scale=softmax_scale(D), causal=causal, dtype=dtype)


def check(o, lse, q, k, v, causal, dtype, what):
    o_ref, l_ref = ref(q, k, v, causal, dtype)
    return parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, what)


UNEQUAL = [(1, 300), (77, 1000), (256, 1000), (300, 129), (1000, 64), (65, 1), (513, 512)]


@pytest.mark.parametrize("Sq,Sk", UNEQUAL)
@pytest.mark.parametrize("D,dtype", [(64, "f16"), (128, "bf16")])
@pytest.mark.parametrize("causal", [False, True])
def test_unequal_lengths(Sq, Sk, D, dtype, causal):
    q, _, _ = make_inputs(1, 2, Sq, D, dtype, seed=500 + Sq)
    _, k, v = make_inputs(1, 2, Sk, D, dtype, seed=600 + Sk)
    say("case Sq", Sq, "Sk", Sk, "D", D, dtype, "causal" if causal else "full")
    o, lse = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    st = check(o, lse, q, k, v, causal, dtype, "Sq%d Sk%d D%d" % (Sq, Sk, D))
    if causal and Sq > Sk:
        # rows that see no key: exactly zero output, lse = -inf
        n = Sq - Sk
        assert torch.all(o[:, :, :n] == 0) and torch.all(torch.isneginf(lse[:, :, :n]))
    say("   max|dO| %.3g" % st["max_abs"])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D,dtype", [(64, "f16"), (128, "bf16")])
def test_bshd_layout(causal, D, dtype):
    """[B, S, H, D] storage viewed as [B, H, S, D] for inputs and output."""
    B, H, S = 2, 3, 333
    q, k, v = make_inputs(B, H, S, D, dtype, seed=700 + D)
    say("case bshd", B, H, S, D, dtype, causal)
    qs, ks, vs = (t.transpose(1, 2).contiguous().to(DEV) for t in (q, k, v))   # [B, S, H, D]
    ostore = torch.full((B, S, H, D), 7.0, dtype=q.dtype, device=DEV)
    o, lse = fa.forward(qs.transpose(1, 2), ks.transpose(1, 2), vs.transpose(1, 2), causal=causal,
                        out=ostore.transpose(1, 2))
    torch.cuda.synchronize()
    assert o.data_ptr() == ostore.data_ptr()
    check(ostore.transpose(1, 2), lse, q, k, v, causal, dtype, "bshd D%d" % D)


def test_rows_inside_wider_buffers():
    """Rows of q, k, v and o are slices of wider rows (row stride D + 64)."""
    B, H, Sq, Sk, D = 1, 4, 200, 450, 128
    q, _, _ = make_inputs(B, H, Sq, D, "f16", seed=801)
    _, k, v = make_inputs(B, H, Sk, D, "f16", seed=802)
    say("case wide rows")

    def widen(t):
        w = torch.full(t.shape[:-1] + (D + 64,), 3.0, dtype=t.dtype)
        w[..., :D] = t
        return w.to(DEV)

    qw, kw, vw = widen(q), widen(k), widen(v)
    ow = torch.full((B, H, Sq, D + 64), 5.0, dtype=q.dtype, device=DEV)
    o, lse = fa.forward(qw[..., :D], kw[..., :D], vw[..., :D], causal=True, out=ow[..., :D])
    torch.cuda.synchronize()
    assert torch.all(ow[..., D:] == 5.0), "padding columns of the output were written"
    check(ow[..., :D], lse, q, k, v, True, "f16", "wide rows")


@pytest.mark.parametrize("causal", [False, True])
def test_kv_shared_across_heads(causal):
    """K and V with head stride 0: every head attends to the same keys."""
    B, H, S, D = 2, 6, 300, 128
    q, _, _ = make_inputs(B, H, S, D, "bf16", seed=901)
    _, k1, v1 = make_inputs(B, 1, S, D, "bf16", seed=902)
    say("case shared kv", causal)
    kd, vd = k1.to(DEV).expand(B, H, S, D), v1.to(DEV).expand(B, H, S, D)
    assert kd.stride(1) == 0
    o, lse = fa.forward(q.to(DEV), kd, vd, causal=causal)
    torch.cuda.synchronize()
    check(o, lse, q, k1.expand(B, H, S, D), v1.expand(B, H, S, D), causal, "bf16", "shared kv")


def test_strided_matches_contiguous_bitwise():
    """The strided entry point on a [B, S, H, D] layout gives exactly the bits
    of fa_fwd on the same values stored contiguously."""
    B, H, S, D = 1, 8, 1024, 128
    q, k, v = make_inputs(B, H, S, D, "bf16", seed=1001, q_mult=4.0)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1 = torch.empty_like(qd)
    l1 = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    assert fa.fa_fwd(qd, kd, vd, o1, l1, B, H, S, D, softmax_scale(D), 1, fa.BF16, None) == 0
    qs, ks, vs = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (qd, kd, vd))
    o2, l2 = fa.forward(qs, ks, vs, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_rejected_layouts():
    B, H, S, D = 1, 2, 64, 64
    q, k, v = (t.to(DEV) for t in make_inputs(B, H, S, D, "f16", seed=1101))
    wide = torch.zeros((B, H, S, D + 4), dtype=q.dtype, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.forward(wide[..., :D], k, v)          # row stride D + 4: not a multiple of 8
    assert e.value.status == 8
    with pytest.raises(fa.FaError) as e:
        fa.forward(q, k, v, out=torch.empty((B, 1, S, D), dtype=q.dtype, device=DEV).expand(B, H, S, D))
    assert e.value.status == 8                   # output heads would share memory
    with pytest.raises(fa.FaError) as e:
        fa.forward(q, k, v, out=q)               # output aliases an input
    assert e.value.status == 7
