"""GPU parity of head dimension 256 (the general kernel behind fa_fwd,
fa_fwd_strided and fa_fwd_ext at D = 256) against the fp64 oracle."""
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


def test_d256_backward_is_rejected():
    q = torch.zeros(1, 1, 16, D, dtype=torch.float16, device=DEV)
    lse = torch.zeros(1, 1, 16, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError):
        fa.backward(q, q.clone(), q.clone(), q.clone(), lse, q.clone())
