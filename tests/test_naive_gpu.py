"""GPU parity of the unfused comparison path (fa_naive_fwd) against the fp64
oracle, and its agreement with the fused kernel."""
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


@pytest.mark.parametrize("S", [1, 17, 64, 65, 255, 256, 257, 1000])
@pytest.mark.parametrize("D,dtype", [(64, "f16"), (128, "bf16")])
@pytest.mark.parametrize("causal", [False, True])
def test_naive_matches_oracle(S, D, dtype, causal):
    q, k, v = make_inputs(2, 2, S, D, dtype, seed=1200 + S)
    say("case naive", S, D, dtype, causal)
    o, lse = fa.naive_forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_fwd(bits(q), bits(k), bits(v), scale=softmax_scale(D),
                                        causal=causal, dtype=dtype)
    parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, "naive S%d D%d" % (S, D))


def test_naive_workload_rows_and_fused_agreement():
    """The 1x32x2048x128 fp16 workload: sampled rows against the oracle, and
    the whole output against the fused kernel (both within the parity bound
    of the oracle, so within twice of each other)."""
    w = WORKLOADS["llama_noncausal_1x32x2048x128_f16"]
    q, k, v = workload_inputs(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    say("case naive workload", w.name)
    o, lse = fa.naive_forward(qd, kd, vd, causal=w.causal)
    of, lf = fa.forward(qd, kd, vd, causal=w.causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(w.B * w.H * w.S, size=256, replace=False)).astype(np.int64)
    o_ref, l_ref = oracle.attention_rows(bits(q), bits(k), bits(v), rows, scale=w.scale,
                                         causal=w.causal, dtype=w.dtype)
    parity.assert_parity(to64(o).reshape(-1, w.D)[rows], to64(lse).reshape(-1)[rows], o_ref, l_ref,
                         w.dtype, "naive workload rows")
    assert (o.float() - of.float()).abs().max().item() <= 2 * parity.O_TOL[w.dtype] + 2e-3
    assert (lse - lf).abs().max().item() <= 2e-4 * max(1.0, lf.abs().max().item())


def test_naive_causal_row0_with_stale_workspace():
    """Row 0 of a causal call sees only key 0, so its output is exactly V[0];
    the workspace starts filled with large finite garbage, none of which may
    leak into the result."""
    q, k, v = make_inputs(1, 3, 300, 64, "f16", seed=1301)
    ws = torch.full((fa.fa_naive_workspace_bytes(1, 3, 600, 64),), 0x7f, dtype=torch.uint8, device=DEV)
    o, _ = fa.naive_forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])
