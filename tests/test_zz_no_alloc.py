"""The allocation-free backward (fa_bwd_noalloc) through the C ABI against
fa_bwd with a caller-owned workspace: bitwise
equal gradients on two calls in a row, the second with a smaller input
(the shared scratch array keeps the first call's contents), and a call
beyond the array's size refused with FA_ERR_SCRATCH before anything is
enqueued."""
import pytest
import torch

import tiled_attention_15_amd as fa
from workloads import make_inputs, softmax_scale

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(B, H, Sq, Sk, D, dtype, causal, seed):
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=seed, Sk=Sk)
    q = q[:, :, :Sq].contiguous()
    g, _, _ = make_inputs(B, H, Sq, D, dtype, seed=seed + 1)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.forward(qd, kd, vd, causal=causal)
    code = fa.BF16 if dtype == "bf16" else fa.F16
    sc = softmax_scale(D)
    stream = torch.cuda.current_stream()
    # reference: fa_bwd with its own workspace
    need = fa.fa_bwd_workspace_bytes(B, H, Sq, D, True)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ref = [torch.empty_like(t) for t in (qd, kd, vd)]
    assert fa.fa_bwd(qd, kd, vd, o, gd, lse, ref[0], ref[1], ref[2], B, H, Sq, Sk, D, sc, causal, code, True,
                     ws, need, stream) == 0
    got = [torch.full_like(t, float("nan")) for t in (qd, kd, vd)]
    st = fa.fa_bwd_noalloc(qd, kd, vd, o, gd, lse, got[0], got[1], got[2], B, H, Sq, Sk, D, sc, causal, code,
                           stream)
    assert st == 0, fa.fa_status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name
    return got


def test_noalloc_matches_fa_bwd_twice_second_smaller():
    print("case noalloc 1x8x1000x128 bf16 causal", flush=True)
    _case(1, 8, 1000, 1000, 128, "bf16", True, seed=5100)
    print("case noalloc 1x2x300x400x64 f16 non-causal", flush=True)
    _case(1, 2, 300, 400, 64, "f16", False, seed=5200)


def test_noalloc_refuses_beyond_its_scratch():
    cap = fa.fa_bwd_noalloc_scratch_bytes()
    assert cap == 16 << 20
    rows = cap // 4 + 256          # one 256-byte-rounded row block too many
    B, H, D = 1, 1, 64
    Sq = Sk = rows
    t = torch.empty((1,), dtype=torch.float16, device=DEV)      # never read: refused on the host
    lse = torch.empty((1,), dtype=torch.float32, device=DEV)
    st = fa.fa_bwd_noalloc(t, t, t, t, t, lse, t, t, t, B, H, Sq, Sk, D, 0.125, True, fa.F16, None)
    assert st == 10, fa.fa_status_string(st)
