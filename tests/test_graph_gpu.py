"""The C ABI under HIP graph capture: the library allocates nothing, clears
nothing with memset and synchronises nothing, so its calls can be captured
into a graph (through torch.cuda.CUDAGraph, which captures the caller's
stream).  The captured forward, backward and masked/dropout forward are
replayed several times, with new inputs copied in eagerly between replays,
and every replay must equal the eager calls on the same inputs bit for
bit."""
import numpy as np
import pytest
import torch

import tiled_attention_15_amd as fa
from workloads import make_inputs, softmax_scale

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("D,dtype,causal", [(128, "bf16", True), (64, "f16", False)])
def test_graph_replays_equal_eager_calls(D, dtype, causal):
    B, H, S = 1, 8, 1024
    say("case graph capture", B, H, S, D, dtype, causal)
    code = fa.BF16 if dtype == "bf16" else fa.F16
    scale = softmax_scale(D)
    sets = []
    for r in range(4):
        q, k, v = make_inputs(B, H, S, D, dtype, seed=5700 + 10 * r)
        g, _, _ = make_inputs(B, H, S, D, dtype, seed=5701 + 10 * r)
        sets.append(tuple(t.to(DEV) for t in (q, k, v, g)))
    mask = torch.from_numpy((np.random.default_rng(5790).random((S, S)) < 0.9).astype(np.uint8)).to(DEV)
    ms = (0, 0, S)
    need = fa.fa_bwd_workspace_bytes(B, H, S, D, True)

    # static buffers the graph reads and writes
    q, k, v, g = (t.clone() for t in sets[0])
    o, o2 = torch.empty_like(q), torch.empty_like(q)
    lse, lse2 = (torch.empty((B, H, S), dtype=torch.float32, device=DEV) for _ in range(2))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)

    def calls(stream):
        assert fa.fa_fwd(q, k, v, o, lse, B, H, S, D, scale, int(causal), code, stream) == 0
        assert fa.fa_bwd(q, k, v, o, g, lse, dq, dk, dv, B, H, S, S, D, scale, int(causal), code, True, ws, need,
                         stream) == 0
        assert fa.fa_fwd_ext(q, k, v, o2, lse2, B, H, S, S, D, mask, ms, 0.1, 11, 2, scale, int(causal), code,
                             stream) == 0

    calls(torch.cuda.current_stream())       # eager first call (reads the device's properties once)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for r in range(1, 4):
        for dst, src in zip((q, k, v, g), sets[r]):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv, o2, lse2)]
        # the same calls eagerly on the same inputs, into the same buffers
        calls(torch.cuda.current_stream())
        torch.cuda.synchronize()
        want = (o, lse, dq, dk, dv, o2, lse2)
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv", "o_ext", "lse_ext"), got, want):
            assert torch.equal(a, b), (r, name)
        # and the eager result is the forward of these inputs, not of the captured ones
        oc, _ = fa.forward(*sets[r][:3], causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(oc, o), r
