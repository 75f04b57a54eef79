"""GPU checks through the diagnostic launch of the tuned forward (fa_fwd_diag):

* the kernel's own error: O stored in fp32 before its rounding to 16 bits,
  held to the raw tolerance (max |dO| <= 2e-3 for fp16, 1e-2 for bf16, with
  no half-ulp allowance) against the fp64 oracle on every workload shape;
  the 16-bit O must be the round-to-nearest-even of that fp32 O, bit for bit;
* the diagnostic instance computes what the product instance computes (O and
  lse bitwise equal);
* blocks are independent of the order workgroups take them (reversed order:
  bitwise equal outputs), on the XCD-grouped and the plain schedule;
* the K/V tiles each wave actually runs its softmax on, counted in the
  kernel, equal the causal skip rule of "catlass FlashAttention tuning for a
  13B service" (gsyq.cn), "Causal Mask implementation" (mode 2): per query
  block min(ceil(Sk / 64), ceil(min(Sq, (qb+1) B_r) + Sk - Sq) / 64)), at
  least one, every wave of a 256-row block running all of them, the two wave
  groups of a key-split block sharing them (one padding tile when odd).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import parity
import tiled_attention_15_amd as fa
from workloads import WORKLOADS, bits, make_inputs, softmax_scale, workload_inputs
from workload_ref import workload_reference

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RAW_TOL = {"f16": 2e-3, "bf16": 1e-2}


def say(*a):
    print(*a, flush=True)


def to64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def code(dtype):
    return fa.BF16 if dtype == "bf16" else fa.F16


def run_diag(qd, kd, vd, causal, scale, dtype, flags=0, want_o32=True, want_tiles=True):
    B, H, Sq, D = qd.shape
    Sk = kd.shape[2]
    o = torch.full((B, H, Sq, D), float("nan"), dtype=qd.dtype, device=DEV)
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=DEV)
    o32 = torch.full((B, H, Sq, D), float("nan"), dtype=torch.float32, device=DEV) if want_o32 else None
    n = fa.fa_fwd_diag_tile_slots(B, H, Sq, D, causal)
    assert n > 0
    tiles = torch.full((n,), -1, dtype=torch.int32, device=DEV) if want_tiles else None
    st = fa.fa_fwd_diag(qd, kd, vd, o, lse, o32, tiles, B, H, Sq, Sk, D, scale, causal, code(dtype), flags,
                        torch.cuda.current_stream())
    assert st == 0, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return o, lse, o32, tiles


def expected_tiles(B, H, Sq, Sk, D, causal, dtype):
    """Per block (n = (b*H + h) * nqb + qb) and wave: the tiles the rule
    visits, from the rule itself (not from the library)."""
    br = fa.fa_fwd_plan(B, H, Sq, D, causal, code(dtype))[0]
    split = br == 128
    nkv = -(-Sk // 64)
    nqb = -(-Sq // br)
    per_block = []
    for qb in range(nqb):
        if causal:
            last = min(Sq, (qb + 1) * br) + (Sk - Sq)    # keys < last are visible to some row
            nt = max(1, min(nkv, -(-last // 64))) if last > 0 else 1
        else:
            nt = nkv
        per_block.append(nt)
    per_wave = np.array([[(nt + 1) // 2] * 8 if split else [nt] * 8 for nt in per_block], np.int64)
    return split, np.tile(per_wave, (B * H, 1)), np.array(per_block * (B * H), np.int64)


def check_tiles(tiles, B, H, Sq, Sk, D, causal, dtype, what):
    split, per_wave, per_block = expected_tiles(B, H, Sq, Sk, D, causal, dtype)
    got = (tiles.cpu().numpy().astype(np.int64) & 0xFFFFFFFF).reshape(-1, 8)
    assert got.shape == per_wave.shape, (got.shape, per_wave.shape)
    assert np.array_equal(got, per_wave), "%s: tile counts differ from the skip rule (first bad block %d)" % (
        what, int(np.argmax(np.any(got != per_wave, axis=1))))
    if Sq == Sk:
        # and they add up to the planner's count (plus one padding tile per
        # odd key-split block)
        plan_tiles = fa.fa_fwd_plan(B, H, Sq, D, causal, code(dtype))[3]
        total = int(got[:, 0].sum()) if not split else int(got[:, 0].sum() + got[:, 4].sum())
        pad = int((per_block % 2).sum()) if split else 0
        assert total == plan_tiles + pad, (what, total, plan_tiles, pad)


WL = [n for n in WORKLOADS if WORKLOADS[n].D <= 128]


@pytest.mark.parametrize("name", WL)
def test_kernel_own_error_and_counts_on_workloads(name):
    w = WORKLOADS[name]
    say("diag workload", name)
    q, k, v = workload_inputs(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse, o32, tiles = run_diag(qd, kd, vd, w.causal, w.scale, w.dtype)
    # the product launch computes the same bits
    op, lp = fa.forward(qd, kd, vd, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, op) and torch.equal(lse, lp), "diagnostic instance differs from the product instance"
    assert torch.isfinite(o32).all().item()
    # O (16-bit) is the round-to-nearest-even of the fp32 O
    o32c = o32.cpu()
    assert torch.equal(o32c.to(o.dtype), o.cpu()), "16-bit O is not RNE of the fp32 O"
    check_tiles(tiles, w.B, w.H, w.S, w.S, w.D, w.causal, w.dtype, name)
    rows, o_ref, l_ref = workload_reference(w, q, k, v)
    og = o32c.to(torch.float64).numpy().reshape(-1, w.D)[rows]
    raw = float(np.max(np.abs(og - o_ref)))
    st16 = parity.compare(to64(o).reshape(-1, w.D)[rows], to64(lse).reshape(-1)[rows], o_ref, l_ref, w.dtype)
    say(name, "rows", rows.size, "fp32-O max|dO| %.3e (tol %.0e)" % (raw, RAW_TOL[w.dtype]),
        "16-bit O max|dO| %.3e ulp-net %.3e lse %.2e" % (st16["max_abs"], st16["max_ulp_net"],
                                                         st16["lse_max_scaled"]))
    assert raw <= RAW_TOL[w.dtype], "kernel's own error %.3e above %.0e on %s" % (raw, RAW_TOL[w.dtype], name)


@pytest.mark.parametrize("name", ["long_causal_1x32x8192x128_bf16_q4", "gpt_causal_2x12x2048x64_f16",
                                  "llama_noncausal_1x32x2048x128_f16"])
def test_reverse_grid_order_is_bitwise_equal(name):
    """32 and 24 heads: the XCD-grouped schedule (B*H a multiple of 8) and
    the key-split route of the GPT shape."""
    w = WORKLOADS[name]
    q, k, v = workload_inputs(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a = run_diag(qd, kd, vd, w.causal, w.scale, w.dtype, flags=0)
    b = run_diag(qd, kd, vd, w.causal, w.scale, w.dtype, flags=fa.DIAG_REVERSE_ORDER)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


SHAPES = [
    # (B, H, Sq, Sk, D, dtype, causal): unsplit and key-split routes, ragged,
    # unequal lengths, rows that see no key, B*H a multiple of 8 or not
    (1, 130, 333, 333, 128, "bf16", True),
    (1, 136, 1000, 1000, 64, "f16", True),
    (1, 130, 300, 700, 128, "bf16", True),
    (1, 86, 700, 300, 128, "f16", True),
    (2, 3, 777, 777, 128, "bf16", True),
    (1, 4, 1000, 1000, 64, "f16", True),
    (1, 2, 300, 900, 128, "f16", True),
    (1, 2, 900, 300, 64, "bf16", True),
    (1, 3, 1, 1, 128, "bf16", True),
    (2, 2, 513, 513, 128, "f16", False),
    (1, 130, 333, 500, 64, "bf16", False),
]


@pytest.mark.parametrize("case", SHAPES, ids=["%dx%dx%dx%dx%d%s%s" % (c[0], c[1], c[2], c[3], c[4], c[5],
                                                                     "c" if c[6] else "n") for c in SHAPES])
def test_counts_order_and_own_error(case):
    B, H, Sq, Sk, D, dtype, causal = case
    say("case diag", case)
    q, k, v = make_inputs(B, H, max(Sq, Sk), D, dtype, seed=4100 + Sq + Sk + D, q_mult=4.0, Sk=Sk)
    q = q[:, :, :Sq].contiguous()
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sc = softmax_scale(D)
    o, lse, o32, tiles = run_diag(qd, kd, vd, causal, sc, dtype)
    check_tiles(tiles, B, H, Sq, Sk, D, causal, dtype, str(case))
    r = run_diag(qd, kd, vd, causal, sc, dtype, flags=fa.DIAG_REVERSE_ORDER)
    assert torch.equal(o, r[0]) and torch.equal(lse, r[1]) and torch.equal(o32, r[2]) and torch.equal(tiles, r[3])
    o_ref, l_ref = oracle.attention_fwd(bits(q), bits(k), bits(v), scale=sc, causal=causal, dtype=dtype)
    assert torch.equal(o32.cpu().to(o.dtype), o.cpu())
    st = parity.assert_parity(to64(o), to64(lse), o_ref, l_ref, dtype, str(case))
    raw = float(np.max(np.abs(to64(o32) - o_ref)))
    say("   fp32-O max|dO| %.3e" % raw, st)
    assert raw <= RAW_TOL[dtype]


def test_diag_rejects():
    q = torch.zeros((1, 1, 64, 256), dtype=torch.float16, device=DEV)
    o = torch.empty_like(q)
    assert fa.fa_fwd_diag(q, q, q, o, None, None, None, 1, 1, 64, 64, 256, 0.1, 0, fa.F16, 0, None) == 3
    q = q[..., :128].contiguous()
    o = torch.empty_like(q)
    assert fa.fa_fwd_diag(q, q, q, o, None, None, None, 1, 1, 64, 64, 128, 0.1, 0, fa.F16, 2, None) == 3
    o32 = torch.empty((1, 1, 64, 128), dtype=torch.float32, device=DEV)
    # fp32 output overlapping the input
    assert fa.fa_fwd_diag(q, q, q, o, None, q, None, 1, 1, 64, 64, 128, 0.1, 0, fa.F16, 0, None) == 7
    assert fa.fa_fwd_diag(q, q, q, o, None, o32, None, 1, 1, 64, 64, 128, 0.1, 0, fa.F16, 0, None) == 0
    torch.cuda.synchronize()
