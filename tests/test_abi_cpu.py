"""C ABI checks that need no GPU: the library loads, exports every entry
point include/fa.h declares, and rejects bad arguments on the host before
anything is launched.  No call here reaches a kernel launch."""
import ctypes
import json
import math
import os
import re

import pytest

import tiled_attention_15_amd as fa
from tiled_attention_15_amd import build as fabuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fabuild.LIB):
        fabuild.build()
    return fa._load()


def declared_entry_points():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_entry_points()
    assert {"fa_fwd", "fa_status_string", "fa_version", "fa_fwd_plan"} <= set(names)
    raw = ctypes.CDLL(fabuild.LIB)
    for n in names:
        assert hasattr(raw, n), n


def test_version_and_status_strings(lib):
    assert fa.fa_version() >= 10000
    for code in range(10):
        s = fa.fa_status_string(code)
        assert s and s != "unknown status", code
    assert fa.fa_status_string(99) == "unknown status"


# fake, 16-byte aligned, non-overlapping "device" addresses: validation never dereferences them.
# Every call below must fail a host check; as a safety net the calls are not made at all where a
# GPU is visible, so a call that wrongly passed validation could never launch on fake addresses.
Q, K, V, O, L = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0      # counts devices without initialising them
    except Exception:
        return False


fake_addresses = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses are only passed "
                                    "where no GPU is visible")
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, S=256, D=64, scale=0.125, causal=0, dtype=0)


def call(**kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S"], a["D"],
                     a["scale"], a["causal"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(o=0), 1),
    (dict(B=0), 2), (dict(H=0), 2), (dict(S=0), 2), (dict(S=-5), 2), (dict(B=-1), 2),
    (dict(S=1 << 23, D=128), 2),
    (dict(D=96), 3), (dict(D=512), 3), (dict(D=0), 3), (dict(dtype=2), 3), (dict(dtype=-1), 3),
    (dict(q=Q + 8), 4), (dict(o=O + 2), 4), (dict(lse=L + 4), 4),
    (dict(scale=0.0), 5), (dict(scale=-1.0), 5), (dict(scale=float("nan")), 5),
    (dict(scale=float("inf")), 5),
    (dict(o=Q), 7), (dict(o=K + 64), 7), (dict(lse=V), 7), (dict(lse=O + 16), 7),
])
@fake_addresses
def test_rejects_bad_arguments(lib, kw, code):
    assert call(**kw) == code


def test_null_lse_is_not_an_error_in_validation(lib):
    # lse=NULL passes validation; check through the planner (no launch)
    br, _, grid, _ = fa.fa_fwd_plan(1, 2, 256, 64, False, 0)
    assert grid == 2 * -(-256 // br)


def _expected_tiles(B, H, S, br, bc, causal):
    nqb, nkv = -(-S // br), -(-S // bc)
    tot = 0
    for qb in range(nqb):
        tot += min(nkv, -(-min(S, (qb + 1) * br) // bc)) if causal else nkv
    return tot * B * H


@pytest.mark.parametrize("S", [1, 2, 17, 63, 64, 65, 255, 256, 257, 1000, 2048, 8192, 16384])
@pytest.mark.parametrize("causal", [False, True])
def test_plan_tile_counts(lib, S, causal):
    br, bc, grid, tiles = fa.fa_fwd_plan(2, 3, S, 128, causal, 1)
    assert br % 32 == 0 and bc == 64
    assert grid == 2 * 3 * -(-S // br)
    assert tiles == _expected_tiles(2, 3, S, br, bc, causal)


def test_plan_matches_pages_skip_table_reading(lib):
    """The pages' diagonal-skip table (128x128 tiles) prints total = T^2 and
    skipped = T^2/2.  The exact count visited is T(T+1)/2, so skipped is
    T(T-1)/2; with this library's tiles the skipped fraction likewise tends
    to one half as S grows."""
    facts = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_facts.json")))
    table = facts["causal_diagonal_skip_table"]
    tb = table["tile"][0]
    for S, total, skipped_printed in table["rows"]:
        T = S // tb
        assert T * T == total
        assert skipped_printed == total // 2
        visited = _expected_tiles(1, 1, S, tb, tb, True)
        assert visited == T * (T + 1) // 2
        assert total - visited == T * (T - 1) // 2
        br, bc, _, tiles = fa.fa_fwd_plan(1, 1, S, 128, True, 1)
        full = -(-S // br) * -(-S // bc)
        frac_skipped = 1 - tiles / full
        assert abs(frac_skipped - 0.5) <= bc / (2 * S) + br / (2 * S) + 1e-12


def test_python_forward_rejects_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


# fa_fwd_strided: a [B, H, S, D] layout given by element strides
def scall(B=2, H=3, Sq=100, Sk=150, D=64, qs=None, ks=None, vs=None, os_=None, **kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, scale=0.125, causal=1, dtype=0)
    a.update(kw)
    qs = qs or (H * Sq * D, Sq * D, D)
    ks = ks or (H * Sk * D, Sk * D, D)
    vs = vs or (H * Sk * D, Sk * D, D)
    os_ = os_ or (H * Sq * D, Sq * D, D)
    return fa.fa_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], B, H, Sq, Sk, D, qs, ks, vs,
                             os_, a["scale"], a["causal"], a["dtype"], None)


@fake_addresses
def test_strided_rejects_bad_arguments(lib):
    D = 64
    assert scall(Sk=0) == 2 and scall(Sq=0) == 2
    assert scall(qs=(3 * 100 * D, 100 * D, D + 4)) == 8            # row stride not a multiple of 8
    assert scall(ks=(3 * 150 * D, 150 * D, 56)) == 8               # row stride < D
    assert scall(vs=(-8, 150 * D, D)) == 8                         # negative stride
    assert scall(os_=(3 * 100 * D, 0, D)) == 8                     # heads of o share memory
    assert scall(os_=(3 * 100 * D, 64, D)) == 8                    # rows of one head overlap the next head's
    assert scall(B=1, os_=(0, 100 * D, D), o=K + 64) == 7          # batch stride 0 is fine at B=1; o overlaps k
    assert scall(o=K) == 7 and scall(lse=Q + 64) == 7              # aliasing
    assert scall(q=Q + 8) == 4
    assert scall(qs=(3 * 100 * D, 100 * D, 1 << 26)) == 2          # head span beyond 2^31 bytes
    assert scall(D=96, qs=(0, 0, 96), ks=(0, 0, 96), vs=(0, 0, 96), os_=(300 * 96, 100 * 96, 96)) == 3


@fake_addresses
def test_strided_accepts_layouts_up_to_the_launch(lib):
    """Valid layouts pass every host check; with null stream and fake
    addresses a launch would be made, so only the checks that come before it
    are exercised here, through layouts that must be rejected one step later
    (an unaligned lse)."""
    D = 128
    B, H, Sq, Sk = 2, 4, 100, 300
    bshd_q = (Sq * H * D, D, H * D)
    bshd_kv = (Sk * H * D, D, H * D)
    shared = (Sk * D, 0, D)
    for qs, ks, vs in ((bshd_q, bshd_kv, bshd_kv), (None, shared, shared)):
        assert scall(B=B, H=H, Sq=Sq, Sk=Sk, D=D, qs=qs, ks=ks, vs=vs, os_=bshd_q, lse=L + 4) == 4


@fake_addresses
def test_naive_rejects_bad_arguments(lib):
    W = 0x10000000
    B, H, S, D = 1, 2, 256, 64
    need = fa.fa_naive_workspace_bytes(B, H, S, D)
    Sp = 256
    assert need >= B * H * (S * Sp * 6 + D * Sp * 2)
    assert fa.fa_naive_workspace_bytes(1, 1, 16385, 64) == 0     # beyond the 16384-key limit
    assert fa.fa_naive_workspace_bytes(1, 1, 0, 64) == 0

    def ncall(**kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, B=B, H=H, S=S, D=D, scale=0.125, causal=1, dtype=0,
                 ws=W, wsb=need)
        a.update(kw)
        return fa.fa_naive_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S"],
                               a["D"], a["scale"], a["causal"], a["dtype"], a["ws"], a["wsb"], None)

    assert ncall(ws=0) == 1
    assert ncall(wsb=need - 1) == 2
    assert ncall(S=20000, wsb=1 << 40) == 2
    assert ncall(ws=W + 8) == 4
    assert ncall(ws=Q) == 7                  # workspace overlaps q
    assert ncall(o=K) == 7
    assert ncall(scale=0.0) == 5
    assert ncall(D=96) == 3
    assert ncall(D=256) == 3                 # the unfused path stops at D = 128
    assert fa.fa_naive_workspace_bytes(1, 1, 256, 256) == 0


@fake_addresses
def test_bwd_rejects_bad_arguments(lib):
    B, H, Sq, Sk, D = 1, 2, 300, 200, 64
    DO, DQ, DK, DV, W = 0x600000, 0x700000, 0x800000, 0x900000, 0x10000000
    for det in (0, 1):          # the flag is ignored: the workspace holds D_i only
        need = fa.fa_bwd_workspace_bytes(B, H, Sq, D, det)
        rows = B * H * Sq
        assert need == (rows * 4 + 255) // 256 * 256
    assert fa.fa_bwd_workspace_bytes(1, 1, 0, 64, 1) == 0
    assert fa.fa_bwd_workspace_bytes(1, 1, 16, 96, 1) == 0
    need = fa.fa_bwd_workspace_bytes(B, H, Sq, D, 0)

    def bcall(**kw):
        a = dict(q=Q, k=K, v=V, o=O, do=DO, lse=L, dq=DQ, dk=DK, dv=DV, B=B, H=H, Sq=Sq, Sk=Sk, D=D,
                 scale=0.125, causal=1, dtype=1, det=0, ws=W, wsb=need)
        a.update(kw)
        return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                         a["B"], a["H"], a["Sq"], a["Sk"], a["D"], a["scale"], a["causal"], a["dtype"],
                         a["det"], a["ws"], a["wsb"], None)

    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"):
        assert bcall(**{name: 0}) == 1, name
    assert bcall(Sq=0) == 2 and bcall(B=0) == 2
    assert bcall(wsb=need - 1) == 2
    assert bcall(D=96) == 3 and bcall(dtype=2) == 3
    assert bcall(D=512) == 3
    need256 = fa.fa_bwd_workspace_bytes(B, H, Sq, 256, 0)
    assert need256 == need                              # D_i only: independent of D
    assert bcall(D=256, wsb=need256, ws=W + 4) == 4      # D = 256 passes the shape checks
    assert bcall(Sk=1 << 24, wsb=1 << 40) == 2          # head span beyond 32-bit offsets
    assert bcall(dk=DK + 8) == 4 and bcall(ws=W + 4) == 4
    assert bcall(scale=float("nan")) == 5 and bcall(scale=-1.0) == 5
    assert bcall(dq=Q) == 7                  # output over an input
    assert bcall(dv=DK + 64) == 7            # two outputs overlap
    assert bcall(ws=DO) == 7                 # workspace over an input
    assert bcall(dk=W + 256) == 7            # output inside the workspace


@fake_addresses
def test_ext_rejects_bad_arguments(lib):
    B, H, Sq, Sk, D = 2, 2, 100, 120, 64
    M = 0x20000000

    def ecall(**kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, B=B, H=H, Sq=Sq, Sk=Sk, D=D, mask=M,
                 ms=(H * Sq * 128, Sq * 128, 128), p=0.1, seed=1, off=0, scale=0.125, causal=1,
                 dtype=0)
        a.update(kw)
        return fa.fa_fwd_ext(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Sq"],
                             a["Sk"], a["D"], a["mask"], a["ms"], a["p"], a["seed"], a["off"],
                             a["scale"], a["causal"], a["dtype"], None)

    assert ecall(q=0) == 1 and ecall(o=0) == 1
    assert ecall(Sq=0) == 2 and ecall(D=80) == 3 and ecall(dtype=3) == 3
    assert ecall(o=O + 8) == 4 and ecall(lse=L + 4) == 4
    assert ecall(scale=0.0) == 5
    for bad in (1.0, -0.01, float("nan"), 0.9999999):
        assert ecall(p=bad) == 9, bad
    assert ecall(mask=M + 2) == 9                       # mask not 4-byte aligned
    assert ecall(ms=None) == 9                          # strides missing
    assert ecall(ms=(0, 0, 118)) == 9                   # row stride < Sk
    assert ecall(ms=(0, 0, 130)) == 9                   # row stride not a multiple of 4
    assert ecall(ms=(-128, 0, 128)) == 9                # negative stride
    assert ecall(ms=(0, 0, 1 << 26)) == 9               # one head's rows beyond 2^31 bytes
    assert ecall(o=M + 64) == 7                         # output over the mask
    assert ecall(lse=K) == 7
    assert ecall(Sq=1 << 24, Sk=1 << 24, ms=(0, 0, 1 << 24)) == 2    # head span beyond 32-bit offsets


def test_plan_d256_uses_128_row_blocks(lib):
    """D = 256: 128-row blocks (the pair split) of 64-key tiles."""
    for causal in (0, 1):
        br, bc, grid, tiles = fa.fa_fwd_plan(2, 3, 1000, 256, causal, 1)
        assert (br, bc) == (128, 64)
        nqb = (1000 + 127) // 128
        assert grid == 2 * 3 * nqb
        nkv = (1000 + 63) // 64
        want = sum(min(nkv, (min(1000, (qb + 1) * 128) + 63) // 64) if causal else nkv for qb in range(nqb))
        assert tiles == want * 6


@fake_addresses
def test_bwd_ext_rejects_bad_arguments(lib):
    B, H, Sq, Sk, D = 1, 2, 100, 120, 64
    DO, DQ, DK, DV, W, M = 0x600000, 0x700000, 0x800000, 0x900000, 0x10000000, 0x20000000
    need = fa.fa_bwd_workspace_bytes(B, H, Sq, D, 1)

    def call(**kw):
        a = dict(q=Q, k=K, v=V, o=O, do=DO, lse=L, dq=DQ, dk=DK, dv=DV, Sq=Sq, Sk=Sk, D=D, mask=M,
                 ms=(0, 0, 128), p=0.1, ws=W, wsb=need)
        a.update(kw)
        return fa.fa_bwd_ext(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                             B, H, a["Sq"], a["Sk"], a["D"], a["mask"], a["ms"], a["p"], 1, 0, 0.125, 1, 0,
                             a["ws"], a["wsb"], None)

    assert call(ws=0) == 1 and call(dq=0) == 1
    assert call(D=512) == 3
    assert call(p=1.0) == 9 and call(p=-0.5) == 9
    assert call(mask=M + 1) == 9 and call(ms=(0, 0, 100)) == 9 and call(ms=(0, 0, 126)) == 9
    assert call(ms=(0, 0, 1 << 25)) == 9                 # mask rows beyond 2^31 bytes
    assert call(dk=M) == 7                                # an output over the mask
    assert call(wsb=need - 1) == 2


@fake_addresses
def test_bwd_strided_validation(lib):
    """fa_bwd_strided: layout rules per tensor (q, k, v, o, dout inputs; dq, dk,
    dv outputs), the aliasing rule on byte spans, and valid [B, S, H, D]
    layouts passing every check before the launch (shown by an unaligned
    workspace being the first thing rejected)."""
    B, H, Sq, Sk, D = 2, 4, 100, 300, 64
    sz_q, sz_k = B * H * Sq * D * 2, B * H * Sk * D * 2
    base = 0x40000000
    addr = {}
    for i, name in enumerate(("q", "k", "v", "o", "do", "dq", "dk", "dv")):
        addr[name] = base + i * 0x1000000
    W, M = base + 9 * 0x1000000, base + 10 * 0x1000000
    assert sz_k < 0x1000000
    bhsd_q, bhsd_k = (H * Sq * D, Sq * D, D), (H * Sk * D, Sk * D, D)
    bshd_q, bshd_k = (Sq * H * D, D, H * D), (Sk * H * D, D, H * D)
    need = fa.fa_bwd_workspace_bytes(B, H, Sq, D, 0)

    def call(strides=None, det=0, mask=None, ms=None, p=0.0, **kw):
        a = dict(addr, ws=W, wsb=need, D=D)
        a.update(kw)
        if strides is None:
            strides = [s for t in (bhsd_q, bhsd_k, bhsd_k, bhsd_q, bhsd_q, bhsd_q, bhsd_k, bhsd_k) for s in t]
        return fa.fa_bwd_strided(a["q"], a["k"], a["v"], a["o"], a["do"], L, a["dq"], a["dk"], a["dv"], B, H,
                                 Sq, Sk, a["D"], strides, mask, ms, p, 1, 0, 0.125, 1, 1, det, a["ws"], a["wsb"],
                                 None)

    def with_tensor(t, st):
        s = [x for u in (bhsd_q, bhsd_k, bhsd_k, bhsd_q, bhsd_q, bhsd_q, bhsd_k, bhsd_k) for x in u]
        s[3 * t:3 * t + 3] = st
        return s

    assert call(ws=W + 4) == 4                                   # contiguous: every layout check passes
    bshd = [x for t in (bshd_q, bshd_k, bshd_k, bshd_q, bshd_q, bshd_q, bshd_k, bshd_k) for x in t]
    assert call(bshd, ws=W + 4) == 4                             # [B, S, H, D] views of every tensor
    shared_kv = with_tensor(1, (Sk * D, 0, D))
    assert call(shared_kv, ws=W + 4) == 4                        # one K shared by the heads of a batch
    assert call(with_tensor(6, (Sk * D, 0, D))) == 8             # dk heads sharing memory
    assert call(with_tensor(5, (H * Sq * D, Sq * D, D + 4))) == 8    # row stride not a multiple of 8
    assert call(with_tensor(2, (H * Sk * D, Sk * D, 56))) == 8       # row stride < D
    assert call(with_tensor(4, (-8, Sq * D, D))) == 8                # negative stride
    assert call(with_tensor(7, (H * Sk * D, 64, D))) == 8            # dv rows run into the next head
    assert call(with_tensor(0, (0, 0, 1 << 22))) == 2                # a head beyond 32-bit offsets
    with pytest.raises(ValueError):
        call(strides=[D] * 23)
    # aliasing on the spans of strided tensors
    wide = with_tensor(5, (H * Sq * D * 4, Sq * D * 4, D * 4))       # dq spread over 4x its size
    assert call(wide, dk=addr["dq"] + sz_q + 64) == 7                 # dk inside dq's span
    assert call(dq=addr["o"] + 128) == 7 and call(ws=addr["dv"]) == 7
    assert call(mask=M, ms=(0, 0, 300), dq=M + 64) == 7               # output over the mask
    # one workspace size whatever the flag: there is no atomic dq accumulator
    assert fa.fa_bwd_workspace_bytes(B, H, Sq, D, 1) == need == (B * H * Sq * 4 + 255) // 256 * 256
    assert call(mask=M, ms=(0, 0, 300), ws=W + 4) == 4
    assert call(p=0.2, ws=W + 4) == 4 and call(det=1, ws=W + 4) == 4
    assert call(wsb=need - 1) == 2
    assert call(p=1.0) == 9 and call(mask=M + 1, ms=(0, 0, 300)) == 9


@fake_addresses
def test_fwd_ext_strided_validation(lib):
    """fa_fwd_ext_strided: per-tensor layout rules, span aliasing, and valid
    [B, S, H, D] / head-shared layouts passing every check (an unaligned lse
    is then the first thing rejected)."""
    B, H, Sq, Sk, D = 2, 4, 100, 300, 128
    base = 0x40000000
    Qa, Ka, Va, Oa, La, M = (base + i * 0x1000000 for i in range(6))
    bhsd_q, bhsd_k = (H * Sq * D, Sq * D, D), (H * Sk * D, Sk * D, D)
    bshd_q, bshd_k = (Sq * H * D, D, H * D), (Sk * H * D, D, H * D)

    def call(st=(bhsd_q, bhsd_k, bhsd_k, bhsd_q), **kw):
        a = dict(q=Qa, k=Ka, v=Va, o=Oa, lse=La, mask=None, ms=None, p=0.0, D=D)
        a.update(kw)
        flat = [x for t in st for x in t]
        return fa.fa_fwd_ext_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], B, H, Sq, Sk, a["D"], flat,
                                     a["mask"], a["ms"], a["p"], 1, 0, 0.125, 1, 1, None)

    assert call(lse=La + 4) == 4
    assert call((bshd_q, bshd_k, bshd_k, bshd_q), lse=La + 4) == 4
    assert call((bhsd_q, (Sk * D, 0, D), (Sk * D, 0, D), bhsd_q), lse=La + 4) == 4   # shared K, V
    assert call((bhsd_q, bhsd_k, bhsd_k, (H * Sq * D, 0, D))) == 8                    # o heads collide
    assert call((bhsd_q, (H * Sk * D, Sk * D, D + 8 - 4), bhsd_k, bhsd_q)) == 8        # row stride % 8
    assert call((bhsd_q, bhsd_k, (0, 0, 120), bhsd_q)) == 8                           # row stride < D
    assert call(((0, 0, 1 << 22), bhsd_k, bhsd_k, bhsd_q)) == 2                       # head span > 2^31 B
    assert call(o=Qa + 256) == 7 and call(lse=Oa + 64) == 7
    assert call(mask=M, ms=(0, 0, 300), o=M + 64) == 7
    assert call(mask=M, ms=(0, 0, 298)) == 9 and call(p=1.0) == 9
    assert call(D=96) == 3 and call(q=0) == 1
    with pytest.raises(ValueError):
        fa.fa_fwd_ext_strided(Qa, Ka, Va, Oa, La, B, H, Sq, Sk, D, [D] * 11, None, None, 0.0, 0, 0, 0.1, 0, 0,
                              None)


def test_split_is_chosen_for_small_grids(lib):
    """The key-split instance (128-row blocks) is planned for D = 64 and 128
    when twice the 256-row block count fits the 256 compute units, or for a
    causal call with fewer blocks than compute units."""
    br, bc, grid, _ = fa.fa_fwd_plan(2, 12, 2048, 64, True, 0)     # the GPT-shaped workload: 192 blocks
    assert (br, bc, grid) == (128, 64, 2 * 12 * 16)
    br, _, grid, _ = fa.fa_fwd_plan(4, 64, 2048, 64, True, 0)      # 2048 blocks of 256 rows
    assert (br, grid) == (256, 4 * 64 * 8)
    assert fa.fa_fwd_plan(1, 32, 1024, 128, False, 1)[0] == 128    # 128 blocks: the doubled grid fits
    assert fa.fa_fwd_plan(1, 33, 1024, 128, False, 1)[0] == 256    # 132 blocks, non-causal: no split
    assert fa.fa_fwd_plan(1, 33, 1024, 128, True, 1)[0] == 128     # causal, fewer blocks than CUs
    assert fa.fa_fwd_plan(1, 64, 1024, 128, True, 1)[0] == 256     # 256 blocks
    assert fa.fa_fwd_plan(1, 2, 2048, 256, True, 1)[0] == 128      # D = 256: the pair split's blocks
