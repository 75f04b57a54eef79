"""Oracle references for the full-size workload checks (test helper).

workload_reference(w, q, k, v) evaluates the fp64 oracle on the rows the
GPU workload tests compare: every row of every head, except on the
16384-long workload, where every row of eight heads (one from each XCD's
share of the heads) and 512 random rows of each other head are compared.
"""
import numpy as np

import oracle
from workloads import bits


def xcd_heads(BH):
    """Eight heads, one from each XCD's share when the kernel groups heads by
    XCD (B*H a multiple of 8: head x*BH/8 + k runs on XCD x), at different
    offsets inside the shares; otherwise the first eight."""
    if BH % 8 == 0:
        hpx = BH // 8
        return [x * hpx + (x % hpx) for x in range(8)]
    return list(range(min(8, BH)))


# Heads of the workload compared in full (every row): all of them, except on
# the 16384-long workload, where eight full heads (one per XCD share) and
# FULL_OTHERS_ROWS random rows of every other head are compared.
FULL_OTHERS_ROWS = 512


def workload_reference(w, q, k, v):
    """The oracle on the rows the workload test compares: (rows, o_ref [n, D],
    lse_ref [n]) with rows flat ids (b*H + h)*S + i, every row for all heads
    except on the longest workload (see above)."""
    BH = w.B * w.H
    qb, kb, vb = bits(q), bits(k), bits(v)
    if w.S <= 8192:
        full = list(range(BH))
        extra = np.zeros(0, np.int64)
    else:
        full = xcd_heads(BH)
        rng = np.random.default_rng(w.seed)
        others = [h for h in range(BH) if h not in full]
        extra = np.sort(np.concatenate([h * w.S + rng.choice(w.S, FULL_OTHERS_ROWS, replace=False)
                                        for h in others])).astype(np.int64)
    rows, os_, ls_ = [], [], []
    for h in full:
        b, hh = divmod(h, w.H)
        sl = (slice(b, b + 1), slice(hh, hh + 1))
        o_ref, l_ref = oracle.attention_fwd(np.ascontiguousarray(qb[sl]), np.ascontiguousarray(kb[sl]),
                                            np.ascontiguousarray(vb[sl]), scale=w.scale, causal=w.causal,
                                            dtype=w.dtype)
        rows.append(h * w.S + np.arange(w.S, dtype=np.int64))
        os_.append(o_ref.reshape(-1, w.D))
        ls_.append(l_ref.reshape(-1))
    if extra.size:
        o_ref, l_ref = oracle.attention_rows(qb, kb, vb, extra, scale=w.scale, causal=w.causal, dtype=w.dtype)
        rows.append(extra)
        os_.append(o_ref)
        ls_.append(l_ref)
    return np.concatenate(rows), np.concatenate(os_), np.concatenate(ls_)
