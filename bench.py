"""Benchmark of the fused attention forward on one MI355X.

One step is one fa_fwd call over the whole workload batch (every query row
of every head), inputs already resident in device memory.  The default
workload is the long-sequence causal case: B=1, H=32, S=8192, D=128, bf16
Q/K/V drawn i.i.d. N(0,1) (Q x4), scale 1/sqrt(128).

Prints ONE JSON line:
  value      algorithmic TFLOP/s (FlashAttention-2 convention 4*B*H*S^2*D,
             halved when causal) over the timed steps;
  roofline   the same figure against the dense bf16/fp16 matrix-core peak,
             from HIP events on the stream the kernel runs on, plus the HBM
             traffic per launch read from the committed rocprofv3 counter
             summary when it was taken on the current kernel source;
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of rows of
             the same workload on this host's cores (rank 0, one GPU only).

  naive_unfused  the same attention computed the unfused way (scores and
             probabilities written to device memory, four kernels of this
             library), timed the same way, with the fused kernel's speedup.
  backward   the gradients (fa_bwd, bitwise reproducible) on the same
             inputs, in TFLOP/s at 2.5x the forward's flops.
  mask_dropout  the forward with an explicit mask and/or dropout (fa_fwd_ext).
             The backward and mask_dropout objects carry their own
             cpu_baseline: the fp64 oracle on the first heads of the workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--cpu-seconds T] [--no-cpu-baseline] [--no-naive]
                       [--no-backward] [--no-ext] [--cold N]
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import HEADLINE, WORKLOADS, bits, workload_inputs  # noqa: E402

# MI355X published dense matrix-core peak for fp16/bf16 (2.4 GHz, 256 CUs).
MFMA_PEAK_TFLOPS = 2516.6
HBM_PEAK_GBS = 8000.0
# The fused kernel and its parameter block: the HBM counters in profiles/ stay
# valid while these are unchanged.
KERNEL_SOURCES = ["tiled_attention_15_amd/csrc/fa_fwd_kernel.h", "tiled_attention_15_amd/csrc/fa_fwd_kernel.hip",
                  "tiled_attention_15_amd/csrc/fa_launch.h", "tiled_attention_15_amd/csrc/fa_tile.h"]


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name):
    """HBM bytes per launch from profiles/traffic_<workload>.md, or None when
    the file is absent or was taken on another kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.md" % workload_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def warm_up(step, launches, seconds):
    """At least `launches` calls of step(), and more until `seconds` of wall
    time have passed with the GPU busy: the shader clock ramps up over the
    first tens of milliseconds of sustained work, so a fixed handful of
    launches can leave the timed region on a still-rising clock."""
    import torch
    for _ in range(launches):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            step()
        n += 4
        torch.cuda.synchronize()
    return launches + n


def timed_steps(step, steps, stream):
    """Mean milliseconds per call over `steps` back-to-back calls of step()
    (after its warm-up), timed with HIP events on `stream`.  One untimed call
    is queued first, so that the GPU is busy while the start event is
    recorded and the timed calls are enqueued: otherwise the host's time
    between the start event and the first launch lands in the timed region
    (about a millisecond after the warm-up's final synchronisation)."""
    import torch
    step()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def gpu_leg(w, steps, warmup, cold=0, warmup_s=1.0):
    """Times `steps` back-to-back launches (the headline figure) after a
    warm-up of at least `warmup` launches and `warmup_s` seconds, with the
    shader clock stamped on the same stream just before and after the timed
    launches; then 50 launches timed one by one (median and minimum); with
    cold > 0, that many launches each preceded by a 512 MiB device write that
    evicts the caches."""
    import statistics
    import torch
    import tiled_attention_15_amd as fa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = workload_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    code = fa.BF16 if w.dtype == "bf16" else fa.F16

    def step():
        st = fa.fa_fwd(qd, kd, vd, o, lse, w.B, w.H, w.S, w.D, w.scale, w.causal, code, stream)
        if st != 0:
            raise fa.FaError(st)

    warm_launches = warm_up(step, warmup, warmup_s)
    # events on the stream the kernel is enqueued on (torch's current stream)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ck0 = fa.clock_stamps(dev, stream)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    ck1 = fa.clock_stamps(dev, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    per_xcd = fa.clock_mhz(ck0, ck1)
    if not torch.isfinite(o).all().item():
        raise RuntimeError("non-finite output in the benchmark run")

    def one_by_one(n, before=None):
        times = []
        for _ in range(n):
            if before is not None:
                before()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        return {"median_ms": round(statistics.median(times), 6), "min_ms": round(min(times), 6), "launches": n}

    stats = {"warm": one_by_one(50)}
    if cold > 0:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        stats["cold"] = one_by_one(cold, lambda: scratch.fill_(1))
        stats["cold"]["between_launches"] = "512 MiB device write"
        del scratch
    clock = {"sclk_mhz_mean": round(sum(per_xcd.values()) / max(1, len(per_xcd)), 1),
             "sclk_mhz_per_xcd": {str(x): round(m, 1) for x, m in sorted(per_xcd.items())},
             "warmup_launches": warm_launches, "warmup_s_min": warmup_s,
             "method": "shader-clock and 100 MHz real-time counters read on every XCD by a stamp kernel "
                       "launched on the same stream just before and after the timed launches"}
    hashes = {"q": hashlib.sha256(bits(q).tobytes()).hexdigest(),
              "k": hashlib.sha256(bits(k).tobytes()).hexdigest(),
              "v": hashlib.sha256(bits(v).tobytes()).hexdigest()}
    return ev_ms / steps, wall / steps * 1e3, stats, clock, hashes


def naive_leg(w, steps, warmup):
    """The unfused comparison path (scores and probabilities materialised in
    device memory) on the same inputs, timed like the fused kernel."""
    import torch
    import tiled_attention_15_amd as fa

    dev = torch.device("cuda:0")
    need = fa.fa_naive_workspace_bytes(w.B, w.H, w.S, w.D)
    if need <= 0:
        return None
    q, k, v = workload_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    code = fa.BF16 if w.dtype == "bf16" else fa.F16

    def step():
        st = fa.fa_naive_fwd(qd, kd, vd, o, lse, w.B, w.H, w.S, w.D, w.scale, w.causal, code, ws,
                             need, stream)
        if st != 0:
            raise fa.FaError(st, "fa_naive_fwd")

    warm_up(step, warmup, 0.2)
    ms = timed_steps(step, steps, stream)
    del ws
    return {"ms_per_step": round(ms, 4), "value": round(w.flops() / (ms * 1e-3) / 1e12, 3),
            "unit": "TFLOP/s", "workspace_bytes": int(need), "steps": steps,
            "path": "scores (fp32) and probabilities materialised in device memory: four kernels "
                    "(Q K^T, row softmax, V transpose, P V)"}


def backward_leg(w, steps, warmup):
    """The backward (fa_bwd, bitwise reproducible) on the same inputs, then the
    backward of the masked / dropout forward, timed like the forward.
    Algorithmic flops: FlashAttention-2 convention, 2.5 x the forward's (five
    S x S x D products), whatever the kernels recompute."""
    import torch
    import tiled_attention_15_amd as fa
    from workloads import make_inputs

    dev = torch.device("cuda:0")
    q, k, v = workload_inputs(w)
    g, _, _ = make_inputs(w.B, w.H, w.S, w.D, w.dtype, seed=w.seed + 1000)
    qd, kd, vd, gd = q.to(dev), k.to(dev), v.to(dev), g.to(dev)
    o, lse = fa.forward(qd, kd, vd, causal=w.causal, scale=w.scale)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    stream = torch.cuda.current_stream(dev)
    code = fa.BF16 if w.dtype == "bf16" else fa.F16
    flops = 2.5 * w.flops()
    out = {"unit": "TFLOP/s", "flops_per_step": flops, "steps": steps}
    if fa.fa_bwd_workspace_bytes(w.B, w.H, w.S, w.D, True) <= 0:
        out["skipped"] = "the backward takes D in {64, 128, 256}"
        return out
    need = fa.fa_bwd_workspace_bytes(w.B, w.H, w.S, w.D, True)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step():
        st = fa.fa_bwd(qd, kd, vd, o, gd, lse, dq, dk, dv, w.B, w.H, w.S, w.S, w.D, w.scale,
                       w.causal, code, True, ws, need, stream)
        if st != 0:
            raise fa.FaError(st, "fa_bwd")

    warm_up(step, warmup, 0.2)
    ms = timed_steps(step, steps, stream)
    if not (torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()):
        raise RuntimeError("non-finite gradient in the benchmark run")
    tf = flops / (ms * 1e-3) / 1e12
    out["deterministic"] = {
        "ms_per_step": round(ms, 4), "value": round(tf, 3),
        "frac_of_mfma_peak": round(tf / MFMA_PEAK_TFLOPS, 4), "workspace_bytes": int(need)}
    del ws
    # the backward of the masked / dropout forward: one [S, S] mask shared by
    # all heads (90% kept) and dropout 0.1
    import numpy as np
    ld = (w.S + 3) // 4 * 4
    rng = np.random.default_rng(2400)
    mask = torch.zeros((w.S, ld), dtype=torch.uint8)
    mask[:, :w.S] = torch.from_numpy((rng.random((w.S, w.S)) < 0.9).astype(np.uint8))
    md = mask.to(dev)
    ms = (0, 0, ld)
    lse_x = torch.empty_like(lse)
    o_x = torch.empty_like(o)
    st = fa.fa_fwd_ext(qd, kd, vd, o_x, lse_x, w.B, w.H, w.S, w.S, w.D, md, ms, 0.1, 1234, 0, w.scale, w.causal,
                       code, stream)
    if st != 0:
        raise fa.FaError(st, "fa_fwd_ext")
    need = fa.fa_bwd_workspace_bytes(w.B, w.H, w.S, w.D, True)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step_x():
        st = fa.fa_bwd_ext(qd, kd, vd, o_x, gd, lse_x, dq, dk, dv, w.B, w.H, w.S, w.S, w.D, md, ms, 0.1, 1234, 0,
                           w.scale, w.causal, code, ws, need, stream)
        if st != 0:
            raise fa.FaError(st, "fa_bwd_ext")

    warm_up(step_x, warmup, 0.2)
    ms_x = timed_steps(step_x, steps, stream)
    tf = flops / (ms_x * 1e-3) / 1e12
    out["mask_dropout"] = {"ms_per_step": round(ms_x, 4), "value": round(tf, 3),
                           "frac_of_mfma_peak": round(tf / MFMA_PEAK_TFLOPS, 4),
                           "mask": "one [S, S] uint8 mask shared by all heads, 90% kept", "dropout_p": 0.1}
    return out


def ext_leg(w, steps, warmup):
    """The masked/dropout forward (fa_fwd_ext) on the same inputs: without
    mask or dropout, with a shared random boolean mask (90% of scores kept),
    with dropout 0.1, and with both.  TFLOP/s at the forward's algorithmic
    flops (a mask hides scores but the convention counts the full causal
    product)."""
    import numpy as np
    import torch
    import tiled_attention_15_amd as fa

    dev = torch.device("cuda:0")
    q, k, v = workload_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=dev)
    ld = (w.S + 3) // 4 * 4
    rng = np.random.default_rng(2400)
    mask = torch.zeros((w.S, ld), dtype=torch.uint8)
    mask[:, :w.S] = torch.from_numpy((rng.random((w.S, w.S)) < 0.9).astype(np.uint8))
    md = mask.to(dev)
    stream = torch.cuda.current_stream(dev)
    code = fa.BF16 if w.dtype == "bf16" else fa.F16
    out = {"unit": "TFLOP/s", "steps": steps, "mask_layout": "one [S, S] uint8 mask shared by all heads, 90% kept",
           "dropout_p": 0.1}
    for name, m, p in (("plain", None, 0.0), ("mask", md, 0.0), ("dropout", None, 0.1), ("mask_dropout", md, 0.1)):
        ms = None if m is None else (0, 0, ld)

        def step():
            st = fa.fa_fwd_ext(qd, kd, vd, o, lse, w.B, w.H, w.S, w.S, w.D, m, ms, p, 1234, 0,
                               w.scale, w.causal, code, stream)
            if st != 0:
                raise fa.FaError(st, "fa_fwd_ext")

        warm_up(step, warmup, 0.2)
        ms_step = timed_steps(step, steps, stream)
        tf = w.flops() / (ms_step * 1e-3) / 1e12
        out[name] = {"ms_per_step": round(ms_step, 4), "value": round(tf, 3),
                     "frac_of_mfma_peak": round(tf / MFMA_PEAK_TFLOPS, 4)}
    return out


def copy_leg(mib, steps, warmup):
    """A plain device copy of known size: its HBM byte counters per dispatch
    calibrate the counters read on the attention kernel."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    return {"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": ms,
            "gbs_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}


def cpu_leg(w, seconds):
    """The fp64 oracle on a bounded sample of the workload's query rows."""
    import numpy as np
    import oracle

    q, k, v = workload_inputs(w)
    qb, kb, vb = bits(q), bits(k), bits(v)
    rng = np.random.default_rng(12345)
    total = w.B * w.H * w.S

    def sample(n):
        rows = np.sort(rng.choice(total, size=min(n, total), replace=False)).astype(np.int64)
        pos = rows % w.S
        vis = (pos + 1) if w.causal else np.full(rows.shape, w.S)
        return rows, float(np.sum(4.0 * w.D * vis))

    def timed(rows):
        t0 = time.perf_counter()
        oracle.attention_rows(qb, kb, vb, rows, scale=w.scale, causal=w.causal, dtype=w.dtype)
        return time.perf_counter() - t0

    # grow the sample until it takes most of the budget (the per-row cost falls as
    # more rows share each head's decoded K/V, so one extrapolation is not enough)
    n = 64 * oracle.max_threads()
    while True:
        rows, flops = sample(n)
        t = timed(rows)
        if t >= 0.6 * seconds or n >= total:
            break
        n = int(min(total, n * max(2.0, 0.9 * seconds / max(t, 1e-3))))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.max_threads(),
        "cpu_model": cpu_model,
        "wall_s": round(t, 3),
        "kind": "oracle",
        "sample": "%d of %d query rows (random, seed 12345) of %s, fp64 oracle row by row; "
                  "%.1f s wall; flops counted per row as 4*D*visible_keys" % (
                      rows.size, total, w.name, t),
    }


def oracle_heads_leg(w, seconds, what):
    """The fp64 oracle on the first h heads of the workload (heads are
    independent, so these are exact gradients / outputs of those heads),
    h grown until the run takes most of `seconds`.  what: "backward" (the
    plain backward, flops 2.5x the forward's per head) or "mask_dropout"
    (the forward with the shared 90% mask and dropout 0.1)."""
    import numpy as np
    import oracle
    from workloads import make_inputs

    q, k, v = workload_inputs(w)
    g, _, _ = make_inputs(w.B, w.H, w.S, w.D, w.dtype, seed=w.seed + 1000)
    qb, kb, vb, gb = bits(q), bits(k), bits(v), bits(g)
    per_head = w.flops() / (w.B * w.H) * (2.5 if what == "backward" else 1.0)
    mask = None
    if what == "mask_dropout":
        ld = (w.S + 3) // 4 * 4
        rng = np.random.default_rng(2400)
        mask = np.zeros((w.S, ld), np.uint8)
        mask[:, :w.S] = (rng.random((w.S, w.S)) < 0.9).astype(np.uint8)

    def run(h):
        sl = (slice(0, 1), slice(0, h))
        qs, ks, vs, gs = (np.ascontiguousarray(x[sl]) for x in (qb, kb, vb, gb))
        t0 = time.perf_counter()
        if what == "backward":
            oracle.attention_bwd(qs, ks, vs, gs, scale=w.scale, causal=w.causal, dtype=w.dtype)
        else:
            oracle.attention_fwd_ext(qs, ks, vs, scale=w.scale, causal=w.causal, dtype=w.dtype, mask=mask,
                                     mask_strides=(0, 0, mask.shape[1]), dropout_p=0.1, seed=1234, offset=0)
        return time.perf_counter() - t0

    h = 1
    while True:
        t = run(h)
        if t >= 0.6 * seconds or h >= w.H:
            break
        h = int(min(w.H, max(h + 1, math.ceil(h * 0.9 * seconds / max(t, 1e-3)))))
    return {"value": per_head * h / t / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "wall_s": round(t, 3), "kind": "oracle",
            "sample": "heads 0..%d of batch 0 (of %d heads) of %s, the fp64 oracle's full %s of those "
                      "heads; %.1f s wall; flops counted as for the GPU figure" % (
                          h - 1, w.B * w.H, w.name,
                          "backward" if what == "backward" else "masked/dropout forward", t)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, choices=list(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="minimum wall time of warm-up launches before the timed region "
                         "(in addition to --warmup launches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-naive", action="store_true",
                    help="skip the unfused comparison path")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward (gradient) timing")
    ap.add_argument("--no-ext", action="store_true",
                    help="skip the masked / dropout forward timing")
    ap.add_argument("--cold", type=int, default=0,
                    help="also time this many launches one by one with a 512 MiB cache-evicting write "
                         "before each (cold caches)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of attention, time a plain device-to-device copy of this many "
                         "MiB (the reference kernel for scaling HBM byte counters)")
    a = ap.parse_args()
    if a.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(heads shard across GPUs with no exchange; see the design notes)" % a.gpus,
              file=sys.stderr)
        sys.exit(2)
    if a.copy_mib:
        print(json.dumps(copy_leg(a.copy_mib, a.steps, a.warmup)), flush=True)
        return
    w = WORKLOADS[a.workload]
    ms, wall_ms, launch_stats, clock, hashes = gpu_leg(w, a.steps, a.warmup, a.cold, a.warmup_seconds)
    tflops = w.flops() / (ms * 1e-3) / 1e12
    traffic = measured_traffic(w.name)
    out = {
        "metric": "attention fwd TFLOPS + % of MI355X MFMA peak, S=8192 D=128 causal",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded i.i.d. N(0,1) Q/K/V (Q x%g), resident in HBM" % w.q_mult,
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "D": w.D,
                   "causal": w.causal, "q_mult": w.q_mult, "seed": w.seed},
        "inputs_sha256": hashes,
        "tokens_per_s": round(w.B * w.S / (ms * 1e-3), 1),
        "pct_of_mfma_peak": round(100.0 * tflops / MFMA_PEAK_TFLOPS, 2),
        "hbm_gbs_algorithmic": round(w.bytes() / (ms * 1e-3) / 1e9, 2),
        "wall_ms_per_step": round(wall_ms, 6),
        "launch_stats": launch_stats,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic},
        # the peak is quoted at 2.4 GHz; the same fraction against the clock
        # the chip delivered over the timed region
        "clock": dict(clock, frac_at_delivered_clock=round(
            tflops / (MFMA_PEAK_TFLOPS * clock["sclk_mhz_mean"] / 2400.0), 4) if clock["sclk_mhz_mean"] else None),
        "cpu_baseline": None,
    }
    if not a.no_naive:
        nv = naive_leg(w, max(10, min(20, a.steps)), 2)
        if nv is not None:
            nv["fused_speedup"] = round(nv["ms_per_step"] / ms, 2)
        out["naive_unfused"] = nv
    if not a.no_backward:
        out["backward"] = backward_leg(w, max(10, min(20, a.steps)), 2)
    if not a.no_ext:
        out["mask_dropout"] = ext_leg(w, max(10, min(20, a.steps)), 2)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_leg(w, a.cpu_seconds)
        # the oracle timed beside the backward and the masked/dropout forward too
        if not a.no_backward and "skipped" not in out["backward"]:
            out["backward"]["cpu_baseline"] = oracle_heads_leg(w, a.cpu_seconds / 2, "backward")
        if not a.no_ext:
            out["mask_dropout"]["cpu_baseline"] = oracle_heads_leg(w, a.cpu_seconds / 2, "mask_dropout")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
