"""Benchmark: paged decode attention, batch 64 x 32 heads x 128, bf16, B=16.

One step is one decode-attention pass over the whole batch (the partition
kernel, then the log-sum-exp merge kernel) with the KV cache already resident
in HBM. Before every step a 2 GiB buffer is read so the step starts with
cold caches (MI355X has a 256 MB last-level cache); the step itself is timed
with HIP events on the stream the kernels run on. Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload 2] [--partition-tokens P]

Inputs are synthetic and seeded (see workloads/): context lengths uniform in
[1, 2048], frames drawn from a randomly permuted pool of 20,000, q/k/v
standard-normal values rounded to bf16.

With the default workload the run then times workloads 1 and 3-8 (below), each in
a child process with the same --steps/--warmup, and adds their figures to the
line under "other_workloads" (--no-others skips this).

Other workloads (--workload N): 1 the worked example, 3 eight 32k-token
sequences, 4 forks of shared prompts (through paged_attn_decode_grouped
unless --ungrouped), 5 batch 256 with the step's kv_append (--permuted-pool
for its pool-order variant); 6 and 7 paged prefill (a 512-token chunk after
a cached prefix, whole prompts); 8 prefix-cached prefill rounds, with and
without caching. Decode and prefill dispatch their longest work first unless
--decode-batch-order / --prefill-batch-order. --head-dim / --dtype /
--block-size / --seqs / --max-ctx run workload 2 at another head dim
(H = 4096 / d, so a token's row keeps its size), storage dtype, block size,
batch or context range. --gpus N > 1 exits: the
library runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak
METRIC = "paged decode attention: KV GB/s (% of HBM peak) + µs/step, bf16 batch 64"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SOURCES = {"paged_decode": ("paged_decode.h", "paged_decode.hip", "paged_decode_f32.hip",
                                  "paged_decode_f16.hip", "paged_decode_bf16.hip", "pa_device.h",
                                  "pa_launch.h"),
                  "paged_prefill": ("paged_prefill.hip", "pa_device.h", "pa_launch.h",
                                    "pa_prefill.h")}


def _code_only(text: str) -> str:
    """Source text without comments and blank lines: what the compiler sees
    (string literals in these files hold no comment markers)."""
    import re

    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_digest(kind: str = "paged_decode") -> str:
    """Digest of the code (comments excluded) a kernel is built from: hardware
    counters taken on one digest are reported only while it still holds."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "paged_kv_cache_126_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, digest: str, kind: str = "paged_decode"):
    """HBM bytes per kernel launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def _draw_rows(w, stream, ids, device):
    """Generator rows for identities ``ids`` on the host: numpy's evaluation,
    or (``device``) torch's on the GPU in chunks, spot-checked bit for bit
    against numpy's on each chunk's first and last identity."""
    from workloads import values as V

    if device is None:
        return V.draw_np(w.seed, stream, ids, w.H, w.D, w.dtype)
    import torch

    from oracle.oracle import STORAGE

    out = np.empty((len(ids), w.H, w.D), dtype=STORAGE[w.dtype])
    step = max(1, (1 << 28) // (w.H * w.D))
    for i in range(0, len(ids), step):
        part = ids[i:i + step]
        t = V.draw_torch(w.seed, stream, torch.from_numpy(part).to(device), w.H, w.D, w.dtype, device)
        host = t.cpu().numpy() if w.dtype == "f32" else t.view(torch.int16).cpu().numpy().view(np.uint16)
        ends = np.unique([0, len(part) - 1])
        want = V.draw_np(w.seed, stream, part[ends], w.H, w.D, w.dtype)
        if not np.array_equal(host[ends].view(np.uint8), want.view(np.uint8)):
            raise RuntimeError("device and host evaluations of the value generator differ")
        out[i:i + len(part)] = host
    return out


def _compact_caches(w, tables, ctx, slot_ident, device=None):
    """Host K/V caches holding only the frames ``tables`` use, renumbered
    compactly (a relabelling of frames leaves attention unchanged), filled by
    the oracle side's own replay (``slot_ident``). Returns (k, v, tables)."""
    from oracle.oracle import STORAGE
    from workloads import values as V

    used = np.unique(np.concatenate([tables[i, :-(-int(c) // w.B)] for i, c in enumerate(ctx)]))
    remap = np.zeros(max(int(tables.max()), int(used.max())) + 1, dtype=np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    tab = np.where(tables >= 0, remap[np.clip(tables, 0, None)], 0).astype(np.int32)
    nb = len(used)
    nan = V.nan_bits(w.dtype)
    k = np.full((nb, w.B, w.H, w.D), nan, dtype=STORAGE[w.dtype])
    v = k.copy()
    slots_all = (used[:, None] * w.B + np.arange(w.B)[None, :]).reshape(-1)
    ids = slot_ident[slots_all]
    keep = ids >= 0
    new_slots = np.arange(nb * w.B, dtype=np.int64)[keep]
    k.reshape(nb * w.B, w.H, w.D)[new_slots] = _draw_rows(w, V.STREAM_K, ids[keep], device)
    v.reshape(nb * w.B, w.H, w.D)[new_slots] = _draw_rows(w, V.STREAM_V, ids[keep], device)
    return k, v, tab


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_info() -> dict:
    """The host CPU as /proc/cpuinfo and the scheduler describe it."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if info:
                        break  # first processor's block only
                    continue
                key, val = (x.strip() for x in line.split(":", 1))
                if key in ("vendor_id", "cpu family", "model", "model name", "stepping",
                           "cpu MHz", "cache size", "cpu cores", "siblings"):
                    info[key] = val
    except OSError:
        pass
    info["logical_cpus"] = os.cpu_count()
    try:
        info["usable_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    return info


def _time_bounded(fn, budget_s: float, max_runs: int = 500):
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= max_runs:
            break
    return float(np.median(times)), len(times)


def cpu_baseline_prefill(w, budget_s: float = 12.0):
    """The fp64 oracle's paged prefill on a bounded sample of a prefill
    workload: the sequence with the fewest visible (query, key) pairs, all
    heads, through the oracle side's own replay."""
    from oracle import blockmgr as obm
    from oracle.oracle import default
    from workloads import values as V

    orc = default()
    snap = obm.replay(w)[0][-1]
    n = np.asarray(w.query_lens, dtype=np.int64)
    ctx = snap.context_lens.astype(np.int64)
    pairs = n * (ctx - n) + n * (n + 1) // 2
    sample = np.sort(np.argsort(pairs, kind="stable")[:1])
    k, v, tab = _compact_caches(w, snap.tables[sample], snap.context_lens[sample], snap.slot_ident)
    sub_n = n[sample]
    qs = np.concatenate([[0], np.cumsum(sub_n)]).astype(np.int32)
    ids = np.concatenate([w.idents(int(si), np.arange(int(ctx[si] - n[si]), int(ctx[si])))
                          for si in sample])
    q = V.draw_np(w.seed, V.STREAM_Q, ids, w.H, w.D, w.dtype)
    sub_ctx = snap.context_lens[sample]
    t, runs = _time_bounded(
        lambda: orc.paged_prefill(q, k, v, tab, sub_ctx, qs, w.B, w.scale, w.dtype), budget_s, 20)
    flops = 4 * w.D * w.H * int(pairs[sample].sum())
    return {
        "value": flops / t / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(), "kind": "oracle",
        "cpu_model": _cpu_model(),
        "sample": f"{len(sample)} of {w.num_seqs} sequences (all {w.H} heads, "
                  f"{int(sub_n.sum())} queries, {int(pairs[sample].sum())} visible pairs), "
                  f"fp64 C oracle, median of {runs} runs",
        "seconds_per_sample": t,
    }


def cpu_baseline_prefix(w, budget_s: float = 12.0):
    """The fp64 oracle on a bounded sample of the prefix-cached rounds: the
    oracle side's own replay of the rounds (its prefix cache), then its paged
    prefill over the positions one request of the last round must compute,
    the request with the fewest visible (query, key) pairs. The rate counts
    that request's prompt tokens (reused + computed), as the GPU figure does."""
    from oracle.oracle import default
    from oracle.prefixcache import replay_rounds
    from workloads import values as V

    orc = default()
    rounds, _ = replay_rounds(w)
    rd = rounds[-1]
    ctx = rd.context_lens.astype(np.int64)
    n = ctx - rd.reused.astype(np.int64)
    pairs = n * (ctx - n) + n * (n + 1) // 2
    cand = np.flatnonzero(n > 0)
    i = int(cand[np.argmin(pairs[cand])])
    k, v, tab = _compact_caches(w, rd.tables[[i]], rd.context_lens[[i]], rd.slot_ident)
    c = rd.seqs[i]
    ids = w.idents(c, np.arange(int(rd.reused[i]), int(ctx[i])))
    q = V.draw_np(w.seed, V.STREAM_Q, ids, w.H, w.D, w.dtype)
    qs = np.array([0, int(n[i])], dtype=np.int64)
    sub_ctx = rd.context_lens[[i]]
    t, runs = _time_bounded(
        lambda: orc.paged_prefill(q, k, v, tab, sub_ctx, qs, w.B, w.scale, w.dtype), budget_s, 50)
    return {
        "value": float(ctx[i]) / t, "unit": "tokens/s", "cores": orc.num_threads(), "kind": "oracle",
        "cpu_model": _cpu_model(),
        "sample": f"1 request of the last round ({int(ctx[i])} prompt tokens, {int(rd.reused[i])} "
                  f"reused, {int(n[i])} computed, all {w.H} heads), after the oracle's own replay of "
                  f"all {len(rounds)} rounds; fp64 C oracle, median of {runs} runs",
        "seconds_per_sample": t,
    }


def cpu_baseline(w, device=None):
    """The fp64 oracle on the whole decode step of workload ``w`` (every
    sequence and head of its last attention point, through the oracle side's
    own replay), on the host's cores: the median of 3 runs for the two
    smallest workloads, one run for the others; also one thread, once, on
    the two smallest. The oracle's host caches are filled from the value
    generator (on ``device`` when given, checked against the host draw)."""
    from oracle import blockmgr as obm
    from oracle.oracle import default
    from workloads import values as V

    orc = default()
    cores = orc.num_threads()
    snaps, _ = obm.replay(w)
    snap = snaps[-1]
    ctx = snap.context_lens
    t0 = time.perf_counter()
    k, v, tab = _compact_caches(w, snap.tables, ctx, snap.slot_ident, device)
    prep_s = time.perf_counter() - t0
    q = V.draw_np(w.seed, V.STREAM_Q, w.q_idents(len(snaps) - 1), w.H, w.D, w.dtype)
    small = int(ctx.sum()) * w.H <= 4_000_000  # the worked example and the batch-64 step

    def run():
        orc.paged_decode(q, k, v, tab, ctx, w.B, w.scale, w.dtype)

    def timed(n):
        ts = []
        for _ in range(n):
            t1 = time.perf_counter()
            run()
            ts.append(time.perf_counter() - t1)
        return float(np.median(ts))

    runs = 3 if small else 1
    t = timed(runs)
    kv_bytes = 2 * w.H * w.D * w.elem_bytes * int(ctx.sum())
    res = {
        "value": kv_bytes / t / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
        "cpu_model": _cpu_model(), "cpu": _cpu_info(),
        "sample": f"the whole step: all {w.num_seqs} sequences x {w.H} heads "
                  f"({int(ctx.sum())} tokens, {kv_bytes / 1e6:.1f} MB of KV), fp64 C oracle, "
                  f"{'median of 3 runs' if runs == 3 else 'one run'}",
        "seconds_per_step": t,
        "host_cache_fill_s": round(prep_s, 3),
    }
    if small:
        orc.set_num_threads(1)
        try:
            t1 = timed(1)
        finally:
            orc.set_num_threads(cores)
        res["one_thread"] = {"value": kv_bytes / t1 / 1e9, "unit": "GB/s", "seconds_per_step": t1,
                             "sample": "the same whole step, one run on one thread"}
    return res


MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix peak

def frame_patterns(w, buf, sink, part_tokens: int, flush, args, dev) -> dict:
    """Read bandwidth of three frame access patterns over ``buf`` (the step's
    K/V size, frames of the workload's geometry, a seeded random frame order;
    pa_frame_read, kernel-stamped, cold): one head's B rows of a token-major
    [.., B, H, D] frame (the decode kernel's pattern and the target's layout),
    one head's B rows of a head-major [.., H, B, D] frame (contiguous, as in
    page 1's per-head K and V caches), and whole frames. A workgroup reads
    one head of the frames one partition covers, or, for whole frames, the
    same bytes in 1/H as many frames."""
    import torch

    import paged_kv_cache_126_amd as pkv

    row = w.D * w.elem_bytes
    frame = w.B * w.H * row
    n = (buf.numel() * buf.element_size()) // frame
    fpu = max(1, -(-part_tokens // w.B))
    order = torch.from_numpy(np.random.default_rng(7).permutation(n).astype(np.int32)).to(dev)
    specs = {
        "token_major_one_head": (w.H, row, w.B, w.H * row, row, fpu),
        "head_major_one_head": (w.H, w.B * row, w.B, row, row, fpu),
        "whole_frames": (1, 0, w.B * w.H, row, row, max(1, fpu // w.H)),
    }
    out = {"what": ("pa_frame_read over the step's K/V bytes in a random frame order, "
                    f"{frame} B frames, one workgroup per (head, {fpu} frames)"), "GB/s": {}}
    for name, (g, gs, pc, ps, pb, f) in specs.items():
        f = max(f, -(-n // 65535))  # pa_frame_read launches at most 65,535 units
        for _ in range(3):
            pkv.lib.frame_read(buf, order, frame, g, gs, pc, ps, pb, f, sink)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(20)]
        for c0, c1 in evs:
            if not args.no_flush:
                flush()
            with pkv.kernel_timing(c0, c1):
                pkv.lib.frame_read(buf, order, frame, g, gs, pc, ps, pb, f, sink)
        torch.cuda.synchronize()
        us = float(np.mean([c0.elapsed_time(c1) for c0, c1 in evs])) * 1e3
        out["GB/s"][name] = round(n * frame / us / 1e3, 1)
    log(f"[bench] frame access patterns: " + ", ".join(f"{k} {v:.0f} GB/s" for k, v in out["GB/s"].items()))
    return out


def prefill_roofline(w, flops: int, compulsory: int, kernel_ms: float, traffic) -> dict:
    """Roofline of one prefill launch. The attainable rate is the lower of the
    matrix peak and the HBM peak times the launch's intensity (algorithmic
    flops over compulsory bytes); ``bound`` names that roof, and
    ``achieved``/``peak`` are in its unit (compulsory bytes per second for an
    HBM-bound launch). The matrix cores issue the algorithmic flops: the
    weighted sum takes each weight once, in fp16 (with split weights, a bf16
    high part and residual, they would issue 1.5x)."""
    sec = kernel_ms * 1e-3
    tflops = flops / sec / 1e12
    intensity = flops / compulsory
    hbm_roof_tflops = HBM_PEAK_GBS * 1e9 * intensity / 1e12
    issued = flops
    out = {"kernel": "prefill_kernel"}
    if hbm_roof_tflops < MFMA_PEAK_TFLOPS:
        gbs = compulsory / sec / 1e9
        out.update(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                   frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        out.update(bound="mfma", achieved=round(tflops, 2), peak=MFMA_PEAK_TFLOPS,
                   unit="TFLOP/s", frac=round(tflops / MFMA_PEAK_TFLOPS, 4))
    out.update(traffic=traffic, launch_us=round(kernel_ms * 1e3, 2),
               algorithmic_flops_per_launch=flops, compulsory_bytes_per_launch=compulsory,
               intensity_flop_per_byte=round(intensity, 1),
               achieved_tflops=round(tflops, 2),
               attainable_tflops=round(min(MFMA_PEAK_TFLOPS, hbm_roof_tflops), 1),
               frac_of_mfma_peak=round(tflops / MFMA_PEAK_TFLOPS, 4),
               mfma_issued_flops_per_launch=int(issued),
               mfma_issued_frac_of_mfma_peak=round(issued / sec / 1e12 / MFMA_PEAK_TFLOPS, 4))
    return out


OTHER_WORKLOADS = (1, 3, 4, 5, 6, 7, 8)


def other_workloads(args) -> dict:
    """Time the other workloads, each in a child process running this script
    (after the headline's timed region, one at a time), and keep the figures
    that summarise each: the rate, the step time and the dominant kernel's
    roofline."""
    out = {}
    for wl in OTHER_WORKLOADS:
        cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", str(wl),
               "--steps", str(args.steps), "--warmup", str(args.warmup), "--no-cpu-baseline",
               "--no-others"]
        if args.no_flush:
            cmd.append("--no-flush")
        log(f"[bench] other workload {wl}: {' '.join(cmd[2:])}")
        t0 = time.perf_counter()
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        lines = [x for x in r.stdout.splitlines() if x.startswith("{")]
        if r.returncode != 0 or not lines:
            out[str(wl)] = {"error": f"exit {r.returncode}: {r.stderr.strip()[-300:]}"}
            log(f"[bench] other workload {wl} failed (exit {r.returncode})")
            continue
        res = json.loads(lines[-1])
        roof = res.get("roofline") or {}
        keep = {
            "workload": res["config"].get("workload"), "metric": res["metric"],
            "value": res["value"], "unit": res["unit"], "ms_per_step": res["ms_per_step"],
            "dtype": res["dtype"],
            "roofline": {k: roof.get(k) for k in ("kernel", "bound", "achieved", "peak", "unit",
                                                   "frac", "launch_us") if k in roof},
        }
        for k in ("pct_hbm_peak", "speedup_vs_no_caching", "dispatch_order"):
            if k in res:
                keep[k] = res[k]
        if "access_patterns" in roof:
            keep["roofline"]["access_patterns_GB/s"] = roof["access_patterns"]["GB/s"]
        out[str(wl)] = keep
        log(f"[bench] other workload {wl} ({keep['workload']}): {keep['value']} {keep['unit']}, "
            f"{keep['ms_per_step'] * 1e3:.1f} us/step, {time.perf_counter() - t0:.1f} s")
    return out


def bench_prefill(args, w, pt, cache, dev):
    """Prefill workloads: time paged_attn_prefill (one launch per step)."""
    import torch

    import paged_kv_cache_126_amd as pkv
    from workloads import values as V

    qs, ids = w.prefill_queries(pt.context_lens)
    T = int(qs[-1])
    q = V.draw_torch(w.seed, V.STREAM_Q, ids, w.H, w.D, w.dtype, dev).contiguous()
    out = torch.empty((T, w.H, w.D), dtype=torch.float32, device=dev)
    bt = torch.from_numpy(pt.tables).to(dev)
    cl = torch.from_numpy(pt.context_lens).to(dev)
    qsd = torch.from_numpy(qs.astype(np.int32)).to(dev)
    max_ctx, max_q = int(pt.context_lens.max()), int(np.diff(qs).max())
    from paged_kv_cache_126_amd.driver import prefill_order

    order = None if args.prefill_batch_order else torch.from_numpy(
        prefill_order(pt.context_lens, qs, max_q)).to(dev)
    # algorithmic work: 4 D flops per (query, visible key) per head
    n = np.asarray(w.query_lens, dtype=np.int64)
    ctx = pt.context_lens.astype(np.int64)
    pairs = int(np.sum(n * (ctx - n) + n * (n + 1) // 2))
    flops = 4 * w.D * w.H * pairs
    # bytes a single pass must move: every visible K and V row once, q in, out (fp32) back
    compulsory = w.H * w.D * (2 * w.elem_bytes * int(ctx.sum()) + (w.elem_bytes + 4) * T)
    digest = kernel_source_digest("paged_prefill")
    flush_buf = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def step(work_order=order, split=False):
        pkv.paged_attn_prefill(q, cache.k, cache.v, bt, cl, qsd, w.B, w.scale, out, max_ctx, max_q,
                               work_order=work_order, split_weights=split)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Plain launches between stream events (the step time) alternate with
    # launches that stamp the kernel's own start and end (its duration) and,
    # for context, plain launches in the default order and (bf16) stamped
    # launches with split weights, so that all of them see the same clock and
    # cache conditions.
    split_too = w.dtype == "bf16"
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    for e0, e1, k0, k1, b0, b1, s0, s1 in evs:
        if not args.no_flush:
            torch.sum(flush_buf, dim=0, out=flush_sink)
        e0.record()
        step()
        e1.record()
        if not args.no_flush:
            torch.sum(flush_buf, dim=0, out=flush_sink)
        with pkv.kernel_timing(k0, k1):
            step()
        if order is not None:
            if not args.no_flush:
                torch.sum(flush_buf, dim=0, out=flush_sink)
            b0.record()
            step(None)
            b1.record()
        if split_too:
            if not args.no_flush:
                torch.sum(flush_buf, dim=0, out=flush_sink)
            with pkv.kernel_timing(s0, s1):
                step(split=True)
    torch.cuda.synchronize()
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("prefill produced non-finite outputs: unwritten cache rows were read")
    split_ms = float(np.mean([e[6].elapsed_time(e[7]) for e in evs])) if split_too else None
    batch_order_ms = None
    if order is not None:
        batch_order_ms = float(np.mean([e[4].elapsed_time(e[5]) for e in evs]))
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    kms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    tflops = flops / (kms * 1e-3) / 1e12          # the kernel alone (roofline)
    step_tflops = flops / (ms * 1e-3) / 1e12      # whole step between stream events (value)
    log(f"[bench] prefill {args.steps} steps: {ms * 1e3:.1f} us (kernel alone {kms * 1e3:.1f}), "
        f"{step_tflops:.1f} TFLOP/s per step, kernel alone {tflops:.1f} TFLOP/s"
        + ("" if split_ms is None else f"; split weights: kernel alone {split_ms * 1e3:.1f} us"))
    res = {
        "metric": "paged prefill attention: TFLOP/s (% of MFMA peak) + us/step",
        "value": round(step_tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "step": "prefill attention",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "queries": T,
                   "sum_ctx": int(ctx.sum()), "visible_pairs": pairs, "flops": flops,
                   "cache_flush_between_steps": not args.no_flush},
        "us_per_step": round(ms * 1e3, 2),
        "dispatch_order": ("default (sequence by sequence)" if order is None else
                           "costliest sequence first, its later query tiles first "
                           "(driver.prefill_order)"),
        "default_order_us_per_step": None if batch_order_ms is None else round(batch_order_ms * 1e3, 2),
        "weighted_sum": ("fp16 operands: each weight rounded once to fp16"
                         + (", bf16 V converted to fp16 on chip" if split_too else "")),
        "split_weights_kernel_us": None if split_ms is None else round(split_ms * 1e3, 2),
        "roofline": prefill_roofline(w, flops, compulsory, kms, measured_traffic(
            w.name, digest, "paged_prefill")),
        "kernel_source_digest": digest,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        res["cpu_baseline"] = cpu_baseline_prefill(w)
    print(json.dumps(res), flush=True)


def bench_prefix(args, w, dev):
    """Prefix-sharing rounds: one step replays every round (write the prompt
    rows the block manager asks for with kv_append, paged_attn_prefill over
    them, then write the rows of the tokens the round's decode steps
    generate, which later rounds' prompts reuse), once with prefix caching
    and once without."""
    import torch

    import paged_kv_cache_126_amd as pkv
    from paged_kv_cache_126_amd.driver import DeviceCache, plan_prefix_rounds, prefill_order
    from workloads import values as V

    def prepare(caching):
        pool = None if caching else w.frames_without_caching
        t0 = time.perf_counter()
        rounds, mgr = plan_prefix_rounds(w, caching, pool_frames=pool)
        host_s = time.perf_counter() - t0
        cache = DeviceCache(w.NB if caching else pool, w.B, w.H, w.D, V.torch_dtype(w.dtype), dev,
                            poison=True)
        launches = []
        for rd in rounds:
            wb = rd.writes
            ids = torch.from_numpy(w.idents_rows(wb.seqs, wb.positions)).to(dev)
            k_new = V.draw_torch(w.seed, V.STREAM_K, ids, w.H, w.D, w.dtype, dev).contiguous()
            v_new = V.draw_torch(w.seed, V.STREAM_V, ids, w.H, w.D, w.dtype, dev).contiguous()
            q = V.draw_torch(w.seed, V.STREAM_Q, ids, w.H, w.D, w.dtype, dev).contiguous()
            T = int(rd.query_start[-1])
            n = np.diff(rd.query_start).astype(np.int64)
            ctx = rd.context_lens.astype(np.int64)
            pairs = int(np.sum(n * (ctx - n) + n * (n + 1) // 2))
            # the K/V rows of the tokens the round's decode steps generate, in
            # one write after the round's prefill (the next round's prompts
            # reuse the blocks that hold them; decode attention is not timed)
            dec = [st.writes for st in (rd.decode or [])]
            dseqs = np.concatenate([d.seqs for d in dec]) if dec else np.zeros(0, np.int64)
            dpos = np.concatenate([d.positions for d in dec]) if dec else np.zeros(0, np.int64)
            dslots = np.concatenate([d.slots for d in dec]) if dec else np.zeros(0, np.int64)
            dk = dv = None
            if len(dslots):
                dids = torch.from_numpy(w.idents_rows(dseqs, dpos)).to(dev)
                dk = V.draw_torch(w.seed, V.STREAM_K, dids, w.H, w.D, w.dtype, dev).contiguous()
                dv = V.draw_torch(w.seed, V.STREAM_V, dids, w.H, w.D, w.dtype, dev).contiguous()
            launches.append(dict(
                dk=dk, dv=dv, dslots=torch.from_numpy(dslots).to(dev), drows=len(dslots),
                k_new=k_new, v_new=v_new, slots=torch.from_numpy(wb.slots).to(dev), q=q,
                out=torch.empty((T, w.H, w.D), dtype=torch.float32, device=dev),
                bt=torch.from_numpy(rd.tables).to(dev), cl=torch.from_numpy(rd.context_lens).to(dev),
                qs=torch.from_numpy(rd.query_start).to(dev), max_ctx=int(ctx.max()),
                max_q=int(n.max()), rows=len(wb.slots), flops=4 * w.D * w.H * pairs,
                order=None if args.prefill_batch_order else
                torch.from_numpy(prefill_order(rd.context_lens, rd.query_start, int(n.max()))).to(dev)))
        return rounds, mgr, cache, launches, host_s

    flush_buf = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def timed(cache, launches):
        def step(evs=None, stamp=False):
            for i, L in enumerate(launches):
                if evs:
                    evs[i][0].record()
                if L["rows"]:
                    pkv.kv_append(L["k_new"], L["v_new"], L["slots"], cache.k, cache.v)
                if evs:
                    evs[i][1].record()
                if stamp:
                    with pkv.kernel_timing(evs[i][3], evs[i][4]):  # the kernel's own start and end
                        pkv.paged_attn_prefill(L["q"], cache.k, cache.v, L["bt"], L["cl"], L["qs"],
                                               w.B, w.scale, L["out"], L["max_ctx"], L["max_q"],
                                               work_order=L["order"])
                else:
                    pkv.paged_attn_prefill(L["q"], cache.k, cache.v, L["bt"], L["cl"], L["qs"], w.B,
                                           w.scale, L["out"], L["max_ctx"], L["max_q"],
                                           work_order=L["order"])
                if evs:
                    evs[i][2].record()
                if L["drows"]:
                    pkv.kv_append(L["dk"], L["dv"], L["dslots"], cache.k, cache.v)
                if evs:
                    evs[i][5].record()

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        # pass 0: the step time, events around the whole step only (events
        # recorded between kernels cost stream time themselves)
        sevs = []
        for _ in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if not args.no_flush:
                torch.sum(flush_buf, dim=0, out=flush_sink)
            e0.record()
            step()
            e1.record()
            sevs.append((e0, e1))
        # pass 1: events between the phases (the breakdown); pass 2: the
        # prefill kernel stamping its own start and end (its duration)
        all_evs = []
        for stamp in (False, True):
            for _ in range(args.steps):
                evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in launches]
                if not args.no_flush:
                    torch.sum(flush_buf, dim=0, out=flush_sink)
                step(evs, stamp)
                all_evs.append((stamp, evs))
        torch.cuda.synchronize()
        kern_evs = [e for st, e in all_evs if st]
        all_evs = [e for st, e in all_evs if not st]
        step_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in sevs]))
        append_ms = float(np.mean([sum(r[0].elapsed_time(r[1]) + r[2].elapsed_time(r[5]) for r in e)
                                   for e in all_evs]))
        prefill_ms = float(np.mean([sum(r[1].elapsed_time(r[2]) for r in e) for e in all_evs]))
        kernel_ms = float(np.mean([sum(r[3].elapsed_time(r[4]) for r in e) for e in kern_evs]))
        return step_ms, append_ms, prefill_ms, kernel_ms

    res = {}
    for caching in (True, False):
        rounds, mgr, cache, launches, host_s = prepare(caching)
        step_ms, append_ms, prefill_ms, kernel_ms = timed(cache, launches)
        # every query's keys were written before its prefill: a non-finite
        # output means the step read unwritten (NaN-filled) cache rows
        if not all(bool(torch.isfinite(L["out"]).all()) for L in launches):
            raise RuntimeError("prefix rounds produced non-finite outputs: unwritten cache rows were read")
        tokens = int(sum(int(rd.context_lens.sum()) for rd in rounds))
        reused = int(sum(int(rd.reused.sum()) for rd in rounds))
        res[caching] = dict(step_ms=step_ms, append_ms=append_ms, prefill_ms=prefill_ms,
                            kernel_ms=kernel_ms,
                            tokens=tokens, reused=reused, host_plan_s=host_s,
                            rows=sum(L["rows"] for L in launches),
                            decode_rows=sum(L["drows"] for L in launches),
                            flops=sum(L["flops"] for L in launches),
                            evictions=getattr(mgr, "evictions", 0), frames=cache.k.shape[0])
        log(f"[bench] prefix caching {'on' if caching else 'off'}: step {step_ms * 1e3:.1f} us "
            f"(append {append_ms * 1e3:.1f}, prefill {prefill_ms * 1e3:.1f}), "
            f"{reused}/{tokens} tokens reused, host plan {host_s * 1e3:.1f} ms")
        del cache, launches
    on, off = res[True], res[False]
    value = on["tokens"] / (on["step_ms"] * 1e-3)
    tflops = on["flops"] / (on["kernel_ms"] * 1e-3) / 1e12
    out = {
        "metric": "prefix-cached prefill: prompt tokens served per second (reused + computed)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(on["step_ms"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "step": f"{w.rounds} rounds of (kv_append of the prompt rows not reused, paged prefill "
                "over them, kv_append of the rows of the tokens the round's decode steps generate); "
                "decode attention is not timed",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "rounds": w.rounds,
                   "prompt_tokens": on["tokens"], "reused_tokens": on["reused"],
                   "written_rows": on["rows"], "decode_rows": on["decode_rows"],
                   "evictions": on["evictions"],
                   "frames": on["frames"], "cache_flush_between_steps": not args.no_flush},
        "phases_us": {"append": round(on["append_ms"] * 1e3, 2),
                      "prefill": round(on["prefill_ms"] * 1e3, 2)},
        "without_caching": {"value": round(off["tokens"] / (off["step_ms"] * 1e-3), 1),
                            "ms_per_step": round(off["step_ms"], 5),
                            "append_us": round(off["append_ms"] * 1e3, 2),
                            "prefill_us": round(off["prefill_ms"] * 1e3, 2),
                            "written_rows": off["rows"], "frames": off["frames"]},
        "speedup_vs_no_caching": round(off["step_ms"] / on["step_ms"], 3),
        "host_plan_ms": {"native": round(on["host_plan_s"] * 1e3, 2),
                         "what": "block manager + slot lists for all rounds, before timing"},
        "roofline": {"kernel": "prefill_kernel", "bound": "mfma", "achieved": round(tflops, 2),
                     "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops_per_step": on["flops"],
                     "launch_us_per_step": round(on["kernel_ms"] * 1e3, 2),
                     "mfma_issued_frac_of_mfma_peak": round(tflops / MFMA_PEAK_TFLOPS, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline_prefix(w)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--head-dim", type=int, default=0, choices=(0, 16, 32, 64, 128, 256),
                    help="workload 2 with this head dim (H = 4096 / d, the same bytes per token)")
    ap.add_argument("--dtype", default="", choices=("", "bf16", "f16", "f32"),
                    help="workload 2 with this storage dtype")
    ap.add_argument("--seqs", type=int, default=0, help="workload 2 with this many sequences")
    ap.add_argument("--max-ctx", type=int, default=0,
                    help="workload 2 with contexts drawn from U[1, max-ctx]")
    ap.add_argument("--block-size", type=int, default=0,
                    help="workloads 2 and 3: tokens per frame (default 16; the pool keeps its "
                         "slot count)")
    ap.add_argument("--permuted-pool", action="store_true",
                    help="workload 5: a seeded permuted frame pool instead of first in, first out "
                         "in id order (the sensitivity variant)")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--prefill-batch-order", action="store_true",
                    help="dispatch prefill work in the default order, sequence by sequence in "
                         "batch order (by default the costliest sequences go first, "
                         "driver.prefill_order)")
    ap.add_argument("--decode-batch-order", action="store_true",
                    help="dispatch decode work in batch order (by default longest first: "
                         "driver.decode_order / group_order)")
    ap.add_argument("--ungrouped", action="store_true",
                    help="time paged_attn_decode even where sequences share frames (by default "
                         "forked sequences go through paged_attn_decode_grouped)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="with the default workload, skip timing the other workloads (1, 3-8) in "
                         "child processes after the headline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="first run one plain device-to-device copy of BYTES (a known-size "
                         "reference for hardware traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has "
              "no cross-GPU step; each GPU would serve its own sequences", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_126_amd as pkv
    from paged_kv_cache_126_amd.driver import DeviceCache, execute, plan
    from workloads import configs
    from workloads import values as V

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pkv.load()
    dev = torch.device("cuda:0")
    if args.block_size and args.workload not in (2, 3):
        print("--block-size applies to workloads 2 and 3 only", file=sys.stderr)
        sys.exit(2)
    reshaped = bool(args.head_dim or args.dtype or args.seqs or args.max_ctx)
    if reshaped and args.workload != 2:
        print("--head-dim, --dtype, --seqs and --max-ctx apply to workload 2 only", file=sys.stderr)
        sys.exit(2)
    if args.permuted_pool and args.workload != 5:
        print("--permuted-pool applies to workload 5 only", file=sys.stderr)
        sys.exit(2)
    if reshaped:
        S, C, B = args.seqs or 64, args.max_ctx or 2048, args.block_size or 16
        # a pool of 20,000 16-token frames, or enough for S contexts of C tokens
        NB = max(20000 * 16 // B, S * -(-C // B) * 11 // 10)
        w = configs.config2(S=S, max_ctx=C, NB=NB, B=B, D=args.head_dim or 128,
                            dtype=args.dtype or "bf16")
    elif args.block_size:
        w = {2: configs.config2, 3: configs.config3}[args.workload](B=args.block_size)
    elif args.permuted_pool:
        w = configs.config5(permuted=True)
    else:
        w = configs.FULL[args.workload]()
    log(f"[bench] workload {w.name}: {w.description}")
    if args.copy_calibration > 0:
        # a plain device copy of known size, for scaling hardware byte counters
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy of {args.copy_calibration} bytes done")
    if isinstance(w, configs.PrefixWorkload):
        bench_prefix(args, w, dev)
        return

    t0 = time.perf_counter()
    events, plan_mgr = plan(w)
    host_s = time.perf_counter() - t0
    cache = DeviceCache(w.NB, w.B, w.H, w.D, V.torch_dtype(w.dtype), dev, poison=True)
    points = []

    def rows(seqs, positions):
        ids = np.empty(len(seqs), dtype=np.int64)
        for s in np.unique(seqs):
            m = seqs == s
            ids[m] = w.idents(int(s), positions[m])
        idt = torch.from_numpy(ids).to(dev)
        return (V.draw_torch(w.seed, V.STREAM_K, idt, w.H, w.D, w.dtype, dev).contiguous(),
                V.draw_torch(w.seed, V.STREAM_V, idt, w.H, w.D, w.dtype, dev).contiguous())

    # The large-model workload's step is "append one token per sequence, then
    # attend": its last write batch is held back and replayed inside every
    # timed step (rewriting the same rows is idempotent).
    from paged_kv_cache_126_amd.driver import WriteBatch

    step_append = None
    if args.workload == 5:
        idx = max(i for i, e in enumerate(events) if isinstance(e, WriteBatch))
        step_append = events[idx]
        events = events[:idx] + events[idx + 1:]
    execute(events, cache, rows, points.append, chunk_rows=max(256, (1 << 25) // (w.H * w.D)))
    pt = points[-1]
    append_args = None
    if step_append is not None:
        k_new, v_new = rows(step_append.seqs, step_append.positions)
        slots = torch.from_numpy(step_append.slots).to(dev)
        append_args = (k_new, v_new, slots)
        cache.append(*append_args)
    torch.cuda.synchronize()
    log(f"[bench] cache written: {w.NB} frames, sum ctx {int(pt.context_lens.sum())}"
        + (f"; step appends {len(step_append.slots)} tokens" if step_append is not None else ""))

    if w.query_lens is not None:
        bench_prefill(args, w, pt, cache, dev)
        return
    q = V.draw_torch(w.seed, V.STREAM_Q, w.q_idents(pt.step), w.H, w.D, w.dtype, dev).contiguous()
    bt = torch.from_numpy(pt.tables).to(dev)
    cl = torch.from_numpy(pt.context_lens).to(dev)
    out = torch.empty((w.num_seqs, w.H, w.D), dtype=torch.float32, device=dev)
    max_ctx = int(pt.context_lens.max())
    policy = ungrouped_policy = pt.cache_policy
    # Forks of one prompt share their leading frames: the grouped pass reads
    # each shared row once for the whole group (so streaming loads suit it).
    from paged_kv_cache_126_amd.driver import share_groups

    group_start, group_shared = share_groups(pt.tables, pt.context_lens, w.B)
    grouped = not args.ungrouped and bool((group_shared > 0).any())
    groups = None
    if grouped:
        groups = (torch.from_numpy(group_start).to(dev), torch.from_numpy(group_shared).to(dev))
        policy = pkv.lib.PA_CACHE_STREAM
    # Dispatch order: longest work first (sequences; groups for the grouped
    # call). An ordered launch takes longer partitions by default.
    from paged_kv_cache_126_amd.driver import decode_order, group_order

    seq_order = grp_order = None
    if not args.decode_batch_order:
        seq_order = torch.from_numpy(decode_order(pt.context_lens, pt.tables)).to(dev)
        if grouped:
            grp_order = torch.from_numpy(group_order(group_start, group_shared,
                                                     pt.context_lens)).to(dev)
    shape = pkv.lib.make_shape(q, cache.k, bt, max_ctx, pkv.lib.PA_F32, args.partition_tokens, policy,
                               seq_order)
    ws = pkv.alloc_workspace(shape, dev)
    part_tokens = pkv.partition_tokens(shape)
    # the same launches in batch order, for context (their own default partition size)
    shape_batch = pkv.lib.make_shape(q, cache.k, bt, max_ctx, pkv.lib.PA_F32, args.partition_tokens,
                                     policy)
    ws_batch = pkv.alloc_workspace(shape_batch, dev)
    sum_ctx = int(pt.context_lens.sum())
    kv_bytes = 2 * w.H * w.D * w.elem_bytes * sum_ctx
    # distinct cache rows the step reads (less than sum_ctx when frames are shared)
    uniq_slots = np.unique(np.concatenate([
        pt.tables[s_, np.arange(c) // w.B].astype(np.int64) * w.B + np.arange(c) % w.B
        for s_, c in enumerate(pt.context_lens.tolist()) if c > 0]))
    kv_bytes_unique = 2 * w.H * w.D * w.elem_bytes * len(uniq_slots)
    # block-manager memory use at this point: distinct cached tokens over the
    # slots of the frames holding them (waste is the unfilled tail slots)
    frames_used = len(np.unique(uniq_slots // w.B))
    memory = {"frames_used": int(frames_used), "tokens_stored": int(len(uniq_slots)),
              "utilisation": round(len(uniq_slots) / (frames_used * w.B), 5)}
    # Cache flush between steps: read a 2 GiB buffer (8x the 256 MB last-level
    # cache). A read leaves clean lines; a write would leave dirty lines whose
    # write-back competes with the timed step.
    flush_buf = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def flush():
        torch.sum(flush_buf, dim=0, out=flush_sink)

    def attend(phase, pol, ordered=True):
        if phase == "grouped":
            pkv.paged_attn_decode_grouped(q, cache.k, cache.v, bt, cl, w.B, w.scale, out, max_ctx,
                                          groups[0], groups[1], ws if ordered else ws_batch,
                                          args.partition_tokens, cache_policy=pol,
                                          dispatch_order=grp_order if ordered else None)
        else:
            pkv.paged_attn_decode(q, cache.k, cache.v, bt, cl, w.B, w.scale, out, max_ctx,
                                  ws if ordered else ws_batch, args.partition_tokens, phase=phase,
                                  cache_policy=pol, dispatch_order=seq_order if ordered else None)

    def step(evs=None, use_groups=grouped, phases=False, ordered=True):
        """One step: [kv_append,] then the partition pass and the merge pass
        (the grouped call queues both). evs[0] start, evs[2] end; with
        `phases`, also evs[3] after the append and evs[1] after the
        partition pass (after both for the grouped call); with six events,
        evs[4], evs[5] the partition kernel's own start and end. Events
        recorded between kernels cost stream time themselves, so the step
        time comes from steps timed with the first two only."""
        if evs is not None:
            evs[0].record()
        if append_args is not None:
            cache.append(*append_args)
            if phases:
                evs[3].record()
        first = "grouped" if use_groups else "partitions"
        pol = policy if use_groups else ungrouped_policy
        if evs is not None and len(evs) > 4:
            with pkv.kernel_timing(evs[4], evs[5]):
                attend(first, pol, ordered)
        else:
            attend(first, pol, ordered)
        if phases:
            evs[1].record()
        if not use_groups:
            attend("merge", pol, ordered)
        if evs is not None:
            evs[2].record()

    for i in range(args.warmup):
        if not args.no_flush:
            flush()
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    # Pass 1 (the step time): plain launches bracketed by stream events.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if not args.no_flush:
            flush()
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Pass 1b (the breakdown): events between the phases as well.
    pevs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        if not args.no_flush:
            flush()
        step(pevs[i], phases=True)
    torch.cuda.synchronize()
    # Pass 2 (the kernel's duration): the same steps with the partition
    # kernel stamping its own start and end. Kept apart because a stamped
    # launch adds dispatch work that the stream events of pass 1 would count.
    kevs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for i in range(args.steps):
        if not args.no_flush:
            flush()
        step(kevs[i])
    torch.cuda.synchronize()
    # Context for the grouped call: the same steps through paged_attn_decode.
    ungrouped_ctx = None
    if grouped:
        uevs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        for i in range(args.steps):
            if not args.no_flush:
                flush()
            # batch order: sorting by length would split the fork families whose
            # shared frames this pass relies on reading close together in time
            step(uevs[i], use_groups=False, ordered=False)
        torch.cuda.synchronize()
        ums = float(np.mean([e[0].elapsed_time(e[2]) for e in uevs]))
        ungrouped_ctx = {"us_per_step": round(ums * 1e3, 2),
                         "GB/s": round(kv_bytes / (ums * 1e-3) / 1e9, 1),
                         "cache_policy": "reuse" if ungrouped_policy else "stream",
                         "what": "the same steps through paged_attn_decode in batch order (every "
                                 "sequence reads its own rows; shared frames hit in cache)"}
        log(f"[bench] ungrouped: step {ums * 1e3:.1f} us")
    # Context: the same steps dispatched in batch order.
    batch_order_ctx = None
    if seq_order is not None:
        bevs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        for i in range(args.steps):
            if not args.no_flush:
                flush()
            step(bevs[i], ordered=False)
        torch.cuda.synchronize()
        bms = float(np.mean([e[0].elapsed_time(e[2]) for e in bevs]))
        batch_order_ctx = {"us_per_step": round(bms * 1e3, 2),
                           "GB/s": round(kv_bytes / (bms * 1e-3) / 1e9, 1),
                           "partition_tokens": pkv.partition_tokens(shape_batch)}
        log(f"[bench] batch order: step {bms * 1e3:.1f} us")
    part_start = 3 if append_args is not None else 0
    append_ms = np.array([e[0].elapsed_time(e[3]) for e in pevs]) if append_args else np.zeros(1)
    part_ms = np.array([e[part_start].elapsed_time(e[1]) for e in pevs])
    kern_ms = np.array([e[4].elapsed_time(e[5]) for e in kevs])  # kernel alone, no dispatch gap
    merge_ms = np.array([e[1].elapsed_time(e[2]) for e in pevs])
    # the library queues no merge when no sequence spans two partitions (no
    # workspace); the events around that call then time only themselves
    merge_launched = ws is not None
    step_ms = np.array([e[0].elapsed_time(e[2]) for e in evs])
    ms = float(step_ms.mean())
    log(f"[bench] {args.steps} steps: step {ms * 1e3:.1f} us (median {np.median(step_ms) * 1e3:.1f}), "
        + (f"grouped call {part_ms.mean() * 1e3:.1f} us (grouped partition kernel alone "
           f"{kern_ms.mean() * 1e3:.1f})" if grouped else
           f"partition kernel {part_ms.mean() * 1e3:.1f} us (kernel alone {kern_ms.mean() * 1e3:.1f}), "
           + (f"merge {merge_ms.mean() * 1e3:.1f} us" if merge_launched else
              "no merge launch (no sequence spans two partitions)"))
        + (f", kv_append {append_ms.mean() * 1e3:.1f} us" if append_args else ""))

    # Streaming-read ceiling: the same non-temporal 16-byte loads over a
    # buffer of the step's K/V size, no arithmetic (pa_stream_read), cold.
    ceil_buf = torch.ones(kv_bytes_unique // 2, dtype=torch.int16, device=dev)
    ceil_sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        pkv.lib.stream_read(ceil_buf, ceil_sink)
    cevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(20)]
    for c0, c1 in cevs:
        if not args.no_flush:
            flush()
        with pkv.kernel_timing(c0, c1):
            pkv.lib.stream_read(ceil_buf, ceil_sink)
    torch.cuda.synchronize()
    ceil_us = float(np.mean([c0.elapsed_time(c1) for c0, c1 in cevs])) * 1e3
    ceil_gbs = kv_bytes_unique / ceil_us / 1e3
    patterns = frame_patterns(w, ceil_buf, ceil_sink, part_tokens, flush, args, dev)
    del ceil_buf
    log(f"[bench] streaming-read ceiling over {kv_bytes_unique / 1e9:.3f} GB: {ceil_us:.1f} us, "
        f"{ceil_gbs:.0f} GB/s")

    # Copy-on-write frame copies (shared-prefix workload): the step's copies,
    # redirected to frames the schedule never uses so the cache stays intact.
    from paged_kv_cache_126_amd.driver import CopyBlocks

    cow = None
    cow_pairs = [e.pairs for e in events if isinstance(e, CopyBlocks)]
    if cow_pairs:
        pairs = np.concatenate(cow_pairs).copy()
        spare = plan_mgr.free_list()[-len(pairs):]
        if len(spare) == len(pairs):
            pairs[:, 1] = spare
            pairs_dev = torch.from_numpy(pairs).to(dev)
            cts = []
            for i in range(args.steps):
                if not args.no_flush:
                    flush()
                c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                c0.record()
                cache.copy_blocks(pairs_dev)
                c1.record()
                torch.cuda.synchronize()
                cts.append(c0.elapsed_time(c1))
            cbytes = 2 * 2 * len(pairs) * w.B * w.H * w.D * w.elem_bytes  # K and V, read + write
            cus = float(np.mean(cts)) * 1e3
            cow = {"pairs": len(pairs), "us": round(cus, 2), "bytes": cbytes,
                   "GB/s": round(cbytes / cus / 1e3, 1)}
            log(f"[bench] copy-on-write: {len(pairs)} frame copies in {cus:.1f} us")

    # warm (no flush) back-to-back rate, reported beside the cold headline
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / args.steps

    gbs = kv_bytes / (ms * 1e-3) / 1e9
    # The roofline counts the bytes the method must move: each distinct cache
    # row once (equal to kv_bytes unless sequences share frames).
    # Duration: the partition kernel's own start-to-end stamps (the same
    # interval rocprofv3's kernel trace reports), averaged over the timed steps.
    part_gbs = kv_bytes_unique / (kern_ms.mean() * 1e-3) / 1e9
    digest = kernel_source_digest()
    traffic = measured_traffic(w.name, digest)
    res = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "step": "kv_append + decode attention" if append_args else "decode attention",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.num_seqs, "heads": w.H, "head_dim": w.D,
            "block_size": w.B, "num_blocks": w.NB, "description": w.description,
            "sum_ctx": sum_ctx, "kv_bytes": kv_bytes, "kv_bytes_unique": kv_bytes_unique,
            "partition_tokens": part_tokens,
            "out_dtype": "f32", "cache_flush_between_steps": not args.no_flush,
            "cache_policy": "reuse" if policy else "stream",
            "memory": memory,
        },
        "us_per_step": round(ms * 1e3, 2),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "warm_us_per_step": round(warm_ms * 1e3, 2),
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "launch": ("paged_attn_decode_grouped (grouped partition pass + merge pass)" if grouped
                   else "paged_attn_decode_partitions + paged_attn_merge"),
        "groups": ({"count": int(len(group_shared)), "sequences_in_shared_groups":
                    int(sum(b - a for a, b, sh in zip(group_start[:-1], group_start[1:], group_shared)
                            if sh > 0)),
                    "shared_tokens": sorted({int(x) for x in group_shared})[-4:]} if grouped else None),
        "ungrouped": ungrouped_ctx,
        "dispatch_order": ("batch order" if seq_order is None else
                           "longest first (driver.group_order)" if grouped else
                           "longest first, fork families together (driver.decode_order)"),
        "batch_order": batch_order_ctx,
        "kernels_us": {"partition": round(float(part_ms.mean()) * 1e3, 2),
                       "partition_kernel_alone": round(float(kern_ms.mean()) * 1e3, 2),
                       "merge": (None if grouped or not merge_launched
                                 else round(float(merge_ms.mean()) * 1e3, 2)),
                       "merge_launched": (not grouped) and merge_launched,
                       "kv_append": round(float(append_ms.mean()) * 1e3, 2) if append_args else None,
                       "what": ("partition = the grouped call (both passes) between stream events; "
                                "partition_kernel_alone = the grouped partition kernel's own stamps"
                                if grouped else "between stream events; kernel alone = its own stamps")},
        "roofline": {
            "kernel": "decode_group_kernel" if grouped else "decode_partition_kernel", "bound": "hbm",
            "achieved": round(part_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(part_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes_unique,
            "launch_us": round(float(kern_ms.mean()) * 1e3, 2),
            "read_ceiling": {"GB/s": round(ceil_gbs, 1), "us": round(ceil_us, 2),
                             "what": "pa_stream_read: the same non-temporal 16-byte loads over "
                                     "as many bytes, in order, nothing else"},
            "frac_of_read_ceiling": round(part_gbs / ceil_gbs, 4),
            "access_patterns": patterns,
        },
        "kernel_source_digest": digest,
        "cow_frame_copies": cow,
        "host_plan_ms": {"native": round(host_s * 1e3, 2),
                         "what": "block manager replay of the whole schedule (prefill, forks, "
                                 "decode steps) before timing"},
    }
    default_run = (args.workload == 2 and not args.block_size and not args.partition_tokens
                   and not args.head_dim and not args.dtype and not args.seqs and not args.max_ctx
                   and not args.decode_batch_order and not args.ungrouped)
    if default_run and not args.no_others:
        res["other_workloads"] = other_workloads(args)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on the whole step")
        res["cpu_baseline"] = cpu_baseline(w, dev)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
