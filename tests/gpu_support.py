"""Shared set-up for the GPU tests: run a workload through the HIP path, and
compute the oracle's answer for the same seeded inputs on the host.

The two sides share only the seeded generator (workloads.values) and the
workload description (workloads.configs). The GPU side plans with the
product block manager and writes the cache with kv_append; the oracle side
plans with its own block manager and scatters on the host.
"""
from __future__ import annotations

import math
import sys

import numpy as np

from oracle import blockmgr as obm
from oracle.oracle import STORAGE, default as oracle_default
from workloads import values as V

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    import pytest
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_126_amd as pkv

    pkv.load()  # raises (fails the test) if the HIP library is missing


def rows_fn(w, device):
    """Device K/V rows for (seqs, positions) from the shared generator."""
    import torch

    def rows(seqs, positions):
        ids = np.empty(len(seqs), dtype=np.int64)
        for s in np.unique(seqs):
            m = seqs == s
            ids[m] = w.idents(int(s), positions[m])
        idt = torch.from_numpy(ids).to(device)
        k = V.draw_torch(w.seed, V.STREAM_K, idt, w.H, w.D, w.dtype, device)
        v = V.draw_torch(w.seed, V.STREAM_V, idt, w.H, w.D, w.dtype, device)
        return k.contiguous(), v.contiguous()

    return rows


def pad_frame_for(w) -> int:
    """A frame the schedule never allocates (stays NaN), for table padding."""
    from paged_kv_cache_126_amd.driver import plan

    _, mgr = plan(w)
    fl = mgr.free_list()
    return fl[-1] if fl else -1


def run_gpu(w, partition_tokens: int = 0, out_dtype=None, phases: bool = False, poison=True,
            keep_cache=False, cache_policy=None, grouped: bool = False, order=None):
    """Play workload ``w`` on cuda:0. Returns a list of (AttendPoint, out cpu
    tensor) and, with keep_cache, the DeviceCache. ``grouped`` runs
    paged_attn_decode_grouped with the groups ``share_groups`` finds in each
    attention point's tables, and checks at every point that its output
    equals paged_attn_decode's at the same partition size, bit for bit.
    ``order`` ("longest": driver.decode_order / group_order; "random": a
    seeded permutation) sets the dispatch order of every launch."""
    import torch

    import paged_kv_cache_126_amd as pkv
    from paged_kv_cache_126_amd.driver import (DeviceCache, decode_order, execute, group_order, plan,
                                               share_groups)

    dev = torch.device("cuda:0")
    pad = pad_frame_for(w)
    events, _ = plan(w, pad=pad)
    tdt = V.torch_dtype(w.dtype)
    cache = DeviceCache(w.NB, w.B, w.H, w.D, tdt, dev, poison=poison)
    results = []

    def on_attend(pt):
        q = V.draw_torch(w.seed, V.STREAM_Q, w.q_idents(pt.step), w.H, w.D, w.dtype, dev).contiguous()
        bt = torch.from_numpy(pt.tables).to(dev)
        cl = torch.from_numpy(pt.context_lens).to(dev)
        odt = torch.float32 if out_dtype is None else out_dtype
        out = torch.full((w.num_seqs, w.H, w.D), float("nan"), dtype=odt, device=dev)
        max_ctx = int(pt.context_lens.max())
        policy = pt.cache_policy if cache_policy is None else cache_policy
        gs, gsh = share_groups(pt.tables, pt.context_lens, w.B)
        rng = np.random.default_rng(w.seed + pt.step)
        seq_ord = grp_ord = None
        if order == "longest":
            seq_ord = decode_order(pt.context_lens, pt.tables)
            grp_ord = group_order(gs, gsh, pt.context_lens)
        elif order == "random":
            seq_ord = rng.permutation(w.num_seqs).astype(np.int32)
            grp_ord = rng.permutation(len(gsh)).astype(np.int32)
        seq_ord = None if seq_ord is None else torch.from_numpy(seq_ord).to(dev)
        grp_ord = None if grp_ord is None else torch.from_numpy(grp_ord).to(dev)
        shape = pkv.lib.make_shape(q, cache.k, bt, max_ctx, pkv.lib.dtype_code(out), partition_tokens,
                                   policy, seq_ord)
        ws = pkv.alloc_workspace(shape, dev)
        kw = dict(partition_tokens=partition_tokens, cache_policy=policy, dispatch_order=seq_ord)
        if grouped:
            pkv.paged_attn_decode_grouped(q, cache.k, cache.v, bt, cl, w.B, w.scale, out, max_ctx,
                                          torch.from_numpy(gs).to(dev), torch.from_numpy(gsh).to(dev),
                                          ws, partition_tokens, cache_policy=policy,
                                          dispatch_order=grp_ord)
            ref = torch.full_like(out, float("nan"))
            pkv.paged_attn_decode(q, cache.k, cache.v, bt, cl, w.B, w.scale, ref, max_ctx, ws, **kw)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), (f"grouped != ungrouped at step {pt.step} ({len(gsh)} groups): "
                                           f"max diff {float((out - ref).abs().max()):.3e}")
        elif phases:
            pkv.paged_attn_decode(q, cache.k, cache.v, bt, cl, w.B, w.scale, out, max_ctx, ws,
                                  phase="partitions", **kw)
            pkv.paged_attn_decode(q, cache.k, cache.v, bt, cl, w.B, w.scale, out, max_ctx, ws,
                                  phase="merge", **kw)
        else:
            pkv.paged_attn_decode(q, cache.k, cache.v, bt, cl, w.B, w.scale, out, max_ctx, ws, **kw)
        torch.cuda.synchronize()
        results.append((pt, out.cpu()))

    execute(events, cache, rows_fn(w, dev), on_attend, chunk_rows=max(256, (1 << 25) // (w.H * w.D)))
    torch.cuda.synchronize()
    return (results, cache) if keep_cache else results


def run_gpu_prefill(w, out_dtype=None, order=None, split_weights=False):
    """Play prefill workload ``w`` on cuda:0: write every token with kv_append,
    then one paged_attn_prefill over each sequence's last query_lens tokens
    (``split_weights`` passed on). ``order`` ("cost": driver.prefill_order;
    "random": a seeded permutation of the work items) dispatches the query
    tiles in that order, and checks that the output equals the
    default-order launch's bit for bit. Returns (AttendPoint, query_start,
    out cpu tensor [T, H, D])."""
    import torch

    import paged_kv_cache_126_amd as pkv
    from paged_kv_cache_126_amd.driver import DeviceCache, execute, plan, prefill_order

    dev = torch.device("cuda:0")
    events, _ = plan(w, pad=pad_frame_for(w))
    cache = DeviceCache(w.NB, w.B, w.H, w.D, V.torch_dtype(w.dtype), dev, poison=True)
    res = []

    def on_attend(pt):
        qs, ids = w.prefill_queries(pt.context_lens)
        T = int(qs[-1])
        q = V.draw_torch(w.seed, V.STREAM_Q, ids, w.H, w.D, w.dtype, dev).contiguous()
        odt = torch.float32 if out_dtype is None else out_dtype
        out = torch.full((T, w.H, w.D), float("nan"), dtype=odt, device=dev)
        args = (q, cache.k, cache.v, torch.from_numpy(pt.tables).to(dev),
                torch.from_numpy(pt.context_lens).to(dev), torch.from_numpy(qs.astype(np.int32)).to(dev),
                w.B, w.scale, out, int(pt.context_lens.max()), int(np.diff(qs).max()))
        pkv.paged_attn_prefill(*args, split_weights=split_weights)
        if order is not None:
            mq = int(np.diff(qs).max())
            items = len(pt.context_lens) * -(-mq // pkv.PA_PREFILL_TILE)
            work = (prefill_order(pt.context_lens, qs, mq) if order == "cost" else
                    np.random.default_rng(w.seed).permutation(items).astype(np.int32))
            first = out.clone()
            out.fill_(float("nan"))
            pkv.paged_attn_prefill(*args, work_order=torch.from_numpy(work).to(dev),
                                   split_weights=split_weights)
            torch.cuda.synchronize()
            assert torch.equal(out, first), f"dispatch order {order} changed the output"
        torch.cuda.synchronize()
        res.append((pt, qs, out.cpu()))

    execute(events, cache, rows_fn(w, dev), on_attend, chunk_rows=max(256, (1 << 25) // (w.H * w.D)))
    torch.cuda.synchronize()
    return res[-1]


def oracle_prefill(w, pad):
    """fp64 oracle output [T, H, D] of prefill workload ``w``."""
    orc = oracle_default()
    snap = obm.replay(w, pad_frame=pad)[0][-1]
    k, v = oracle_caches(w, snap)
    qs, ids = w.prefill_queries(snap.context_lens)
    q = V.draw_np(w.seed, V.STREAM_Q, ids, w.H, w.D, w.dtype)
    return snap, orc.paged_prefill(q, k, v, snap.tables, snap.context_lens, qs, w.B, w.scale, w.dtype)


def _widen_rows(w, ids, dev):
    """fp64 K and V rows [n, H, D] of identities ``ids`` (generator rows drawn
    on the device and checked against the host draw, widened exactly by the
    oracle's decoders)."""
    import torch

    orc = oracle_default()
    ids = np.asarray(ids, dtype=np.int64)
    idt = torch.from_numpy(ids).to(dev)
    k = orc.widen(_rows_checked(w, ids, idt, V.STREAM_K, dev), w.dtype)
    v = orc.widen(_rows_checked(w, ids, idt, V.STREAM_V, dev), w.dtype)
    return k, v


def oracle_prefill_full(w, context_lens, device: str = "cuda:0"):
    """fp64 output [T, H, D] of prefill workload ``w``: every query of every
    sequence, by the dense causal form over the sequence's logical rows
    (oracle/dense.py, pinned against the C oracle)."""
    import torch

    from oracle import dense

    orc = oracle_default()
    dev = torch.device(device)
    qs, qids = w.prefill_queries(context_lens)
    q_all = orc.widen(V.draw_np(w.seed, V.STREAM_Q, qids, w.H, w.D, w.dtype), w.dtype)
    scale = float(np.float32(w.scale))
    out = np.empty((int(qs[-1]), w.H, w.D), dtype=np.float64)
    for s in range(len(context_lens)):
        n = int(qs[s + 1] - qs[s])
        if n == 0:
            continue
        ctx = int(context_lens[s])
        k, v = _widen_rows(w, w.idents(s, np.arange(ctx)), dev)
        out[qs[s]:qs[s + 1]] = dense.causal_attention(q_all[qs[s]:qs[s + 1]], k, v, scale, ctx - n)
    return out


def oracle_caches(w, snap):
    """Host K/V caches built by the oracle's scatter from a replay snapshot."""
    return _caches_from_idents(w, w.NB, snap.slot_ident)


def oracle_outputs(w, pad):
    """fp64 oracle outputs [S, H, D] at every attention point of ``w``."""
    orc = oracle_default()
    snaps, _ = obm.replay(w, pad_frame=pad)
    outs = []
    for i, snap in enumerate(snaps):
        k, v = oracle_caches(w, snap)
        q = V.draw_np(w.seed, V.STREAM_Q, w.q_idents(i), w.H, w.D, w.dtype)
        outs.append((snap, orc.paged_decode(q, k, v, snap.tables, snap.context_lens, w.B, w.scale,
                                            w.dtype)))
    return outs


def _rows_checked(w, ids, ids_dev, stream, dev):
    """Host copy of the generator's rows for identities ``ids`` (all heads),
    drawn by torch on ``dev`` from ``ids_dev`` (the same identities on the
    device); the first and last rows are checked bit for bit against the
    numpy draw of the same recipe."""
    t = V.draw_torch(w.seed, stream, ids_dev, w.H, w.D, w.dtype, dev)
    host = (t.cpu().numpy() if w.dtype == "f32" else t.view(_torch().int16).cpu().numpy().view(np.uint16))
    del t
    ends = np.unique([0, len(ids) - 1])
    want = V.draw_np(w.seed, stream, ids[ends], w.H, w.D, w.dtype)
    assert np.array_equal(host[ends].view(np.uint8), want.view(np.uint8)), "generator draws differ"
    return host


def _torch():
    import torch

    return torch


def oracle_full(w, step: int, ctx: np.ndarray, chunk_tokens: int = 1 << 14, device: str = "cuda:0"):
    """fp64 oracle output [S, H, D] of attention point ``step`` for every
    sequence and head, by the contiguous definition over each sequence's
    logical tokens. The oracle's inputs are the generator's rows for the
    sequence's value identities (no block table, no device cache): drawn by
    torch on the GPU for speed, copied to the host, and spot-checked against
    the numpy draw. Sequences are attended in chunks of about
    ``chunk_tokens`` tokens, so host memory stays small."""
    torch = _torch()
    orc = oracle_default()
    dev = torch.device(device)
    S = len(ctx)
    out = np.empty((S, w.H, w.D), dtype=np.float64)
    q_all = V.draw_np(w.seed, V.STREAM_Q, w.q_idents(step), w.H, w.D, w.dtype)
    s0 = 0
    while s0 < S:
        s1, tok = s0, 0
        while s1 < S and (s1 == s0 or tok + int(ctx[s1]) <= chunk_tokens):
            tok += int(ctx[s1])
            s1 += 1
        ids = np.concatenate([w.idents(s, np.arange(int(ctx[s]))) for s in range(s0, s1)])
        start = np.concatenate([[0], np.cumsum(ctx[s0:s1].astype(np.int64))])
        ids = ids.astype(np.int64)
        idt = torch.from_numpy(ids).to(dev)
        k = _rows_checked(w, ids, idt, V.STREAM_K, dev)
        v = _rows_checked(w, ids, idt, V.STREAM_V, dev)
        out[s0:s1] = orc.dense_attention(q_all[s0:s1], k, v, start, w.scale, w.dtype)
        del k, v, idt
        s0 = s1
    return out


def max_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.all(np.isfinite(a)), "non-finite values in the GPU output"
    return float(np.max(np.abs(a - b))) if a.size else 0.0


__all__ = ["TOL", "say", "require_gpu", "run_gpu", "oracle_outputs", "oracle_full", "max_err",
           "pad_frame_for", "oracle_caches", "math"]


def run_gpu_prefix(w, caching: bool = True, pool_frames=None, snapshot_caches: bool = False):
    """Play prefix-sharing workload ``w`` on cuda:0, round by round: write the
    rows the block manager asks for with kv_append, one paged_attn_prefill
    over the written positions, then the round's decode steps (kv_append of
    the step's tokens, paged_attn_decode over the step's requests). Returns
    a list of (PrefillRound, prefill out cpu tensor [T, H, D], (k, v) cpu
    caches after the round or None, [decode out cpu tensor per step])."""
    import torch

    import paged_kv_cache_126_amd as pkv
    from paged_kv_cache_126_amd.driver import DeviceCache, plan_prefix_rounds

    dev = torch.device("cuda:0")
    rounds, _ = plan_prefix_rounds(w, caching, pool_frames=pool_frames)
    NB = w.NB if pool_frames is None else pool_frames
    cache = DeviceCache(NB, w.B, w.H, w.D, V.torch_dtype(w.dtype), dev, poison=True)
    rows = rows_fn(w, dev)
    res = []
    for rd in rounds:
        wb = rd.writes
        if len(wb.slots):
            k_new, v_new = rows(wb.seqs, wb.positions)
            cache.append(k_new, v_new, torch.from_numpy(wb.slots).to(dev))
        T = int(rd.query_start[-1])
        ids = w.idents_rows(wb.seqs, wb.positions)
        q = V.draw_torch(w.seed, V.STREAM_Q, torch.from_numpy(ids).to(dev), w.H, w.D, w.dtype,
                         dev).contiguous()
        out = torch.full((T, w.H, w.D), float("nan"), dtype=torch.float32, device=dev)
        pkv.paged_attn_prefill(q, cache.k, cache.v, torch.from_numpy(rd.tables).to(dev),
                               torch.from_numpy(rd.context_lens).to(dev),
                               torch.from_numpy(rd.query_start).to(dev), w.B, w.scale, out,
                               int(rd.context_lens.max()), int(np.diff(rd.query_start).max()))
        torch.cuda.synchronize()
        pout = out.cpu()
        douts = []
        for st in rd.decode or []:
            wb = st.writes
            k_new, v_new = rows(wb.seqs, wb.positions)
            cache.append(k_new, v_new, torch.from_numpy(wb.slots).to(dev))
            ids = torch.from_numpy(w.idents_rows(wb.seqs, wb.positions)).to(dev)
            qd = V.draw_torch(w.seed, V.STREAM_Q, ids, w.H, w.D, w.dtype, dev).contiguous()
            bt = torch.from_numpy(st.tables).to(dev)
            cl = torch.from_numpy(st.context_lens).to(dev)
            dout = torch.full((len(wb.seqs), w.H, w.D), float("nan"), dtype=torch.float32,
                              device=dev)
            max_ctx = int(st.context_lens.max())
            shape = pkv.lib.make_shape(qd, cache.k, bt, max_ctx, pkv.lib.PA_F32, 0,
                                       pkv.lib.PA_CACHE_REUSE)
            ws = pkv.alloc_workspace(shape, dev)
            pkv.paged_attn_decode(qd, cache.k, cache.v, bt, cl, w.B, w.scale, dout, max_ctx, ws,
                                  cache_policy=pkv.lib.PA_CACHE_REUSE)
            douts.append(dout.cpu())
        torch.cuda.synchronize()
        snap = (cache.k.cpu(), cache.v.cpu()) if snapshot_caches else None
        res.append((rd, pout, snap, douts))
    return res


def oracle_prefix_rounds(w, caching: bool = True, pool_frames=None, with_decode: bool = True):
    """The oracle's rounds of ``w`` with fp64 outputs [T, H, D] over the
    positions each request writes, its host caches after each round, and
    (with_decode) the fp64 decode outputs of every decode step."""
    from oracle.prefixcache import replay_rounds

    orc = oracle_default()
    rounds, _ = replay_rounds(w, caching=caching, pool_frames=pool_frames)
    NB = w.NB if pool_frames is None else pool_frames
    res = []
    for rd in rounds:
        k, v = _caches_from_idents(w, NB, rd.slot_ident)
        counts = rd.context_lens.astype(np.int64) - rd.reused
        qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        ids = np.concatenate([w.idents(c, np.arange(int(rd.reused[i]), int(rd.context_lens[i])))
                              for i, c in enumerate(rd.seqs)])
        q = V.draw_np(w.seed, V.STREAM_Q, ids, w.H, w.D, w.dtype)
        out = orc.paged_prefill(q, k, v, rd.tables, rd.context_lens, qs, w.B, w.scale, w.dtype)
        douts = []
        if with_decode:
            for pt in rd.decode:
                qids = np.array([w.idents(c, [int(n) - 1])[0] for c, n in zip(pt.seqs, pt.context_lens)])
                qd = V.draw_np(w.seed, V.STREAM_Q, qids, w.H, w.D, w.dtype)
                douts.append(orc.paged_decode(qd, k, v, pt.tables, pt.context_lens, w.B, w.scale,
                                              w.dtype))
        res.append((rd, qs, out, (k, v), douts))
    return res


def _caches_from_idents(w, NB, slot_ident):
    """NaN-filled host caches with the identity's rows scattered by the oracle."""
    orc = oracle_default()
    nan = V.nan_bits(w.dtype)
    k = np.full((NB, w.B, w.H, w.D), nan, dtype=STORAGE[w.dtype])
    v = k.copy()
    slots = np.nonzero(slot_ident >= 0)[0].astype(np.int64)
    ids = slot_ident[slots]
    orc.kv_append(V.draw_np(w.seed, V.STREAM_K, ids, w.H, w.D, w.dtype),
                  V.draw_np(w.seed, V.STREAM_V, ids, w.H, w.D, w.dtype), slots, k, v, w.B, w.dtype)
    return k, v


def oracle_prefix_full(w, rd, device: str = "cuda:0"):
    """fp64 outputs of one prefix-cache round ``rd`` (a driver PrefillRound):
    the prefill output [T, H, D] over every written position of every
    request, and each decode step's output [len(step), H, D], by the dense
    causal form over each conversation's logical rows (oracle/dense.py).
    A conversation's decode queries sit at the positions right after its
    prompt, so one causal call per conversation covers the prefill queries
    and every decode query of the round."""
    import torch

    from oracle import dense

    orc = oracle_default()
    dev = torch.device(device)
    scale = float(np.float32(w.scale))
    T = int(rd.query_start[-1])
    pre = np.empty((T, w.H, w.D), dtype=np.float64)
    steps = rd.decode or []
    final = {int(c): int(n) for i, (c, n) in enumerate(zip(rd.seqs, rd.context_lens))}
    for st in steps:
        for c, n in zip(st.writes.seqs, st.context_lens):
            final[int(c)] = max(final[int(c)], int(n))
    outs = {}
    for i, c in enumerate(rd.seqs):
        c = int(c)
        lo, ctx, last = int(rd.reused[i]), int(rd.context_lens[i]), final[c]
        k, v = _widen_rows(w, w.idents(c, np.arange(last)), dev)
        q = orc.widen(V.draw_np(w.seed, V.STREAM_Q, w.idents(c, np.arange(lo, last)), w.H, w.D,
                                w.dtype), w.dtype)
        o = dense.causal_attention(q, k, v, scale, lo)  # queries at positions lo .. last - 1
        pre[rd.query_start[i]:rd.query_start[i + 1]] = o[:ctx - lo]
        outs[c] = (lo, o)
    dec = []
    for st in steps:
        d = np.empty((len(st.writes.seqs), w.H, w.D), dtype=np.float64)
        for j, (c, n) in enumerate(zip(st.writes.seqs, st.context_lens)):
            lo, o = outs[int(c)]
            d[j] = o[int(n) - 1 - lo]
        dec.append(d)
    return pre, dec


def oracle_prefix_sampled(w, picks):
    """fp64 outputs for sampled (conversation, position, head): causal
    attention of that token's query over tokens 0 .. position of its
    conversation, by the C oracle's contiguous definition."""
    orc = oracle_default()
    res = {}
    for c, pos, h in picks:
        ids = w.idents(c, np.arange(pos + 1))
        k = V.draw_np(w.seed, V.STREAM_K, ids, w.H, w.D, w.dtype, heads=[h])
        v = V.draw_np(w.seed, V.STREAM_V, ids, w.H, w.D, w.dtype, heads=[h])
        q = V.draw_np(w.seed, V.STREAM_Q, w.idents(c, [pos]), w.H, w.D, w.dtype, heads=[h])
        o = orc.dense_attention(q, k, v, np.array([0, pos + 1], dtype=np.int64), w.scale, w.dtype)
        res[(c, pos, h)] = o[0, 0]
    return res
