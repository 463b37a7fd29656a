"""Plays a decode schedule through the block manager and the library.

A schedule is any object with the attributes ``NB``, ``B``, ``num_seqs``,
``prefill`` ([(seq, n_tokens)]), ``forks`` ([(parent, child)]), ``steps``
(per decode step, the sequences appending one token, in order),
``attend_after`` (step indices after which attention runs; -1 = after the
prefill) and ``frame_order`` (initial free list or None).

:func:`plan` runs only the host block manager and returns the ordered list of
frame copies (copy-on-write), KV writes and attention points: what a serving
loop would hand the device. :class:`DeviceCache` plus :func:`execute` carry
them out on the GPU with ``kv_copy_blocks`` and ``kv_append``. Within one
decode step every copy is issued before any write, so a copy always reads the
shared frame as it was before the step.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .native_blocks import NativeBlockManager


@dataclass
class WriteBatch:
    seqs: np.ndarray       # int64 [N]: sequence of each row
    positions: np.ndarray  # int64 [N]: token position inside that sequence
    slots: np.ndarray      # int64 [N]: destination slot (frame * B + offset)


@dataclass
class CopyBlocks:
    pairs: np.ndarray      # int64 [n, 2]: (source frame, new private frame), copy-on-write


@dataclass
class AttendPoint:
    step: int                 # index in schedule.attend_after order
    tables: np.ndarray        # int32 [S, max_blocks]
    context_lens: np.ndarray  # int32 [S]
    shared_frames: bool = False  # some frame is referenced by two or more sequences

    @property
    def cache_policy(self) -> int:
        """The decode cache hint that fits these tables (see pa_cache_policy)."""
        from .lib import PA_CACHE_REUSE, PA_CACHE_STREAM

        return PA_CACHE_REUSE if self.shared_frames else PA_CACHE_STREAM


def make_manager(num_frames: int, block_size: int, order=None, prefix_caching: bool = False):
    """The host block manager (C++, include/paged_blocks.h)."""
    return NativeBlockManager(num_frames, block_size, order, prefix_caching)


def plan(schedule, pad: int = -1, max_blocks: int | None = None):
    """Host-only replay. Returns (events, manager); each event is a
    WriteBatch or an AttendPoint, in the order a serving loop issues them."""
    mgr = make_manager(schedule.NB, schedule.B, schedule.frame_order)
    B = schedule.B
    sids = list(range(schedule.num_seqs))
    events = []
    seqs, poss, slots, copies = [], [], [], []

    def flush():
        if copies:
            events.append(CopyBlocks(np.array(copies, dtype=np.int64).reshape(-1, 2)))
            copies.clear()
        if seqs:
            events.append(WriteBatch(np.concatenate(seqs), np.concatenate(poss), np.concatenate(slots)))
            seqs.clear(), poss.clear(), slots.clear()

    n_attend = 0

    def attend():
        nonlocal n_attend
        flush()
        events.append(AttendPoint(n_attend, mgr.tables(sids, pad, max_blocks), mgr.context_lens(sids),
                                  bool(mgr.ref.max() > 1)))
        n_attend += 1

    for s, n in schedule.prefill:
        sl = mgr.init_sequence(s, n)
        seqs.append(np.full(n, s, dtype=np.int64))
        poss.append(np.arange(n, dtype=np.int64))
        slots.append(sl)
    for parent, child in schedule.forks:
        mgr.fork(parent, child)
    if -1 in schedule.attend_after:
        attend()
    else:
        flush()
    for k, step in enumerate(schedule.steps):
        if len(step):
            step = np.asarray(step, dtype=np.int64)
            # position of each appended token: the sequence's length before
            # the step plus its earlier appearances in the step
            uniq, inv = np.unique(step, return_inverse=True)
            base = mgr.context_lens(uniq.tolist()).astype(np.int64)[inv]
            seen = {}
            rank = np.empty(len(step), dtype=np.int64)
            for i, sq in enumerate(step.tolist()):
                rank[i] = seen.get(sq, 0)
                seen[sq] = rank[i] + 1
            sl, cow = mgr.append_tokens(step.tolist())
            for src, dst, _ in cow[cow[:, 0] >= 0]:
                copies.append((int(src), int(dst)))  # copy-on-write of the shared frame
            seqs.append(step)
            poss.append(base + rank)
            slots.append(sl)
        if k in schedule.attend_after:
            attend()
        else:
            flush()
    flush()
    return events, mgr


def share_groups(tables: np.ndarray, context_lens: np.ndarray, block_size: int,
                 max_group: int = 4, min_shared: int = 1):
    """Groups of consecutive sequences whose block-table rows start with the
    same frames (forks of one prompt), for ``paged_attn_decode_grouped``.

    Greedy over the batch order: a group starts at sequence i and takes the
    following sequences while they share at least ``min_shared`` leading
    frames with sequence i, up to ``max_group`` members. A group's shared
    length is the run of leading frames common to all its members, in
    tokens, cut to its shortest member's context. Sequences sharing nothing
    with their neighbours form groups of one with no shared tokens. Returns
    int32 ``group_start`` [G + 1] and ``group_shared`` [G].
    """
    tables = np.asarray(tables)
    ctx = np.asarray(context_lens, dtype=np.int64)
    S = len(ctx)
    nblk = -(-ctx // block_size)  # table entries in use

    def common(i, j):
        n = int(min(nblk[i], nblk[j]))
        neq = np.flatnonzero(tables[i, :n] != tables[j, :n])
        return n if len(neq) == 0 else int(neq[0])

    starts, shared = [0], []
    i = 0
    while i < S:
        j, run = i + 1, int(nblk[i])
        while j < S and j - i < max_group:
            c = common(i, j)
            if c < min_shared:
                break
            run = min(run, c)
            j += 1
        members = ctx[i:j]
        shared.append(0 if j - i == 1 else int(min(run * block_size, members.min())))
        starts.append(j)
        i = j
    return np.asarray(starts, dtype=np.int32), np.asarray(shared, dtype=np.int32)


def decode_order(context_lens, tables=None) -> np.ndarray:
    """Dispatch order for decode (``pa_decode_shape.dispatch_order``): the
    sequences by context length, longest first, ties in batch order. int32 [S].

    With the batch's block ``tables``, sequences whose rows start with the
    same frame (the branches of one prompt, "PagedAttention: Virtual Memory
    Guide for LLM Inference", "2. Zero-Copy Branching via Copy-on-Write")
    form a family that stays together: families by their longest member,
    longest first (ties: the family whose first member comes first in the
    batch), members longest first, then in batch order. Branches dispatched
    together read their shared frames close in time, so the repeats hit in
    cache (with ``PA_CACHE_REUSE``); sorted by length alone they drift apart.
    Without shared first frames this is the plain length order."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    S = len(ctx)
    if tables is None or S == 0:
        return np.argsort(-ctx, kind="stable").astype(np.int32)
    tables = np.asarray(tables)
    idx = np.arange(S, dtype=np.int64)
    # family key: the first frame; a sequence with no token is its own family
    key = np.where(ctx > 0, tables[:, 0].astype(np.int64), -1 - idx)
    _, fam = np.unique(key, return_inverse=True)
    fam_len = np.zeros(fam.max() + 1, dtype=np.int64)
    np.maximum.at(fam_len, fam, ctx)
    fam_first = np.full(fam.max() + 1, S, dtype=np.int64)
    np.minimum.at(fam_first, fam, idx)
    # np.lexsort sorts by the last key first
    return np.lexsort((idx, -ctx, fam_first[fam], -fam_len[fam])).astype(np.int32)


def group_order(group_start, group_shared, context_lens) -> np.ndarray:
    """Dispatch order for ``paged_attn_decode_grouped``: groups by the rows
    their workgroups read (the shared tokens once, then each member's own),
    most first. int32 [G]."""
    gs = np.asarray(group_start, dtype=np.int64)
    sh = np.asarray(group_shared, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    work = np.array([sh[g] + np.sum(np.maximum(ctx[gs[g]:gs[g + 1]] - sh[g], 0))
                     for g in range(len(sh))], dtype=np.int64)
    return np.argsort(-work, kind="stable").astype(np.int32)


def prefill_order(context_lens, query_start, max_query_len=None) -> np.ndarray:
    """Dispatch order for ``paged_attn_prefill``'s work items (query tile t
    of sequence s is item s * Tq + t, Tq = ceil(max_query_len /
    PA_PREFILL_TILE)): sequences by the number of (query, key) pairs their
    queries see, most first, ties in batch order; within a sequence its
    later tiles, which see more keys, first. A longest-first schedule leaves
    the shortest work for the launch's tail, and a sequence's tiles stay
    together, so the keys they share are still in cache when the next tile
    reads them (measured: sorting all tiles by cost instead, across
    sequences, was slower). ``max_query_len`` must be the value the call is
    made with (default: the largest query count). int32 [S * Tq]."""
    from .lib import PA_PREFILL_TILE

    ctx = np.asarray(context_lens, dtype=np.int64)
    n = np.clip(np.diff(np.asarray(query_start, dtype=np.int64)), 0, ctx)
    mq = int(n.max(initial=0)) if max_query_len is None else int(max_query_len)
    n = np.minimum(n, mq)
    tq = max(1, -(-mq // PA_PREFILL_TILE))
    pairs = n * (ctx - n) + n * (n + 1) // 2
    seqs = np.argsort(-pairs, kind="stable")
    return (seqs[:, None] * tq + np.arange(tq - 1, -1, -1)[None, :]).reshape(-1).astype(np.int32)


class DeviceCache:
    """K and V caches [NB, B, H, D] in device memory, optionally NaN-filled."""

    def __init__(self, NB: int, B: int, H: int, D: int, dtype, device="cuda", poison: bool = True):
        import torch

        self.k = torch.empty((NB, B, H, D), dtype=dtype, device=device)
        self.v = torch.empty_like(self.k)
        if poison:
            self.k.fill_(float("nan"))
            self.v.fill_(float("nan"))
        self.B = B

    def append(self, k_new, v_new, slots, stream=None) -> None:
        from .lib import kv_append

        kv_append(k_new, v_new, slots, self.k, self.v, stream=stream)

    def copy_blocks(self, pairs, stream=None) -> None:
        from .lib import kv_copy_blocks

        kv_copy_blocks(self.k, self.v, pairs, stream=stream)


def execute(events, cache: DeviceCache, rows, on_attend, chunk_rows: int = 1 << 16) -> None:
    """Apply the events on the device.

    ``rows(seqs, positions)`` returns device tensors (k_new, v_new) [N, H, D]
    for those tokens; ``on_attend(point)`` is called at each AttendPoint once
    every earlier write has been queued. Large write batches are applied in
    chunks of ``chunk_rows`` tokens.
    """
    import torch

    dev = cache.k.device
    for ev in events:
        if isinstance(ev, CopyBlocks):
            cache.copy_blocks(torch.from_numpy(np.ascontiguousarray(ev.pairs)).to(dev))
        elif isinstance(ev, WriteBatch):
            for lo in range(0, len(ev.slots), chunk_rows):
                hi = min(lo + chunk_rows, len(ev.slots))
                k_new, v_new = rows(ev.seqs[lo:hi], ev.positions[lo:hi])
                sl = torch.from_numpy(np.ascontiguousarray(ev.slots[lo:hi])).to(dev)
                cache.append(k_new, v_new, sl)
        else:
            on_attend(ev)


@dataclass
class DecodeStep:
    """One decode step of a round: one generated token per listed request."""
    writes: WriteBatch        # the step's K/V rows (one per request)
    tables: np.ndarray        # int32 [len(seqs), max_blocks] after the appends
    context_lens: np.ndarray  # int32 [len(seqs)]


@dataclass
class PrefillRound:
    """One round of requests of a prefix-sharing workload, planned on the host."""
    seqs: list                # request (conversation) ids, in arrival order
    writes: WriteBatch        # the K/V rows the round must write: every position not reused
    tables: np.ndarray        # int32 [S, max_blocks]
    context_lens: np.ndarray  # int32 [S]: prompt lengths
    query_start: np.ndarray   # int32 [S + 1]: queries are the written positions, per request
    reused: np.ndarray        # int64 [S]: leading prompt tokens found in the cache
    decode: list = None       # DecodeStep per decode step after the prefill


def plan_prefix_rounds(w, caching: bool = True, pad: int = -1, pool_frames: int | None = None):
    """Host-only replay of a prefix-sharing workload (``w.rounds``,
    ``w.requests(r)`` -> [(id, prompt_len)], ``w.tokens(id, positions)``).

    With ``caching`` each request reuses the cached frames of its leading full
    blocks and writes (and queries) only the rest; without it every request
    takes fresh frames for its whole prompt. Requests of a round end before
    the next round. ``pool_frames`` replaces the workload's pool by one of
    that many frames in id order (a run without caching needs more).
    Returns (rounds, manager)."""
    if pool_frames is None:
        mgr = make_manager(w.NB, w.B, w.frame_order, caching)
    else:
        mgr = make_manager(pool_frames, w.B, None, caching)
    out = []
    for r in range(w.rounds):
        reqs = w.requests(r)
        seqs, poss, slots, reused = [], [], [], []
        for c, n in reqs:
            if caching:
                pos, sl = mgr.init_sequence_tokens(c, w.tokens(c, np.arange(n)))
            else:
                sl = mgr.init_sequence(c, n)
                pos = np.arange(n, dtype=np.int64)
            seqs.append(np.full(len(pos), c, dtype=np.int64))
            poss.append(pos)
            slots.append(np.asarray(sl, dtype=np.int64))
            reused.append(n - len(pos))
        ids = [c for c, _ in reqs]
        counts = np.array([len(p) for p in poss], dtype=np.int64)
        qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        rd = PrefillRound(ids, WriteBatch(np.concatenate(seqs), np.concatenate(poss),
                                          np.concatenate(slots)),
                          mgr.tables(ids, pad), mgr.context_lens(ids), qs,
                          np.array(reused, dtype=np.int64), [])
        for step in (w.decode_steps(r) if hasattr(w, "decode_steps") else []):
            pos = mgr.context_lens(step).astype(np.int64)
            toks = np.array([int(w.tokens(c, [p])[0]) for c, p in zip(step, pos)], dtype=np.int64)
            sl, _ = mgr.append_tokens(step, toks if caching else None)
            rd.decode.append(DecodeStep(WriteBatch(np.asarray(step, dtype=np.int64), pos, sl),
                                        mgr.tables(step, pad), mgr.context_lens(step)))
        out.append(rd)
        for c in ids:
            mgr.free_sequence(c)
    return out, mgr
