"""The oracle's prefix cache over the frame pool (test infrastructure only).

Restates the reuse that "PagedAttention: Virtual Memory Guide for LLM
Inference" describes in "2. Native Synergy with RadixAttention and Prompt
Caching" (a filled block never changes, so an identical prefix can map to the
frames already holding it) and that "Solving the LLM Memory Wall" states in
its algorithmic step 5 (sequences sharing a prefix point at the same physical
block; a finished request returns its blocks to the pool).

The pages give no keying, lookup or eviction rule; the readings taken here:

* A cached frame is known by the whole token prefix it completes: the tuple
  of every token id from position 0 through the last position of its block.
  Two full blocks are interchangeable exactly when these tuples are equal
  (same tokens at the same positions after the same history). This is the
  plain definition, with no hashing.
* A new request reuses the longest run of its leading full blocks whose
  prefixes are cached; the first miss ends the run. Its partial last block
  is never shared.
* A block enters the cache when it fills: for a prompt, at request start,
  for every full block not reused; for a generated token, when it completes
  the block. If an equal prefix is cached already, nothing changes.
* The cache holds one reference on each frame it keeps. A frame whose only
  reference is the cache's stays cached after its request ends.
* Every cache entry and every reuse is an event with a rising counter; a
  request's reuses come first, in block order, then its new entries in
  block order. When the free list is empty, the cached frame that only the
  cache references and whose latest event is oldest leaves the cache and
  returns to the pool; allocation then proceeds first-in first-out.
* A request whose frames cannot all be found (free plus evictable, not
  counting the frames it reuses) fails with nothing changed.
* A branch (fork) starts with its parent's frames, tokens and length, each
  frame gaining a user, as in :mod:`oracle.blockmgr`. A token appended into a
  partial last frame that has other users first moves the writer to a
  private copy of it (the copy's frame is found like any other, evicting if
  it must); a block filled by an appended token enters the cache.

The cache contents are modelled as the identity written to each slot (-1 for
never written), as in :mod:`oracle.blockmgr`.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from oracle.blockmgr import new_paging, release, share, take


class PrefixCache:
    """Block tables over a FIFO pool, with reuse of cached full-block prefixes."""

    def __init__(self, num_blocks: int, block_size: int, order=None, enabled: bool = True):
        self.pg = new_paging(num_blocks, block_size, order)
        self.B = block_size
        self.enabled = enabled            # off: plain demand paging, nothing cached
        self.frame_of_prefix: dict = {}   # token prefix tuple -> frame
        self.prefix_of_frame: dict = {}   # frame -> token prefix tuple
        self.last_event: dict = {}        # frame -> counter value of its latest event
        self.clock = 0
        self.tables: dict = {}
        self.tokens: dict = {}
        self.evicted: list = []

    def _event(self, frame: int) -> None:
        self.clock += 1
        self.last_event[frame] = self.clock

    def _evictable(self) -> list:
        return [f for f in self.prefix_of_frame if self.pg.users[f] == 1]

    def _take_frame(self) -> int:
        if not self.pg.free:
            candidates = self._evictable()
            if not candidates:
                raise MemoryError("no free frame and no evictable cached frame")
            victim = candidates[0]
            for f in candidates[1:]:
                if self.last_event[f] < self.last_event[victim]:
                    victim = f
            del self.frame_of_prefix[self.prefix_of_frame.pop(victim)]
            del self.last_event[victim]
            release(self.pg, victim)
            self.evicted.append(victim)
        return take(self.pg)

    def _enter(self, sid, b: int) -> None:
        prefix = tuple(self.tokens[sid][:(b + 1) * self.B])
        if not self.enabled or prefix in self.frame_of_prefix:
            return
        frame = self.tables[sid][b]
        self.frame_of_prefix[prefix] = frame
        self.prefix_of_frame[frame] = prefix
        share(self.pg, frame)
        self._event(frame)

    def start_request(self, sid, token_ids) -> int:
        """Open request ``sid``; returns how many leading tokens were reused."""
        toks = [int(t) for t in token_ids]
        B = self.B
        reused = []
        for b in range(len(toks) // B if self.enabled else 0):
            f = self.frame_of_prefix.get(tuple(toks[:(b + 1) * B]))
            if f is None:
                break
            reused.append(f)
        fresh = (len(toks) + B - 1) // B - len(reused)
        evictable = [f for f in self._evictable() if f not in reused]
        if fresh > len(self.pg.free) + len(evictable):
            raise MemoryError("frame pool exhausted")
        for f in reused:
            share(self.pg, f)
            self._event(f)
        table = list(reused)
        for _ in range(fresh):
            table.append(self._take_frame())
        self.tables[sid] = table
        self.tokens[sid] = toks
        for b in range(len(reused), len(toks) // B):
            self._enter(sid, b)
        return len(reused) * B

    def append(self, sid, token_id):
        """One generated token. Returns (slot, (shared frame, private copy))
        when the token's frame was copied first, else (slot, None)."""
        t = len(self.tokens[sid])
        row = self.tables[sid]
        copied = None
        if t % self.B == 0:
            row.append(self._take_frame())
        elif self.pg.users[row[-1]] > 1:
            mine = self._take_frame()
            copied = (row[-1], mine)
            release(self.pg, row[-1])
            row[-1] = mine
        self.tokens[sid].append(int(token_id))
        if (t + 1) % self.B == 0:
            self._enter(sid, t // self.B)
        return row[t // self.B] * self.B + t % self.B, copied

    def fork(self, parent, child) -> None:
        """``child`` starts with ``parent``'s frames and tokens."""
        for f in self.tables[parent]:
            share(self.pg, f)
        self.tables[child] = list(self.tables[parent])
        self.tokens[child] = list(self.tokens[parent])

    def end_request(self, sid) -> None:
        for f in self.tables.pop(sid):
            release(self.pg, f)
        del self.tokens[sid]

    def slots(self, sid, positions) -> np.ndarray:
        table = np.asarray(self.tables[sid], dtype=np.int64)
        pos = np.asarray(positions, dtype=np.int64)
        return table[pos // self.B] * self.B + pos % self.B


@dataclass
class DecodePoint:
    seqs: list                # conversations that appended a token in this step, in order
    tables: np.ndarray        # int32 [len(seqs), max_blocks] after the step
    context_lens: np.ndarray  # int32 [len(seqs)]: lengths after the step


@dataclass
class Round:
    seqs: list                # conversations of the round, in arrival order
    tables: np.ndarray        # int32 [S, max_blocks], padded (after the prefill)
    context_lens: np.ndarray  # int32 [S]: prompt lengths
    reused: np.ndarray        # int64 [S]: leading tokens found in the cache
    slot_ident: np.ndarray    # int64 [NB * B]: identity in each slot after the round's writes
    free_list: list           # after the round's requests ended
    decode: list              # DecodePoint per decode step of the round


def replay_rounds(w, pad_frame: int = -1, caching: bool = True, pool_frames: int | None = None):
    """Play a :class:`workloads.configs.PrefixWorkload`; one Round per round.

    Each request writes the identities of its positions from ``reused`` on;
    with ``caching`` off nothing is reused and every request writes its
    whole prompt. Then the round's decode steps append one generated token
    per listed request (its token id is the next position's). Attention at
    a decode step only reads positions written by then, and a frame is
    reallocated within a round only after eviction, when no request of the
    round references it; so one snapshot of the slots after the round serves
    every attention point of the round. ``pool_frames`` replaces the
    workload's pool by one of that many frames in id order."""
    if pool_frames is None:
        pc = PrefixCache(w.NB, w.B, w.frame_order, enabled=caching)
    else:
        pc = PrefixCache(pool_frames, w.B, None, enabled=caching)
    slot_ident = np.full(pc.pg.num_frames * w.B, -1, dtype=np.int64)
    rounds = []
    for r in range(w.rounds):
        reqs = w.requests(r)
        reused = []
        for c, n in reqs:
            k = pc.start_request(c, w.tokens(c, np.arange(n)))
            reused.append(k)
            pos = np.arange(k, n)
            slot_ident[pc.slots(c, pos)] = w.idents(c, pos)
        def table_of(seqs):
            mb = max(1, max(len(pc.tables[c]) for c in seqs))
            t = np.full((len(seqs), mb), pad_frame, dtype=np.int32)
            for i, c in enumerate(seqs):
                t[i, :len(pc.tables[c])] = pc.tables[c]
            return t

        seqs = [c for c, _ in reqs]
        tables = table_of(seqs)
        decode = []
        for step in w.decode_steps(r):
            for c in step:
                pos = len(pc.tokens[c])
                slot, _ = pc.append(c, int(w.tokens(c, [pos])[0]))
                slot_ident[slot] = w.idents(c, [pos])[0]
            decode.append(DecodePoint(list(step), table_of(step),
                                      np.array([len(pc.tokens[c]) for c in step], dtype=np.int32)))
        for c in seqs:
            pc.end_request(c)
        rounds.append(Round(seqs, tables, np.array([n for _, n in reqs], dtype=np.int32),
                            np.array(reused, dtype=np.int64), slot_ident.copy(),
                            list(pc.pg.free), decode))
    return rounds, pc
