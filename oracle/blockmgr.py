"""The oracle's frame bookkeeping and schedule replay (test infrastructure only).

The state is one record, :class:`Paging`: the free frames, a user count per
frame, and per sequence its row of frames and its length. Plain functions
change it, one per rule. The rules, as the pages state them:

* Free frames leave from the front and return at the back (the pool of
  "PagedAttention: Virtual Memory Guide for LLM Inference", section
  "1. Demand Paging during Autoregressive Decoding"; the order is fixed by
  the worked example of "PagedAttention, simply explained", section "How
  PagedAttention solves it": prompts A, B, C, D take frames 0, 1, 2-3, 4 and
  the next frame handed out is 5, then 6).
* A prompt of L tokens holds ceil(L / B) frames (page 1, section 1; page 3's
  example, where 12 tokens at B = 10 take two frames).
* The token at position t (t = tokens the sequence already holds) goes to
  offset t mod B of the sequence's last frame; when t mod B == 0 there is no
  room and a new frame is appended first (page 1, section 1; page 3: D grows
  from 9 to 10 tokens in its first frame and takes frame 5 for the 11th).
* A branch starts with its parent's frames and length, and each of those
  frames gains a user (page 1, section "2. Zero-Copy Branching via
  Copy-on-Write").
* Writing into a frame that has other users first gives the writer a private
  frame holding a copy, and the shared frame loses that user (same section).
* A frame whose users drop to zero returns to the pool; finishing a sequence
  drops one user from each of its frames (page 1, section 1; "Solving the
  LLM Memory Wall", algorithmic step 5).

Readings where the pages leave a step open:

* t = 0 (an empty sequence) is the t mod B == 0 case: a new frame.
* A prompt that needs more frames than are free takes none and raises
  MemoryError (page 2's allocator checks the free count before taking).
* The cache contents are modelled as the *identity* of the token written to
  each slot (``frame * B + offset``), -1 for a slot never written. A
  copy-on-write copies the whole frame's identities, as a byte copy of the
  frame does to its contents.
"""
from __future__ import annotations

import collections
import math
from dataclasses import dataclass

import numpy as np


@dataclass
class Paging:
    """Frames and sequences of one pool."""

    block_size: int
    free: collections.deque  # free frame ids, next to hand out on the left
    users: np.ndarray        # int64 [num_frames]: how many table rows (or caches) use each frame
    table: dict              # sequence -> list of frame ids, logical block order
    length: dict             # sequence -> tokens held

    @property
    def num_frames(self) -> int:
        return len(self.users)


def new_paging(num_frames: int, block_size: int, order=None) -> Paging:
    """All frames free, handed out in ``order`` (default 0, 1, 2, ...)."""
    free = collections.deque(range(num_frames) if order is None else (int(f) for f in order))
    if sorted(free) != list(range(num_frames)):
        raise ValueError("order must be a permutation of the frame ids")
    return Paging(block_size, free, np.zeros(num_frames, dtype=np.int64), {}, {})


def frames_for(tokens: int, block_size: int) -> int:
    """Frames that hold ``tokens`` tokens: the ceiling of tokens / B."""
    return -(-tokens // block_size)


def take(pg: Paging) -> int:
    """The frame at the front of the free list, now with one user."""
    if not pg.free:
        raise MemoryError("no free frame")
    f = pg.free.popleft()
    pg.users[f] = 1
    return f


def share(pg: Paging, f: int) -> None:
    """One more user of frame ``f``."""
    pg.users[f] += 1


def release(pg: Paging, f: int) -> None:
    """One user fewer; a frame left with none goes to the back of the free
    list. A frame that has no user already is left as it is."""
    if pg.users[f] > 0:
        pg.users[f] -= 1
        if pg.users[f] == 0:
            pg.free.append(f)


def start(pg: Paging, seq, tokens: int) -> None:
    """Sequence ``seq`` with a prompt of ``tokens`` tokens."""
    n = frames_for(tokens, pg.block_size)
    if n > len(pg.free):
        raise MemoryError("not enough free frames for the prompt")
    pg.table[seq] = [take(pg) for _ in range(n)]
    pg.length[seq] = tokens


def extend(pg: Paging, seq):
    """Room for one more token of ``seq``. Returns (shared frame, private
    copy) when the token's frame had to be copied first, else None."""
    row = pg.table[seq]
    t = pg.length[seq]
    copied = None
    if t % pg.block_size == 0:
        row.append(take(pg))
    else:
        last = row[-1]
        if pg.users[last] > 1:
            row[-1] = take(pg)
            release(pg, last)
            copied = (last, row[-1])
    pg.length[seq] = t + 1
    return copied


def branch(pg: Paging, parent, child) -> None:
    """``child`` starts as a copy of ``parent``'s row and length."""
    for f in pg.table[parent]:
        share(pg, f)
    pg.table[child] = list(pg.table[parent])
    pg.length[child] = pg.length[parent]


def finish(pg: Paging, seq) -> None:
    """``seq`` ends; an unknown sequence is ignored."""
    row = pg.table.pop(seq, None)
    if row is None:
        return
    del pg.length[seq]
    for f in row:
        release(pg, f)


def slots_of(pg: Paging, seq, positions) -> np.ndarray:
    """Slot (frame * B + offset) of each position of ``seq``."""
    B = pg.block_size
    row = np.asarray(pg.table[seq], dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    return row[pos // B] * B + pos % B


def memory_efficiency(tokens: int, block_size: int) -> float:
    """Share of allocated slots that hold tokens (page 2, "Performance Analysis")."""
    frames = math.ceil(tokens / block_size)
    return tokens / (frames * block_size) if frames else 1.0


@dataclass
class Snapshot:
    tables: np.ndarray        # int32 [S, max_blocks], padded with pad_frame
    context_lens: np.ndarray  # int32 [S]
    slot_ident: np.ndarray    # int64 [NB * B]: identity written to each slot, -1 if none
    free_list: list


def replay(w, pad_frame: int = -1, max_blocks: int | None = None):
    """Play a workload schedule; returns (one Snapshot per attention point,
    the final Paging).

    ``w`` is a :class:`workloads.configs.Workload`. Sequences are prefilled in
    schedule order, branched, then each decode step appends one token to
    each listed sequence in the listed order.
    """
    pg = new_paging(w.NB, w.B, w.frame_order)
    B = w.B
    slot_ident = np.full(w.NB * B, -1, dtype=np.int64)

    for s, n in w.prefill:
        start(pg, s, n)
        if n:
            pos = np.arange(n)
            slot_ident[slots_of(pg, s, pos)] = w.idents(s, pos)
    for parent, child in w.forks:
        branch(pg, parent, child)

    snaps = []

    def snap():
        S = w.num_seqs
        lens = np.array([pg.length[s] for s in range(S)], dtype=np.int32)
        mb = max_blocks or max(1, max(len(pg.table[s]) for s in range(S)))
        tables = np.full((S, mb), pad_frame, dtype=np.int32)
        for s in range(S):
            row = pg.table[s]
            tables[s, :len(row)] = row
        snaps.append(Snapshot(tables, lens, slot_ident.copy(), list(pg.free)))

    if -1 in w.attend_after:
        snap()
    for k, seqs in enumerate(w.steps):
        for s in seqs:
            t = pg.length[s]
            copied = extend(pg, s)
            if copied is not None:
                src, dst = copied
                slot_ident[dst * B:(dst + 1) * B] = slot_ident[src * B:(src + 1) * B]
            slot_ident[slots_of(pg, s, [t])] = w.idents(s, [t])
        if k in w.attend_after:
            snap()
    return snaps, pg
