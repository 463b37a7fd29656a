"""The oracle's block manager and schedule replay (test infrastructure only).

A direct restatement of the memory manager described on "PagedAttention:
Virtual Memory Guide for LLM Inference" (sections "1. Demand Paging during
Autoregressive Decoding", "2. Zero-Copy Branching via Copy-on-Write" and
"Reference Implementation: Block Table & Paged Cache Manager"), checked
against the worked allocation example of "PagedAttention, simply explained"
(section "How PagedAttention solves it").

Rules as the pages state them:

* the pool's free list is first-in first-out: allocation takes the head,
  a frame whose reference count drops to zero goes to the tail;
* a prompt of L tokens takes ceil(L / B) frames at once;
* appending token t (t = tokens already held) takes a new frame exactly when
  t mod B == 0, else writes into the last frame at offset t mod B;
* forking copies the table and adds one reference to every frame in it;
* appending into a shared (reference count > 1) partial last frame first
  copies that frame to a newly allocated one (copy-on-write) and drops one
  reference on the old frame.

Readings where the pages leave a step open:

* t = 0 (an empty sequence) takes the new-frame branch, since 0 mod B == 0;
  the page's listing would read the last table entry of an empty table first.
* The cache is modelled as the *identity* of the token written to each slot
  (``frame * B + offset``), with -1 for a slot never written. A copy-on-write
  copies the whole frame's identities, which is what a byte copy of the
  frame does to its contents.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


class PhysicalBlockPool:
    """Free frames in FIFO order plus a reference count per frame."""

    def __init__(self, num_blocks: int, order=None):
        self.num_blocks = num_blocks
        self.free_blocks = list(range(num_blocks)) if order is None else [int(f) for f in order]
        assert sorted(self.free_blocks) == list(range(num_blocks))
        self.ref_counts = {i: 0 for i in range(num_blocks)}

    def allocate(self) -> int:
        if not self.free_blocks:
            raise MemoryError("frame pool exhausted")
        block_id = self.free_blocks.pop(0)
        self.ref_counts[block_id] = 1
        return block_id

    def add_reference(self, block_id: int) -> None:
        self.ref_counts[block_id] += 1

    def free(self, block_id: int) -> None:
        if self.ref_counts[block_id] <= 0:
            return
        self.ref_counts[block_id] -= 1
        if self.ref_counts[block_id] == 0:
            self.free_blocks.append(block_id)

    @property
    def free_count(self) -> int:
        return len(self.free_blocks)


class SequenceGroupMemoryManager:
    """Block tables and lengths per request; demand paging, fork and CoW."""

    def __init__(self, pool: PhysicalBlockPool, block_size: int):
        self.pool = pool
        self.block_size = block_size
        self.block_tables: dict = {}
        self.seq_lens: dict = {}

    def init_sequence(self, request_id, prompt_tokens: int) -> None:
        n = math.ceil(prompt_tokens / self.block_size)
        self.block_tables[request_id] = [self.pool.allocate() for _ in range(n)]
        self.seq_lens[request_id] = prompt_tokens

    def append_token(self, request_id):
        """Returns (old_frame, new_frame) when a copy-on-write happened, else None."""
        cur_len = self.seq_lens[request_id]
        table = self.block_tables[request_id]
        copied = None
        if cur_len % self.block_size == 0:
            table.append(self.pool.allocate())
        else:
            cur_block_id = table[-1]
            if self.pool.ref_counts[cur_block_id] > 1:
                new_block_id = self.pool.allocate()
                self.pool.free(cur_block_id)
                table[-1] = new_block_id
                copied = (cur_block_id, new_block_id)
        self.seq_lens[request_id] = cur_len + 1
        return copied

    def fork_sequence(self, parent_id, child_id) -> None:
        parent_table = self.block_tables[parent_id]
        for b_id in parent_table:
            self.pool.add_reference(b_id)
        self.block_tables[child_id] = list(parent_table)
        self.seq_lens[child_id] = self.seq_lens[parent_id]

    def free_sequence(self, request_id) -> None:
        if request_id in self.block_tables:
            for b_id in self.block_tables[request_id]:
                self.pool.free(b_id)
            del self.block_tables[request_id]
            del self.seq_lens[request_id]


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
    """Play a workload schedule; one Snapshot per attention point.

    ``w`` is a :class:`workloads.configs.Workload`. Sequences are prefilled in
    schedule order, forked, then each decode step appends one token to each
    listed sequence in the listed order.
    """
    pool = PhysicalBlockPool(w.NB, w.frame_order)
    mgr = SequenceGroupMemoryManager(pool, w.B)
    B = w.B
    slot_ident = np.full(w.NB * B, -1, dtype=np.int64)

    def slots_of(s, positions):
        table = np.asarray(mgr.block_tables[s], dtype=np.int64)
        positions = np.asarray(positions, dtype=np.int64)
        return table[positions // B] * B + positions % B

    for s, n in w.prefill:
        mgr.init_sequence(s, n)
        if n:
            pos = np.arange(n)
            slot_ident[slots_of(s, pos)] = w.idents(s, pos)
    for parent, child in w.forks:
        mgr.fork_sequence(parent, child)

    snaps = []

    def snap():
        S = w.num_seqs
        lens = np.array([mgr.seq_lens[s] for s in range(S)], dtype=np.int32)
        mb = max_blocks or max(1, max(len(mgr.block_tables[s]) for s in range(S)))
        tables = np.full((S, mb), pad_frame, dtype=np.int32)
        for s in range(S):
            t = mgr.block_tables[s]
            tables[s, :len(t)] = t
        snaps.append(Snapshot(tables, lens, slot_ident.copy(), list(pool.free_blocks)))

    if -1 in w.attend_after:
        snap()
    for k, seqs in enumerate(w.steps):
        for s in seqs:
            t = mgr.seq_lens[s]
            copied = mgr.append_token(s)
            if copied is not None:
                old, new = copied
                slot_ident[new * B:(new + 1) * B] = slot_ident[old * B:(old + 1) * B]
            slot_ident[slots_of(s, [t])] = w.idents(s, [t])
        if k in w.attend_after:
            snap()
    return snaps, mgr, pool
