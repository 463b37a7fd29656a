"""Host-side block manager: frame pool, block tables and slot mapping.

This is the control plane the kernels are fed by. It follows the memory
manager described on "PagedAttention: Virtual Memory Guide for LLM
Inference" (sections "1. Demand Paging during Autoregressive Decoding",
"2. Zero-Copy Branching via Copy-on-Write" and "Reference Implementation:
Block Table & Paged Cache Manager") and the worked example of
"PagedAttention, simply explained":

* free frames are handed out first-in first-out; a frame whose reference
  count falls to zero rejoins the tail of the free list;
* a prompt of L tokens takes ceil(L / B) frames at once;
* token t of a sequence (t = tokens it already holds) goes to offset t mod B
  of its last frame; a new frame is taken exactly when t mod B == 0 (this
  includes t = 0, the first token of an empty sequence);
* fork shares every frame of the parent and adds one reference to each;
* appending into a shared partial last frame first moves the sequence to a
  private copy of that frame (copy-on-write): the caller copies the frame's
  first t mod B rows on the device, then writes the new token.

Slots are ``frame * B + offset``; with caches laid out [NB, B, H, D] a slot is
the row index of the cache viewed as [NB * B, H, D].
"""
from __future__ import annotations

import hashlib
from collections import deque
from dataclasses import dataclass

import numpy as np


class BlockPool:
    """Physical frames: FIFO free list plus a reference count per frame."""

    def __init__(self, num_frames: int, order=None):
        if num_frames <= 0:
            raise ValueError("num_frames must be positive")
        self.num_frames = int(num_frames)
        if order is None:
            self._free = deque(range(self.num_frames))
        else:
            order = [int(f) for f in order]
            if sorted(order) != list(range(self.num_frames)):
                raise ValueError("order must be a permutation of the frame ids")
            self._free = deque(order)
        self.ref = np.zeros(self.num_frames, dtype=np.int64)

    @property
    def free_count(self) -> int:
        return len(self._free)

    def free_list(self) -> list:
        return list(self._free)

    def allocate(self) -> int:
        if not self._free:
            raise MemoryError("frame pool exhausted")
        f = self._free.popleft()
        self.ref[f] = 1
        return f

    def allocate_many(self, n: int) -> list:
        """n frames in FIFO order, or MemoryError with nothing taken."""
        if n > len(self._free):
            raise MemoryError(f"frame pool exhausted: need {n}, have {len(self._free)}")
        out = [self._free.popleft() for _ in range(n)]
        self.ref[out] = 1
        return out

    def add_ref(self, frame: int) -> None:
        self.ref[frame] += 1

    def free(self, frame: int) -> None:
        """Drop one reference; a frame reaching zero goes to the free tail.
        Freeing a frame that holds no reference does nothing."""
        if self.ref[frame] <= 0:
            return
        self.ref[frame] -= 1
        if self.ref[frame] == 0:
            self._free.append(frame)


@dataclass(frozen=True)
class AppendResult:
    slot: int                    # where the new token's K/V rows go
    cow_src: int | None = None   # frame to copy from (copy-on-write), or None
    cow_dst: int | None = None   # the sequence's new private frame
    cow_rows: int = 0            # rows of cow_src to copy (offsets 0 .. cow_rows - 1)


class SeqManager:
    """Per-sequence block tables and lengths over one BlockPool."""

    def __init__(self, pool: BlockPool, block_size: int):
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self.pool = pool
        self.B = int(block_size)
        self._tables: dict = {}
        self._lens: dict = {}

    # ------------------------------------------------------------ lifecycle
    def _allocate(self) -> int:
        return self.pool.allocate()

    def init_sequence(self, sid, n_tokens: int) -> np.ndarray:
        """Allocate ceil(n_tokens / B) frames; return the n_tokens slots."""
        if sid in self._tables:
            raise KeyError(f"sequence {sid!r} exists")
        n_tokens = int(n_tokens)
        frames = self.pool.allocate_many(-(-n_tokens // self.B))
        self._tables[sid] = frames
        self._lens[sid] = n_tokens
        return self.slots(sid, np.arange(n_tokens))

    def append_token(self, sid) -> AppendResult:
        t = self._lens[sid]
        table = self._tables[sid]
        off = t % self.B
        cow = (None, None, 0)
        if off == 0:
            table.append(self._allocate())
        else:
            last = table[-1]
            if self.pool.ref[last] > 1:
                new = self._allocate()
                self.pool.free(last)
                table[-1] = new
                cow = (last, new, off)
        self._lens[sid] = t + 1
        return AppendResult(table[-1] * self.B + off, *cow)

    def append_tokens(self, sids, token_ids=None):
        """Append one token to each listed sequence, in order. Returns
        (slots int64 [n], cow int64 [n, 3]: source frame, new frame, rows
        to copy, or -1, -1, 0)."""
        sids = list(sids)
        slots = np.empty(len(sids), dtype=np.int64)
        cow = np.tile(np.array([-1, -1, 0], dtype=np.int64), (len(sids), 1))
        for i, sid in enumerate(sids):
            r = (self.append_token(sid) if token_ids is None
                 else self.append_token_id(sid, token_ids[i]))
            slots[i] = r.slot
            if r.cow_src is not None:
                cow[i] = (r.cow_src, r.cow_dst, r.cow_rows)
        return slots, cow

    @property
    def ref(self) -> np.ndarray:
        """Reference count of every frame."""
        return self.pool.ref

    def free_list(self) -> list:
        return self.pool.free_list()

    def fork(self, parent, child) -> None:
        if child in self._tables:
            raise KeyError(f"sequence {child!r} exists")
        table = self._tables[parent]
        for f in table:
            self.pool.add_ref(f)
        self._tables[child] = list(table)
        self._lens[child] = self._lens[parent]

    def free_sequence(self, sid) -> None:
        """Release a finished sequence's frames; unknown ids are ignored."""
        table = self._tables.pop(sid, None)
        if table is None:
            return
        del self._lens[sid]
        for f in table:
            self.pool.free(f)

    # ------------------------------------------------------------ queries
    def block_table(self, sid) -> list:
        return list(self._tables[sid])

    def context_len(self, sid) -> int:
        return self._lens[sid]

    def slots(self, sid, positions) -> np.ndarray:
        """Slots (frame * B + offset) of token positions of a sequence."""
        pos = np.asarray(positions, dtype=np.int64)
        table = np.asarray(self._tables[sid], dtype=np.int64)
        return table[pos // self.B] * self.B + pos % self.B

    def tables(self, sids, pad: int, max_blocks: int | None = None) -> np.ndarray:
        """int32 [len(sids), max_blocks] block tables, unused columns = pad."""
        width = max((len(self._tables[s]) for s in sids), default=0)
        mb = max(1, width if max_blocks is None else max_blocks)
        if width > mb:
            raise ValueError("max_blocks smaller than the longest table")
        out = np.full((len(sids), mb), pad, dtype=np.int32)
        for r, s in enumerate(sids):
            t = self._tables[s]
            out[r, :len(t)] = t
        return out

    def context_lens(self, sids) -> np.ndarray:
        return np.array([self._lens[s] for s in sids], dtype=np.int32)

    def waste_slots(self, sid) -> int:
        """Allocated but unused slots of a sequence (< B by construction)."""
        return len(self._tables[sid]) * self.B - self._lens[sid]


def memory_efficiency(tokens: int, block_size: int) -> float:
    """Used share of the slots allocated for ``tokens`` tokens (page 2's
    "Performance Analysis" figure: B = 4 and 7 tokens give 7 / 8)."""
    frames = -(-int(tokens) // int(block_size))
    return tokens / (frames * block_size) if frames else 1.0


class PrefixCachingSeqManager(SeqManager):
    """SeqManager that reuses frames of identical full blocks across requests.

    "PagedAttention: Virtual Memory Guide for LLM Inference" ("2. Native
    Synergy with RadixAttention and Prompt Caching"): a block is immutable
    once filled, so a request whose prompt starts with the same tokens can
    point at the frames already holding them. "Solving the LLM Memory Wall"
    (algorithmic step 5): sequences sharing a prefix point to the same
    physical block.

    Policy:

    * A full block is keyed by a chain digest over its tokens and the digest
      of the block before it, so a key names the block's tokens together with
      every token in front of them.
    * The cache holds one reference on each frame it indexes. A block is
      indexed when it fills (at request start for a prompt's full blocks, or
      when an appended token completes it); a block whose key is already
      indexed keeps its own frame and the index is left as it was.
    * A new request reuses the longest run of leading full blocks whose keys
      are indexed, stopping at the first miss; the partial last block is
      never shared.
    * Each indexed frame has a last-use time: when it was indexed or last
      reused (one tick per event; a request's reuses in block order, then its
      new entries in block order). When the free list is empty, the indexed
      frame with the oldest last use among those referenced by the index
      alone is dropped from the index and freed, then allocation proceeds.
    * A request that cannot get all its frames takes none and changes
      nothing.
    """

    def __init__(self, pool: BlockPool, block_size: int):
        super().__init__(pool, block_size)
        self._index: dict = {}          # digest -> frame
        self._digest_of: dict = {}      # frame -> digest
        self._last_use: dict = {}       # frame -> tick, for indexed frames
        self._tick = 0
        self._tokens: dict = {}         # sid -> token ids held
        self._chain: dict = {}          # sid -> digests of its full blocks
        self.hit_blocks = 0
        self.miss_blocks = 0
        self.evictions = 0

    @staticmethod
    def _digest(prev: bytes, tokens) -> bytes:
        h = hashlib.blake2b(digest_size=16)
        h.update(prev)
        h.update(np.asarray(tokens, dtype=np.int64).tobytes())
        return h.digest()

    def _touch(self, frame: int) -> None:
        self._tick += 1
        self._last_use[frame] = self._tick

    def init_sequence(self, sid, n_tokens: int) -> np.ndarray:
        raise RuntimeError("a prefix-caching manager needs the prompt's token ids: "
                           "use init_sequence_tokens")

    def append_token(self, sid) -> AppendResult:
        raise RuntimeError("a prefix-caching manager needs each token's id: use append_token_id")

    def _idle(self) -> list:
        return [f for f in self._last_use if self.pool.ref[f] == 1]

    def _allocate(self) -> int:
        if self.pool.free_count == 0:
            idle = self._idle()
            if not idle:
                raise MemoryError("frame pool exhausted and every cached frame is in use")
            f = min(idle, key=self._last_use.__getitem__)
            del self._index[self._digest_of.pop(f)]
            del self._last_use[f]
            self.pool.free(f)
            self.evictions += 1
        return self.pool.allocate()

    def _register(self, sid, b: int) -> None:
        """Block b of sid has just filled: key it, and index it if new."""
        toks = self._tokens[sid][b * self.B:(b + 1) * self.B]
        chain = self._chain[sid]
        d = self._digest(chain[b - 1] if b > 0 else b"", toks)
        chain.append(d)
        if d not in self._index:
            frame = self._tables[sid][b]
            self._index[d] = frame
            self._digest_of[frame] = d
            self.pool.add_ref(frame)  # the index's own reference
            self._touch(frame)

    def init_sequence_tokens(self, sid, token_ids):
        """Start a request with prompt ``token_ids``. Returns (positions,
        slots) of the tokens whose K/V must be written: tokens of reused
        blocks are already in the cache."""
        if sid in self._tables:
            raise KeyError(f"sequence {sid!r} exists")
        toks = np.asarray(token_ids, dtype=np.int64).reshape(-1)
        n, B = len(toks), self.B
        hits, chain = [], []
        prev = b""
        for b in range(n // B):
            d = self._digest(prev, toks[b * B:(b + 1) * B])
            f = self._index.get(d)
            if f is None:
                break
            hits.append(f)
            chain.append(d)
            prev = d
        need = -(-n // B) - len(hits)
        spare = sum(1 for f in self._idle() if f not in hits)
        if need > self.pool.free_count + spare:
            raise MemoryError(f"frame pool exhausted: need {need}, can free "
                              f"{self.pool.free_count + spare}")
        for f in hits:
            self.pool.add_ref(f)
            self._touch(f)
        table = hits + [self._allocate() for _ in range(need)]
        self.hit_blocks += len(hits)
        self.miss_blocks += need
        self._tables[sid] = table
        self._lens[sid] = n
        self._tokens[sid] = [int(t) for t in toks]
        self._chain[sid] = chain
        for b in range(len(hits), n // B):
            self._register(sid, b)
        pos = np.arange(len(hits) * B, n, dtype=np.int64)
        return pos, self.slots(sid, pos)

    def append_token_id(self, sid, token_id) -> AppendResult:
        """Append one token; the block it completes is keyed and indexed."""
        t = self._lens[sid]
        r = SeqManager.append_token(self, sid)
        self._tokens[sid].append(int(token_id))
        if (t + 1) % self.B == 0:
            self._register(sid, t // self.B)
        return r

    def fork(self, parent, child) -> None:
        super().fork(parent, child)
        self._tokens[child] = list(self._tokens[parent])
        self._chain[child] = list(self._chain[parent])

    def free_sequence(self, sid) -> None:
        super().free_sequence(sid)
        self._tokens.pop(sid, None)
        self._chain.pop(sid, None)

    @property
    def cached_frames(self) -> int:
        return len(self._index)
