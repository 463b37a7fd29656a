"""ctypes binding of the host block manager (include/paged_blocks.h).

``NativeBlockManager`` is the frame pool and the sequences' block tables:
demand paging, fork with copy-on-write, and (with ``prefix_caching=True``)
reuse of cached full blocks across requests. Argument marshalling only: the
work happens in the library's C++ code (csrc/block_manager.cpp).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from .lib import load

PB_OK, PB_EINVAL, PB_ENOMEM, PB_ESTATE = 0, -1, -2, -3

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


@dataclass
class AppendResult:
    slot: int                    # where the new token's K/V rows go
    cow_src: int | None = None   # frame to copy from (copy-on-write), or None
    cow_dst: int | None = None   # the sequence's new private frame
    cow_rows: int = 0            # rows of cow_src to copy (offsets 0 .. cow_rows - 1)


class PbStats(ctypes.Structure):
    _fields_ = [("free_frames", _I64), ("cached_frames", _I64), ("hit_blocks", _I64),
                ("miss_blocks", _I64), ("evictions", _I64), ("sequences", _I64)]


_BOUND = None


def _lib():
    global _BOUND
    if _BOUND is None:
        L = load()
        L.pb_create.argtypes = [_I64, _I32, _P, _I32, ctypes.POINTER(_P)]
        L.pb_destroy.argtypes = [_P]
        L.pb_destroy.restype = None
        L.pb_init_sequence.argtypes = [_P, _I64, _I64, _P]
        L.pb_init_sequence_tokens.argtypes = [_P, _I64, _P, _I64, _P, _P]
        L.pb_append_tokens.argtypes = [_P, _P, _P, _I64, _P, _P, _P]
        L.pb_fork.argtypes = [_P, _I64, _I64]
        L.pb_free_sequence.argtypes = [_P, _I64]
        L.pb_block_tables.argtypes = [_P, _P, _I64, _I32, _I32, _P, _P]
        L.pb_table_length.argtypes = [_P, _I64, _P]
        L.pb_free_list.argtypes = [_P, _P, _I64, _P]
        L.pb_ref_counts.argtypes = [_P, _P]
        L.pb_get_stats.argtypes = [_P, ctypes.POINTER(PbStats)]
        for f in ("pb_create", "pb_init_sequence", "pb_init_sequence_tokens", "pb_append_tokens",
                  "pb_fork", "pb_free_sequence", "pb_block_tables", "pb_table_length",
                  "pb_free_list", "pb_ref_counts", "pb_get_stats"):
            getattr(L, f).restype = ctypes.c_int
        _BOUND = L
    return _BOUND


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(fn: str, rc: int):
    if rc == PB_OK:
        return
    if rc == PB_ENOMEM:
        raise MemoryError(f"{fn}: frame pool exhausted")
    if rc == PB_ESTATE:
        raise RuntimeError(f"{fn}: not available on this manager")
    raise ValueError(f"{fn}: invalid argument")


class NativeBlockManager:
    """Frame pool + sequences, in the C++ library. See include/paged_blocks.h."""

    def __init__(self, num_frames: int, block_size: int, order=None, prefix_caching: bool = False):
        L = _lib()
        self.B = int(block_size)
        self.num_frames = int(num_frames)
        self.prefix_caching = bool(prefix_caching)
        o = None if order is None else np.ascontiguousarray(order, dtype=np.int32)
        h = _P()
        _check("pb_create", L.pb_create(self.num_frames, self.B, None if o is None else _ptr(o),
                                        int(self.prefix_caching), ctypes.byref(h)))
        self._h = h
        self._L = L

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._L.pb_destroy(h)
            self._h = None

    # ------------------------------------------------------------ lifecycle
    def init_sequence(self, sid, n_tokens: int) -> np.ndarray:
        slots = np.empty(int(n_tokens), dtype=np.int64)
        _check("pb_init_sequence", self._L.pb_init_sequence(self._h, int(sid), int(n_tokens),
                                                            _ptr(slots)))
        return slots

    def init_sequence_tokens(self, sid, token_ids):
        """(positions, slots) of the prompt positions to write (from the
        first one not reused)."""
        toks = np.ascontiguousarray(token_ids, dtype=np.int64).reshape(-1)
        slots = np.empty(len(toks), dtype=np.int64)
        reused = _I64(0)
        _check("pb_init_sequence_tokens",
               self._L.pb_init_sequence_tokens(self._h, int(sid), _ptr(toks), len(toks),
                                               ctypes.byref(reused), _ptr(slots)))
        k = int(reused.value)
        return np.arange(k, len(toks), dtype=np.int64), slots[k:]

    def append_tokens(self, sids, token_ids=None):
        """Append one token to each listed sequence, in order. Returns
        (slots int64 [n], cow int64 [n, 3]: source frame, new frame, rows)."""
        s = np.ascontiguousarray(sids, dtype=np.int64).reshape(-1)
        t = None if token_ids is None else np.ascontiguousarray(token_ids, dtype=np.int64).reshape(-1)
        slots = np.empty(len(s), dtype=np.int64)
        cow = np.empty((len(s), 3), dtype=np.int64)
        done = _I64(0)
        _check("pb_append_tokens",
               self._L.pb_append_tokens(self._h, _ptr(s), None if t is None else _ptr(t), len(s),
                                        _ptr(slots), _ptr(cow), ctypes.byref(done)))
        return slots, cow

    def _one(self, sid, token_id):
        slots, cow = self.append_tokens([sid], None if token_id is None else [token_id])
        src, dst, rows = (int(x) for x in cow[0])
        return AppendResult(int(slots[0]), None if src < 0 else src, None if src < 0 else dst, rows)

    def append_token(self, sid) -> AppendResult:
        return self._one(sid, None)

    def append_token_id(self, sid, token_id) -> AppendResult:
        return self._one(sid, int(token_id))

    def fork(self, parent, child) -> None:
        _check("pb_fork", self._L.pb_fork(self._h, int(parent), int(child)))

    def free_sequence(self, sid) -> None:
        _check("pb_free_sequence", self._L.pb_free_sequence(self._h, int(sid)))

    # ------------------------------------------------------------ queries
    def _table_len(self, sid) -> int:
        n = _I64(0)
        _check("pb_table_length", self._L.pb_table_length(self._h, int(sid), ctypes.byref(n)))
        return int(n.value)

    def tables(self, sids, pad: int, max_blocks: int | None = None) -> np.ndarray:
        s = np.ascontiguousarray(list(sids), dtype=np.int64)
        width = max((self._table_len(x) for x in s), default=0)
        mb = max(1, width if max_blocks is None else int(max_blocks))
        if width > mb:
            raise ValueError("max_blocks smaller than the longest table")
        out = np.empty((len(s), mb), dtype=np.int32)
        _check("pb_block_tables", self._L.pb_block_tables(self._h, _ptr(s), len(s), int(pad), mb,
                                                          _ptr(out), None))
        return out

    def context_lens(self, sids) -> np.ndarray:
        s = np.ascontiguousarray(list(sids), dtype=np.int64)
        width = max(1, max((self._table_len(x) for x in s), default=1))
        tab = np.empty((len(s), width), dtype=np.int32)
        lens = np.empty(len(s), dtype=np.int32)
        _check("pb_block_tables", self._L.pb_block_tables(self._h, _ptr(s), len(s), -1, width,
                                                          _ptr(tab), _ptr(lens)))
        return lens

    def block_table(self, sid) -> list:
        n = self._table_len(sid)
        return [int(f) for f in self.tables([sid], -1, max(1, n))[0, :n]]

    def context_len(self, sid) -> int:
        return int(self.context_lens([sid])[0])

    def slots(self, sid, positions) -> np.ndarray:
        pos = np.asarray(positions, dtype=np.int64)
        table = np.asarray(self.block_table(sid), dtype=np.int64)
        return table[pos // self.B] * self.B + pos % self.B

    def free_list(self) -> list:
        out = np.empty(self.num_frames, dtype=np.int32)
        n = _I64(0)
        _check("pb_free_list", self._L.pb_free_list(self._h, _ptr(out), len(out), ctypes.byref(n)))
        return [int(f) for f in out[:n.value]]

    @property
    def ref(self) -> np.ndarray:
        out = np.empty(self.num_frames, dtype=np.int32)
        _check("pb_ref_counts", self._L.pb_ref_counts(self._h, _ptr(out)))
        return out

    def stats(self) -> dict:
        st = PbStats()
        _check("pb_get_stats", self._L.pb_get_stats(self._h, ctypes.byref(st)))
        return {f: int(getattr(st, f)) for f, _ in PbStats._fields_}

    @property
    def evictions(self) -> int:
        return self.stats()["evictions"]

    @property
    def cached_frames(self) -> int:
        return self.stats()["cached_frames"]
