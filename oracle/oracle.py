"""Python front end of the C oracle (``oracle/oracle.c``) plus workload replay.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it; the product library never imports it. It shares no code with
the HIP path. Values come from :mod:`workloads.values`; block tables and slots
come from :mod:`oracle.blockmgr`, this oracle's own block manager.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_D = ctypes.c_double


class OracleError(RuntimeError):
    pass


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """Handle on one build of liboracle.so (tests may load mutated builds)."""

    def __init__(self, path: str = DEFAULT_LIB):
        if not os.path.exists(path):
            from oracle.build import build

            build(out=path)
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.oracle_paged_decode.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I64, _I, _D, _I, _P]
        L.oracle_paged_decode_split.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I64, _I, _D,
                                                _I, _I, _P]
        L.oracle_dense_attention.argtypes = [_P, _P, _P, _P, _I, _I, _I, _D, _I, _P]
        L.oracle_paged_prefill.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I64, _I, _D, _I,
                                           _P]
        L.oracle_kv_append.argtypes = [_P, _P, _P, _I64, _I, _I, _I, _I64, _I, _P, _P]
        L.oracle_gather.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I64, _I, _I, _P]
        L.oracle_widen.argtypes = [_P, _I64, _I, _P]
        L.oracle_set_num_threads.argtypes = [_I]
        L.oracle_set_num_threads.restype = None
        for f in ("oracle_paged_decode", "oracle_paged_decode_split", "oracle_dense_attention",
                  "oracle_paged_prefill",
                  "oracle_kv_append", "oracle_gather", "oracle_widen", "oracle_num_threads"):
            getattr(L, f).restype = _I

    @staticmethod
    def _check(rc: int, what: str):
        if rc != 0:
            raise OracleError(f"{what} failed with code {rc}")

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        """OpenMP threads of the calls that follow (for timing)."""
        self.lib.oracle_set_num_threads(int(n))

    def paged_decode(self, q, k_cache, v_cache, block_tables, context_lens, B: int,
                     scale: float, dtype: str) -> np.ndarray:
        """fp64 [S, H, D] output of decode attention through the block tables."""
        q = np.ascontiguousarray(q, dtype=STORAGE[dtype])
        k_cache = np.ascontiguousarray(k_cache, dtype=STORAGE[dtype])
        v_cache = np.ascontiguousarray(v_cache, dtype=STORAGE[dtype])
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        S, H, D = q.shape
        NB = k_cache.shape[0]
        assert k_cache.shape == (NB, B, H, D) and v_cache.shape == k_cache.shape
        assert bt.ndim == 2 and bt.shape[0] == S and cl.shape == (S,)
        out = np.zeros((S, H, D), dtype=np.float64)
        rc = self.lib.oracle_paged_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl),
                                          S, H, D, B, NB, bt.shape[1], float(np.float32(scale)),
                                          DTYPE_CODE[dtype], _ptr(out))
        self._check(rc, "oracle_paged_decode")
        return out

    def paged_decode_split(self, q, k_cache, v_cache, block_tables, context_lens, B: int,
                           scale: float, dtype: str, P: int) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=STORAGE[dtype])
        k_cache = np.ascontiguousarray(k_cache, dtype=STORAGE[dtype])
        v_cache = np.ascontiguousarray(v_cache, dtype=STORAGE[dtype])
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        S, H, D = q.shape
        NB = k_cache.shape[0]
        out = np.zeros((S, H, D), dtype=np.float64)
        rc = self.lib.oracle_paged_decode_split(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt),
                                                _ptr(cl), S, H, D, B, NB, bt.shape[1],
                                                float(np.float32(scale)), DTYPE_CODE[dtype], P,
                                                _ptr(out))
        self._check(rc, "oracle_paged_decode_split")
        return out

    def paged_prefill(self, q, k_cache, v_cache, block_tables, context_lens, query_start, B: int,
                      scale: float, dtype: str) -> np.ndarray:
        """fp64 [T, H, D]: causal attention of each sequence's last tokens (see oracle.c)."""
        q = np.ascontiguousarray(q, dtype=STORAGE[dtype])
        k_cache = np.ascontiguousarray(k_cache, dtype=STORAGE[dtype])
        v_cache = np.ascontiguousarray(v_cache, dtype=STORAGE[dtype])
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        qs = np.ascontiguousarray(query_start, dtype=np.int32)
        T, H, D = q.shape
        S = cl.shape[0]
        NB = k_cache.shape[0]
        assert qs.shape == (S + 1,) and qs[-1] == T and k_cache.shape == (NB, B, H, D)
        out = np.zeros((T, H, D), dtype=np.float64)
        rc = self.lib.oracle_paged_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl),
                                           _ptr(qs), S, H, D, B, NB, bt.shape[1],
                                           float(np.float32(scale)), DTYPE_CODE[dtype], _ptr(out))
        self._check(rc, "oracle_paged_prefill")
        return out

    def dense_attention(self, q, k_rows, v_rows, seq_start, scale: float, dtype: str) -> np.ndarray:
        """fp64 [S, H, D]; sequence s attends to rows seq_start[s]:seq_start[s+1]."""
        q = np.ascontiguousarray(q, dtype=STORAGE[dtype])
        k_rows = np.ascontiguousarray(k_rows, dtype=STORAGE[dtype])
        v_rows = np.ascontiguousarray(v_rows, dtype=STORAGE[dtype])
        st = np.ascontiguousarray(seq_start, dtype=np.int64)
        S, H, D = q.shape
        assert st.shape == (S + 1,) and k_rows.shape[1:] == (H, D)
        out = np.zeros((S, H, D), dtype=np.float64)
        rc = self.lib.oracle_dense_attention(_ptr(q), _ptr(k_rows), _ptr(v_rows), _ptr(st), S, H, D,
                                             float(np.float32(scale)), DTYPE_CODE[dtype], _ptr(out))
        self._check(rc, "oracle_dense_attention")
        return out

    def kv_append(self, k_new, v_new, slot_mapping, k_cache, v_cache, B: int, dtype: str) -> None:
        """In-place host scatter of token rows into the two caches."""
        k_new = np.ascontiguousarray(k_new, dtype=STORAGE[dtype])
        v_new = np.ascontiguousarray(v_new, dtype=STORAGE[dtype])
        sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
        N, H, D = k_new.shape
        NB = k_cache.shape[0]
        assert k_cache.shape == (NB, B, H, D) and k_cache.dtype == STORAGE[dtype]
        rc = self.lib.oracle_kv_append(_ptr(k_new), _ptr(v_new), _ptr(sm), N, H, D, B, NB,
                                       DTYPE_CODE[dtype], _ptr(k_cache), _ptr(v_cache))
        self._check(rc, "oracle_kv_append")

    def gather(self, cache, block_tables, context_lens, B: int, dtype: str) -> np.ndarray:
        cache = np.ascontiguousarray(cache, dtype=STORAGE[dtype])
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        NB, _, H, D = cache.shape
        S = cl.shape[0]
        out = np.zeros((int(cl.clip(min=0).sum()), H, D), dtype=STORAGE[dtype])
        rc = self.lib.oracle_gather(_ptr(cache), _ptr(bt), _ptr(cl), S, H, D, B, NB, bt.shape[1],
                                    DTYPE_CODE[dtype], _ptr(out))
        self._check(rc, "oracle_gather")
        return out

    def widen(self, a, dtype: str) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=STORAGE[dtype])
        out = np.zeros(a.shape, dtype=np.float64)
        rc = self.lib.oracle_widen(_ptr(a), a.size, DTYPE_CODE[dtype], _ptr(out))
        self._check(rc, "oracle_widen")
        return out


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
