"""Seeded synthetic values for q, K and V, drawn by counter.

This module is the one source of input values for both the HIP path (through
torch on the device) and the CPU oracle (through numpy on the host). It holds
no attention or paging arithmetic: it only turns an integer counter into a
standard-normal value stored in the cache dtype.

Draw recipe (the same on both sides, bit for bit):

* counter ``c = ident * (H * D) + h * D + e`` for the token (or query)
  identity ``ident``, head ``h`` and element ``e``;
* ``x = mix(mix(lo(c) ^ key) ^ (hi(c) + 0x85EBCA6B))`` where ``key`` mixes
  the seed and the stream id (K, V or Q), ``lo``/``hi`` are the 32-bit halves
  and ``mix`` is the 32-bit "lowbias32" integer hash (xor-shift / multiply);
* the top 16 bits of ``x`` index a table of 65,536 standard-normal quantiles,
  ``Phi^-1((i + 0.5) / 65536)``, rounded once (round to nearest even) to the
  storage dtype.

So every value is a discretised N(0, 1) draw, reproducible from its position
alone. Integer operations are written so that no intermediate exceeds 2^49,
which keeps numpy int64 and torch int64 (CPU or GPU) results identical.
"""
from __future__ import annotations

import functools

import numpy as np

STREAM_K = 1
STREAM_V = 2
STREAM_Q = 3

DTYPES = ("f32", "f16", "bf16")

_M32 = 0xFFFFFFFF


def _mul32(x, c: int):
    """(x * c) mod 2^32 for 0 <= x < 2^32, without int64 overflow."""
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + (((hi * c) & 0xFFFF) << 16)) & _M32


def _mix32(x):
    """lowbias32 hash of a value in [0, 2^32), array-module agnostic."""
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _mix32_scalar(x: int) -> int:
    return int(_mix32(np.int64(x & _M32)))


def stream_key(seed: int, stream: int) -> int:
    return _mix32_scalar(_mix32_scalar(seed * 0x9E3779B9 + 0x632BE5AB) ^ stream)


def _index16(counter, key: int):
    lo = counter & _M32
    hi = counter >> 32
    x = _mix32(lo ^ key)
    x = _mix32(x ^ ((hi + 0x85EBCA6B) & _M32))
    return x >> 16


def _f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even) and return the 16-bit patterns."""
    b = x32.astype(np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


@functools.lru_cache(maxsize=None)
def quantile_table(dtype: str) -> np.ndarray:
    """65,536 N(0,1) quantiles stored in ``dtype``.

    Returns float32 values for "f32" and raw uint16 bit patterns for "f16"
    and "bf16".
    """
    from scipy.special import ndtri

    q = ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0)
    if dtype == "f32":
        return q.astype(np.float32)
    if dtype == "f16":
        return q.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return _f32_to_bf16_bits(q.astype(np.float32))
    raise ValueError(f"unknown dtype {dtype!r}")


def draw_np(seed: int, stream: int, idents, H: int, D: int, dtype: str, heads=None) -> np.ndarray:
    """Values for identities ``idents`` as a host array ``[len(idents), H, D]``.

    float32 for "f32"; uint16 bit patterns for "f16" and "bf16". With
    ``heads`` given, only those heads are drawn: ``[len(idents), len(heads), D]``
    holding exactly the values the full draw has at those heads.
    """
    idents = np.asarray(idents, dtype=np.int64).reshape(-1)
    hs = np.arange(H, dtype=np.int64) if heads is None else np.asarray(heads, dtype=np.int64)
    hd = (hs[:, None] * D + np.arange(D, dtype=np.int64)[None, :]).reshape(-1)
    counter = idents[:, None] * (H * D) + hd[None, :]
    idx = _index16(counter, stream_key(seed, stream))
    return quantile_table(dtype)[idx].reshape(len(idents), len(hs), D)


_TORCH_TABLES: dict = {}


def _torch_table(dtype: str, device):
    import torch

    k = (dtype, str(device))
    t = _TORCH_TABLES.get(k)
    if t is None:
        host = quantile_table(dtype)
        if dtype == "f32":
            t = torch.from_numpy(host.copy()).to(device)
        else:
            t = torch.from_numpy(host.view(np.int16).copy()).to(device)
        _TORCH_TABLES[k] = t
    return t


def torch_dtype(dtype: str):
    import torch

    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def draw_torch(seed: int, stream: int, idents, H: int, D: int, dtype: str, device):
    """Same values as :func:`draw_np`, produced by torch on ``device``.

    Returns a tensor ``[len(idents), H, D]`` of the torch dtype for ``dtype``.
    """
    import torch

    if not isinstance(idents, torch.Tensor):
        idents = torch.as_tensor(np.asarray(idents, dtype=np.int64))
    idents = idents.to(device=device, dtype=torch.int64).reshape(-1)
    hd = torch.arange(H * D, dtype=torch.int64, device=device)
    counter = idents[:, None] * (H * D) + hd[None, :]
    idx = _index16(counter, stream_key(seed, stream))
    vals = _torch_table(dtype, device)[idx]
    if dtype != "f32":
        vals = vals.view(torch_dtype(dtype))
    return vals.reshape(-1, H, D)


def nan_bits(dtype: str):
    """A quiet-NaN pattern in the storage representation (poison fill)."""
    if dtype == "f32":
        return np.float32(np.nan)
    if dtype == "f16":
        return np.uint16(0x7E00)
    return np.uint16(0x7FC0)
