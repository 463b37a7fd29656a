"""Pins of oracle/dense.py (fp64 causal attention with library matrix products).

Each ``pin_*`` takes a module exposing ``causal_attention`` (the oracle's
:mod:`oracle.dense`, or a copy of it with a planted mistake). The reference
is the C oracle's paged prefill, itself pinned by brute force and closed
forms (tests/oracle_pins.py), plus closed forms of the causal sum.
"""
from __future__ import annotations

import math
import sys

import numpy as np

from oracle.oracle import STORAGE, default as oracle_default
from workloads.values import STREAM_K, STREAM_Q, STREAM_V, draw_np, nan_bits


def _paged_problem(seed, dtype, H, D, B, ctxs, nqs):
    """Random sequences in a permuted pool; returns what the C oracle's
    prefill takes and the logical rows the dense form takes."""
    rng = np.random.default_rng(seed)
    nblk = [-(-c // B) for c in ctxs]
    NB = sum(nblk) + 2
    perm = rng.permutation(NB)
    pad = int(perm[-1])
    tables = np.full((len(ctxs), max(nblk)), pad, dtype=np.int32)
    k = np.full((NB, B, H, D), nan_bits(dtype), dtype=STORAGE[dtype])
    v = k.copy()
    rows, used = [], 0
    for s, c in enumerate(ctxs):
        tables[s, :nblk[s]] = perm[used:used + nblk[s]]
        used += nblk[s]
        ids = 10000 * (s + 1) + np.arange(c)
        kr = draw_np(seed, STREAM_K, ids, H, D, dtype)
        vr = draw_np(seed, STREAM_V, ids, H, D, dtype)
        for i in range(c):
            f = tables[s, i // B]
            k[f, i % B] = kr[i]
            v[f, i % B] = vr[i]
        rows.append((kr, vr))
    qs = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32)
    q = draw_np(seed, STREAM_Q, np.arange(int(qs[-1])) + 777, H, D, dtype)
    return q, k, v, tables, np.asarray(ctxs, dtype=np.int32), qs, rows


def pin_matches_c_oracle(mod):
    """Random causal problems (whole prompts, chunks, one query) in every
    storage dtype: within 1e-12 of the C oracle's paged prefill."""
    orc = oracle_default()
    cases = [("bf16", 2, 64, 16, [70, 33, 5], [70, 10, 1]),
             ("f16", 3, 32, 7, [41, 90], [41, 50]),
             ("f32", 1, 16, 4, [17, 1, 29], [3, 1, 29])]
    for seed, (dtype, H, D, B, ctxs, nqs) in enumerate(cases):
        q, k, v, tables, cl, qs, rows = _paged_problem(50 + seed, dtype, H, D, B, ctxs, nqs)
        scale = float(np.float32(D ** -0.5))
        ref = orc.paged_prefill(q, k, v, tables, cl, qs, B, scale, dtype)
        for s, (kr, vr) in enumerate(rows):
            n = int(nqs[s])
            got = mod.causal_attention(orc.widen(q[qs[s]:qs[s + 1]], dtype), orc.widen(kr, dtype),
                                       orc.widen(vr, dtype), scale, int(cl[s]) - n)
            err = float(np.max(np.abs(got - ref[qs[s]:qs[s + 1]])))
            assert err <= 1e-12, (dtype, s, err)


def pin_one_visible_key_returns_its_row(mod):
    """The first query of a whole prompt sees key 0 only: its output is v_0."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((6, 2, 8))
    v = rng.standard_normal((6, 2, 8))
    q = rng.standard_normal((6, 2, 8))
    o = mod.causal_attention(q, k, v, 0.7, 0)
    assert np.array_equal(o[0], v[0])


def pin_equal_scores_give_the_mean(mod):
    """q = 0: every visible key weighs the same, so query i (position
    first + i) returns the mean of rows 0 .. first + i."""
    rng = np.random.default_rng(4)
    k = rng.standard_normal((20, 3, 5))
    v = rng.standard_normal((20, 3, 5))
    first, n = 12, 8
    o = mod.causal_attention(np.zeros((n, 3, 5)), k, v, 0.5, first)
    for i in range(n):
        p = first + i
        for h in range(3):
            for e in range(5):
                mean = math.fsum(v[:p + 1, h, e]) / (p + 1)
                assert abs(o[i, h, e] - mean) <= 1e-15, (i, h, e)


def pin_later_keys_are_ignored(mod):
    """Rows after the last query's position, and rows after each query's own
    position, do not change its output (bit for bit)."""
    rng = np.random.default_rng(5)
    k = rng.standard_normal((30, 2, 8))
    v = rng.standard_normal((30, 2, 8))
    q = rng.standard_normal((10, 2, 8))
    base = mod.causal_attention(q, k, v, 0.3, 15)
    k2, v2 = k.copy(), v.copy()
    k2[25:] = 1e9
    v2[25:] = -7.0
    assert np.array_equal(mod.causal_attention(q, k2, v2, 0.3, 15), base)
    k3, v3 = k.copy(), v.copy()
    k3[20:] = 3.0  # visible to queries 5.. only
    v3[20:] = 3.0
    assert np.array_equal(mod.causal_attention(q, k3, v3, 0.3, 15)[:5], base[:5])
    assert not np.allclose(mod.causal_attention(q, k3, v3, 0.3, 15)[5:], base[5:])


ALL = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def run_all(mod) -> list:
    failed = []
    for pin in ALL:
        try:
            pin(mod)
        except Exception as exc:  # noqa: BLE001
            failed.append((pin.__name__, f"{type(exc).__name__}: {exc}"[:200]))
    return failed


if __name__ == "__main__":
    import importlib.util

    spec = importlib.util.spec_from_file_location("mutant_dense", sys.argv[1])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    failed = run_all(mod)
    for name, why in failed:
        print(name, why)
    sys.exit(len(failed))
