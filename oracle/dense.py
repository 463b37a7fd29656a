"""fp64 causal attention of many queries with library matrix products.

TEST INFRASTRUCTURE ONLY: the GPU tests use it to check every output of the
full-size prefill workloads, where the C oracle's per-query walk would take
minutes. The product library never imports it, and it shares no code with
the HIP path.

It computes the same definition as ``oracle_paged_prefill`` in oracle.c
("Solving the LLM Memory Wall: A Deep Dive into PagedAttention", "1. The
Mathematical Foundation"): query i of a sequence, at position p_i, attends
to the keys j <= p_i with weights softmax_j(scale * q_i . k_j) and returns
sum_j w_j v_j. The rows are the sequence's K and V in logical order, so
there is no block table here: paging only decides where the rows are read.

Steps, all in fp64: the scores of every (query, key) pair as one matrix
product per head; keys after a query's position get -inf; the exact
two-pass softmax (maximum, exponentials, sum); the output as a second
matrix product divided by the sum. The products are library routines
(numpy matmul); their summation order is the library's.

Pinned against the C oracle (itself pinned by brute force and closed forms)
to 1e-12 on random causal problems of every storage dtype, and by closed
forms of its own (one visible key returns its value row; equal scores give
the mean of the visible rows); planted mistakes in a copy of this file
must each fail a pin (tests/test_oracle_mutants.py).
"""
from __future__ import annotations

import numpy as np


def causal_attention(q, k, v, scale: float, first: int) -> np.ndarray:
    """Attention of n queries at positions first .. first + n - 1 over keys
    0 .. first + n - 1 of one sequence.

    ``q`` [n, H, D], ``k`` and ``v`` [ctx, H, D] (ctx >= first + n; rows
    past the last query's position are ignored), all fp64 (widened exactly
    by the caller). ``scale`` multiplies q . k. Returns fp64 [n, H, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, H, D = q.shape
    last = first + n  # keys 0 .. last - 1 can be visible
    kh = np.ascontiguousarray(k[:last].transpose(1, 0, 2))  # [H, last, D]
    vh = np.ascontiguousarray(v[:last].transpose(1, 0, 2))
    qh = np.ascontiguousarray(q.transpose(1, 0, 2))          # [H, n, D]
    a = scale * np.matmul(qh, kh.transpose(0, 2, 1))         # [H, n, last] scores
    pos = first + np.arange(n)
    hidden = np.arange(last)[None, :] > pos[:, None]         # key j after query i's position
    a[:, hidden] = -np.inf
    m = a.max(axis=2, keepdims=True)
    w = np.exp(a - m)
    z = w.sum(axis=2, keepdims=True)
    o = np.matmul(w, vh) / z                                 # [H, n, D]
    return np.ascontiguousarray(o.transpose(1, 0, 2))
