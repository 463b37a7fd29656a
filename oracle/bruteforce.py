"""Exact-arithmetic brute force for tiny decode-attention cases (test only).

Scores are exact rationals (``fractions.Fraction``) of the stored values;
exponentials, sums and the division use ``decimal`` at 60 significant digits.
The result is therefore the softmax attention of "Solving the LLM Memory
Wall: A Deep Dive into PagedAttention" (section "1. The Mathematical
Foundation") to far below fp64 resolution. Block translation follows "The
Mathematics of Block Translation" on "PagedAttention: Virtual Memory Guide
for LLM Inference": token i sits in frame table[i // B] at offset i % B.
"""
from __future__ import annotations

import decimal
from fractions import Fraction

_CTX = decimal.Context(prec=60)


def _dec(x: Fraction) -> decimal.Decimal:
    return decimal.Decimal(x.numerator) / decimal.Decimal(x.denominator)


def decode_one(q, k_cache, v_cache, table, ctx: int, h: int, B: int, scale: float):
    """Attention output for one (sequence, head), as a list of floats.

    q: [D] floats; k_cache / v_cache: nested [NB][B][H][D] floats;
    table: logical block -> frame; ctx: tokens attended.
    """
    if ctx <= 0:
        return [0.0] * len(q)
    with decimal.localcontext(_CTX):
        return _decode_one(q, k_cache, v_cache, table, ctx, h, B, scale)


def _decode_one(q, k_cache, v_cache, table, ctx, h, B, scale):
    qf = [Fraction(x) for x in q]
    sc = Fraction(scale)
    rows_k, rows_v = [], []
    for i in range(ctx):
        b, o = divmod(i, B)
        f = table[b]
        rows_k.append(k_cache[f][o][h])
        rows_v.append(v_cache[f][o][h])
    a = [sc * sum(qe * Fraction(ke) for qe, ke in zip(qf, kr)) for kr in rows_k]
    m = max(a)
    w = [_dec(ai - m).exp() for ai in a]
    z = sum(w, decimal.Decimal(0))
    out = []
    for e in range(len(q)):
        num = sum((wj * _dec(Fraction(rows_v[j][e])) for j, wj in enumerate(w)), decimal.Decimal(0))
        out.append(float(num / z))
    return out
