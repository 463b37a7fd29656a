"""GPU parity over the shapes the kernels accept beyond the named workloads:
every decode head dimension, block sizes on the compiled fast paths and off
them, each storage dtype, and prefill at both head dimensions with block
sizes from 1 to 64, sequences with no queries, a context whose block table
is too long to stage in LDS (the direct table-read path), and head counts
that take the head-per-XCD launch mapping.

Each case is a small seeded workload (random context lengths, a permuted
frame pool) written through the product block manager and kv_append, and
compared element by element with the fp64 oracle on the oracle's own replay.
The decode launch forms for many short contexts (two wavefronts) and for
long ones over enough workgroups (sixteen wavefronts on twice the heads)
need larger batches: those cases compare every output with the oracle's
contiguous definition over each sequence's logical tokens.
"""
from __future__ import annotations

import numpy as np
import pytest

from tests.gpu_support import (TOL, max_err, oracle_full, oracle_outputs, oracle_prefill,
                               pad_frame_for, require_gpu, run_gpu, run_gpu_prefill, say)
from workloads.configs import Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def shape_workload(dtype, D, B, ctx, H=3, query_lens=None, seed=9, spare=4):
    ctx = [int(c) for c in ctx]
    rng = np.random.default_rng(seed)
    NB = sum(-(-c // B) for c in ctx) + spare
    return Workload(
        name=f"shape_{dtype}_D{D}_B{B}", seed=seed, dtype=dtype, H=H, D=D, B=B, NB=NB,
        num_seqs=len(ctx), prefill=[(s, c) for s, c in enumerate(ctx)],
        frame_order=rng.permutation(NB),
        query_lens=None if query_lens is None else np.asarray(query_lens, dtype=np.int64),
        description=f"{dtype}, D={D}, B={B}, H={H}, ctx {ctx}")


DECODE_CASES = [
    # (dtype, D, B): fast-path block sizes 8 / 32 / 64, off-path 1 / 7 / 24
    ("bf16", 64, 8), ("f16", 256, 64), ("bf16", 32, 7), ("f32", 128, 16), ("f16", 128, 1),
    ("bf16", 16, 32), ("f32", 64, 24), ("f16", 32, 64),
]


@pytest.mark.parametrize("dtype,D,B", DECODE_CASES)
@pytest.mark.parametrize("pt", [0, 1 << 6])
@pytest.mark.parametrize("H", [3, 6, 8])
def test_decode_shapes(dtype, D, B, pt, H):
    """H = 8 takes the launches whose workgroups serve up to 8 adjacent
    heads (rows under 256 bytes), H = 6 a smaller grouping that divides it,
    H = 3 the one-head launches of every shape."""
    rng = np.random.default_rng(D * 131 + B)
    ctx = list(rng.integers(1, 400, size=5)) + [1, B, B + 1]
    w = shape_workload(dtype, D, B, ctx, H=H)
    # pt = 64 forces several partitions per sequence (the library rounds it
    # up to a whole number of the kernel's chunks); 0 takes its default
    say(f"[gpu] decode {w.description}, partition tokens {pt or 'default'}")
    part = pt
    res = run_gpu(w, partition_tokens=part)
    ref = oracle_outputs(w, pad_frame_for(w))
    for (pt_, out), (snap, o) in zip(res, ref):
        assert np.array_equal(pt_.tables, snap.tables)
        err = max_err(out.numpy(), o)
        say(f"  max-abs err {err:.3e} (tol {TOL[dtype]})")
        assert err <= TOL[dtype]


# (dtype, D, H, S, tokens per chunk, heads per workgroup): S sequences of up
# to 200 tokens (at most 64 chunks) over at least 4096 workgroups, which the
# decode launch serves with two wavefronts per workgroup instead of eight,
# and with twice the heads where 2 * hp divides H and the halved grid still
# has at least 4096 workgroups (the first three cases); H = 33 keeps one
# head, and 128 sequences of 32 heads keep it at the default partition size
# for lack of workgroups (their four 64-token partitions have enough)
TWO_WAVE_CASES = [("bf16", 128, 32, 256, 16, 1), ("f16", 64, 64, 256, 16, 2),
                  ("f32", 128, 32, 256, 8, 1), ("bf16", 128, 33, 128, 16, 1),
                  ("bf16", 128, 32, 128, 16, 1)]


@pytest.mark.parametrize("dtype,D,H,S,chunk,hp", TWO_WAVE_CASES)
def test_decode_short_contexts_two_wave_launch(dtype, D, H, S, chunk, hp):
    """Many short contexts: the two-wavefront launches (twice the heads per
    workgroup where that fits) of the ungrouped and the grouped pass (bit
    for bit equal, checked inside run_gpu) against the oracle, at the
    default partition size and at 64-token partitions."""
    rng = np.random.default_rng(D + H + S)
    ctx = list(rng.integers(1, 201, size=S - 2)) + [1, 200]
    assert max(ctx) <= 64 * chunk and S * (H // hp) >= 4096
    w = shape_workload(dtype, D, 16, ctx, H=H, seed=11)
    ref = oracle_outputs(w, pad_frame_for(w))
    for pt in (0, 64):
        parts = 1 if pt == 0 else -(-max(ctx) // pt)
        doubled = H % (2 * hp) == 0 and S * (H // (2 * hp)) * parts >= 4096
        say(f"[gpu] decode {S} short contexts, {dtype} D={D} H={H} "
            f"({2 * hp if doubled else hp} heads per workgroup), partition tokens {pt or 'default'}")
        res = run_gpu(w, partition_tokens=pt, grouped=True)
        for (pt_, out), (snap, o) in zip(res, ref):
            assert np.array_equal(pt_.tables, snap.tables)
            err = max_err(out.numpy(), o)
            say(f"  max-abs err {err:.3e} (tol {TOL[dtype]})")
            assert err <= TOL[dtype]


# (dtype, D, H, S, heads per workgroup of the default form, longest context,
# partition tokens): contexts of 1,536 tokens or more in four partitions (or
# one), over at least 1,024 workgroups at twice the heads, which the decode
# launch serves with sixteen wavefronts on 2 * hp heads (the wide form): the
# groupings of 16, 8, 4 and 2 heads, 512-byte rows (fp32 d = 128, bf16
# d = 256), and the ordered default of one 4,096-token partition
WIDE_CASES = [("bf16", 16, 16, 256, 8, 6144, 1536), ("bf16", 32, 16, 128, 4, 6144, 1536),
              ("f16", 64, 8, 128, 2, 6144, 1536), ("f32", 128, 4, 128, 1, 6144, 1536),
              ("bf16", 256, 4, 128, 1, 6144, 1536), ("f32", 64, 8, 64, 1, 6144, 1536),
              ("bf16", 128, 8, 256, 1, 4096, 0)]


@pytest.mark.parametrize("dtype,D,H,S,hp,max_ctx,pt", WIDE_CASES)
def test_decode_long_contexts_wide_launch(dtype, D, H, S, hp, max_ctx, pt):
    """Long contexts over enough workgroups: the sixteen-wavefront launches
    on twice the heads, of the ungrouped and the grouped pass (bit for bit
    equal, checked inside run_gpu), dispatched longest first as the
    benchmark does; every output against the fp64 oracle's contiguous
    definition."""
    import torch

    rng = np.random.default_rng(D + H + S + max_ctx)
    ctx = list(rng.integers(1, max_ctx + 1, size=S - 2)) + [1, max_ctx]
    part = pt if pt else 4096  # the ordered default for contexts of 2,049-4,096 tokens
    parts = -(-max_ctx // part)
    assert max_ctx >= 1536 and (parts == 1 or parts >= 4) and H % (2 * hp) == 0
    assert S * (H // (2 * hp)) * parts >= 1024
    w = shape_workload(dtype, D, 16, ctx, H=H, seed=16)
    say(f"[gpu] decode {S} long contexts, {dtype} D={D} H={H} ({2 * hp} heads per workgroup), "
        f"partition tokens {pt or 'default'}")
    results = run_gpu(w, partition_tokens=pt, grouped=True, order="longest")
    for pt_, out in results:
        o = out.numpy()
        assert np.all(np.isfinite(o)), "non-finite output"
        ref = oracle_full(w, pt_.step, pt_.context_lens)
        err = max_err(o, ref)
        say(f"  all {o.shape[0]} x {o.shape[1]} (seq, head) outputs, max-abs err {err:.3e} "
            f"(tol {TOL[dtype]})")
        assert err <= TOL[dtype]
    del results
    torch.cuda.empty_cache()


PREFILL_CASES = [
    # (dtype, D, B, contexts, query lengths)
    ("bf16", 64, 16, [300, 45, 129, 1], [300, 0, 20, 1]),
    ("f16", 64, 8, [257, 130, 64], [100, 130, 64]),
    ("f16", 128, 64, [200, 513, 31], [200, 129, 0]),
    ("bf16", 128, 7, [150, 99, 260], [40, 99, 260]),
    # B = 1 and 2,200 keys: 2,200 table entries, more than the kernel stages in LDS
    ("bf16", 128, 1, [2200, 40], [130, 40]),
    # B = 16 and 33,000 keys (2,063 frames): wavefronts whose pieces share a
    # frame read its number from the table a tile ahead, at any length
    ("bf16", 64, 16, [33000, 100], [40, 100]),
]


@pytest.mark.parametrize("dtype,D,B,ctx,qlens", PREFILL_CASES)
def test_prefill_shapes(dtype, D, B, ctx, qlens):
    w = shape_workload(dtype, D, B, ctx, H=2, query_lens=qlens, seed=10)
    say(f"[gpu] prefill {w.description}, queries {qlens}")
    pt, qs, out = run_gpu_prefill(w)
    snap, ref = oracle_prefill(w, pad_frame_for(w))
    assert np.array_equal(pt.tables, snap.tables)
    assert int(qs[-1]) == sum(qlens)
    err = max_err(out.numpy(), ref)
    say(f"  {int(qs[-1])} queries, max-abs err {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,H,order", [("bf16", 8, "cost"), ("f16", 16, "random")])
def test_prefill_heads_on_xcds(dtype, H, order):
    """Head counts that are multiples of 8 take the launch mapping that pins
    head h to XCD h mod 8; every output is compared with the oracle, in the
    default order and in another dispatch order (bit for bit)."""
    ctx, qlens = [700, 129, 400, 5], [512, 129, 1, 5]
    w = shape_workload(dtype, 128, 16, ctx, H=H, query_lens=qlens, seed=12)
    say(f"[gpu] prefill {w.description}, queries {qlens}, order {order}")
    pt, qs, out = run_gpu_prefill(w, order=order)
    snap, ref = oracle_prefill(w, pad_frame_for(w))
    assert np.array_equal(pt.tables, snap.tables)
    err = max_err(out.numpy(), ref)
    say(f"  {int(qs[-1])} queries, max-abs err {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]



@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_idle_wavefronts(dtype):
    """Query counts on each side of the 32-query wavefront and 128-query tile
    boundaries: in the last tile of such a sequence the wavefronts past its
    last query compute nothing, yet still stage K/V for the others; every
    output is compared with the oracle, also in a random dispatch order."""
    qlens = [1, 31, 32, 33, 64, 95, 96, 97, 127, 128, 129, 161]
    ctx = [q + e for q, e in zip(qlens, [0, 300, 17, 0, 129, 64, 1, 250, 0, 33, 400, 2])]
    w = shape_workload(dtype, 128, 16, ctx, H=8, query_lens=qlens, seed=14)
    say(f"[gpu] prefill {w.description}, queries {qlens}")
    pt, qs, out = run_gpu_prefill(w, order="random")
    snap, ref = oracle_prefill(w, pad_frame_for(w))
    assert np.array_equal(pt.tables, snap.tables)
    assert int(qs[-1]) == sum(qlens)
    err = max_err(out.numpy(), ref)
    say(f"  {int(qs[-1])} queries, max-abs err {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("scale", [0.0, -0.125, -1.5])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_nonpositive_scale(dtype, scale):
    """Any finite scale: zero (every visible key weighs the same, so the
    output is the mean of the value rows) and negative ones, for decode
    (forced partitions, so the merge runs too) and for prefill (causal
    masks, whose keys must still weigh exactly 0), against the oracle."""
    from dataclasses import replace

    ctx, qlens = [300, 45, 129, 1, 70], [300, 45, 20, 1, 33]
    w = replace(shape_workload(dtype, 128, 16, ctx, H=2, query_lens=qlens, seed=15), scale_value=scale)
    say(f"[gpu] scale {scale}: {w.description}")
    res = run_gpu(w, partition_tokens=64)
    ref = oracle_outputs(w, pad_frame_for(w))
    for (pt, out), (snap, o) in zip(res, ref):
        err = max_err(out.numpy(), o)
        say(f"  decode max-abs err {err:.3e}")
        assert err <= TOL[dtype]
    pt, qs, out = run_gpu_prefill(w)
    snap, ref = oracle_prefill(w, pad_frame_for(w))
    err = max_err(out.numpy(), ref)
    say(f"  prefill {int(qs[-1])} queries, max-abs err {err:.3e}")
    assert err <= TOL[dtype]
