"""Seeded random sweeps on the GPU against the fp64 oracle: decode over
random dtypes, head dims, block sizes (on and off the compiled fast paths),
head counts, batch sizes, context mixes (empty, single-token, block-aligned,
long) and forced partition sizes; prefill over random chunk shapes, head
counts and dispatch orders; grouped decode over random fork families; decode
batches large enough for the short launch form, and long-context batches
that take the sixteen-wavefront form. Every case is
compared element by element; grouped decode is also compared bit for bit
with the ungrouped pass."""
from __future__ import annotations

import numpy as np
import pytest

from tests.gpu_support import (TOL, max_err, oracle_default, oracle_full, oracle_outputs,
                               oracle_prefill, pad_frame_for, require_gpu, run_gpu, run_gpu_prefill,
                               say)
from tests.test_gpu_shapes import shape_workload
from workloads import values as V

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16")
HEAD_DIMS = (16, 32, 64, 128, 256)
BLOCKS = (1, 3, 8, 10, 16, 32, 64, 100)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _contexts(rng, S, B):
    kinds = rng.integers(0, 5, size=S)
    ctx = []
    for k in kinds:
        if k == 0:
            ctx.append(int(rng.integers(1, 600)))
        elif k == 1:
            ctx.append(1)
        elif k == 2:
            ctx.append(int(B * rng.integers(1, 8)))          # ends on a block boundary
        elif k == 3:
            ctx.append(int(rng.integers(600, 1500)))
        else:
            ctx.append(int(rng.integers(0, 3)))               # empty or nearly
    return ctx


@pytest.mark.parametrize("seed", range(24))
def test_decode_random_shapes(seed):
    rng = np.random.default_rng(5000 + seed)
    dtype = DTYPES[seed % 3]
    D = int(rng.choice(HEAD_DIMS))
    B = int(rng.choice(BLOCKS))
    H = int(rng.integers(1, 7))
    S = int(rng.integers(1, 13))
    ctx = _contexts(rng, S, B)
    pt = int(rng.choice([0, 16, 64, 200]))
    w = shape_workload(dtype, D, B, ctx, H=H, seed=60 + seed)
    say(f"[gpu] fuzz decode seed {seed}: {w.description}, partition tokens {pt or 'default'}")
    res = run_gpu(w, partition_tokens=pt)
    ref = oracle_outputs(w, pad_frame_for(w))
    for (p, out), (snap, o) in zip(res, ref):
        assert np.array_equal(p.tables, snap.tables)
        err = max_err(out.numpy(), o)
        say(f"  max-abs err {err:.3e}")
        assert err <= TOL[dtype]


@pytest.mark.parametrize("seed", range(8))
def test_decode_random_short_launches(seed):
    """Batches large enough for the short launch form (contexts of at most
    64 chunks over 4,096 workgroups or more: two wavefronts, and twice the
    heads per workgroup where they divide H): random dtype, head dim, block
    size, head count and partition size, with empty, single-token and
    block-aligned contexts, through the ungrouped and the grouped pass (bit
    for bit equal, checked inside run_gpu)."""
    rng = np.random.default_rng(7000 + seed)
    dtype = DTYPES[seed % 3]
    D = int(rng.choice(HEAD_DIMS))
    B = int(rng.choice(BLOCKS))
    H = int(rng.choice([12, 16, 24, 33, 40]))
    row = D * (4 if dtype == "f32" else 2)
    hp = 1 if row >= 256 else 256 // row  # the row's preferred grouping, at most
    # enough sequences for the doubled grouping's grid; contexts of at most
    # 256 tokens stay within 64 chunks at every shape (chunks are 4 tokens
    # or more)
    S = -(-8192 * hp // H) + int(rng.integers(0, 100))
    cap = 256
    ctx = [int(c) for c in rng.integers(1, cap + 1, size=S)]
    ctx[:4] = [0, 1, B, min(cap, 2 * B)]
    pt = int(rng.choice([0, 16, 64]))
    w = shape_workload(dtype, D, B, ctx, H=H, seed=70 + seed)
    say(f"[gpu] fuzz short decode seed {seed}: {dtype} D={D} B={B} H={H} S={S} contexts up to "
        f"{max(ctx)}, partition tokens {pt or 'default'}")
    res = run_gpu(w, partition_tokens=pt, grouped=True)
    ref = oracle_outputs(w, pad_frame_for(w))
    for (p, out), (snap, o) in zip(res, ref):
        assert np.array_equal(p.tables, snap.tables)
        err = max_err(out.numpy(), o)
        say(f"  max-abs err {err:.3e}")
        assert err <= TOL[dtype]


@pytest.mark.parametrize("seed", range(6))
def test_decode_random_wide_launches(seed):
    """Batches that take the sixteen-wavefront form (contexts of 1,536 tokens
    or more in four or more partitions of at least that length, 1,024
    workgroups or more at twice the heads): random dtype, head dim, block
    size (on and off the compiled fast paths), head count (a multiple of
    twice the row's grouping) and partition size, with empty, single-token and block-aligned
    contexts, dispatched longest first, through the ungrouped and the
    grouped pass (bit for bit equal, checked inside run_gpu); every output
    against the oracle's contiguous definition."""
    import torch

    rng = np.random.default_rng(8000 + seed)
    dtype = DTYPES[seed % 3]
    D = HEAD_DIMS[seed % 5]
    B = int(rng.choice(BLOCKS))
    row = D * (4 if dtype == "f32" else 2)
    hp = 1 if row >= 256 else 256 // row  # the row's preferred grouping
    H = 2 * hp * int(rng.integers(1, 6))  # a multiple of the doubled grouping
    pt = int(rng.choice([1536, 2048]))
    parts = int(rng.integers(4, 6))
    groups = H // (2 * hp)  # workgroups per (sequence, partition) at the doubled grouping
    S = -(-1024 // (groups * parts)) + int(rng.integers(0, 16))
    cap = parts * pt
    ctx = [int(c) for c in rng.integers(1, cap + 1, size=S)]
    ctx[:5] = [0, 1, B, 2 * B, cap]
    w = shape_workload(dtype, D, B, ctx, H=H, seed=80 + seed)
    say(f"[gpu] fuzz wide decode seed {seed}: {dtype} D={D} B={B} H={H} S={S} contexts up to "
        f"{cap}, partition tokens {pt}, {2 * hp} heads per workgroup")
    results = run_gpu(w, partition_tokens=pt, grouped=True, order="longest")
    for p, out in results:
        o = out.numpy()
        ref = oracle_full(w, p.step, p.context_lens)
        err = max_err(o, ref)
        say(f"  all {o.shape[0]} x {o.shape[1]} (seq, head) outputs, max-abs err {err:.3e}")
        assert err <= TOL[dtype]
    del results
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed", range(24))
def test_prefill_random_shapes(seed):
    rng = np.random.default_rng(6000 + seed)
    dtype = ("bf16", "f16")[seed % 2]
    D = (64, 128)[(seed // 2) % 2]
    B = int(rng.choice(BLOCKS))
    S = int(rng.integers(1, 7))
    # head counts on both launch mappings (multiples of 8: head h on XCD h mod 8)
    H = (2, 8, 3, 16, 1, 8)[seed % 6]
    ctx = [int(c) for c in rng.integers(1, 700, size=S)]
    qlens = [int(rng.integers(0, c + 1)) if rng.random() < 0.7 else c for c in ctx]
    w = shape_workload(dtype, D, B, ctx, H=H, query_lens=qlens, seed=80 + seed)
    order = ("cost", "random", None)[seed % 3]
    split = seed % 4 == 0  # bf16: weights as a bf16 value plus its residual
    say(f"[gpu] fuzz prefill seed {seed}: {w.description}, queries {qlens}, order {order}, "
        f"split weights {split}")
    pt, qs, out = run_gpu_prefill(w, order=order, split_weights=split)
    snap, ref = oracle_prefill(w, pad_frame_for(w))
    assert np.array_equal(pt.tables, snap.tables)
    err = max_err(out.numpy(), ref)
    say(f"  {int(qs[-1])} queries, max-abs err {err:.3e}")
    assert err <= (1e-4 if split and dtype == "bf16" else TOL[dtype])


@pytest.mark.parametrize("seed", range(10))
def test_grouped_random_forks(seed):
    """Families of 1-6 forks of one prompt (split into groups of at most 4
    by share_groups), each sharing a random number of the prompt's frames
    and adding frames of its own."""
    import torch

    import paged_kv_cache_126_amd as pkv
    from paged_kv_cache_126_amd.driver import share_groups

    rng = np.random.default_rng(7000 + seed)
    dtype = DTYPES[seed % 3]
    D = int(rng.choice((32, 64, 128)))
    B = int(rng.choice((8, 16, 32, 10)))
    H = int(rng.integers(1, 5))
    mb = 24
    rows, ctx = [], []
    frame = 0
    for _ in range(int(rng.integers(2, 6))):
        base = np.arange(frame, frame + mb)
        frame += mb
        for _ in range(int(rng.integers(1, 7))):
            r = base.copy()
            keep = int(rng.integers(0, mb + 1))
            r[keep:] = np.arange(frame, frame + mb - keep)
            frame += mb - keep
            rows.append(r)
            ctx.append(int(rng.integers(0, mb * B + 1)))
    NB = frame + 1
    perm = rng.permutation(NB).astype(np.int32)
    tables = perm[np.stack(rows)].astype(np.int32)          # scatter the frames over the pool
    ctx = np.asarray(ctx, dtype=np.int32)
    S = len(ctx)
    ids = np.arange(NB * B, dtype=np.int64) + 10**6 * seed
    k = V.draw_np(9, V.STREAM_K, ids, H, D, dtype).reshape(NB, B, H, D)
    v = V.draw_np(9, V.STREAM_V, ids, H, D, dtype).reshape(NB, B, H, D)
    q = V.draw_np(10, V.STREAM_Q, np.arange(S, dtype=np.int64) + 1000 * seed, H, D, dtype)
    scale = float(np.float32(D ** -0.5))
    ref = oracle_default().paged_decode(q, k, v, tables, ctx, B, scale, dtype)
    gs, gsh = share_groups(tables, ctx, B)
    dev = torch.device("cuda:0")
    tdt = V.torch_dtype(dtype)

    def dev_t(x):
        x = np.ascontiguousarray(x)
        if dtype == "f32":
            return torch.from_numpy(x).to(dev)
        return torch.from_numpy(x.view(np.int16)).to(dev).view(tdt)

    tq, tk, tv = dev_t(q), dev_t(k), dev_t(v)
    bt, cl = torch.from_numpy(tables).to(dev), torch.from_numpy(ctx).to(dev)
    mc = max(int(ctx.max()), 1)
    for pt in (0, 16 if dtype != "f32" else 64):
        out = torch.full((S, H, D), float("nan"), dtype=torch.float32, device=dev)
        two = torch.full_like(out, float("nan"))
        shape = pkv.lib.make_shape(tq, tk, bt, mc, pkv.lib.PA_F32, pt)
        ws = pkv.alloc_workspace(shape, dev)
        pkv.paged_attn_decode_grouped(tq, tk, tv, bt, cl, B, scale, out, mc,
                                      torch.from_numpy(gs).to(dev), torch.from_numpy(gsh).to(dev),
                                      ws, pt)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        pkv.paged_attn_decode(tq, tk, tv, bt, cl, B, scale, two, mc, ws, pt)
        torch.cuda.synchronize()
        assert np.array_equal(o, two.cpu().numpy())
        err = max_err(o, ref)
        say(f"[gpu] fuzz grouped seed {seed}: {dtype} D={D} B={B} H={H}, {S} seqs in "
            f"{len(gsh)} groups (shared {sorted(set(gsh.tolist()))[-3:]}), P{pt}: err {err:.3e}")
        assert err <= TOL[dtype]
