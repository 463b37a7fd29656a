"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Small variants of the five workloads are compared element by element with
the paged fp64 oracle; the full-size decode workloads, in the launch
configuration the benchmark times, are compared on every output with the
contiguous fp64 oracle over each sequence's logical tokens. Tolerances are the
acceptance bars: max-abs 1e-5 for fp32 inputs, 2e-3 for bf16/fp16 inputs.
KV append and block translation are compared bit for bit.
"""
from dataclasses import replace

import numpy as np
import pytest

from tests.gpu_support import (TOL, max_err, oracle_caches, oracle_outputs, oracle_prefill,
                               oracle_full, oracle_prefill_full, oracle_prefix_full,
                               oracle_prefix_rounds, pad_frame_for, require_gpu, run_gpu,
                               run_gpu_prefill, run_gpu_prefix, say)
from workloads import configs
from workloads import values as V

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _check_against_oracle(w, gpu_results, label):
    ref = oracle_outputs(w, pad_frame_for(w))
    assert len(gpu_results) == len(ref)
    for (pt, out), (snap, o) in zip(gpu_results, ref):
        assert np.array_equal(pt.tables, snap.tables)
        assert np.array_equal(pt.context_lens, snap.context_lens)
        err = max_err(out.float().numpy(), o)
        say(f"  {label} step {pt.step}: max-abs err {err:.3e} (tol {TOL[w.dtype]})")
        assert err <= TOL[w.dtype], (label, pt.step, err)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_small_workload_parity(cfg):
    w = configs.small(cfg)
    say(f"[gpu] small workload {w.name}: {w.description}")
    _check_against_oracle(w, run_gpu(w), w.name)


@pytest.mark.parametrize("cfg,pt", [(2, 16), (2, 64), (2, 1 << 20), (5, 48), (5, 1 << 20), (1, 64),
                                    (3, 512), (4, 96)])
def test_partition_sizes(cfg, pt):
    """Forcing many splits, or none, still matches the oracle."""
    w = configs.small(cfg)
    say(f"[gpu] {w.name} with partition_tokens={pt}")
    _check_against_oracle(w, run_gpu(w, partition_tokens=pt), f"{w.name}/P{pt}")


def test_two_phase_launch_equals_combined():
    w = configs.small(3)
    say(f"[gpu] {w.name}: partitions + merge entry points vs paged_attn_decode")
    a = run_gpu(w, partition_tokens=256)
    b = run_gpu(w, partition_tokens=256, phases=True)
    for (_, x), (_, y) in zip(a, b):
        assert np.array_equal(x.numpy(), y.numpy())


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_parity(cfg):
    """The full workload in the launch configuration the benchmark times
    (longest work first, default partition size): every output, every
    sequence and head, against the fp64 oracle's contiguous definition over
    the sequence's logical tokens. These caches pass 2^31 bytes (2.6 GB for
    the batch-64 workload, 8.6 GB for batch 256), so the 64-bit frame
    offsets are covered here."""
    import torch

    w = configs.FULL[cfg]()
    say(f"[gpu] full workload {w.name}: {w.description}")
    results = run_gpu(w, order="longest")  # as the benchmark dispatches
    for pt, out in results:
        o = out.numpy()
        assert np.all(np.isfinite(o)), "non-finite output"
        ref = oracle_full(w, pt.step, pt.context_lens)
        err = max_err(o, ref)
        say(f"  {w.name} step {pt.step}: all {o.shape[0]} x {o.shape[1]} (seq, head) outputs, "
            f"{o.size} values, max-abs err {err:.3e} (tol {TOL[w.dtype]})")
        assert err <= TOL[w.dtype]
    del results
    torch.cuda.empty_cache()


def test_full_size_short_contexts_parity():
    """The batch-64 workload's geometry with 2,048 sequences of up to 128
    tokens, at full size in the benchmark's launch configuration: the launch
    takes the short form (two wavefronts and two heads per workgroup), and
    every output is checked against the fp64 oracle."""
    import torch

    w = configs.config2(S=2048, max_ctx=128, NB=20000)
    say(f"[gpu] full workload {w.name}: {w.description}")
    results = run_gpu(w, order="longest")
    for pt, out in results:
        o = out.numpy()
        assert np.all(np.isfinite(o)), "non-finite output"
        ref = oracle_full(w, pt.step, pt.context_lens)
        err = max_err(o, ref)
        say(f"  {w.name} step {pt.step}: all {o.shape[0]} x {o.shape[1]} (seq, head) outputs, "
            f"max-abs err {err:.3e} (tol {TOL[w.dtype]})")
        assert err <= TOL[w.dtype]
    del results
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("pt", [0, 16, 64])
def test_grouped_decode_equals_ungrouped(cfg, pt):
    """paged_attn_decode_grouped over the groups the host finds (forks of one
    prompt; singletons elsewhere) equals paged_attn_decode at the same
    partition size bit for bit (checked inside run_gpu at every attention
    point), and the oracle within tolerance. Forced 16/64-token partitions
    put the shared/own boundary inside, at and past partition edges."""
    w = configs.small(cfg)
    say(f"[gpu] {w.name}: grouped decode, partition_tokens={pt}")
    _check_against_oracle(w, run_gpu(w, partition_tokens=pt, grouped=True), f"{w.name}/grouped/P{pt}")


@pytest.mark.parametrize("cfg", [1, 2, 4, 5])
def test_dispatch_order_leaves_outputs_unchanged(cfg):
    """A random dispatch order (sequences, or groups in the grouped pass)
    gives the batch-order outputs bit for bit at the same partition size;
    longest-first with its own default partition size matches the oracle."""
    w = configs.small(cfg)
    say(f"[gpu] {w.name}: dispatch orders")
    grouped = cfg == 4
    base = run_gpu(w, partition_tokens=16, grouped=grouped)
    shuffled = run_gpu(w, partition_tokens=16, grouped=grouped, order="random")
    for (_, x), (_, y) in zip(base, shuffled):
        assert np.array_equal(x.numpy(), y.numpy())
    _check_against_oracle(w, run_gpu(w, grouped=grouped, order="longest"), f"{w.name}/longest")


def test_grouped_decode_full_size_shared_prefix():
    """The shared-prefix workload at full size, grouped as the benchmark
    runs it: bit-equal to the ungrouped pass (inside run_gpu) and every
    output against the oracle's contiguous definition."""
    import torch

    w = configs.FULL[4]()
    say(f"[gpu] full workload {w.name}, grouped: {w.description}")
    results = run_gpu(w, grouped=True, order="longest")
    for pt, out in results:
        ref = oracle_full(w, pt.step, pt.context_lens)
        err = max_err(out.numpy(), ref)
        say(f"  {w.name} grouped step {pt.step}: all {out.numel()} values, max-abs err {err:.3e}")
        assert err <= TOL[w.dtype]
    del results
    torch.cuda.empty_cache()


def test_grouped_decode_shared_prefix_wide_form():
    """The shared-prefix workload with 2,000-token prompts at 8 heads: its
    contexts (2,001-2,200 tokens) take one 4,096-token partition in the
    ordered launch, and its 256 sequences keep 1,024 workgroups at two heads
    each, so both passes run in the sixteen-wavefront form, and the grouped
    pass folds each family's shared chunks into four members' states there.
    Grouped equals ungrouped bit for bit (inside run_gpu); every output
    against the oracle's contiguous definition."""
    import torch

    w = configs.config4(prompt_len=2000, H=8)
    say(f"[gpu] {w.name}, grouped, sixteen-wavefront form: {w.description}")
    results = run_gpu(w, grouped=True, order="longest")
    for pt, out in results:
        assert 2048 < int(pt.context_lens.max()) <= 4096 and w.num_seqs * w.H // 2 >= 1024
        ref = oracle_full(w, pt.step, pt.context_lens)
        err = max_err(out.numpy(), ref)
        say(f"  {w.name} grouped step {pt.step}: all {out.numel()} values, max-abs err {err:.3e}")
        assert err <= TOL[w.dtype]
    del results
    torch.cuda.empty_cache()


def test_grouped_decode_edge_groups():
    """Hand-built groups: members whose context is all shared but for a few
    tokens past the last whole chunk, a member with an empty context, a
    claimed shared length longer than the shortest member, a shared length
    that is not a whole chunk, groups of 1 to 4. Checked against the
    oracle's paged decode and, bit for bit, against paged_attn_decode."""
    import torch

    import paged_kv_cache_126_amd as pkv
    from tests.gpu_support import oracle_default

    dev = torch.device("cuda:0")
    H, D, B, NB = 3, 64, 16, 64
    dtype = "bf16"
    rng = np.random.default_rng(77)
    ids = np.arange(NB * B, dtype=np.int64)
    k = V.draw_np(5, V.STREAM_K, ids, H, D, dtype).reshape(NB, B, H, D)
    v = V.draw_np(5, V.STREAM_V, ids, H, D, dtype).reshape(NB, B, H, D)
    base = rng.permutation(NB)[:12].astype(np.int32)
    rows, ctx = [], []
    # group A: 3 members, identical tables, identical contexts (all shared)
    for _ in range(3):
        rows.append(base.copy()); ctx.append(100)
    # group B: 4 members sharing 5 frames, own tails of different lengths
    for i in range(4):
        r = base.copy(); r[5:] = rng.permutation(NB)[:7]; rows.append(r); ctx.append([90, 81, 150, 80][i])
    # group C: 2 members, one with an empty context
    rows.append(base.copy()); ctx.append(37)
    rows.append(base.copy()); ctx.append(0)
    # group D: a single sequence
    rows.append(rng.permutation(NB)[:12].astype(np.int32)); ctx.append(191)
    tables = np.stack(rows).astype(np.int32)
    ctx = np.asarray(ctx, dtype=np.int32)
    S = len(ctx)
    group_start = np.array([0, 3, 7, 9, 10], dtype=np.int32)
    # claimed shared tokens: A all (more than the context: cut to it), B 5
    # frames minus 3 tokens (not a whole chunk), C 40 (cut to 0), D 0
    group_shared = np.array([1000, 5 * B - 3, 40, 0], dtype=np.int32)
    q = V.draw_np(6, V.STREAM_Q, np.arange(S, dtype=np.int64), H, D, dtype)
    scale = D ** -0.5
    ref = oracle_default().paged_decode(q, k, v, tables, ctx, B, scale, dtype)
    # bf16 values travel as their 16-bit patterns
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
                  for x in (q, k, v))
    bt = torch.from_numpy(tables).to(dev)
    cl = torch.from_numpy(ctx).to(dev)
    for pt in (0, 16, 48):
        out = torch.full((S, H, D), float("nan"), dtype=torch.float32, device=dev)
        shape = pkv.lib.make_shape(tq, tk, bt, int(ctx.max()), pkv.lib.PA_F32, pt)
        ws = pkv.alloc_workspace(shape, dev)
        P = pkv.partition_tokens(shape)
        pkv.paged_attn_decode_grouped(tq, tk, tv, bt, cl, B, scale, out, int(ctx.max()),
                                      torch.from_numpy(group_start).to(dev),
                                      torch.from_numpy(group_shared).to(dev), ws, pt)
        two = torch.full_like(out, float("nan"))
        pkv.paged_attn_decode(tq, tk, tv, bt, cl, B, scale, two, int(ctx.max()), ws, pt)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.array_equal(o, two.cpu().numpy()), pt
        err = max_err(o, ref)
        say(f"  edge groups P{P}: max-abs err {err:.3e}")
        assert err <= TOL[dtype]


def test_kv_append_bit_exact_with_cow():
    """The whole device cache (written by kv_append, copy-on-write copies
    included, NaN poison elsewhere) equals the oracle's host scatter, bit for bit."""
    from oracle import blockmgr as obm

    for w in (configs.small(4), configs.small(1), configs.small(5)):
        say(f"[gpu] kv_append bit-exact on {w.name}")
        results, cache = run_gpu(w, keep_cache=True)
        snap = obm.replay(w, pad_frame=pad_frame_for(w))[0][-1]
        k, v = oracle_caches(w, snap)
        view = np.int32 if w.dtype == "f32" else np.int16
        import torch

        tview = torch.int32 if w.dtype == "f32" else torch.int16
        assert np.array_equal(cache.k.view(tview).cpu().numpy(), k.view(view))
        assert np.array_equal(cache.v.view(tview).cpu().numpy(), v.view(view))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_kv_append_skips_padding_and_out_of_range_slots(dtype):
    """Tokens whose slot is negative (padding) or past the pool's last slot
    write nothing; the rest land bit for bit where the oracle's scatter puts
    them, and every other slot keeps its previous bytes (the oracle is given
    the out-of-range slots as padding, the rule the library documents)."""
    import torch

    import paged_kv_cache_126_amd as pkv
    from oracle.oracle import default

    rng = np.random.default_rng(90)
    NB, B, H, D, N = 9, 4, 2, 64, 24
    slots = np.empty(N, dtype=np.int64)
    slots[:20] = rng.permutation(NB * B)[:20]
    slots[20:] = [-1, -7, NB * B, NB * B + 1000]
    slots = slots[rng.permutation(N)]
    kn = V.draw_np(90, V.STREAM_K, np.arange(N), H, D, dtype)
    vn = V.draw_np(90, V.STREAM_V, np.arange(N), H, D, dtype)
    base_k = V.draw_np(91, V.STREAM_K, np.arange(NB * B), H, D, dtype).reshape(NB, B, H, D)
    base_v = V.draw_np(91, V.STREAM_V, np.arange(NB * B), H, D, dtype).reshape(NB, B, H, D)
    ref_k, ref_v = base_k.copy(), base_v.copy()
    default().kv_append(kn, vn, np.where(slots < NB * B, slots, -1), ref_k, ref_v, B, dtype)

    view = np.int32 if dtype == "f32" else np.int16
    tview = torch.int32 if dtype == "f32" else torch.int16
    tdt = V.torch_dtype(dtype)
    dev = torch.device("cuda:0")

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(view)).to(dev).view(tdt)

    k, v = to_dev(base_k), to_dev(base_v)
    say(f"[gpu] kv_append with padding and out-of-range slots, {dtype}: {slots.tolist()}")
    pkv.kv_append(to_dev(kn), to_dev(vn), torch.from_numpy(slots).to(dev), k, v)
    torch.cuda.synchronize()
    assert np.array_equal(k.view(tview).cpu().numpy(), ref_k.view(view))
    assert np.array_equal(v.view(tview).cpu().numpy(), ref_v.view(view))
    assert not np.array_equal(ref_k.view(view), base_k.view(view))  # something was written


def test_gather_bit_exact():
    """Block translation: the device gather of every sequence's rows in logical
    order equals the oracle's gather, bit for bit."""
    import torch

    import paged_kv_cache_126_amd as pkv
    from oracle import blockmgr as obm
    from oracle.oracle import default

    for w in (configs.small(2), configs.small(1), configs.small(4)):
        say(f"[gpu] paged_gather on {w.name}")
        pad = pad_frame_for(w)
        results, cache = run_gpu(w, keep_cache=True)
        pt = results[-1][0]
        snap = obm.replay(w, pad_frame=pad)[0][-1]
        k, _ = oracle_caches(w, snap)
        ref = default().gather(k, snap.tables, snap.context_lens, w.B, w.dtype)
        dev = cache.k.device
        cl = pt.context_lens.astype(np.int64)
        starts = torch.from_numpy(np.concatenate([[0], np.cumsum(cl)[:-1]])).to(dev)
        out = torch.empty((int(cl.sum()), w.H, w.D), dtype=cache.k.dtype, device=dev)
        pkv.paged_gather(cache.k, torch.from_numpy(pt.tables).to(dev),
                         torch.from_numpy(pt.context_lens).to(dev), starts, out,
                         int(pt.context_lens.max()))
        torch.cuda.synchronize()
        view = torch.int32 if w.dtype == "f32" else torch.int16
        got = out.view(view).cpu().numpy()
        assert np.array_equal(got, ref.view(np.int32 if w.dtype == "f32" else np.int16))


def test_frame_permutation_is_bit_identical():
    """Another physical placement of the same logical tokens gives the same
    output bits: the kernel's arithmetic order depends only on positions."""
    w = configs.small(2)
    say(f"[gpu] {w.name}: two frame orders")
    a = run_gpu(w)
    rng = np.random.default_rng(77)
    b = run_gpu(replace(w, frame_order=rng.permutation(w.NB)))
    for (pa, x), (pb, y) in zip(a, b):
        assert not np.array_equal(pa.tables, pb.tables)
        assert np.array_equal(x.numpy(), y.numpy())


def test_shared_frames_equal_private_copies():
    """Shared-prefix tables give the same bits as private copies of the frames."""
    import torch

    import paged_kv_cache_126_amd as pkv

    w = configs.small(4)
    say(f"[gpu] {w.name}: shared prompt frames vs private copies")
    results, cache = run_gpu(w, keep_cache=True)
    pt, out_shared = results[-1]
    tables = pt.tables.copy()
    used = set(int(f) for f in tables.reshape(-1) if f >= 0)
    spare = [f for f in range(w.NB) if f not in used]
    # give every branch but the parent its own copy of each shared frame
    for s in range(w.num_seqs):
        if w.share_len is not None and w.share_len[s] > 0:
            nshared = int(w.share_len[s]) // w.B
            for b in range(nshared):
                f_new = spare.pop()
                cache.k[f_new] = cache.k[int(tables[s, b])]
                cache.v[f_new] = cache.v[int(tables[s, b])]
                tables[s, b] = f_new
    dev = cache.k.device
    q = V.draw_torch(w.seed, V.STREAM_Q, w.q_idents(pt.step), w.H, w.D, w.dtype, dev).contiguous()
    out = torch.empty((w.num_seqs, w.H, w.D), dtype=torch.float32, device=dev)
    bt = torch.from_numpy(tables).to(dev)
    cl = torch.from_numpy(pt.context_lens).to(dev)
    mc = int(pt.context_lens.max())
    shape = pkv.lib.make_shape(q, cache.k, bt, mc, 0)
    pkv.paged_attn_decode(q, cache.k, cache.v, bt, cl, w.B, w.scale, out, mc,
                          pkv.alloc_workspace(shape, dev))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), out_shared.numpy())


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_single_token_context_returns_v0_exactly(dtype):
    """ctx = 1: the weight is exactly 1, so the output is that token's V row."""
    import torch

    import paged_kv_cache_126_amd as pkv

    H, D, B, NB, S = 3, 128 if dtype != "f32" else 16, 16, 12, 5
    say(f"[gpu] ctx=1 exactness, {dtype}")
    dev = torch.device("cuda:0")
    tdt = V.torch_dtype(dtype)
    k = torch.full((NB, B, H, D), float("nan"), dtype=tdt, device=dev)
    v = torch.full_like(k, float("nan"))
    kn = V.draw_torch(9, V.STREAM_K, np.arange(S), H, D, dtype, dev).contiguous()
    vn = V.draw_torch(9, V.STREAM_V, np.arange(S), H, D, dtype, dev).contiguous()
    frames = np.array([7, 2, 9, 0, 4])
    pkv.kv_append(kn, vn, torch.from_numpy(frames * B + 0).to(dev), k, v)
    bt = torch.from_numpy(np.full((S, 2), 11, dtype=np.int32)).to(dev)
    bt[:, 0] = torch.from_numpy(frames.astype(np.int32)).to(dev)
    cl = torch.ones(S, dtype=torch.int32, device=dev)
    q = V.draw_torch(9, V.STREAM_Q, np.arange(S), H, D, dtype, dev).contiguous()
    out = torch.empty((S, H, D), dtype=torch.float32, device=dev)
    pkv.paged_attn_decode(q, k, v, bt, cl, B, D ** -0.5, out, 1)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), vn.float().cpu())


def test_zero_context_gives_zeros_and_neighbours_unaffected():
    import torch

    import paged_kv_cache_126_amd as pkv

    say("[gpu] ctx = 0 rows")
    w = configs.small(2)
    results, cache = run_gpu(w, keep_cache=True)
    pt, ref = results[-1]
    dev = cache.k.device
    cl_np = pt.context_lens.copy()
    cl_np[[1, 4]] = 0
    q = V.draw_torch(w.seed, V.STREAM_Q, w.q_idents(pt.step), w.H, w.D, w.dtype, dev).contiguous()
    out = torch.full((w.num_seqs, w.H, w.D), float("nan"), dtype=torch.float32, device=dev)
    bt = torch.from_numpy(pt.tables).to(dev)
    cl = torch.from_numpy(cl_np).to(dev)
    mc = int(pt.context_lens.max())
    shape = pkv.lib.make_shape(q, cache.k, bt, mc, 0)
    pkv.paged_attn_decode(q, cache.k, cache.v, bt, cl, w.B, w.scale, out, mc,
                          pkv.alloc_workspace(shape, dev))
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[[1, 4]] == 0)
    keep = [s for s in range(w.num_seqs) if s not in (1, 4)]
    assert np.array_equal(o[keep], ref.numpy()[keep])


def _narrow_ok(got, ref, dtype, fp32_tol=1e-5):
    """A 16-bit output rounds the fp32 result to nearest even: it must lie
    within one unit in the last place (of the 16-bit format, at the oracle's
    magnitude) plus the fp32 accumulation error of the fp64 oracle value."""
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    y = got.float().numpy().astype(np.float64)
    mant = 8 if dtype == "bf16" else 11
    mag = np.maximum(np.abs(ref), 2.0 ** -14)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - (mant - 1))
    err = np.abs(y - ref)
    assert got.dtype == tdt
    return float(np.max(err - ulp)) <= fp32_tol


@pytest.mark.parametrize("cfg", [2, 4])
def test_narrow_output_dtype_within_one_ulp(cfg):
    """A bf16/fp16 output is the fp32 result rounded to nearest even."""
    import torch

    w = configs.small(cfg)
    say(f"[gpu] {w.name}: output in {w.dtype}")
    tdt = V.torch_dtype(w.dtype)
    gpu = run_gpu(w, out_dtype=tdt)
    ref = oracle_outputs(w, pad_frame_for(w))
    for (pt, out), (_, o) in zip(gpu, ref):
        assert _narrow_ok(out, o, w.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_copy_blocks_bit_exact(dtype):
    """kv_copy_blocks copies whole frames bit for bit, leaves every other frame
    untouched and skips pairs naming a frame outside the pool. The pairs keep
    the documented contract: destinations distinct and never a source."""
    import torch

    import paged_kv_cache_126_amd as pkv

    say(f"[gpu] kv_copy_blocks, {dtype}")
    NB, B, H, D = 40, 16, 4, 128 if dtype == "bf16" else 32
    dev = torch.device("cuda:0")
    n = NB * B
    k = V.draw_torch(31, V.STREAM_K, np.arange(n), H, D, dtype, dev).reshape(NB, B, H, D).contiguous()
    v = V.draw_torch(31, V.STREAM_V, np.arange(n), H, D, dtype, dev).reshape(NB, B, H, D).contiguous()
    pairs = np.array([[3, 17], [5, 0], [39, 21], [6, 2], [3, 30], [-1, 9], [7, NB]], dtype=np.int64)
    ref_k, ref_v = k.cpu().clone(), v.cpu().clone()
    for src, dst in pairs:
        if 0 <= src < NB and 0 <= dst < NB:
            ref_k[dst] = k.cpu()[src]
            ref_v[dst] = v.cpu()[src]
    pkv.kv_copy_blocks(k, v, torch.from_numpy(pairs).to(dev))
    torch.cuda.synchronize()
    view = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(k.cpu().view(view), ref_k.view(view))
    assert torch.equal(v.cpu().view(view), ref_v.view(view))


def test_cache_policies_give_identical_bits():
    """Non-temporal and cached loads fetch the same bytes: outputs are equal."""
    from paged_kv_cache_126_amd.lib import PA_CACHE_REUSE, PA_CACHE_STREAM

    for cfg in (2, 4):
        w = configs.small(cfg)
        say(f"[gpu] {w.name}: stream vs reuse cache policy")
        a = run_gpu(w, cache_policy=PA_CACHE_STREAM)
        b = run_gpu(w, cache_policy=PA_CACHE_REUSE)
        for (_, x), (_, y) in zip(a, b):
            assert np.array_equal(x.numpy(), y.numpy())


@pytest.mark.parametrize("cfg", [6, 7])
def test_prefill_small_parity(cfg):
    """Causal multi-query attention on the matrix cores against the fp64
    oracle, every query of every sequence (ragged query and key tiles);
    dispatched in a random sequence order too, with identical bits."""
    w = configs.small(cfg)
    say(f"[gpu] prefill {w.name}: {w.description}")
    pt, qs, out = run_gpu_prefill(w, order="random")
    snap, ref = oracle_prefill(w, pad_frame_for(w))
    assert np.array_equal(pt.tables, snap.tables)
    err = max_err(out.numpy(), ref)
    say(f"  {w.name}: {int(qs[-1])} queries, max-abs err {err:.3e} (tol {TOL[w.dtype]})")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("cfg", [6, 7])
def test_prefill_full_size_parity(cfg):
    """The full prefill workloads as the benchmark dispatches them: every
    query of every sequence and head against the fp64 dense causal form over
    the sequence's logical rows (oracle/dense.py, pinned against the C
    oracle)."""
    w = configs.FULL[cfg]()
    say(f"[gpu] prefill {w.name}: {w.description}")
    pt, qs, out = run_gpu_prefill(w, order="cost")  # as the benchmark dispatches
    o = out.numpy()
    assert np.all(np.isfinite(o))
    ref = oracle_prefill_full(w, pt.context_lens)
    err = max_err(o, ref)
    say(f"  {w.name}: all {o.shape[0]} queries x {w.H} heads, {o.size} values, max-abs err {err:.3e} "
        f"(tol {TOL[w.dtype]})")
    assert err <= TOL[w.dtype]


def test_prefill_split_weights():
    """split_weights = 1 keeps V in bf16 and enters each weight as a bf16
    value plus its residual (~16 significant bits): within 1e-4 of the fp64
    oracle, where the default fp16 weights (11 bits) are held to the usual
    tolerance; for fp16 caches the flag changes nothing, bit for bit."""
    w = configs.small(6)
    say(f"[gpu] prefill {w.name}: split weights against fp16 weights")
    pt, qs, split = run_gpu_prefill(w, order="random", split_weights=True)
    plain = run_gpu_prefill(w)[2]
    _, ref = oracle_prefill(w, pad_frame_for(w))
    e_split, e_plain = max_err(split.numpy(), ref), max_err(plain.numpy(), ref)
    say(f"  max-abs err {e_split:.3e} split, {e_plain:.3e} fp16 weights")
    assert e_split <= 1e-4 and e_plain <= TOL[w.dtype]
    w = replace(configs.small(6), dtype="f16", name="prefill_S3_H2_C150_f16")
    a = run_gpu_prefill(w)[2]
    b = run_gpu_prefill(w, split_weights=True)[2]
    assert torch_equal_bits(a, b)


def torch_equal_bits(a, b) -> bool:
    """Bit-for-bit equality of two fp32 tensors (NaN payloads included)."""
    import torch

    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_wide_values_redone_split(D):
    """bf16 V values of magnitude 2^16 or more (and an infinity) do not fit
    fp16: every work item (query tile of one sequence, one head) that stages
    such a row redoes its tiles with split weights, so its outputs equal the
    split_weights launch's bit for bit and are within the split form's
    precision of the oracle, relative to the largest value. 65,280, the
    largest bf16 value under 2^16, fits fp16 exactly and keeps the fp16
    weights. The other items stay within the usual tolerance."""
    import torch

    import paged_kv_cache_126_amd as pkv
    from oracle.oracle import default as oracle_default

    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(4321 + D)
    B, H = 16, 4
    ctx = np.array([300, 200, 150, 40], dtype=np.int32)
    qlen = np.array([300, 72, 150, 40], dtype=np.int32)
    nblk = (ctx + B - 1) // B
    mb = int(nblk.max())
    NB = int(nblk.sum()) + 3
    frames = torch.randperm(NB, generator=gen).numpy().astype(np.int32)
    tables = np.full((len(ctx), mb), NB - 1, dtype=np.int32)
    used = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = frames[used:used + n]
        used += n
    k = torch.randn(NB, B, H, D, generator=gen).to(torch.bfloat16)
    v = torch.randn(NB, B, H, D, generator=gen).to(torch.bfloat16)

    def row(s, t):
        return int(tables[s, t // B]), t % B

    # (sequence, token, head) -> values of that V row
    wide = {(0, 5, 1): 7.0e4 * torch.randn(D, generator=gen),     # up to ~2^18
            (1, 140, 0): torch.full((D,), -65536.0),               # exactly 2^16
            (3, 10, 2): torch.full((D,), float("inf"))}
    fits = {(2, 60, 3): torch.full((D,), 65280.0)}                 # largest bf16 under 2^16
    for (s, t, h), val in {**wide, **fits}.items():
        f, o = row(s, t)
        v[f, o, h] = val.to(torch.bfloat16)
    qs = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    T = int(qs[-1])
    q = torch.randn(T, H, D, generator=gen).to(torch.bfloat16)
    scale = D ** -0.5
    say(f"[gpu] prefill wide V values: D {D}, contexts {ctx.tolist()}, queries {qlen.tolist()}")
    outs = []
    for split in (False, True):
        out = torch.full((T, H, D), float("nan"), dtype=torch.float32, device=dev)
        pkv.paged_attn_prefill(q.to(dev), k.to(dev), v.to(dev), torch.from_numpy(tables).to(dev),
                               torch.from_numpy(ctx).to(dev), torch.from_numpy(qs).to(dev), B,
                               scale, out, int(ctx.max()), int(qlen.max()), split_weights=split)
        torch.cuda.synchronize()
        outs.append(out.cpu())
    fast, split = outs
    bits = lambda x: x.contiguous().view(torch.int16).numpy().view(np.uint16)
    ref = oracle_default().paged_prefill(bits(q), bits(k), bits(v), tables, ctx, qs, B, scale, "bf16")
    for s in range(len(ctx)):
        rows = slice(int(qs[s]), int(qs[s + 1]))
        for h in range(H):
            a, b, r = fast[rows, h], split[rows, h], ref[rows, h]
            hit = [key for key in wide if key[0] == s and key[2] == h]
            if hit:
                assert torch_equal_bits(a, b), f"sequence {s} head {h} was not redone"
                if s != 3:  # the infinity makes NaNs (0 x inf) as well as infinities
                    vmax = float(wide[hit[0]].to(torch.bfloat16).float().abs().max())
                    err = float(np.max(np.abs(a.numpy() - r)))
                    say(f"  sequence {s} head {h}: redone, max-abs err {err:.3e} (values up to {vmax:.3g})")
                    assert err <= 1e-4 * vmax
            else:
                err = float(np.max(np.abs(a.numpy() - r)))
                big = any(key[0] == s and key[2] == h for key in fits)
                tol = TOL["bf16"] * (65280.0 if big else 1.0)
                assert err <= tol, f"sequence {s} head {h}: {err:.3e}"
                if big:
                    say(f"  sequence {s} head {h}: 65280 rows kept fp16 weights, max-abs err {err:.3e}")
                    assert not torch_equal_bits(a, b)


def test_binding_rejects_malformed_orders():
    """The binding checks an order's dtype and length before anything is
    launched: a prefill work order must be int32 [S * ceil(max_query_len /
    PA_PREFILL_TILE)], a decode dispatch order a 1-D int32 tensor."""
    import torch

    import paged_kv_cache_126_amd as pkv

    dev = torch.device("cuda:0")
    S, H, D, B, NB, mq = 3, 2, 128, 16, 8, 200
    q = torch.zeros((S * mq, H, D), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((NB, B, H, D), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((S, 16), dtype=torch.int32, device=dev)
    cl = torch.full((S,), mq, dtype=torch.int32, device=dev)
    qs = torch.arange(0, (S + 1) * mq, mq, dtype=torch.int32, device=dev)
    out = torch.zeros((S * mq, H, D), dtype=torch.float32, device=dev)
    items = S * -(-mq // pkv.PA_PREFILL_TILE)
    args = (q, k, k, bt, cl, qs, B, 0.088, out, mq, mq)
    with pytest.raises(TypeError):
        pkv.paged_attn_prefill(*args, work_order=torch.arange(S, dtype=torch.int32, device=dev))
    with pytest.raises(TypeError):
        pkv.paged_attn_prefill(*args, work_order=torch.arange(items, dtype=torch.int64, device=dev))
    qd = torch.zeros((S, H, D), dtype=torch.bfloat16, device=dev)
    od = torch.zeros((S, H, D), dtype=torch.float32, device=dev)
    with pytest.raises(TypeError):
        pkv.paged_attn_decode(qd, k, k, bt, cl, B, 0.088, od, mq,
                              dispatch_order=torch.arange(S, dtype=torch.int64, device=dev))
    torch.cuda.synchronize()


@pytest.mark.parametrize("split", [False, True])
def test_prefill_narrow_output_rounds_the_fp32_result(split):
    """Prefill with a bf16 output: the same launch's fp32 result rounded to
    nearest even, bit for bit, and so within the fp32 result's error plus half
    a bf16 unit of the oracle. With split weights the fp32 result is within
    the oracle's fp32 accumulation error, so the bf16 output is within one
    unit of the oracle."""
    import torch

    w = configs.small(6)
    say(f"[gpu] prefill {w.name}: bf16 output, split weights {split}")
    out = run_gpu_prefill(w, out_dtype=torch.bfloat16, split_weights=split)[2]
    wide = run_gpu_prefill(w, split_weights=split)[2]
    assert torch.equal(out.view(torch.int16), wide.to(torch.bfloat16).view(torch.int16))
    _, ref = oracle_prefill(w, pad_frame_for(w))
    if split:
        assert _narrow_ok(out, ref, w.dtype)
    else:
        half_ulp = np.abs(ref) * 2.0 ** -8 + 2.0 ** -133
        assert np.all(np.abs(out.float().numpy() - ref) <= TOL[w.dtype] + half_ulp)


@pytest.mark.parametrize("dtype,D,B", [("f16", 128, 16), ("bf16", 128, 16), ("f16", 64, 8),
                                       ("bf16", 64, 32)])
def test_prefill_constant_values_reproduced(dtype, D, B):
    """Every value row of head h equal to one vector c_h: each output is a
    convex combination of identical rows, so it equals c_h whatever the
    softmax weights are (a property of the definition, no oracle needed).
    The bound (5e-5, fp32 accumulation over up to 700 keys) fails if l sums
    other weights than the ones applied to the rows: a query that sees a
    few keys would then be off by a rounding of its weights, up to 2^-11
    (fp16) or 2^-9 (bf16) relative."""
    import torch

    import paged_kv_cache_126_amd as pkv

    dev = torch.device("cuda:0")
    tdt = V.torch_dtype(dtype)
    gen = torch.Generator().manual_seed(1234 + D + B)
    H = 4
    ctx = np.array([1, 2, 3, 33, 300, 700], dtype=np.int32)
    nblk = (ctx + B - 1) // B
    mb = int(nblk.max())
    NB = int(nblk.sum()) + 3
    frames = torch.randperm(NB, generator=gen).numpy().astype(np.int32)
    tables = np.full((len(ctx), mb), NB - 1, dtype=np.int32)
    used = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = frames[used:used + n]
        used += n
    k = torch.randn(NB, B, H, D, generator=gen).to(tdt).to(dev)
    c = torch.randn(H, D, generator=gen).to(tdt)
    v = c.reshape(1, 1, H, D).expand(NB, B, H, D).contiguous().to(dev)
    qs = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    T = int(qs[-1])
    q = torch.randn(T, H, D, generator=gen).to(tdt).to(dev)
    out = torch.full((T, H, D), float("nan"), dtype=torch.float32, device=dev)
    say(f"[gpu] prefill constant values: {dtype}, D {D}, block {B}, contexts {ctx.tolist()}")
    pkv.paged_attn_prefill(q, k, v, torch.from_numpy(tables).to(dev), torch.from_numpy(ctx).to(dev),
                           torch.from_numpy(qs).to(dev), B, D ** -0.5, out, int(ctx.max()),
                           int(ctx.max()))
    torch.cuda.synchronize()
    err = float((out.cpu() - c.float().reshape(1, H, D)).abs().max())
    say(f"  {T} queries, max-abs deviation from the value row {err:.3e}")
    assert err <= 5e-5


def test_prefix_cache_small_parity():
    """Prefix caching across rounds of requests: each round writes only the
    positions its requests do not reuse, prefills them through tables that
    point at cached frames, then generates tokens with decode steps (blocks
    the generated tokens fill are cached for later rounds). Tables and caches
    bit for bit, prefill and decode outputs within tolerance, against the
    oracle's own prefix cache and scatter."""
    import torch

    w = configs.small(8)
    say(f"[gpu] prefix cache {w.name}: {w.description}")
    gpu = run_gpu_prefix(w, snapshot_caches=True)
    ref = oracle_prefix_rounds(w)
    tview = torch.int32 if w.dtype == "f32" else torch.int16
    view = np.int32 if w.dtype == "f32" else np.int16
    for r, ((rd, out, (k, v), douts), (ord_, qs, oref, (ok, ov), drefs)) in enumerate(zip(gpu, ref)):
        assert rd.seqs == ord_.seqs
        assert np.array_equal(rd.tables, ord_.tables) and np.array_equal(rd.reused, ord_.reused)
        assert np.array_equal(rd.query_start, qs)
        assert np.array_equal(k.view(tview).numpy(), ok.view(view))
        assert np.array_equal(v.view(tview).numpy(), ov.view(view))
        err = max_err(out.numpy(), oref)
        assert len(douts) == len(drefs) == len(ord_.decode)
        derr = 0.0
        for st, pt, d, dr in zip(rd.decode, ord_.decode, douts, drefs):
            assert np.array_equal(st.tables, pt.tables)
            assert np.array_equal(st.context_lens, pt.context_lens)
            derr = max(derr, max_err(d.numpy(), dr))
        say(f"  round {r}: {len(rd.seqs)} requests, {int(rd.reused.sum())} of "
            f"{int(rd.context_lens.sum())} tokens reused, prefill max-abs err {err:.3e}, "
            f"{len(douts)} decode steps, max-abs err {derr:.3e}")
        assert err <= TOL[w.dtype] and derr <= TOL[w.dtype]
    assert any(g[0].reused.any() for g in gpu)


def test_prefix_cache_matches_uncached_run():
    """The same rounds without caching (every prompt written and queried in
    full) give the same outputs at the positions the cached run queries."""
    w = configs.small(8)
    say(f"[gpu] prefix cache {w.name}: cached vs uncached")
    a = run_gpu_prefix(w)
    b = run_gpu_prefix(w, caching=False, pool_frames=w.frames_without_caching)
    ref = oracle_prefix_rounds(w, caching=False, pool_frames=w.frames_without_caching)
    for (ra, oa, _, da), (rb, ob, _, db), (_, qs_ref, oref, _, dref) in zip(a, b, ref):
        assert not rb.reused.any()
        assert max_err(ob.numpy(), oref) <= TOL[w.dtype]
        for x, y, z in zip(da, db, dref):  # decode steps: cached, uncached, oracle
            assert max_err(x.numpy(), z) <= TOL[w.dtype] and max_err(y.numpy(), z) <= TOL[w.dtype]
        for i in range(len(ra.seqs)):
            lo = int(ra.reused[i])
            n = int(ra.context_lens[i]) - lo
            x = oa.numpy()[ra.query_start[i]:ra.query_start[i] + n]
            y = ob.numpy()[rb.query_start[i] + lo:rb.query_start[i] + lo + n]
            assert max_err(x, y) <= TOL[w.dtype]


def test_prefix_cache_full_size_parity():
    """The full workload (64 conversations over 8 system prompts, 4 rounds
    of prompts and generated tokens, frames evicted under pool pressure):
    every prefill output of every round and every decode output of every
    decode step, against the fp64 dense causal form over each
    conversation's tokens."""
    w = configs.FULL[8]()
    say(f"[gpu] prefix cache {w.name}: {w.description}")
    gpu = run_gpu_prefix(w)
    for r, (rd, out, _, douts) in enumerate(gpu):
        o = out.numpy()
        assert np.all(np.isfinite(o))
        pre, dec = oracle_prefix_full(w, rd)
        err = max_err(o, pre)
        derr = max((max_err(d.numpy(), x) for d, x in zip(douts, dec)), default=0.0)
        say(f"  round {r}: {int(rd.reused.sum())} of {int(rd.context_lens.sum())} tokens reused, "
            f"{o.size} prefill values max-abs err {err:.3e}; {len(douts)} decode steps max-abs err "
            f"{derr:.3e}")
        assert err <= TOL[w.dtype] and derr <= TOL[w.dtype]


def test_kernel_timing_events_leave_results_unchanged():
    """Launches stamped with kernel-timing events give the same bits as plain
    launches, and the stamps bracket a positive duration inside the
    stream-recorded events around the call."""
    import torch

    import paged_kv_cache_126_amd as pkv

    w = configs.small(2)
    say(f"[gpu] {w.name}: kernel-timing events")
    res, cache = run_gpu(w, keep_cache=True)
    pt = res[-1][0]
    dev = cache.k.device
    q = V.draw_torch(w.seed, V.STREAM_Q, w.q_idents(pt.step), w.H, w.D, w.dtype, dev).contiguous()
    out = torch.empty((w.num_seqs, w.H, w.D), dtype=torch.float32, device=dev)
    bt = torch.from_numpy(pt.tables).to(dev)
    cl = torch.from_numpy(pt.context_lens).to(dev)
    max_ctx = int(pt.context_lens.max())
    ws = pkv.alloc_workspace(pkv.lib.make_shape(q, cache.k, bt, max_ctx, pkv.lib.PA_F32, 0,
                                                pt.cache_policy), dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    with pkv.kernel_timing(ev[1], ev[2]):
        pkv.paged_attn_decode(q, cache.k, cache.v, bt, cl, w.B, w.scale, out, max_ctx, ws,
                              cache_policy=pt.cache_policy)
    ev[3].record()
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), res[-1][1].numpy())
    outer = ev[0].elapsed_time(ev[3])
    inner = ev[1].elapsed_time(ev[2])
    say(f"  stream events {outer * 1e3:.1f} us, kernel stamps {inner * 1e3:.1f} us")
    assert 0 < inner <= outer


@pytest.mark.parametrize("make", [
    lambda: configs.config2(S=8, H=4, NB=2000, seed=101),
    lambda: configs.config2(S=8, H=4, NB=2000, seed=102),
    lambda: configs.config5(S=24, H=4, NB=4000, seed=101),
    lambda: configs.config5(S=24, H=4, NB=4000, seed=102),
    lambda: configs.config5(S=24, H=4, NB=4000, permuted=True),
], ids=["cfg2_seed101", "cfg2_seed102", "cfg5_seed101", "cfg5_seed102", "cfg5_permuted"])
def test_robustness_seeds_and_permuted_pool(make):
    """The decode workloads under other seeds (structure and values) and the
    batch-256 step on a permuted pool: element-wise against the oracle."""
    w = make()
    say(f"[gpu] {w.name}: {w.description}")
    gpu = run_gpu(w)
    ref = oracle_outputs(w, pad_frame_for(w))
    for (pt, out), (snap, o) in zip(gpu, ref):
        assert np.array_equal(pt.tables, snap.tables)
        err = max_err(out.numpy(), o)
        say(f"  max-abs err {err:.3e}")
        assert err <= TOL[w.dtype]


def test_frame_read_probe_runs_and_leaves_sink():
    """The frame-pattern probe reads a buffer of frames in a given order in
    the three patterns the bench times (one head's rows of a token-major
    frame, one head's rows of a head-major frame, whole frames), touching
    nothing else; its launch-event stamps bracket a positive duration."""
    import torch

    import paged_kv_cache_126_amd as pkv

    dev = torch.device("cuda:0")
    B, H, row = 16, 8, 256
    frame = B * H * row
    n = 300
    buf = torch.ones(n * frame // 2, dtype=torch.int16, device=dev)
    order = torch.from_numpy(np.random.default_rng(3).permutation(n).astype(np.int32)).to(dev)
    sink = torch.full((1,), 12345, dtype=torch.int32, device=dev)
    patterns = [(H, row, B, H * row, row, 32), (H, B * row, B, row, row, 32), (1, 0, B * H, row, row, 4)]
    for groups, gs, pieces, ps, pb, fpu in patterns:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with pkv.kernel_timing(e0, e1):
            pkv.lib.frame_read(buf, order, frame, groups, gs, pieces, ps, pb, fpu, sink)
        torch.cuda.synchronize()
        assert e0.elapsed_time(e1) > 0
    assert int(sink.item()) == 12345


def test_stream_read_probe_runs_and_leaves_sink():
    """The streaming-read probe reads the whole buffer without touching
    anything else (its sink stays as it was for ordinary data)."""
    import torch

    import paged_kv_cache_126_amd as pkv

    dev = torch.device("cuda:0")
    for n in (16, 4096 * 16 + 48, 1 << 24):
        buf = torch.ones(n // 2, dtype=torch.int16, device=dev)
        sink = torch.full((1,), 7, dtype=torch.int32, device=dev)
        pkv.lib.stream_read(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) == 7


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_graph_capture_replays_equal_eager(cfg):
    """A decode step (kv_append + partition + merge; grouped on the
    shared-prefix workload) captured in a HIP graph: every replay, with
    eager launches and synchronisations in between, equals the eager
    result bit for bit. The library's launches allocate nothing and set no
    memory, so capture needs nothing special."""
    import torch

    import paged_kv_cache_126_amd as pkv
    from paged_kv_cache_126_amd.driver import share_groups

    w = configs.small(cfg)
    say(f"[gpu] graph capture, {w.name}")
    res, cache = run_gpu(w, keep_cache=True)
    pt, _ = res[-1]
    dev = torch.device("cuda:0")
    q = V.draw_torch(w.seed, V.STREAM_Q, w.q_idents(pt.step), w.H, w.D, w.dtype, dev).contiguous()
    bt = torch.from_numpy(pt.tables).to(dev)
    cl = torch.from_numpy(pt.context_lens).to(dev)
    mc = int(pt.context_lens.max())
    out = torch.zeros((w.num_seqs, w.H, w.D), dtype=torch.float32, device=dev)
    shape = pkv.lib.make_shape(q, cache.k, bt, mc, pkv.lib.PA_F32, 16)  # forced splits: merge runs
    ws = pkv.alloc_workspace(shape, dev)
    gs, gsh = share_groups(pt.tables, pt.context_lens, w.B)
    gsd, gshd = torch.from_numpy(gs).to(dev), torch.from_numpy(gsh).to(dev)
    # rewrite the last rows of every sequence (idempotent) as the step's append
    last = np.array([int(pt.tables[s, (c - 1) // w.B]) * w.B + (c - 1) % w.B
                     for s, c in enumerate(pt.context_lens.tolist()) if c > 0], dtype=np.int64)
    k_new = cache.k.reshape(-1, w.H, w.D)[torch.from_numpy(last).to(dev)].contiguous()
    v_new = cache.v.reshape(-1, w.H, w.D)[torch.from_numpy(last).to(dev)].contiguous()
    slots = torch.from_numpy(last).to(dev)

    def step():
        pkv.kv_append(k_new, v_new, slots, cache.k, cache.v)
        if (gsh > 0).any():
            pkv.paged_attn_decode_grouped(q, cache.k, cache.v, bt, cl, w.B, w.scale, out, mc, gsd,
                                          gshd, ws, 16)
        else:
            pkv.paged_attn_decode(q, cache.k, cache.v, bt, cl, w.B, w.scale, out, mc, ws, 16)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        other = torch.zeros_like(out)
        pkv.paged_attn_decode(q, cache.k, cache.v, bt, cl, w.B, w.scale, other, mc, ws, 16)
        torch.cuda.synchronize()
        assert torch.equal(other, ref)
    del g
