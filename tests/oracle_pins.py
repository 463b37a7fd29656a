"""Pins of the C oracle against things other than itself.

Each ``pin_*`` takes an :class:`oracle.oracle.Oracle` handle and raises
AssertionError when the oracle disagrees with what the pages or mathematics
fix. The tests run them on the real build; the mutation test runs them on
copies of the oracle with a planted mistake and expects at least one to fail.

Independent references used here: the pages' address formula for an
interleaved K/V frame, numpy's own float16 decoding, exact rational brute
force, closed forms of the softmax, and invariances of the definition
(frame permutation, shared versus duplicated frames, partition merging).

Run as ``python -m tests.oracle_pins <liboracle.so>`` to print the failing
pins of that build (exit status = number of failing pins).
"""
from __future__ import annotations

import math
import sys

import numpy as np

from oracle import bruteforce
from workloads.values import STREAM_K, STREAM_Q, STREAM_V, draw_np, nan_bits

STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}


def np_widen(a, dtype):
    """Decode stored values with numpy (independent of the oracle's decoders)."""
    a = np.asarray(a)
    with np.errstate(invalid="ignore"):
        return _np_widen(a, dtype)


def _np_widen(a, dtype):
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return a.astype(np.uint16).view(np.float16).astype(np.float64)
    return (a.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Case:
    """A random paged problem: frames drawn from a permuted pool, NaN poison elsewhere."""

    def __init__(self, seed, S, H, D, B, dtype, max_ctx, spare=3, min_ctx=1):
        rng = np.random.default_rng(seed)
        self.S, self.H, self.D, self.B, self.dtype = S, H, D, B, dtype
        self.ctx = rng.integers(min_ctx, max_ctx + 1, size=S).astype(np.int32)
        nblk = [(-(-int(c) // B)) for c in self.ctx]
        self.NB = sum(nblk) + spare
        perm = rng.permutation(self.NB)
        self.poison_frame = int(perm[-1])
        mb = max(max(nblk), 1)
        self.tables = np.full((S, mb), self.poison_frame, dtype=np.int32)
        shape = (self.NB, B, H, D)
        self.k = np.full(shape, nan_bits(dtype), dtype=STORAGE[dtype])
        self.v = np.full(shape, nan_bits(dtype), dtype=STORAGE[dtype])
        self.rows_k, self.rows_v = [], []
        pos = 0
        for s in range(S):
            self.tables[s, :nblk[s]] = perm[pos:pos + nblk[s]]
            pos += nblk[s]
            idents = 1000 * s + np.arange(self.ctx[s]) + seed * 100000
            kr = draw_np(seed, STREAM_K, idents, H, D, dtype)
            vr = draw_np(seed, STREAM_V, idents, H, D, dtype)
            self.rows_k.append(kr)
            self.rows_v.append(vr)
            for i in range(self.ctx[s]):
                f = self.tables[s, i // B]
                self.k[f, i % B] = kr[i]
                self.v[f, i % B] = vr[i]
        self.q = draw_np(seed, STREAM_Q, np.arange(S) + seed * 7919, H, D, dtype)
        self.scale = float(np.float32(1.0 / math.sqrt(D)))

    def decode(self, orc, **kw):
        return orc.paged_decode(self.q, self.k, self.v, self.tables, self.ctx, self.B, self.scale,
                                self.dtype, **kw)


def pin_widen_f16(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.widen(bits, "f16")
    ref = np_widen(bits, "f16")
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def pin_widen_bf16(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.widen(bits, "bf16")
    ref = np_widen(bits, "bf16")
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def pin_bruteforce(orc):
    """Exact rational / 60-digit brute force on tiny random cases, all dtypes."""
    cases = [(11, 3, 2, 8, 1, "f32", 9), (12, 2, 2, 4, 2, "f16", 24), (13, 3, 1, 8, 3, "bf16", 20),
             (14, 2, 2, 6, 4, "f32", 17), (15, 2, 2, 8, 10, "bf16", 24), (16, 2, 1, 5, 10, "f16", 23)]
    for seed, S, H, D, B, dt, mc in cases:
        c = Case(seed, S, H, D, B, dt, mc)
        out = c.decode(orc)
        kf = np_widen(c.k, dt).tolist()
        vf = np_widen(c.v, dt).tolist()
        qf = np_widen(c.q, dt)
        for s in range(S):
            for h in range(H):
                ref = bruteforce.decode_one(qf[s, h].tolist(), kf, vf, c.tables[s].tolist(),
                                            int(c.ctx[s]), h, B, c.scale)
                err = np.max(np.abs(out[s, h] - np.array(ref)))
                assert err <= 1e-14, (seed, s, h, err)


def pin_ctx1_returns_v0(orc):
    """One token: softmax weight 1, so the output is that token's V row exactly."""
    for dt in ("f32", "f16", "bf16"):
        c = Case(21, 4, 2, 16, 10, dt, 1)
        out = c.decode(orc)
        for s in range(c.S):
            assert np.array_equal(out[s], np_widen(c.rows_v[s][0], dt))


def pin_zero_query_is_mean(orc):
    """q = 0 gives equal weights: the output is the mean of the V rows."""
    c = Case(22, 3, 2, 8, 4, "f32", 40, min_ctx=5)
    c.q[:] = 0
    out = c.decode(orc)
    for s in range(c.S):
        vv = np_widen(c.rows_v[s], "f32")
        for h in range(c.H):
            for e in range(c.D):
                mean = math.fsum(vv[:, h, e]) / c.ctx[s]
                assert abs(out[s, h, e] - mean) <= 1e-15, (s, h, e)


def pin_zero_scale_is_mean(orc):
    """scale = 0 makes every score 0, so every weight is equal: the output is
    the mean of the V rows (bf16 storage, any q)."""
    c = Case(23, 3, 2, 16, 4, "bf16", 40, min_ctx=5)
    c.scale = 0.0
    out = c.decode(orc)
    for s in range(c.S):
        vv = np_widen(c.rows_v[s], "bf16")
        for h in range(c.H):
            for e in range(c.D):
                mean = math.fsum(vv[:, h, e]) / c.ctx[s]
                assert abs(out[s, h, e] - mean) <= 1e-15, (s, h, e)


def pin_negative_scale_is_negated_query(orc):
    """scale * (q . k) = (-scale) * ((-q) . k): a negative scale gives the
    output of the positive scale with q's sign flipped, bit for bit (the
    flip is exact in every storage dtype, and so are the negated products)."""
    for dtype, flip in (("bf16", 0x8000), ("f16", 0x8000), ("f32", None)):
        c = Case(24, 3, 2, 8, 4, dtype, 30)
        c.scale = -0.35
        neg = c.decode(orc)
        c.q = (-c.q if flip is None else (c.q ^ np.uint16(flip)))
        c.scale = 0.35
        pos = c.decode(orc)
        assert np.array_equal(neg, pos), dtype
        # and it is not the positive-scale output of the original q
        c.q = (-c.q if flip is None else (c.q ^ np.uint16(flip)))
        assert not np.allclose(c.decode(orc), pos), dtype


def pin_peaked_score_selects_row(orc):
    """Key j aligned with a large query dominates: output = v_j to ~e^-60."""
    c = Case(23, 2, 2, 8, 3, "f32", 30, min_ctx=6)
    for s in range(c.S):
        j = int(c.ctx[s]) // 2 + s
        for h in range(c.H):
            c.q[s, h] = 0
            c.q[s, h, 0] = 30.0
        # zero every key of this sequence, then make key j large along e=0
        for i in range(c.ctx[s]):
            f = c.tables[s, i // c.B]
            c.k[f, i % c.B] = 0
        f = c.tables[s, j // c.B]
        c.k[f, j % c.B, :, 0] = 2.0 / c.scale  # score 60 for token j, 0 elsewhere
    out = c.decode(orc)
    for s in range(c.S):
        j = int(c.ctx[s]) // 2 + s
        vj = np_widen(c.rows_v[s][j], "f32")
        assert np.max(np.abs(out[s] - vj)) <= 1e-12 * (1 + np.max(np.abs(vj)))


def _interleaved_image(c):
    """Frames laid out as the address formula on page 1 assumes:
    each token's K and V rows side by side, [NB][B][2][H][D]."""
    img = np.empty((c.NB, c.B, 2, c.H, c.D), dtype=c.k.dtype)
    img[:, :, 0] = c.k
    img[:, :, 1] = c.v
    return img.tobytes()


def pin_translation_address_formula(orc):
    """Gather through the oracle == bytes at the page-1 address formula:
    Address(K_i) = BlockTable[i // B] * FrameSize + (i mod B) * (2 * H * d * bytes),
    plus h * d * bytes for head h inside the token's K row."""
    for dt in ("f32", "bf16"):
        c = Case(31, 4, 2, 16, 10, dt, 47)
        e = 4 if dt == "f32" else 2
        img = _interleaved_image(c)
        token = 2 * c.H * c.D * e
        frame = c.B * token
        got = orc.gather(c.k, c.tables, c.ctx, c.B, dt).tobytes()
        row = c.H * c.D * e
        n = 0
        for s in range(c.S):
            for i in range(int(c.ctx[s])):
                b, o = i // c.B, i % c.B
                base = int(c.tables[s, b]) * frame + o * token
                for h in range(c.H):
                    want = img[base + h * c.D * e: base + (h + 1) * c.D * e]
                    have = got[n * row + h * c.D * e: n * row + (h + 1) * c.D * e]
                    assert want == have, (dt, s, i, h)
                n += 1
        assert n * row == len(got)


def pin_decode_reads_formula_rows(orc):
    """The attention path reads K_i and V_i at the formula's address: make only
    the K row at Address(K_i) match the query, and the output is the V row at
    the same address (up to e^-60)."""
    c = Case(32, 3, 2, 8, 10, "f32", 35, min_ctx=12)
    img = np.frombuffer(_interleaved_image(c), dtype=np.float32)
    for s in range(c.S):
        i = int(c.ctx[s]) - 1 - 3 * s
        b, o = i // c.B, i % c.B
        token = 2 * c.H * c.D
        base = int(c.tables[s, b]) * c.B * token + o * token
        kk = np.zeros((c.NB, c.B, c.H, c.D), dtype=np.float32)
        flat = kk.reshape(-1)
        # the page-1 formula addresses the interleaved image; map that K row back
        for h in range(c.H):
            addr = base + h * c.D
            fr, rem = divmod(addr, c.B * token)
            oo, rem = divmod(rem, token)
            kv, rem = divmod(rem, c.H * c.D)
            assert kv == 0
            flat[((fr * c.B + oo) * c.H) * c.D + rem: ((fr * c.B + oo) * c.H) * c.D + rem + 1] = 60.0 / c.scale
        q = np.zeros((c.S, c.H, c.D), dtype=np.float32)
        q[:, :, 0] = 1.0
        out = orc.paged_decode(q, kk, c.v, c.tables, c.ctx, c.B, c.scale, "f32")
        for h in range(c.H):
            vaddr = base + c.H * c.D + h * c.D
            want = img[vaddr: vaddr + c.D].astype(np.float64)
            assert np.max(np.abs(out[s, h] - want)) <= 1e-12 * (1 + np.max(np.abs(want))), (s, h)


def pin_frame_permutation_invariance(orc):
    """Relabelling physical frames (moving their contents along) changes nothing."""
    for dt, seed in (("f32", 41), ("bf16", 42), ("f16", 43)):
        c = Case(seed, 5, 2, 16, 4, dt, 60)
        base = c.decode(orc)
        rng = np.random.default_rng(seed)
        for _ in range(3):
            pi = rng.permutation(c.NB)
            k2 = np.empty_like(c.k)
            v2 = np.empty_like(c.v)
            k2[pi] = c.k
            v2[pi] = c.v
            t2 = pi[c.tables].astype(np.int32)
            out = orc.paged_decode(c.q, k2, v2, t2, c.ctx, c.B, c.scale, dt)
            assert np.array_equal(out, base)


def pin_shared_vs_private_frames(orc):
    """Two sequences pointing at the same prefix frames equal the same
    sequences with private copies of those frames."""
    c = Case(51, 4, 2, 8, 4, "f16", 30, spare=40, min_ctx=14)
    # sequence 1..3 share sequence 0's first 3 frames (same bytes)
    shared = c.tables.copy()
    k, v = c.k.copy(), c.v.copy()
    for s in range(1, c.S):
        for b in range(3):
            k[c.tables[s, b]] = k[c.tables[0, b]]
            v[c.tables[s, b]] = v[c.tables[0, b]]
            shared[s, b] = c.tables[0, b]
    private = orc.paged_decode(c.q, k, v, c.tables, c.ctx, c.B, c.scale, "f16")
    sharing = orc.paged_decode(c.q, k, v, shared, c.ctx, c.B, c.scale, "f16")
    assert np.array_equal(private, sharing)


def pin_paged_equals_dense(orc):
    """Paged attention equals contiguous attention over the same logical rows."""
    for dt, seed in (("bf16", 61), ("f32", 62)):
        c = Case(seed, 6, 3, 16, 16, dt, 100)
        paged = c.decode(orc)
        st = np.concatenate([[0], np.cumsum(c.ctx)]).astype(np.int64)
        dense = orc.dense_attention(c.q, np.concatenate(c.rows_k), np.concatenate(c.rows_v), st,
                                    c.scale, dt)
        assert np.max(np.abs(paged - dense)) <= 1e-12


def pin_gather_then_dense_torch(orc):
    """A structurally different second opinion ("Solving the LLM Memory Wall",
    "Implementation": the forward pass gathers each sequence's blocks
    through its table, flattens them, trims to the sequence length and runs
    ordinary scaled dot-product attention): the same computation in torch
    fp64 on the CPU, with its own widening, equals the oracle within 1e-12."""
    import torch

    for dt, seed in (("bf16", 81), ("f16", 82), ("f32", 83)):
        c = Case(seed, 5, 3, 16, 7, dt, 60)
        k_all = torch.from_numpy(np_widen(c.k, dt))
        v_all = torch.from_numpy(np_widen(c.v, dt))
        q_all = torch.from_numpy(np_widen(c.q, dt))
        want = c.decode(orc)
        for s in range(c.S):
            n = int(c.ctx[s])
            blocks = torch.from_numpy(c.tables[s, :-(-n // c.B)].astype(np.int64))
            k = k_all[blocks].reshape(-1, c.H, c.D)[:n]          # [n, H, D]
            v = v_all[blocks].reshape(-1, c.H, c.D)[:n]
            scores = torch.einsum("hd,nhd->hn", q_all[s], k) * c.scale
            o = torch.einsum("hn,nhd->hd", torch.softmax(scores, dim=-1), v)
            assert np.max(np.abs(o.numpy() - want[s])) <= 1e-12, (dt, s)


def pin_split_merge_identity(orc):
    """Partitioned attention merged by log-sum-exp equals the single pass."""
    c = Case(71, 4, 2, 8, 5, "f32", 90, min_ctx=2)
    base = c.decode(orc)
    for P in (1, 3, 7, 16, 64, 200):
        out = orc.paged_decode_split(c.q, c.k, c.v, c.tables, c.ctx, c.B, c.scale, "f32", P)
        assert np.max(np.abs(out - base)) <= 1e-12, P


def pin_kv_append_scatter(orc):
    """Host scatter == numpy fancy-index assignment; negative slots skipped."""
    for dt in ("f32", "f16", "bf16"):
        rng = np.random.default_rng(81)
        NB, B, H, D, N = 9, 4, 2, 8, 20
        slots = rng.permutation(NB * B)[:N].astype(np.int64)
        slots[[3, 11]] = -1
        kn = draw_np(81, STREAM_K, np.arange(N), H, D, dt)
        vn = draw_np(81, STREAM_V, np.arange(N), H, D, dt)
        kc = np.full((NB, B, H, D), nan_bits(dt), dtype=STORAGE[dt])
        vc = kc.copy()
        ref_k, ref_v = kc.copy(), vc.copy()
        keep = slots >= 0
        ref_k.reshape(NB * B, H, D)[slots[keep]] = kn[keep]
        ref_v.reshape(NB * B, H, D)[slots[keep]] = vn[keep]
        orc.kv_append(kn, vn, slots, kc, vc, B, dt)
        assert kc.tobytes() == ref_k.tobytes() and vc.tobytes() == ref_v.tobytes()


def pin_gather_matches_numpy(orc):
    c = Case(91, 5, 3, 8, 3, "f16", 20)
    got = orc.gather(c.v, c.tables, c.ctx, c.B, "f16")
    ref = np.concatenate(c.rows_v)
    assert got.tobytes() == ref.tobytes()


def _prefill_case(seed, S, H, D, B, dtype, max_ctx, full=False):
    c = Case(seed, S, H, D, B, dtype, max_ctx, min_ctx=1)
    rng = np.random.default_rng(seed + 1)
    n = c.ctx.copy() if full else np.array([int(rng.integers(1, k + 1)) for k in c.ctx], dtype=np.int32)
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q = draw_np(seed, STREAM_Q, np.arange(qs[-1]) + 5000 * seed, H, D, dtype)
    return c, n, qs, q


def pin_prefill_single_query_equals_decode(orc):
    """One query per sequence (its last token) is decode attention."""
    for dt in ("f32", "bf16"):
        c = Case(101, 5, 2, 16, 4, dt, 60)
        qs = np.arange(c.S + 1, dtype=np.int32)
        pre = orc.paged_prefill(c.q, c.k, c.v, c.tables, c.ctx, qs, c.B, c.scale, dt)
        dec = c.decode(orc)
        assert np.array_equal(pre, dec)


def pin_prefill_last_query_equals_decode(orc):
    """In a full prefill the last query sees the whole context: it equals decode."""
    c, n, qs, q = _prefill_case(102, 4, 2, 8, 3, "f16", 40, full=True)
    pre = orc.paged_prefill(q, c.k, c.v, c.tables, c.ctx, qs, c.B, c.scale, "f16")
    last = q[qs[1:] - 1]
    dec = orc.paged_decode(last, c.k, c.v, c.tables, c.ctx, c.B, c.scale, "f16")
    assert np.array_equal(pre[qs[1:] - 1], dec)


def pin_prefill_is_causal(orc):
    """Query at position p ignores every token after p and depends on token p."""
    c, n, qs, q = _prefill_case(103, 3, 2, 8, 4, "f32", 30, full=True)
    base = orc.paged_prefill(q, c.k, c.v, c.tables, c.ctx, qs, c.B, c.scale, "f32")
    s, p = 1, int(c.ctx[1]) // 2
    k2, v2 = c.k.copy(), c.v.copy()
    for i in range(p + 1, int(c.ctx[s])):
        f = c.tables[s, i // c.B]
        k2[f, i % c.B] = 7.0
        v2[f, i % c.B] = -3.0
    after = orc.paged_prefill(q, k2, v2, c.tables, c.ctx, qs, c.B, c.scale, "f32")
    row = qs[s] + p
    assert np.array_equal(after[:row + 1], base[:row + 1])
    assert not np.array_equal(after[row + 1:qs[s + 1]], base[row + 1:qs[s + 1]])
    k3 = c.k.copy()
    f = c.tables[s, p // c.B]
    k3[f, p % c.B] = 5.0
    moved = orc.paged_prefill(q, k3, c.v, c.tables, c.ctx, qs, c.B, c.scale, "f32")
    assert not np.array_equal(moved[row], base[row])


def pin_prefill_bruteforce(orc):
    """Every query of a chunked prefill against the rational brute force."""
    for seed, dt, B in ((104, "bf16", 3), (105, "f32", 10)):
        c, n, qs, q = _prefill_case(seed, 3, 2, 6, B, dt, 22)
        out = orc.paged_prefill(q, c.k, c.v, c.tables, c.ctx, qs, c.B, c.scale, dt)
        kf, vf, qf = np_widen(c.k, dt).tolist(), np_widen(c.v, dt).tolist(), np_widen(q, dt)
        for s in range(c.S):
            for r in range(int(n[s])):
                pos = int(c.ctx[s]) - int(n[s]) + r
                t = qs[s] + r
                for h in range(c.H):
                    ref = bruteforce.decode_one(qf[t, h].tolist(), kf, vf, c.tables[s].tolist(),
                                                pos + 1, h, c.B, c.scale)
                    assert np.max(np.abs(out[t, h] - np.array(ref))) <= 1e-14, (seed, s, r, h)


ALL = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def run_all(orc) -> list:
    failed = []
    for pin in ALL:
        try:
            pin(orc)
        except Exception as exc:  # noqa: BLE001 - any failure counts
            failed.append((pin.__name__, f"{type(exc).__name__}: {exc}"[:200]))
    return failed


if __name__ == "__main__":
    from oracle.oracle import Oracle

    failed = run_all(Oracle(sys.argv[1]))
    for name, why in failed:
        print(name, why)
    sys.exit(len(failed))
