"""Pins of a prefix-cache module (the oracle's :mod:`oracle.prefixcache`, or
a copy with a planted mistake). Each ``pin_*`` takes the module, which
exposes ``PrefixCache`` and ``replay_rounds``.

The hand-worked example below was executed by hand from the rules stated in
the oracle's header (full-prefix keys, longest leading run, one reference
held by the cache, oldest-latest-event eviction, all-or-nothing requests).
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import blockmgr as obm
from workloads import configs

# 6 frames handed out 0..5, B = 2. Each step: ("start", request, tokens,
# expected reused tokens, expected table), with MemoryError for a request
# that must fail and change nothing, or ("end", request).
HAND_STEPS = [
    ("start", "A", [1, 2, 3, 4, 5], 0, [0, 1, 2]),   # cold; (1,2)->0, (1,2,3,4)->1 cached
    ("start", "B", [1, 2, 3, 9], 2, [0, 3]),         # first block reused; (1,2,3,9)->3
    ("end", "A"),                                    # 1 stays cached, 2 is freed
    ("start", "F", [3, 4, 5, 6], 0, [4, 5]),         # (3,4) equals block 1 of A but not its prefix
    ("start", "G", [1, 2, 3, 4, 8], 4, [0, 1, 2]),   # reuses A's frames, one of them idle
    ("start", "H", [5, 5, 5], MemoryError, None),    # nothing free, nothing evictable
    ("end", "B"),
    ("end", "F"),                                    # 3, 4 and 5 idle in the cache
    ("start", "H", [5, 5, 5], 0, [3, 4]),            # evicts 3 (oldest), then 4
    ("end", "G"),
    ("end", "H"),
    ("start", "J", [3, 4, 5, 6, 7], 0, [2, 4, 5]),   # (3,4) gone: no reuse although (3,4,5,6)
                                                     # is cached; evicts 5, not 0 (0 was reused
                                                     # after 5 was cached)
]
HAND_EVICTED = [3, 4, 5]
HAND_FINAL = {0: (1, 2), 1: (1, 2, 3, 4), 3: (5, 5), 2: (3, 4), 4: (3, 4, 5, 6)}


def _users(pc) -> dict:
    return {f: int(n) for f, n in enumerate(pc.pg.users)}


def check_invariants(pc, slot_ident=None):
    """Reference counts = table uses + one for the cache; the free list and
    the referenced frames partition the pool; cached prefixes are whole
    blocks; a cached frame's slots hold the last block of its prefix."""
    uses = {f: 0 for f in range(pc.pg.num_frames)}
    for t in pc.tables.values():
        for f in t:
            uses[f] += 1
    for f in pc.prefix_of_frame:
        uses[f] += 1
    assert uses == _users(pc), "reference counts"
    free = list(pc.pg.free)
    assert len(set(free)) == len(free)
    assert set(free) == {f for f, n in uses.items() if n == 0}, "free list"
    for prefix, f in pc.frame_of_prefix.items():
        assert pc.prefix_of_frame[f] == prefix and len(prefix) % pc.B == 0, "cache keys"
        if slot_ident is not None:
            assert list(slot_ident[f * pc.B:(f + 1) * pc.B]) == list(prefix[-pc.B:]), "content"


def pin_hand_worked_example(mod):
    pc = mod.PrefixCache(6, 2)
    for st in HAND_STEPS:
        if st[0] == "end":
            pc.end_request(st[1])
            continue
        _, sid, toks, reused, table = st
        if reused is MemoryError:
            before = (_users(pc), list(pc.pg.free), dict(pc.frame_of_prefix),
                      dict(pc.last_event))
            try:
                pc.start_request(sid, toks)
            except MemoryError:
                pass
            else:
                raise AssertionError(f"{sid} should not fit")
            after = (_users(pc), list(pc.pg.free), dict(pc.frame_of_prefix),
                     dict(pc.last_event))
            assert before == after, "a failed request changed the state"
            continue
        got = pc.start_request(sid, toks)
        assert got == reused, (sid, got)
        assert pc.tables[sid] == table, (sid, pc.tables[sid])
        check_invariants(pc)
    assert pc.evicted == HAND_EVICTED, pc.evicted
    assert list(pc.pg.free) == []
    assert {f: p for p, f in pc.frame_of_prefix.items()} == HAND_FINAL


def random_ops(seed, n_ops=400, fork=False):
    """A random stream of request starts, token appends, request ends and
    (with ``fork``) branches, over a vocabulary of 1 to 3 tokens, B in 1..3,
    a pool of 3 to 11 frames."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    NB = int(rng.integers(3, 12))
    vocab = int(rng.integers(1, 4))
    ops, live = [], []
    for i in range(n_ops):
        u = rng.random()
        if u < 0.4 or not live:
            ops.append(("start", i, rng.integers(0, vocab, size=int(rng.integers(0, 4 * B + 2))).tolist()))
            live.append(i)
        elif u < 0.7:
            ops.append(("append", live[int(rng.integers(0, len(live)))], int(rng.integers(0, vocab))))
        elif u < 0.8 and fork:
            ops.append(("fork", live[int(rng.integers(0, len(live)))], i))
            live.append(i)
        else:
            ops.append(("end", live.pop(int(rng.integers(0, len(live))))))
    return B, NB, ops


def pin_random_streams_keep_invariants(mod):
    """Under random streams (half of them with branches): the invariants hold
    after every step, every reused position already holds the request's own
    token, every position of every live request reads back its own token
    through its table (so a copy-on-write copied what it had to), and a
    failed start or append leaves the state as it was."""
    for seed in range(24):
        B, NB, ops = random_ops(seed, fork=seed % 2 == 1)
        pc = mod.PrefixCache(NB, B)
        slot_ident = np.full(NB * B, -1, dtype=np.int64)
        for op in ops:
            state = (_users(pc), list(pc.pg.free))
            try:
                if op[0] == "start":
                    k = pc.start_request(op[1], op[2])
                    assert k % B == 0 and k <= len(op[2])
                    pos = np.arange(len(op[2]))
                    slots = pc.slots(op[1], pos)
                    toks = np.asarray(op[2], dtype=np.int64)
                    assert np.array_equal(slot_ident[slots[:k]], toks[:k]), "reused wrong content"
                    slot_ident[slots[k:]] = toks[k:]
                elif op[0] == "append" and op[1] in pc.tables:
                    slot, copied = pc.append(op[1], op[2])
                    if copied is not None:
                        src, dst = copied
                        slot_ident[dst * B:(dst + 1) * B] = slot_ident[src * B:(src + 1) * B]
                    slot_ident[slot] = op[2]
                elif op[0] == "fork" and op[1] in pc.tables:
                    pc.fork(op[1], op[2])
                elif op[0] == "end" and op[1] in pc.tables:
                    pc.end_request(op[1])
            except MemoryError:
                assert state == (_users(pc), list(pc.pg.free))
            check_invariants(pc, slot_ident)
            for sid, toks in pc.tokens.items():
                got = slot_ident[pc.slots(sid, np.arange(len(toks)))]
                assert np.array_equal(got, np.asarray(toks, dtype=np.int64)), ("read back", sid)


def pin_reuse_is_maximal(mod):
    """With a pool large enough that nothing is evicted, a request reuses
    every leading full block whose prefix some earlier request held."""
    rng = np.random.default_rng(5)
    B = 2
    pc = mod.PrefixCache(400, B)
    seen = set()
    for i in range(60):
        toks = rng.integers(0, 2, size=int(rng.integers(0, 12))).tolist()
        expect = 0
        while expect + B <= len(toks) and tuple(toks[:expect + B]) in seen:
            expect += B
        assert pc.start_request(i, toks) == expect, (i, toks)
        for b in range(len(toks) // B):
            seen.add(tuple(toks[:(b + 1) * B]))
        if rng.random() < 0.5:
            pc.end_request(i)
    assert not pc.evicted


def pin_caching_off_is_demand_paging(mod):
    """With the cache off, a round's prompts take ceil(L / B) frames each and
    its decode steps append by the t mod B rule: the oracle's plain block
    manager gives the same tables at every point."""
    w = configs.small(8)
    NB = w.frames_without_caching
    rounds, _ = mod.replay_rounds(w, caching=False, pool_frames=NB)
    pg = obm.new_paging(NB, w.B)
    assert any(rd.decode for rd in rounds)
    for rd in rounds:
        assert not rd.reused.any()
        for i, (c, n) in enumerate(zip(rd.seqs, rd.context_lens)):
            obm.start(pg, c, int(n))
            t = pg.table[c]
            assert list(rd.tables[i, :len(t)]) == t
        for pt in rd.decode:
            for i, c in enumerate(pt.seqs):
                obm.extend(pg, c)
            for i, c in enumerate(pt.seqs):
                t = pg.table[c]
                assert list(pt.tables[i, :len(t)]) == t and pt.context_lens[i] == pg.length[c]
        for c in rd.seqs:
            obm.finish(pg, c)


def pin_rounds_hold_every_prompt(mod):
    """After each round of the small prefix workload every position of every
    request, reused or written, prompt or generated, reads back its own
    identity through the request's table at every attention point; some
    positions are reused and some frames evicted; a later round reuses
    blocks that generated tokens completed."""
    w = configs.small(8)
    rounds, pc = mod.replay_rounds(w)
    assert any(rd.reused.any() for rd in rounds) and pc.evicted

    def check(seqs, tables, lens, slot_ident):
        for i, c in enumerate(seqs):
            pos = np.arange(int(lens[i]))
            slots = tables[i][pos // w.B].astype(np.int64) * w.B + pos % w.B
            assert np.array_equal(slot_ident[slots], w.idents(c, pos))

    reused_generated = False
    for r, rd in enumerate(rounds):
        check(rd.seqs, rd.tables, rd.context_lens, rd.slot_ident)
        for pt in rd.decode:
            check(pt.seqs, pt.tables, pt.context_lens, rd.slot_ident)
        for i, c in enumerate(rd.seqs):
            n = int(rd.context_lens[i])
            assert rd.reused[i] % w.B == 0 and rd.reused[i] <= n - n % w.B
            for k in range(r):  # a generated token of an earlier round lies in the reused blocks
                if w.active[c, k] and w.gen(c, k) > 0 and w.prompt_len(c, k) < rd.reused[i]:
                    reused_generated = True
    assert reused_generated


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

    spec = importlib.util.spec_from_file_location("mutant_prefixcache", sys.argv[1])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    failed = run_all(mod)
    for name, why in failed:
        print(name, why)
    sys.exit(len(failed))
