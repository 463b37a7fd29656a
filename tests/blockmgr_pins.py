"""Pins of a block manager module against the pages' worked examples.

Each ``pin_*`` takes a module exposing ``new_paging``, ``start``,
``extend``, ``branch``, ``finish``, ``memory_efficiency`` and ``replay`` (the
oracle's :mod:`oracle.blockmgr`, or a copy of it with a planted mistake).
"""
from __future__ import annotations

import json
import math
import os
import sys
from dataclasses import replace

import numpy as np

from workloads import configs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pin_p3_worked_example(mod):
    g = _golden("p3_worked_example.json")
    w = replace(configs.config1(), attend_after=[-1, 0, 1, 2])
    assert w.B == g["block_size"] and w.NB == g["num_frames"]
    assert [n for _, n in w.prefill] == [g["prefill"][r] for r in g["requests"]]
    snaps, _ = mod.replay(w)
    assert len(snaps) == len(g["states"])
    for snap, state in zip(snaps, g["states"]):
        for s, r in enumerate(g["requests"]):
            want = state["tables"][r]
            table = [int(f) for f in snap.tables[s] if f >= 0]
            assert table == want, (state["after"], r, table)
            fill = [min(w.B, int(snap.context_lens[s]) - b * w.B) for b in range(len(table))]
            assert fill == state["fill"][r], (state["after"], r, fill)
            written = [int((snap.slot_ident[f * w.B:(f + 1) * w.B] >= 0).sum()) for f in table]
            assert written == state["fill"][r], (state["after"], r, written)
        fl = snap.free_list
        assert fl[:len(state["free_head"])] == state["free_head"]
        assert fl[-len(state["free_tail"]):] == state["free_tail"]
        assert len(fl) == state["free_count"]


def pin_p1_demo(mod):
    g = _golden("p1_demo.json")
    pg = mod.new_paging(g["num_frames"], g["block_size"])
    st, dv = g["stated"], g["derived"]
    mod.start(pg, "req_alpha", g["prompt_tokens"])
    assert pg.table["req_alpha"] == st["alpha_table_after_prompt"]
    assert g["num_frames"] - len(pg.free) == st["frames_allocated_by_prompt"]
    assert len(pg.free) == dv["free_after_prompt"]
    before = len(pg.free)
    mod.branch(pg, "req_alpha", "req_beta")
    assert before - len(pg.free) == st["extra_frames_used_by_fork"]
    assert pg.table["req_beta"] == dv["beta_table_after_fork"]
    assert len(pg.free) == dv["free_after_fork"]
    assert {str(k): int(pg.users[k]) for k in (0, 1)} == dv["ref_counts_after_fork"]
    assert pg.length["req_alpha"] == st["append_allocates_one_new_block_because_length_was"]
    mod.extend(pg, "req_alpha")
    assert pg.table["req_alpha"] == dv["alpha_table_after_append"]
    assert pg.table["req_beta"] == dv["beta_table_after_append"]
    assert len(pg.free) == dv["free_after_append"]
    mod.finish(pg, "req_alpha")
    mod.finish(pg, "req_beta")
    assert len(pg.free) == st["free_after_cleanup_of"] == dv["free_after_cleanup"]
    assert list(pg.free)[-5:] == dv["free_list_tail_after_cleanup"]


def pin_p2_efficiency(mod):
    g = _golden("p2_efficiency.json")
    B, n = g["block_size"], g["sequence_length"]
    pg = mod.new_paging(10, B)
    mod.start(pg, 0, n)
    blocks = len(pg.table[0])
    assert blocks == g["blocks_allocated"]
    assert blocks * B == g["slots_allocated"]
    assert blocks * B - n == g["wasted_slots"]
    tol = g["approx_abs_tolerance"]
    assert abs(mod.memory_efficiency(n, B) - g["memory_efficiency_approx"]) <= tol["memory_efficiency_approx"]
    assert abs(n / g["contiguous_prealloc_slots"] - g["contiguous_efficiency_approx"]) <= tol["contiguous_efficiency_approx"]


def pin_waste_below_one_block(mod):
    """Allocated slots minus tokens stays within [0, B - 1] (page 3's closing
    bound; page 1's 'Maximum Waste per Request')."""
    rng = np.random.default_rng(7)
    for B in (1, 3, 10, 16):
        pg = mod.new_paging(4000, B)
        lens = rng.integers(0, 60, size=12)
        for s, n in enumerate(lens):
            mod.start(pg, s, int(n))
        for _ in range(40):
            for s in range(len(lens)):
                if rng.random() < 0.6:
                    mod.extend(pg, s)
                    waste = len(pg.table[s]) * B - pg.length[s]
                    assert 0 <= waste <= B - 1, (B, s, waste)


def pin_copy_on_write(mod):
    """Appending into a shared partial frame copies that one frame only."""
    pg = mod.new_paging(20, 4)
    mod.start(pg, "p", 10)               # frames 0, 1, 2 (last holds 2 tokens)
    mod.branch(pg, "p", "c")
    assert pg.users[2] == 2 and len(pg.free) == 17
    copied = mod.extend(pg, "c")         # shared partial frame 2 -> copy into 3
    assert copied == (2, 3)
    assert pg.table["c"] == [0, 1, 3] and pg.table["p"] == [0, 1, 2]
    assert pg.users[2] == 1 and pg.users[3] == 1 and pg.users[0] == 2
    assert mod.extend(pg, "p") is None   # now private: no copy
    assert pg.table["p"] == [0, 1, 2]
    mod.extend(pg, "p")
    mod.extend(pg, "p")                  # length 12 -> new frame 4
    assert pg.table["p"] == [0, 1, 2, 4]
    mod.finish(pg, "c")                  # c's private frame 3 returns; 0, 1 keep one user
    assert list(pg.free)[-1] == 3 and pg.users[0] == 1 and pg.users[3] == 0


def pin_pool_exhaustion(mod):
    pg = mod.new_paging(3, 2)
    mod.start(pg, 0, 6)
    try:
        mod.extend(pg, 0)
    except MemoryError:
        pass
    else:
        raise AssertionError("no MemoryError when the pool is empty")
    pg = mod.new_paging(3, 2)
    try:
        mod.start(pg, 0, 7)              # four frames from a pool of three
    except MemoryError:
        assert len(pg.free) == 3 and 0 not in pg.table
    else:
        raise AssertionError("no MemoryError for a prompt larger than the pool")


def pin_replay_cow_contents(mod):
    """After replaying the shared-prefix schedule, every sequence's tokens,
    read through its table, carry the identities the schedule assigned."""
    w = configs.config4(prompts=2, n=3, prompt_len=45, H=1, NB=200, max_tail=40)
    w.B = 8
    snaps, _ = mod.replay(w)
    snap = snaps[-1]
    for s in range(w.num_seqs):
        ctx = int(snap.context_lens[s])
        pos = np.arange(ctx)
        slots = snap.tables[s][pos // w.B].astype(np.int64) * w.B + pos % w.B
        assert np.array_equal(snap.slot_ident[slots], w.idents(s, pos)), s


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

    spec = importlib.util.spec_from_file_location("mutant_blockmgr", sys.argv[1])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    failed = run_all(mod)
    for name, why in failed:
        print(name, why)
    sys.exit(len(failed))
