"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Each mutant is one plausible slip (a wrong index, a dropped term, a wrong
sign, a transposed operand). The mutated source is built in a temporary
directory and the pins run against it in a child process, so a crash also
counts as detected. The real oracle source is never modified.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
BLOCKMGR = os.path.join(ROOT, "oracle", "blockmgr.py")
PREFIXCACHE = os.path.join(ROOT, "oracle", "prefixcache.py")
DENSE = os.path.join(ROOT, "oracle", "dense.py")

C_MUTANTS = {
    "offset_in_block": ("int64_t off = i % B;", "int64_t off = (i + 1) % B;"),
    "logical_block": ("int64_t b = i / B;", "int64_t b = i / (B + 1);"),
    "head_dim_transposed": ("row_off[i] = ((f * B + off) * H + h) * D;",
                            "row_off[i] = ((f * B + off) * H) * D + h;"),
    "scale_dropped": ("a[j] = scale * dot;", "a[j] = dot;"),
    "v_read_from_k": ("acc += a[j] * load(vc, dtype, row_off[j] + e);",
                      "acc += a[j] * load(kc, dtype, row_off[j] + e);"),
    "last_token_dropped": ("attend_rows(q, ((int64_t)s * H + h) * D, k_cache, v_cache, row_off, ctx, D,",
                           "attend_rows(q, ((int64_t)s * H + h) * D, k_cache, v_cache, row_off, ctx - 1, D,"),
    "softmax_sign": ("a[j] = exp(a[j] - m);", "a[j] = exp(m - a[j]);"),
    "f16_exponent_bias": ("expo - 25", "expo - 24"),
    "f16_subnormal_scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "bf16_hidden_bit": ("(double)(128 + frac)", "(double)(frac)"),
    "append_offset_dropped": ("size_t dst = (size_t)(frame * B + off) * row_bytes;",
                              "size_t dst = (size_t)(frame * B) * row_bytes;"),
    "gather_offset": ("(const char*)cache + (size_t)(f * B + i % B) * row_bytes",
                      "(const char*)cache + (size_t)(f * B + (i + 1) % B) * row_bytes"),
    "merge_weight_dropped": ("L += exp(m[p] - M) * l[p];", "L += l[p];"),
    "query_head_transposed": ("attend_rows(q, ((int64_t)s * H + h) * D, k_cache",
                              "attend_rows(q, ((int64_t)h * S + s) * D, k_cache"),
    "dense_head_dropped": ("row_off[j] = ((seq_start[s] + j) * H + h) * D;",
                           "row_off[j] = ((seq_start[s] + j) * H) * D;"),
    "normaliser_dropped": ("out[e] = acc / z;", "out[e] = acc;"),
    "prefill_not_causal": ("row_off, pos + 1, D, scale", "row_off, ctx, D, scale"),
    "prefill_excludes_self": ("row_off, pos + 1, D, scale", "row_off, pos, D, scale"),
    "prefill_position": ("int64_t pos = ctx - n + r;", "int64_t pos = r;"),
}

PY_MUTANTS = {
    "lifo_pool": ("f = pg.free.popleft()", "f = pg.free.pop()"),
    "free_to_head": ("            pg.free.append(f)", "            pg.free.appendleft(f)"),
    "new_frame_rule": ("if t % pg.block_size == 0:", "if (t + 1) % pg.block_size == 0:"),
    "prefill_floor": ("return -(-tokens // block_size)", "return tokens // block_size"),
    "no_cow": ("if pg.users[last] > 1:", "if pg.users[last] > 99:"),
    "cow_keeps_old_user": ("            release(pg, last)\n", "            pass\n"),
    "fork_no_ref": ("        share(pg, f)\n    pg.table[child]", "        pass\n    pg.table[child]"),
    "fork_aliases_row": ("pg.table[child] = list(pg.table[parent])", "pg.table[child] = pg.table[parent]"),
    "cow_no_copy": ("slot_ident[dst * B:(dst + 1) * B] = slot_ident[src * B:(src + 1) * B]", "pass"),
    "free_ignores_refcount": ("if pg.users[f] == 0:", "if True:"),
}


# Prefix cache (oracle/prefixcache.py). A value may list several (find,
# replace) pairs for one mistake made in more than one place.
PC_MUTANTS = {
    "key_block_only": [("prefix = tuple(self.tokens[sid][:(b + 1) * self.B])",
                        "prefix = tuple(self.tokens[sid][b * self.B:(b + 1) * self.B])"),
                       ("f = self.frame_of_prefix.get(tuple(toks[:(b + 1) * B]))",
                        "f = self.frame_of_prefix.get(tuple(toks[b * B:(b + 1) * B]))")],
    "mru_eviction": ("if self.last_event[f] < self.last_event[victim]:",
                     "if self.last_event[f] > self.last_event[victim]:"),
    "reuse_not_an_event": ("share(self.pg, f)\n            self._event(f)",
                           "share(self.pg, f)"),
    "no_stop_at_miss": ("            if f is None:\n                break",
                        "            if f is None:\n                continue"),
    "cache_holds_no_ref": ("self.prefix_of_frame[frame] = prefix\n        share(self.pg, frame)",
                           "self.prefix_of_frame[frame] = prefix"),
    "partial_block_cached": ("for b in range(len(reused), len(toks) // B):",
                             "for b in range(len(reused), (len(toks) + B - 1) // B):"),
    "failure_not_atomic": ("if fresh > len(self.pg.free) + len(evictable):", "if False:"),
    "evict_in_use": ("if self.pg.users[f] == 1]", "if self.pg.users[f] >= 1]"),
    "branch_no_ref": ("        for f in self.tables[parent]:\n            share(self.pg, f)",
                      "        for f in self.tables[parent]:\n            pass"),
    "branch_no_cow": ("elif self.pg.users[row[-1]] > 1:", "elif False:"),
    "entry_replaces_existing": ("if not self.enabled or prefix in self.frame_of_prefix:",
                                "if not self.enabled:"),
}


# Dense causal attention (oracle/dense.py).
DENSE_MUTANTS = {
    "mask_excludes_own_key": ("np.arange(last)[None, :] > pos[:, None]",
                              "np.arange(last)[None, :] >= pos[:, None]"),
    "scale_dropped": ("a = scale * np.matmul(", "a = np.matmul("),
    "v_read_from_k": ("o = np.matmul(w, vh) / z", "o = np.matmul(w, kh) / z"),
    "normaliser_dropped": ("o = np.matmul(w, vh) / z", "o = np.matmul(w, vh)"),
    "first_ignored": ("pos = first + np.arange(n)", "pos = np.arange(n)"),
}


def _mutate(src_path, find, repl, dst_path):
    with open(src_path) as f:
        src = f.read()
    pairs = find if isinstance(find, list) else [(find, repl)]
    for a, b in pairs:
        assert src.count(a) == 1, f"mutation anchor not unique: {a!r}"
        src = src.replace(a, b)
    with open(dst_path, "w") as f:
        f.write(src)


def _run_c_mutant(name, tmp):
    from oracle.build import build

    find, repl = C_MUTANTS[name]
    src = os.path.join(tmp, f"{name}.c")
    lib = os.path.join(tmp, f"lib{name}.so")
    _mutate(ORACLE_C, find, repl, src)
    build(src=src, out=lib, extra=["-Wno-unused-variable", "-Wno-unused-parameter"])
    r = subprocess.run([sys.executable, "-m", "tests.oracle_pins", lib], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout + r.stderr


def _run_py_mutant(name, tmp):
    find, repl = PY_MUTANTS[name]
    dst = os.path.join(tmp, f"blockmgr_{name}.py")
    _mutate(BLOCKMGR, find, repl, dst)
    r = subprocess.run([sys.executable, "-m", "tests.blockmgr_pins", dst], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout + r.stderr


def _run_pc_mutant(name, tmp):
    m = PC_MUTANTS[name]
    find, repl = (m, None) if isinstance(m, list) else m
    dst = os.path.join(tmp, f"prefixcache_{name}.py")
    _mutate(PREFIXCACHE, find, repl, dst)
    r = subprocess.run([sys.executable, "-m", "tests.prefixcache_pins", dst], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout + r.stderr


def _run_dense_mutant(name, tmp):
    find, repl = DENSE_MUTANTS[name]
    dst = os.path.join(tmp, f"dense_{name}.py")
    _mutate(DENSE, find, repl, dst)
    r = subprocess.run([sys.executable, "-m", "tests.dense_pins", dst], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout + r.stderr


RUNNERS = {"c": _run_c_mutant, "py": _run_py_mutant, "pc": _run_pc_mutant, "dense": _run_dense_mutant}


def test_every_oracle_mutant_is_caught(tmp_path):
    tmp = str(tmp_path)
    jobs = ([("c", n) for n in C_MUTANTS] + [("py", n) for n in PY_MUTANTS]
            + [("pc", n) for n in PC_MUTANTS] + [("dense", n) for n in DENSE_MUTANTS])
    with ThreadPoolExecutor(max_workers=6) as ex:
        futs = {(k, n): ex.submit(RUNNERS[k], n, tmp) for k, n in jobs}
    survivors = []
    for (k, n), fut in futs.items():
        rc, out = fut.result()
        if rc == 0:
            survivors.append(f"{k}:{n}")
    assert not survivors, f"mutants not caught by any pin: {survivors}"


def test_unmutated_oracle_passes_pin_runner():
    from oracle.oracle import DEFAULT_LIB

    r = subprocess.run([sys.executable, "-m", "tests.oracle_pins", DEFAULT_LIB], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "tests.blockmgr_pins", BLOCKMGR], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "tests.prefixcache_pins", PREFIXCACHE], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "tests.dense_pins", DENSE], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
