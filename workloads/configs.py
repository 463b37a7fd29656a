"""The seeded synthetic workloads, as plain data.

Each workload is a *schedule*: which sequences are prefilled with how many
tokens, which are forked from which, which sequences append one token at each
decode step, and after which steps decode attention runs. It also fixes the
shapes, the storage dtype, the frame-pool size and the pool's initial free
order. Nothing here allocates frames or computes slots; a block manager plays
the schedule.

Token values are identified by an integer *identity* per (sequence, position):
a forked child shares its parent's identities for the shared prompt, so the
bytes it attends to are the same bytes the parent wrote. Query values are
identified by ``step * num_seqs + seq``. Values themselves come from
:mod:`workloads.values`.

The structure draws use ``numpy.random.default_rng(seed)`` with seed equal to
the workload number (1-8), in the order documented per workload.
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass, field

import numpy as np


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str                 # storage dtype of q, K and V: "f32", "f16", "bf16"
    H: int                     # heads (q heads == kv heads)
    D: int                     # head dim
    B: int                     # tokens per block
    NB: int                    # frames in the pool
    num_seqs: int
    prefill: list              # [(seq, n_tokens)] in allocation order
    forks: list = field(default_factory=list)     # [(parent, child)] after prefill
    steps: list = field(default_factory=list)     # per decode step: seqs appending, in order
    attend_after: list = field(default_factory=lambda: [-1])  # -1 = after prefill/forks
    frame_order: np.ndarray | None = None         # initial free list; None = 0..NB-1
    share_len: np.ndarray | None = None           # per seq: prompt positions shared with parent
    share_src: np.ndarray | None = None           # per seq: parent whose identities are shared
    query_lens: np.ndarray | None = None          # prefill: per seq, its last tokens that are queries
    description: str = ""
    scale_value: float | None = None              # multiplier of q . k; None = 1 / sqrt(D)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D) if self.scale_value is None else float(self.scale_value)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def ident_stride(self) -> int:
        total = {}
        for s, n in self.prefill:
            total[s] = total.get(s, 0) + n
        longest = max(total.values(), default=0) + len(self.steps) + 1
        return int(longest)

    def idents(self, seq: int, positions) -> np.ndarray:
        """Value identities of sequence ``seq`` at token ``positions``."""
        pos = np.asarray(positions, dtype=np.int64)
        out = seq * self.ident_stride + pos
        if self.share_len is not None and self.share_len[seq] > 0:
            src = int(self.share_src[seq])
            shared = pos < self.share_len[seq]
            out = np.where(shared, self.idents(src, pos), out)
        return out

    def q_idents(self, step_index: int) -> np.ndarray:
        """Query identities for the attention run ``step_index`` (0-based)."""
        return step_index * self.num_seqs + np.arange(self.num_seqs, dtype=np.int64)

    def prefill_queries(self, context_lens) -> tuple:
        """Prefill workloads: (query_start [S+1], identities [T]) of the query
        tokens, each sequence's last query_lens[s] tokens in order. A query
        token's value is drawn from the query stream under the token's own
        identity."""
        n = np.asarray(self.query_lens, dtype=np.int64)
        start = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
        ids = np.concatenate([self.idents(s, np.arange(int(c) - int(n[s]), int(c)))
                              for s, c in enumerate(np.asarray(context_lens))] or [np.zeros(0, np.int64)])
        return start, ids


def config1() -> Workload:
    """Worked allocation example: B=10, 100 frames, prefill 8/5/12/9, 3 steps."""
    return Workload(
        name="cfg1_worked_example", seed=1, dtype="f32", H=2, D=16, B=10, NB=100,
        num_seqs=4,
        prefill=[(0, 8), (1, 5), (2, 12), (3, 9)],
        steps=[[0, 1, 2, 3]] * 3,
        attend_after=[0, 1, 2],
        description="B=10, 100 frames, FIFO; prefill A:8 B:5 C:12 D:9; 3 decode steps; "
                    "2 heads x 16, fp32",
    )


def config2(S: int = 64, H: int = 32, NB: int | None = None, max_ctx: int = 2048,
            B: int = 16, seed: int = 2, D: int = 128, dtype: str = "bf16") -> Workload:
    """Decode batch 64, bf16, ctx ~ U{1..2048}, permuted 20k-frame pool.

    Draw order: ``ctx = integers(1, max_ctx + 1, S)``, then ``permutation(NB)``.
    Another block size keeps the pool's slot count (NB = 20000 * 16 / B).
    Another seed (structure and values) gives a robustness variant. Another
    head dim D (with the default H) keeps H * D = 4096, so a token's row
    keeps its size; another dtype changes only the storage type.
    """
    NB = NB if NB is not None else 20000 * 16 // B
    if D != 128 and H == 32:
        H = 4096 // D
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, max_ctx + 1, size=S)
    order = rng.permutation(NB)
    if D != 128 or dtype != "bf16":
        name = f"cfg2_S{S}_H{H}_d{D}_{dtype}"
    else:
        name = "cfg2_batch64_bf16" if (S, H) == (64, 32) else f"cfg2_S{S}_H{H}"
    if max_ctx != 2048:
        name += f"_ctx{max_ctx}"
    if B != 16:
        name += f"_B{B}"
    if seed != 2:
        name += f"_seed{seed}"
    return Workload(
        name=name, seed=seed, dtype=dtype, H=H, D=D, B=B, NB=NB, num_seqs=S,
        prefill=[(s, int(ctx[s])) for s in range(S)], frame_order=order,
        description=f"S={S}, H={H}, d={D}, B={B}, {dtype}, ctx U[1,{max_ctx}], permuted pool of {NB}",
    )


def config3(S: int = 8, H: int = 40, ctx: int = 32768, NB: int | None = None,
            B: int = 16) -> Workload:
    """Long context: every sequence exactly 32,768 tokens, permuted pool.

    Another block size keeps the pool's slot count (NB = 20000 * 16 / B).
    """
    NB = NB if NB is not None else 20000 * 16 // B
    rng = np.random.default_rng(3)
    order = rng.permutation(NB)
    name = "cfg3_long_ctx_bf16" if (S, H, ctx) == (8, 40, 32768) else f"cfg3_S{S}_H{H}_L{ctx}"
    if B != 16:
        name += f"_B{B}"
    return Workload(
        name=name, seed=3, dtype="bf16", H=H, D=128, B=B, NB=NB, num_seqs=S,
        prefill=[(s, ctx) for s in range(S)], frame_order=order,
        description=f"S={S}, H={H}, d=128, B={B}, bf16, ctx {ctx}, permuted pool of {NB}",
    )


def config4(prompts: int = 64, n: int = 4, prompt_len: int = 1000, H: int = 32,
            NB: int = 8192, max_tail: int = 200) -> Workload:
    """Shared-prefix parallel sampling: each prompt forked into n branches.

    Sequence ``p * n + b`` is branch ``b`` of prompt ``p``; branch 0 is the
    prefilled parent. Draw order: ``tails = integers(1, max_tail + 1, prompts * n)``.
    Tails are appended one token per decode step, all live branches in
    sequence order, then attention runs once.
    """
    rng = np.random.default_rng(4)
    S = prompts * n
    tails = rng.integers(1, max_tail + 1, size=S)
    prefill = [(p * n, prompt_len) for p in range(prompts)]
    forks = [(p * n, p * n + b) for p in range(prompts) for b in range(1, n)]
    steps = []
    for t in range(int(tails.max())):
        steps.append([s for s in range(S) if tails[s] > t])
    share_len = np.zeros(S, dtype=np.int64)
    share_src = np.zeros(S, dtype=np.int64)
    for p in range(prompts):
        for b in range(1, n):
            share_len[p * n + b] = prompt_len
            share_src[p * n + b] = p * n
    return Workload(
        name="cfg4_shared_prefix_f16" if (prompts, H) == (64, 32) else f"cfg4_P{prompts}_H{H}",
        seed=4, dtype="f16", H=H, D=128, B=32, NB=NB, num_seqs=S,
        prefill=prefill, forks=forks, steps=steps, attend_after=[len(steps) - 1],
        share_len=share_len, share_src=share_src,
        description=f"{prompts} prompts x {prompt_len} tokens, n={n} branches, tails U[1,{max_tail}], "
                    f"B=32, H={H}, d=128, fp16, FIFO pool of {NB}",
    )


def config5(S: int = 256, H: int = 64, NB: int = 32768, cap: int = 8192, seed: int = 5,
            permuted: bool = False) -> Workload:
    """Large-model decode step: lognormal contexts, append then attend.

    Draw order: ``z = standard_normal(S)``; ``ctx = clip(rint(exp(ln 1000 + 0.8 z)), 1, cap)``;
    with ``permuted``, then ``permutation(NB)`` for the pool (the sensitivity
    variant; the default pool is first in, first out in id order).
    ``ctx`` counts the token appended by the step, so the prefill is ctx - 1.
    Another seed (structure and values) gives a robustness variant.
    """
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(S)
    ctx = np.clip(np.rint(np.exp(np.log(1000.0) + 0.8 * z)), 1, cap).astype(np.int64)
    order = rng.permutation(NB) if permuted else None
    name = "cfg5_batch256_f16" if (S, H) == (256, 64) else f"cfg5_S{S}_H{H}"
    if permuted:
        name += "_permuted"
    if seed != 5:
        name += f"_seed{seed}"
    return Workload(
        name=name, seed=seed, dtype="f16", H=H, D=128, B=16, NB=NB, num_seqs=S,
        prefill=[(s, int(ctx[s]) - 1) for s in range(S)],
        steps=[list(range(S))], attend_after=[0], frame_order=order,
        description=f"S={S}, H={H}, d=128, B=16, fp16, lognormal ctx (median 1000, sigma 0.8, "
                    f"cap {cap}); append one token then attend; "
                    f"{'permuted' if permuted else 'FIFO'} pool of {NB}",
    )


def config6(S: int = 16, H: int = 32, chunk: int = 512, max_prefix: int = 1536,
            NB: int = 4096) -> Workload:
    """Chunked prefill: each sequence holds a cached prefix ~ U{0..max_prefix}
    and appends a chunk of ``chunk`` tokens whose queries attend causally.

    Draw order: ``prefix = integers(0, max_prefix + 1, S)``, then ``permutation(NB)``.
    """
    rng = np.random.default_rng(6)
    prefix = rng.integers(0, max_prefix + 1, size=S)
    order = rng.permutation(NB)
    ctx = prefix + chunk
    return Workload(
        name="prefill_chunk512_bf16" if (S, H, chunk) == (16, 32, 512) else f"prefill_S{S}_H{H}_C{chunk}",
        seed=6, dtype="bf16", H=H, D=128, B=16, NB=NB, num_seqs=S,
        prefill=[(s, int(ctx[s])) for s in range(S)], frame_order=order,
        query_lens=np.full(S, chunk, dtype=np.int64),
        description=f"S={S}, H={H}, d=128, B=16, bf16, cached prefix U[0,{max_prefix}] + chunk of "
                    f"{chunk} causal queries, permuted pool of {NB}",
    )


def config7(S: int = 8, H: int = 32, max_ctx: int = 2048, NB: int = 2048,
            dtype: str = "f16") -> Workload:
    """Whole-prompt prefill: ctx ~ U{1..max_ctx}; every token is a query.

    Draw order: ``ctx = integers(1, max_ctx + 1, S)``, then ``permutation(NB)``.
    """
    rng = np.random.default_rng(7)
    ctx = rng.integers(1, max_ctx + 1, size=S)
    order = rng.permutation(NB)
    return Workload(
        name=f"prefill_full_{dtype}" if (S, H) == (8, 32) else f"prefill_full_S{S}_H{H}_{dtype}",
        seed=7, dtype=dtype, H=H, D=128, B=16, NB=NB, num_seqs=S,
        prefill=[(s, int(ctx[s])) for s in range(S)], frame_order=order,
        query_lens=ctx.astype(np.int64),
        description=f"S={S}, H={H}, d=128, B=16, {dtype}, whole prompts ctx U[1,{max_ctx}] as causal "
                    f"queries, permuted pool of {NB}",
    )


FULL = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5, 6: config6, 7: config7}


def small(cfg_id: int) -> Workload:
    """Reduced variants the oracle finishes in seconds, with the same structure."""
    if cfg_id == 1:
        return config1()
    if cfg_id == 2:
        return config2(S=8, H=4, NB=2000)
    if cfg_id == 3:
        return config3(S=2, H=2, ctx=32768, NB=4200)
    if cfg_id == 4:
        return config4(prompts=3, H=4, NB=600)
    if cfg_id == 5:
        return config5(S=24, H=4, NB=4000)
    if cfg_id == 6:
        return config6(S=3, H=2, chunk=150, max_prefix=200, NB=200)
    if cfg_id == 7:
        return config7(S=3, H=2, max_ctx=300, NB=200, dtype="bf16")
    if cfg_id == 8:
        return config8(P=2, C=6, R=4, H=2, sys_min=20, sys_max=60, turn_min=5, turn_max=40,
                       p_active=0.6, gen_min=2, gen_max=12, NB=36)
    raise ValueError(cfg_id)


@dataclass
class PrefixWorkload:
    """Rounds of requests whose prompts share leading tokens.

    Conversation ``c`` opens with system prompt ``conv_sys[c]`` (shared by
    every conversation that uses it). In round ``r`` each conversation with
    ``active[c, r]`` grows by ``turn_len[c, r]`` tokens and sends one request
    whose prompt is its whole history so far; requests of a round arrive in
    conversation order. After the round's prefill each request generates
    ``gen_len[c, r]`` tokens, one per decode step (step g appends a token to
    every request with more than g to generate, in conversation order, then
    decode attention runs over the round's requests); the generated tokens
    join the conversation's history. All requests end before the next round.
    A conversation that sits a round out keeps its history, and its cached
    blocks may be evicted meanwhile.

    Token ids double as value identities: position ``i`` of a conversation
    whose system prompt ``p`` is longer than ``i`` holds ``p * stride + i``,
    any later position ``(P + c) * stride + i``. Equal token prefixes thus
    hold equal values, as the K/V of a real model would. A query token's
    value is drawn from the query stream under its own identity.

    Structure draws use ``numpy.random.default_rng(seed)``: ``sys_len``,
    then ``conv_sys``, then ``turn_len``, then ``active``, then ``gen_len``,
    then the pool order.
    """

    name: str
    seed: int
    dtype: str
    H: int
    D: int
    B: int
    NB: int
    sys_len: np.ndarray       # int64 [P]
    conv_sys: np.ndarray      # int64 [C]
    turn_len: np.ndarray      # int64 [C, R]
    active: np.ndarray        # bool [C, R]
    gen_len: np.ndarray | None = None  # int64 [C, R]: tokens generated per round (None: 0)
    frame_order: np.ndarray | None = None
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def num_seqs(self) -> int:
        return int(len(self.conv_sys))

    @property
    def rounds(self) -> int:
        return int(self.turn_len.shape[1])

    def gen(self, c: int, r: int) -> int:
        return 0 if self.gen_len is None else int(self.gen_len[c, r])

    def history(self, c: int, r: int) -> int:
        """Tokens of conversation ``c`` once round ``r`` is done (r = -1:
        before the first round)."""
        grown = self.turn_len[c, :r + 1].copy()
        if self.gen_len is not None:
            grown = grown + self.gen_len[c, :r + 1]
        return int(self.sys_len[self.conv_sys[c]] + (grown * self.active[c, :r + 1]).sum())

    def prompt_len(self, c: int, r: int) -> int:
        """Prompt of conversation ``c``'s request in round ``r``."""
        return self.history(c, r - 1) + int(self.turn_len[c, r])

    @functools.cached_property
    def stride(self) -> int:
        return max(self.history(c, self.rounds - 1) for c in range(self.num_seqs)) + 1

    def tokens(self, c: int, positions) -> np.ndarray:
        """Token ids (= value identities) of conversation ``c`` at ``positions``."""
        pos = np.asarray(positions, dtype=np.int64)
        p = int(self.conv_sys[c])
        P = len(self.sys_len)
        own = (P + c) * self.stride + pos
        return np.where(pos < self.sys_len[p], p * self.stride + pos, own)

    def idents(self, c: int, positions) -> np.ndarray:
        return self.tokens(c, positions)

    def idents_rows(self, convs, positions) -> np.ndarray:
        """Identities of rows given as parallel (conversation, position) arrays."""
        convs = np.asarray(convs, dtype=np.int64)
        out = np.empty(len(convs), dtype=np.int64)
        for c in np.unique(convs):
            m = convs == c
            out[m] = self.idents(int(c), np.asarray(positions)[m])
        return out

    @property
    def frames_without_caching(self) -> int:
        """Frames the busiest round takes when nothing is shared."""
        return max(sum(-(-(n + self.gen(c, r)) // self.B) for c, n in self.requests(r))
                   for r in range(self.rounds))

    def decode_steps(self, r: int) -> list:
        """Per decode step of round ``r``: the conversations appending a token."""
        reqs = [c for c, _ in self.requests(r)]
        steps = max((self.gen(c, r) for c in reqs), default=0)
        return [[c for c in reqs if self.gen(c, r) > g] for g in range(steps)]

    def requests(self, r: int) -> list:
        """[(conversation, prompt length)] of round ``r`` in arrival order."""
        return [(c, self.prompt_len(c, r)) for c in range(self.num_seqs) if self.active[c, r]]


def config8(P: int = 8, C: int = 64, R: int = 4, H: int = 32, sys_min: int = 512,
            sys_max: int = 1536, turn_min: int = 32, turn_max: int = 256, p_active: float = 0.75,
            gen_min: int = 16, gen_max: int = 64, NB: int = 2816,
            dtype: str = "bf16") -> PrefixWorkload:
    """Prefix caching across requests: C conversations over P shared system
    prompts, R rounds of multi-turn requests, each a whole-history prompt
    followed by gen_len ~ U{gen_min..gen_max} generated tokens; each
    conversation takes part in a round with probability p_active (every
    conversation in round 0)."""
    rng = np.random.default_rng(8)
    sys_len = rng.integers(sys_min, sys_max + 1, size=P).astype(np.int64)
    conv_sys = rng.integers(0, P, size=C).astype(np.int64)
    turn_len = rng.integers(turn_min, turn_max + 1, size=(C, R)).astype(np.int64)
    active = rng.random((C, R)) < p_active
    active[:, 0] = True
    gen_len = rng.integers(gen_min, gen_max + 1, size=(C, R)).astype(np.int64)
    order = rng.permutation(NB)
    full = (P, C, R, H) == (8, 64, 4, 32)
    return PrefixWorkload(
        name=f"prefix_cache_{dtype}" if full else f"prefix_cache_P{P}_C{C}_R{R}_H{H}",
        seed=8, dtype=dtype, H=H, D=128, B=16, NB=NB, sys_len=sys_len, conv_sys=conv_sys,
        turn_len=turn_len, active=active, gen_len=gen_len, frame_order=order,
        description=f"{C} conversations over {P} system prompts U[{sys_min},{sys_max}], {R} rounds "
                    f"of turns U[{turn_min},{turn_max}] + generated U[{gen_min},{gen_max}], "
                    f"whole-history prompts, H={H}, d=128, B=16, {dtype}, permuted pool of {NB}",
    )


FULL[8] = config8
