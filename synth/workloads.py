"""Seeded synthetic request streams for the five workload shapes.

A workload is a list of requests.  Each has a prompt (the key matched in
the tree), the tokens it feeds at its decode steps (one per step), and the
requests that must finish before it arrives.  Token ids are uniform in
[0, 1000) from numpy's PCG64 seeded with the workload seed; Q/K/V values
come from ``synth.gen`` with the same seed.

These shapes stand in for the pages' few-shot, branching-sample (fork) and
multi-turn chat benchmarks; no benchmark data is used or reproduced.
"""

from dataclasses import dataclass, field

import numpy as np

VOCAB = 1000


@dataclass
class Request:
    rid: int
    prompt: list
    gen: list = field(default_factory=list)
    after: tuple = ()


@dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16"
    num_slots: int
    requests: list
    max_ctx: int
    skip_extend_attention: bool = False  # K/V written by kv_store only
    page_size: int = 1  # KV slots per page of the pool (num_slots a multiple of it)

    @property
    def sm_scale(self):
        return 1.0 / float(np.sqrt(self.head_dim))


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _tokens(rng, n):
    return [int(t) for t in rng.integers(0, VOCAB, size=n)]


def _distinct_first(rng, n, avoid):
    """n token runs' first tokens, pairwise distinct and not in ``avoid``."""
    firsts = []
    while len(firsts) < n:
        t = int(rng.integers(0, VOCAB))
        if t not in firsts and t not in avoid:
            firsts.append(t)
    return firsts


def tiny(num_slots=512, with_wave2=None, seed=0):
    """1 layer, Hq = Hkv = 4, D = 64, fp32.  Four requests share a 32-token
    prefix and add distinct 16-token suffixes; each decodes 8 tokens.  The
    first request runs alone; the other three arrive when it finishes.
    With a pool of 160 slots a second wave of four requests (same prefix,
    fresh suffixes) arrives after the first wave and forces eviction."""
    if with_wave2 is None:
        with_wave2 = num_slots < 512
    rng = _rng(seed)
    prefix = _tokens(rng, 32)
    firsts = _distinct_first(rng, 8, avoid=())
    reqs = []
    for i in range(4):
        suffix = [firsts[i]] + _tokens(rng, 15)
        reqs.append(Request(i, prefix + suffix, _tokens(rng, 8), () if i == 0 else (0,)))
    if with_wave2:
        for i in range(4):
            suffix = [firsts[4 + i]] + _tokens(rng, 15)
            reqs.append(Request(4 + i, prefix + suffix, _tokens(rng, 8), (1, 2, 3)))
    return Workload("tiny", seed, 4, 4, 64, "f32", num_slots, reqs, max_ctx=64)


def few_shot(seed=1, batch=64, prefix_len=1024, suffix_len=128, decode_steps=0,
             num_slots=262144):
    """Llama-3-8B attention shape (Hq 32, Hkv 8, D 128, bf16).  A warm-up
    request holds the shared few-shot prefix; then ``batch`` requests add
    distinct suffixes and run one extend pass (plus ``decode_steps``)."""
    rng = _rng(seed)
    prefix = _tokens(rng, prefix_len)
    reqs = [Request(0, list(prefix), [], ())]
    for i in range(batch):
        reqs.append(Request(1 + i, prefix + _tokens(rng, suffix_len),
                            _tokens(rng, decode_steps), (0,)))
    return Workload("few_shot", seed, 32, 8, 128, "bf16", num_slots, reqs,
                    max_ctx=prefix_len + suffix_len + decode_steps)


def fork(seed=2, prompts=16, prompt_len=2048, branches=8, decode_steps=256,
         num_slots=262144):
    """16 cold prompts of 2048 tokens; each forks into 8 branches that match
    the whole prompt and decode 256 tokens (batch 128)."""
    rng = _rng(seed)
    reqs, rid = [], 0
    heads = []
    for p in range(prompts):
        reqs.append(Request(rid, _tokens(rng, prompt_len), [], ()))
        heads.append(rid)
        rid += 1
    for p in range(prompts):
        for b in range(branches):
            reqs.append(Request(rid, list(reqs[heads[p]].prompt), _tokens(rng, decode_steps),
                                (heads[p],)))
            rid += 1
    return Workload("fork", seed, 32, 8, 128, "bf16", num_slots, reqs,
                    max_ctx=prompt_len + decode_steps)


def chat(seed=3, sessions=256, turns=4, system_len=512, user_lo=128, user_hi=384,
         gen_len=128, pool_fraction=0.6):
    """Multi-turn chat tree: a shared system prompt; each turn appends
    U{128..384} user tokens to the whole history and generates 128 tokens;
    turn k+1 arrives when turn k finishes.  The pool is a fraction of the
    working set (system prompt + every user and generated token)."""
    rng = _rng(seed)
    system = _tokens(rng, system_len)
    reqs = [Request(0, list(system), [], ())]
    rid = 1
    working_set = system_len
    max_ctx = 0
    for s in range(sessions):
        history = list(system)
        prev = 0
        for t in range(turns):
            u = int(rng.integers(user_lo, user_hi + 1))
            history = history + _tokens(rng, u)
            gen = _tokens(rng, gen_len)
            reqs.append(Request(rid, list(history), gen, (prev,)))
            working_set += u + gen_len
            history = history + gen
            max_ctx = max(max_ctx, len(history))
            prev = rid
            rid += 1
    num_slots = int(pool_fraction * working_set)
    return Workload("chat", seed, 32, 8, 128, "bf16", num_slots, reqs, max_ctx=max_ctx)


def long_context(seed=4, batch=32, shared_len=16384, private_len=16384, decode_steps=128,
                 num_slots=1 << 20):
    """Hq 64, Hkv 8, D 128, bf16: 32 requests of 32768-token context whose
    first 16384 tokens are shared; 128 decode steps.  Prompt K/V is written
    with the scatter kernel only (no extend attention)."""
    rng = _rng(seed)
    shared = _tokens(rng, shared_len)
    reqs = [Request(0, list(shared), [], ())]
    for i in range(batch):
        reqs.append(Request(1 + i, shared + _tokens(rng, private_len),
                            _tokens(rng, decode_steps), (0,)))
    return Workload("long_context", seed, 64, 8, 128, "bf16", num_slots, reqs,
                    max_ctx=shared_len + private_len + decode_steps,
                    skip_extend_attention=True)


def paged(wl, page_size):
    """The same workload over a pool of page_size-slot pages: the pool is
    rounded up to whole pages."""
    import copy
    out = copy.copy(wl)
    out.page_size = int(page_size)
    out.num_slots = -(-wl.num_slots // page_size) * page_size
    return out
