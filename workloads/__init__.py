"""Seeded synthetic workloads for paged decode attention.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``.  This module
only draws random numbers and lays out *what* is asked of the cache: shapes,
context lengths, the order in which requests are admitted, forked, grown and
freed, and which token rows each sequence holds.  It holds none of the method's
arithmetic: no attention, no allocator logic, no slot or address computation.

The five workloads follow the pages' settings:

1. tiny fp32 paged decode (parity case; lengths {1, 17, 40, 100});
2. one Llama-3-8B decode layer, batch 64, 1024-token contexts (32 q / 8 kv
   heads, head_dim 128, bf16) - the shape of the per-token footprint in
   [KVP] Observation-2 and of the workshop in [ROC];
3. a ragged serving mix at the Llama-3-8B shape: prompt ~ Exp(1024) plus
   output ~ Exp(256) tokens, capped at 8192 ([ROC] Workshop), served from a
   pool fragmented by an earlier generation of requests;
4. the one-GPU share of Yi-34B under two-way tensor parallelism ([KVP] section
   4 setup): 28 q / 4 kv heads, batch 128, 1024 tokens, paged and contiguous
   at ``reqId x S`` with S = 8192 ([VAC] 5.2.3);
5. shared prompts with parallel samples at the Yi-6B shape ([PAS] Key points,
   [ROC] "Fragmentation is lost users"): 40 prompts of 2048 tokens, 8 samples
   each, 256 private tokens per sample.  Variant ``prompt_len=2056`` leaves
   the last prompt block half full, so the first private write copies it.

Every context length is the length *after* the decode step's append: a
sequence is prefilled with ``L - 1`` tokens and the step appends token ``L-1``
and attends over all ``L``.  The tiny workload also runs in the other
reading (``contexts_before_append=True``): its lengths are the contexts
before the step, which appends token ``L`` and attends over ``L + 1``.

Values: q, K and V rows are N(0, 1) float32 draws from a seeded
``torch.Generator``, cast to bfloat16 with round-to-nearest-even where the
workload is bf16.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

BASE_SEED = 2410


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str            # "f32" | "bf16"
    num_layers: int          # distinct layer pools (rotated by the bench)
    num_blocks: int          # 0: derived from the plan
    max_seq_len: int         # S: per-request cap (and contiguous stride)
    context: int = 0         # uniform context length (0: drawn)
    prompt_len: int = 0      # shared-prompt workloads
    samples: int = 0
    private_len: int = 0
    seed: int = BASE_SEED
    contexts_before_append: bool = False   # tiny workload: the other reading of its lengths

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


CONFIGS = {
    1: Config(1, "tiny paged decode, fp32", 4, 4, 2, 64, 16, "f32", 1, 64, 128,
              seed=BASE_SEED + 1),
    2: Config(2, "Llama-3-8B decode layer, batch 64, context 1024", 64, 32, 8, 128, 16,
              "bf16", 8, 4096, 8192, context=1024, seed=BASE_SEED + 2),
    3: Config(3, "ragged serving mix at the Llama-3-8B shape, batch 256", 256, 32, 8, 128, 16,
              "bf16", 4, 0, 8192, seed=BASE_SEED + 3),
    4: Config(4, "Yi-34B one-GPU tensor-parallel share, batch 128, context 1024", 128, 28, 4,
              128, 16, "bf16", 4, 8192, 8192, context=1024, seed=BASE_SEED + 4),
    5: Config(5, "shared-prefix parallel sampling at the Yi-6B shape, batch 320", 320, 32, 4,
              128, 16, "bf16", 4, 12288, 8192, prompt_len=2048, samples=8,
              private_len=256, seed=BASE_SEED + 5),
}

TINY_LENGTHS = (1, 17, 40, 100)


def get(cid: int, **overrides) -> Config:
    """Workload ``cid`` (1..5), optionally with fields replaced (e.g. batch)."""
    return replace(CONFIGS[cid], **overrides)


# --------------------------------------------------------------------------
# plans: the order of admissions, forks, growth and frees
# --------------------------------------------------------------------------

@dataclass
class Plan:
    """What to do to the cache, in order, before and during one decode step.

    ``ops`` are tuples over integer handles:
      ("add", h) | ("fork", parent_h, child_h) | ("free", h) |
      ("reserve", [h...], [count...])
    ``rows[h]`` lists, for handle h, the logical row id of each of its
    positions (shared prompt positions of forked samples name the same rows);
    handles without an entry get no content (warm-up traffic).
    ``step`` is the decode step's reserve: one new token for every handle of
    the batch, in batch order.  ``lengths[s]`` is batch sequence s's context
    after the step.
    """

    ops: list = field(default_factory=list)
    rows: dict = field(default_factory=dict)
    batch_handles: list = field(default_factory=list)
    lengths: np.ndarray = None
    num_rows: int = 0
    num_blocks: int = 0
    step: tuple = None


def ragged_lengths(n: int, rng: np.random.Generator):
    """(prompt, generated) lengths: Exp(1024) and Exp(256), each >= 1, sum <= 8192."""
    prompt = np.maximum(1, np.rint(rng.exponential(1024.0, n))).astype(np.int64)
    gen = np.maximum(1, np.rint(rng.exponential(256.0, n))).astype(np.int64)
    prompt = np.minimum(prompt, 8191)
    gen = np.minimum(gen, 8192 - prompt)
    return prompt, gen


def plan(cfg: Config) -> Plan:
    """The admission plan of a workload (deterministic in ``cfg.seed``)."""
    rng = np.random.default_rng(cfg.seed)
    p = Plan()
    bs = cfg.block_size
    b = cfg.batch
    if cfg.cid == 1:
        lengths = np.array(TINY_LENGTHS[:b], dtype=np.int64)
        if cfg.contexts_before_append:
            lengths = lengths + 1
        if b > len(TINY_LENGTHS):
            extra = rng.integers(1, 129, b - len(TINY_LENGTHS))
            lengths = np.concatenate([lengths, extra])
        _uniform_like(p, cfg, lengths)
    elif cfg.cid in (2, 4):
        _uniform_like(p, cfg, np.full(b, cfg.context, dtype=np.int64))
    elif cfg.cid == 3:
        _ragged(p, cfg, rng)
    elif cfg.cid == 5:
        _shared_prefix(p, cfg)
    else:
        raise ValueError(cfg.cid)
    if not p.num_blocks:
        p.num_blocks = cfg.num_blocks
    return p


def _uniform_like(p: Plan, cfg: Config, lengths: np.ndarray) -> None:
    b = len(lengths)
    p.batch_handles = list(range(b))
    p.lengths = lengths
    nxt = 0
    for h in range(b):
        p.ops.append(("add", h))
        p.rows[h] = list(range(nxt, nxt + int(lengths[h])))
        nxt += int(lengths[h])
    p.num_rows = nxt
    p.ops.append(("reserve", list(range(b)), [int(n) - 1 for n in lengths]))
    p.step = ("reserve", list(range(b)), [1] * b)


def _ragged(p: Plan, cfg: Config, rng: np.random.Generator) -> None:
    b = cfg.batch
    bs = cfg.block_size
    prompt, gen = ragged_lengths(b, rng)
    lengths = prompt + gen
    blocks_needed = int(sum(-(-int(n) // bs) for n in lengths))
    nb = cfg.num_blocks or int(np.ceil(1.5 * blocks_needed))
    p.num_blocks = nb
    # warm-up generation: same distribution, admitted until the pool is full,
    # then freed in a seeded random order so that reuse follows that order
    wrng = np.random.default_rng(cfg.seed + 1)
    used = 0
    warm = []
    while True:
        wp, wg = ragged_lengths(1, wrng)
        n = int(wp[0] + wg[0])
        need = -(-n // bs)
        if used + need > nb:
            break
        used += need
        warm.append(n)
    handle = b
    warm_handles = []
    for n in warm:
        p.ops.append(("add", handle))
        p.ops.append(("reserve", [handle], [n]))
        warm_handles.append(handle)
        handle += 1
    for i in wrng.permutation(len(warm_handles)):
        p.ops.append(("free", warm_handles[int(i)]))
    # measured batch: prompts at admission, then generated tokens one per
    # live sequence per iteration; the last generated token is the step's
    p.batch_handles = list(range(b))
    p.lengths = lengths.astype(np.int64)
    nxt = 0
    for h in range(b):
        p.ops.append(("add", h))
        p.ops.append(("reserve", [h], [int(prompt[h])]))
        p.rows[h] = list(range(nxt, nxt + int(lengths[h])))
        nxt += int(lengths[h])
    p.num_rows = nxt
    for r in range(int(gen.max()) - 1):
        live = [h for h in range(b) if gen[h] - 1 > r]
        if live:
            p.ops.append(("reserve", live, [1] * len(live)))
    p.step = ("reserve", list(range(b)), [1] * b)


def _shared_prefix(p: Plan, cfg: Config) -> None:
    n_prompts = cfg.batch // cfg.samples
    assert n_prompts * cfg.samples == cfg.batch
    plen = cfg.prompt_len
    priv = cfg.private_len
    # parents are added first (handles 0..n_prompts-1 are the first sample
    # of each prompt); batch order is prompt-major: prompt i's samples are
    # batch entries i*samples .. i*samples+samples-1
    handles = []
    nxt = 0
    prompt_rows = []
    for i in range(n_prompts):
        h = i * cfg.samples
        p.ops.append(("add", h))
        p.ops.append(("reserve", [h], [plen]))
        prompt_rows.append(list(range(nxt, nxt + plen)))
        nxt += plen
    for i in range(n_prompts):
        parent = i * cfg.samples
        for j in range(1, cfg.samples):
            p.ops.append(("fork", parent, parent + j))
    for i in range(n_prompts):
        for j in range(cfg.samples):
            h = i * cfg.samples + j
            handles.append(h)
            p.rows[h] = prompt_rows[i] + list(range(nxt, nxt + priv))
            nxt += priv
    p.num_rows = nxt
    p.batch_handles = handles
    p.lengths = np.full(cfg.batch, plen + priv, dtype=np.int64)
    for _ in range(priv - 1):
        p.ops.append(("reserve", list(handles), [1] * len(handles)))
    p.step = ("reserve", list(handles), [1] * len(handles))


def free_order(num_blocks: int, seed: int) -> np.ndarray:
    """Seeded permutation of all block ids: the order blocks are handed out."""
    return np.random.default_rng(seed).permutation(num_blocks).astype(np.int32)


# --------------------------------------------------------------------------
# values
# --------------------------------------------------------------------------

def normal(shape, seed: int, dtype: str, device="cpu"):
    """Seeded N(0, 1) float32 draws, cast to ``dtype`` ("f32" | "bf16")."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def values(cfg: Config, pl: Plan, device="cpu", layer: int = 0):
    """(q, k_rows, v_rows) of one layer: q ``[B][Hq][d]``, rows ``[num_rows][Hkv][d]``."""
    s = cfg.seed * 1000 + 10 * layer
    q = normal((len(pl.batch_handles), cfg.num_q_heads, cfg.head_dim), s + 1, cfg.kv_dtype, device)
    k = normal((pl.num_rows, cfg.num_kv_heads, cfg.head_dim), s + 2, cfg.kv_dtype, device)
    v = normal((pl.num_rows, cfg.num_kv_heads, cfg.head_dim), s + 3, cfg.kv_dtype, device)
    return q, k, v


def run_ops(ops, alloc, rids=None, on_reserve=None) -> dict:
    """Carry out plan ops on any allocator with add/fork/free_seq/reserve.

    ``rids`` maps plan handles to the allocator's request ids (filled in as
    requests are added or forked).  ``on_reserve(handles, counts, slots,
    pairs)`` is called after every reserve, e.g. to copy and append on a device.
    """
    rids = {} if rids is None else rids
    for op in ops:
        kind = op[0]
        if kind == "add":
            rids[op[1]] = alloc.add()
        elif kind == "fork":
            rids[op[2]] = alloc.fork(rids[op[1]])
        elif kind == "free":
            alloc.free_seq(rids.pop(op[1]))
        elif kind == "reserve":
            handles, counts = op[1], op[2]
            slots, pairs = alloc.reserve([rids[h] for h in handles], counts)
            if on_reserve is not None:
                on_reserve(handles, counts, slots, pairs)
        else:
            raise ValueError(kind)
    return rids
