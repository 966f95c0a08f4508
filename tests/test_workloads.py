"""The seeded workloads, run through the oracle allocator (CPU only)."""

import numpy as np
import pytest

import workloads as W
from oracle import allocator as AL


def _run(cfg):
    pl = W.plan(cfg)
    a = AL.RefAllocator(pl.num_blocks, cfg.block_size, max(cfg.batch * 4, 64) + 4096,
                        cfg.max_seq_len)
    a.set_free_order(W.free_order(pl.num_blocks, cfg.seed))
    copies = []
    rids = W.run_ops(pl.ops, a, on_reserve=lambda h, c, s, p: copies.extend(p))
    W.run_ops([pl.step], a, rids, on_reserve=lambda h, c, s, p: copies.extend(p))
    AL.check_invariants(a)
    got = [a.length(rids[h]) for h in pl.batch_handles]
    assert got == [int(x) for x in pl.lengths]
    return pl, a, rids, copies


def test_tiny_workload_uses_13_of_64_blocks():
    pl, a, rids, copies = _run(W.get(1))
    assert list(pl.lengths) == [1, 17, 40, 100]
    assert a.stats()["used_blocks"] == 1 + 2 + 3 + 7
    assert copies == []


@pytest.mark.parametrize("cid,batch", [(2, 4), (4, 3), (3, 6)])
def test_uniform_and_ragged_plans(cid, batch):
    cfg = W.get(cid, batch=batch, num_blocks=0 if cid == 3 else 64 * batch + 8)
    pl, a, rids, copies = _run(cfg)
    assert copies == []
    if cid == 3:
        assert np.all(pl.lengths >= 2) and np.all(pl.lengths <= 8192)
        # fragmented: the measured batch's blocks are not handed out in id order
        t = a.table(rids[0])
        assert t != sorted(t) or len(t) < 3


def test_ragged_lengths_distribution():
    prompt, gen = W.ragged_lengths(20000, np.random.default_rng(0))
    assert prompt.min() >= 1 and gen.min() >= 1 and (prompt + gen).max() <= 8192
    assert abs(prompt.mean() - 1024) < 40 and abs(gen.mean() - 256) < 10


@pytest.mark.parametrize("prompt_len,expect", [(48, 0), (56, 7)])
def test_shared_prefix_copies(prompt_len, expect):
    cfg = W.get(5, batch=16, prompt_len=prompt_len, private_len=20, num_blocks=256)
    pl, a, rids, copies = _run(cfg)
    assert len(copies) == expect * 2     # 2 prompts x (samples - 1)
    # samples of one prompt still share the full prompt blocks
    t0, t1 = a.table(rids[0]), a.table(rids[1])
    assert t0[: prompt_len // 16] == t1[: prompt_len // 16]


def test_full_shared_prefix_plan_copy_counts():
    # the 2048-token prompt fills its last block: no copy; 2056 leaves it half
    # full: 7 copies per prompt, 280 in all
    for plen, expect in ((2048, 0), (2056, 280)):
        cfg = W.get(5, prompt_len=plen, private_len=2)
        pl = W.plan(cfg)
        a = AL.RefAllocator(pl.num_blocks, 16, 400, 8192)
        copies = []
        rids = W.run_ops(pl.ops, a, on_reserve=lambda h, c, s, p: copies.extend(p))
        W.run_ops([pl.step], a, rids, on_reserve=lambda h, c, s, p: copies.extend(p))
        assert len(copies) == expect


def test_values_are_seeded():
    cfg = W.get(1)
    pl = W.plan(cfg)
    a = W.values(cfg, pl)
    b = W.values(cfg, pl)
    for x, y in zip(a, b):
        assert (x == y).all()
    assert a[1].shape == (pl.num_rows, 2, 64)
