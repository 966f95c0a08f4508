"""Pins of the allocator and capacity oracles.

* The pages' printed per-token footprints (KV-allocation-patterns page,
  Observation-2) and the workshop's admission readouts ("Running Out of
  Cache": 52 vs 333 requests, 6.4x, 15% vs 99% in use).
* The waste rule: under one block per sequence (same page, paging paragraph).
* Sharing and copy-on-write checked by a token-label content model: no
  sequence ever sees a token it did not write or inherit.
* All-or-nothing growth when blocks run out.
"""

import copy
import json
import math
import os

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import allocator as AL
from oracle import capacity as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_per_token_footprints_match_the_page():
    g = _golden("footprints.json")
    for m in g["models"]:
        got = C.kv_bytes_per_token(m["num_layers"], m["num_kv_heads"], m["head_dim"], g["elt_bytes"])
        assert got == m["kb_per_token"] * 1024, m["model"]


def test_workshop_closed_forms_match_the_page():
    w = _golden("workshop.json")
    tokens = C.cache_tokens(w["cache_bytes"], w["model_bytes_per_token"])
    mean_len = w["prompt_mean"] + w["output_mean"]
    contiguous = C.contiguous_admissions(tokens, w["max_len"])
    paged = C.paged_admissions(tokens, w["block_size"], mean_len)
    assert contiguous == w["contiguous_requests"]
    assert paged == w["paged_requests"]
    assert round(paged / contiguous, 1) == w["ratio"]
    assert math.floor(100 * C.contiguous_utilisation([mean_len], w["max_len"])) == w["contiguous_pct_in_use"]


def test_workshop_admissions_by_driving_the_allocator():
    w = _golden("workshop.json")
    tokens = C.cache_tokens(w["cache_bytes"], w["model_bytes_per_token"])
    bs = w["block_size"]
    mean_len = w["prompt_mean"] + w["output_mean"]
    # paged: admit mean-length requests until no block is left
    a = AL.RefAllocator(tokens // bs, bs, max_seqs=4096, max_seq_len=w["max_len"])
    admitted = 0
    while True:
        rid = a.add()
        try:
            a.reserve([rid], [mean_len])
        except AL.AllocError as e:
            assert e.status == AL.ERR_NO_BLOCKS
            a.free_seq(rid)
            break
        admitted += 1
    assert admitted == w["paged_requests"]
    # contiguous: each request holds a reqId whose sub-tensor is max_len long
    c = AL.RefAllocator(0, bs, max_seqs=tokens // w["max_len"], max_seq_len=w["max_len"],
                        layout=AL.CONTIGUOUS)
    n = 0
    with pytest.raises(AL.AllocError) as ei:
        while True:
            rid = c.add()
            c.reserve([rid], [mean_len])
            n += 1
    assert ei.value.status == AL.ERR_NO_REQ_ID
    assert n == w["contiguous_requests"]
    assert math.floor(100 * c.stats()["utilisation"]) == w["contiguous_pct_in_use"]


def test_workshop_paged_utilisation_with_exponential_lengths():
    # Prompt and output lengths exponential with the workshop's means; the
    # share of allocated blocks holding tokens rounds to the page's 99%.
    w = _golden("workshop.json")
    rng = np.random.default_rng(5)
    n = 4000
    lengths = (np.maximum(1, np.rint(rng.exponential(w["prompt_mean"], n)))
               + np.maximum(1, np.rint(rng.exponential(w["output_mean"], n))))
    lengths = np.minimum(lengths, w["max_len"]).astype(int)
    a = AL.RefAllocator(int(sum(-(-x // 16) for x in lengths)), 16, n, w["max_len"])
    for x in lengths:
        a.reserve([a.add()], [int(x)])
    util = a.stats()["utilisation"]
    assert abs(util - C.paged_utilisation(lengths, 16)) < 1e-15
    assert round(100 * util) == w["paged_pct_in_use"]
    assert a.stats()["free_blocks"] == 0


def test_allocate_on_fill_takes_a_block_only_when_the_last_is_full():
    a = AL.RefAllocator(8, 4, 4, 64)
    a.set_free_order([5, 2, 7, 0, 1, 3, 4, 6])
    r = a.add()
    slots = []
    for _ in range(9):
        s, pairs = a.reserve([r])
        assert pairs == []
        slots += s
        AL.check_invariants(a)
    # blocks in the given order; rows filled in position order
    assert slots == [20, 21, 22, 23, 8, 9, 10, 11, 28]
    assert a.table(r) == [5, 2, 7]
    assert a.stats()["tokens"] == 9 and a.stats()["used_blocks"] == 3


def test_fork_shares_and_first_write_copies():
    # Two samples share a half-full block: the first writer copies it, the
    # last holder writes in place; full shared blocks are never copied.
    m = AL.ContentModel(AL.RefAllocator(16, 4, 8, 64))
    p = m.add()
    m.reserve([p], [6])
    c = m.fork(p)
    assert m.a.table(c) == m.a.table(p)
    assert m.a.refcount[m.a.table(p)[0]] == 2
    slots, pairs = m.reserve([p, c])
    assert len(pairs) == 1 and pairs[0][0] == m.a.table(c)[1]
    assert m.a.table(p)[0] == m.a.table(c)[0]
    assert m.a.table(p)[1] != m.a.table(c)[1]
    m.check()
    AL.check_invariants(m.a)
    assert m.a.stats()["cow_copies"] == 1


def test_eight_samples_make_seven_copies():
    m = AL.ContentModel(AL.RefAllocator(64, 16, 16, 256))
    p = m.add()
    m.reserve([p], [24])
    kids = [m.fork(p) for _ in range(7)]
    _, pairs = m.reserve([p] + kids)
    assert len(pairs) == 7
    _, pairs = m.reserve([p] + kids)
    assert pairs == []
    m.check()
    AL.check_invariants(m.a)


def test_full_shared_prompt_is_never_copied():
    m = AL.ContentModel(AL.RefAllocator(64, 16, 16, 256))
    p = m.add()
    m.reserve([p], [32])
    kids = [m.fork(p) for _ in range(3)]
    for _ in range(20):
        _, pairs = m.reserve([p] + kids)
        assert pairs == []
    m.check()
    AL.check_invariants(m.a)


def test_out_of_blocks_leaves_state_unchanged():
    a = AL.RefAllocator(4, 4, 4, 64)
    r1, r2 = a.add(), a.add()
    a.reserve([r1], [9])
    before = copy.deepcopy(a.__dict__)
    with pytest.raises(AL.AllocError) as ei:
        a.reserve([r1, r2], [3, 5])
    assert ei.value.status == AL.ERR_NO_BLOCKS
    assert a.__dict__ == before
    # pre-empt r1 and retry
    a.free_seq(r1)
    a.reserve([r2], [16])
    AL.check_invariants(a)
    assert a.stats()["free_blocks"] == 0


def test_errors():
    a = AL.RefAllocator(4, 4, 2, 8)
    r = a.add()
    a.add()
    with pytest.raises(AL.AllocError) as ei:
        a.add()
    assert ei.value.status == AL.ERR_NO_REQ_ID
    with pytest.raises(AL.AllocError) as ei:
        a.reserve([r, r])
    assert ei.value.status == AL.ERR_INVALID_ARG
    with pytest.raises(AL.AllocError) as ei:
        a.reserve([r], [9])
    assert ei.value.status == AL.ERR_INVALID_ARG
    with pytest.raises(AL.AllocError) as ei:
        a.free_seq(7)
    assert ei.value.status == AL.ERR_UNKNOWN_SEQ


def test_contiguous_slots_follow_reqid_times_s():
    a = AL.RefAllocator(0, 16, 4, 100, layout=AL.CONTIGUOUS)
    r0, r1 = a.add(), a.add()
    slots, pairs = a.reserve([r1, r0], [2, 3])
    assert slots == [100, 101, 0, 1, 2] and pairs == []
    with pytest.raises(AL.AllocError):
        a.fork(r0)


def test_swap_round_trip_restores_contents_and_takes_blocks_off_the_stack():
    m = AL.ContentModel(AL.RefAllocator(10, 4, 4, 64))
    r = m.add()
    m.reserve([r], [10])                 # blocks 0, 1, 2 (ascending free order)
    assert m.a.table(r) == [0, 1, 2]
    m.swap_out(r)
    # given back in table order onto the free stack, block 2 on top
    assert m.a.free[-3:] == [0, 1, 2]
    st_out = m.a.stats()
    assert st_out["used_blocks"] == 0 and st_out["live_seqs"] == 0
    assert st_out["swapped_seqs"] == 1 and st_out["swapped_tokens"] == 10
    m.check()
    m.swap_in(r)
    # ceil(10 / 4) = 3 blocks off the top of the stack: the table comes back reversed
    assert m.a.table(r) == [2, 1, 0]
    assert m.a.length(r) == 10 and m.a.stats()["swapped_seqs"] == 0
    m.check()
    AL.check_invariants(m.a)
    m.reserve([r], [3])                  # 2 rows fill block 0, then a new block
    m.check()
    assert m.a.table(r) == [2, 1, 0, 3]


def test_swapping_out_one_sharer_leaves_the_others_their_blocks():
    m = AL.ContentModel(AL.RefAllocator(12, 4, 4, 64))
    p = m.add()
    m.reserve([p], [6])
    c = m.fork(p)
    shared = m.a.table(p)
    m.swap_out(p)
    assert m.a.table(c) == shared and all(m.a.refcount[b] == 1 for b in shared)
    assert m.a.stats()["shared_blocks"] == 0
    m.reserve([c], [3])                  # c is now the only holder: writes in place
    m.check()
    m.swap_in(p)                         # p comes back into private blocks
    assert set(m.a.table(p)).isdisjoint(m.a.table(c))
    m.reserve([p], [2])
    m.check()
    AL.check_invariants(m.a)


def test_preemption_by_swapping_frees_room_and_the_request_resumes():
    # 6 blocks of 4: two requests of 11 tokens fill the pool (one row left in
    # each last block)
    m = AL.ContentModel(AL.RefAllocator(6, 4, 4, 64))
    a, b = m.add(), m.add()
    m.reserve([a, b], [11, 11])
    c = m.add()
    with pytest.raises(AL.AllocError) as e:
        m.reserve([c], [5])
    assert e.value.status == AL.ERR_NO_BLOCKS
    m.swap_out(b)                        # the pre-empted request
    m.reserve([c], [5])
    with pytest.raises(AL.AllocError) as e:
        m.swap_in(b)                     # needs 3 blocks, 1 free: nothing changes
    assert e.value.status == AL.ERR_NO_BLOCKS and m.a.seqs[b].swapped
    m.free_seq(c)
    m.swap_in(b)
    m.reserve([a, b])                    # both write their last free row in place
    assert m.a.stats()["free_blocks"] == 0
    m.check()
    AL.check_invariants(m.a)


def test_swap_errors():
    a = AL.RefAllocator(8, 4, 4, 64)
    r = a.add()
    a.reserve([r], [5])
    with pytest.raises(AL.AllocError) as e:
        a.swap_in(r)                     # resident
    assert e.value.status == AL.ERR_INVALID_ARG
    a.swap_out(r)
    for call in (lambda: a.reserve([r]), lambda: a.fork(r), lambda: a.table(r),
                 lambda: a.swap_out(r)):
        with pytest.raises(AL.AllocError) as e:
            call()
        assert e.value.status == AL.ERR_INVALID_ARG
    with pytest.raises(AL.AllocError) as e:
        a.swap_out(7)
    assert e.value.status == AL.ERR_UNKNOWN_SEQ
    a.free_seq(r)                        # a swapped-out request can be dropped
    assert a.stats()["swapped_seqs"] == 0 and a.stats()["free_blocks"] == 8
    c = AL.RefAllocator(0, 16, 4, 64, layout=AL.CONTIGUOUS)
    q = c.add()
    with pytest.raises(AL.AllocError) as e:
        c.swap_out(q)
    assert e.value.status == AL.ERR_INVALID_ARG


_ops = st.lists(st.tuples(st.sampled_from(["add", "fork", "grow", "free", "swapout", "swapin"]),
                          st.integers(0, 1 << 30), st.integers(0, 40)), max_size=60)


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(_ops, st.sampled_from([1, 2, 4, 16]), st.integers(4, 40))
def test_random_operation_sequences_keep_every_invariant(ops, bs, nb):
    m = AL.ContentModel(AL.RefAllocator(nb, bs, 6, 120))
    for kind, pick, count in ops:
        live = sorted(m.history)
        resident = [r for r in live if r not in m.images]
        try:
            if kind == "add":
                m.add()
            elif kind == "fork" and resident:
                m.fork(resident[pick % len(resident)])
            elif kind == "free" and live:
                m.free_seq(live[pick % len(live)])
            elif kind == "swapout" and resident:
                m.swap_out(resident[pick % len(resident)])
            elif kind == "swapin" and m.images:
                out = sorted(m.images)
                before = copy.deepcopy(m.a.__dict__)
                try:
                    m.swap_in(out[pick % len(out)])
                except AL.AllocError as e:
                    assert e.status == AL.ERR_NO_BLOCKS and m.a.__dict__ == before
            elif kind == "grow" and resident:
                chosen = [r for i, r in enumerate(resident) if (pick >> i) & 1] or resident[:1]
                before = copy.deepcopy(m.a.__dict__)
                try:
                    m.reserve(chosen, [count % 7] * len(chosen))
                except AL.AllocError as e:
                    assert e.status in (AL.ERR_NO_BLOCKS, AL.ERR_INVALID_ARG)
                    assert m.a.__dict__ == before
        except AL.AllocError as e:
            assert e.status in (AL.ERR_NO_REQ_ID, AL.ERR_NO_BLOCKS)
        AL.check_invariants(m.a)
        m.check()
    for r in sorted(m.history):
        m.free_seq(r)
    assert m.a.stats()["free_blocks"] == nb
    AL.check_invariants(m.a)


def test_invariant_checker_catches_planted_mistakes():
    a = AL.RefAllocator(8, 4, 4, 64)
    r = a.add()
    a.reserve([r], [6])
    AL.check_invariants(a)
    bad = copy.deepcopy(a)
    bad.refcount[bad.table(r)[0]] += 1
    with pytest.raises(AssertionError):
        AL.check_invariants(bad)
    bad = copy.deepcopy(a)
    bad.seqs[r].table.append(bad.free.pop())
    with pytest.raises(AssertionError):
        AL.check_invariants(bad)
    # a write into a shared block (no copy) is caught by the content model
    m = AL.ContentModel(AL.RefAllocator(8, 4, 4, 64))
    p = m.add()
    m.reserve([p], [2])
    c = m.fork(p)
    m.a.refcount[m.a.table(p)[0]] = 1   # plant: forget the share
    m.reserve([p])
    m.reserve([c])                        # overwrites p's third token in place
    with pytest.raises(AssertionError):
        m.check()
    # a swap-in that brings back the wrong rows is caught too
    m = AL.ContentModel(AL.RefAllocator(8, 4, 4, 64))
    r = m.add()
    m.reserve([r], [6])
    m.swap_out(r)
    m.images[r][1], m.images[r][4] = m.images[r][4], m.images[r][1]   # plant: two rows swapped
    with pytest.raises(AssertionError):
        m.check()
