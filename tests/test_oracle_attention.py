"""Pins of the attention oracle against things other than itself.

Brute force on tiny inputs, closed forms (two-token logistic form, uniform
weights, constant values), library routines (scipy's softmax, torch's bfloat16
conversion), permutation invariance of the block placement and the contiguous
``reqId x S`` layout.  A dropped term, a wrong sign, a wrong scale, a
transposed operand or a wrong query-to-KV-head map fails at least one case.
"""

import math

import numpy as np
import pytest
import scipy.special

from oracle import attention as A


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("hq,hkv,d,length", [
    (1, 1, 4, 1), (2, 1, 3, 5), (4, 2, 8, 7), (6, 3, 5, 16), (8, 8, 4, 3),
    (4, 2, 6, 0), (7, 1, 2, 9), (8, 2, 16, 33),
])
def test_numpy_matches_bruteforce(hq, hkv, d, length):
    rng = np.random.default_rng(100 + hq * 31 + length)
    q = _rand(rng, hq, d)
    k = _rand(rng, length, hkv, d)
    v = _rand(rng, length, hkv, d)
    scale = 1.0 / math.sqrt(d)
    got = A.attend(q, k, v, scale)
    ref = np.array(A.attend_bruteforce(q.tolist(), k.tolist(), v.tolist(), scale))
    assert got.shape == (hq, d)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_two_tokens_logistic_closed_form():
    # With two keys the softmax weight of key 0 is the logistic function of
    # the logit difference: w0 = 1 / (1 + exp(-(z0 - z1))).
    rng = np.random.default_rng(7)
    d = 8
    q = _rand(rng, 1, d)
    k = _rand(rng, 2, 1, d)
    v = _rand(rng, 2, 1, d)
    scale = 0.37
    delta = scale * (q[0] @ k[0, 0] - q[0] @ k[1, 0])
    w0 = scipy.special.expit(delta)
    expect = w0 * v[0, 0] + (1.0 - w0) * v[1, 0]
    got = A.attend(q, k, v, scale)[0]
    assert np.max(np.abs(got - expect)) <= 1e-14


def test_length_one_returns_v_exactly():
    rng = np.random.default_rng(8)
    q = _rand(rng, 4, 16)
    k = _rand(rng, 1, 2, 16)
    v = _rand(rng, 1, 2, 16)
    got = A.attend(q, k, v, 0.25)
    for h in range(4):
        assert np.array_equal(got[h], v[0, h // 2])


def test_zero_query_gives_column_mean():
    rng = np.random.default_rng(9)
    k = _rand(rng, 13, 2, 8)
    v = _rand(rng, 13, 2, 8)
    got = A.attend(np.zeros((4, 8)), k, v, 0.5)
    for h in range(4):
        assert np.allclose(got[h], v[:, h // 2, :].mean(axis=0), rtol=0, atol=1e-14)


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(10)
    q = _rand(rng, 2, 8)
    k = 3.0 * _rand(rng, 40, 1, 8)
    got = A.attend(q, k, np.ones((40, 1, 8)), 1.0)
    assert np.max(np.abs(got - 1.0)) <= 1e-14


def test_one_hot_values_give_the_softmax_weights():
    # V[t] = e_t turns the output into the weight vector itself; it must be
    # non-negative, sum to one and equal scipy's softmax of the scaled logits.
    rng = np.random.default_rng(11)
    length, d = 12, 16
    q = _rand(rng, 2, d)
    k = _rand(rng, length, 1, d)
    v = np.zeros((length, 1, d))
    for t in range(length):
        v[t, 0, t] = 1.0
    scale = 1.0 / math.sqrt(d)
    out = A.attend(q, k, v, scale)
    for h in range(2):
        w = out[h, :length]
        assert np.all(w >= 0) and abs(w.sum() - 1.0) <= 1e-14
        assert np.all(out[h, length:] == 0)
        ref = scipy.special.softmax(scale * (k[:, 0, :] @ q[h]))
        assert np.max(np.abs(w - ref)) <= 1e-15


def test_query_heads_read_their_group_kv_head():
    # KV head g holds the constant value g; query head h must return h // G.
    hq, hkv, d, length = 12, 3, 4, 5
    rng = np.random.default_rng(12)
    q = _rand(rng, hq, d)
    k = _rand(rng, length, hkv, d)
    v = np.zeros((length, hkv, d))
    for g in range(hkv):
        v[:, g, :] = g
    out = A.attend(q, k, v, 1.0)
    for h in range(hq):
        assert np.allclose(out[h], h // (hq // hkv), atol=1e-14)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(13)
    length, d = 20, 8
    k = _rand(rng, length, 1, d)
    v = _rand(rng, length, 1, d)
    j = 13
    k[j] *= 5.0
    q = 10.0 * k[j, 0][None, :] / np.linalg.norm(k[j, 0])
    out = A.attend(q, k, v, 1.0)
    # every other logit is at least this far below key j's
    gap = min(q[0] @ (k[j, 0] - k[t, 0]) for t in range(length) if t != j)
    assert gap > 20
    assert np.max(np.abs(out[0] - v[j, 0])) <= 2 * length * math.exp(-gap) * np.max(np.abs(v))


def test_empty_context_is_zero():
    out = A.attend(np.ones((2, 4)), np.zeros((0, 1, 4)), np.zeros((0, 1, 4)), 1.0)
    assert np.array_equal(out, np.zeros((2, 4)))


def _place(logical, order, bs, nb):
    """Scatter logical rows [L][Hkv][d] into blocks given by ``order``."""
    length, hkv, d = logical.shape
    pool = np.full((nb, hkv, bs, d), np.nan)
    table = []
    for j in range(-(-length // bs)):
        table.append(int(order[j]))
    for t in range(length):
        pool[table[t // bs], :, t % bs, :] = logical[t]
    return pool, table


def test_gather_is_independent_of_block_placement():
    rng = np.random.default_rng(14)
    bs, nb, length, hkv, d = 4, 16, 23, 2, 5
    kl = _rand(rng, length, hkv, d)
    vl = _rand(rng, length, hkv, d)
    q = _rand(rng, 4, d)
    outs = []
    for seed in (1, 2, 3):
        order = np.random.default_rng(seed).permutation(nb)
        kp, table = _place(kl, order, bs, nb)
        vp, _ = _place(vl, order, bs, nb)
        assert np.array_equal(A.gather_paged(kp, table, length, bs), kl)
        outs.append(A.decode_paged(q[None], kp, vp, [table], [length], bs, 0.3)[0])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    assert np.array_equal(outs[0], A.attend(q, kl, vl, 0.3))


def test_contiguous_layout_matches_paged():
    # Request r's sub-tensor sits at r x S in the [max_seqs][Hkv][S][d] tensor.
    rng = np.random.default_rng(15)
    bmax, hkv, s, d = 3, 2, 32, 4
    lengths = [5, 32, 17]
    pool = np.full((bmax, hkv, s, d), np.nan)
    logical = []
    for r, n in enumerate(lengths):
        x = _rand(rng, n, hkv, d)
        logical.append(x)
        for t in range(n):
            pool[r, :, t, :] = x[t]
    flat = pool.reshape(-1)
    for r, n in enumerate(lengths):
        got = A.gather_contiguous(pool, r, n)
        assert np.array_equal(got, logical[r])
        # the same rows, read by plain flat offsets from reqId x S
        base = r * (hkv * s * d)
        for t in range(n):
            for h in range(hkv):
                off = base + h * s * d + t * d
                assert np.array_equal(flat[off:off + d], logical[r][t, h])


def test_append_scatter_worked_example():
    # BS = 4: slot 5 is block 1 row 1, slot 0 is block 0 row 0; -1 is skipped.
    pool = np.zeros((3, 2, 4, 2), dtype=np.float32)
    rows = np.arange(12, dtype=np.float32).reshape(3, 2, 2) + 1
    out = A.append_scatter(pool, [5, -1, 0], rows)
    expect = np.zeros_like(pool)
    expect[1, 0, 1] = [1, 2]
    expect[1, 1, 1] = [3, 4]
    expect[0, 0, 0] = [9, 10]
    expect[0, 1, 0] = [11, 12]
    assert np.array_equal(out, expect)
    assert np.array_equal(pool, np.zeros_like(pool)), "input must not change"


def test_copy_blocks_worked_example():
    pool = np.arange(4 * 1 * 2 * 1, dtype=np.int32).reshape(4, 1, 2, 1)
    out = A.copy_blocks(pool, [(1, 3), (1, 0)])
    assert out[:, 0, :, 0].tolist() == [[2, 3], [2, 3], [4, 5], [2, 3]]


def test_bf16_decoding_matches_torch():
    torch = pytest.importorskip("torch")
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x3EAA, 0x4049,
                     0x0080, 0x7F7F], dtype=np.uint16)
    got = A.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    assert got[0] == 1.0 and got[1] == -2.0 and got[4] == 2.0 ** -133


def test_tile_readers_worked_example():
    # d = 4, VE = 2, BS = 3: K tile [2][3][2], V tile [4][3]; token row o is
    # (K) chunks 0 and 1 of row o, (V) column o.
    k = np.arange(12).reshape(1, 1, 2, 3, 2)
    rows = A.k_rows(k)
    assert rows.shape == (1, 1, 3, 4)
    assert rows[0, 0].tolist() == [[0, 1, 6, 7], [2, 3, 8, 9], [4, 5, 10, 11]]
    v = np.arange(12).reshape(1, 1, 4, 3)
    assert A.v_rows(v)[0, 0].tolist() == [[0, 3, 6, 9], [1, 4, 7, 10], [2, 5, 8, 11]]


def test_pair_tiles_worked_example():
    # fp32 (VE = 4), d = 8, BS = 2: one tile pair of 32 elements labelled by
    # position.  K tile = elements 0..15 as [2][2][4]: token 0 holds chunk 0
    # of row 0 (0..3) and chunk 1 of row 0 (8..11); V tile = elements 16..31
    # as [8][2]: token o of dim e is 16 + 2e + o.
    pair = np.arange(32, dtype=np.float32).reshape(1, 1, 32)
    kt, vt = A.pair_tiles(pair, 8, 2)
    assert kt.shape == (1, 1, 2, 2, 4) and vt.shape == (1, 1, 8, 2)
    assert A.k_rows(kt)[0, 0].tolist() == [[0, 1, 2, 3, 8, 9, 10, 11], [4, 5, 6, 7, 12, 13, 14, 15]]
    assert A.v_rows(vt)[0, 0].tolist() == [[16, 18, 20, 22, 24, 26, 28, 30],
                                           [17, 19, 21, 23, 25, 27, 29, 31]]
    # bf16 bits (VE = 8), d = 8, BS = 1, two heads: head 1's K row is
    # elements 16..23, its V row 24..31
    bits = np.arange(32, dtype=np.uint16).reshape(1, 2, 16)
    kt, vt = A.pair_tiles(bits, 8, 1)
    assert kt.shape == (1, 2, 1, 1, 8) and vt.shape == (1, 2, 8, 1)
    assert A.k_rows(kt)[0, 1, 0].tolist() == list(range(16, 24))
    assert A.v_rows(vt)[0, 1, 0].tolist() == list(range(24, 32))
    # 32-token blocks, fp32 (VE = 4), d = 4: two pairs of 16 rows.  Pair 0:
    # K elements 0..63 (row r: 4r .. 4r+3), V 64..127 (dim e, row r: 64 +
    # 16e + r); pair 1 the same from 128.  Block row 17 is row 1 of pair 1.
    region = np.arange(256, dtype=np.float32).reshape(1, 256)
    kt, vt = A.pair_tiles(region, 4, 32)
    assert kt.shape == (1, 1, 32, 4) and vt.shape == (1, 4, 32)
    kr, vr = A.k_rows(kt)[0], A.v_rows(vt)[0]
    assert kr[0].tolist() == [0, 1, 2, 3] and kr[15].tolist() == [60, 61, 62, 63]
    assert kr[16].tolist() == [128, 129, 130, 131] and kr[17].tolist() == [132, 133, 134, 135]
    assert vr[0].tolist() == [64, 80, 96, 112] and vr[17].tolist() == [193, 209, 225, 241]


def test_contiguous_rows_follow_reqid_times_s():
    # 2 requests, S = 4, BS = 2: request r's blocks are 2r and 2r+1
    rows = np.arange(4 * 1 * 2 * 1).reshape(4, 1, 2, 1)
    per_req = A.contiguous_rows(rows, 2, 4)
    assert per_req[:, 0, :, 0].tolist() == [[0, 1, 2, 3], [4, 5, 6, 7]]
    # flat offset of request r's sub-tensor is r x S x Hkv x d
    assert per_req.reshape(-1).tolist() == rows.reshape(-1).tolist()
