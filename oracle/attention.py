"""Oracle: gather through block tables, textbook decode attention, append scatter.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain float64 NumPy;
nothing is blocked, fused or reordered beyond the definitions below.

Cache layout.  The pages fix none; the C library documents this one, and the
functions here read it as written there:

* One array holds a layer's K and V: one region of ``2*d*BS`` elements per
  (block, KV head), shape ``[units][Hkv][region]``.  A region holds
  ``BS/sub`` tile pairs of ``sub = min(BS, 16)`` token rows: the K tile of
  those rows (``d*sub`` elements), then their V tile (``d*sub``).  The K tile
  is ``[d/VE][sub][VE]`` (the row of a token cut into 16-byte chunks of
  ``VE`` elements, chunk-major), the V tile is ``[d][sub]`` (dimension-major).
  ``pair_tiles`` turns a region into the block's K tile ``[d/VE][BS][VE]``
  and V tile ``[d][BS]``; ``k_rows`` / ``v_rows`` turn those into plain token
  rows ``[units][Hkv][BS][d]``, which is what the gathers read.
* paged: ``units`` are the physical blocks; block ``b`` holds BS consecutive
  token rows of every KV head.
* contiguous: request ``r`` owns the ``S/BS`` consecutive blocks starting at
  block ``r*S/BS``, i.e. the sub-tensor at ``reqId x S`` where S is one
  request's maximum cache size ([VAC] 5.2.3, request-level KV-cache indexing).
  ``contiguous_rows`` views that as ``[max_seqs][Hkv][S][d]``.

A "slot" names one token row: ``slot = u*BS + o`` (``u`` the block, ``o`` the row
inside it); in the contiguous layout that is ``reqId*S + position``.
"""

from __future__ import annotations

import math

import numpy as np


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 numbers given as their raw 16-bit patterns.

    A bfloat16 is the upper half of an IEEE binary32, so shifting the pattern
    into the high 16 bits of a 32-bit word gives the same number as a float32;
    widening to float64 is then exact.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        bits = bits.view(np.uint16)
    as_u32 = bits.astype(np.uint32) << np.uint32(16)
    return as_u32.view(np.float32).astype(np.float64)


def f32_to_f64(x: np.ndarray) -> np.ndarray:
    """Exact widening of float32 values to float64."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# reading the documented tile layout
# --------------------------------------------------------------------------

def pair_tiles(cache: np.ndarray, head_dim: int, block_size: int):
    """K tiles and V tiles of a cache held as (block, head) regions.

    ``cache`` holds raw elements (any dtype; VE = 16 bytes / element size),
    shape ``[..., 2*d*BS]``: per (block, KV head) ``BS/sub`` tile pairs of
    ``sub = min(BS, 16)`` rows, each the K tile ``[d/VE][sub][VE]`` of those
    rows, then their V tile ``[d][sub]``.  Returns the block's tiles
    ``(k_tiles [..., d/VE, BS, VE], v_tiles [..., d, BS])``: row ``o`` of the
    block is row ``o % sub`` of pair ``o // sub``.
    """
    cache = np.asarray(cache)
    assert cache.shape[-1] == 2 * head_dim * block_size, "last axis must be one region"
    lead = cache.shape[:-1]
    sub = min(block_size, 16)
    ve = 16 // cache.itemsize
    pairs = cache.reshape(*lead, block_size // sub, 2, head_dim * sub)
    k = pairs[..., 0, :].reshape(*lead, block_size // sub, head_dim // ve, sub, ve)
    v = pairs[..., 1, :].reshape(*lead, block_size // sub, head_dim, sub)
    # pair p's rows are the block's rows p*sub .. p*sub + sub - 1
    k = np.moveaxis(k, -4, -3).reshape(*lead, head_dim // ve, block_size, ve)
    v = np.moveaxis(v, -3, -2).reshape(*lead, head_dim, block_size)
    return k, v


def k_rows(k_tiles: np.ndarray) -> np.ndarray:
    """K tiles ``[..., d/VE, BS, VE]`` as token rows ``[..., BS, d]``.

    Element (row o, dim e) of a tile is chunk ``e // VE``, row ``o``, lane
    ``e % VE``.
    """
    *lead, nq, bs, ve = k_tiles.shape
    return np.swapaxes(k_tiles, -3, -2).reshape(*lead, bs, nq * ve)


def v_rows(v_tiles: np.ndarray) -> np.ndarray:
    """V tiles ``[..., d, BS]`` as token rows ``[..., BS, d]``."""
    return np.swapaxes(v_tiles, -1, -2)


def contiguous_rows(rows: np.ndarray, max_seqs: int, max_len: int) -> np.ndarray:
    """Token rows ``[max_seqs*S/BS][Hkv][BS][d]`` of a contiguous cache as
    ``[max_seqs][Hkv][S][d]``: request r's blocks, in order, are its tokens."""
    units, hkv, bs, d = rows.shape
    assert units == max_seqs * (max_len // bs)
    per = max_len // bs
    return rows.reshape(max_seqs, per, hkv, bs, d).transpose(0, 2, 1, 3, 4).reshape(
        max_seqs, hkv, max_len, d)


# --------------------------------------------------------------------------
# gather ([ROC] paging paragraph and Terms: block table; [PAS] Summary)
# --------------------------------------------------------------------------

def gather_paged(pool: np.ndarray, table, length: int, block_size: int) -> np.ndarray:
    """Logical K (or V) of one sequence, read through its block table.

    The block table maps the sequence's positions to physical cache blocks
    ([ROC], paging paragraph and the "Block table" term): position ``t`` lives
    in physical block ``table[t // BS]`` at row ``t % BS``.  Blocks need not be
    adjacent ([PAS] Summary).

    pool:   ``[num_blocks][Hkv][BS][d]`` (any float dtype)
    return: ``[length][Hkv][d]`` float64
    """
    nb, hkv, bs, d = pool.shape
    assert bs == block_size
    out = np.empty((length, hkv, d), dtype=np.float64)
    for t in range(length):
        b = int(table[t // block_size])
        assert 0 <= b < nb, f"block id {b} out of range at position {t}"
        out[t] = pool[b, :, t % block_size, :]
    return out


def gather_contiguous(pool: np.ndarray, req_id: int, length: int) -> np.ndarray:
    """Logical K (or V) of one request in a per-request contiguous layout.

    Request ``req_id`` owns the non-overlapping sub-tensor at offset
    ``reqId x S`` of the layer's tensor ([VAC] 5.2.3); in this per-request
    view the token at position ``t`` of KV head ``h`` is row ``t`` of head ``h``.

    pool:   ``[max_seqs][Hkv][S][d]``
    return: ``[length][Hkv][d]`` float64
    """
    bmax, hkv, s, d = pool.shape
    assert 0 <= req_id < bmax and 0 <= length <= s
    out = np.empty((length, hkv, d), dtype=np.float64)
    for t in range(length):
        out[t] = pool[req_id, :, t, :]
    return out


# --------------------------------------------------------------------------
# attention for one decode step
# --------------------------------------------------------------------------

def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``h`` under grouped-query attention.

    The pages say nothing about head grouping; the reading taken is the common
    contiguous grouping: query heads ``g*G .. g*G+G-1`` share KV head ``g``
    with ``G = Hq / Hkv``.
    """
    assert num_q_heads % num_kv_heads == 0
    return h // (num_q_heads // num_kv_heads)


def attention_weights(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Softmax weights of one decode query over a sequence's cached keys.

    q: ``[Hq][d]``, k: ``[L][Hkv][d]`` -> ``[Hq][L]`` float64.
    ``w[h, t] = exp(z_t - max z) / sum_u exp(z_u - max z)`` with
    ``z_t = scale * <q_h, k_t>`` on the KV head of ``h``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    hq = q.shape[0]
    length, hkv, _ = k.shape
    w = np.zeros((hq, length), dtype=np.float64)
    if length == 0:
        return w
    for h in range(hq):
        kv = kv_head_of(h, hq, hkv)
        z = float(scale) * (k[:, kv, :] @ q[h])
        e = np.exp(z - z.max())
        w[h] = e / e.sum()
    return w


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Single-token decode attention, softmax(scale * q K^T) V, per query head.

    q: ``[Hq][d]``, k and v: ``[L][Hkv][d]`` -> ``[Hq][d]`` float64.
    An empty context (L == 0) gives a zero output row (a convention of this
    library; no sequence on the pages is empty).
    """
    q = np.asarray(q, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, d = q.shape
    length, hkv, _ = np.shape(k)
    out = np.zeros((hq, d), dtype=np.float64)
    if length == 0:
        return out
    w = attention_weights(q, k, scale)
    for h in range(hq):
        out[h] = w[h] @ v[:, kv_head_of(h, hq, hkv), :]
    return out


def attend_bruteforce(q, k, v, scale) -> list:
    """The same attention as ``attend`` written as plain Python loops.

    Used only to check ``attend`` on tiny inputs.  Returns nested lists.
    """
    hq = len(q)
    d = len(q[0])
    length = len(k)
    hkv = len(k[0]) if length else 1
    group = hq // hkv
    out = [[0.0] * d for _ in range(hq)]
    if length == 0:
        return out
    for h in range(hq):
        kv = h // group
        logits = []
        for t in range(length):
            acc = 0.0
            for i in range(d):
                acc += float(q[h][i]) * float(k[t][kv][i])
            logits.append(float(scale) * acc)
        top = max(logits)
        expo = [math.exp(z - top) for z in logits]
        total = math.fsum(expo)
        for i in range(d):
            out[h][i] = math.fsum(expo[t] * float(v[t][kv][i]) for t in range(length)) / total
    return out


def decode_paged(q, k_pool, v_pool, tables, lens, block_size, scale) -> np.ndarray:
    """Decode attention for a batch whose cache sits in a paged pool.

    q: ``[B][Hq][d]``; pools ``[NB][Hkv][BS][d]``; ``tables[s]`` the block
    table of sequence ``s``; ``lens[s]`` its context length.  -> ``[B][Hq][d]``.
    """
    out = np.zeros(np.shape(q), dtype=np.float64)
    for s in range(len(lens)):
        length = int(lens[s])
        k = gather_paged(k_pool, tables[s], length, block_size)
        v = gather_paged(v_pool, tables[s], length, block_size)
        out[s] = attend(q[s], k, v, scale)
    return out


# --------------------------------------------------------------------------
# append ([KVP] Observation-1: one new token per request per iteration)
# --------------------------------------------------------------------------

def append_scatter(pool: np.ndarray, slots, new_rows: np.ndarray) -> np.ndarray:
    """Pool after writing each new token's row into its slot.

    Each decode iteration adds exactly one token to every running request
    ([KVP] Observation-1); its K (or V) row goes to the slot the allocator gave
    it.  ``pool`` is token rows ``[units][Hkv][BS][d]`` of raw values (any
    dtype, compared bytewise by callers), ``new_rows`` is ``[n][Hkv][d]`` of the
    same dtype and ``slots[i] = u*BS + o``; a negative slot means "skip this
    row".  Returns a new array; the input is not modified.
    """
    out = np.array(pool, copy=True)
    units, hkv, unit, d = out.shape
    for i, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0:
            continue
        u, o = divmod(slot, unit)
        assert u < units, f"slot {slot} beyond the pool"
        out[u, :, o, :] = new_rows[i]
    return out


def copy_blocks(pool: np.ndarray, pairs) -> np.ndarray:
    """Pool after the copy-on-write copies: block ``dst`` takes block ``src``'s rows.

    Shared blocks are copied only when one of the sharers writes ([PAS] Summary,
    [ROC] "Fragmentation is lost users").  ``pool`` is ``[NB][...]`` (rows or
    tiles: a block is copied whole).
    """
    out = np.array(pool, copy=True)
    for src, dst in pairs:
        out[int(dst)] = pool[int(src)]
    return out
