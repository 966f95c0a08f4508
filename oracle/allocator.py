"""Oracle: a plain model of the host block allocator, and its invariants.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix:

* The cache is cut into fixed blocks of a few tokens, 16 by default; a
  sequence's blocks need not be adjacent and a block table maps its positions
  to blocks ([ROC] paging paragraph, block-size paragraph; [PAS] Summary).
* A sequence takes a new block only when its last block is full, so each
  sequence wastes less than one block ([ROC] paging paragraph).
* Each running request grows by exactly one token per iteration until it ends
  ([KVP] Observation-1).
* Blocks can be shared between samples of one prompt and between requests, and
  a shared block is copied only when written ([PAS] Summary and Key points;
  [ROC] "Fragmentation is lost users").
* A finished or pre-empted request's cache is given back ([ROC]
  "Fragmentation is lost users" and the "Pre-emption" term).
* A pre-empted request's cache can be evicted and swapped back in later
  ([ROC] "Fragmentation is lost users"; [PAS] Summary: the scheduler
  pre-empts requests).
* Utilisation is the share of reserved cache that holds real tokens ([ROC]
  readouts; [PAS] Key points).
* In the contiguous per-request layout the library hands out a reqId in
  ``[0, B)`` and a request's cache sits at ``reqId x S`` ([VAC] 5.2.3).

Readings where the pages are silent (the C library documents the same rules):

* The free list is a stack (last freed, first reused).  Initially blocks are
  taken in ascending id order; ``set_free_order`` replaces that order while no
  block is in use, so that ``order[0]`` is taken first.
* A freed sequence returns its blocks in table order, each pushed when its
  share count reaches zero.  reqIds are a stack too, ``0`` handed out first.
* ``reserve`` is all-or-nothing.  Sequences are processed in the order given.
  A sequence whose next position falls inside a last block that is still shared
  (share count > 1) first copies that block to a fresh one and drops its share
  of the old one; the last remaining holder writes in place.  Full shared
  blocks are never written, hence never copied.
* Swapping (paged only): ``swap_out`` gives a request's blocks back exactly as
  ``free_seq`` does but keeps its id and length; its contents leave as whole
  blocks.  ``swap_in`` takes ``ceil(L / BS)`` blocks off the free stack, all
  or nothing, in the order they come off, and fills them with those contents,
  so sharing is not restored.  A swapped-out request cannot grow, fork or be
  read until it is swapped in; it can be freed.
* Stats: ``tokens`` counts token rows physically held (a shared row once),
  ``reserved_tokens`` is ``used_blocks x BS`` (paged) or ``live requests x S``
  (contiguous), ``utilisation = tokens / reserved_tokens``.
"""

from __future__ import annotations

from dataclasses import dataclass, field

OK = 0
ERR_INVALID_ARG = -1
ERR_NO_BLOCKS = -2
ERR_NO_REQ_ID = -3
ERR_UNKNOWN_SEQ = -4

PAGED = 0
CONTIGUOUS = 1


class AllocError(Exception):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


@dataclass
class _Seq:
    table: list = field(default_factory=list)
    length: int = 0
    swapped: bool = False


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class RefAllocator:
    """Host-side allocator model: one instance models one pool."""

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int,
                 max_seq_len: int, layout: int = PAGED):
        if layout == PAGED:
            if num_blocks <= 0 or block_size <= 0:
                raise AllocError(ERR_INVALID_ARG, "paged pool needs blocks")
        if max_seqs <= 0 or max_seq_len <= 0:
            raise AllocError(ERR_INVALID_ARG, "max_seqs and max_seq_len must be > 0")
        self.layout = layout
        self.num_blocks = num_blocks if layout == PAGED else 0
        self.block_size = block_size
        self.max_seqs = max_seqs
        self.max_seq_len = max_seq_len
        self.refcount = [0] * self.num_blocks
        self.fill = [0] * self.num_blocks
        # stack: the end of the list is taken first
        self.free = list(range(self.num_blocks - 1, -1, -1))
        self.free_ids = list(range(max_seqs - 1, -1, -1))
        self.seqs: dict[int, _Seq] = {}
        self.cow_copies = 0

    # -- placement ---------------------------------------------------------
    def set_free_order(self, order) -> None:
        order = [int(b) for b in order]
        if self.layout != PAGED:
            raise AllocError(ERR_INVALID_ARG, "no blocks in a contiguous pool")
        if len(self.free) != self.num_blocks:
            raise AllocError(ERR_INVALID_ARG, "free order can only be set while no block is used")
        if sorted(order) != list(range(self.num_blocks)):
            raise AllocError(ERR_INVALID_ARG, "free order must be a permutation of all blocks")
        self.free = order[::-1]

    # -- sequences ---------------------------------------------------------
    def add(self) -> int:
        if not self.free_ids:
            raise AllocError(ERR_NO_REQ_ID, "all request ids are in use")
        rid = self.free_ids.pop()
        self.seqs[rid] = _Seq()
        return rid

    def _get(self, rid: int) -> _Seq:
        if rid not in self.seqs:
            raise AllocError(ERR_UNKNOWN_SEQ, f"request {rid} is not live")
        return self.seqs[rid]

    def _resident(self, rid: int) -> _Seq:
        s = self._get(rid)
        if s.swapped:
            raise AllocError(ERR_INVALID_ARG, f"request {rid} is swapped out")
        return s

    def fork(self, parent: int) -> int:
        if self.layout != PAGED:
            raise AllocError(ERR_INVALID_ARG, "sharing needs the paged layout")
        p = self._resident(parent)
        if not self.free_ids:
            raise AllocError(ERR_NO_REQ_ID, "all request ids are in use")
        rid = self.free_ids.pop()
        self.seqs[rid] = _Seq(table=list(p.table), length=p.length)
        for b in p.table:
            self.refcount[b] += 1
        return rid

    def _give_back(self, s: _Seq) -> None:
        for b in s.table:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.fill[b] = 0
                self.free.append(b)
        s.table = []

    def free_seq(self, rid: int) -> None:
        s = self._get(rid)
        self._give_back(s)
        del self.seqs[rid]
        self.free_ids.append(rid)

    # -- pre-emption by swapping -----------------------------------------------
    def swap_out(self, rid: int) -> list:
        """Evict rid's cache; return the blocks whose contents leave, in order."""
        if self.layout != PAGED:
            raise AllocError(ERR_INVALID_ARG, "swapping needs the paged layout")
        s = self._resident(rid)
        blocks = list(s.table)
        self._give_back(s)
        s.swapped = True
        return blocks

    def swap_in(self, rid: int) -> list:
        """Bring rid back into fresh blocks; return its new table."""
        if self.layout != PAGED:
            raise AllocError(ERR_INVALID_ARG, "swapping needs the paged layout")
        s = self._get(rid)
        if not s.swapped:
            raise AllocError(ERR_INVALID_ARG, f"request {rid} is not swapped out")
        n = ceil_div(s.length, self.block_size)
        if n > len(self.free):
            raise AllocError(ERR_NO_BLOCKS, f"need {n} blocks, {len(self.free)} free")
        for j in range(n):
            b = self.free.pop()
            self.refcount[b] = 1
            self.fill[b] = min(self.block_size, s.length - j * self.block_size)
            s.table.append(b)
        s.swapped = False
        return list(s.table)

    # -- growth --------------------------------------------------------------
    def blocks_needed(self, req_ids, counts) -> tuple[int, int]:
        """(fresh blocks, copy-on-write copies) a reserve call would take."""
        bs = self.block_size
        share = {}
        need = 0
        copies = 0
        for rid, c in zip(req_ids, counts):
            s = self.seqs[rid]
            if c == 0:
                continue
            if s.length % bs != 0:
                last = s.table[-1]
                rc = share.get(last, self.refcount[last])
                if rc > 1:
                    copies += 1
                    share[last] = rc - 1
            need += ceil_div(s.length + c, bs) - ceil_div(s.length, bs)
        return need + copies, copies

    def reserve(self, req_ids, counts=None):
        """Grow each listed sequence; return (slots, cow_pairs).

        ``counts[i]`` tokens are added to ``req_ids[i]`` (one each if None).
        Slots come out in order: all of ``req_ids[0]``'s, then ``req_ids[1]``'s.
        """
        req_ids = [int(r) for r in req_ids]
        counts = [1] * len(req_ids) if counts is None else [int(c) for c in counts]
        if len(counts) != len(req_ids):
            raise AllocError(ERR_INVALID_ARG, "one count per request")
        if len(set(req_ids)) != len(req_ids):
            raise AllocError(ERR_INVALID_ARG, "a request may appear once per call")
        for rid, c in zip(req_ids, counts):
            s = self._resident(rid)
            if c < 0:
                raise AllocError(ERR_INVALID_ARG, "negative token count")
            if s.length + c > self.max_seq_len:
                raise AllocError(ERR_INVALID_ARG, "request would exceed max_seq_len")
        slots: list[int] = []
        pairs: list[tuple[int, int]] = []
        if self.layout == CONTIGUOUS:
            for rid, c in zip(req_ids, counts):
                s = self.seqs[rid]
                for _ in range(c):
                    slots.append(rid * self.max_seq_len + s.length)
                    s.length += 1
            return slots, pairs
        need, _ = self.blocks_needed(req_ids, counts)
        if need > len(self.free):
            raise AllocError(ERR_NO_BLOCKS, f"need {need} blocks, {len(self.free)} free")
        bs = self.block_size
        for rid, c in zip(req_ids, counts):
            s = self.seqs[rid]
            for _ in range(c):
                pos = s.length
                if pos % bs == 0:
                    b = self.free.pop()
                    self.refcount[b] = 1
                    self.fill[b] = 0
                    s.table.append(b)
                else:
                    b = s.table[-1]
                    if self.refcount[b] > 1:
                        nb = self.free.pop()
                        self.refcount[nb] = 1
                        self.fill[nb] = self.fill[b]
                        self.refcount[b] -= 1
                        s.table[-1] = nb
                        pairs.append((b, nb))
                        self.cow_copies += 1
                        b = nb
                slots.append(b * bs + pos % bs)
                self.fill[b] = pos % bs + 1
                s.length += 1
        return slots, pairs

    # -- readouts ------------------------------------------------------------
    def table(self, rid: int) -> list:
        return list(self._resident(rid).table)

    def length(self, rid: int) -> int:
        return self._get(rid).length

    def stats(self) -> dict:
        resident = [s for s in self.seqs.values() if not s.swapped]
        swapped = [s for s in self.seqs.values() if s.swapped]
        if self.layout == PAGED:
            used = self.num_blocks - len(self.free)
            tokens = sum(self.fill[b] for b in range(self.num_blocks) if self.refcount[b] > 0)
            reserved = used * self.block_size
        else:
            used = 0
            tokens = sum(s.length for s in resident)
            reserved = len(resident) * self.max_seq_len
        return {
            "free_blocks": len(self.free),
            "used_blocks": used,
            "tokens": tokens,
            "logical_tokens": sum(s.length for s in resident),
            "reserved_tokens": reserved,
            "live_seqs": len(resident),
            "cow_copies": self.cow_copies,
            "shared_blocks": sum(1 for rc in self.refcount if rc > 1),
            "utilisation": (tokens / reserved) if reserved else 0.0,
            "swapped_seqs": len(swapped),
            "swapped_tokens": sum(s.length for s in swapped),
        }


def check_invariants(a: RefAllocator) -> None:
    """Raise AssertionError if the allocator state breaks a rule of the pages.

    * every block is either free or referenced, never both, never twice free;
    * a block's share count equals the number of tables that hold it;
    * each table has exactly ceil(L / BS) blocks, so the waste of a sequence,
      ``len(table)*BS - L``, is below one block ([ROC] paging paragraph);
    * the rows a block holds agree with every holder's length.
    """
    if a.layout != PAGED:
        for rid, s in a.seqs.items():
            assert 0 <= rid < a.max_seqs and 0 <= s.length <= a.max_seq_len
        assert len(set(a.free_ids)) == len(a.free_ids)
        assert set(a.free_ids).isdisjoint(a.seqs)
        assert len(a.free_ids) + len(a.seqs) == a.max_seqs
        return
    bs = a.block_size
    held = [0] * a.num_blocks
    for s in a.seqs.values():
        if s.swapped:
            assert s.table == [], "a swapped-out request holds blocks"
            continue
        assert len(s.table) == ceil_div(s.length, bs), "table length != ceil(L/BS)"
        waste = len(s.table) * bs - s.length
        assert 0 <= waste < bs, "waste must be under one block"
        for j, b in enumerate(s.table):
            held[b] += 1
            assert a.fill[b] == min(bs, s.length - j * bs), "block fill disagrees with a holder"
    free = set(a.free)
    assert len(free) == len(a.free), "a block is free twice"
    for b in range(a.num_blocks):
        assert a.refcount[b] == held[b], f"block {b}: share count {a.refcount[b]} != holders {held[b]}"
        assert (b in free) == (held[b] == 0), f"block {b} free/used mismatch"
    assert len(a.free_ids) + len(a.seqs) == a.max_seqs
    assert set(a.free_ids).isdisjoint(a.seqs)


class ContentModel:
    """Token-label model of the pool, to check sharing and copy-on-write.

    Every slot holds a label; ``reserve`` writes ``(rid, position, serial)`` to
    each new slot and copy-on-write pairs copy whole blocks, as the device would.
    ``history`` is what each sequence should see: a fork inherits its parent's
    history; later tokens are its own.  ``check`` gathers every live sequence's
    labels through its table and compares with its history, so a write into a
    block that another sequence still shares shows up at once.
    """

    def __init__(self, alloc: RefAllocator):
        self.a = alloc
        self.rows: dict[int, object] = {}
        self.history: dict[int, list] = {rid: [] for rid in alloc.seqs}
        self.images: dict[int, list] = {}   # swapped-out request -> its rows, whole blocks
        self.serial = 0

    def add(self) -> int:
        rid = self.a.add()
        self.history[rid] = []
        return rid

    def fork(self, parent: int) -> int:
        rid = self.a.fork(parent)
        self.history[rid] = list(self.history[parent])
        return rid

    def free_seq(self, rid: int) -> None:
        self.a.free_seq(rid)
        del self.history[rid]
        self.images.pop(rid, None)

    def swap_out(self, rid: int) -> None:
        """Whole blocks leave, rows past the request's length included."""
        blocks = self.a.swap_out(rid)
        bs = self.a.block_size
        self.images[rid] = [self.rows.get(b * bs + o) for b in blocks for o in range(bs)]

    def swap_in(self, rid: int) -> None:
        table = self.a.swap_in(rid)
        bs = self.a.block_size
        image = self.images.pop(rid)
        for j, b in enumerate(table):
            for o in range(bs):
                label = image[j * bs + o]
                if label is None:
                    self.rows.pop(b * bs + o, None)
                else:
                    self.rows[b * bs + o] = label

    def reserve(self, req_ids, counts=None):
        slots, pairs = self.a.reserve(req_ids, counts)
        bs = self.a.block_size
        for src, dst in pairs:
            for o in range(bs):
                if src * bs + o in self.rows:
                    self.rows[dst * bs + o] = self.rows[src * bs + o]
                else:
                    self.rows.pop(dst * bs + o, None)
        counts = [1] * len(req_ids) if counts is None else counts
        k = 0
        for rid, c in zip(req_ids, counts):
            for _ in range(c):
                label = (rid, len(self.history[rid]), self.serial)
                self.serial += 1
                self.rows[slots[k]] = label
                self.history[rid].append(label)
                k += 1
        return slots, pairs

    def check(self) -> None:
        bs = self.a.block_size
        for rid, hist in self.history.items():
            if rid in self.images:
                image = self.images[rid]
                assert image[:len(hist)] == hist, f"request {rid}'s image holds other tokens"
                continue
            table = self.a.table(rid)
            seen = [self.rows.get(table[t // bs] * bs + t % bs) for t in range(len(hist))]
            assert seen == hist, f"request {rid} sees other tokens than it wrote"
