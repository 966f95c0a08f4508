"""CPU oracle for paged decode attention and its block allocator.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``paged_kv_cache_241_amd`` and its HIP library) never imports,
links or calls it, and this package imports nothing from the product.

Everything here is the plain definition of what the hot path computes, written
out slowly and in float64:

* ``attention``  - gather a sequence's K/V through its block table (or through
  the request-offset rule of a contiguous per-request layout), textbook softmax
  attention, the append scatter, and a pure-Python brute force used to check
  the NumPy version.
* ``allocator``  - a plain model of the host block allocator: free list,
  share counts, allocate-on-fill, fork, copy-on-write, free, utilisation; plus
  an invariant checker and a token-label content model.
* ``capacity``   - per-token KV footprint and the admission closed forms of
  the workshop on the "Running Out of Cache" page.

Sources (the four pages this work follows):

* [KVP]  "Insights into LLM Serving Systems: KV-Cache Memory Allocation
  Patterns" (vAttention paper, section 4, Observations 1 and 2).
* [PAS]  "Efficient Memory Management for Large Language Model Serving with
  PagedAttention" (summary page: Summary, Key points).
* [ROC]  "Running Out of Cache" (serving plate XXIII.3: the paging paragraph,
  the Workshop box, "Fragmentation is lost users", Terms).
* [VAC]  "Leveraging Low-Level CUDA APIs for vAttention's Dynamic Memory"
  (vAttention paper, sections 5.2.1-5.2.3).

Parity status: every function here is pinned by tests under ``tests/`` marked
``not gpu`` (brute force, closed forms, special cases, the pages' printed
footprints and workshop readouts, allocator invariants).  None is
"parity unpinned".
"""

from . import allocator, attention, capacity  # noqa: F401
