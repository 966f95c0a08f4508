"""Oracle: per-token KV footprint and the admission arithmetic of the workshop.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* [KVP] Observation-2 prints the per-token KV footprint, over all layers, of
  Yi-6B, Llama-3-8B and Yi-34B (64, 128 and 240 KB).  With K and V each holding
  one row of ``head_dim`` 16-bit values per KV head per layer, the footprint is
  ``2 * layers * kv_heads * head_dim * bytes_per_element``.
* [ROC] Workshop and "Fragmentation is lost users": about 56 GB of cache,
  Llama 3 8B in BF16, requests of mean prompt 1024 and mean output 256 tokens,
  contiguous reservations of 8192 tokens against 16-token blocks; the page
  reads out 52 against 333 requests (6.4x) and 15% against 99% of the reserved
  cache holding real tokens.
"""

from __future__ import annotations

import math


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elt_bytes: int) -> int:
    """Bytes one token occupies in the KV cache, K plus V, over all layers."""
    return 2 * num_layers * num_kv_heads * head_dim * elt_bytes


def cache_tokens(cache_bytes: int, bytes_per_token: int) -> int:
    """Whole tokens a cache of ``cache_bytes`` can hold."""
    return cache_bytes // bytes_per_token


def contiguous_admissions(tokens: int, max_len: int) -> int:
    """Requests that fit when each reserves ``max_len`` tokens up front."""
    return tokens // max_len


def paged_admissions(tokens: int, block_size: int, request_len: int) -> int:
    """Requests of ``request_len`` tokens that fit in whole blocks of ``block_size``."""
    return (tokens // block_size) // math.ceil(request_len / block_size)


def contiguous_utilisation(lengths, max_len: int) -> float:
    """Share of contiguous reservations that holds real tokens."""
    lengths = list(lengths)
    return sum(lengths) / (len(lengths) * max_len)


def paged_utilisation(lengths, block_size: int) -> float:
    """Share of allocated blocks that holds real tokens (last-block waste only)."""
    lengths = list(lengths)
    return sum(lengths) / sum(math.ceil(n / block_size) * block_size for n in lengths)
