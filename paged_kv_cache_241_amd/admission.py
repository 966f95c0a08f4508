"""Admission and cache utilisation under continuous batching, over libpa.so's allocator.

The "Running Out of Cache" page (Workshop box, "Fragmentation is lost users")
compares a contiguous reservation per request with paged allocation by
simulation: Llama 3 8B in BF16 on one H100 with about 56 GB of KV cache after
weights, Poisson arrivals, prompt and output lengths exponential with means
1024 and 256, a maximum length of 8192, continuous batching; contiguous
reserves 8192 tokens per request, paged takes 16-token blocks as needed; pass
times are roofline estimates from the H100's published figures (989 TFLOP/s
dense BF16, 3.35 TB/s) at 60% and 80% of peak, plus 0.2 ms per pass.  This
module runs that comparison with the library's own allocator making every
admission decision (a host-only pool: no GPU).

Readings where the page is silent:

* A pass advances every running request by one token and prefills the
  requests admitted just before it; a request's first token is out at the end
  of its prefill pass (time to first token = that time - arrival).
* Admission is first come, first served.  Contiguous: a request needs a free
  reqId (max_seqs = cache tokens // 8192).  Paged: its context's blocks, with
  1% of all blocks kept free.
* A paged pass that cannot grow every running request pre-empts the request
  admitted last: its blocks go back and it waits at the head of the queue to
  be prefilled again (recomputation), until the rest fits.
* The roofline pass time: flops = 2 x parameters x tokens processed plus
  attention (4 x layers x hidden per token per context token, half of it for
  a prompt's own causal context); bytes = the weights once, plus the K/V read
  and written.  Time = max(flops / (0.6 x 989 TFLOP/s), bytes / (0.8 x 3.35
  TB/s)) + 0.2 ms.
* Llama 3 8B: 8.03e9 parameters, 32 layers, hidden 4096, 128 KiB of K/V per
  token (the per-token footprint the allocation-patterns page gives).
* The run length.  The page states none, and it matters for the contiguous
  reservation: at 18 requests a second its 52 slots serve fewer requests a
  second than arrive, so the queue never drains and the median time to first
  token grows with the run (300 requests: 0.4 s, 600: 2.8 s, 1000: 6.0 s,
  2000: 14.1 s on seed 2416), while paging stays at about 0.05 s at any
  length.  1000 requests (about 55 s of arrivals) is the default: it is the
  length at which the page's 6.01 s comes out.

The readouts: peak and mean running requests, the time-averaged share of
reserved cache holding real tokens, and the median time to first token.
"""

from __future__ import annotations

import argparse
import json
from collections import deque
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Model:
    params: float = 8.03e9
    layers: int = 32
    hidden: int = 4096
    kv_bytes_per_token: int = 131072
    weight_bytes_per_param: int = 2


@dataclass(frozen=True)
class Hardware:
    flops: float = 989e12
    bandwidth: float = 3.35e12
    flops_share: float = 0.6
    bandwidth_share: float = 0.8
    pass_overhead_s: float = 0.2e-3


@dataclass(frozen=True)
class Workload:
    rate: float = 18.0            # requests per second (Poisson)
    requests: int = 1000
    prompt_mean: float = 1024.0
    output_mean: float = 256.0
    max_len: int = 8192
    seed: int = 2416


def draw_requests(w: Workload):
    """(arrival s, prompt tokens, output tokens) per request, seeded."""
    rng = np.random.default_rng(w.seed)
    gaps = rng.exponential(1.0 / w.rate, w.requests)
    prompt = np.maximum(1, np.rint(rng.exponential(w.prompt_mean, w.requests))).astype(np.int64)
    output = np.maximum(1, np.rint(rng.exponential(w.output_mean, w.requests))).astype(np.int64)
    prompt = np.minimum(prompt, w.max_len - 1)
    output = np.minimum(output, w.max_len - prompt)
    return list(zip(np.cumsum(gaps).tolist(), prompt.tolist(), output.tolist()))


def pass_seconds(prefill_ctx, decode_ctx, m: Model = Model(), hw: Hardware = Hardware()) -> float:
    """Roofline time of one pass: prompts of the given lengths, and one token
    for each running request with the given context."""
    p_tokens = float(sum(prefill_ctx))
    d_tokens = float(len(decode_ctx))
    attn = 4.0 * m.layers * m.hidden * (sum(c * c / 2.0 for c in prefill_ctx) + float(sum(decode_ctx)))
    flops = 2.0 * m.params * (p_tokens + d_tokens) + attn
    kv = m.kv_bytes_per_token * (float(sum(decode_ctx)) + p_tokens + d_tokens)
    nbytes = m.params * m.weight_bytes_per_param + kv
    return max(flops / (hw.flops_share * hw.flops),
               nbytes / (hw.bandwidth_share * hw.bandwidth)) + hw.pass_overhead_s


class NoRoom(Exception):
    """The allocator cannot take the request (no reqId, or no blocks)."""


class LibAllocator:
    """The library's host allocator (a host-only pool), as the simulation sees it."""

    def __init__(self, mode: str, cache_tokens: int, max_len: int = 8192, block_size: int = 16):
        from . import capi
        from .pool import Pool

        self.capi = capi
        self.mode = mode
        if mode == "contiguous":
            self.pool = Pool(1, 0, block_size, 1, 64, "f32", "contiguous",
                             max_seqs=cache_tokens // max_len, max_seq_len=max_len, host_only=True)
            self.watermark = 0
        else:
            nb = cache_tokens // block_size
            self.pool = Pool(1, nb, block_size, 1, 64, "f32", "paged", max_seqs=8192,
                             max_seq_len=max_len, host_only=True)
            self.watermark = nb // 100
        self.block_size = block_size

    def _room(self, fn, *a):
        try:
            return fn(*a)
        except self.capi.PaError as e:
            if e.status in (self.capi.PA_ERR_NO_BLOCKS, self.capi.PA_ERR_NO_REQ_ID):
                raise NoRoom(str(e)) from None
            raise

    def admit(self, tokens: int) -> int:
        if self.mode == "paged":
            need = -(-tokens // self.block_size)
            if self.pool.stats()["free_blocks"] - need < self.watermark:
                raise NoRoom("watermark")
        rid = self._room(self.pool.add)
        try:
            self._room(self.pool.reserve, [rid], [tokens])
        except NoRoom:
            self.pool.free_seq(rid)
            raise
        return rid

    def grow(self, rids) -> None:
        if rids:
            self._room(self.pool.reserve, rids, None)

    def free(self, rid: int) -> None:
        self.pool.free_seq(rid)

    def stats(self) -> dict:
        return self.pool.stats()


@dataclass
class _Req:
    idx: int
    arrival: float
    prompt: int
    output: int
    done: int = 0            # output tokens produced
    rid: int = -1
    ttft: float | None = None


@dataclass
class Result:
    mode: str
    ttft: list = field(default_factory=list)
    peak_running: int = 0
    mean_running: float = 0.0
    utilisation: float = 0.0
    preemptions: int = 0
    passes: int = 0
    seconds: float = 0.0
    trace: list = field(default_factory=list)   # per pass: (admitted idx, pre-empted idx)

    def summary(self) -> dict:
        t = np.array(self.ttft)
        return {"mode": self.mode, "requests": len(self.ttft),
                "median_ttft_s": round(float(np.median(t)), 4),
                "p90_ttft_s": round(float(np.percentile(t, 90)), 4),
                "peak_running": self.peak_running, "mean_running": round(self.mean_running, 1),
                "utilisation": round(self.utilisation, 4), "preemptions": self.preemptions,
                "passes": self.passes, "simulated_s": round(self.seconds, 2)}


def simulate(alloc, reqs, m: Model = Model(), hw: Hardware = Hardware(), mode: str = "") -> Result:
    """Continuous batching over ``alloc`` (admit / grow / free / stats, raising
    NoRoom) until every request in ``reqs`` has finished."""
    res = Result(mode=mode or getattr(alloc, "mode", ""))
    pending = deque(_Req(i, a, p, o) for i, (a, p, o) in enumerate(reqs))
    waiting: deque = deque()
    running: list = []
    t = 0.0
    busy = 0.0
    util_area = 0.0
    run_area = 0.0
    while pending or waiting or running:
        while pending and pending[0].arrival <= t:
            waiting.append(pending.popleft())
        if not waiting and not running:
            t = pending[0].arrival
            continue
        # admit in arrival order while the allocator can hold the context
        admitted = []
        while waiting:
            r = waiting[0]
            try:
                r.rid = alloc.admit(r.prompt + r.done)
            except NoRoom:
                break
            waiting.popleft()
            admitted.append(r)
        # every running request grows by the token it is fed back this pass
        preempted = []
        while running:
            try:
                alloc.grow([r.rid for r in running])
                break
            except NoRoom:
                victim = (admitted or running).pop()
                alloc.free(victim.rid)
                victim.rid = -1
                waiting.appendleft(victim)
                preempted.append(victim.idx)
                res.preemptions += 1
        if not admitted and not running:
            # nothing fits (a lone prompt larger than the free cache): wait
            t = pending[0].arrival if pending else t + hw.pass_overhead_s
            continue
        dt = pass_seconds([r.prompt + r.done for r in admitted],
                          [r.prompt + r.done for r in running], m, hw)
        st = alloc.stats()
        if st["reserved_tokens"]:
            util_area += dt * st["tokens"] / st["reserved_tokens"]
        t += dt
        busy += dt
        res.passes += 1
        res.trace.append((tuple(r.idx for r in admitted), tuple(preempted)))
        for r in admitted:
            if r.ttft is None:
                r.ttft = t - r.arrival
            r.done += 1
        for r in running:
            r.done += 1
        still = []
        for r in running + admitted:
            if r.done >= r.output:
                alloc.free(r.rid)
                res.ttft.append((r.idx, r.ttft))
            else:
                still.append(r)
        running = still
        res.peak_running = max(res.peak_running, len(running))
        run_area += dt * len(running)
    res.ttft = [x for _, x in sorted(res.ttft)]
    res.seconds = t
    res.utilisation = util_area / busy if busy else 0.0
    res.mean_running = run_area / busy if busy else 0.0
    return res


def workshop(rate: float = 18.0, requests: int = 1000, seed: int = 2416,
             cache_bytes: int = 56_000_000_000) -> dict:
    """Both allocations on the same seeded requests."""
    m = Model()
    tokens = cache_bytes // m.kv_bytes_per_token
    reqs = draw_requests(Workload(rate=rate, requests=requests, seed=seed))
    out = {}
    for mode in ("contiguous", "paged"):
        out[mode] = simulate(LibAllocator(mode, tokens), reqs, m, mode=mode).summary()
    return {"rate": rate, "requests": requests, "seed": seed, "cache_tokens": tokens, **out}


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--rate", type=float, default=18.0)
    ap.add_argument("--requests", type=int, default=1000)
    ap.add_argument("--seed", type=int, default=2416)
    args = ap.parse_args(argv)
    print(json.dumps(workshop(args.rate, args.requests, args.seed)))


if __name__ == "__main__":
    main()
