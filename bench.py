"""Benchmark of the paged decode hot path on one MI355X.

One step = one decode iteration of the whole batch over every layer pool:
  host  pa_reserve: one new token per sequence (allocate-on-fill, copy-on-write)
  H2D   slots, context lengths, and block tables when a block was handed out
        (pinned, asynchronous)
  GPU   pa_copy_blocks for any copy-on-write pairs
        pa_append_decode for each layer: the new token's K/V stored into its
        slot and paged attention over the context, in one launch (split-K
        merge if needed); --separate-append uses pa_append_kv + pa_decode
NL distinct layer pools are rotated so that the 256 MB Infinity Cache cannot
serve repeated reads.  Contexts grow by one token per step; the workload's
prefill is set so that the timed steps are centred on the nominal context.

Prints ONE JSON line: KV-read GB/s over the timed steps (metric), the decode
kernels' roofline fraction from HIP events, and the CPU oracle's rate.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth
TIMING_EVERY = 4        # timed steps whose decode launches HIP events bracket
METRIC = "paged decode-attn KV GB/s (% of HBM peak), Llama-3-8B shape, batch 64"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 100 steps (39 ms at the Llama-3-8B shape): over 20, the first step's host work and the
    # closing synchronisation, which no step overlaps, were 1.5% of the timed region
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (2 = the metric's)")
    ap.add_argument("--layout", default="paged", choices=["paged", "contiguous", "vmm"],
                    help="vmm: the contiguous layout with caches mapped on demand (ROCm VMM)")
    ap.add_argument("--prompt-len", type=int, default=0, help="workload 5: prompt length")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--block-size", type=int, default=0, help="tokens per block (0: workload's, 16)")
    ap.add_argument("--batch", type=int, default=0,
                    help="workloads 2 and 4: number of sequences (0: the workload's)")
    ap.add_argument("--context", type=int, default=0,
                    help="workloads 2 and 4: context length (0: the workload's)")
    ap.add_argument("--shared-prefix", type=int, default=0, metavar="TOKENS",
                    help="decode with pa_decode_shared in partitions of TOKENS tokens (samples "
                         "sharing a prompt read its blocks once)")
    ap.add_argument("--separate-append", action="store_true",
                    help="pa_append_kv then pa_decode per layer instead of one pa_append_decode")
    ap.add_argument("--plan-per-layer", action="store_true",
                    help="each layer's call makes its own work plan (pa_decode / pa_append_decode) "
                         "instead of one pa_decode_plan per step and the planned calls")
    ap.add_argument("--layers", type=int, default=0, help="layer pools rotated (0: workload's)")
    ap.add_argument("--time-every", type=int, default=TIMING_EVERY, metavar="K",
                    help="HIP events bracket the decode launches of every K-th timed step")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle sample budget")
    ap.add_argument("--swap-seqs", type=int, default=0, metavar="N",
                    help="after the timed steps, swap N requests out to pinned host memory "
                         "and back in, and report the rates")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hbm-probe", action="store_true",
                    help="skip the achievable-read-bandwidth probe (bench_read_probe)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized buffer 3 times (calibrates byte counters)")
    ap.add_argument("--read-probe", type=int, default=0, metavar="MIB",
                    help="only time plain reductions over a MIB-sized buffer (achievable read rate)")
    return ap.parse_args()


def hbm_probe() -> dict | None:
    """Best read rate of bench_read_probe (plain stream and 4 KiB tiles), GB/s."""
    import subprocess

    exe = os.path.join(ROOT, "bench_read_probe")
    if not os.path.exists(exe):
        return None
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    if res.returncode != 0:
        return None
    best = {}
    for line in res.stdout.splitlines():
        parts = line.split()
        if len(parts) == 3 and not parts[0].endswith("_us"):
            best[parts[0]] = max(best.get(parts[0], 0.0), float(parts[2]))
    return best


def read_probe(mib: int) -> None:
    """Achievable HBM read rate: plain device reductions over a large buffer."""
    import torch

    n = mib * (1 << 20) // 2
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    res = {}
    for name, fn in (("sum", lambda: x.sum(dtype=torch.float32)), ("amax", lambda: x.amax())):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[name] = round(n * 2 * 10 / (a.elapsed_time(b) / 1e3) / 1e9, 1)
    print(json.dumps({"read_probe_bytes": n * 2, "gbs": res}), flush=True)


def copy_probe(mib: int) -> None:
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch

    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


class Bench:
    """The workload built in device memory through libpa.so."""

    def __init__(self, cfg, layout, num_layers, extra_steps, partition_tokens):
        import torch

        import workloads as W
        from paged_kv_cache_241_amd import Pool

        self.torch = torch
        self.cfg = cfg
        # "vmm": the contiguous layout with its caches mapped on demand
        self.vmm = layout == "vmm"
        layout = "contiguous" if self.vmm else layout
        self.layout = layout
        self.nl = num_layers
        self.pt = partition_tokens
        dev = torch.device("cuda")
        self.dev = dev
        pl = W.plan(cfg)
        self.pl = pl
        bs = cfg.block_size
        headroom = len(pl.batch_handles) * (-(-extra_steps // bs) + 1)
        nb = pl.num_blocks + headroom
        self.max_seqs = 4096 if layout == "paged" else cfg.batch
        elt = 2 if cfg.kv_dtype == "bf16" else 4
        # demand paging may map at most what the plain contiguous pool reserves
        full = 2 * num_layers * self.max_seqs * cfg.max_seq_len * cfg.num_kv_heads * cfg.head_dim * elt
        self.pool = Pool(num_layers, nb, bs, cfg.num_kv_heads, cfg.head_dim, cfg.kv_dtype, layout,
                         max_seqs=self.max_seqs, max_seq_len=cfg.max_seq_len, device=dev,
                         vmm_bytes=full if self.vmm else None)
        self.full_bytes = full
        self.reserve_s = 0.0   # host time inside pa_reserve during the prefill
        self.step_reserve_s = 0.0   # host time inside the steps' pa_reserve calls
        if layout == "paged":
            order = np.concatenate([W.free_order(pl.num_blocks, cfg.seed),
                                    np.arange(pl.num_blocks, nb, dtype=np.int32)])
            self.pool.set_free_order(order)
        # per-layer values; the prefill writes every layer through pa_append_kv
        self.q, self.rows = [], []
        for layer in range(num_layers):
            q, kr, vr = W.values(cfg, pl, dev, layer=layer)
            self.q.append(q)
            self.rows.append((kr, vr))
        self.length = {}
        self.rids = {}

        pool = self.pool

        class Tracked:
            def add(_):
                r = pool.add()
                self.length[r] = 0
                return r

            def fork(_, parent):
                r = pool.fork(parent)
                self.length[r] = self.length[parent]
                return r

            def free_seq(_, rid):
                pool.free_seq(rid)
                del self.length[rid]

            def reserve(_, rids, counts):
                t0 = time.perf_counter()
                out = pool.reserve(rids, counts)
                self.reserve_s += time.perf_counter() - t0
                for r, c in zip(rids, counts):
                    self.length[r] += c
                return out

        W.run_ops(pl.ops, Tracked(), self.rids, on_reserve=self._prefill)
        torch.cuda.synchronize()
        self.prefill_mapped = self.pool.vmm_stats()["mapped_bytes"] if self.vmm else 0
        for layer in range(num_layers):   # values no longer needed
            self.rows[layer] = None
        self.batch = [self.rids[h] for h in pl.batch_handles]
        self.rids_np = np.array(self.batch, dtype=np.int32)
        b = len(self.batch)
        self.req_ids = torch.tensor(self.batch, dtype=torch.int32, device=dev)
        g = torch.Generator(device=dev)
        g.manual_seed(cfg.seed + 99)
        tdt = self.pool.torch_dtype
        self.k_new = [torch.randn((b, cfg.num_kv_heads, cfg.head_dim), generator=g, device=dev).to(tdt)
                      for _ in range(num_layers)]
        self.v_new = [torch.randn((b, cfg.num_kv_heads, cfg.head_dim), generator=g, device=dev).to(tdt)
                      for _ in range(num_layers)]
        self.out = torch.empty((b, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
        self.max_context = cfg.max_seq_len   # sizes the workspace: enough for any step
        self.stride = -(-cfg.max_seq_len // bs)
        self.ws = None
        self.scale = float(np.float32(1.0 / np.sqrt(cfg.head_dim)))

    def _prefill(self, handles, counts, slots, pairs):
        torch = self.torch
        if len(pairs):
            self.pool.copy_blocks(torch.from_numpy(np.ascontiguousarray(pairs)).to(self.dev))
        idx, sl = [], []
        k = 0
        for h, c in zip(handles, counts):
            r = self.rids[h]
            p0 = self.length[r] - c
            if h in self.pl.rows:
                idx.extend(self.pl.rows[h][p0:p0 + c])
                sl.extend(int(x) for x in slots[k:k + c])
            k += c
        if not idx:
            return
        it = torch.tensor(idx, dtype=torch.int64, device=self.dev)
        st = torch.tensor(sl, dtype=torch.int32, device=self.dev)
        for layer in range(self.nl):
            kr, vr = self.rows[layer]
            self.pool.append_kv(layer, kr.index_select(0, it).contiguous(),
                                vr.index_select(0, it).contiguous(), st)

    def prepare(self, max_steps: int, separate_append: bool = False, shared_tokens: int = 0,
                plan_per_layer: bool = False):
        """Fixed device buffers, double-buffered pinned staging, ctypes arguments.

        shared_tokens > 0: decode with pa_append_decode_shared (or, with
        separate_append, pa_append_kv + pa_decode_shared) in partitions of
        that many tokens.  Otherwise a split launch's work plan is made once
        per step (pa_decode_plan, then every layer's pa_append_decode_planned
        or pa_decode_planned), or, with plan_per_layer, in each layer's call."""
        import ctypes

        import torch

        from paged_kv_cache_241_amd import capi

        lib = self.pool.lib
        self.lib = lib
        b = len(self.batch)
        bs = self.cfg.block_size
        longest = int(max(self.length[r] for r in self.batch)) + max_steps + 1
        self.stride = -(-longest // bs) if self.layout == "paged" else 1
        dev = self.dev
        # slots, lengths and tables side by side, so that one copy uploads a
        # step's arguments (the tables only when they changed)
        self.n_small = 2 * b
        self.n_all = 2 * b + b * self.stride
        self.args_d = torch.full((self.n_all,), -1, dtype=torch.int32, device=dev)
        self.slots_d = self.args_d[:b]
        self.lens_d = self.args_d[b:2 * b]
        self.tables_d = self.args_d[2 * b:].view(b, self.stride)
        self.stage = []
        for _ in range(2):
            buf = torch.empty(self.n_all, dtype=torch.int32).pin_memory()
            self.stage.append({
                "buf": buf,
                "slots": buf[:b],
                "lens": buf[b:2 * b],
                "tables": buf[2 * b:].view(b, self.stride),
                "pairs": torch.empty((b, 2), dtype=torch.int32).pin_memory(),
                "own": torch.cuda.Event(),   # the staging buffer's event on untimed steps
                "event": None,               # the last event recorded after its upload
            })
        self.pairs_d = torch.empty((b, 2), dtype=torch.int32, device=dev)
        self.ncow = ctypes.c_int32()
        self.rids_c = self.rids_np.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        self.p32 = lambda t: ctypes.cast(t.data_ptr(), ctypes.POINTER(ctypes.c_int32))
        self.stream = torch.cuda.current_stream()
        self.sh = ctypes.c_void_p(self.stream.cuda_stream)
        self.shared_T = shared_tokens
        if shared_tokens:
            self.pt = shared_tokens
            need = self.pool.workspace_bytes(b, self.cfg.num_q_heads,
                                             max(self.cfg.max_seq_len, shared_tokens + 1), shared_tokens)
            self.ws = torch.empty(need, dtype=torch.uint8, device=dev)
            self.sh_seq = torch.zeros(b, dtype=torch.int32, device=dev)
            self.sh_groups = torch.zeros((b, 2), dtype=torch.int32, device=dev)
            self.update_groups()
        if self.ws is None:
            need = self.pool.workspace_bytes(b, self.cfg.num_q_heads, self.cfg.max_seq_len, self.pt)
            self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        self.ws_bytes = self.ws.numel()
        self.dtype_code = capi.PA_BF16 if self.cfg.kv_dtype == "bf16" else capi.PA_F32
        self.check = capi.check
        self.separate_append = separate_append
        self.plan_once = not plan_per_layer and not shared_tokens
        self.plans_made = 0     # steps whose launches ran from a plan made once
        self.planned = ctypes.c_int32()
        self.nstep = 0
        # the tables only change when a block is handed out: upload on demand
        self.tables_dirty = True

    def update_groups(self):
        """Groups of the batch sharing a block prefix (pa_shared_groups), to the device."""
        seq, groups, mm, ms = self.pool.shared_groups(self.batch, self.shared_T)
        self.sh_seq.copy_(self.torch.from_numpy(np.ascontiguousarray(seq)))
        if len(groups):
            self.sh_groups[: len(groups)].copy_(self.torch.from_numpy(np.ascontiguousarray(groups)))
        self.sh_ng, self.sh_mm, self.sh_ms = len(groups), mm, ms

    def step(self, ev=None):
        """One decode iteration over all layers; returns the contexts it attended."""
        import ctypes

        lib, pool, cfg = self.lib, self.pool, self.cfg
        st = self.stage[self.nstep % 2]
        self.nstep += 1
        if st["event"] is not None:
            st["event"].synchronize()        # its previous uploads have run
        b = len(self.batch)
        t0 = time.perf_counter()
        self.check(lib.pa_reserve(pool.handle, self.rids_c, b, None, self.p32(st["slots"]), b,
                                  self.p32(st["pairs"]), b, ctypes.byref(self.ncow)), "pa_reserve")
        self.step_reserve_s += time.perf_counter() - t0
        slots = st["slots"].numpy()
        if self.layout == "paged" and (self.ncow.value or bool((slots % cfg.block_size == 0).any())):
            self.tables_dirty = True
        if self.tables_dirty and self.layout == "paged":
            self.check(lib.pa_get_block_tables(pool.handle, self.rids_c, b, self.stride,
                                               self.p32(st["tables"]), self.p32(st["lens"])),
                       "pa_get_block_tables")
            n = self.n_all
            self.tables_dirty = False
            if self.shared_T:
                self.update_groups()
        else:
            self.check(lib.pa_get_block_tables(pool.handle, self.rids_c, b, 0, None,
                                               self.p32(st["lens"])), "pa_get_block_tables")
            n = self.n_small
        self.args_d[:n].copy_(st["buf"][:n], non_blocking=True)
        if self.ncow.value:
            n = self.ncow.value
            self.pairs_d[:n].copy_(st["pairs"][:n], non_blocking=True)
            self.check(lib.pa_copy_blocks(pool.handle, self.pairs_d.data_ptr(), n, self.sh),
                       "pa_copy_blocks")
        if ev is None:
            st["own"].record(self.stream)
            st["event"] = st["own"]
        lens = st["lens"].numpy().astype(np.int64)
        max_context = int(lens.max())
        tables = self.tables_d.data_ptr() if self.layout == "paged" else None
        req = self.req_ids.data_ptr() if self.layout != "paged" else None
        if self.separate_append:
            for layer in range(self.nl):
                self.check(lib.pa_append_kv(pool.handle, layer, self.k_new[layer].data_ptr(),
                                            self.v_new[layer].data_ptr(), self.slots_d.data_ptr(),
                                            b, self.sh), "pa_append_kv")
        if ev is not None:
            # the timing event also marks this staging buffer's upload as done
            # (every event recorded on the stream holds the GPU ~5 us; a
            # separate one for the staging cost 1.3% of the step)
            ev[0].record(self.stream)
            st["event"] = ev[0]
        if self.plan_once:
            # one work plan for every layer: they all attend the same lengths
            self.check(lib.pa_decode_plan(pool.handle, self.lens_d.data_ptr(), b, cfg.num_q_heads,
                                          max_context, self.pt, self.ws.data_ptr(), self.ws_bytes,
                                          ctypes.byref(self.planned), self.sh), "pa_decode_plan")
            self.plans_made += self.planned.value
        for layer in range(self.nl):
            tail = (self.q[layer].data_ptr(), self.dtype_code, cfg.num_q_heads, self.scale, tables,
                    self.stride, req, self.lens_d.data_ptr(), b, max_context, self.pt,
                    self.out.data_ptr(), self.ws.data_ptr(), self.ws_bytes, self.sh)
            if self.shared_T:
                shared_tail = (self.q[layer].data_ptr(), self.dtype_code, cfg.num_q_heads,
                               self.scale, tables, self.stride, self.lens_d.data_ptr(), b, max_context,
                               self.shared_T, self.sh_seq.data_ptr(), self.sh_groups.data_ptr(),
                               self.sh_ng, self.sh_mm, self.sh_ms, self.out.data_ptr(),
                               self.ws.data_ptr(), self.ws_bytes, self.sh)
                if self.separate_append:
                    self.check(lib.pa_decode_shared(pool.handle, layer, *shared_tail), "pa_decode_shared")
                else:
                    self.check(lib.pa_append_decode_shared(
                        pool.handle, layer, self.k_new[layer].data_ptr(), self.v_new[layer].data_ptr(),
                        self.slots_d.data_ptr(), *shared_tail), "pa_append_decode_shared")
            elif self.separate_append:
                fn = lib.pa_decode_planned if self.plan_once else lib.pa_decode
                self.check(fn(pool.handle, layer, *tail), "pa_decode")
            else:
                fn = lib.pa_append_decode_planned if self.plan_once else lib.pa_append_decode
                self.check(fn(pool.handle, layer, self.k_new[layer].data_ptr(),
                              self.v_new[layer].data_ptr(), self.slots_d.data_ptr(), *tail),
                           "pa_append_decode")
        if ev is not None:
            ev[1].record(self.stream)
        return lens


def swap_probe(bench, n: int) -> dict:
    """Swap the first n requests of the batch out to pinned host images and
    back in (pa_swap_out / pa_swap_in), timed with HIP events on the stream
    the calls are queued on.  The images hold every rotated layer's blocks."""
    import torch

    pool = bench.pool
    rids = bench.batch[:n]
    images = [torch.empty(pool.swap_bytes(r), dtype=torch.uint8, pin_memory=True) for r in rids]
    total = sum(im.numel() for im in images)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    ev[0].record(bench.stream)
    for r, im in zip(rids, images):
        pool.swap_out(r, im, bench.stream)
    ev[1].record(bench.stream)
    for r, im in zip(rids, images):
        pool.swap_in(r, im, bench.stream)
    ev[2].record(bench.stream)
    torch.cuda.synchronize()
    bench.tables_dirty = True
    t_out = ev[0].elapsed_time(ev[1]) / 1e3
    t_in = ev[1].elapsed_time(ev[2]) / 1e3
    return {"seqs": n, "bytes": total, "out_ms": round(t_out * 1e3, 3), "in_ms": round(t_in * 1e3, 3),
            "out_gbs": round(total / t_out / 1e9, 2), "in_gbs": round(total / t_in / 1e9, 2),
            "image": "pinned host memory"}


COUNTERS_GLOB = os.path.join(ROOT, "profiles", "*_hbm_counters.md")


def measured_traffic(workload: str, steps: int, warmup: int):
    """HBM bytes per decode step of one layer from the committed counter summaries, or None.

    Each summary's machine lines give, per workload, the rocprofv3 FETCH_SIZE /
    WRITE_SIZE bytes of one layer's launches and the device sources' digest
    they were taken with; a line that names `steps` and `warmup` holds only
    for a run with those counts (the contexts it decodes depend on them).  A
    figure is used only while the sources still hash the same.
    """
    import glob

    fields = {}
    for path in sorted(glob.glob(COUNTERS_GLOB)):
        try:
            text = open(path).read()
        except OSError:
            continue
        for line in text.splitlines():
            if "traffic_bytes_per_launch=" in line:
                kv = dict(item.split("=", 1) for item in line.split() if "=" in item)
                if kv.get("workload") == workload:
                    fields = kv
    if not fields:
        return None
    if "steps" in fields and (int(fields["steps"]) != steps or int(fields.get("warmup", -1)) != warmup):
        return None
    if kernel_source_digest() != fields.get("kernel_src_sha256_16"):
        return None
    return int(fields["traffic_bytes_per_launch"])


# the sources every decode kernel (partition, plan, merge, shared) is compiled from
KERNEL_SOURCES = ("kernels.hip", "decode_partition.hpp", "decode_common.hpp", "kernels.hpp",
                  "decode_shared.hip")


def kernel_source_digest() -> str:
    """First 16 hex digits of SHA-256 over the decode kernels' sources, in order."""
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_241_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kv_bytes(cfg, lens) -> int:
    elt = 2 if cfg.kv_dtype == "bf16" else 4
    return int(lens.sum()) * cfg.num_kv_heads * cfg.head_dim * elt * 2


def unique_kv_fraction(bench) -> float:
    """Share of the batch's logical K/V bytes that lie in distinct blocks.

    Samples of one prompt share its full blocks, and a shared block has to come
    from HBM only once per launch, so the roofline counts every distinct block
    (with the most rows any sharer uses) once.  1.0 when nothing is shared."""
    if bench.layout != "paged":
        return 1.0
    tables, lens = bench.pool.block_tables(bench.rids_np)
    bs = bench.cfg.block_size
    rows_of = {}
    logical = 0
    for row, n in zip(tables, lens):
        n = int(n)
        for j in range(-(-n // bs)):
            rows = min(bs, n - j * bs)
            blk = int(row[j])
            rows_of[blk] = max(rows_of.get(blk, 0), rows)
            logical += rows
    return sum(rows_of.values()) / logical if logical else 1.0


def algorithmic_bytes(cfg, lens, fused_append: bool, kv_fraction: float = 1.0) -> int:
    """Bytes a decode launch must move: K/V (times the share in distinct blocks),
    q, out, block-table entries, lengths; with the fused append also the new
    rows (read once, written once) and slots."""
    elt = 2 if cfg.kv_dtype == "bf16" else 4
    b = len(lens)
    tables = int(sum(-(-int(n) // cfg.block_size) for n in lens)) * 4
    total = (int(round(kv_bytes(cfg, lens) * kv_fraction)) +
             b * cfg.num_q_heads * cfg.head_dim * (elt + 4) + tables + b * 4)
    if fused_append:
        total += b * cfg.num_kv_heads * cfg.head_dim * elt * 2 * 2 + b * 4
    return total


def _oracle_slice(job: dict) -> tuple:
    """One host core's share of the oracle baseline, run in a child process:
    gather through the block table (or at reqId x S) + fp64 attention, cycling
    over its sequences until `seconds` have passed.  BLAS is held to one
    thread.  Returns (KV bytes attended, sequence-decodes, seconds)."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as A

    conv = A.bf16_bits_to_f64 if job["bf16"] else A.f32_to_f64
    kvb, lens, q, bs = job["kvb"], job["lens"], job["q"], job["bs"]
    done = n = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            for i, length in enumerate(lens):
                length = int(length)
                blocks = job["blocks"][i][: -(-length // bs)]
                kt, vt = A.pair_tiles(kvb[blocks], job["head_dim"], bs)
                kr, vr = conv(A.k_rows(kt)), conv(A.v_rows(vt))
                if job["paged"]:
                    local = range(len(blocks))
                    k = A.gather_paged(kr, local, length, bs)
                    v = A.gather_paged(vr, local, length, bs)
                else:
                    span = len(blocks) * bs
                    k = A.gather_contiguous(A.contiguous_rows(kr, 1, span), 0, length)
                    v = A.gather_contiguous(A.contiguous_rows(np.ascontiguousarray(vr), 1, span), 0, length)
                A.attend(q[i], k, v, job["scale"])
                done += length * job["token_bytes"]
                n += 1
                if time.perf_counter() - t0 >= job["seconds"]:
                    return done, n, time.perf_counter() - t0


# host cores a GPU machine gives one GPU's jobs
CPU_SHARE = 16


def cpu_baseline(bench, seconds: float) -> dict | None:
    """The oracle (fp64 gather + attend) on the host's cores over a bounded
    sample of the workload's first layer: one child process per core, each
    cycling over its slice of the sequences for `seconds` seconds with BLAS
    held to one thread, then the same on one core alone.  The value is the
    sum of the processes' rates."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    import torch

    cfg = bench.cfg
    pool = bench.pool
    if pool.kv_cache is None:   # a demand-paged pool's cache cannot be read back
        return None
    paged = bench.layout == "paged"
    # the layer's raw tile pairs [units][Hkv][2][d*BS]
    if cfg.kv_dtype == "bf16":
        kvb = pool.kv_cache[0].view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        kvb = pool.kv_cache[0].cpu().numpy()
    q = bench.q[0].float().cpu().numpy().astype(np.float64)
    if paged:
        tables, lens = pool.block_tables(bench.rids_np)
    else:
        _, lens = pool.block_tables(bench.rids_np, 1)
    bs = cfg.block_size
    per = cfg.max_seq_len // bs
    elt = 2 if cfg.kv_dtype == "bf16" else 4
    cores = max(1, min(len(os.sched_getaffinity(0)), CPU_SHARE))

    def job(seqs, secs):
        # the slice's blocks copied out of the layer, renumbered in order
        blocks, parts, off = [], [], 0
        for s in seqs:
            nblk = -(-int(lens[s]) // bs)
            ids = (tables[s][:nblk] if paged else
                   np.arange(bench.batch[s] * per, bench.batch[s] * per + nblk))
            parts.append(kvb[ids])
            blocks.append(np.arange(off, off + nblk))
            off += nblk
        return {"kvb": np.concatenate(parts), "blocks": blocks, "head_dim": cfg.head_dim,
                "lens": [int(lens[s]) for s in seqs], "q": q[list(seqs)], "bs": bs, "paged": paged,
                "bf16": cfg.kv_dtype == "bf16", "scale": bench.scale, "seconds": secs,
                "token_bytes": cfg.num_kv_heads * cfg.head_dim * elt * 2}

    b = len(lens)
    slices = [list(range(i, b, cores)) for i in range(min(cores, b))]
    with ProcessPoolExecutor(max_workers=len(slices), mp_context=mp.get_context("spawn")) as ex:
        parts = list(ex.map(_oracle_slice, [job(sl, seconds) for sl in slices]))
    rate = sum(d / t for d, _, t in parts)
    n_all = sum(n for _, n, _ in parts)
    one_d, one_n, one_t = _oracle_slice(job(list(range(b)), seconds / 2))
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": len(slices), "kind": "oracle",
            "sample": f"{n_all} sequence-decodes of one layer ({b} sequences dealt round-robin to "
                      f"{len(slices)} processes, one per host core, each cycling over its share for "
                      f"{seconds:.0f} s: gather through the block table + fp64 attention, BLAS "
                      f"threads 1 per process); affinity {len(os.sched_getaffinity(0))} cores, "
                      f"at most {CPU_SHARE} used",
            "single_core": {"value": round(one_d / one_t / 1e9, 4), "unit": "GB/s",
                            "sample": f"{one_n} sequence-decodes in {one_t:.1f} s, one process, "
                                      "BLAS threads 1"}}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                                   "(multi-GPU sharding is described, not built)"}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.read_probe:
        read_probe(args.read_probe)
        return
    import torch

    import workloads as W

    over = {}
    if args.config == 5 and args.prompt_len:
        over["prompt_len"] = args.prompt_len
    base = W.get(args.config, **over)
    if args.block_size:
        over["block_size"] = args.block_size
        if base.num_blocks:
            over["num_blocks"] = base.num_blocks * base.block_size // args.block_size
        base = W.get(args.config, **over)
    if args.batch or args.context:
        if not base.context:
            print(json.dumps({"error": "--batch and --context apply to the uniform-context workloads 2 and 4"}))
            sys.exit(2)
        over["batch"] = args.batch or base.batch
        over["context"] = args.context or base.context
        steps = args.warmup + args.steps + 2
        need = -(-over["batch"] * min(over["context"] + steps, base.max_seq_len) // base.block_size) + 16
        over["num_blocks"] = max(base.num_blocks, need)
        base = W.get(args.config, **over)
    nominal = base.context
    if nominal:
        # centre the timed steps on the nominal context, and keep the last
        # step within the per-request cap
        over["context"] = min(nominal - args.warmup - (args.steps - 1) // 2,
                              base.max_seq_len - args.warmup - args.steps - 1)
    cfg = W.get(args.config, **over)
    if not cfg.context:
        # drawn or listed contexts grow by one token a step: lift the
        # per-request cap where the longest would outgrow it (the tiny
        # workload's 100-token context passes its 128-token cap in 29 steps)
        longest = int(W.plan(cfg).lengths.max())
        grown = -(-(longest + args.warmup + args.steps + 1) // cfg.block_size) * cfg.block_size
        if grown > cfg.max_seq_len:
            over["max_seq_len"] = grown
            cfg = W.get(args.config, **over)
    nl = args.layers or cfg.num_layers
    bench = Bench(cfg, args.layout, nl, args.warmup + args.steps + 1, args.partition_tokens)
    bench.prepare(args.warmup + args.steps, args.separate_append, args.shared_prefix,
                  args.plan_per_layer)
    for _ in range(args.warmup):
        bench.step()
    torch.cuda.synchronize()
    # HIP events bracket the decode launches of every K-th timed step
    # (--time-every, default TIMING_EVERY; the first one included); the other
    # steps record only the staging buffer's event.  Each event recorded on
    # the stream holds the GPU ~5 us, so timing every step would itself lower
    # the whole-step rate (every 4th against every 8th step: 5936 against
    # 5951 GB/s whole step on the Llama-3-8B layer, three runs each, within
    # run-to-run spread).
    timed = [i for i in range(args.steps) if i % max(args.time_every, 1) == 0]
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in timed}
    total_kv = 0
    lens_seen = []
    lens_all = []
    torch.cuda.synchronize()
    bench.step_reserve_s = 0.0
    t0 = time.perf_counter()
    for i in range(args.steps):
        lens = bench.step(evs.get(i))
        total_kv += kv_bytes(cfg, lens) * nl
        lens_all.append(lens)
        lens_seen.append(float(lens.mean()))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dt = t1 - t0
    n_launches = len(timed) * nl
    decode_ms = sum(a.elapsed_time(b) for a, b in evs.values())
    per_launch_s = decode_ms / 1e3 / n_launches
    kv_frac = unique_kv_fraction(bench)
    timed_lens = [lens_all[i] for i in timed]
    total_alg = sum(algorithmic_bytes(cfg, ln, not args.separate_append, kv_frac) for ln in timed_lens) * nl
    timed_kv = sum(kv_bytes(cfg, ln) for ln in timed_lens) * nl
    achieved = total_alg / n_launches / per_launch_s / 1e9
    value = total_kv / dt / 1e9
    b = len(bench.batch)
    part = args.shared_prefix or bench.pool.partition_tokens(b, int(max(lens)), args.partition_tokens)
    stats = bench.pool.stats()
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": cfg.name + ("" if args.layout == "paged" else ", contiguous reqId x S layout") +
                        (f" (run with batch {b}, context about {cfg.context + args.warmup + (args.steps - 1) // 2})"
                         if args.batch or args.context else ""),
            "batch": b, "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
            "head_dim": cfg.head_dim, "block_size": cfg.block_size, "kv_dtype": cfg.kv_dtype,
            "mean_context_timed": round(float(np.mean(lens_seen)), 2),
            "layers_rotated": nl, "partition_tokens": part, "layout": args.layout,
            "decode": ("shared prefixes read once (" +
                       ("pa_append_kv + pa_decode_shared" if args.separate_append else "pa_append_decode_shared") +
                       ")") if args.shared_prefix else
                      ("pa_append_kv + pa_decode" if args.separate_append else "pa_append_decode") +
                      ("_planned" if bench.plan_once else ""),
            "work_plan": ("none (shared-prefix launch)" if args.shared_prefix else
                          "in each layer's call, where the launch uses one" if args.plan_per_layer else
                          "once per step (pa_decode_plan), used by every layer" if bench.plans_made else
                          "none (no launch of this size uses one)"),
        },
        # logical K/V bytes count a shared block once per sharer; the share of
        # HBM's peak is taken on the distinct bytes
        "pct_of_hbm_peak": round(100 * value * kv_frac / HBM_PEAK_GBS, 2),
        "value_distinct_gbs": round(value * kv_frac, 2),
        "decode_us_per_layer": round(per_launch_s * 1e6, 3),
        "decode_kv_gbs": round(timed_kv / n_launches / per_launch_s / 1e9, 2),
        "decode_launches_timed": n_launches,
        "tokens_per_s_per_layer": round(b / per_launch_s, 1),
        "pool_utilisation": round(stats["utilisation"], 4),
        "roofline": {
            "bound": "hbm",
            "kernel": (("pa_decode_shared" if args.separate_append else "pa_append_decode_shared") +
                       " (decode_shared_kernel: shared pass and private partitions; "
                       "decode_merge_kernel)" if args.shared_prefix else
                       ("pa_decode" if args.separate_append else "pa_append_decode") +
                       " (decode_partition_kernel; decode_merge_kernel when contexts are split, "
                       "and decode_plan_kernel for large split launches, " +
                       ("in each layer's call" if args.plan_per_layer else "once per step") + ")"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "kv_unique_fraction": round(kv_frac, 4),
            "basis": "algorithmic bytes per launch" + (" (distinct blocks once)" if kv_frac < 1.0 else ""),
            "traffic": None,
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0)",
        },
    }
    # the counters were taken on each workload as it stands: no other batch,
    # context, prompt, block size, layer count, partition size or plan mode
    as_counted = not (args.batch or args.context or args.block_size or args.layers or
                      args.partition_tokens or args.prompt_len or args.plan_per_layer)
    if args.layout in ("paged", "contiguous") and as_counted:
        key = (f"cfg{args.config}-{args.layout}" + (f"-shared{args.shared_prefix}" if args.shared_prefix else "") +
               ("" if args.separate_append else "-fused"))
        traffic = measured_traffic(key, args.steps, args.warmup)
        roof = res["roofline"]
        roof["traffic"] = traffic
        if traffic is not None and kv_frac < 1.0:
            # shared blocks may be served by the caches, so where blocks are
            # shared the fraction is taken on the bytes HBM actually moved
            roof["achieved_algorithmic"] = roof["achieved"]
            roof["achieved"] = round(traffic / per_launch_s / 1e9, 2)
            roof["frac"] = round(traffic / per_launch_s / 1e9 / HBM_PEAK_GBS, 4)
            roof["basis"] = "measured HBM bytes (traffic) per launch"
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(bench, args.cpu_seconds)
        if cpu is not None:
            res["cpu_baseline"] = cpu
    if args.swap_seqs:
        res["swap"] = swap_probe(bench, args.swap_seqs)
    if bench.vmm:
        v = bench.pool.vmm_stats()
        res["vmm"] = {
            "page_bytes": v["page_bytes"], "mapped_bytes": v["mapped_bytes"],
            "contiguous_reservation_bytes": bench.full_bytes,
            "mapped_share": round(v["mapped_bytes"] / bench.full_bytes, 4),
            "prefill_mapped_bytes": bench.prefill_mapped,
            "prefill_reserve_s": round(bench.reserve_s, 4),
            "prefill_map_rate_gbs": round(bench.prefill_mapped / bench.reserve_s / 1e9, 2) if bench.reserve_s else None,
            # pages mapped by the warm-up and timed steps' pa_reserve calls
            # (inside the timed region where contexts cross a page)
            "steps_mapped_bytes": v["mapped_bytes"] - bench.prefill_mapped,
            "timed_reserve_s": round(bench.step_reserve_s, 4),
        }
    if not args.no_hbm_probe:
        probe = hbm_probe()
        if probe:
            res["hbm_read_probe_gbs"] = probe
            res["roofline"]["frac_of_probe_best"] = round(achieved / max(probe.values()), 4)
            if "decode_pattern" in probe:
                res["roofline"]["frac_of_decode_pattern"] = round(achieved / probe["decode_pattern"], 4)
            if "decode_mapped_kv8k" in probe and args.config == 2 and as_counted:
                # the same tiles in the decode's own order and the library's
                # layout (K and V of a block side by side), no arithmetic
                res["roofline"]["frac_of_decode_mapped"] = round(achieved / probe["decode_mapped_kv8k"], 4)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
