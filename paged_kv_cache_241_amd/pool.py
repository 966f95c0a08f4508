"""A paged KV cache over torch device memory, driven through libpa.so.

PyTorch supplies the device memory (the cache array, q, out, tables,
workspace) and the stream; every allocator step and every kernel is the C
library's.  Method names follow the C ABI (``pa_seq_add`` -> ``add``, ...).
"""

from __future__ import annotations

import ctypes

import numpy as np

from . import capi

_DTYPES = {"f32": capi.PA_F32, "bf16": capi.PA_BF16}
_LAYOUTS = {"paged": capi.PA_PAGED, "contiguous": capi.PA_CONTIGUOUS}


def _ptr32(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream_handle(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Pool:
    """The KV cache of ``num_layers`` layers plus the host block allocator.

    ``kv_cache`` is the one array include/pa.h lays out, one region per
    (block, KV head): ``[num_layers][units][num_kv_heads][2 * head_dim * block_size]``,
    each region ``block_size / sub`` tile pairs of ``sub = min(block_size, 16)``
    token rows (K tile ``[head_dim/VE][sub][VE]``, then V tile ``[head_dim][sub]``),
    with ``VE = 16 / element bytes`` and ``units = num_blocks`` (paged) or
    ``max_seqs * max_seq_len / block_size`` (contiguous: request r owns the
    ``max_seq_len / block_size`` consecutive blocks from ``r * max_seq_len / block_size``).
    """

    def __init__(self, num_layers: int, num_blocks: int, block_size: int, num_kv_heads: int,
                 head_dim: int, kv_dtype: str = "bf16", layout: str = "paged",
                 max_seqs: int = 256, max_seq_len: int = 8192, device="cuda", fill=None,
                 host_only: bool = False, vmm_bytes: int | None = None):
        """``host_only``: no cache memory is allocated and only the host
        allocator calls may be used (the library never touches the caches in
        those calls); device calls then fail.

        ``vmm_bytes``: a demand-paged contiguous pool (pa_create_pool_vmm) whose
        cache the library backs with up to that many bytes of physical pages
        as requests grow; ``kv_cache`` is then None (the library owns the
        memory and unbacked ranges must not be read)."""
        import torch

        self.lib = capi.load()
        self.kv_dtype = kv_dtype
        self.layout = layout
        self.desc = capi.pa_pool_desc(num_layers, num_blocks if layout == "paged" else 0,
                                      block_size, num_kv_heads, head_dim, _DTYPES[kv_dtype],
                                      _LAYOUTS[layout], max_seqs, max_seq_len)
        nbytes = self.lib.pa_cache_bytes(ctypes.byref(self.desc))
        if nbytes == 0:
            raise capi.PaError(capi.PA_ERR_INVALID_ARG, "Pool", "invalid pool description")
        tdt = torch.bfloat16 if kv_dtype == "bf16" else torch.float32
        units = num_blocks if layout == "paged" else max_seqs * (max_seq_len // block_size)
        kv_shape = (num_layers, units, num_kv_heads, 2 * head_dim * block_size)
        self.vmm = vmm_bytes is not None
        if self.vmm:
            if layout != "contiguous":
                raise ValueError("demand paging backs the contiguous layout")
            self.kv_cache = None
            h = ctypes.c_void_p()
            capi.check(self.lib.pa_create_pool_vmm(ctypes.byref(self.desc), int(vmm_bytes),
                                                   ctypes.byref(h)), "pa_create_pool_vmm")
            self._finish(h, num_layers, num_blocks, block_size, num_kv_heads, head_dim, max_seqs,
                         max_seq_len, tdt)
            return
        if host_only:
            self.kv_cache = None
            self._fake = torch.empty(16, dtype=torch.uint8)
        elif fill is None:
            self.kv_cache = torch.empty(kv_shape, dtype=tdt, device=device)
        else:
            self.kv_cache = torch.full(kv_shape, fill, dtype=tdt, device=device)
        if host_only:
            # any 16-byte aligned address: allocator calls never dereference it
            ptr = (self._fake.data_ptr() + 15) // 16 * 16
        else:
            assert self.kv_cache.numel() * self.kv_cache.element_size() == nbytes
            ptr = self.kv_cache.data_ptr()
        h = ctypes.c_void_p()
        capi.check(self.lib.pa_create_pool(ctypes.byref(self.desc), ptr, ctypes.byref(h)),
                   "pa_create_pool")
        self._finish(h, num_layers, num_blocks, block_size, num_kv_heads, head_dim, max_seqs,
                     max_seq_len, tdt)

    def _finish(self, h, num_layers, num_blocks, block_size, num_kv_heads, head_dim, max_seqs,
                max_seq_len, tdt):
        self.handle = h
        self.num_layers, self.num_blocks, self.block_size = num_layers, num_blocks, block_size
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.max_seqs, self.max_seq_len = max_seqs, max_seq_len
        self.torch_dtype = tdt
        self._device = self.vmm or self.kv_cache is not None

    def vmm_stats(self) -> dict:
        st = capi.pa_vmm_stats()
        capi.check(self.lib.pa_vmm_info(self.handle, ctypes.byref(st)), "pa_vmm_info")
        return {name: getattr(st, name) for name, _ in capi.pa_vmm_stats._fields_}

    def vmm_trim(self) -> int:
        """Unmap the pages of request ids that are not live (synchronise first)."""
        freed = ctypes.c_int64()
        capi.check(self.lib.pa_vmm_trim(self.handle, ctypes.byref(freed)), "pa_vmm_trim")
        return freed.value

    # -- lifetime --------------------------------------------------------------
    def close(self) -> None:
        if getattr(self, "handle", None) is not None and self.handle.value:
            if getattr(self, "vmm", False):
                # destroying unmaps the caches: nothing queued may still read them
                import torch

                torch.cuda.synchronize()
            capi.check(self.lib.pa_destroy_pool(self.handle), "pa_destroy_pool")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- host allocator --------------------------------------------------------
    def bytes_per_token(self) -> int:
        return int(self.lib.pa_bytes_per_token(ctypes.byref(self.desc)))

    def set_free_order(self, order) -> None:
        order = np.ascontiguousarray(order, dtype=np.int32)
        capi.check(self.lib.pa_set_free_order(self.handle, _ptr32(order), len(order)),
                   "pa_set_free_order")

    def add(self) -> int:
        rid = ctypes.c_int32()
        capi.check(self.lib.pa_seq_add(self.handle, ctypes.byref(rid)), "pa_seq_add")
        return rid.value

    def fork(self, parent: int) -> int:
        rid = ctypes.c_int32()
        capi.check(self.lib.pa_seq_fork(self.handle, parent, ctypes.byref(rid)), "pa_seq_fork")
        return rid.value

    def free_seq(self, rid: int) -> None:
        capi.check(self.lib.pa_seq_free(self.handle, rid), "pa_seq_free")

    def reserve(self, req_ids, counts=None):
        """Grow requests; returns (slots int32[total], cow pairs int32[k][2])."""
        rids = np.ascontiguousarray(req_ids, dtype=np.int32)
        n = len(rids)
        if counts is None:
            cnt = None
            total = n
        else:
            cnt = np.ascontiguousarray(counts, dtype=np.int32)
            total = int(cnt.sum())
        slots = np.empty(max(total, 1), dtype=np.int32)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        ncow = ctypes.c_int32()
        capi.check(self.lib.pa_reserve(self.handle, _ptr32(rids), n,
                                       _ptr32(cnt) if cnt is not None else None,
                                       _ptr32(slots), total, _ptr32(pairs), n, ctypes.byref(ncow)),
                   "pa_reserve")
        return slots[:total], pairs[: ncow.value]

    def block_tables(self, req_ids, stride: int | None = None):
        """(tables int32[n][stride] padded with -1, lengths int32[n])."""
        rids = np.ascontiguousarray(req_ids, dtype=np.int32)
        n = len(rids)
        lens = np.empty(max(n, 1), dtype=np.int32)
        if stride is None:
            capi.check(self.lib.pa_get_block_tables(self.handle, _ptr32(rids), n, 0, None,
                                                    _ptr32(lens)), "pa_get_block_tables")
            stride = max(1, -(-int(lens[:n].max(initial=0)) // self.block_size))
        tables = np.empty((max(n, 1), stride), dtype=np.int32)
        capi.check(self.lib.pa_get_block_tables(self.handle, _ptr32(rids), n, stride,
                                                _ptr32(tables), _ptr32(lens)), "pa_get_block_tables")
        return tables[:n], lens[:n]

    # -- shared prefixes ------------------------------------------------------
    def shared_groups(self, req_ids, partition_tokens: int):
        """Groups of consecutive requests with a common block prefix (pa_shared_groups):
        (seq_shared int32[n], groups int32[g][2], max_members, max_shared)."""
        rids = np.ascontiguousarray(req_ids, dtype=np.int32)
        n = len(rids)
        seq_shared = np.zeros(max(n, 1), dtype=np.int32)
        groups = np.zeros((max(n, 1), 2), dtype=np.int32)
        ng, mm, ms = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        capi.check(self.lib.pa_shared_groups(self.handle, _ptr32(rids), n, int(partition_tokens),
                                             _ptr32(seq_shared), _ptr32(groups), ctypes.byref(ng),
                                             ctypes.byref(mm), ctypes.byref(ms)), "pa_shared_groups")
        return seq_shared[:n], groups[: ng.value], mm.value, ms.value

    def decode_shared(self, layer: int, q, scale: float, block_tables, context_lens, max_context: int,
                      partition_tokens: int, seq_shared, groups, max_members: int, max_shared: int,
                      out=None, workspace=None, stream=None, append=None):
        """pa_decode_shared: seq_shared int32 [B] and groups int32 [g][2] on the device.

        ``append=(k, v, slots)`` stores each sequence's new token first, in the
        same launch (pa_append_decode_shared); k, v are [B][Hkv][D], slots int32 [B].
        """
        import torch

        assert self._device, "host-only pool"
        b, hq, d = q.shape
        assert q.is_cuda and q.is_contiguous() and q.dtype == self.torch_dtype and d == self.head_dim
        for t in (block_tables, context_lens, seq_shared, groups):
            assert t.is_cuda and t.dtype == torch.int32 and t.is_contiguous()
        assert tuple(seq_shared.shape) == (b,) and tuple(context_lens.shape) == (b,)
        if out is None:
            out = torch.empty((b, hq, d), dtype=torch.float32, device=q.device)
        assert out.is_cuda and out.is_contiguous() and out.dtype == torch.float32 and tuple(out.shape) == (b, hq, d)
        if workspace is None:
            # at least two partitions: the shared pass always writes partials
            need = self.workspace_bytes(b, hq, max(int(max_context), int(partition_tokens) + 1),
                                        partition_tokens)
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        assert workspace.is_cuda and workspace.is_contiguous()
        tail = (q.data_ptr(), _DTYPES[self.kv_dtype], hq, float(scale),
                block_tables.data_ptr(), int(block_tables.shape[1]), context_lens.data_ptr(), b,
                int(max_context), int(partition_tokens), seq_shared.data_ptr(),
                groups.data_ptr() if groups.numel() else None, int(groups.shape[0]), int(max_members),
                int(max_shared), out.data_ptr(), workspace.data_ptr(),
                workspace.numel() * workspace.element_size(), _stream_handle(stream))
        if append is None:
            capi.check(self.lib.pa_decode_shared(self.handle, layer, *tail), "pa_decode_shared")
        else:
            k, v, slots = append
            for t in (k, v):
                assert t.is_cuda and t.is_contiguous() and t.dtype == self.torch_dtype
                assert tuple(t.shape) == (b, self.num_kv_heads, self.head_dim)
            assert slots.is_cuda and slots.dtype == torch.int32 and tuple(slots.shape) == (b,)
            capi.check(self.lib.pa_append_decode_shared(self.handle, layer, k.data_ptr(), v.data_ptr(),
                                                        slots.data_ptr(), *tail), "pa_append_decode_shared")
        return out

    def check_shared_args(self, seq_shared, context_lens, partition_tokens: int, slots=None) -> None:
        """pa_check_shared_args on host int32 arrays."""
        sh = np.ascontiguousarray(seq_shared, dtype=np.int32)
        ln = np.ascontiguousarray(context_lens, dtype=np.int32)
        sl = None if slots is None else np.ascontiguousarray(slots, dtype=np.int32)
        n = len(sh)
        capi.check(self.lib.pa_check_shared_args(
            self.handle, _ptr32(sh) if n else None, _ptr32(ln) if n else None,
            _ptr32(sl) if sl is not None else None, n, int(partition_tokens)), "pa_check_shared_args")

    # -- pre-emption by swapping ---------------------------------------------
    def swap_bytes(self, rid: int) -> int:
        """Bytes of request rid's swap image (include/pa.h lays it out)."""
        n = ctypes.c_size_t()
        capi.check(self.lib.pa_swap_bytes(self.handle, rid, ctypes.byref(n)), "pa_swap_bytes")
        return n.value

    def _image(self, image, stream):
        if image is None:  # no copy: nothing touches the device
            return ctypes.c_void_p(None), 0, ctypes.c_void_p(None)
        return (ctypes.c_void_p(image.data_ptr()), image.numel() * image.element_size(),
                _stream_handle(stream))

    def swap_out(self, rid: int, image=None, stream=None) -> None:
        """Copy rid's blocks into ``image`` (a pinned host or device uint8
        tensor of at least swap_bytes(rid) bytes) and give the blocks back;
        ``image=None`` drops the contents (pre-emption by recomputation)."""
        ptr, cap, st = self._image(image, stream)
        capi.check(self.lib.pa_swap_out(self.handle, rid, ptr, cap, st), "pa_swap_out")

    def swap_in(self, rid: int, image=None, stream=None) -> None:
        """Give swapped-out rid fresh blocks and copy ``image`` back into them
        (``image=None``: no copy, the caller rewrites the rows)."""
        ptr, cap, st = self._image(image, stream)
        capi.check(self.lib.pa_swap_in(self.handle, rid, ptr, cap, st), "pa_swap_in")

    def stats(self) -> dict:
        st = capi.pa_stats()
        capi.check(self.lib.pa_get_stats(self.handle, ctypes.byref(st)), "pa_get_stats")
        return {name: getattr(st, name) for name, _ in capi.pa_stats._fields_}

    # -- host-side checks of device arrays (host copies; nothing is launched) ---
    def check_decode_args(self, block_tables, context_lens, max_context: int, req_ids=None,
                          slots=None) -> None:
        """pa_check_decode_args on host int32 arrays: tables [B][stride]
        (paged), lengths [B], request ids [B] (contiguous; None: s), the fused
        append's slots [B] (None: no append)."""
        lens = np.ascontiguousarray(context_lens, dtype=np.int32)
        b = len(lens)
        tables, stride = None, 0
        if self.layout == "paged" and block_tables is not None:
            tables = np.ascontiguousarray(block_tables, dtype=np.int32)
            stride = int(tables.shape[1]) if tables.ndim == 2 else 0
        rids = None if req_ids is None else np.ascontiguousarray(req_ids, dtype=np.int32)
        sl = None if slots is None else np.ascontiguousarray(slots, dtype=np.int32)
        capi.check(self.lib.pa_check_decode_args(
            self.handle, _ptr32(tables) if tables is not None else None, stride,
            _ptr32(rids) if rids is not None else None, _ptr32(lens) if b else None,
            _ptr32(sl) if sl is not None else None, b, int(max_context)), "pa_check_decode_args")

    def check_slots(self, slots) -> None:
        sl = np.ascontiguousarray(slots, dtype=np.int32)
        capi.check(self.lib.pa_check_slots(self.handle, _ptr32(sl) if len(sl) else None, len(sl)),
                   "pa_check_slots")

    def check_block_pairs(self, pairs) -> None:
        pr = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
        capi.check(self.lib.pa_check_block_pairs(self.handle, _ptr32(pr) if len(pr) else None, len(pr)),
                   "pa_check_block_pairs")

    # -- device ----------------------------------------------------------------
    def copy_blocks(self, pairs, stream=None) -> None:
        """pairs: device int32 tensor [n][2] of (src, dst) blocks."""
        n = int(pairs.shape[0]) if pairs is not None else 0
        if n == 0:
            return
        assert self._device, "host-only pool"
        assert pairs.dtype.is_floating_point is False and pairs.is_cuda and pairs.is_contiguous()
        assert tuple(pairs.shape) == (n, 2)
        capi.check(self.lib.pa_copy_blocks(self.handle, pairs.data_ptr(), n, _stream_handle(stream)),
                   "pa_copy_blocks")

    def append_kv(self, layer: int, k, v, slots, stream=None) -> None:
        """k, v: device [n][Hkv][D] in the cache dtype; slots: device int32 [n]."""
        n = int(slots.shape[0])
        if n == 0:
            return
        assert self._device, "host-only pool"
        for t in (k, v):
            assert t.is_cuda and t.is_contiguous() and t.dtype == self.torch_dtype
            assert tuple(t.shape) == (n, self.num_kv_heads, self.head_dim)
        assert slots.is_cuda and slots.is_contiguous() and str(slots.dtype) == "torch.int32"
        capi.check(self.lib.pa_append_kv(self.handle, layer, k.data_ptr(), v.data_ptr(),
                                         slots.data_ptr(), n, _stream_handle(stream)), "pa_append_kv")

    def partition_tokens(self, num_seqs: int, max_context: int, partition_tokens: int = 0) -> int:
        return int(self.lib.pa_decode_partition_tokens(self.handle, num_seqs, max_context,
                                                        partition_tokens))

    def workspace_bytes(self, num_seqs: int, num_q_heads: int, max_context: int,
                        partition_tokens: int = 0) -> int:
        return int(self.lib.pa_decode_workspace_bytes(self.handle, num_seqs, num_q_heads,
                                                      max_context, partition_tokens))

    def decode_plan(self, context_lens, num_q_heads: int, max_context: int, workspace,
                    partition_tokens: int = 0, stream=None) -> bool:
        """pa_decode_plan: the work plan of a split decode into ``workspace``,
        for every layer's ``decode(..., planned=True)`` with these lengths and
        sizes; False when such a launch uses no plan (nothing is enqueued)."""
        import torch

        assert self._device, "host-only pool"
        assert context_lens.is_cuda and context_lens.dtype == torch.int32 and context_lens.is_contiguous()
        b = int(context_lens.shape[0])
        assert workspace is None or (workspace.is_cuda and workspace.is_contiguous())
        made = ctypes.c_int32(0)
        capi.check(self.lib.pa_decode_plan(
            self.handle, context_lens.data_ptr(), b, int(num_q_heads), int(max_context),
            int(partition_tokens), workspace.data_ptr() if workspace is not None else None,
            workspace.numel() * workspace.element_size() if workspace is not None else 0,
            ctypes.byref(made), _stream_handle(stream)), "pa_decode_plan")
        return bool(made.value)

    def decode(self, layer: int, q, scale: float, block_tables, context_lens, max_context: int,
               out=None, partition_tokens: int = 0, req_ids=None, workspace=None, stream=None,
               append=None, planned: bool = False):
        """Decode attention for q [B][Hq][D]; returns out fp32 [B][Hq][D].

        ``append=(k, v, slots)`` stores each sequence's new token first, in the
        same launch (pa_append_decode); k, v are [B][Hkv][D], slots int32 [B].
        ``planned``: the plan ``decode_plan`` left in ``workspace`` is used
        (pa_decode_planned / pa_append_decode_planned).
        """
        import torch

        assert self._device, "host-only pool"
        b, hq, d = q.shape
        assert q.is_cuda and q.is_contiguous() and q.dtype == self.torch_dtype and d == self.head_dim
        assert context_lens.is_cuda and context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (b,)
        stride = 0
        if self.layout == "paged":
            assert block_tables.is_cuda and block_tables.dtype == torch.int32
            assert block_tables.is_contiguous() and block_tables.shape[0] == b
            stride = int(block_tables.shape[1])
        if req_ids is not None:
            assert req_ids.is_cuda and req_ids.dtype == torch.int32 and tuple(req_ids.shape) == (b,)
        if out is None:
            out = torch.empty((b, hq, d), dtype=torch.float32, device=q.device)
        assert out.is_cuda and out.is_contiguous() and out.dtype == torch.float32 and tuple(out.shape) == (b, hq, d)
        need = self.workspace_bytes(b, hq, max_context, partition_tokens)
        if need and workspace is None:
            assert not planned, "a planned decode reads its plan from the caller's workspace"
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        assert workspace is None or (workspace.is_cuda and workspace.is_contiguous())
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        args = (q.data_ptr(), _DTYPES[self.kv_dtype], hq, float(scale),
                block_tables.data_ptr() if self.layout == "paged" else None, stride,
                req_ids.data_ptr() if req_ids is not None else None, context_lens.data_ptr(), b,
                int(max_context), int(partition_tokens), out.data_ptr(), ws_ptr, ws_bytes,
                _stream_handle(stream))
        if append is None:
            name = "pa_decode_planned" if planned else "pa_decode"
            capi.check(getattr(self.lib, name)(self.handle, layer, *args), name)
        else:
            k, v, slots = append
            for t in (k, v):
                assert t.is_cuda and t.is_contiguous() and t.dtype == self.torch_dtype
                assert tuple(t.shape) == (b, self.num_kv_heads, self.head_dim)
            assert slots.is_cuda and slots.dtype == torch.int32 and tuple(slots.shape) == (b,)
            name = "pa_append_decode_planned" if planned else "pa_append_decode"
            capi.check(getattr(self.lib, name)(self.handle, layer, k.data_ptr(), v.data_ptr(),
                                               slots.data_ptr(), *args), name)
        return out

    def append_decode_noalloc(self, layer: int, q, scale: float, block_tables, context_lens,
                              max_context: int, k, v, slots, out=None, partition_tokens: int = 0,
                              req_ids=None, stream=None):
        """pa_append_decode_noalloc: pa_append_decode without a workspace (the
        split-K partials go to the library's own device scratch)."""
        import torch

        assert self._device, "host-only pool"
        b, hq, d = q.shape
        assert q.is_cuda and q.is_contiguous() and q.dtype == self.torch_dtype and d == self.head_dim
        assert context_lens.is_cuda and context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (b,)
        stride = 0
        if self.layout == "paged":
            assert block_tables.is_cuda and block_tables.dtype == torch.int32
            assert block_tables.is_contiguous() and block_tables.shape[0] == b
            stride = int(block_tables.shape[1])
        if req_ids is not None:
            assert req_ids.is_cuda and req_ids.dtype == torch.int32 and tuple(req_ids.shape) == (b,)
        for t in (k, v):
            assert t.is_cuda and t.is_contiguous() and t.dtype == self.torch_dtype
            assert tuple(t.shape) == (b, self.num_kv_heads, self.head_dim)
        assert slots.is_cuda and slots.dtype == torch.int32 and tuple(slots.shape) == (b,)
        if out is None:
            out = torch.empty((b, hq, d), dtype=torch.float32, device=q.device)
        assert out.is_cuda and out.is_contiguous() and out.dtype == torch.float32 and tuple(out.shape) == (b, hq, d)
        capi.check(self.lib.pa_append_decode_noalloc(
            self.handle, layer, k.data_ptr(), v.data_ptr(), slots.data_ptr(), q.data_ptr(),
            _DTYPES[self.kv_dtype], hq, float(scale),
            block_tables.data_ptr() if self.layout == "paged" else None, stride,
            req_ids.data_ptr() if req_ids is not None else None, context_lens.data_ptr(), b,
            int(max_context), int(partition_tokens), out.data_ptr(), _stream_handle(stream)),
            "pa_append_decode_noalloc")
        return out
