"""Device-memory plumbing around the C ABI, on top of PyTorch (memory and streams only).

* ``PagedKVCache``     — the two pools (torch tensors) plus the library's cache handle;
* ``DeviceDescriptors`` — uploads a composed batch and its work list to the device in one
  copy from a ring of pinned staging buffers (an event guards each buffer, so the host can
  compose the next pass while the previous copy is still queued);
* ``Workspace``         — device scratch for split-key partials (no initialisation needed),
  grown on demand.

No arithmetic of the method happens here.
"""
from __future__ import annotations

import ctypes
import time

import numpy as np
import torch

from . import fg

TORCH_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def num_cus(device=None) -> int:
    return int(torch.cuda.get_device_properties(device or torch.cuda.current_device())
               .multi_processor_count)


def stream_handle(stream=None) -> int:
    s = stream or torch.cuda.current_stream()
    return int(s.cuda_stream)


def v_group(block_size: int) -> int:
    """Keys per group of the V pool layout (include/fg.h): min(8, block_size)."""
    return min(8, int(block_size))


def pool_shapes(num_blocks, block_size, num_kv_heads, head_dim):
    """(K pool shape, V pool shape) of the layout include/fg.h declares."""
    g = v_group(block_size)
    return ((num_blocks, num_kv_heads, block_size, head_dim),
            (num_blocks, num_kv_heads, block_size // g, head_dim, g))


class PagedKVCache:
    """Pools: K [NB][Hkv][bs][D], V [NB][Hkv][bs/g][D][g] (g = min(8, bs)) in the cache
    dtype."""

    def __init__(self, num_blocks, block_size, num_kv_heads, head_dim, dtype, device="cuda",
                 free_ids=None, k_pool=None, v_pool=None):
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.num_kv_heads, self.head_dim, self.dtype = int(num_kv_heads), int(head_dim), dtype
        tdt = TORCH_DTYPES[dtype]
        ks, vs = pool_shapes(self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        if k_pool is None:
            k_pool = torch.empty(ks, dtype=tdt, device=device)
        if v_pool is None:
            v_pool = torch.empty(vs, dtype=tdt, device=device)
        assert k_pool.is_contiguous() and v_pool.is_contiguous()
        assert tuple(k_pool.shape) == ks, (tuple(k_pool.shape), ks)
        assert tuple(v_pool.shape) == vs, (tuple(v_pool.shape), vs)
        assert k_pool.dtype == tdt and v_pool.dtype == tdt
        self.k_pool, self.v_pool = k_pool, v_pool
        self.handle = fg.fg_blocked_cache_init(num_blocks, block_size, num_kv_heads, head_dim,
                                               dtype, k_pool.data_ptr(), v_pool.data_ptr(),
                                               free_ids)

    def close(self):
        if self.handle is not None:
            fg.fg_blocked_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001  (interpreter shutdown)
            pass


class DeviceDescriptors:
    """One int32 device buffer holding [query_start | n_query | context_len | block_table |
    work records] of the current pass, and the fg_ragged_batch struct pointing into it."""

    def __init__(self, device="cuda", ring: int = 3):
        self.device = torch.device(device)
        self.ring = [None] * ring
        self.events = [None] * ring
        self.slot = 0
        self.dev = None
        self.cstruct = fg.FgRaggedBatch()
        self.work_ptr = 0
        self._pending = []  # slots uploaded with record=False and not yet released
        self.wait_s = 0.0   # host seconds spent waiting for a staging buffer to come free

    def _staging(self, n):
        i = self.slot
        self.slot = (self.slot + 1) % len(self.ring)
        if i in self._pending:
            raise RuntimeError("descriptor ring reused before release(): call release() at "
                               "least once every ring uploads")
        if self.events[i] is not None:
            t0 = time.perf_counter()
            self.events[i].synchronize()        # the copy that last read this buffer is done
            self.wait_s += time.perf_counter() - t0
        if self.ring[i] is None or self.ring[i].numel() < n:
            self.ring[i] = torch.empty(max(n, 1024), dtype=torch.int32, pin_memory=True)
        return i, self.ring[i]

    def upload(self, hb: fg.HostBatch, work: np.ndarray | None = None, stream=None,
               record: bool = True):
        """Copy the batch (and work list) to the device on `stream`.  The pinned staging
        buffer is reused `ring` uploads later, once the event guarding it has completed:
        with record=True an event recorded right after the copy; with record=False the caller
        hands one in through release() (an event it records later on the same stream anyway,
        e.g. after the pass's kernels), which saves a marker between the copy and the next
        kernel."""
        S, stride = hb.num_seqs, hb.table_stride
        nw = 0 if work is None else int(work.size)
        parts = [hb.query_start[:S + 1], hb.n_query[:S], hb.context_len[:S],
                 hb.block_table[:S].reshape(-1)]
        sizes = [S + 1, S, S, S * stride]
        total = sum(sizes) + nw
        i, host = self._staging(total)
        h = host.numpy()
        off = 0
        for p, n in zip(parts, sizes):
            h[off:off + n] = p
            off += n
        if nw:
            h[off:off + nw] = work.reshape(-1)
        if self.dev is None or self.dev.numel() < total:
            self.dev = torch.empty(max(total, 1024), dtype=torch.int32, device=self.device)
        s = stream or torch.cuda.current_stream()
        with torch.cuda.stream(s):
            self.dev[:total].copy_(host[:total], non_blocking=True)
            ev = None
            if record:
                ev = torch.cuda.Event()
                ev.record(s)
        self.events[i] = ev
        if record:
            self._pending = []
        else:
            self._pending.append(i)
        base = self.dev.data_ptr()
        offs = np.cumsum([0] + sizes)
        p32 = lambda k: ctypes.cast(base + 4 * int(offs[k]), fg.i32p)
        c = self.cstruct
        c.num_seqs, c.num_tokens, c.table_stride, c.seq_capacity = S, hb.num_tokens, stride, S
        c.query_start, c.n_query, c.context_len, c.block_table = p32(0), p32(1), p32(2), p32(3)
        c.seq_index = None
        c.seq_id = None
        self.work_ptr = base + 4 * int(offs[4]) if nw else 0
        return c


    def release(self, event):
        """Guard the staging buffers of the uploads made with record=False since the last
        release by `event`, recorded on the upload stream after their copies.  Call it at least
        once every `ring` uploads: a buffer is reused only after its guard completed."""
        for i in self._pending:
            self.events[i] = event
        self._pending = []


class Workspace:
    def __init__(self, device="cuda"):
        self.device = torch.device(device)
        self.buf = None

    def ensure(self, nbytes: int):
        if nbytes <= 0:
            return 0, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(int(nbytes), dtype=torch.uint8, device=self.device)
        return self.buf.data_ptr(), self.buf.numel()
