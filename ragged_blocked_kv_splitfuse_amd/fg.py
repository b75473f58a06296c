"""ctypes binding of the C ABI declared in include/fg.h (argument marshalling only).

Every function here has the name of the C entry point it calls and takes host arrays as
numpy arrays and device memory as integer addresses (e.g. ``tensor.data_ptr()``) plus a
stream handle (``torch.cuda.current_stream().cuda_stream``).  Every step of the pass runs in
the library; nothing here computes.  The library must be built (``python -m
ragged_blocked_kv_splitfuse_amd.build``): loading fails loudly otherwise, there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfg.so")
FG_ITEM_INTS = 12
FG_STREAM_ROWS = 16   # query rows of a stream work item (include/fg.h)
FG_TILE_ROWS = 256    # query rows of a tile work item

FG_OK, FG_E_ARG, FG_E_DESC, FG_E_NO_BLOCKS, FG_E_UNSUPPORTED, FG_E_HIP, FG_E_WORKSPACE = range(7)
FG_F32, FG_BF16 = 0, 1
DTYPES = {"f32": FG_F32, "bf16": FG_BF16}

EXPORTS = [
    "fg_blocked_cache_init", "fg_blocked_cache_destroy", "fg_blocked_cache_num_free",
    "fg_blocked_cache_free_ids", "fg_blocked_cache_release", "fg_splitfuse_compose",
    "fg_splitfuse_commit", "fg_splitfuse_retire", "fg_validate_batch", "fg_validate_work",
    "fg_kv_append", "fg_attention_plan", "fg_ragged_attention_workspace_size",
    "fg_ragged_attention", "fg_ragged_attention_noalloc", "fg_linear_bf16",
    "fg_linear_qkv_bf16",
    "fg_status_string", "fg_last_error",
]
FG_NOALLOC_WORKSPACE_BYTES = 64 << 20   # include/fg.h

i32p = ctypes.POINTER(ctypes.c_int32)
i64p = ctypes.POINTER(ctypes.c_int64)


class FgCacheConfig(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class FgSeqState(ctypes.Structure):
    _fields_ = [("seq_id", ctypes.c_int64), ("n_cached", ctypes.c_int32),
                ("prompt_len", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("blocks", i32p),
                ("n_scheduled", ctypes.c_int32), ("stop_len", ctypes.c_int32)]


class FgRaggedBatch(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("table_stride", ctypes.c_int32), ("seq_capacity", ctypes.c_int32),
                ("query_start", i32p), ("n_query", i32p), ("context_len", i32p),
                ("block_table", i32p), ("seq_index", i32p), ("seq_id", i64p)]


class FgPlanInfo(ctypes.Structure):
    _fields_ = [("num_work", ctypes.c_int32), ("num_groups", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64),
                ("num_q_heads", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("num_items", ctypes.c_int32), ("work_ints", ctypes.c_int32)]


class FgError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{fg_status_string(status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m ragged_blocked_kv_splitfuse_amd.build`")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def load(path):
    """Use another build of the library (e.g. the host-only sanitizer build in tests)."""
    global _lib
    _lib = _declare(ctypes.CDLL(path))
    return _lib


def _declare(L):
    """Set argument and return types of the entry points the loaded library exports.

    A host-only build (the sanitizer build used in tests) lacks the device entry points;
    calling one of those raises AttributeError from ctypes, so nothing falls back silently.
    """
    st, vp = ctypes.c_int, ctypes.c_void_p
    sigs = {
        "fg_blocked_cache_init": ([ctypes.POINTER(FgCacheConfig), vp, vp, vp, ctypes.c_int32,
                                   ctypes.POINTER(vp)], st),
        "fg_blocked_cache_destroy": ([vp], st),
        "fg_blocked_cache_num_free": ([vp], ctypes.c_int32),
        "fg_blocked_cache_free_ids": ([vp, vp, ctypes.c_int32, i32p], st),
        "fg_blocked_cache_release": ([vp, vp, ctypes.c_int32], st),
        "fg_splitfuse_compose": ([vp, ctypes.POINTER(FgSeqState), ctypes.c_int32, ctypes.c_int32,
                                  ctypes.POINTER(FgRaggedBatch)], st),
        "fg_splitfuse_commit": ([ctypes.POINTER(FgSeqState), ctypes.c_int32], st),
        "fg_splitfuse_retire": ([vp, ctypes.POINTER(FgSeqState), ctypes.c_int32, i32p], st),
        "fg_validate_batch": ([vp, ctypes.POINTER(FgRaggedBatch)], st),
        "fg_validate_work": ([vp, ctypes.POINTER(FgRaggedBatch), ctypes.POINTER(FgPlanInfo), vp,
                              ctypes.c_size_t], st),
        "fg_ragged_attention_workspace_size": ([vp, ctypes.POINTER(FgRaggedBatch), ctypes.c_int32,
                                                ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)],
                                               st),
        "fg_kv_append": ([vp, ctypes.POINTER(FgRaggedBatch), vp, vp, vp], st),
        "fg_attention_plan": ([vp, ctypes.POINTER(FgRaggedBatch), ctypes.c_int32, ctypes.c_int32,
                               ctypes.POINTER(FgPlanInfo), vp, ctypes.c_int32], st),
        "fg_ragged_attention": ([vp, ctypes.POINTER(FgRaggedBatch), ctypes.POINTER(FgPlanInfo),
                                 vp, vp, ctypes.c_int32, ctypes.c_float, vp, vp,
                                 ctypes.c_size_t, vp], st),
        "fg_ragged_attention_noalloc": ([vp, ctypes.POINTER(FgRaggedBatch),
                                         ctypes.POINTER(FgPlanInfo), vp, vp, ctypes.c_int32,
                                         ctypes.c_float, vp, vp], st),
        "fg_linear_bf16": ([vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp], st),
        "fg_linear_qkv_bf16": ([vp, vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                ctypes.c_int32, vp], st),
        "fg_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "fg_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sigs.items():
        if hasattr(L, name):
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
    return L


def fg_status_string(status: int) -> str:
    return lib().fg_status_string(status).decode()


def fg_last_error() -> str:
    return lib().fg_last_error().decode()


def _check(status: int, ok=(FG_OK,)):
    if status not in ok:
        raise FgError(status, fg_last_error())
    return status


def _ptr(a: np.ndarray | None, ctype=ctypes.c_int32):
    """Typed pointer to a numpy array (for struct fields; slow-ish, use at setup)."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.cast(_addr(a), ctypes.POINTER(ctype))


def _addr(a: np.ndarray | None):
    """Address of a contiguous numpy array, cheap enough for per-call marshalling."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.__array_interface__["data"][0]


# ---- cache handle ---------------------------------------------------------------------

def fg_blocked_cache_init(num_blocks, block_size, num_kv_heads, head_dim, dtype,
                          k_pool_ptr, v_pool_ptr, free_ids=None):
    cfg = FgCacheConfig(num_blocks, block_size, num_kv_heads, head_dim, DTYPES.get(dtype, dtype))
    h = ctypes.c_void_p()
    if free_ids is None:
        _check(lib().fg_blocked_cache_init(ctypes.byref(cfg), k_pool_ptr, v_pool_ptr, None, -1,
                                           ctypes.byref(h)))
    else:
        ids = np.ascontiguousarray(free_ids, dtype=np.int32)
        _check(lib().fg_blocked_cache_init(ctypes.byref(cfg), k_pool_ptr, v_pool_ptr, _addr(ids),
                                           len(ids), ctypes.byref(h)))
    return h


def fg_blocked_cache_destroy(handle):
    _check(lib().fg_blocked_cache_destroy(handle))


def fg_blocked_cache_num_free(handle) -> int:
    return int(lib().fg_blocked_cache_num_free(handle))


def fg_blocked_cache_free_ids(handle) -> np.ndarray:
    n = ctypes.c_int32()
    _check(lib().fg_blocked_cache_free_ids(handle, None, 0, ctypes.byref(n)))
    out = np.zeros(n.value, np.int32)
    _check(lib().fg_blocked_cache_free_ids(handle, _addr(out), n.value, ctypes.byref(n)))
    return out


def fg_blocked_cache_release(handle, blocks):
    b = np.ascontiguousarray(blocks, dtype=np.int32)
    _check(lib().fg_blocked_cache_release(handle, _addr(b), len(b)))


# ---- sequences and batches (host side) -------------------------------------------------

class SeqStates:
    """A caller-owned array of fg_seq_state plus the block storage it points into."""

    def __init__(self, states, max_blocks):
        n = len(states)
        self.max_blocks = int(max_blocks)
        per_seq = [int(getattr(s, "max_blocks", max_blocks)) for s in states]
        self.blocks = np.full((max(n, 1), max([self.max_blocks, 1, *per_seq])), -1, np.int32)
        self.arr = (FgSeqState * max(n, 1))()
        self.n = n
        for i, s in enumerate(states):
            nb = len(s.blocks)
            self.blocks[i, :nb] = s.blocks
            a = self.arr[i]
            a.seq_id = s.seq_id
            a.n_cached = s.n_cached
            a.prompt_len = s.prompt_len
            a.n_blocks = nb
            a.max_blocks = per_seq[i]
            a.blocks = ctypes.cast(_addr(self.blocks) + i * self.blocks.strides[0], i32p)
            a.n_scheduled = 0
            a.stop_len = int(getattr(s, "stop_len", 0))

    def n_cached(self, i):
        return int(self.arr[i].n_cached)

    def owned(self, i):
        return self.blocks[i, :self.arr[i].n_blocks].tolist()


class HostBatch:
    """Host arrays of a fg_ragged_batch with fixed capacities."""

    def __init__(self, seq_capacity, table_stride):
        S = max(int(seq_capacity), 1)
        self.query_start = np.zeros(S + 1, np.int32)
        self.n_query = np.zeros(S, np.int32)
        self.context_len = np.zeros(S, np.int32)
        self.block_table = np.full((S, max(int(table_stride), 1)), -1, np.int32)
        self.seq_index = np.zeros(S, np.int32)
        self.seq_id = np.zeros(S, np.int64)
        self.c = FgRaggedBatch(0, 0, self.block_table.shape[1], int(seq_capacity),
                               _ptr(self.query_start), _ptr(self.n_query), _ptr(self.context_len),
                               _ptr(self.block_table), _ptr(self.seq_index),
                               _ptr(self.seq_id, ctypes.c_int64))

    @property
    def num_seqs(self):
        return int(self.c.num_seqs)

    @property
    def num_tokens(self):
        return int(self.c.num_tokens)

    @property
    def table_stride(self):
        return int(self.c.table_stride)


def fg_splitfuse_compose(handle, seqs: SeqStates, token_budget: int, out: HostBatch) -> int:
    """Returns the status (FG_OK or FG_E_NO_BLOCKS); other statuses raise."""
    return _check(lib().fg_splitfuse_compose(handle, seqs.arr, seqs.n, int(token_budget),
                                             ctypes.byref(out.c)), ok=(FG_OK, FG_E_NO_BLOCKS))


def fg_splitfuse_commit(seqs: SeqStates):
    _check(lib().fg_splitfuse_commit(seqs.arr, seqs.n))


def fg_splitfuse_retire(handle, arr, n: int) -> int:
    """Retire finished sequences of the fg_seq_state array ``arr[0..n)``; returns n_live."""
    n_live = ctypes.c_int32(0)
    _check(lib().fg_splitfuse_retire(handle, arr, int(n), ctypes.byref(n_live)))
    return int(n_live.value)


def fg_validate_batch(handle, batch: HostBatch):
    _check(lib().fg_validate_batch(handle, ctypes.byref(batch.c)))


def fg_validate_work(handle, batch: HostBatch, info: FgPlanInfo, work, workspace_bytes: int):
    w = np.ascontiguousarray(work, dtype=np.int32)
    _check(lib().fg_validate_work(handle, ctypes.byref(batch.c), ctypes.byref(info),
                                  _addr(w) if w.size else None, int(workspace_bytes)))


def fg_ragged_attention_workspace_size(handle, batch: HostBatch, num_q_heads: int,
                                       num_cus: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().fg_ragged_attention_workspace_size(handle, ctypes.byref(batch.c),
                                                    int(num_q_heads), int(num_cus),
                                                    ctypes.byref(n)))
    return int(n.value)


def fg_attention_plan(handle, batch: HostBatch, num_q_heads: int, num_cus: int, work=None):
    """Returns (FgPlanInfo, the work list as a flat int32 array of info.work_ints).

    The list is info.num_items items of FG_ITEM_INTS int32, then info.num_work record codes
    (include/fg.h).  ``work`` may be a reusable 1-D int32 buffer; the returned list is a view
    of it when it is large enough (one call), else a new array (two calls)."""
    info = FgPlanInfo()
    cap = 0 if work is None else int(work.size)
    st = lib().fg_attention_plan(handle, ctypes.byref(batch.c), int(num_q_heads), int(num_cus),
                                 ctypes.byref(info), _addr(work) if cap else None, cap)
    if st == FG_OK and info.work_ints == 0:
        return info, np.zeros(0, np.int32)
    if st == FG_OK and info.work_ints <= cap:
        return info, work.reshape(-1)[:info.work_ints]
    if st not in (FG_OK, FG_E_ARG) or info.work_ints <= cap:
        _check(st)
    work = np.zeros(max(info.work_ints, 1), np.int32)
    _check(lib().fg_attention_plan(handle, ctypes.byref(batch.c), int(num_q_heads), int(num_cus),
                                   ctypes.byref(info), _addr(work), info.work_ints))
    return info, work[:info.work_ints]


# ---- device work ------------------------------------------------------------------------

def fg_kv_append(handle, dev: FgRaggedBatch, k_new_ptr, v_new_ptr, stream):
    _check(lib().fg_kv_append(handle, ctypes.byref(dev), k_new_ptr, v_new_ptr, stream))


def fg_ragged_attention(handle, dev: FgRaggedBatch, info: FgPlanInfo, work_dev_ptr, q_ptr,
                        num_q_heads, scale, out_ptr, workspace_ptr, workspace_bytes, stream):
    _check(lib().fg_ragged_attention(handle, ctypes.byref(dev), ctypes.byref(info),
                                     work_dev_ptr or None, q_ptr,
                                     int(num_q_heads), float(scale), out_ptr, workspace_ptr,
                                     int(workspace_bytes), stream))


def fg_ragged_attention_noalloc(handle, dev: FgRaggedBatch, info: FgPlanInfo, work_dev_ptr,
                                q_ptr, num_q_heads, scale, out_ptr, stream):
    _check(lib().fg_ragged_attention_noalloc(handle, ctypes.byref(dev), ctypes.byref(info),
                                             work_dev_ptr or None, q_ptr, int(num_q_heads),
                                             float(scale), out_ptr, stream))


def fg_linear_bf16(x_ptr, w_ptr, y_ptr, T, K, N, stream):
    """y[T][N] = x[T][K] . w[N][K]^T in bf16 (device pointers)."""
    _check(lib().fg_linear_bf16(x_ptr, w_ptr, y_ptr, int(T), int(K), int(N), stream))


def fg_linear_qkv_bf16(x_ptr, wqkv_ptr, q_ptr, k_ptr, v_ptr, T, K, Nq, Nkv, stream):
    """q[T][Nq], k[T][Nkv], v[T][Nkv] = x[T][K] . w_qkv[Nq + 2*Nkv][K]^T in bf16 (device
    pointers; w_qkv stacks Wq, Wk and Wv)."""
    _check(lib().fg_linear_qkv_bf16(x_ptr, wqkv_ptr, q_ptr, k_ptr, v_ptr, int(T), int(K),
                                    int(Nq), int(Nkv), stream))
