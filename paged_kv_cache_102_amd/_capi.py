"""ctypes binding of libpagedkv (include/pagedkv.h), same names as the C ABI.

Argument marshalling only: host arrays are numpy, device buffers are torch
CUDA tensors (their data pointers are passed through), streams default to
torch's current stream.  A non-zero status raises PkvError.  The library
must be built (``__graft_entry__.build()``); importing this module without
it raises ImportError -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
_lib = C.CDLL(LIB_PATH)

PKV_OK, PKV_ERR_INVALID, PKV_ERR_OOM, PKV_ERR_UNSUPPORTED, PKV_ERR_HIP = range(5)
PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
BLOCK_SIZE = 16

_i32p = C.POINTER(C.c_int32)
_i64p = C.POINTER(C.c_int64)
_vp = C.c_void_p


class pkv_stats(C.Structure):
    _fields_ = [("num_blocks", C.c_int32), ("num_free", C.c_int32), ("num_used", C.c_int32),
                ("num_shared", C.c_int32), ("num_refs", C.c_int64), ("usage_percent", C.c_double)]


_SIGS = {
    "pkv_status_string": (C.c_char_p, [C.c_int]),
    "pkv_pool_create": (C.c_int, [C.c_int32, C.c_int32, _i32p, C.POINTER(_vp)]),
    "pkv_pool_destroy": (None, [_vp]),
    "kv_block_alloc": (C.c_int, [_vp, C.c_int32, _i32p]),
    "kv_block_share": (C.c_int, [_vp, C.c_int32, _i32p]),
    "kv_block_free": (C.c_int, [_vp, C.c_int32, _i32p]),
    "kv_block_cow": (C.c_int, [_vp, C.c_int32, _i32p, _i32p]),
    "kv_block_refcount": (C.c_int, [_vp, C.c_int32, _i32p]),
    "kv_pool_stats": (C.c_int, [_vp, C.POINTER(pkv_stats)]),
    "kv_pool_free_list": (C.c_int, [_vp, C.c_int32, _i32p, _i32p]),
    "pkv_prefix_cache_enable": (C.c_int, [_vp]),
    "pkv_prefix_match": (C.c_int, [_vp, _i32p, C.c_int32, C.c_int32, _i32p, _i32p]),
    "pkv_prefix_register": (C.c_int, [_vp, _i32p, C.c_int32, _i32p]),
    "pkv_prefix_stats": (C.c_int, [_vp, _i32p, _i32p]),
    "kv_block_swap": (C.c_int, [_vp, _vp, C.c_int32, _i32p, _i32p, _i32p, _i32p]),
    "pkv_window_release": (C.c_int, [_vp, C.c_int32, C.c_int32, _i32p, _i32p, C.c_int32, _i32p,
                                     C.c_int32, _i32p]),
    "paged_kv_append_slots": (C.c_int, [_vp, C.c_int32, C.c_int32, _i32p, _i32p, _i32p, _i64p,
                                        C.c_int64, _i32p, C.c_int32, _i32p, _i32p, C.c_int32,
                                        _i32p]),
    "paged_block_table_update": (C.c_int, [_vp, C.c_int64, _vp, C.c_int32, _vp]),
    "paged_kv_write": (C.c_int, [_vp, _vp, _vp, _vp, _vp, C.c_int32, C.c_int32, C.c_int32,
                                 C.c_int32, C.c_int, _vp]),
    "paged_kv_append": (C.c_int, [_vp, _vp, _vp, _vp, _vp, C.c_int32, C.c_int32, C.c_int32,
                                  C.c_int32, C.c_int, _vp, C.c_int64, _vp, C.c_int32, _vp]),
    "paged_kv_copy_blocks": (C.c_int, [_vp, _vp, _vp, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                       C.c_int, _vp]),
    "paged_attention_workspace_size": (C.c_size_t, [C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                                    C.c_int32, C.c_int32]),
    "paged_attention_decode": (C.c_int, [_vp, _vp, _vp, _vp, _vp, C.c_int32, C.c_int32, C.c_int32,
                                         C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_float,
                                         C.c_int32, _vp, C.c_size_t, C.c_int, _vp, _vp]),
    "paged_attention_prefill": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, C.c_int32, C.c_int32,
                                          C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                          C.c_int32, C.c_float, C.c_int32, C.c_int, _vp, _vp]),
    "paged_attention_prefill_fp8": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, C.c_int32, C.c_int32,
                                              C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                              C.c_int32, C.c_int32, C.c_float, C.c_int32,
                                              C.c_float, C.c_float, _vp, _vp]),
    "paged_attention_decode_window": (C.c_int, [_vp, _vp, _vp, _vp, _vp, C.c_int32, C.c_int32,
                                                C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                                C.c_int32, C.c_float, C.c_int32, C.c_int32, _vp,
                                                C.c_size_t, C.c_int, C.c_float, C.c_float, _vp,
                                                _vp]),
    "paged_kv_append_decode": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                         C.c_int32, C.c_int32, C.c_int32, C.c_float, C.c_int32,
                                         _vp, C.c_size_t, C.c_int, _vp, _vp]),
    "paged_attention_decode_noalloc": (C.c_int, [_vp, _vp, _vp, _vp, _vp, C.c_int32, C.c_int32,
                                                 C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                                 C.c_int32, C.c_float, C.c_int32, C.c_int,
                                                 C.c_float, C.c_float, _vp, _vp]),
    "paged_kv_swap_blocks": (C.c_int, [_vp, _vp, _vp, _vp, _vp, C.c_int32, C.c_int32, C.c_int32,
                                       C.c_int32, C.c_int32, C.c_int, _vp]),
    "paged_attention_decode_fp8": (C.c_int, [_vp, _vp, _vp, _vp, _vp, C.c_int32, C.c_int32,
                                             C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                             C.c_float, C.c_float, C.c_float, _vp, C.c_size_t, _vp,
                                             _vp]),
    "paged_kv_write_fp8": (C.c_int, [_vp, _vp, C.c_int, _vp, _vp, _vp, C.c_int32, C.c_int32,
                                     C.c_int32, C.c_int32, C.c_float, C.c_float, _vp]),
    "pkv_profile_begin": (C.c_int, [C.c_int32]),
    "pkv_profile_end": (C.c_int, [_i32p, C.POINTER(C.c_double)]),
    "pkv_profile_durations": (C.c_int, [C.POINTER(C.c_float), C.c_int32, _i32p]),
    "pkv_stream_read": (C.c_int, [_vp, C.c_size_t, _vp, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.pkv_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def _check(st: int, where: str):
    if st != PKV_OK:
        raise PkvError(st, where)


def pkv_status_string(status: int) -> str:
    return _lib.pkv_status_string(status).decode()


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_i32p)


# --------------------------------------------------------------------------- pool
class Pool:
    """Owns a pkv_pool handle."""

    def __init__(self, handle):
        self.handle = handle
        # held here: at interpreter exit the module's globals may be gone
        # before the last pool is collected
        self._destroy = _lib.pkv_pool_destroy

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h:
            self._destroy(h)


def pkv_pool_create(num_blocks: int, block_size: int = BLOCK_SIZE, init_order=None) -> Pool:
    h = _vp()
    if init_order is None:
        st = _lib.pkv_pool_create(num_blocks, block_size, None, C.byref(h))
    else:
        arr, ptr = _i32(init_order)
        st = _lib.pkv_pool_create(num_blocks, block_size, ptr, C.byref(h))
    _check(st, "pkv_pool_create")
    return Pool(h)


def kv_block_alloc(pool: Pool, n: int) -> np.ndarray:
    out = np.empty(max(n, 0), dtype=np.int32)
    _check(_lib.kv_block_alloc(pool.handle, n, out.ctypes.data_as(_i32p)), "kv_block_alloc")
    return out


def kv_block_share(pool: Pool, ids) -> None:
    arr, ptr = _i32(ids)
    _check(_lib.kv_block_share(pool.handle, arr.size, ptr), "kv_block_share")


def kv_block_free(pool: Pool, ids) -> None:
    arr, ptr = _i32(ids)
    _check(_lib.kv_block_free(pool.handle, arr.size, ptr), "kv_block_free")


def kv_block_cow(pool: Pool, block_id: int):
    out, copy = C.c_int32(), C.c_int32()
    _check(_lib.kv_block_cow(pool.handle, block_id, C.byref(out), C.byref(copy)), "kv_block_cow")
    return out.value, bool(copy.value)


def kv_block_refcount(pool: Pool, block_id: int) -> int:
    out = C.c_int32()
    _check(_lib.kv_block_refcount(pool.handle, block_id, C.byref(out)), "kv_block_refcount")
    return out.value


def kv_pool_stats(pool: Pool) -> dict:
    s = pkv_stats()
    _check(_lib.kv_pool_stats(pool.handle, C.byref(s)), "kv_pool_stats")
    return {f: getattr(s, f) for f, _ in pkv_stats._fields_}


def kv_pool_free_list(pool: Pool) -> np.ndarray:
    n = C.c_int32()
    _check(_lib.kv_pool_free_list(pool.handle, 0, None, C.byref(n)), "kv_pool_free_list")
    out = np.empty(n.value, dtype=np.int32)
    _check(_lib.kv_pool_free_list(pool.handle, n.value, out.ctypes.data_as(_i32p), C.byref(n)),
           "kv_pool_free_list")
    return out


def pkv_prefix_cache_enable(pool: Pool) -> None:
    _check(_lib.pkv_prefix_cache_enable(pool.handle), "pkv_prefix_cache_enable")


def pkv_prefix_match(pool: Pool, tokens, max_blocks: int | None = None) -> np.ndarray:
    """Ids of the cached blocks holding the longest indexed prefix of tokens
    (one reference taken on each)."""
    arr, ptr = _i32(tokens)
    cap = arr.size // BLOCK_SIZE if max_blocks is None else max_blocks
    out = np.empty(max(cap, 1), dtype=np.int32)
    n = C.c_int32()
    _check(_lib.pkv_prefix_match(pool.handle, ptr, arr.size, cap, out.ctypes.data_as(_i32p),
                                 C.byref(n)), "pkv_prefix_match")
    return out[:n.value].copy()


def pkv_prefix_register(pool: Pool, tokens, block_ids) -> None:
    arr, ptr = _i32(tokens)
    ids, iptr = _i32(block_ids)
    if ids.size < arr.size // BLOCK_SIZE:
        raise ValueError("fewer block ids than full blocks")
    _check(_lib.pkv_prefix_register(pool.handle, ptr, arr.size, iptr), "pkv_prefix_register")


def pkv_prefix_stats(pool: Pool):
    a, b = C.c_int32(), C.c_int32()
    _check(_lib.pkv_prefix_stats(pool.handle, C.byref(a), C.byref(b)), "pkv_prefix_stats")
    return a.value, b.value


def kv_block_swap(from_pool: Pool, to_pool: Pool, ids):
    """Moves the references ids (held in from_pool) to fresh blocks of
    to_pool.  Returns (new ids int32 [n], pairs int32 [k][2] of (old, new))."""
    arr, ptr = _i32(ids)
    n = arr.size
    out = np.empty(max(n, 1), dtype=np.int32)
    pairs = np.empty((max(n, 1), 2), dtype=np.int32)
    k = C.c_int32()
    _check(_lib.kv_block_swap(from_pool.handle, to_pool.handle, n, ptr,
                              out.ctypes.data_as(_i32p), pairs.ctypes.data_as(_i32p),
                              C.byref(k)), "kv_block_swap")
    return out[:n].copy(), pairs[:k.value].copy()


def pkv_window_release(pool: Pool, block_tables: np.ndarray, context_lens, window: int):
    """block_tables int32 [B][max_blocks] is updated in place.  Returns the
    table updates int32 [n][2] of (flat index, -1)."""
    assert block_tables.dtype == np.int32 and block_tables.flags.c_contiguous
    B, mb = block_tables.shape
    lens, lptr = _i32(context_lens)
    cap = int(np.count_nonzero(block_tables >= 0))
    upd = np.empty((max(cap, 1), 2), dtype=np.int32)
    nu = C.c_int32()
    _check(_lib.pkv_window_release(pool.handle, B, mb, block_tables.ctypes.data_as(_i32p), lptr,
                                   window, upd.ctypes.data_as(_i32p), cap, C.byref(nu)),
           "pkv_window_release")
    return upd[:nu.value].copy()


def paged_kv_append_slots(pool: Pool, block_tables: np.ndarray, context_lens: np.ndarray,
                          num_new=None):
    """block_tables int32 [B][max_blocks] and context_lens int32 [B] are
    updated in place.  Returns (slot_mapping int64, table_updates int32 [n][2],
    cow_pairs int32 [n][2])."""
    assert block_tables.dtype == np.int32 and block_tables.flags.c_contiguous
    assert context_lens.dtype == np.int32 and context_lens.flags.c_contiguous
    B, mb = block_tables.shape
    if num_new is None:
        nn, nn_ptr, total = None, None, B
    else:
        nn, nn_ptr = _i32(num_new)
        total = int(nn.sum())
    upd_cap = total + B
    slots = np.empty(max(total, 1), dtype=np.int64)
    upd = np.empty((upd_cap, 2), dtype=np.int32)
    cows = np.empty((max(B, 1), 2), dtype=np.int32)
    nu, nc = C.c_int32(), C.c_int32()
    st = _lib.paged_kv_append_slots(pool.handle, B, mb, block_tables.ctypes.data_as(_i32p),
                                    context_lens.ctypes.data_as(_i32p), nn_ptr,
                                    slots.ctypes.data_as(_i64p), total,
                                    upd.ctypes.data_as(_i32p), upd_cap, C.byref(nu),
                                    cows.ctypes.data_as(_i32p), B, C.byref(nc))
    _check(st, "paged_kv_append_slots")
    return slots[:total], upd[:nu.value], cows[:nc.value]



class AppendPlanner:
    """paged_kv_append_slots bound once to a pool and to host tables and
    lengths (int32 [B][max_blocks] and [B], updated in place and never
    reallocated), with output buffers kept between calls: per call only the
    counts of new tokens are converted.  Returns what paged_kv_append_slots
    returns, as arrays of the caller's own."""

    def __init__(self, pool: Pool, block_tables: np.ndarray, context_lens: np.ndarray):
        assert block_tables.dtype == np.int32 and block_tables.flags.c_contiguous
        assert context_lens.dtype == np.int32 and context_lens.flags.c_contiguous
        self._pool, self._tables, self._lens = pool, block_tables, context_lens
        self._B, self._mb = block_tables.shape
        self._tp = block_tables.ctypes.data_as(_i32p)
        self._lp = context_lens.ctypes.data_as(_i32p)
        self._nn = np.ones(self._B, dtype=np.int32)
        self._nnp = self._nn.ctypes.data_as(_i32p)
        self._cows = np.empty((max(self._B, 1), 2), dtype=np.int32)
        self._cp = self._cows.ctypes.data_as(_i32p)
        self._nu, self._nc = C.c_int32(), C.c_int32()
        self._nur, self._ncr = C.byref(self._nu), C.byref(self._nc)
        self._fn = _lib.paged_kv_append_slots
        self._grow(self._B)

    def _grow(self, total: int):
        self._cap = total
        self._slots = np.empty(max(total, 1), dtype=np.int64)
        self._sp = self._slots.ctypes.data_as(_i64p)
        self._upd = np.empty((total + self._B, 2), dtype=np.int32)
        self._up = self._upd.ctypes.data_as(_i32p)

    def __call__(self, num_new=None):
        if num_new is None:
            nn_ptr, total = None, self._B
        else:
            self._nn[:] = num_new
            nn_ptr, total = self._nnp, int(self._nn.sum())
        if total > self._cap:
            self._grow(total)
        _check(self._fn(self._pool.handle, self._B, self._mb, self._tp, self._lp, nn_ptr, self._sp,
                        total, self._up, self._upd.shape[0], self._nur, self._cp, self._B,
                        self._ncr), "paged_kv_append_slots")
        return (self._slots[:total].copy(), self._upd[:self._nu.value].copy(),
                self._cows[:self._nc.value].copy())

# --------------------------------------------------------------------------- device calls
def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dev(t, name):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")
    return t.data_ptr()


def _dev_or_pinned(t, name):
    """Device tensor, or host tensor in pinned (device-accessible) memory."""
    if not t.is_contiguous() or not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a contiguous device or pinned host tensor")
    return t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return PKV_BF16
    if t.dtype == torch.uint8:
        return PKV_FP8_E4M3
    raise ValueError(f"unsupported cache dtype {t.dtype}")


def paged_block_table_update(block_tables, updates, stream=None) -> None:
    n = updates.shape[0]
    if n == 0:
        return
    _check(_lib.paged_block_table_update(_dev(block_tables, "block_tables"), block_tables.numel(),
                                         _dev_or_pinned(updates, "updates"), n, _stream(stream)),
           "paged_block_table_update")


def paged_kv_write(k_new, v_new, slot_mapping, k_cache, v_cache, num_kv_heads: int,
                   head_dim: int, num_blocks: int, stream=None) -> None:
    n = slot_mapping.shape[0]
    if n == 0:
        return
    _check(_lib.paged_kv_write(_dev(k_new, "k_new"), _dev(v_new, "v_new"),
                               _dev_or_pinned(slot_mapping, "slot_mapping"),
                               _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), n,
                               num_kv_heads, head_dim, num_blocks, _dtype_code(k_cache),
                               _stream(stream)), "paged_kv_write")


def paged_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, num_kv_heads: int,
                    head_dim: int, num_blocks: int, block_tables, updates, stream=None) -> None:
    n = slot_mapping.shape[0]
    nu = updates.shape[0]
    if n == 0 and nu == 0:
        return
    _check(_lib.paged_kv_append(_dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                _dev_or_pinned(slot_mapping, "slot_mapping"),
                                _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), n,
                                num_kv_heads, head_dim, num_blocks, _dtype_code(k_cache),
                                _dev(block_tables, "block_tables"), block_tables.numel(),
                                _dev_or_pinned(updates, "updates") if nu else None, nu,
                                _stream(stream)), "paged_kv_append")


def paged_kv_copy_blocks(k_cache, v_cache, pairs, num_kv_heads: int, head_dim: int,
                         num_blocks: int, stream=None) -> None:
    n = pairs.shape[0]
    if n == 0:
        return
    _check(_lib.paged_kv_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                     _dev_or_pinned(pairs, "pairs"), n, num_kv_heads, head_dim,
                                     num_blocks, _dtype_code(k_cache), _stream(stream)),
           "paged_kv_copy_blocks")


def paged_kv_swap_blocks(src_k, src_v, dst_k, dst_v, pairs, num_kv_heads: int, head_dim: int,
                         src_num_blocks: int, dst_num_blocks: int, stream=None) -> None:
    """Copies blocks pairs[i][0] of (src_k, src_v) to pairs[i][1] of (dst_k,
    dst_v); caches and pairs on the device or in pinned host memory."""
    n = pairs.shape[0]
    if n == 0:
        return
    if _dtype_code(src_k) != _dtype_code(dst_k):
        raise ValueError("source and destination caches differ in dtype")
    _check(_lib.paged_kv_swap_blocks(_dev_or_pinned(src_k, "src_k"), _dev_or_pinned(src_v, "src_v"),
                                     _dev_or_pinned(dst_k, "dst_k"), _dev_or_pinned(dst_v, "dst_v"),
                                     _dev_or_pinned(pairs, "pairs"), n, num_kv_heads, head_dim,
                                     src_num_blocks, dst_num_blocks, _dtype_code(src_k),
                                     _stream(stream)), "paged_kv_swap_blocks")


def paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                   max_context_len, partition_size=0) -> int:
    return int(_lib.paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                   max_context_len, partition_size))


def paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, out, *,
                           num_kv_heads: int, num_blocks: int, max_context_len: int,
                           scale: float, partition_size: int = 0, workspace=None,
                           stream=None) -> None:
    B, Hq, D = q.shape
    mb = block_tables.shape[1]
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.paged_attention_decode(_dev(q, "q"), _dev(k_cache, "k_cache"),
                                       _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
                                       _dev(context_lens, "context_lens"), B, Hq, num_kv_heads, D,
                                       num_blocks, mb, max_context_len, scale, partition_size,
                                       ws_ptr, ws_bytes, _dtype_code(k_cache), _dev(out, "out"),
                                       _stream(stream)), "paged_attention_decode")


def paged_attention_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, out, *,
                            num_kv_heads: int, num_blocks: int, max_context_len: int,
                            max_query_len: int, scale: float, window: int = 0,
                            stream=None) -> None:
    """q [T][Hq][D] (chunk rows of all sequences, in order), query_start
    int32 [B + 1]; out [T][Hq][D] fp32; window 0 = no sliding window."""
    T, Hq, D = q.shape
    B = context_lens.shape[0]
    mb = block_tables.shape[1]
    _check(_lib.paged_attention_prefill(_dev(q, "q"), _dev(k_cache, "k_cache"),
                                        _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
                                        _dev(context_lens, "context_lens"),
                                        _dev(query_start, "query_start"), B, Hq, num_kv_heads, D,
                                        num_blocks, mb, max_context_len, max_query_len, scale,
                                        window, _dtype_code(k_cache), _dev(out, "out"),
                                        _stream(stream)),
           "paged_attention_prefill")


def paged_attention_prefill_fp8(q, k_cache, v_cache, block_tables, context_lens, query_start, out,
                                *, num_kv_heads: int, num_blocks: int, max_context_len: int,
                                max_query_len: int, scale: float, k_scale: float, v_scale: float,
                                window: int = 0, stream=None) -> None:
    """paged_attention_prefill over FP8 E4M3 caches (uint8 codes) with tensor
    scales; q bf16 [T][Hq][D], out fp32."""
    T, Hq, D = q.shape
    B = context_lens.shape[0]
    mb = block_tables.shape[1]
    _check(_lib.paged_attention_prefill_fp8(_dev(q, "q"), _dev(k_cache, "k_cache"),
                                            _dev(v_cache, "v_cache"),
                                            _dev(block_tables, "block_tables"),
                                            _dev(context_lens, "context_lens"),
                                            _dev(query_start, "query_start"), B, Hq, num_kv_heads,
                                            D, num_blocks, mb, max_context_len, max_query_len,
                                            scale, window, k_scale, v_scale, _dev(out, "out"),
                                            _stream(stream)),
           "paged_attention_prefill_fp8")


def paged_kv_write_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, num_kv_heads: int,
                       head_dim: int, num_blocks: int, k_scale: float, v_scale: float,
                       stream=None) -> None:
    """k_new, v_new: bf16 or fp32 [T][Hkv][D]; caches: uint8 FP8 E4M3 codes."""
    n = slot_mapping.shape[0]
    if n == 0:
        return
    _check(_lib.paged_kv_write_fp8(_dev(k_new, "k_new"), _dev(v_new, "v_new"), _dtype_code(k_new),
                                   _dev_or_pinned(slot_mapping, "slot_mapping"),
                                   _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), n,
                                   num_kv_heads, head_dim, num_blocks, k_scale, v_scale,
                                   _stream(stream)), "paged_kv_write_fp8")


def paged_attention_decode_fp8(q, k_cache, v_cache, block_tables, context_lens, out, *,
                               num_kv_heads: int, num_blocks: int, max_context_len: int,
                               scale: float, k_scale: float, v_scale: float, workspace=None,
                               stream=None) -> None:
    B, Hq, D = q.shape
    mb = block_tables.shape[1]
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.paged_attention_decode_fp8(_dev(q, "q"), _dev(k_cache, "k_cache"),
                                           _dev(v_cache, "v_cache"),
                                           _dev(block_tables, "block_tables"),
                                           _dev(context_lens, "context_lens"), B, Hq, num_kv_heads,
                                           D, num_blocks, mb, max_context_len, scale, k_scale,
                                           v_scale, ws_ptr, ws_bytes, _dev(out, "out"),
                                           _stream(stream)), "paged_attention_decode_fp8")


def paged_attention_decode_window(q, k_cache, v_cache, block_tables, context_lens, out, *,
                                  num_kv_heads: int, num_blocks: int, max_context_len: int,
                                  scale: float, window: int, partition_size: int = 0,
                                  k_scale: float = 1.0, v_scale: float = 1.0, workspace=None,
                                  stream=None) -> None:
    B, Hq, D = q.shape
    mb = block_tables.shape[1]
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.paged_attention_decode_window(_dev(q, "q"), _dev(k_cache, "k_cache"),
                                              _dev(v_cache, "v_cache"),
                                              _dev(block_tables, "block_tables"),
                                              _dev(context_lens, "context_lens"), B, Hq,
                                              num_kv_heads, D, num_blocks, mb, max_context_len,
                                              scale, window, partition_size, ws_ptr, ws_bytes,
                                              _dtype_code(k_cache), k_scale, v_scale,
                                              _dev(out, "out"), _stream(stream)),
           "paged_attention_decode_window")


def paged_kv_append_decode(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                           lens_in, lens_out, updates, out, *, num_kv_heads: int, num_blocks: int,
                           max_context_len: int, scale: float, window: int = 0, workspace=None,
                           stream=None) -> None:
    """One decode step in one launch (see pagedkv.h): k_new / v_new [B][Hkv][D]
    bf16 rows, slot_mapping int64 [B] and updates int32 [n][2] (device or
    pinned host tensors), lens_in / lens_out two distinct int32 [B] device
    buffers."""
    B, Hq, D = q.shape
    mb = block_tables.shape[1]
    n_upd = int(updates.shape[0]) if updates is not None and updates.numel() else 0
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.paged_kv_append_decode(_dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                       _dev_or_pinned(slot_mapping, "slot_mapping"),
                                       _dev(k_cache, "k_cache"),
                                       _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
                                       _dev(lens_in, "lens_in"), _dev(lens_out, "lens_out"),
                                       _dev_or_pinned(updates, "updates") if n_upd else None,
                                       n_upd, B, Hq,
                                       num_kv_heads, D, num_blocks, mb, max_context_len, scale,
                                       window, ws_ptr, ws_bytes, _dtype_code(k_cache),
                                       _dev(out, "out"), _stream(stream)),
           "paged_kv_append_decode")


def paged_attention_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, out, *,
                                   num_kv_heads: int, num_blocks: int, max_context_len: int,
                                   scale: float, window: int = 0, k_scale: float = 1.0,
                                   v_scale: float = 1.0, stream=None) -> None:
    """Decode without a workspace: partial states in the library's static
    per-GPU scratch (calls on one GPU must not overlap)."""
    B, Hq, D = q.shape
    mb = block_tables.shape[1]
    _check(_lib.paged_attention_decode_noalloc(_dev(q, "q"), _dev(k_cache, "k_cache"),
                                               _dev(v_cache, "v_cache"),
                                               _dev(block_tables, "block_tables"),
                                               _dev(context_lens, "context_lens"), B, Hq,
                                               num_kv_heads, D, num_blocks, mb, max_context_len,
                                               scale, window, _dtype_code(k_cache), k_scale,
                                               v_scale, _dev(out, "out"), _stream(stream)),
           "paged_attention_decode_noalloc")


def pkv_profile_begin(every: int = 1) -> None:
    """Times decode calls 0, every, 2 every, ... until pkv_profile_end."""
    _check(_lib.pkv_profile_begin(every), "pkv_profile_begin")


def pkv_profile_end():
    n, ms = C.c_int32(), C.c_double()
    _check(_lib.pkv_profile_end(C.byref(n), C.byref(ms)), "pkv_profile_end")
    return n.value, ms.value


def pkv_profile_durations(capacity: int = 8192):
    """Durations (ms) of the launches timed so far in this session."""
    buf = (C.c_float * max(capacity, 1))()
    n = C.c_int32()
    _check(_lib.pkv_profile_durations(buf, capacity, C.byref(n)), "pkv_profile_durations")
    return [buf[i] for i in range(min(n.value, capacity))]


def pkv_stream_read(buf, sink, stream=None) -> None:
    _check(_lib.pkv_stream_read(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                _dev(sink, "sink"), _stream(stream)), "pkv_stream_read")
