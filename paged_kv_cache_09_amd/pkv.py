"""Thin ctypes binding of libpkv.so (see include/pkv.h for every contract).

Argument marshalling only: device pointers are passed as integers (anything
with a ``data_ptr()`` method, e.g. a torch tensor, is accepted), host arrays
as numpy arrays, streams as integers. A negative return code raises
:class:`PkvError` carrying the library's message. Importing this module fails
loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIB may name another build of the library in this directory (the
# per-wave timeline build, libpkv_timeline.so); the default is libpkv.so.
LIB_PATH = os.path.join(_HERE, os.path.basename(os.environ.get("PKV_LIB", "libpkv.so")))

F32, F16, BF16, Q8_0, Q4_0 = 0, 1, 2, 3, 4
OK, EINVAL, ECAPACITY, EOUT_OF_BLOCKS, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 32 << 20  # static scratch array per GPU (allocation-free decode)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python -m paged_kv_cache_09_amd.build` (no CPU fallback exists)")


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "layers", "num_blocks", "block_size", "kv_heads", "head_dim", "dtype", "max_seq_len",
        "max_seqs")]


class PkvError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"pkv error {code}: {message}")
        self.code = code


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_U = ctypes.c_uintptr_t if hasattr(ctypes, "c_uintptr_t") else ctypes.c_size_t

_lib = ctypes.CDLL(LIB_PATH)
_SIGS = {
    "pkv_pool_bytes": (_SZ, [ctypes.POINTER(Shape)]),
    "pkv_kv_pool_alloc": (_I, [ctypes.POINTER(Shape), _P, _SZ, ctypes.POINTER(_P)]),
    "pkv_kv_pool_free": (_I, [_P]),
    "pkv_block_alloc": (_I, [_P, _I, _P]),
    "pkv_block_claim": (_I, [_P, _P, _I]),
    "pkv_block_ref": (_I, [_P, _P, _I]),
    "pkv_block_free": (_I, [_P, _P, _I]),
    "pkv_block_refcount": (_I, [_P, ctypes.c_int32]),
    "pkv_prepare_append": (_I, [_P, _P, _I, _I, _P, _P, _P, _I, ctypes.POINTER(_I)]),
    "pkv_prepare_write": (_I, [_P, _P, _I, _I, _P, _P, _P, ctypes.c_int64, _P, _I,
                               ctypes.POINTER(_I)]),
    "pkv_block_table_upload": (_I, [_P, _P, _I, _I, _P, _P, _U]),
    "pkv_copy_blocks": (_I, [_P, _P, _I, _U]),
    "pkv_kv_append": (_I, [_P, _I, _P, _P, _P, _I, _U]),
    "pkv_paged_attn_decode": (_I, [_P, _I, _P, _I, ctypes.c_float, _P, _I, _P, _SZ, _U]),
    "pkv_append_paged_attn_decode": (_I, [_P, _I, _P, _P, _P, _I, ctypes.c_float, _P, _I, _P,
                                          _SZ, _U]),
    "pkv_paged_attn_decode_noalloc": (_I, [_P, _I, _P, _I, ctypes.c_float, _P, _I, _U]),
    "pkv_decode_workspace_bytes": (_SZ, [_P, _I, _I, _I]),
    "pkv_pool_stats": (_I, [_P, _P]),
    "pkv_schedule_stats": (_I, [_P, _P]),
    "pkv_probe_stream_read": (_I, [_P, ctypes.c_int64, _P, _I, _U]),
    "pkv_probe_gather": (_I, [_P, _I, _P, _I, _U]),
    "pkv_prefix_match": (_I, [_P, _P, _I, _P, _I]),
    "pkv_prefix_insert": (_I, [_P, _P, _I, _P, _I]),
    "pkv_prefix_stats": (_I, [_P, _P]),
    "pkv_last_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


def _ptr(x) -> int:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _np(a, dtype) -> np.ndarray:
    arr = np.ascontiguousarray(a, dtype=dtype)
    return arr


def _addr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def last_error() -> str:
    return _lib.pkv_last_error().decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise PkvError(rc, last_error())
    return rc


def make_shape(layers, num_blocks, kv_heads, head_dim, dtype, max_seq_len, max_seqs,
               block_size=16) -> Shape:
    return Shape(layers, num_blocks, block_size, kv_heads, head_dim, dtype, max_seq_len, max_seqs)


def pool_bytes(shape: Shape) -> int:
    return int(_lib.pkv_pool_bytes(ctypes.byref(shape)))


def kv_pool_alloc(shape: Shape, dev_base=None, dev_bytes: int = 0):
    h = _P()
    _check(_lib.pkv_kv_pool_alloc(ctypes.byref(shape), _ptr(dev_base), int(dev_bytes),
                                  ctypes.byref(h)))
    return h


def kv_pool_free(pool) -> None:
    _check(_lib.pkv_kv_pool_free(pool))


def block_alloc(pool, n: int) -> np.ndarray:
    out = np.zeros(max(n, 1), dtype=np.int32)
    _check(_lib.pkv_block_alloc(pool, int(n), _addr(out)))
    return out[:n]


def block_claim(pool, ids) -> None:
    a = _np(ids, np.int32)
    _check(_lib.pkv_block_claim(pool, _addr(a), a.size))


def block_ref(pool, ids) -> None:
    a = _np(ids, np.int32)
    _check(_lib.pkv_block_ref(pool, _addr(a), a.size))


def block_free(pool, ids) -> None:
    a = _np(ids, np.int32)
    _check(_lib.pkv_block_free(pool, _addr(a), a.size))


def block_refcount(pool, block_id: int) -> int:
    return _check(_lib.pkv_block_refcount(pool, int(block_id)))


def prepare_append(pool, block_table: np.ndarray, ctx_lens):
    """Slot assignment; ``block_table`` (int32 [B][max_blocks]) is updated in place.

    Returns (slots int64 [B], cow_pairs int32 [n][2]).
    """
    if block_table.dtype != np.int32 or not block_table.flags["C_CONTIGUOUS"]:
        raise TypeError("block_table must be a C-contiguous int32 array (updated in place)")
    ctx = _np(ctx_lens, np.int32)
    B, mb = block_table.shape
    slots = np.zeros(B, dtype=np.int64)
    pairs = np.zeros((B, 2), dtype=np.int32)
    n = _I(0)
    _check(_lib.pkv_prepare_append(pool, _addr(block_table), B, mb, _addr(ctx), _addr(slots),
                                   _addr(pairs), B, ctypes.byref(n)))
    return slots, pairs[:n.value].copy()


def prepare_write(pool, block_table: np.ndarray, ctx_before, n_new):
    """Slots for n_new[s] tokens per sequence after ctx_before[s] cached ones;
    ``block_table`` (int32 [B][max_blocks]) is updated in place.

    Returns (slots int64 [sum n_new], cow_pairs int32 [n][2]).
    """
    if block_table.dtype != np.int32 or not block_table.flags["C_CONTIGUOUS"]:
        raise TypeError("block_table must be a C-contiguous int32 array (updated in place)")
    before = _np(ctx_before, np.int32)
    nn = _np(n_new, np.int32)
    B, mb = block_table.shape
    total = int(nn.astype(np.int64).sum())
    slots = np.zeros(max(total, 1), dtype=np.int64)
    pairs = np.zeros((B, 2), dtype=np.int32)
    n = _I(0)
    _check(_lib.pkv_prepare_write(pool, _addr(block_table), B, mb, _addr(before), _addr(nn),
                                  _addr(slots), total, _addr(pairs), B, ctypes.byref(n)))
    return slots[:total].copy(), pairs[:n.value].copy()


def block_table_upload(pool, block_table, ctx_lens, slots=None, stream: int = 0) -> None:
    bt = _np(block_table, np.int32)
    ctx = _np(ctx_lens, np.int32)
    sl = None if slots is None else _np(slots, np.int64)
    _check(_lib.pkv_block_table_upload(pool, _addr(bt), bt.shape[0], bt.shape[1], _addr(ctx),
                                       None if sl is None else _addr(sl), int(stream)))


def copy_blocks(pool, pairs, stream: int = 0) -> None:
    a = _np(pairs, np.int32).reshape(-1, 2)
    _check(_lib.pkv_copy_blocks(pool, _addr(a) if a.size else None, a.shape[0], int(stream)))


def kv_append(pool, layer: int, k_new, v_new, dev_slots, batch: int, stream: int = 0) -> None:
    _check(_lib.pkv_kv_append(pool, int(layer), _ptr(k_new), _ptr(v_new), _ptr(dev_slots),
                              int(batch), int(stream)))


def paged_attn_decode(pool, layer: int, q, q_heads: int, scale: float, out,
                      partition_tokens: int = 0, workspace=None, ws_bytes: int = 0,
                      stream: int = 0) -> None:
    _check(_lib.pkv_paged_attn_decode(pool, int(layer), _ptr(q), int(q_heads), float(scale),
                                      _ptr(out), int(partition_tokens), _ptr(workspace),
                                      int(ws_bytes), int(stream)))


def paged_attn_decode_noalloc(pool, layer: int, q, q_heads: int, scale: float, out,
                              partition_tokens: int = 0, stream: int = 0) -> None:
    _check(_lib.pkv_paged_attn_decode_noalloc(pool, int(layer), _ptr(q), int(q_heads),
                                              float(scale), _ptr(out), int(partition_tokens),
                                              int(stream)))


def append_paged_attn_decode(pool, layer: int, k_new, v_new, q, q_heads: int, scale: float,
                             out, partition_tokens: int = 0, workspace=None, ws_bytes: int = 0,
                             stream: int = 0) -> None:
    _check(_lib.pkv_append_paged_attn_decode(pool, int(layer), _ptr(k_new), _ptr(v_new), _ptr(q),
                                             int(q_heads), float(scale), _ptr(out),
                                             int(partition_tokens), _ptr(workspace),
                                             int(ws_bytes), int(stream)))


def decode_workspace_bytes(pool, batch: int, q_heads: int, partition_tokens: int = 0) -> int:
    return int(_lib.pkv_decode_workspace_bytes(pool, int(batch), int(q_heads),
                                               int(partition_tokens)))


def pool_stats(pool) -> dict:
    out = np.zeros(4, dtype=np.int64)
    _check(_lib.pkv_pool_stats(pool, _addr(out)))
    return {"free": int(out[0]), "used": int(out[1]), "shared": int(out[2]),
            "waste_tokens": int(out[3])}


def probe_stream_read(buf, nbytes: int, out, waves: int, stream: int = 0) -> None:
    _check(_lib.pkv_probe_stream_read(_ptr(buf), int(nbytes), _ptr(out), int(waves), int(stream)))


def probe_gather(pool, layer: int, out, waves: int, stream: int = 0) -> None:
    _check(_lib.pkv_probe_gather(pool, int(layer), _ptr(out), int(waves), int(stream)))


def schedule_stats(pool) -> dict:
    out = np.zeros(4, dtype=np.int64)
    _check(_lib.pkv_schedule_stats(pool, _addr(out)))
    return {"full_builds": int(out[0]), "updates": int(out[1]), "bins": bool(out[2]),
            "waves": int(out[3])}


def prefix_match(pool, tokens, max_ids: int | None = None) -> np.ndarray:
    """Ids of the cached leading full blocks of ``tokens`` (each gains a reference)."""
    t = _np(tokens, np.int32)
    cap = t.size if max_ids is None else int(max_ids)
    ids = np.zeros(max(cap, 1), dtype=np.int32)
    k = _lib.pkv_prefix_match(pool, _addr(t), t.size, _addr(ids), cap)
    _check(min(k, 0))
    return ids[:k].copy()


def prefix_insert(pool, tokens, bt_row) -> int:
    t = _np(tokens, np.int32)
    row = _np(bt_row, np.int32)
    k = _lib.pkv_prefix_insert(pool, _addr(t), t.size, _addr(row), row.size)
    _check(min(k, 0))
    return int(k)


def prefix_stats(pool) -> dict:
    out = np.zeros(4, dtype=np.int64)
    _check(_lib.pkv_prefix_stats(pool, _addr(out)))
    return {"cached": int(out[0]), "evictable": int(out[1]), "hits": int(out[2]),
            "evictions": int(out[3])}
