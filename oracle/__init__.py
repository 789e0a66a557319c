"""Plain fp64 CPU oracle for paged KV-cache decode (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the GPU library
and imports nothing from it.

Parts:
  * ``oracle.c`` (built to ``liboracle.so`` by :func:`build`): closed-form KV
    size, append, gather and fp64 softmax attention, plus a partitioned
    (per-partition max/sum, then merge) form of the same attention; the q8_0
    quantised cache (quantisation of new rows, exact dequantisation).
  * :mod:`oracle.brute`: the same attention in pure-Python loops, for tiny
    inputs.
  * :mod:`oracle.block_model`: a plain model of on-demand block allocation,
    refcounted sharing and copy-on-write.

The wrappers below take numpy arrays and only marshal arguments.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

F32, F16, BF16, Q8_0, Q4_0 = 0, 1, 2, 3, 4
QUANTISED = (Q8_0, Q4_0)
_NP_STORAGE = {F32: np.float32, F16: np.uint16, BF16: np.uint16, Q8_0: np.uint8, Q4_0: np.uint8}
Q8_GROUP = 32


def code_row_bytes(dtype: int, head_dim: int) -> int:
    """Code bytes of one quantised row: head_dim (q8_0) or head_dim / 2 (q4_0)."""
    return head_dim // 2 if dtype == Q4_0 else head_dim


def q_tile_bytes(dtype: int, head_dim: int, block_size: int = 16) -> int:
    """Bytes of one quantised (block, kv head) tile: codes, then fp16 scales."""
    return block_size * code_row_bytes(dtype, head_dim) + block_size * (head_dim // Q8_GROUP) * 2


def q8_tile_bytes(head_dim: int, block_size: int = 16) -> int:
    return q_tile_bytes(Q8_0, head_dim, block_size)


def input_dtype(dtype: int) -> int:
    """Storage type of q, k_new and v_new for a cache of `dtype` (bf16 when quantised)."""
    return BF16 if dtype in QUANTISED else dtype


_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O3 -fopenmp, no fast-math, no contraction of a*b+c)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.run(
            ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
             "-ffp-contract=off",
             "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        i64 = ctypes.c_int64
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [i32]
        L.orc_kv_bytes_per_token.restype = i64
        L.orc_kv_bytes_per_token.argtypes = [i64, i64, i64, i64]
        L.orc_elem_to_double.restype = ctypes.c_double
        L.orc_elem_to_double.argtypes = [P, i64, i32]
        L.orc_append.restype = None
        L.orc_append.argtypes = [i32, i32, i32, i32, i32, P, P, P, i32, P, P, P]
        L.orc_gather.restype = None
        L.orc_gather.argtypes = [i32, i32, i32, i32, P, P, P, i32, i32, P, P]
        L.orc_decode.restype = None
        L.orc_decode.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, i32, P, P,
                                 ctypes.c_double, P]
        L.orc_float_to_half.restype = None
        L.orc_float_to_half.argtypes = [P, i64, P]
        L.orc_q8_quantize.restype = None
        L.orc_q8_quantize.argtypes = [P, i64, P, P]
        L.orc_q4_quantize.restype = None
        L.orc_q4_quantize.argtypes = [P, i64, P, P]
        L.orc_decode_partitioned.restype = None
        L.orc_decode_partitioned.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, i32, P,
                                             P, ctypes.c_double, i32, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _storage(a: np.ndarray, dtype: int) -> np.ndarray:
    want = _NP_STORAGE[dtype]
    if a.dtype != want:
        raise TypeError(f"expected storage dtype {np.dtype(want)} for code {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def set_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops (for timing; results do not depend on it)."""
    lib().orc_set_threads(int(n))


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    return int(lib().orc_kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_elem))


def elem_to_double(storage: np.ndarray, dtype: int) -> np.ndarray:
    s = _storage(storage.reshape(-1), dtype)
    L = lib()
    return np.array([L.orc_elem_to_double(_ptr(s), i, dtype) for i in range(s.size)])


def float_to_half_bits(x) -> np.ndarray:
    """fp32 values -> IEEE binary16 bit patterns (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.zeros(x.size, dtype=np.uint16)
    lib().orc_float_to_half(_ptr(x), x.size, _ptr(out))
    return out


def q8_quantize(x):
    """q8_0 groups of 32 fp32 values -> (int8 codes [n][32], fp16 scale bits [n])."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, Q8_GROUP)
    codes = np.zeros(x.shape, dtype=np.int8)
    d = np.zeros(x.shape[0], dtype=np.uint16)
    lib().orc_q8_quantize(_ptr(x), x.shape[0], _ptr(codes), _ptr(d))
    return codes, d


def q4_quantize(x):
    """q4_0 groups of 32 fp32 values -> (4-bit codes 0..15 [n][32] as uint8, fp16 scale bits [n])."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, Q8_GROUP)
    codes = np.zeros(x.shape, dtype=np.uint8)
    d = np.zeros(x.shape[0], dtype=np.uint16)
    lib().orc_q4_quantize(_ptr(x), x.shape[0], _ptr(codes), _ptr(d))
    return codes, d


def _head_dim_of_qtile(dtype, tile_bytes, block_size):
    # tile = bs * (D * c) + bs * D / 16 with c = 1 (q8_0) or 1/2 (q4_0)
    per_row = tile_bytes // block_size
    D = per_row * 16 // 17 if dtype == Q8_0 else per_row * 16 // 9
    assert q_tile_bytes(dtype, D, block_size) == tile_bytes
    return D


def _pool_shape(pool, dtype, block_size, head_dim):
    """(NB, Hkv) of a layer array: [NB][Hkv][bs][D], or [NB][Hkv][tile bytes] when quantised."""
    if dtype in QUANTISED:
        assert pool.ndim == 3 and pool.shape[2] == q_tile_bytes(dtype, head_dim, block_size)
    else:
        assert pool.ndim == 4 and pool.shape[2] == block_size and pool.shape[3] == head_dim
    return pool.shape[0], pool.shape[1]


def append(k_pool, v_pool, block_table, ctx_lens, k_new, v_new, *, dtype, block_size=16):
    """In-place append into one layer's K/V pool arrays ([NB][Hkv][bs][D], or
    [NB][Hkv][tile bytes] uint8 for q8_0 / q4_0, whose new rows come in bf16)."""
    k_pool = _storage(k_pool, dtype)
    v_pool = _storage(v_pool, dtype)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    kn = _storage(k_new, input_dtype(dtype))
    vn = _storage(v_new, input_dtype(dtype))
    B, Hkv, D = kn.shape
    assert _pool_shape(k_pool, dtype, block_size, D)[1] == Hkv
    _check_tables(bt, ctx, k_pool.shape[0], block_size)
    lib().orc_append(B, Hkv, D, block_size, dtype, _ptr(k_pool), _ptr(v_pool), _ptr(bt),
                     bt.shape[1], _ptr(ctx), _ptr(kn), _ptr(vn))
    return k_pool, v_pool


def gather(k_pool, v_pool, bt_row, n_tokens, g, *, dtype, block_size=16):
    """Contiguous fp64 K and V rows [n_tokens][D] of kv head g for one sequence."""
    k_pool = _storage(k_pool, dtype)
    v_pool = _storage(v_pool, dtype)
    row = np.ascontiguousarray(bt_row, dtype=np.int32)
    if dtype in QUANTISED:
        NB, Hkv, tb = k_pool.shape
        D = _head_dim_of_qtile(dtype, tb, block_size)
    else:
        NB, Hkv, bs, D = k_pool.shape
    _check_tables(row[None, :], np.array([n_tokens]), NB, block_size)
    ok = np.zeros((max(n_tokens, 1), D))
    ov = np.zeros((max(n_tokens, 1), D))
    lib().orc_gather(Hkv, D, block_size, dtype, _ptr(k_pool), _ptr(v_pool), _ptr(row),
                     n_tokens, g, _ptr(ok), _ptr(ov))
    return ok[:n_tokens], ov[:n_tokens]


def _check_tables(bt, ctx, num_blocks, block_size):
    """Every table entry a sequence reads must name a block of the pool."""
    if bt.shape[0] != ctx.shape[0]:
        raise ValueError("block table and context lengths disagree on the batch")
    for s, L in enumerate(ctx):
        n = (int(L) + block_size - 1) // block_size
        if L < 0 or n > bt.shape[1]:
            raise ValueError(f"sequence {s}: length {L} does not fit the table")
        row = bt[s, :n]
        if n and (row.min() < 0 or row.max() >= num_blocks):
            raise ValueError(f"sequence {s}: table entry outside [0, {num_blocks})")


def decode(k_pool, v_pool, block_table, ctx_lens, q, scale, *, dtype, block_size=16,
           partition_tokens: int = 0):
    """fp64 attention output [B][Hq][D] for one layer read through the block table.

    ``partition_tokens`` > 0 computes the partitioned form (per-partition
    max/sum/output, then merged); 0 computes the plain definition.
    """
    k_pool = _storage(k_pool, dtype)
    v_pool = _storage(v_pool, dtype)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    qq = _storage(q, input_dtype(dtype))
    B, Hq, D = qq.shape
    NB, Hkv = _pool_shape(k_pool, dtype, block_size, D)
    assert Hq % Hkv == 0
    _check_tables(bt, ctx, NB, block_size)
    out = np.zeros((B, Hq, D))
    L = lib()
    if partition_tokens > 0:
        L.orc_decode_partitioned(B, Hq, Hkv, D, block_size, dtype, _ptr(k_pool), _ptr(v_pool),
                                 _ptr(bt), bt.shape[1], _ptr(ctx), _ptr(qq), float(scale),
                                 int(partition_tokens), _ptr(out))
    else:
        L.orc_decode(B, Hq, Hkv, D, block_size, dtype, _ptr(k_pool), _ptr(v_pool), _ptr(bt),
                     bt.shape[1], _ptr(ctx), _ptr(qq), float(scale), _ptr(out))
    return out
