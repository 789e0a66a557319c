"""One decode step on host copies of the pool, in the oracle's own terms (test infrastructure).

The block bookkeeping follows :mod:`oracle.block_model` (on-demand blocks,
refcounted sharing, copy-on-write); the byte writes follow ``orc_append``.
The oracle picks its own fresh block ids (any id free before the step), so
its physical placement generally differs from the library's; what must agree
is the logical content of every sequence and the attention output, neither
of which depends on placement.
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle.block_model import BlockModel

BLOCK = 16


def run_step(k_layers, v_layers, pre_tables, shared, ctx, k_new_layers, v_new_layers, *,
             dtype, num_blocks, max_blocks, block_size=BLOCK):
    """Apply one decode step to host pools.

    k_layers / v_layers: lists (one per layer) of storage arrays [NB][Hkv][16][D]
    ([NB][Hkv][tile bytes] for q8_0), updated in place. k_new_layers /
    v_new_layers: per-layer [B][Hkv][D] rows.
    Returns (post_table int32 [B][max_blocks], kinds).
    """
    model = BlockModel(num_blocks)
    used = sorted({b for row in pre_tables for b in row})
    model.claim(used)
    for b, rc in shared:
        model.ref([b] * (rc - 1))
    kinds = model.plan_append(pre_tables, ctx, block_size)
    free_ids = iter(sorted(set(range(num_blocks)) - set(used)))
    B = len(pre_tables)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    for s, row in enumerate(pre_tables):
        table[s, :len(row)] = row
    for s, kind in enumerate(kinds):
        j = (int(ctx[s]) - 1) // block_size
        if kind == "new":
            table[s, j] = next(free_ids)
        elif kind == "cow":
            src = int(table[s, j])
            dst = next(free_ids)
            for kl, vl in zip(k_layers, v_layers):
                kl[dst] = kl[src]
                vl[dst] = vl[src]
            table[s, j] = dst
    for kl, vl, kn, vn in zip(k_layers, v_layers, k_new_layers, v_new_layers):
        oracle.append(kl, vl, table, ctx, kn, vn, dtype=dtype, block_size=block_size)
    return table, kinds


def run_write(k_layers, v_layers, pre_tables, shared, ctx_before, n_new, k_rows_layers,
              v_rows_layers, *, dtype, num_blocks, max_blocks, block_size=BLOCK):
    """Write n_new[s] tokens per sequence after ctx_before[s] cached ones into host
    pools (every layer), the oracle's own block placement.

    k_rows_layers / v_rows_layers: per-layer rows [sum n_new][Hkv][D], sequence by
    sequence in position order. Returns (post_table int32 [B][max_blocks], plan).
    """
    model = BlockModel(num_blocks)
    used = sorted({b for row in pre_tables for b in row})
    model.claim(used)
    for b, rc in shared:
        model.ref([b] * (rc - 1))
    plan = model.plan_write(pre_tables, ctx_before, n_new, block_size)
    free_ids = iter(sorted(set(range(num_blocks)) - set(used)))
    B = len(pre_tables)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    for s, row in enumerate(pre_tables):
        table[s, :len(row)] = row
    for s, j, kind in plan:
        if kind == "new":
            table[s, j] = next(free_ids)
        elif kind == "cow":
            src = int(table[s, j])
            dst = next(free_ids)
            for kl, vl in zip(k_layers, v_layers):
                kl[dst] = kl[src]
                vl[dst] = vl[src]
            table[s, j] = dst
    # token t of every sequence that has one, written as a one-token append
    offsets = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int64)
    for t in range(int(max(n_new)) if len(n_new) else 0):
        has = np.array([t < n for n in n_new])
        ctx = np.where(has, np.asarray(ctx_before) + t + 1, 0).astype(np.int32)
        rows = np.where(has, offsets[:-1] + t, 0)
        for kl, vl, kr, vr in zip(k_layers, v_layers, k_rows_layers, v_rows_layers):
            oracle.append(kl, vl, table, ctx, np.ascontiguousarray(kr[rows]),
                          np.ascontiguousarray(vr[rows]), dtype=dtype, block_size=block_size)
    return table, plan


def q_format(tile_bytes, block_size=BLOCK):
    """(code bytes per row, head_dim) of a quantised tile: rows of head_dim codes
    (q8_0, 17 * head_dim / 16 bytes with the scales) or head_dim / 2 bytes of
    nibbles (q4_0, 9 * head_dim / 16 bytes); the two never have equal sizes."""
    per_row16 = tile_bytes * 16 // block_size
    if per_row16 % 17 == 0:
        D = per_row16 // 17
        return D, D
    assert per_row16 % 9 == 0, "not a quantised tile size"
    D = per_row16 // 9
    return D // 2, D


def q4_code_index(rows, is_v, head_dim):
    """Tile byte offsets of each row's q4_0 code bytes in element order
    ([n][head_dim/2]): word w (4 bytes, elements 8w .. 8w+7) of row r lies at
    r*CB + 4*((w % 4)*G + w // 4) in the K region and at
    (r - r % G)*CB + 4*(w*G + r % G) in the V region (G = head_dim/32,
    CB = head_dim/2), as orc_append writes them."""
    G, CB = head_dim // 32, head_dim // 2
    r = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(CB)[None, :]
    w, b = j // 4, j % 4
    if is_v:
        return (r - r % G) * CB + 4 * (w * G + r % G) + b
    return r * CB + 4 * ((w % 4) * G + w // 4) + b


def q8_code_index(rows, is_v, head_dim, block_size=BLOCK):
    """Tile byte offsets of each row's q8_0 codes in element order
    ([n][head_dim]), as orc_append writes them: rows R = min(block_size, 16) at
    a time (u = r // R, rr = r % R), element d = 8w + j in chunk w (P = D/8
    chunks per row, NV = P/4); K: w = 4k + q at
    u*R*D + (k//2)*R*64 + (q*R + rr)*16 + (k%2)*8 + j; V: at
    u*R*D + ((rr%NV)//2)*R*64 + ((rr//NV)*P + w)*16 + (rr%2)*8 + j."""
    D = head_dim
    P, R = D // 8, min(block_size, 16)
    NV = P // 4
    r = np.asarray(rows, dtype=np.int64)[:, None]
    u, rr = r // R, r % R
    d = np.arange(D)[None, :]
    w, j = d // 8, d % 8
    if is_v:
        return u * R * D + ((rr % NV) // 2) * R * 64 + ((rr // NV) * P + w) * 16 + (rr % 2) * 8 + j
    k, q = w // 4, w % 4
    return u * R * D + (k // 2) * R * 64 + (q * R + rr) * 16 + (k % 2) * 8 + j


def q8_row_bytes(pool, blocks, rows, is_v, block_size=BLOCK):
    """Bytes of quantised rows (q8_0 or q4_0) as [n][Hkv][code bytes + 2 * D/32 scale
    bytes]: codes in element order, scales in group order. A tile is block_size rows
    of codes (q8_0 codes placed as q8_code_index says, q4_0 words as
    q4_code_index says), then fp16 scales ordered
    [row][group] (K region) or [group][row] (V region)."""
    cb, D = q_format(pool.shape[2], block_size)
    ng = D // 32
    rows = np.asarray(rows, dtype=np.int64)
    blocks = np.asarray(blocks, dtype=np.int64)
    if cb == D:
        code_idx = q8_code_index(rows, is_v, D, block_size)
    else:
        code_idx = q4_code_index(rows, is_v, D)
    grp = np.arange(ng)[None, :]
    si = grp * block_size + rows[:, None] if is_v else rows[:, None] * ng + grp
    sb = block_size * cb + 2 * si
    scale_idx = np.stack([sb, sb + 1], axis=2).reshape(len(rows), 2 * ng)
    idx = np.concatenate([code_idx, scale_idx], axis=1)
    return np.take_along_axis(pool[blocks], idx[:, None, :], axis=2)


def logical_rows(k_pool, v_pool, table, ctx, block_size=BLOCK):
    """Raw bytes of every sequence's K and V rows in logical order: list of (K, V)
    arrays [L][Hkv][D] (q8_0 pools [NB][Hkv][tile bytes]: codes then scale bytes)."""
    out = []
    for s, L in enumerate(ctx):
        t = np.arange(int(L))
        blocks = table[s][t // block_size]
        rows = t % block_size
        if k_pool.ndim == 3:
            out.append((q8_row_bytes(k_pool, blocks, rows, False, block_size),
                        q8_row_bytes(v_pool, blocks, rows, True, block_size)))
        else:
            out.append((k_pool[blocks, :, rows, :], v_pool[blocks, :, rows, :]))
    return out
