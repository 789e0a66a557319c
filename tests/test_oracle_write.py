"""Pins of the oracle's multi-token write (no GPU): after writing n_new[s]
tokens behind ctx_before[s] cached ones, every sequence reads back its old
rows followed by exactly the given new rows (q8_0: their quantisation), and
nothing outside the written rows and copied blocks changes
(news.hamidun.com "KV-Cache", prefill/decode paragraph: a prompt's K/V rows
are all written to the cache)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import step as ostep
from paged_kv_cache_09_amd import workloads as W
from tests.helpers import to_storage


@pytest.mark.parametrize("name,changes,n_lo,n_hi", [
    ("tiny_f32", dict(num_blocks=64), 1, 30),
    ("shared_prefix_cow_bf16", dict(batch=6, num_blocks=64 + 6 * 20, layers=2), 1, 200),
    ("mha13b_f16", dict(batch=5, q_heads=4, kv_heads=4, num_blocks=5 * 150), 0, 100),
    ("llama8b_q8", dict(batch=4, num_blocks=4 * 180, layers=2), 1, 700),
    ("llama8b_q4", dict(batch=4, num_blocks=4 * 180, layers=2), 1, 700),
])
def test_write_reads_back_old_rows_then_new_rows(name, changes, n_lo, n_hi):
    cfg = W.scaled(W.CONFIGS[name], **changes)
    w = W.make(cfg, device="cpu", layers=cfg.layers, form="step", fill="nan", extra_blocks=50)
    before_ctx, n_new, k_rows, v_rows = W.write_rows(w, n_lo, n_hi)
    ks, vs = [], []
    for layer in range(w.layers):
        kl, vl = w.layer_views(layer)
        ks.append(to_storage(kl))
        vs.append(to_storage(vl))
    old = [ostep.logical_rows(ks[l], vs[l], w.table("pre"), before_ctx) for l in range(w.layers)]
    k0 = [k.copy() for k in ks]
    kr, vr = to_storage(k_rows), to_storage(v_rows)
    table, plan = ostep.run_write(ks, vs, w.pre_tables, w.shared, before_ctx, n_new,
                                  [kr] * w.layers, [vr] * w.layers, dtype=cfg.dtype,
                                  num_blocks=cfg.num_blocks, max_blocks=w.max_blocks)
    after_ctx = before_ctx + n_new
    offs = np.concatenate([[0], np.cumsum(n_new)])
    for layer in range(w.layers):
        new = ostep.logical_rows(ks[layer], vs[layer], table, after_ctx)
        for s in range(w.B):
            L0 = int(before_ctx[s])
            for which, rows in ((0, kr), (1, vr)):
                got = new[s][which]
                assert np.array_equal(got[:L0], old[layer][s][which])
                want = rows[offs[s]:offs[s + 1]]
                if cfg.dtype in W.QUANTISED:
                    x = (want.astype(np.uint32) << 16).view(np.float32)
                    n = want.shape[0]
                    if cfg.dtype == W.Q8_0:
                        codes, d = oracle.q8_quantize(x.reshape(-1, 32))
                        cb = codes.reshape(n, cfg.kv_heads, cfg.head_dim).view(np.uint8)
                    else:  # q4_0: element i in byte i // 2, low nibble for even i
                        codes, d = oracle.q4_quantize(x.reshape(-1, 32))
                        c = codes.reshape(n, cfg.kv_heads, cfg.head_dim)
                        cb = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
                    want = np.concatenate([cb, d.reshape(n, cfg.kv_heads, -1).view(np.uint8)],
                                          axis=2)
                assert np.array_equal(got[L0:], want)
    # blocks that nobody's table names after the write are untouched
    named = {int(b) for b in table.ravel() if b >= 0} | {int(b) for r in w.pre_tables for b in r}
    for b in range(cfg.num_blocks):
        if b not in named:
            assert np.array_equal(ks[0][b], k0[0][b], equal_nan=cfg.dtype not in W.QUANTISED)
