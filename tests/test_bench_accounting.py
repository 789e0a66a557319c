"""Byte accounting behind bench.py's metric and roofline (no GPU).

The algorithmic bytes of one fused append + decode launch are the per-unit terms
of the decode step (every KV row read once, with the new row read from the new
K/V inputs and written to the pool; q; the fp32 output; the block-table entries
and lengths; the slots), written out here on their own; unique KV bytes count a
shared physical block once, with the most rows any sharer reads from it.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from paged_kv_cache_09_amd import workloads as W  # noqa: E402


def test_algorithmic_bytes_of_the_8b_shaped_layer():
    cfg = W.CONFIGS["llama8b_bf16"]  # 32 q / 8 kv heads, head_dim 128, bf16, blocks of 16
    ctx = np.array([128, 129, 2048, 1000], dtype=np.int32)
    B, e = len(ctx), 2
    kv = int(ctx.sum()) * 2 * 8 * 128 * e          # K and V rows, pool reads + the new rows' writes
    new_in = B * 2 * 8 * 128 * e                     # k_new, v_new
    q = B * 32 * 128 * e
    out = B * 32 * 128 * 4
    table = int(sum((L + 15) // 16 for L in ctx)) * 4
    lengths, slots = B * 4, B * 8
    assert bench.kv_bytes(cfg, ctx) == kv
    assert bench.decode_algorithmic_bytes(cfg, ctx) == kv + new_in + q + out + table + lengths + slots


def test_quantised_rows_count_codes_and_scales():
    for name, row in (("llama8b_q8", 128 + 8), ("llama8b_q4", 64 + 8)):
        cfg = W.CONFIGS[name]
        ctx = np.array([17, 300], dtype=np.int32)
        assert bench.kv_bytes(cfg, ctx) == int(ctx.sum()) * 2 * 8 * row


def test_unique_bytes_count_a_shared_block_once():
    cfg = W.CONFIGS["tiny_f32"]  # 2 kv heads, head_dim 64, fp32: 256-byte rows, blocks of 16
    row = 2 * 2 * 256
    # both sequences read block 3 in full; block 5 is shared with 4 and 9 rows used
    table = np.array([[3, 5, 7], [3, 5, -1]], dtype=np.int32)
    ctx = np.array([16 + 16 + 2, 16 + 9], dtype=np.int32)
    assert bench.unique_kv_bytes(cfg, table, ctx) == (16 + 16 + 2) * row
    assert bench.kv_bytes(cfg, ctx) == (34 + 25) * row
    # nothing shared: unique == logical
    table2 = np.array([[0, 1, 2], [3, 4, -1]], dtype=np.int32)
    assert bench.unique_kv_bytes(cfg, table2, ctx) == bench.kv_bytes(cfg, ctx)


def test_kernel_code_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// a\nint f(int x) { return x + 1; } /* b */\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", [str(src)])
    h0 = bench.kernel_source_hash()
    src.write_text("// changed words\nint f(int x)  {\n  return x + 1;   }\n/* other\n words */")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash() != h0
