"""Benchmark: PagedAttention decode steps on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config llama8b_bf16]

A step is one pass of the whole decode hot path over the batch: host slot
assignment (block allocation / copy-on-write), block-table upload, copy-on-
write copies, then for every layer the K/V append and the paged attention
(with its split merge). The default workload is the Llama-3.1-8B-shaped
layer stack: 32 layers, batch 64, 32 q / 8 kv heads, head_dim 128, bf16 KV,
context lengths uniform in [128, 2048], blocks scattered through a 17 GiB
pool (far larger than the last-level cache, so every layer's reads come
from HBM). Every step grows each sequence by one token, as decode does.

Prints one JSON line. `value` = KV bytes read by all layers of all timed
steps / wall time between synchronisations (GB/s). The `roofline` object is
for the per-layer decode call (decode_kernel with the append fused, and
reduce_kernel when segments are split), timed with HIP events on the launch
stream around repeats of back-to-back calls that rotate over the layers
(mean, and p10 / p50 / p90 of the repeats). The unfused kv_append and the
copy-on-write copies are also timed alone; `cpu_baseline` is the fp64 oracle
on the host cores (and on one core) for a bounded sample of the same layer.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
# the code HBM traffic depends on: the kernels and the host schedule that
# decides between the split and the bins form
KERNEL_SRCS = [os.path.join(ROOT, "paged_kv_cache_09_amd", "csrc", f)
               for f in ("pkv_kernels.hip", "pkv_host.cpp")]
TRAFFIC = os.path.join(ROOT, "profiles", "decode_traffic.json")


def kernel_source_hash() -> str:
    """SHA-256 of the kernel and schedule sources' code: comments removed and
    whitespace collapsed, so that counters stay attached to unchanged code."""
    import hashlib
    import re
    parts = []
    for path in KERNEL_SRCS:
        with open(path, encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        parts.append(" ".join(src.split()))
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()


def measured_traffic(config: str):
    """HBM bytes per layer launch (decode + reduce) from the committed counter runs,
    if they were taken on this workload with the current kernel source (else None)."""
    try:
        with open(TRAFFIC) as f:
            t = json.load(f)
        current = kernel_source_hash()
    except (OSError, ValueError):
        return None
    c = t.get("configs", {}).get(config)
    if t.get("kernel_source_sha256") != current or c is None:
        return None
    return int(c["fetch_bytes_per_launch"] + c["write_bytes_per_launch"])


def kv_bytes(cfg, ctx) -> int:
    """KV bytes one layer's decode reads: every cached row of K and V once."""
    import numpy as np
    from paged_kv_cache_09_amd import workloads as W
    return int(np.asarray(ctx, dtype=np.int64).sum()) * 2 * cfg.kv_heads * W.row_bytes(cfg)


def unique_kv_bytes(cfg, table, ctx) -> int:
    """KV bytes one layer's decode must fetch from HBM: every physical block once,
    with the most rows any sequence reads from it (a shared block is read by each
    sharer but fetched once)."""
    import numpy as np
    from paged_kv_cache_09_amd import workloads as W
    bs = cfg.block_size
    ctx = np.asarray(ctx, dtype=np.int64)
    nb = (ctx + bs - 1) // bs
    j = np.arange(table.shape[1])[None, :]
    valid = j < nb[:, None]
    rows = np.clip(ctx[:, None] - j * bs, 0, bs)
    ids = np.asarray(table)[valid].astype(np.int64)
    best = np.zeros(int(ids.max()) + 1 if ids.size else 1, dtype=np.int64)
    np.maximum.at(best, ids, rows[valid])
    return int(best.sum()) * 2 * cfg.kv_heads * W.row_bytes(cfg)


def decode_algorithmic_bytes(cfg, ctx) -> int:
    """Bytes one fused append + decode launch must move: every KV row once (the new
    row comes from k_new/v_new), the new rows written to the pool, q, the fp32
    output, the block-table entries once, the lengths and the slots."""
    import numpy as np
    from paged_kv_cache_09_amd import workloads as W
    e_in = W.TORCH_DTYPE[cfg.dtype].itemsize  # q, k_new, v_new (bf16 for q8_0)
    B = len(ctx)
    bs = cfg.block_size
    nblk = int(((np.asarray(ctx, dtype=np.int64) + bs - 1) // bs).sum())  # table entries
    # kv_bytes counts every row once, the new one included; that one is read
    # from k_new / v_new (input dtype) rather than the pool, and written to it
    new_rows = B * 2 * cfg.kv_heads * cfg.head_dim * e_in
    return (kv_bytes(cfg, ctx) + new_rows + B * cfg.q_heads * cfg.head_dim * e_in +
            B * cfg.q_heads * cfg.head_dim * 4 + nblk * 4 + B * 4 + B * 8)


def cpu_baseline(w, budget_s: float = 12.0):
    """The fp64 oracle on the host cores, on a bounded sample of the same workload (one layer)."""
    import numpy as np
    import torch

    import oracle

    cfg = w.cfg

    def storage(t):
        t = t.detach().contiguous().cpu()
        if t.dtype in (torch.float32, torch.uint8):
            return t.numpy().copy()
        return t.view(torch.int16).numpy().view(np.uint16).copy()

    cache = {}

    def run(seqs):
        key = tuple(seqs)
        if key in cache:
            kc, vc, bt, ctx, q = cache[key]
            t0 = time.perf_counter()
            oracle.decode(kc, vc, bt, ctx, q, 1.0 / math.sqrt(cfg.head_dim), dtype=cfg.dtype)
            return time.perf_counter() - t0, ctx
        used = sorted({b for s in seqs for b in w.pre_tables[s]} |
                      {int(w.new_blocks[s]) for s in seqs if w.new_blocks[s] >= 0})
        remap = {b: i for i, b in enumerate(used)}
        idx = torch.tensor(used, dtype=torch.long, device=w.pool.device)
        kl, vl = w.layer_views(0)
        kc, vc = storage(kl.index_select(0, idx)), storage(vl.index_select(0, idx))
        bt = np.full((len(seqs), w.max_blocks), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            row = [remap[b] for b in w.pre_tables[s]]
            if w.new_blocks[s] >= 0:
                row.append(remap[int(w.new_blocks[s])])
            bt[i, :len(row)] = row
        ctx = np.ascontiguousarray(w.ctx[seqs], dtype=np.int32)
        sel = torch.tensor(seqs, dtype=torch.long, device=w.pool.device)
        q = storage(w.q.index_select(0, sel))
        cache[key] = (kc, vc, bt, ctx, q)
        t0 = time.perf_counter()
        oracle.decode(kc, vc, bt, ctx, q, 1.0 / math.sqrt(cfg.head_dim), dtype=cfg.dtype)
        return time.perf_counter() - t0, ctx

    oracle.build(force=False)
    # The oracle decodes one layer of the whole batch in well under a second on
    # many cores, so the sample is that layer decoded repeatedly until about
    # budget_s of CPU work has accumulated.
    seqs = list(range(w.B))
    t, ctx = run(seqs)
    reps, total = 1, t
    while total < budget_s and reps < 10000:
        dt, _ = run(seqs)
        total += dt
        reps += 1
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    res = {"value": round(kv_bytes(cfg, ctx) * reps / total / 1e9, 4), "unit": "GB/s",
           "cores": cores, "kind": "oracle",
           "sample": f"one layer of all {w.B} sequences ({int(ctx.sum())} context tokens) "
                     f"decoded {reps} times, {total:.1f} s of oracle time",
           "seq_tokens_per_s": round(float(ctx.sum()) * reps / total, 1)}
    # the same oracle on one core, on the first 8 sequences of that layer
    oracle.set_threads(1)
    try:
        few = seqs[:8]
        t1, ctx1 = run(few)
        reps1, total1 = 1, t1
        while total1 < budget_s / 4 and reps1 < 10000:
            dt, _ = run(few)
            total1 += dt
            reps1 += 1
    finally:
        oracle.set_threads(cores)
    res["single_core"] = {
        "value": round(kv_bytes(cfg, ctx1) * reps1 / total1 / 1e9, 4), "unit": "GB/s",
        "cores": 1,
        "sample": f"one layer of {len(few)} sequences ({int(ctx1.sum())} context tokens) "
                  f"decoded {reps1} times, {total1:.1f} s"}
    return res


def log(msg: str):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama8b_bf16")
    ap.add_argument("--partition", type=int, default=None,
                    help="decode partition tokens (default: the workload's own; 0 = balanced)")
    ap.add_argument("--decode-reps", type=int, default=50,
                    help="timed repeats of the back-to-back per-layer launches (roofline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (3 times) and "
                         "exit: reference for calibrating HBM byte counters")
    ap.add_argument("--probe", choices=("stream", "gather"), default=None,
                    help="instead of the decode step, time a bandwidth probe over one layer of "
                         "--config: 'gather' reads every K/V tile the decode reads through the "
                         "block table (equal shares per wave, no compute), 'stream' a contiguous "
                         "buffer of the same bytes; both with the decode's 16-byte "
                         "nontemporal loads")
    ap.add_argument("--probe-waves", type=int, nargs="+", default=[2048, 4096],
                    help="waves of the probe launch (one JSON line each)")
    ap.add_argument("--unfused", action="store_true",
                    help="kv_append and paged_attn_decode as two launches per layer")
    ap.add_argument("--request-stream", type=int, default=0, metavar="STEPS",
                    help="instead of the decode step, run the block manager under a synthetic "
                         "request stream of STEPS scheduler steps (host only) and report "
                         "paged vs contiguous waste")
    ap.add_argument("--block-size", type=int, default=None,
                    help="tokens per pool block (8, 16 or 32; default: the workload's, 16)")
    ap.add_argument("--write-chunk", type=int, default=0, metavar="TOKENS",
                    help="instead of the decode step, time the multi-token paged write of a "
                         "prompt chunk of TOKENS tokens per sequence (prefill side)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the decode path has "
              "no multi-GPU form here (it would shard by sequence or by kv-head group, with no "
              "exchange; a sequence split across GPUs would exchange only its split partials).",
              file=sys.stderr)
        sys.exit(2)

    if args.request_stream:
        from paged_kv_cache_09_amd import stream as S
        cfg = S.StreamConfig(steps=args.request_stream)
        if args.block_size:
            cfg = S.dataclasses.replace(cfg, block_size=args.block_size,
                                        num_blocks=cfg.num_blocks * 16 // args.block_size)
        sim = S.PagedStream(cfg)
        t0 = time.perf_counter()
        summary = sim.run(S.draw_requests(cfg))
        wall = time.perf_counter() - t0
        sim.close()
        print(json.dumps({"metric": "KV waste under a request stream (host block manager)",
                          "value": summary["paged_waste_pct"], "unit": "% of allocated slots",
                          "higher_is_better": False, "data": "synthetic",
                          "config": {"workload": f"Poisson arrivals {cfg.arrival_rate}/step, "
                                                 f"prompt U[{cfg.prompt_lo},{cfg.prompt_hi}], "
                                                 f"output U[{cfg.output_lo},{cfg.output_hi}], "
                                                 f"{cfg.num_blocks} blocks of {cfg.block_size}, "
                                                 f"max_seq_len {cfg.max_seq_len}"},
                          "wall_s": round(wall, 3), **summary}), flush=True)
        return

    import numpy as np
    import torch

    if args.copy_probe:
        src = torch.empty(args.copy_probe, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe}), flush=True)
        return

    from paged_kv_cache_09_amd import workloads as W
    from paged_kv_cache_09_amd.session import DecodeSession

    if args.write_chunk:
        return main_write(args)
    if args.probe:
        return main_probe(args)
    cfg = W.CONFIGS[args.config]
    if args.block_size:
        # same token capacity in blocks of another size
        cfg = W.scaled(cfg, block_size=args.block_size,
                       num_blocks=cfg.num_blocks * cfg.block_size // args.block_size)
    part = cfg.partition_tokens if args.partition is None else args.partition
    growth = args.warmup + args.steps + 1
    # spare blocks so every sequence can grow by `growth` tokens
    bs = cfg.block_size
    cfg = W.scaled(cfg, num_blocks=cfg.num_blocks + cfg.batch * ((growth + bs - 1) // bs + 1))
    log(f"building {cfg.name}: {cfg.layers} layers")
    w = W.make(cfg, device="cuda", layers=cfg.layers, form="step", fill="random",
               extra_blocks=(growth + bs - 1) // bs + 1)
    sess = DecodeSession(w)
    log("pool ready; warm-up")
    out = sess.new_out()
    stream = torch.cuda.current_stream()
    layers = list(range(cfg.layers))

    cow_pairs = None  # the first copy-on-write pairs a step made (timed alone at the end)

    def one_step():
        nonlocal cow_pairs
        sess.step(out, layers=layers, partition_tokens=part, fused=not args.unfused)
        if cow_pairs is None and len(sess.pairs):
            cow_pairs = sess.pairs.copy()

    total_kv = 0
    total_unique = 0
    for _ in range(args.warmup):
        one_step()
        sess.ctx += 1
    torch.cuda.synchronize()
    log("timed steps")

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # each step's lengths and table, for the byte counts taken after the timed region
    snaps = []
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        one_step()
        snaps.append((sess.ctx.copy(), sess.table.copy()))
        sess.ctx += 1
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    elapsed = max(wall, ev_ms / 1e3)
    for ctx_s, table_s in snaps:
        total_kv += kv_bytes(cfg, ctx_s) * cfg.layers
        total_unique += unique_kv_bytes(cfg, table_s, ctx_s) * cfg.layers

    log("decode-only launches")
    # the per-layer kernel alone: back-to-back launches over all layers, same upload
    sess.ctx -= 1  # the uploaded table matches the last step's lengths
    ctx_now = sess.ctx.copy()
    reps = args.decode_reps
    def layer_call(layer):
        if args.unfused:
            sess.decode(layer, out, part)
        else:
            sess.append_decode(layer, out, part)

    for layer in layers[:4]:
        layer_call(layer)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    evs[0].record(stream)
    t_issue = time.perf_counter()
    for r in range(reps):
        for layer in layers:  # re-appending the same rows is idempotent
            layer_call(layer)
        evs[r + 1].record(stream)
    # host time to issue one call: while it stays below the launch time the
    # GPU never waits for the host and the events time the kernels alone
    issue_s = (time.perf_counter() - t_issue) / (reps * len(layers))
    torch.cuda.synchronize()
    per_rep = np.array([evs[r].elapsed_time(evs[r + 1]) / 1e3 / len(layers)
                        for r in range(reps)])
    per_launch_s = float(per_rep.mean())
    p10, p50, p90 = (float(x) for x in np.percentile(per_rep, [10, 50, 90]))
    # algorithmic bytes with the KV counted as fetched (shared blocks once); the
    # logical figure (every sharer's rows) is reported beside it
    alg_logical = decode_algorithmic_bytes(cfg, ctx_now)
    alg = alg_logical - kv_bytes(cfg, ctx_now) + unique_kv_bytes(cfg, sess.table, ctx_now)
    achieved = alg / per_launch_s / 1e9

    log("kv_append alone")
    # the unfused append (kv_append through the uploaded slots), one launch per layer
    a_reps = 20
    for layer in layers[:4]:
        sess.append(layer)
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(a_reps):
        for layer in layers:
            sess.append(layer)
    a1.record(stream)
    torch.cuda.synchronize()
    append_s = a0.elapsed_time(a1) / 1e3 / (a_reps * len(layers))

    res = {
        "metric": "paged decode KV-read GB/s (% of HBM peak) + seq-tokens/s, 8B-shaped layer",
        "value": round(total_kv / elapsed / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W.DTYPE_NAME[cfg.dtype],
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.layers} layers x batch {cfg.batch}, "
                        f"{cfg.q_heads} q / {cfg.kv_heads} kv heads, head_dim {cfg.head_dim}, "
                        f"block {cfg.block_size}, context {int(w.ctx.min())}..{int(w.ctx.max())} "
                        "growing 1/step",
            "layers": cfg.layers, "batch": cfg.batch, "q_heads": cfg.q_heads,
            "kv_heads": cfg.kv_heads, "head_dim": cfg.head_dim, "block_size": cfg.block_size,
            "partition_tokens": part, "pool_gib": round(w.pool.numel() / 2**30, 2),
        },
        "pct_of_hbm_peak": round(100 * total_unique / elapsed / 1e9 / HBM_PEAK_GBS, 2),
        "seq_tokens_per_s": round(float(sum(int(c) for c in ctx_now)) * cfg.layers *
                                  args.steps / elapsed, 1),
        "decode_tokens_per_s": round(cfg.batch * args.steps / elapsed, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(cfg.name),
            "kernel": "per-layer call: decode_kernel (fused append + paged attention) and, for "
                      "split segments, reduce_kernel; timed together",
            "avg_launch_us": round(per_launch_s * 1e6, 3),
            "host_issue_us_per_call": round(issue_s * 1e6, 3),
            "launch_us_p10_p50_p90": [round(p10 * 1e6, 3), round(p50 * 1e6, 3),
                                      round(p90 * 1e6, 3)],
            "timed_launches": reps * len(layers),
            "algorithmic_bytes_per_launch": alg,
            "logical_bytes_per_launch": alg_logical,
        },
        "kv_append_alone_us_per_layer": round(append_s * 1e6, 3),
    }
    if w.shared:  # shared blocks are read by every sharer but fetched from HBM once
        res["unique_kv_GBps"] = round(total_unique / elapsed / 1e9, 2)
    if not args.no_cpu_baseline:
        log("cpu baseline")
        res["cpu_baseline"] = cpu_baseline(w)
        res["gpu_over_cpu"] = round(res["value"] / res["cpu_baseline"]["value"], 1)
    if cow_pairs is not None:
        # copy-on-write copies alone, with the pairs of the step that made them; run last,
        # since copying them again overwrites rows appended since (timing only)
        log("copy_blocks alone")
        from paged_kv_cache_09_amd import pkv
        c_reps = 20
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(c_reps):
            pkv.copy_blocks(sess.pool, cow_pairs, sess.stream)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_s = c0.elapsed_time(c1) / 1e3 / c_reps
        copy_bytes = 2 * len(cow_pairs) * cfg.layers * 2 * W.tile_bytes(cfg) * cfg.kv_heads
        res["copy_blocks_alone"] = {"pairs": int(len(cow_pairs)), "us": round(copy_s * 1e6, 3),
                                    "GBps": round(copy_bytes / copy_s / 1e9, 2)}
    sess.close()
    print(json.dumps(res), flush=True)


def main_probe(args):
    """Bandwidth probes over one layer of a workload (measurements bounding the
    decode from above; see pkv_probe_* in include/pkv.h)."""
    import numpy as np
    import torch
    from paged_kv_cache_09_amd import pkv, workloads as W
    from paged_kv_cache_09_amd.session import DecodeSession
    cfg = W.CONFIGS[args.config]
    w = W.make(cfg, device="cuda", layers=1, form="step", fill="random", extra_blocks=1)
    sess = DecodeSession(w)
    sess.prepare()
    sess.upload()
    torch.cuda.synchronize()
    tile = W.row_bytes(cfg) * 16
    tiles = int(((np.asarray(sess.ctx, dtype=np.int64) + 15) // 16).sum()) * cfg.kv_heads
    nbytes = 2 * tiles * tile  # K and V tiles of one layer
    stream = torch.cuda.current_stream()
    buf = None
    if args.probe == "stream":
        buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        buf.fill_(3)
    reps = max(5, args.decode_reps)
    for waves in args.probe_waves:
        out = torch.empty(waves * 64, dtype=torch.int32, device="cuda")

        def launch():
            if args.probe == "stream":
                pkv.probe_stream_read(buf, nbytes, out, waves, stream.cuda_stream)
            else:
                pkv.probe_gather(sess.pool, 0, out, waves, stream.cuda_stream)

        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        evs[0].record(stream)
        for r in range(reps):
            launch()
            evs[r + 1].record(stream)
        torch.cuda.synchronize()
        per = np.array([evs[r].elapsed_time(evs[r + 1]) / 1e3 for r in range(reps)])
        gbs = nbytes / per.mean() / 1e9
        print(json.dumps({
            "metric": f"probe: {args.probe} read GB/s", "value": round(gbs, 2), "unit": "GB/s",
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "avg_launch_us": round(per.mean() * 1e6, 3),
            "launch_us_p10_p50_p90": [round(float(x) * 1e6, 3) for x in np.percentile(per, [10, 50, 90])],
            "bytes_per_launch": nbytes, "waves": waves, "launches": reps,
            "config": {"workload": f"{cfg.name}: one layer's K and V tiles "
                                   f"({tiles} tiles of {tile} bytes each)"}}), flush=True)
    sess.close()


def main_write(args):
    """Multi-token paged write (a prompt chunk per sequence, every layer): one
    kv_append launch per layer scatters all the chunk's rows through per-token
    slots. Bytes moved = rows read from the inputs + rows written to the pool."""
    import numpy as np
    import torch

    from paged_kv_cache_09_amd import workloads as W
    from paged_kv_cache_09_amd.session import DecodeSession

    cfg = W.CONFIGS[args.config]
    chunk = args.write_chunk
    cfg = W.scaled(cfg, num_blocks=cfg.num_blocks + cfg.batch * ((chunk + 15) // 16 + 1))
    log(f"building {cfg.name}: {cfg.layers} layers, write chunk {chunk}")
    w = W.make(cfg, device="cuda", layers=cfg.layers, form="step", fill="random",
               extra_blocks=(chunk + 15) // 16 + 1)
    before_ctx, _, k_rows, v_rows = W.write_rows(w, chunk, chunk)
    n_new = np.full(w.B, chunk, dtype=np.int32)
    sess = DecodeSession(w)
    slots, pairs = sess.prepare_write(before_ctx, n_new)
    t_host = sess.last_prepare_s
    sess.copy_blocks()
    rows = int(n_new.sum())
    in_bytes = rows * 2 * cfg.kv_heads * cfg.head_dim * W.TORCH_DTYPE[cfg.dtype].itemsize
    out_bytes = rows * 2 * cfg.kv_heads * W.row_bytes(cfg)
    layers = list(range(cfg.layers))
    stream = torch.cuda.current_stream()
    for _ in range(max(1, args.warmup)):
        for layer in layers:
            sess.write(layer, k_rows, v_rows)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        for layer in layers:  # rewriting the same rows is idempotent
            sess.write(layer, k_rows, v_rows)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = e0.elapsed_time(e1) / 1e3 / (args.steps * len(layers))
    achieved = (in_bytes + out_bytes) / per_launch / 1e9
    res = {
        "metric": "paged KV multi-token write GB/s (prefill chunk)",
        "value": round((in_bytes + out_bytes) * len(layers) * args.steps / wall / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": W.DTYPE_NAME[cfg.dtype],
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.layers} layers x batch {cfg.batch}, "
                               f"{chunk} new tokens per sequence behind "
                               f"{int(before_ctx.min())}..{int(before_ctx.max())} cached",
                   "rows_per_layer": rows, "block_size": 16},
        "host_prepare_write_ms": round(t_host * 1e3, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "append kernel, one launch per layer",
                     "avg_launch_us": round(per_launch * 1e6, 3),
                     "algorithmic_bytes_per_launch": in_bytes + out_bytes},
    }
    sess.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
