"""Per-wave timeline of one decode launch (diagnostics).

Needs the timeline build of the library, whose decode kernel records per
wave its start, the arrival of its descriptor, first tile, end of its runs
and end of its merges
(s_memrealtime, 100 MHz), its XCD, tiles and segments:

    python -m paged_kv_cache_09_amd.build --timeline
    PKV_LIB=libpkv_timeline.so python -m paged_kv_cache_09_amd.timeline --config llama8b_bf16

It runs a few decode steps of the workload, then the per-layer launches
back to back, and summarises the last launch (times in us from the first
wave's start): when waves start and get their first tile, when their runs
end (by XCD and by wave slot of the bin), how the bins' end times relate to
their tile counts, and how long the LDS merges after the barrier take.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os

os.environ.setdefault("PKV_LIB", "libpkv_timeline.so")

import numpy as np  # noqa: E402
import torch  # noqa: E402

from . import pkv, workloads as W  # noqa: E402
from .session import DecodeSession  # noqa: E402

ENTRIES = 8192  # waves the kernel records (8 int64 each)


def read(nwaves_per_bin: int = 8) -> dict:
    fn = getattr(pkv._lib, "pkv_debug_timeline", None)
    if fn is None:
        raise RuntimeError(f"{pkv.LIB_PATH} has no timeline: build it with --timeline")
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    buf = np.zeros(8 * ENTRIES, dtype=np.int64)
    if fn(buf.ctypes.data, buf.nbytes) != 0:
        raise RuntimeError(pkv.last_error())
    r = buf.reshape(-1, 8)
    return r[r[:, 0] != 0]


def summarise(r: np.ndarray, nw: int = 8) -> dict:
    t0 = r[:, 0].min()
    us = lambda col: (r[:, col] - t0) / 100.0  # noqa: E731
    start, first, end, merged, barrier = us(0), (r[:, 1] - r[:, 0]) / 100.0, us(2), us(3), us(6)
    desc = (r[:, 7] - r[:, 0]) / 100.0
    xcd = r[:, 4] & 0xF
    tiles = (r[:, 4] >> 8) & 0xFFFF
    segs = (r[:, 4] >> 24) & 0xFF
    wave = r[:, 5]
    q = lambda v, p: round(float(np.percentile(v, p)), 2)  # noqa: E731
    busy = (r[:, 2] - r[:, 0]) / 100.0
    out = {
        "waves": int(len(r)),
        "start_us": {"p50": q(start, 50), "max": q(start, 100)},
        "descriptor_after_start_us": {"p10": q(desc, 10), "p50": q(desc, 50), "p90": q(desc, 90)},
        "first_tile_after_start_us": {"p10": q(first, 10), "p50": q(first, 50), "p90": q(first, 90)},
        "runs_end_us": {"min": q(end, 0), "p10": q(end, 10), "p50": q(end, 50), "p90": q(end, 90),
                        "max": q(end, 100)},
        "merges_end_max_us": q(merged, 100),
        "us_per_tile_by_xcd": [round(float(busy[xcd == x].sum() / max(1, tiles[xcd == x].sum())), 3)
                               for x in range(8) if (xcd == x).any()],
        "runs_end_p50_by_wave_slot_us": [q(end[wave % nw == v], 50) for v in range(nw)],
        "tiles_per_wave": {"p50": q(tiles, 50), "max": int(tiles.max())},
        "segments_per_wave_max": int(segs.max()),
    }
    # bins: the nw waves of a workgroup
    b = wave // nw
    nb = int(b.max()) + 1
    btiles = np.bincount(b, weights=tiles, minlength=nb)
    bend = np.array([end[b == i].max() if (b == i).any() else 0.0 for i in range(nb)])
    bbar = np.array([barrier[b == i].max() if (b == i).any() else 0.0 for i in range(nb)])
    bmerge = np.array([merged[b == i].max() if (b == i).any() else 0.0 for i in range(nb)])
    if nb > 1 and btiles.std() > 0:
        out["bins"] = {
            "count": nb,
            "tiles_max_over_mean": round(float(btiles.max() / btiles.mean()), 3),
            "corr_end_tiles": round(float(np.corrcoef(bend, btiles)[0, 1]), 2),
            "heaviest_ends_us": [round(float(bend[i]), 2) for i in np.argsort(-btiles)[:8]],
            "latest_ends_us": [round(float(bend[i]), 2) for i in np.argsort(-bend)[:8]],
            "merge_after_barrier_us": {"p50": q(bmerge - bbar, 50), "max": q(bmerge - bbar, 100)},
        }
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="llama8b_bf16")
    ap.add_argument("--steps", type=int, default=3, help="decode steps before the timed launches")
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    cfg = W.CONFIGS[args.config]
    bs = cfg.block_size
    extra = (args.steps + bs - 1) // bs + 1
    cfg = W.scaled(cfg, num_blocks=cfg.num_blocks + cfg.batch * extra)
    w = W.make(cfg, device="cuda", layers=cfg.layers, form="step", fill="random",
               extra_blocks=extra)
    sess = DecodeSession(w)
    out = sess.new_out()
    for _ in range(args.steps):
        sess.step(out, layers=list(range(cfg.layers)))
        sess.ctx += 1
    sess.ctx -= 1
    torch.cuda.synchronize()
    for rep in range(args.reps):
        for layer in range(cfg.layers):
            sess.append_decode(layer, out, 0)
        torch.cuda.synchronize()
        s = summarise(read())
        s["config"] = cfg.name
        s["rep"] = rep
        print(json.dumps(s), flush=True)
    sess.close()


if __name__ == "__main__":
    main()
