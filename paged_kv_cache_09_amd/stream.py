"""A synthetic request stream driven through the native block manager.

Requests arrive over time with a prompt and an output length; each step the
scheduler admits queued requests whose prompt fits the free blocks (a
multi-token write of the whole prompt), gives every running request one more
token (one decode step), and frees the blocks of requests that have finished.
Blocks are taken only when tokens arrive and returned when a request ends
(thienlv.com, "PagedAttention là gì?", "How does PagedAttention work?"), so
the only waste is the unfilled tail of each request's last block.

The same stream is also accounted for as a contiguous allocator would hold it:
every running request reserves max_seq_len tokens up front (same page, "Why
PagedAttention? The memory-waste problem": a fixed reservation for the maximum
length however few tokens are used). Lengths are synthetic draws: the pages
give no length distribution.

All allocation decisions are the library's (pkv_prepare_write,
pkv_prepare_append, pkv_block_free); this module only sequences the calls and
counts.
"""
from __future__ import annotations

import dataclasses
import time

import numpy as np

from . import pkv


@dataclasses.dataclass(frozen=True)
class StreamConfig:
    seed: int = 11
    steps: int = 2000
    num_blocks: int = 8192
    block_size: int = 16
    max_seq_len: int = 2048
    arrival_rate: float = 0.5     # mean new requests per step (Poisson)
    prompt_lo: int = 16
    prompt_hi: int = 1024
    output_lo: int = 16
    output_hi: int = 512
    max_running: int = 256        # concurrency cap (max number of sequences)


def draw_requests(cfg: StreamConfig):
    """Seeded arrivals: list of (arrival_step, prompt_len, output_len)."""
    rng = np.random.default_rng(cfg.seed)
    out = []
    for step in range(cfg.steps):
        for _ in range(int(rng.poisson(cfg.arrival_rate))):
            p = int(rng.integers(cfg.prompt_lo, cfg.prompt_hi + 1))
            o = int(rng.integers(cfg.output_lo, cfg.output_hi + 1))
            o = min(o, cfg.max_seq_len - p)
            out.append((step, p, max(o, 1)))
    return out


@dataclasses.dataclass
class _Req:
    rid: int
    prompt: int
    output: int
    row: np.ndarray            # int32 [max_blocks] block table row
    ctx: int = 0               # tokens in the cache
    admitted_at: int = -1


class PagedStream:
    """Runs a request stream on a host-only pool of the native block manager."""

    def __init__(self, cfg: StreamConfig):
        self.cfg = cfg
        self.max_blocks = (cfg.max_seq_len + cfg.block_size - 1) // cfg.block_size
        shape = pkv.make_shape(1, cfg.num_blocks, 1, 64, pkv.F16, cfg.max_seq_len,
                               cfg.max_running, block_size=cfg.block_size)
        self.pool = pkv.kv_pool_alloc(shape, None, 0)
        self.queue = []
        self.running = []
        self.done = 0
        self.preempted = 0
        self.log = []          # per step: dict of counts
        self.calls = 0
        self.call_s = 0.0

    def close(self):
        if self.pool is not None:
            pkv.kv_pool_free(self.pool)
            self.pool = None

    def _blocks(self, tokens: int) -> int:
        return (tokens + self.cfg.block_size - 1) // self.cfg.block_size

    def _release(self, r: _Req):
        ids = r.row[r.row >= 0]
        if ids.size:
            pkv.block_free(self.pool, ids)
        r.row[:] = -1
        r.ctx = 0

    def _timed(self, fn, *a):
        t0 = time.perf_counter()
        try:
            return fn(*a)
        finally:
            self.call_s += time.perf_counter() - t0
            self.calls += 1

    def step(self, t: int, arrivals):
        cfg = self.cfg
        for rid, p, o in arrivals:
            self.queue.append(_Req(rid, p, o, np.full(self.max_blocks, -1, np.int32)))
        # 1. one more token for every running request (batch order = admission order);
        #    when blocks run out, the newest request is preempted (its blocks
        #    freed, requeued at the head to be written again) and the step retried
        while self.running:
            table = np.ascontiguousarray(np.stack([r.row for r in self.running]))
            ctx = np.array([r.ctx + 1 for r in self.running], dtype=np.int32)
            try:
                self._timed(pkv.prepare_append, self.pool, table, ctx)
            except pkv.PkvError as e:
                if e.code != pkv.EOUT_OF_BLOCKS:
                    raise
                victim = self.running.pop()
                self._release(victim)
                self.queue.insert(0, victim)
                self.preempted += 1
                continue
            for r, row, L in zip(self.running, table, ctx):
                r.row[:] = row
                r.ctx = int(L)
            break
        # 2. finished requests return their blocks
        still = []
        for r in self.running:
            if r.ctx >= r.prompt + r.output:
                self._release(r)
                self.done += 1
            else:
                still.append(r)
        self.running = still
        # 3. admit from the queue head while the prompt fits (FIFO, no skipping)
        while self.queue and len(self.running) < cfg.max_running:
            r = self.queue[0]
            if pkv.pool_stats(self.pool)["free"] < self._blocks(r.prompt) + 1:
                break
            table = np.ascontiguousarray(r.row[None, :])
            self._timed(pkv.prepare_write, self.pool, table, [0], [r.prompt])
            r.row[:] = table[0]
            r.ctx = r.prompt
            r.admitted_at = t
            self.running.append(self.queue.pop(0))
        st = pkv.pool_stats(self.pool)
        used_tokens = sum(r.ctx for r in self.running)
        self.log.append({
            "running": len(self.running), "queued": len(self.queue),
            "blocks": st["used"], "free": st["free"], "tokens": used_tokens,
            "slots": st["used"] * cfg.block_size,
        })

    def run(self, requests):
        by_step = {}
        for rid, (t, p, o) in enumerate(requests):
            by_step.setdefault(t, []).append((rid, p, o))
        for t in range(self.cfg.steps):
            self.step(t, by_step.get(t, []))
        return self.summary()

    def summary(self) -> dict:
        cfg = self.cfg
        busy = [e for e in self.log if e["running"] > 0]
        tok = sum(e["tokens"] for e in busy)
        slots = sum(e["slots"] for e in busy)
        reserved = sum(e["running"] * cfg.max_seq_len for e in busy)
        pool_tokens = cfg.num_blocks * cfg.block_size
        return {
            "steps": cfg.steps, "finished": self.done, "preempted": self.preempted,
            "paged_waste_pct": round(100.0 * (slots - tok) / max(slots, 1), 3),
            "contiguous_waste_pct": round(100.0 * (reserved - tok) / max(reserved, 1), 3),
            "peak_running": max((e["running"] for e in self.log), default=0),
            "mean_running": round(float(np.mean([e["running"] for e in self.log])), 2),
            "contiguous_max_running": pool_tokens // cfg.max_seq_len,
            "allocator_calls": self.calls,
            "allocator_us_per_call": round(1e6 * self.call_s / max(self.calls, 1), 2),
        }
