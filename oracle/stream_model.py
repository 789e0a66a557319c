"""Counts-only reference for the request stream (test infrastructure).

With on-demand allocation a request holding L tokens holds exactly
ceil(L / block_size) blocks, and frees them all when it ends (thienlv.com,
"PagedAttention là gì?", "How does PagedAttention work?": a physical block is
assigned only when tokens arrive). The scheduling rules are restated here
from their description so that the library's free counts can be checked step
by step: admission FIFO while the prompt's blocks plus one fit; every running
request gains one token per step; when blocks run out the newest running
request is preempted (its blocks freed, requeued first); finished requests
free their blocks after the step.
"""
from __future__ import annotations


def run(requests, *, steps, num_blocks, block_size, max_running):
    """Returns per-step dicts {running, queued, blocks, free, tokens}."""
    def blocks(n):
        return -(-n // block_size)

    queue, running, log = [], [], []
    held = lambda: sum(blocks(r["ctx"]) for r in running)  # noqa: E731
    by_step = {}
    for rid, (t, p, o) in enumerate(requests):
        by_step.setdefault(t, []).append({"rid": rid, "prompt": p, "output": o, "ctx": 0})
    for t in range(steps):
        queue.extend(by_step.get(t, []))
        while running:
            need = sum(blocks(r["ctx"] + 1) for r in running)
            if need <= num_blocks:
                for r in running:
                    r["ctx"] += 1
                break
            victim = running.pop()
            victim["ctx"] = 0
            queue.insert(0, victim)
        running = [r for r in running if r["ctx"] < r["prompt"] + r["output"]]
        while queue and len(running) < max_running:
            r = queue[0]
            if num_blocks - held() < blocks(r["prompt"]) + 1:
                break
            r["ctx"] = r["prompt"]
            running.append(queue.pop(0))
        b = held()
        log.append({"running": len(running), "queued": len(queue), "blocks": b,
                    "free": num_blocks - b, "tokens": sum(r["ctx"] for r in running)})
    return log
