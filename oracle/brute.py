"""Pure-Python brute force of paged decode attention, for tiny inputs only.

Test infrastructure. Plain nested loops over Python floats (double precision),
no numpy arithmetic, so that it shares nothing with ``oracle.c`` beyond the
definition it follows:

* the cache of each sequence is split into blocks of ``block_size`` tokens,
  reached through a per-sequence block table (ahmedhaies.com, "PagedAttention:
  why LLM serving wastes most GPU memory", section "The solution: borrow
  virtual memory from the OS");
* the new query attends to every cached key/value of its sequence
  (news.hamidun.com glossary "KV-Cache", mechanism paragraph);
* query head h reads the kv head shared by its group of q_heads/kv_heads heads
  (ssdnodes.com, "KV cache vs prompt cache", GQA paragraph).

Inputs are Python lists of floats already decoded from their storage type:
``k_pool[block][head][row][d]``, ``v_pool`` alike, ``q[s][h][d]``.
"""
import math


def decode(k_pool, v_pool, block_table, ctx_lens, q, scale, block_size=16):
    out = []
    for s, L in enumerate(ctx_lens):
        heads_out = []
        q_heads = len(q[s])
        kv_heads = len(k_pool[0])
        group = q_heads // kv_heads
        for h in range(q_heads):
            g = h // group
            logits = []
            for t in range(L):
                blk = block_table[s][t // block_size]
                row = t % block_size
                dot = 0.0
                for d in range(len(q[s][h])):
                    dot += q[s][h][d] * k_pool[blk][g][row][d]
                logits.append(scale * dot)
            top = max(logits)
            weights = [math.exp(z - top) for z in logits]
            total = sum(weights)
            vec = [0.0] * len(q[s][h])
            for t in range(L):
                blk = block_table[s][t // block_size]
                row = t % block_size
                for d in range(len(vec)):
                    vec[d] += weights[t] / total * v_pool[blk][g][row][d]
            heads_out.append(vec)
        out.append(heads_out)
    return out
