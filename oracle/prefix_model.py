"""Plain model of automatic prefix caching (test infrastructure).

What the pages fix: blocks holding a prompt prefix shared by several requests
are reused instead of duplicated (thienlv.com, "PagedAttention là gì?",
"Sharing"; ssdnodes.com, "KV cache vs prompt cache", "When local and remote
caching intersect"), and shared blocks stay held while referenced
(ahmedhaies.com, "PagedAttention: why LLM serving wastes most GPU memory",
"Trade-offs", the prefix-caching point). Readings where they are silent: a
full block is reusable by a request whose tokens agree with it from the very
first token through the block's last (its K/V depend on all of them), so the
key of block j is the token tuple tokens[0 : (j + 1) * block_size]; released
cached blocks stay reusable until a block is needed and none is free, then
the least recently released one is dropped.

Blocks are anonymous handles: physical ids are not unique.
"""
from __future__ import annotations


class _Block:
    __slots__ = ("ref", "key", "tag")

    def __init__(self):
        self.ref = 0
        self.key = None
        self.tag = None  # free for the caller (e.g. a placement of its own)


class PrefixModel:
    def __init__(self, num_blocks: int, block_size: int = 16):
        self.bs = block_size
        self.free = num_blocks      # unkeyed, unreferenced blocks
        self.cache = {}             # key -> block
        self.lru = []               # keyed blocks with no reference, oldest first
        self.evictions = 0
        self.hits = 0

    def available(self) -> int:
        return self.free + len(self.lru)

    def key(self, tokens, j):
        """Cache key of full block j of a prompt: every token from the first
        through the block's last (the block's K/V depend on all of them)."""
        return tuple(tokens[:(j + 1) * self.bs])

    def match(self, tokens):
        out = []
        j = 0
        while (j + 1) * self.bs <= len(tokens):
            b = self.cache.get(self.key(tokens, j))
            if b is None:
                break
            if b.ref == 0:
                self.lru.remove(b)
            b.ref += 1
            out.append(b)
            j += 1
        self.hits += len(out)
        return out

    def allocate(self):
        if self.free == 0 and not self.lru:
            raise MemoryError("no block")
        if self.free:
            self.free -= 1
            b = _Block()
        else:
            b = self.lru.pop(0)
            del self.cache[b.key]
            b.key = None
            self.evictions += 1
        b.ref = 1
        return b

    def insert(self, tokens, blocks):
        added = 0
        for j in range(min(len(tokens) // self.bs, len(blocks))):
            key = self.key(tokens, j)
            b = blocks[j]
            if b.key is None and key not in self.cache:
                b.key = key
                self.cache[key] = b
                added += 1
        return added

    def release(self, b):
        b.ref -= 1
        if b.ref == 0:
            if b.key is not None:
                self.lru.append(b)
            else:
                self.free += 1
