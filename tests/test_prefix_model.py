"""Pins of the plain prefix-cache model (oracle/prefix_model.py) on its own.

The behaviour comes from the pages: a prompt prefix's blocks are reused by
later requests instead of being stored twice, and shared blocks are held by
reference counts (thienlv.com, "PagedAttention là gì?", "Sharing";
ahmedhaies.com, "PagedAttention: why LLM serving wastes most GPU memory",
"Trade-offs", the prefix-caching point). Where the pages are silent the
model reads: a block's key is the whole token prefix through its last token,
only full blocks are keyed, released cached blocks stay reusable, and the
least recently released one is evicted first when no block is free. Every
expected value below is worked out by hand from those readings; three
planted mistakes (a block-local key, most-recent-first eviction, released
blocks returned to the free list) each fail at least one pin.
"""
import pytest

from oracle.prefix_model import PrefixModel


def _serve(model, tokens):
    """Match, allocate the rest, register; returns the request's blocks."""
    blocks = model.match(tokens)
    need = -(-len(tokens) // model.bs) - len(blocks)
    blocks += [model.allocate() for _ in range(need)]
    model.insert(tokens, blocks)
    return blocks


def pin_same_first_blocks_match(cls):
    m = cls(8, block_size=4)
    a = list(range(10, 22))            # 3 full blocks
    blocks_a = _serve(m, a)
    got = m.match(a[:8] + [99, 98, 97, 96, 95])  # first 2 blocks shared
    assert len(got) == 2 and got[0] is blocks_a[0] and got[1] is blocks_a[1]
    assert m.hits == 2
    assert blocks_a[0].ref == 2 and blocks_a[2].ref == 1


def pin_first_token_differs_matches_nothing(cls):
    m = cls(8, block_size=4)
    a = list(range(10, 22))
    _serve(m, a)
    b = [7] + a[1:]                    # blocks 1 and 2 hold the same tokens as a's
    assert m.match(b) == []
    assert m.hits == 0


def pin_later_block_needs_the_whole_prefix(cls):
    m = cls(8, block_size=4)
    x, y, z, w = [1, 2, 3, 4], [5, 6, 7, 8], [9, 10, 11, 12], [13, 14, 15, 16]
    _serve(m, x + y)
    _serve(m, z + w)
    # block 0 of x + w is cached (x), block 1 holds w's tokens but after a
    # different prefix: its K/V differ from the cached w block
    assert len(m.match(x + w)) == 1
    assert m.hits == 1


def pin_only_full_blocks_are_keyed(cls):
    m = cls(8, block_size=4)
    a = list(range(10, 20))            # 2 full blocks + 2 tokens
    blocks = m.match(a) + [m.allocate() for _ in range(3)]
    assert m.insert(a, blocks) == 2
    assert len(m.cache) == 2
    assert len(m.match(a[:7])) == 1    # 7 tokens hold one full block
    assert len(m.match(a)) == 2        # the partial third block is not cached


def pin_released_blocks_stay_evictable(cls):
    m = cls(4, block_size=2)
    blocks = _serve(m, [1, 2, 3, 4, 5])  # 2 full blocks cached + 1 partial
    assert m.available() == 1
    for b in blocks:
        m.release(b)
    assert m.free == 2                  # the uncached partial block is free again
    assert len(m.lru) == 2              # the cached ones stay reusable
    assert m.available() == 4
    got = m.match([1, 2, 3, 4, 9])
    assert len(got) == 2 and len(m.lru) == 0


def pin_least_recently_released_is_evicted(cls):
    m = cls(3, block_size=2)
    for t in ([1, 2], [3, 4], [5, 6]):  # each request: one full block, released
        for b in _serve(m, t):
            m.release(b)
    assert m.free == 0 and len(m.lru) == 3 and m.evictions == 0
    for b in _serve(m, [7, 8]):        # needs a block: [1, 2] was released first
        m.release(b)
    assert m.evictions == 1
    assert m.match([1, 2]) == []
    held = m.match([3, 4])             # a hit takes [3, 4] out of the evictable set
    assert len(held) == 1 and m.hits == 1
    _serve(m, [9, 10])                 # evicts [5, 6], the oldest still evictable
    assert m.evictions == 2
    assert m.match([5, 6]) == []
    assert len(m.match([7, 8])) == 1 and m.hits == 2


PINS = [pin_same_first_blocks_match, pin_first_token_differs_matches_nothing,
        pin_later_block_needs_the_whole_prefix, pin_only_full_blocks_are_keyed, pin_released_blocks_stay_evictable,
        pin_least_recently_released_is_evicted]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_model_pin(pin):
    pin(PrefixModel)


class _BlockLocalKey(PrefixModel):
    def key(self, tokens, j):
        return tuple(tokens[j * self.bs:(j + 1) * self.bs])


class _NewestEvicted(PrefixModel):
    def allocate(self):
        if self.free == 0 and self.lru:
            self.lru.insert(0, self.lru.pop())  # evict the most recently released
        return super().allocate()


class _ReleaseFrees(PrefixModel):
    def release(self, b):
        b.ref -= 1
        if b.ref == 0:
            if b.key is not None:
                del self.cache[b.key]
                b.key = None
            self.free += 1


@pytest.mark.parametrize("planted", [_BlockLocalKey, _NewestEvicted, _ReleaseFrees],
                         ids=["block-local key", "newest evicted", "release frees"])
def test_planted_mistakes_fail_a_pin(planted):
    failed = 0
    for pin in PINS:
        try:
            pin(planted)
        except (AssertionError, KeyError, ValueError):
            failed += 1
    assert failed >= 1
