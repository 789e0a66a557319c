"""Plain model of the block bookkeeping behind a decode step (test infrastructure).

It encodes what the pages state about physical blocks, and nothing about how
a library stores them:

* physical blocks are handed out on demand, only when tokens actually arrive
  (thienlv.com, "PagedAttention là gì?", section "How does PagedAttention
  work?", the on-demand allocation point);
* blocks with identical content may be shared by several sequences, and a
  shared block is copied only when one sharer writes to it, as with the
  operating system's copy-on-write (ahmedhaies.com, "PagedAttention: why LLM
  serving wastes most GPU memory", the paragraph after "The solution: borrow
  virtual memory from the OS");
* a shared block stays allocated while anything references it (same page,
  section "Trade-offs", the prefix-caching point), i.e. it is refcounted.

For one decode step, sequences are taken in batch order. Sequence s writes its
new token at logical position p = L_s - 1, logical block j = p // block_size:
  - "new"     the entry for block j is absent: take a free block;
  - "cow"     the block is referenced more than once: take a free block,
              copy the old one into it, drop one reference to the old one;
  - "inplace" the block is referenced exactly once: write it in place.

A multi-token write (a prompt, or a chunk of one, whose K/V rows are all
written to the cache: news.hamidun.com "KV-Cache", prefill/decode paragraph)
applies the same three rules to every logical block its positions touch,
block by block, sequences in batch order.

Which free block is taken is not unique, so the model tracks only what is:
the kind per sequence (or per touched block), the reference count of every
pre-existing block after the step, and how many blocks are free afterwards.
"""


class BlockModel:
    def __init__(self, num_blocks: int):
        self.num_blocks = num_blocks
        self.refcount = [0] * num_blocks
        self.anonymous = 0  # blocks taken during planned steps (ids not modelled)

    def claim(self, ids):
        for b in ids:
            if self.refcount[b] != 0:
                raise ValueError(f"block {b} is not free")
            self.refcount[b] = 1

    def ref(self, ids):
        for b in ids:
            if self.refcount[b] <= 0:
                raise ValueError(f"block {b} is not allocated")
            self.refcount[b] += 1

    def free(self, ids):
        for b in ids:
            if self.refcount[b] <= 0:
                raise ValueError(f"block {b} is not allocated")
            self.refcount[b] -= 1

    def free_count(self) -> int:
        return sum(1 for r in self.refcount if r == 0) - self.anonymous

    def plan_append(self, tables, ctx_lens, block_size: int = 16):
        """Kinds per sequence for one decode step; updates the model in place.

        ``tables[s]`` lists sequence s's physical blocks before the step (absent
        trailing entries are simply not in the list).
        """
        kinds = []
        for s, L in enumerate(ctx_lens):
            p = L - 1
            j = p // block_size
            row_blocks = tables[s]
            if j >= len(row_blocks) or row_blocks[j] < 0:
                kinds.append("new")
                self.anonymous += 1
                continue
            b = row_blocks[j]
            if self.refcount[b] > 1:
                kinds.append("cow")
                self.refcount[b] -= 1
                self.anonymous += 1
            else:
                kinds.append("inplace")
        return kinds

    def plan_write(self, tables, ctx_before, n_new, block_size: int = 16):
        """Kinds per touched block for writing n_new[s] tokens after ctx_before[s]:
        a list of (sequence, logical block, kind); updates the model in place."""
        plan = []
        for s, (l0, n) in enumerate(zip(ctx_before, n_new)):
            if n <= 0:
                continue
            first = l0 // block_size
            last = (l0 + n - 1) // block_size
            row_blocks = tables[s]
            for j in range(first, last + 1):
                if j >= len(row_blocks) or row_blocks[j] < 0:
                    plan.append((s, j, "new"))
                    self.anonymous += 1
                    continue
                b = row_blocks[j]
                if self.refcount[b] > 1:
                    plan.append((s, j, "cow"))
                    self.refcount[b] -= 1
                    self.anonymous += 1
                else:
                    plan.append((s, j, "inplace"))
        return plan
