"""Seeded synthetic decode workloads shared by the tests, the smoke check and the benchmark.

This module draws inputs only; it holds none of the decode arithmetic (no
slot formula, no attention, no append). Both the GPU library and the CPU
oracle consume what it produces.

Each workload describes one decode step of a batch of sequences whose caches
live in 16-token physical blocks scattered through one pool:

* ``ctx[s]``       tokens attended by sequence s, the new token included;
* ``pre_tables``   physical blocks holding each sequence's cached tokens
                   before the step (``ctx[s] - 1`` of them);
* ``new_blocks``   for the plain-decode form, a block picked for the new token
                   when it starts a block (-1 otherwise);
* ``shared``       blocks referenced by several sequences and their
                   reference counts;
* the pool bytes, q, k_new and v_new as torch tensors on the chosen device.

Physical placement follows a seeded permutation of the pool's block ids,
taken in (sequence, logical block) order, so logical neighbours are scattered
through the pool. Cache values, q and the new K/V are N(0, sigma) draws made
in fp32 and rounded to the cache dtype by torch (round to nearest even). A
q8_0 / q4_0 cache holds random codes and random fp16 scales (its q and new
rows are bf16). Rows of the pool that hold no token are NaN (quantised: NaN scales) for
parity runs, so a kernel that reads them poisons its output.

The five shapes follow the pages' statement of the problem (layers, kv heads,
query heads with grouped-query attention, head_dim, block size 16) at the
Llama-3.1-8B and 13B sizes they discuss.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

F32, F16, BF16, Q8_0, Q4_0 = 0, 1, 2, 3, 4
QUANTISED = (Q8_0, Q4_0)
# element type of q, k_new and v_new (and of the cache itself, unless quantised)
TORCH_DTYPE = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16,
               Q8_0: torch.bfloat16, Q4_0: torch.bfloat16}
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}
DTYPE_NAME = {F32: "f32", F16: "f16", BF16: "bf16", Q8_0: "q8_0", Q4_0: "q4_0"}
BLOCK = 16
Q8_GROUP = 32


def code_row_bytes(cfg) -> int:
    """Code bytes of one quantised row: head_dim (q8_0) or head_dim / 2 (q4_0)."""
    return cfg.head_dim // 2 if cfg.dtype == Q4_0 else cfg.head_dim


def row_bytes(cfg) -> int:
    """Pool bytes of one token's K (or V) row of one kv head: head_dim elements,
    or for q8_0 / q4_0 the codes plus one fp16 scale per 32 elements."""
    if cfg.dtype in QUANTISED:
        return code_row_bytes(cfg) + 2 * (cfg.head_dim // Q8_GROUP)
    return cfg.head_dim * ELEM_BYTES[cfg.dtype]


def tile_bytes(cfg) -> int:
    """Bytes of one (block, kv head) tile of K (or V): block_size rows."""
    return cfg.block_size * row_bytes(cfg)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed: int
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    dtype: int
    sigma: float
    num_blocks: int
    layers: int              # layers the benchmark rotates over
    ctx_kind: str            # "fixed" | "uniform" | "uniform_partial" | "shared_prefix"
    ctx_fixed: tuple = ()
    ctx_lo: int = 0
    ctx_hi: int = 0
    prefix_tokens: int = 0   # shared-prefix workloads
    suffix_hi: int = 0
    partition_tokens: int = 0  # split-K partition the workload is quoted with (0: none)
    block_size: int = 16       # tokens per pool block (8, 16 or 32)


CONFIGS = {
    # 1 layer, 4 sequences, 4 q / 2 kv heads, d 64, fp32, 64-block pool.
    "tiny_f32": Config("tiny_f32", 1, 4, 4, 2, 64, F32, 1.0, 64, 1, "fixed",
                       ctx_fixed=(5, 17, 32, 50)),
    # Llama-3.1-8B-shaped layer: 32 q / 8 kv heads, d 128, bf16, batch 64,
    # context uniform in [128, 2048]; 32 layers of pool for the benchmark.
    "llama8b_bf16": Config("llama8b_bf16", 2, 64, 32, 8, 128, BF16, 1.0, 64 * 136, 32,
                           "uniform", ctx_lo=128, ctx_hi=2048),
    # 13B-shaped MHA layer: 40 q = 40 kv heads, d 128, fp16, batch 256,
    # context uniform in [16, 2048] with a partly filled last block, sigma 0.5.
    "mha13b_f16": Config("mha13b_f16", 3, 256, 40, 40, 128, F16, 0.5, 256 * 136, 1,
                         "uniform_partial", ctx_lo=16, ctx_hi=2048),
    # 128 sequences sharing a 1024-token prefix (64 blocks), each with a private
    # suffix of uniform [0, 512] tokens; GQA 32/8, d 128, bf16.
    "shared_prefix_bf16": Config("shared_prefix_bf16", 4, 128, 32, 8, 128, BF16, 1.0, 8192, 8,
                                 "shared_prefix", prefix_tokens=1024, suffix_hi=512),
    # Copy-on-write case of the shared prefix: a 1016-token prompt shared by all
    # 128 sequences (last shared block half full), every sequence at suffix 0.
    "shared_prefix_cow_bf16": Config("shared_prefix_cow_bf16", 4, 128, 32, 8, 128, BF16, 1.0,
                                     8192, 8, "shared_prefix", prefix_tokens=1016,
                                     suffix_hi=0),
    # The shared prefix with quantised caches (no grouped items: the bins form,
    # whose XCD affinity has the prompt fetched from HBM once and re-read from L2).
    "shared_prefix_q8": Config("shared_prefix_q8", 4, 128, 32, 8, 128, Q8_0, 1.0, 8192, 8,
                               "shared_prefix", prefix_tokens=1024, suffix_hi=512),
    "shared_prefix_q4": Config("shared_prefix_q4", 4, 128, 32, 8, 128, Q4_0, 1.0, 8192, 8,
                               "shared_prefix", prefix_tokens=1024, suffix_hi=512),
    # The Llama-3.1-8B-shaped layer with a q8_0 cache (int8 codes, one fp16
    # scale per 32 elements); same lengths and placement as the bf16 one.
    "llama8b_q8": Config("llama8b_q8", 2, 64, 32, 8, 128, Q8_0, 1.0, 64 * 136, 32,
                         "uniform", ctx_lo=128, ctx_hi=2048),
    # ... and with a q4_0 cache (4-bit codes, one fp16 scale per 32 elements).
    "llama8b_q4": Config("llama8b_q4", 2, 64, 32, 8, 128, Q4_0, 1.0, 64 * 136, 32,
                         "uniform", ctx_lo=128, ctx_hi=2048),
    # Long context: batch 4 x 131072 tokens (8192 blocks each), GQA 32/8, d 128,
    # bf16, 512-token split-K partitions.
    "long_ctx_bf16": Config("long_ctx_bf16", 5, 4, 32, 8, 128, BF16, 1.0, 32768, 1, "fixed",
                            ctx_fixed=(131072,) * 4, partition_tokens=512),
}


def scaled(cfg: Config, **changes) -> Config:
    """A copy of ``cfg`` with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(cfg, **changes)


def _children(seed: int, n: int):
    return [np.random.default_rng(c) for c in np.random.SeedSequence(seed).spawn(n)]


def draw_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    B = cfg.batch
    if cfg.ctx_kind == "fixed":
        ctx = np.array(cfg.ctx_fixed, dtype=np.int64)
        assert ctx.size == B
    elif cfg.ctx_kind == "uniform":
        ctx = rng.integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=B)
    elif cfg.ctx_kind == "uniform_partial":
        ctx = rng.integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=B)
        # redraw lengths whose last block would be exactly full
        while True:
            full = ctx % cfg.block_size == 0
            if not full.any():
                break
            ctx[full] = rng.integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=int(full.sum()))
    elif cfg.ctx_kind == "shared_prefix":
        suffix = rng.integers(0, cfg.suffix_hi + 1, size=B) if cfg.suffix_hi > 0 \
            else np.zeros(B, dtype=np.int64)
        ctx = cfg.prefix_tokens + suffix + 1
    else:
        raise ValueError(cfg.ctx_kind)
    return ctx.astype(np.int32)


def _nblk(n_tokens: int, block_size: int = BLOCK) -> int:
    return (n_tokens + block_size - 1) // block_size


@dataclasses.dataclass
class Workload:
    cfg: Config
    layers: int
    ctx: np.ndarray                 # int32 [B], new token included
    pre_tables: list                # list of lists of physical ids (cached tokens)
    new_blocks: np.ndarray          # int32 [B], -1 when the new token needs no block
    shared: list                    # [(block_id, refcount)] for blocks with refcount > 1
    max_blocks: int                 # table width
    pool: torch.Tensor              # uint8 [pool_bytes], K region then V region
    q: torch.Tensor                 # [B][Hq][D] cache dtype
    k_new: torch.Tensor             # [B][Hkv][D]
    v_new: torch.Tensor             # [B][Hkv][D]
    form: str                       # "step": pool holds ctx-1 tokens; "decode": ctx tokens

    @property
    def B(self):
        return self.cfg.batch

    def table(self, which: str = "pre") -> np.ndarray:
        """Block table int32 [B][max_blocks], -1 padded. "post" adds new_blocks."""
        bt = np.full((self.B, self.max_blocks), -1, dtype=np.int32)
        for s, row in enumerate(self.pre_tables):
            bt[s, :len(row)] = row
            if which == "post" and self.new_blocks[s] >= 0:
                bt[s, len(row)] = self.new_blocks[s]
        return bt

    def allocated_ids(self, which: str = "pre") -> list:
        """Distinct physical ids in use (each listed once)."""
        ids = []
        seen = set()
        for s, row in enumerate(self.pre_tables):
            for b in row:
                if b not in seen:
                    seen.add(b)
                    ids.append(b)
            if which == "post" and self.new_blocks[s] >= 0:
                ids.append(int(self.new_blocks[s]))
        return ids

    def layer_views(self, layer: int):
        """Typed views (K, V) of one layer: [NB][Hkv][16][D]."""
        return pool_layer_views(self.pool, self.cfg, self.layers, layer)


def region_bytes(cfg: Config, layers: int) -> int:
    """Bytes of the K region (the V region is the same size)."""
    return layers * cfg.num_blocks * cfg.kv_heads * tile_bytes(cfg)


def pool_layer_views(pool: torch.Tensor, cfg: Config, layers: int, layer: int):
    """(K, V) views of one layer: typed [NB][Hkv][16][D], or uint8
    [NB][Hkv][tile bytes] when quantised."""
    n = region_bytes(cfg, layers)
    if cfg.dtype in QUANTISED:
        shape = (layers, cfg.num_blocks, cfg.kv_heads, tile_bytes(cfg))
        return pool[:n].view(shape)[layer], pool[n:2 * n].view(shape)[layer]
    shape = (layers, cfg.num_blocks, cfg.kv_heads, cfg.block_size, cfg.head_dim)
    tdt = TORCH_DTYPE[cfg.dtype]
    return pool[:n].view(tdt).view(shape)[layer], pool[n:2 * n].view(tdt).view(shape)[layer]


def _fill_q8(pool: torch.Tensor, cfg: Config, layers: int, gen: torch.Generator,
             chunk: int = 1 << 26):
    """Quantised pool contents: q8_0 int8 codes uniform in [-127, 127] and fp16
    scales uniform in [0.005, 0.03]; q4_0 code bytes uniform (two 4-bit codes
    each) and scales of either sign with magnitude uniform in [0.05, 0.3]
    (rounded to fp16 by torch)."""
    D = cfg.head_dim
    CB = code_row_bytes(cfg) * cfg.block_size
    tiles = pool.view(2 * layers * cfg.num_blocks * cfg.kv_heads, tile_bytes(cfg))
    for i in range(0, tiles.shape[0], max(1, chunk // tiles.shape[1])):
        part = tiles[i:i + max(1, chunk // tiles.shape[1])]
        BS = cfg.block_size
        if cfg.dtype == Q8_0:
            codes = torch.randint(-127, 128, (part.shape[0], CB), generator=gen,
                                  device=pool.device, dtype=torch.int16)
            part[:, :CB].copy_(codes.to(torch.int8).view(torch.uint8))
            sc = torch.rand((part.shape[0], BS * (D // Q8_GROUP)), generator=gen,
                            device=pool.device, dtype=torch.float32) * 0.025 + 0.005
        else:
            codes = torch.randint(0, 256, (part.shape[0], CB), generator=gen,
                                  device=pool.device, dtype=torch.int16)
            part[:, :CB].copy_(codes.to(torch.uint8))
            sc = torch.rand((part.shape[0], BS * (D // Q8_GROUP)), generator=gen,
                            device=pool.device, dtype=torch.float32) * 0.25 + 0.05
            sign = torch.randint(0, 2, sc.shape, generator=gen, device=pool.device) * 2 - 1
            sc = sc * sign
        part[:, CB:].copy_(sc.to(torch.float16).view(torch.uint8).view(part.shape[0], -1))


def _fill_normal(t: torch.Tensor, sigma: float, gen: torch.Generator, chunk: int = 1 << 26):
    flat = t.view(-1)
    for i in range(0, flat.numel(), chunk):
        part = flat[i:i + chunk]
        vals = torch.randn(part.numel(), generator=gen, device=t.device, dtype=torch.float32)
        if sigma != 1.0:
            vals.mul_(sigma)
        part.copy_(vals.to(t.dtype))


def make(cfg: Config, *, device="cpu", layers: int | None = None, form: str = "step",
         fill: str = "nan", extra_blocks: int = 0, tensors: bool = True) -> Workload:
    """Build one workload.

    form   "step": the pool holds ctx-1 cached tokens per sequence and the step
           appends the new one; "decode": the pool already holds ctx tokens
           (the new token's block comes from ``new_blocks``).
    fill   "nan": rows holding no token are NaN; "random": every pool row is
           a random draw (benchmark).
    extra_blocks  table columns beyond the longest sequence (room to grow).
    tensors  False: lengths and placement only (pool, q, k_new, v_new are None).
    """
    layers = cfg.layers if layers is None else layers
    r_len, r_perm, r_vals = _children(cfg.seed, 3)
    ctx = draw_lengths(cfg, r_len)
    B = cfg.batch
    perm = r_perm.permutation(cfg.num_blocks).astype(np.int32)
    take = iter(perm.tolist())

    pre_tables = [[] for _ in range(B)]
    shared = []
    if cfg.ctx_kind == "shared_prefix":
        prefix = [next(take) for _ in range(_nblk(cfg.prefix_tokens, cfg.block_size))]
        for s in range(B):
            pre_tables[s] = list(prefix)
        shared = [(b, B) for b in prefix]
        first_private = len(prefix)
    else:
        first_private = 0
    for s in range(B):
        cached = int(ctx[s]) - 1
        for _ in range(first_private, _nblk(cached, cfg.block_size)):
            pre_tables[s].append(next(take))
    new_blocks = np.full(B, -1, dtype=np.int32)
    for s in range(B):
        if _nblk(int(ctx[s]), cfg.block_size) > len(pre_tables[s]):
            new_blocks[s] = next(take)
    max_blocks = max(_nblk(int(c), cfg.block_size) for c in ctx) + extra_blocks
    if not tensors:
        return Workload(cfg, layers, ctx, pre_tables, new_blocks, shared, max_blocks, None, None,
                        None, None, form)

    seed_vals = int(r_vals.integers(0, 2**62))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_vals)
    tdt = TORCH_DTYPE[cfg.dtype]
    nb = region_bytes(cfg, layers)
    pool = torch.empty(2 * nb, dtype=torch.uint8, device=device)
    if cfg.dtype in QUANTISED:
        _fill_q8(pool, cfg, layers, gen)
    else:
        _fill_normal(pool.view(tdt), cfg.sigma, gen)
    q = torch.empty((B, cfg.q_heads, cfg.head_dim), dtype=tdt, device=device)
    k_new = torch.empty((B, cfg.kv_heads, cfg.head_dim), dtype=tdt, device=device)
    v_new = torch.empty((B, cfg.kv_heads, cfg.head_dim), dtype=tdt, device=device)
    _fill_normal(q, cfg.sigma, gen)
    _fill_normal(k_new, cfg.sigma, gen)
    _fill_normal(v_new, cfg.sigma, gen)

    if fill == "nan":
        # rows that hold a token: cached ones (and the new one in "decode" form)
        BS = cfg.block_size
        valid = np.zeros((cfg.num_blocks, BS), dtype=bool)
        for s in range(B):
            n_tok = int(ctx[s]) - (1 if form == "step" else 0)
            row_blocks = list(pre_tables[s])
            if form == "decode" and new_blocks[s] >= 0:
                row_blocks.append(int(new_blocks[s]))
            for j, b in enumerate(row_blocks):
                rows = min(BS, n_tok - j * BS)
                if rows > 0:
                    valid[b, :rows] = True
        mask = torch.from_numpy(~valid).to(device)
        if cfg.dtype in QUANTISED:
            # a row without a token gets NaN scales: K scales are [row][group],
            # V scales [group][row] after the codes of a tile
            ng = cfg.head_dim // Q8_GROUP
            shape = (layers, cfg.num_blocks, cfg.kv_heads, tile_bytes(cfg))
            for r, region in enumerate((pool[:nb], pool[nb:2 * nb])):
                sc = region.view(shape)[..., BS * code_row_bytes(cfg):].view(torch.float16)
                if r == 0:
                    sc.view(layers, cfg.num_blocks, cfg.kv_heads, BS, ng).masked_fill_(
                        mask[None, :, None, :, None], float("nan"))
                else:
                    sc.view(layers, cfg.num_blocks, cfg.kv_heads, ng, BS).masked_fill_(
                        mask[None, :, None, None, :], float("nan"))
        else:
            shape = (layers, cfg.num_blocks, cfg.kv_heads, BS, cfg.head_dim)
            typed = pool.view(tdt)
            n = nb // ELEM_BYTES[cfg.dtype]
            for region in (typed[:n], typed[n:2 * n]):
                region.view(shape).masked_fill_(mask[None, :, None, :, None], float("nan"))
    elif fill != "random":
        raise ValueError(fill)

    return Workload(cfg, layers, ctx, pre_tables, new_blocks, shared, max_blocks, pool, q,
                    k_new, v_new, form)


def write_rows(w: Workload, n_lo: int, n_hi: int, device=None):
    """Rows for a multi-token write after a step-form workload's cached tokens:
    n_new[s] uniform in [n_lo, n_hi] tokens per sequence (a prompt chunk), and
    their K/V rows [sum n_new][Hkv][D] (input dtype, N(0, sigma)).

    Returns (ctx_before int32 [B] = ctx - 1, n_new int32 [B], k_rows, v_rows).
    """
    cfg = w.cfg
    rng = _children(cfg.seed, 4)[3]
    n_new = rng.integers(n_lo, n_hi + 1, size=w.B).astype(np.int32)
    total = int(n_new.sum())
    dev = device if device is not None else (w.pool.device if w.pool is not None else "cpu")
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(rng.integers(0, 2**62)))
    shape = (max(total, 1), cfg.kv_heads, cfg.head_dim)
    k_rows = torch.empty(shape, dtype=TORCH_DTYPE[cfg.dtype], device=dev)
    v_rows = torch.empty(shape, dtype=TORCH_DTYPE[cfg.dtype], device=dev)
    _fill_normal(k_rows, cfg.sigma, gen)
    _fill_normal(v_rows, cfg.sigma, gen)
    return (np.ascontiguousarray(w.ctx - 1, dtype=np.int32), n_new, k_rows[:total],
            v_rows[:total])


def attn_scale(cfg: Config) -> float:
    """Softmax scale passed to both sides: 1/sqrt(head_dim) for every shape."""
    return 1.0 / math.sqrt(cfg.head_dim)
