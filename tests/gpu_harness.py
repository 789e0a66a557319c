"""Parity harness: run one decode step through the C ABI and the same step through the oracle.

The oracle only ever sees generator inputs (pre-step pool bytes, pre-step
tables, lengths, q, k_new, v_new); nothing it consumes comes from the GPU path.
For large workloads the comparison runs on a sample of sequences: the blocks
those sequences reference are copied into a compact host pool and their
tables renumbered, which changes no logical content.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from oracle import step as ostep
from paged_kv_cache_09_amd import pkv
from paged_kv_cache_09_amd import workloads as W
from paged_kv_cache_09_amd.session import DecodeSession
from tests.helpers import to_storage


def say(msg: str):
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def tolerance(cfg) -> float:
    return 1e-5 if cfg.dtype == W.F32 else 2e-3


class OracleSide:
    """Compact host copy of the sampled sequences and the oracle's results for them."""

    def __init__(self, w: W.Workload, seqs):
        self.seqs = list(seqs)
        cfg = w.cfg
        used = sorted({b for s in self.seqs for b in w.pre_tables[s]})
        spare = len(self.seqs)  # room for new / copied blocks
        self.nb = len(used) + spare
        remap = {b: i for i, b in enumerate(used)}
        idx = torch.tensor(used, dtype=torch.long, device=w.pool.device)
        self.k, self.v = [], []
        for layer in range(w.layers):
            kl, vl = w.layer_views(layer)
            shape = (self.nb,) + tuple(kl.shape[1:])
            # unused blocks: NaN (q8_0 tiles: 0xff bytes, i.e. NaN scales)
            fillv = 255 if kl.dtype == torch.uint8 else float("nan")
            kc = torch.full(shape, fillv, dtype=kl.dtype)
            vc = torch.full(shape, fillv, dtype=vl.dtype)
            if used:
                kc[:len(used)] = kl.index_select(0, idx).cpu()
                vc[:len(used)] = vl.index_select(0, idx).cpu()
            self.k.append(to_storage(kc))
            self.v.append(to_storage(vc))
        self.pre = [[remap[b] for b in w.pre_tables[s]] for s in self.seqs]
        refs = {}
        for row in self.pre:
            for b in row:
                refs[b] = refs.get(b, 0) + 1
        self.shared = [(b, n) for b, n in refs.items() if n > 1]
        self.ctx = np.ascontiguousarray(w.ctx[self.seqs], dtype=np.int32)
        sel = torch.tensor(self.seqs, dtype=torch.long, device=w.pool.device)
        self.k_new = to_storage(w.k_new.index_select(0, sel))
        self.v_new = to_storage(w.v_new.index_select(0, sel))
        self.q = to_storage(w.q.index_select(0, sel))
        self.cfg = cfg
        self.layers = w.layers
        self.max_blocks = w.max_blocks

    def run(self):
        bs = self.cfg.block_size
        self.table, self.kinds = ostep.run_step(
            self.k, self.v, self.pre, self.shared, self.ctx,
            [self.k_new] * self.layers, [self.v_new] * self.layers, dtype=self.cfg.dtype,
            num_blocks=self.nb, max_blocks=self.max_blocks, block_size=bs)
        self.out = [oracle.decode(self.k[l], self.v[l], self.table, self.ctx, self.q,
                                  W.attn_scale(self.cfg), dtype=self.cfg.dtype, block_size=bs)
                    for l in range(self.layers)]
        return self

    def logical(self, layer):
        return ostep.logical_rows(self.k[layer], self.v[layer], self.table, self.ctx,
                                  self.cfg.block_size)


def gpu_logical(sess: DecodeSession, layer: int, seqs):
    """Bytes of the sampled sequences' rows read back through the library's table
    (q8_0: each row's codes then its scale bytes in group order)."""
    k, v = sess.w.layer_views(layer)
    res = []
    for s in seqs:
        L = int(sess.ctx[s])
        t = torch.arange(L, device=k.device)
        bs = sess.cfg.block_size
        blocks = torch.from_numpy(sess.table[s].astype(np.int64)).to(k.device)[t // bs]
        rows = t % bs
        if k.dtype == torch.uint8:
            kt, vt = to_storage(k[blocks]), to_storage(v[blocks])
            idx = np.arange(L)
            res.append((ostep.q8_row_bytes(kt, idx, rows.cpu().numpy(), False, bs),
                        ostep.q8_row_bytes(vt, idx, rows.cpu().numpy(), True, bs)))
        else:
            res.append((to_storage(k[blocks, :, rows, :]), to_storage(v[blocks, :, rows, :])))
    return res


def pick_seqs(w: W.Workload, sample: int | None, seed: int = 0):
    B = w.B
    if sample is None or sample >= B:
        return list(range(B))
    rng = np.random.default_rng(seed)
    picks = set(rng.choice(B, size=sample - 2, replace=False).tolist())
    picks.add(int(np.argmax(w.ctx)))
    picks.add(int(np.argmin(w.ctx)))
    return sorted(picks)


def run_step_case(cfg, *, layers=1, partitions=(0,), sample=None, check_untouched=True,
                  label="", fused=False, edit=None):
    """Full step on both sides; returns a dict of max errors per (layer, partition).
    ``edit(w)``, if given, may rewrite the generated inputs before either side runs."""
    say(f"case {label or cfg.name}: build workload B={cfg.batch} layers={layers}")
    w = W.make(cfg, device="cuda", layers=layers, form="step", fill="nan")
    if edit is not None:
        edit(w)
    seqs = pick_seqs(w, sample)
    say(f"case {label or cfg.name}: oracle on {len(seqs)} sequences")
    ora = OracleSide(w, seqs).run()
    before = w.pool.clone() if check_untouched else None
    sess = DecodeSession(w)
    say(f"case {label or cfg.name}: GPU step partitions={list(partitions)} fused={fused}")
    slots, pairs = sess.prepare()
    sess.upload()
    sess.copy_blocks()
    errs = {}
    outs = {}
    for layer in range(layers):
        if not fused:
            sess.append(layer)
        for k, part in enumerate(partitions):
            out = sess.new_out()
            out.fill_(float("nan"))
            if fused and k == 0:
                sess.append_decode(layer, out, part)  # append fused into the first decode
            else:
                sess.decode(layer, out, part)
            torch.cuda.synchronize()
            # every sequence's output is finite, compared or not
            assert bool(torch.isfinite(out).all()), \
                f"non-finite output layer {layer} partition {part}"
            got = out.cpu().numpy()[seqs]
            errs[(layer, part)] = float(np.max(np.abs(got - ora.out[layer])))
            outs[(layer, part)] = out
    say(f"case {label or cfg.name}: max errors {errs}")
    # logical content after the step, byte for byte
    for layer in range(layers):
        mine = gpu_logical(sess, layer, seqs)
        theirs = ora.logical(layer)
        for i, s in enumerate(seqs):
            assert mine[i][0].tobytes() == theirs[i][0].tobytes(), f"K rows of seq {s} layer {layer}"
            assert mine[i][1].tobytes() == theirs[i][1].tobytes(), f"V rows of seq {s} layer {layer}"
    if check_untouched:
        _check_untouched(w, before, slots, pairs, layers)
    sess.close()
    return errs, outs, w


def _check_untouched(w, before, slots, pairs, layers):
    """Only the appended rows and copy-on-write destination blocks may change."""
    cfg = w.cfg
    if cfg.dtype in W.QUANTISED:
        return _check_untouched_q8(w, before, slots, pairs, layers)
    bs = cfg.block_size
    shape = (2, layers, cfg.num_blocks, cfg.kv_heads, bs, cfg.head_dim * W.ELEM_BYTES[cfg.dtype])
    a = w.pool.view(shape)
    b = before.view(shape)
    changed = (a != b).any(dim=-1)  # [2][layers][NB][Hkv][block_size]
    allowed = torch.zeros_like(changed)
    for dst in (int(p[1]) for p in pairs):
        allowed[:, :, dst] = True
    for sl in slots:
        if sl >= 0:
            allowed[:, :, int(sl) // bs, :, int(sl) % bs] = True
    bad = changed & ~allowed
    assert not bool(bad.any()), f"{int(bad.sum())} rows changed outside the written slots"


def _check_untouched_q8(w, before, slots, pairs, layers):
    """Quantised caches: byte by byte, only each new row's codes (where the tile
    layout places them) and scales (K scales [row][group], V
    scales [group][row] after a tile's codes) and whole copy-on-write
    destination tiles may change."""
    cfg = w.cfg
    D = W.code_row_bytes(cfg)  # code bytes per row
    ng = cfg.head_dim // 32
    tb = W.tile_bytes(cfg)
    shape = (2, layers, cfg.num_blocks, cfg.kv_heads, tb)
    changed = (w.pool.view(shape) != before.view(shape))
    allowed = torch.zeros_like(changed)
    for dst in (int(p[1]) for p in pairs):
        allowed[:, :, dst] = True
    for sl in slots:
        if sl < 0:
            continue
        bs = cfg.block_size
        b, r = int(sl) // bs, int(sl) % bs
        if cfg.dtype == W.Q4_0:
            # K words within the row's bytes; V rows interleaved as the layout places them
            allowed[0, :, b, :, r * D:(r + 1) * D] = True
            idx = torch.from_numpy(ostep.q4_code_index([r], True, cfg.head_dim)[0]).to(
                allowed.device)
            allowed[1, :, b, :, idx] = True
        else:  # q8_0: the row's codes where the layout places them
            for kv in (0, 1):
                idx = torch.from_numpy(
                    ostep.q8_code_index([r], bool(kv), cfg.head_dim, bs)[0]).to(allowed.device)
                allowed[kv, :, b, :, idx] = True
        for grp in range(ng):
            ik = bs * D + 2 * (r * ng + grp)
            iv = bs * D + 2 * (grp * bs + r)
            allowed[0, :, b, :, ik:ik + 2] = True
            allowed[1, :, b, :, iv:iv + 2] = True
    bad = changed & ~allowed
    assert not bool(bad.any()), f"{int(bad.sum())} bytes changed outside the written rows"


def run_write_case(cfg, n_lo, n_hi, *, layers=2, partitions=(0, 48, 1 << 20), label=""):
    """Multi-token write (prefill chunk) of every layer, then decode; against the oracle."""
    say(f"write case {label}: build workload B={cfg.batch} layers={layers}")
    w = W.make(cfg, device="cuda", layers=layers, form="step", fill="nan",
               extra_blocks=(n_hi + cfg.block_size - 1) // cfg.block_size + 1)
    before_ctx, n_new, k_rows, v_rows = W.write_rows(w, n_lo, n_hi)
    after_ctx = before_ctx + n_new
    ks, vs = [], []
    for layer in range(layers):
        kl, vl = w.layer_views(layer)
        ks.append(to_storage(kl))
        vs.append(to_storage(vl))
    kr, vr = to_storage(k_rows), to_storage(v_rows)
    say(f"write case {label}: oracle, {int(n_new.sum())} rows")
    table_o, _ = ostep.run_write(ks, vs, w.pre_tables, w.shared, before_ctx, n_new,
                                 [kr] * layers, [vr] * layers, dtype=cfg.dtype,
                                 num_blocks=cfg.num_blocks, max_blocks=w.max_blocks,
                                 block_size=cfg.block_size)
    q = to_storage(w.q)
    ora_out = [oracle.decode(ks[l], vs[l], table_o, after_ctx, q, W.attn_scale(cfg),
                             dtype=cfg.dtype, block_size=cfg.block_size)
               for l in range(layers)]
    before = w.pool.clone()
    sess = DecodeSession(w)
    say(f"write case {label}: GPU write + decode partitions={list(partitions)}")
    slots, pairs = sess.prepare_write(before_ctx, n_new)
    sess.copy_blocks()
    for layer in range(layers):
        sess.write(layer, k_rows, v_rows)
    sess.upload(with_slots=False)
    errs = {}
    for layer in range(layers):
        for part in partitions:
            out = sess.new_out()
            out.fill_(float("nan"))
            sess.decode(layer, out, part)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            assert np.isfinite(got).all(), f"non-finite output layer {layer} partition {part}"
            errs[(layer, part)] = float(np.max(np.abs(got - ora_out[layer])))
    say(f"write case {label}: max errors {errs}")
    seqs = list(range(w.B))
    for layer in range(layers):
        mine = gpu_logical(sess, layer, seqs)
        theirs = ostep.logical_rows(ks[layer], vs[layer], table_o, after_ctx, cfg.block_size)
        for s in seqs:
            assert mine[s][0].tobytes() == theirs[s][0].tobytes(), f"K rows of seq {s} layer {layer}"
            assert mine[s][1].tobytes() == theirs[s][1].tobytes(), f"V rows of seq {s} layer {layer}"
    _check_untouched(w, before, slots, pairs, layers)
    sess.close()
    return errs


def run_prefix_case(cfg, *, num_blocks, n_prefixes, prefix_len, suffix_hi, na, nb, seed,
                    partitions=(0, 1 << 20), label=""):
    """Prefix caching on the GPU path: phase 1 writes na prompts (a shared system
    prompt + own suffix) and registers their full blocks; they end (blocks stay
    cached); phase 2 serves nb new prompts that match cached leading blocks,
    writes only the rest, and decodes. The oracle replays the same steps with
    the plain prefix model and its own block placement."""
    from oracle.prefix_model import PrefixModel

    BS = 16
    rng = np.random.default_rng(seed)
    prefixes = [rng.integers(0, 32000, size=prefix_len).tolist() for _ in range(n_prefixes)]
    prompts = []
    for _ in range(na + nb):
        p = prefixes[int(rng.integers(0, n_prefixes))]
        prompts.append(p + rng.integers(0, 32000, size=int(rng.integers(1, suffix_hi + 1))).tolist())
    max_blocks = max(-(-len(t) // BS) for t in prompts)
    H, D = cfg.kv_heads, cfg.head_dim
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    tdt = W.TORCH_DTYPE[cfg.dtype]

    def rows(n):
        r = torch.randn((n, H, D), generator=gen, device="cuda", dtype=torch.float32)
        return r.to(tdt)

    # an empty one-layer pool: every row NaN (q8_0: 0xff bytes, NaN scales)
    cfg_pool = W.scaled(cfg, num_blocks=num_blocks, batch=nb)
    dev_pool = torch.empty(2 * W.region_bytes(cfg_pool, 1), dtype=torch.uint8, device="cuda")
    if cfg.dtype in W.QUANTISED:
        dev_pool.fill_(255)
    else:
        dev_pool.view(tdt).fill_(float("nan"))
    views = lambda: W.pool_layer_views(dev_pool, cfg_pool, 1, 0)  # noqa: E731
    shape = pkv.make_shape(1, num_blocks, H, D, cfg.dtype, max_blocks * BS, max(na, nb))
    pool = pkv.kv_pool_alloc(shape, dev_pool, dev_pool.numel())
    stream = torch.cuda.current_stream().cuda_stream

    # oracle side: host pool, plain model, own placement (tags = own ids)
    k_o, v_o = (to_storage(t) for t in views())
    model = PrefixModel(num_blocks, BS)
    free_tags = list(range(num_blocks - 1, -1, -1))

    def o_alloc():
        b = model.allocate()
        if b.tag is None:  # a block from the free pool: give it one of our ids
            b.tag = free_tags.pop()
        return b

    def o_release(b):
        if b.key is None and b.ref == 1:  # back to the free pool: its id too
            free_tags.append(b.tag)
        model.release(b)

    def o_write(table_row, start, tok_rows_k, tok_rows_v):
        n = tok_rows_k.shape[0]
        for t in range(n):
            ctx = np.array([start + t + 1], np.int32)
            oracle.append(k_o, v_o, table_row[None, :], ctx, tok_rows_k[t:t + 1],
                          tok_rows_v[t:t + 1], dtype=cfg.dtype)

    def serve(tokens, k_rows, v_rows):
        ids = pkv.prefix_match(pool, tokens, max_blocks)
        mb = model.match(tokens)
        assert len(ids) == len(mb)
        k = len(ids)
        table = np.full((1, max_blocks), -1, np.int32)
        table[0, :k] = ids
        n_new = len(tokens) - k * BS
        slots, pairs = pkv.prepare_write(pool, table, [k * BS], [n_new])
        assert len(pairs) == 0
        dev_slots = torch.from_numpy(slots).cuda()
        pkv.kv_append(pool, 0, k_rows[k * BS:], v_rows[k * BS:], dev_slots, n_new, stream)
        nblk = -(-len(tokens) // BS)
        pkv.prefix_insert(pool, tokens, table[0, :nblk])
        blocks = list(mb) + [o_alloc() for _ in range(nblk - k)]
        o_row = np.full(max_blocks, -1, np.int32)
        o_row[:nblk] = [b.tag for b in blocks]
        o_write(o_row, k * BS, to_storage(k_rows[k * BS:]), to_storage(v_rows[k * BS:]))
        model.insert(tokens, blocks)
        return table[0], blocks, o_row, k

    say(f"prefix case {label}: phase 1, {na} prompts served one after another")
    for i in range(na):
        n = len(prompts[i])
        row, blocks, _, _ = serve(prompts[i], rows(n), rows(n))
        pkv.block_free(pool, row[row >= 0])  # the request ends; its blocks stay cached
        for b in blocks:
            o_release(b)
    torch.cuda.synchronize()
    say(f"prefix case {label}: phase 2, {nb} prompts")
    tables, o_tables, ctx, matched = [], [], [], 0
    for i in range(na, na + nb):
        n = len(prompts[i])
        row, blocks, o_row, k = serve(prompts[i], rows(n), rows(n))
        tables.append(row)
        o_tables.append(o_row)
        ctx.append(n)
        matched += k
    assert matched > 0, "phase 2 matched nothing"
    table = np.ascontiguousarray(np.stack(tables))
    o_table = np.ascontiguousarray(np.stack(o_tables))
    ctx = np.array(ctx, np.int32)
    q = torch.randn((nb, cfg.q_heads, D), generator=gen, device="cuda").to(tdt)
    pkv.block_table_upload(pool, table, ctx, None, stream)
    want = oracle.decode(k_o, v_o, o_table, ctx, to_storage(q), W.attn_scale(cfg),
                         dtype=cfg.dtype)
    errs = {}
    for part in partitions:
        nbytes = pkv.decode_workspace_bytes(pool, nb, cfg.q_heads, part)
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        out = torch.full((nb, cfg.q_heads, D), float("nan"), device="cuda")
        pkv.paged_attn_decode(pool, 0, q, cfg.q_heads, W.attn_scale(cfg), out, part, ws,
                              ws.numel(), stream)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.isfinite(got).all()
        errs[part] = float(np.max(np.abs(got - want)))
    # logical rows through both tables agree byte for byte
    k_g, v_g = (to_storage(t) for t in views())
    mine = ostep.logical_rows(k_g, v_g, table, ctx)
    theirs = ostep.logical_rows(k_o, v_o, o_table, ctx)
    for s in range(nb):
        assert mine[s][0].tobytes() == theirs[s][0].tobytes(), f"K rows of seq {s}"
        assert mine[s][1].tobytes() == theirs[s][1].tobytes(), f"V rows of seq {s}"
    say(f"prefix case {label}: matched {matched} blocks, max errors {errs}")
    pkv.kv_pool_free(pool)
    return errs
