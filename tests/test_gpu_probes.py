"""The bandwidth probes read exactly the bytes they are meant to, each once:
the XOR of every lane's word equals the XOR of all 32-bit words of the
contiguous buffer (stream) or of every K and V tile the block table names for
the uploaded lengths (gather; a workload without shared blocks, so no tile is
named twice)."""
import numpy as np
import pytest
import torch

from paged_kv_cache_09_amd import pkv, workloads as W
from paged_kv_cache_09_amd.session import DecodeSession

pytestmark = pytest.mark.gpu


def _xor_all(words: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(words.astype(np.uint32).ravel(), initial=np.uint32(0)))


@pytest.mark.parametrize("nbytes,waves", [(16, 1), (1 << 20, 7), ((3 << 20) + 48, 2048)])
def test_stream_probe_reads_every_byte_once(nbytes, waves):
    gen = torch.Generator(device="cuda").manual_seed(nbytes)
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=gen)
    out = torch.empty(waves * 64, dtype=torch.int32, device="cuda")
    pkv.probe_stream_read(buf, nbytes, out, waves, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    want = _xor_all(buf.cpu().numpy().view(np.uint32))
    assert _xor_all(out.cpu().numpy().view(np.uint32)) == want


@pytest.mark.parametrize("waves", [1, 5, 64, 2048])
def test_gather_probe_reads_every_named_tile_once(waves):
    cfg = W.scaled(W.CONFIGS["llama8b_bf16"], batch=9, num_blocks=9 * 50, ctx_lo=1, ctx_hi=700)
    w = W.make(cfg, device="cuda", layers=1, form="step", fill="random", extra_blocks=1)
    sess = DecodeSession(w)
    sess.prepare()
    sess.upload()
    out = torch.empty(waves * 64, dtype=torch.int32, device="cuda")
    pkv.probe_gather(sess.pool, 0, out, waves, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    k, v = w.layer_views(0)  # [num_blocks][kv_heads][16][head_dim]
    kw = k.cpu().contiguous().view(torch.int32).numpy().reshape(k.shape[0], -1)
    vw = v.cpu().contiguous().view(torch.int32).numpy().reshape(v.shape[0], -1)
    want = 0
    for s in range(cfg.batch):
        for j in range((int(sess.ctx[s]) + 15) // 16):
            b = int(sess.table[s][j])
            want ^= _xor_all(kw[b]) ^ _xor_all(vw[b])
    assert _xor_all(out.cpu().numpy().view(np.uint32)) == want
    sess.close()


def test_probes_reject_bad_arguments():
    out = torch.empty(64, dtype=torch.int32, device="cuda")
    buf = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PkvError):
        pkv.probe_stream_read(buf, 40, out, 1)   # not a multiple of 16
    with pytest.raises(pkv.PkvError):
        pkv.probe_stream_read(buf, 64, out, 0)   # no wave
