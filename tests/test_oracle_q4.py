"""Pins of the oracle's q4_0 cache (no GPU).

The pages name q4_0 as the cache type that takes about a quarter of an f16
cache (ssdnodes.com, "KV cache vs prompt cache", "Four ways to make the KV
cache smaller", item 2); it is read as llama.cpp's Q4_0 block: per 32
consecutive elements, m = the value of largest magnitude (the first on ties),
scale d = m / -8 stored as fp16, codes q = min(15, trunc(x / d + 8.5)),
value (q - 8) * d. The tests pin the oracle to that definition with cases
whose answer is known without it.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import step as ostep

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_sizes.json")


def _recon(codes, d):
    return (codes.astype(np.float64) - 8) * d.view(np.float16).astype(np.float64)[:, None]


def test_q4_row_is_about_a_quarter_of_f16():
    g = json.load(open(GOLDEN))["quantised_cache_q4_0"]
    per_token = 2 * g["layers"] * g["kv_heads"] * oracle.q_tile_bytes(
        oracle.Q4_0, g["head_dim"]) // 16
    assert per_token == 36864  # 64 code bytes + 4 fp16 scales per row of 128
    assert abs(per_token / g["f16_bytes_per_token"] - g["q4_0_approx_fraction_of_f16"]) < 0.05
    assert abs(per_token / 1024 - g["q4_0_approx_kib_per_token"]) / 32 < 0.15
    gib = per_token * g["tokens"] / 2**30
    assert abs(gib - g["q4_0_approx_gib"]) < 0.15 and gib < g["f16_gib"] / 3


def test_q4_exact_grid():
    # x = (q - 8) * d with d = 2^-3, the first value of largest magnitude being
    # -8 d: the scale is exactly d, the codes exactly q, reconstruction exact
    rng = np.random.default_rng(1)
    q = rng.integers(1, 16, size=(50, 32))        # values -7d .. 7d
    pos = rng.integers(0, 32, size=50)
    q[np.arange(50), pos] = 0                      # one -8 d per group
    x = ((q - 8) * 2.0 ** -3).astype(np.float32)
    codes, d = oracle.q4_quantize(x)
    assert np.array_equal(codes, q.astype(np.uint8))
    assert np.all(d == np.float16(2.0 ** -3).view(np.uint16))
    assert np.array_equal(_recon(codes, d), x.astype(np.float64))


def test_q4_scale_takes_the_sign_of_the_first_largest_value():
    x = np.zeros(32, np.float32)
    x[3], x[9] = -2.0, 2.0                         # tie: the first (negative) one wins
    codes, d = oracle.q4_quantize(x)
    assert np.float16(0.25).view(np.uint16) == d[0]
    assert codes[0, 3] == 0 and codes[0, 9] == 15  # +8 d clamps to code 15 (7 d)
    x[3], x[9] = 2.0, -2.0
    codes, d = oracle.q4_quantize(x)
    assert np.float16(-0.25).view(np.uint16) == d[0]
    assert codes[0, 3] == 0 and codes[0, 9] == 15


def test_q4_rounds_half_up_in_units_of_d():
    # m = -8 -> d = 1, x / d + 8.5 truncated: x = k + 0.5 -> k + 1 (half up)
    x = np.zeros(32, np.float32)
    x[0] = -8.0
    halves = [0.5, 1.5, -0.5, -1.5, 6.5]
    x[1:1 + len(halves)] = halves
    codes, d = oracle.q4_quantize(x)
    vals = _recon(codes, d)[0, 1:1 + len(halves)]
    assert vals.tolist() == [1.0, 2.0, 0.0, -1.0, 7.0]


def test_q4_zero_group():
    codes, d = oracle.q4_quantize(np.zeros((2, 32), np.float32))
    assert np.all(codes == 8) and np.all(d == np.float16(-0.0).view(np.uint16))


def test_q4_error_bound_random():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((4000, 32)) * 10.0 ** rng.uniform(-2, 2, (4000, 1))).astype(np.float32)
    codes, d = oracle.q4_quantize(x)
    dq = d.view(np.float16).astype(np.float64)
    first = np.argmax(np.abs(x) == np.abs(x).max(axis=1, keepdims=True), axis=1)
    m = x[np.arange(len(x)), first].astype(np.float64)
    dexact = m / -8
    assert np.all(codes <= 15)
    err = np.abs(x - _recon(codes, d))
    # half a step, the fp32 rounding of x/d + 8.5, the fp16 rounding of d; a value
    # at -m (code would be 16) clamps to 15: one full step
    clamp = codes == 15
    step = np.abs(dexact)[:, None]
    bound = np.where(clamp, 1.0, 0.5 + 1e-5) * step + 8 * np.abs(dq - dexact)[:, None]
    assert np.all(err <= bound)
    assert np.all(codes[np.arange(len(x)), first] == 0)


def _words(codes):
    """Codes [..][D] (0..15) -> bytes [..][D/8 words][4] in element order (element j
    of a word in byte j // 2, low nibble for even j)."""
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed.reshape(packed.shape[:-1] + (packed.shape[-1] // 4, 4))


def _pack_q4(codes, scales, is_v):
    """One tile [Hkv] of q4_0 bytes from codes [Hkv][R][D] (0..15) and fp16 scales
    [Hkv][R][D/32], in the pool's q4_0 layout (G = D/32 groups, words of 8
    elements, word w = 4k + q = group k, quarter q):
      K: each row's words reordered [q][k] (the G words of one quarter together);
      V: rows taken G at a time, words reordered [w][row of the G];
    then scales [row][group] (K) or [group][row] (V)."""
    H, R, D = codes.shape
    G = D // 32
    wd = _words(codes)                                    # [H][R][4G][4]
    if is_v:
        body = wd.reshape(H, R // G, G, 4 * G, 4).transpose(0, 1, 3, 2, 4)
    else:
        body = wd.reshape(H, R, G, 4, 4).transpose(0, 1, 3, 2, 4)
    sc = scales if not is_v else scales.transpose(0, 2, 1)
    return np.concatenate([np.ascontiguousarray(body).reshape(H, R * D // 2),
                           np.ascontiguousarray(sc).view(np.uint8).reshape(H, -1)], axis=1)


def _unpack_q4_codes(tile, R, D, is_v):
    """Inverse of _pack_q4's code part for one head: codes [R][D]."""
    G = D // 32
    body = tile[:R * D // 2]
    if is_v:
        wd = body.reshape(R // G, 4 * G, G, 4).transpose(0, 2, 1, 3).reshape(R, 4 * G * 4)
    else:
        wd = body.reshape(R, 4, G, 4).transpose(0, 2, 1, 3).reshape(R, 4 * G * 4)
    out = np.empty((R, D), dtype=np.uint8)
    out[:, 0::2] = wd & 15
    out[:, 1::2] = wd >> 4
    return out


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (64, 4, 4)])
def test_q4_decode_equals_fp32_decode_of_the_same_values(D, Hq, Hkv):
    rng = np.random.default_rng(4)
    NB, B = 12, 3
    ctx = np.array([37, 16, 70], dtype=np.int32)
    perm = rng.permutation(NB)
    table = np.full((B, 5), -1, dtype=np.int32)
    k = 0
    for s in range(B):
        n = (ctx[s] + 15) // 16
        table[s, :n] = perm[k:k + n]
        k += n
    kc = rng.integers(0, 16, (NB, Hkv, 16, D)).astype(np.uint8)
    vc = rng.integers(0, 16, (NB, Hkv, 16, D)).astype(np.uint8)
    ks = (rng.uniform(0.05, 0.3, (NB, Hkv, 16, D // 32)) *
          rng.choice([-1, 1], (NB, Hkv, 16, D // 32))).astype(np.float16)
    vs = (rng.uniform(0.05, 0.3, (NB, Hkv, 16, D // 32)) *
          rng.choice([-1, 1], (NB, Hkv, 16, D // 32))).astype(np.float16)
    kq = np.stack([_pack_q4(kc[b], ks[b], False) for b in range(NB)])
    vq = np.stack([_pack_q4(vc[b], vs[b], True) for b in range(NB)])
    kf = (np.repeat(ks.astype(np.float32), 32, axis=3) * (kc.astype(np.float32) - 8))
    vf = (np.repeat(vs.astype(np.float32), 32, axis=3) * (vc.astype(np.float32) - 8))
    q_f32 = rng.standard_normal((B, Hq, D)).astype(np.float32)
    q_bf16 = (q_f32.view(np.uint32) >> 16).astype(np.uint16)
    q_back = (q_bf16.astype(np.uint32) << 16).view(np.float32)
    got = oracle.decode(kq, vq, table, ctx, q_bf16, 0.1, dtype=oracle.Q4_0)
    want = oracle.decode(kf.astype(np.float32), vf.astype(np.float32), table, ctx, q_back, 0.1,
                         dtype=oracle.F32)
    assert np.array_equal(got, want)


def test_q4_append_writes_quantised_row_in_layout():
    rng = np.random.default_rng(5)
    D, Hkv, NB = 128, 2, 6
    tb = oracle.q_tile_bytes(oracle.Q4_0, D)
    kp = rng.integers(0, 256, (NB, Hkv, tb)).astype(np.uint8)
    vp = rng.integers(0, 256, (NB, Hkv, tb)).astype(np.uint8)
    k0, v0 = kp.copy(), vp.copy()
    table = np.array([[3, 1], [4, -1]], dtype=np.int32)
    ctx = np.array([21, 9], dtype=np.int32)   # rows (1, 4) and (4, 8)
    kn = (rng.standard_normal((2, Hkv, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vn = (rng.standard_normal((2, Hkv, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    oracle.append(kp, vp, table, ctx, kn, vn, dtype=oracle.Q4_0)
    for s, (blk, row) in enumerate([(1, 4), (4, 8)]):
        for is_v, (pool, new) in enumerate([(kp, kn), (vp, vn)]):
            x = (new[s].astype(np.uint32) << 16).view(np.float32)
            codes, d = oracle.q4_quantize(x.reshape(-1, 32))
            c = codes.reshape(Hkv, D)
            want = np.concatenate([(c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8),
                                   d.reshape(Hkv, D // 32).view(np.uint8)], axis=1)
            got = ostep.q8_row_bytes(pool, [blk], [row], bool(is_v))[0]
            assert np.array_equal(got, want)
            for h in range(Hkv):  # the same codes read back through this file's layout
                unpacked = _unpack_q4_codes(pool[blk, h], 16, D, bool(is_v))[row]
                assert np.array_equal(unpacked, c[h])
    changed = (kp != k0).sum() + (vp != v0).sum()
    assert changed <= 2 * 2 * Hkv * (D // 2 + 8)
