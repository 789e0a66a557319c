"""Pins of the oracle's q8_0 cache (no GPU).

The pages name q8_0 as the cache type that about halves an f16 cache
(ssdnodes.com, "KV cache vs prompt cache", "Four ways to make the KV cache
smaller", item 2); it is read as llama.cpp's Q8_0 block: per 32 consecutive
elements one fp16 scale d = max|x| / 127 and int8 codes round(x / d), value
d * code. These tests hold the oracle to that definition through cases whose
answer is known without it: exact grids, rounding ties, independent groups,
the error bound, numpy's own fp16 rounding, and attention over the same
values stored as fp32.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import step as ostep

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_sizes.json")


def test_q8_row_is_about_half_of_f16():
    g = json.load(open(GOLDEN))["quantised_cache_q8_0"]
    per_token = 2 * g["layers"] * g["kv_heads"] * oracle.q8_tile_bytes(g["head_dim"]) // 16
    assert per_token == 69632  # 128 codes + 4 fp16 scales per row, 32 layers x 8 heads x K,V
    frac = per_token / g["f16_bytes_per_token"]
    assert abs(frac - g["q8_0_approx_fraction_of_f16"]) < 0.05


def test_float_to_half_matches_numpy():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(20000) * 2.0 ** rng.integers(-30, 17, 20000)).astype(np.float32),
        np.float32([0.0, -0.0, 65504, 65519.99, 65520, 1e9, -1e9, 2 ** -24, 2 ** -25,
                    3 * 2 ** -26, 2 ** -14, 2 ** -14 - 2 ** -25, np.inf, -np.inf]),
        # exact ties between two halves: midpoints of consecutive fp16 values
        ((np.arange(1, 2000, dtype=np.float64) * 2 + 1) * 2.0 ** -11).astype(np.float32),
    ])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = oracle.float_to_half_bits(x)
    assert np.array_equal(got, want)
    nan = oracle.float_to_half_bits(np.float32([np.nan]))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0


def test_q8_exact_grid():
    # x = m * 2^-7 with integer m in [-127, 127] and |m| = 127 present:
    # d = 127 * 2^-7 / 127 = 2^-7 exactly, codes = m exactly, value = x exactly
    rng = np.random.default_rng(1)
    m = rng.integers(-127, 128, size=(50, 32))
    m[:, 0] = np.where(rng.random(50) < 0.5, 127, -127)
    x = (m * 2.0 ** -7).astype(np.float32)
    codes, d = oracle.q8_quantize(x)
    assert np.array_equal(codes, m.astype(np.int8))
    assert np.all(d == np.float16(2.0 ** -7).view(np.uint16))
    recon = d.view(np.float16).astype(np.float64)[:, None] * codes
    assert np.array_equal(recon, x.astype(np.float64))


def test_q8_rounds_half_away_from_zero():
    # d = 2^-7 (one element at 127 * 2^-7); x / d = k + 0.5 exactly
    x = np.zeros(32, dtype=np.float32)
    x[0] = 127 * 2.0 ** -7
    halves = [0.5, 1.5, 2.5, -0.5, -2.5, 126.5]
    x[1:1 + len(halves)] = np.float32(halves) * np.float32(2.0 ** -7)
    codes, _ = oracle.q8_quantize(x)
    assert codes[0, 1:1 + len(halves)].tolist() == [1, 2, 3, -1, -3, 127]


def test_q8_zero_group():
    codes, d = oracle.q8_quantize(np.zeros((2, 32), dtype=np.float32))
    assert not codes.any() and not d.any()


def test_q8_groups_are_32_consecutive_values():
    # one row of 128: group k is the same pattern times 2^k, so every group
    # gets the same codes and a scale 2^k times the first
    rng = np.random.default_rng(2)
    base = rng.standard_normal(32).astype(np.float32)
    row = np.concatenate([base * np.float32(2.0 ** k) for k in range(4)])
    codes, d = oracle.q8_quantize(row)
    for k in range(1, 4):
        assert np.array_equal(codes[k], codes[0])
    dv = d.view(np.float16).astype(np.float64)
    assert np.allclose(dv[1:] / dv[:-1], 2.0, rtol=2e-3)
    # and is not what groups of 16 or 64 would give
    amax = np.abs(row).reshape(4, 32).max(axis=1)
    assert np.allclose(dv, amax / 127, rtol=1e-3)


def test_q8_error_bound_random():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((4000, 32)) * 10.0 ** rng.uniform(-3, 3, (4000, 1))).astype(np.float32)
    codes, d = oracle.q8_quantize(x)
    dq = d.view(np.float16).astype(np.float64)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    dexact = amax / 127
    assert np.all(np.abs(codes).max(axis=1) == 127)
    assert np.all(np.abs(codes.astype(np.int32)) <= 127)
    err = np.abs(x - dq[:, None] * codes)
    # x * (1/d) is rounded to fp32 before the integer decision: up to 127 * 2^-23
    # code units beyond the half-unit bound, then the fp16 rounding of d
    bound = (0.5 + 2e-5) * dexact[:, None] + np.abs(codes) * np.abs(dq - dexact)[:, None]
    assert np.all(err <= bound)
    assert np.array_equal(codes[:100], -oracle.q8_quantize(-x[:100])[0])


def _lane_image_q8(codes, is_v):
    """Code bytes of one 16-row q8_0 tile [16][D] as the decode's 64 lanes read
    them, built lane by lane: 16-byte unit c of lane L at c*1024 + L*16.
    K: lane L = 16*quarter + token holds its token's quarter of groups 2c and
    2c + 1 (8 codes each); V: lane L = (D/8)*v + chunk holds that chunk of rows
    NV*v + 2c and NV*v + 2c + 1 (NV = D/32)."""
    R, D = codes.shape
    P, G = D // 8, D // 32
    out = np.zeros(R * D, dtype=np.uint8)
    raw = codes.view(np.uint8)
    for c in range(G // 2):
        for lane in range(64):
            if is_v:
                chunk, v = lane % P, lane // P
                rows = (G * v + 2 * c, G * v + 2 * c + 1)
                unit = np.concatenate([raw[r, 8 * chunk:8 * chunk + 8] for r in rows])
            else:
                tok, quarter = lane % 16, lane // 16
                unit = np.concatenate([raw[tok, 32 * k + 8 * quarter:32 * k + 8 * quarter + 8]
                                       for k in (2 * c, 2 * c + 1)])
            out[c * 1024 + lane * 16:c * 1024 + lane * 16 + 16] = unit
    return out


def _pack_q8(codes, scales, is_v):
    """One tile [Hkv] of q8_0 bytes from codes [Hkv][16][D] and fp16 scales
    [Hkv][16][D/32], in the documented order (codes as the decode's lanes read
    them; scales K: [row][group], V: [group][row])."""
    H, R, D = codes.shape
    sc = scales if not is_v else scales.transpose(0, 2, 1)
    return np.concatenate([np.stack([_lane_image_q8(codes[h], is_v) for h in range(H)]),
                           np.ascontiguousarray(sc).view(np.uint8).reshape(H, -1)], axis=1)


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (64, 4, 4)])
def test_q8_decode_equals_fp32_decode_of_the_same_values(D, Hq, Hkv):
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
    kc = rng.integers(-127, 128, (NB, Hkv, 16, D)).astype(np.int8)
    vc = rng.integers(-127, 128, (NB, Hkv, 16, D)).astype(np.int8)
    ks = rng.uniform(0.005, 0.03, (NB, Hkv, 16, D // 32)).astype(np.float16)
    vs = rng.uniform(0.005, 0.03, (NB, Hkv, 16, D // 32)).astype(np.float16)
    kq = np.stack([_pack_q8(kc[b], ks[b], False) for b in range(NB)])
    vq = np.stack([_pack_q8(vc[b], vs[b], True) for b in range(NB)])
    kf = (np.repeat(ks.astype(np.float32), 32, axis=3) * kc).astype(np.float32)
    vf = (np.repeat(vs.astype(np.float32), 32, axis=3) * vc).astype(np.float32)
    q_f32 = rng.standard_normal((B, Hq, D)).astype(np.float32)
    q_bf16 = (q_f32.view(np.uint32) >> 16).astype(np.uint16)       # truncation: any bf16 will do
    q_back = (q_bf16.astype(np.uint32) << 16).view(np.float32)
    got = oracle.decode(kq, vq, table, ctx, q_bf16, 0.1, dtype=oracle.Q8_0)
    want = oracle.decode(kf, vf, table, ctx, q_back, 0.1, dtype=oracle.F32)
    assert np.array_equal(got, want)


def test_q8_append_writes_quantised_row_in_layout():
    rng = np.random.default_rng(5)
    D, Hkv, NB = 128, 2, 6
    tb = oracle.q8_tile_bytes(D)
    kp = rng.integers(0, 256, (NB, Hkv, tb)).astype(np.uint8)
    vp = rng.integers(0, 256, (NB, Hkv, tb)).astype(np.uint8)
    k0, v0 = kp.copy(), vp.copy()
    table = np.array([[3, 1], [4, -1]], dtype=np.int32)
    ctx = np.array([21, 9], dtype=np.int32)   # rows (1, 4) and (4, 8)
    kn_f = rng.standard_normal((2, Hkv, D)).astype(np.float32)
    vn_f = rng.standard_normal((2, Hkv, D)).astype(np.float32)
    kn = (kn_f.view(np.uint32) >> 16).astype(np.uint16)
    vn = (vn_f.view(np.uint32) >> 16).astype(np.uint16)
    oracle.append(kp, vp, table, ctx, kn, vn, dtype=oracle.Q8_0)
    for s, (blk, row) in enumerate([(1, 4), (4, 8)]):
        for is_v, (pool, new) in enumerate([(kp, kn), (vp, vn)]):
            x = (new[s].astype(np.uint32) << 16).view(np.float32)   # [Hkv][D]
            codes, d = oracle.q8_quantize(x.reshape(-1, 32))
            got = ostep.q8_row_bytes(pool, [blk], [row], bool(is_v))[0]
            want = np.concatenate([codes.reshape(Hkv, D).view(np.uint8),
                                   d.reshape(Hkv, D // 32).view(np.uint8)], axis=1)
            assert np.array_equal(got, want)
    # nothing else changed: 2 rows x (D codes + 8 scale bytes) per head
    changed = (kp != k0).sum() + (vp != v0).sum()
    assert changed <= 2 * 2 * Hkv * (D + 8)
    for is_v, (pool, before) in enumerate([(kp, k0), (vp, v0)]):
        mask = np.zeros_like(pool, dtype=bool)
        for blk, row in [(1, 4), (4, 8)]:
            # the row's codes, placed as the lanes read them (built independently)
            image = _lane_image_q8(np.full((16, D), 0, dtype=np.int8), bool(is_v))
            marker = np.zeros((16, D), dtype=np.int8)
            marker[row] = 1
            mask[blk, :, :16 * D] |= (_lane_image_q8(marker, bool(is_v)) != image)[None, :]
            for grp in range(D // 32):
                i = 16 * D + 2 * (grp * 16 + row if is_v else row * (D // 32) + grp)
                mask[blk, :, i:i + 2] = True
        assert np.array_equal(pool[~mask], before[~mask])
