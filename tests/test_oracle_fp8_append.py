"""Pins of the fp8 encoder and of the quantised append (per-(block, KV head)
scales that grow as a block fills), against a library conversion, closed-form
error bounds and invariants of the scale policy."""
import numpy as np
import pytest
import torch

import oracle
from oracle.fp8 import FP8_MAX
from oracle.quant_cache import append_tile, pow2_ceil
from workloads import bf16_round


def _torch_e4m3(x):
    """torch's float32 -> float8_e4m3fn conversion (round to nearest even), in range."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_encode_matches_torch_conversion_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 40,
        rng.uniform(-448, 448, 100000).astype(np.float32),
        (rng.standard_normal(50000) * 1e-2).astype(np.float32),
        np.array([0.0, -0.0, 448.0, -448.0, 2 ** -9, 2 ** -10, 3 * 2 ** -10], np.float32),
    ])
    assert np.array_equal(oracle.encode_e4m3fn(x), _torch_e4m3(x))


def test_encode_every_bf16_value_in_range():
    """Every bf16 value of magnitude <= 448 (holding every midpoint of E4M3 and the
    values one bf16 step either side of it) encodes as torch's conversion does."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= FP8_MAX)]
    assert np.array_equal(oracle.encode_e4m3fn(x), _torch_e4m3(x))


def test_encode_inverts_decode_and_saturates():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.encode_e4m3fn(oracle.decode_e4m3fn(codes)), codes)
    assert list(oracle.encode_e4m3fn([449.0, 463.9, 1e6, -1e6])) == [0x7E, 0x7E, 0x7E, 0xFE]
    assert oracle.encode_e4m3fn([np.nan])[0] & 0x7F == 0x7F


def _bf16_rows(rng, shape, scale=1.0):
    return bf16_round(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def _f32(bits):
    return oracle.bf16_to_float64(bits).astype(np.float32)


def _quant_bound(x, s):
    """Round-to-nearest error of E4M3 at scale s: half a step, 2^-4 relative in the
    normal range, s * 2^-10 absolute below it."""
    return np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6)


def _pool(rng, nb, h, bs, d):
    """Garbage codes and scales (what a recycled block holds before it opens)."""
    k = rng.integers(0, 0x7E, (nb, h, bs, d), dtype=np.uint8)
    return k, k[::-1].copy(), rng.uniform(1, 5, (nb, h)).astype(np.float32), \
        rng.uniform(1, 5, (nb, h)).astype(np.float32)


def test_pow2_ceil():
    assert pow2_ceil(np.float32(0)) == 0
    for k in range(-140, 120):
        p = np.float32(2.0 ** k)
        assert pow2_ceil(p) == p
        assert pow2_ceil(np.nextafter(p, np.float32(np.inf))) == np.float32(2.0 ** (k + 1))
        if k > -126:
            assert pow2_ceil(np.nextafter(p, np.float32(0))) == p
    assert pow2_ceil(np.float32(3.0)) == 4 and pow2_ceil(np.float32(0.3)) == np.float32(0.5)


def test_a_block_filled_in_one_call():
    """Fresh blocks filled in one call: the scale is the power of two with
    224 < amax / scale <= 448, codes are torch's conversion of x / scale, and
    every value is within half an E4M3 step of x."""
    rng = np.random.default_rng(1)
    nb, H, BS, D = 6, 3, 16, 64
    kp, vp, ks, vs = _pool(rng, nb, H, BS, D)
    k_new, v_new = _bf16_rows(rng, (2, 2 * BS, H, D)), _bf16_rows(rng, (2, 2 * BS, H, D), 3.0)
    tables = np.array([[4, 1], [0, 5]], dtype=np.int32)
    kp2, vp2, ks2, vs2 = oracle.kv_append_fp8(kp, vp, ks, vs, k_new, v_new, tables,
                                              np.array([0, 0]), BS)
    for pool, sc, new in ((kp2, ks2, k_new), (vp2, vs2, v_new)):
        x = _f32(new)
        for b in range(2):
            for i in range(2):
                blk = tables[b, i]
                for h in range(H):
                    rows = x[b, i * BS:(i + 1) * BS, h]
                    s = sc[blk, h]
                    amax = np.float64(np.max(np.abs(rows)))
                    assert np.log2(s) == np.round(np.log2(s)) and 224 < amax / s <= 448
                    expect = _torch_e4m3(np.clip(rows / s, -448, 448))
                    assert np.array_equal(pool[blk, h], expect)
                    deq = oracle.decode_e4m3fn(pool[blk, h]) * np.float64(s)
                    assert np.all(np.abs(deq - rows) <= _quant_bound(rows, s))
    untouched = [2, 3]
    assert np.array_equal(kp2[untouched], kp[untouched]) and np.array_equal(ks2[untouched], ks[untouched])


def test_token_by_token_equals_one_call_when_the_first_token_is_largest():
    """When the block's first token holds its largest |x|, the scale never grows and
    filling the block one token per call gives the same codes as one call."""
    rng = np.random.default_rng(2)
    nb, H, BS, D = 3, 2, 16, 32
    kp, vp, ks, vs = _pool(rng, nb, H, BS, D)
    x = _bf16_rows(rng, (1, BS, H, D))
    x[0, 0, :, 0] = bf16_round(np.full(H, 9.0, np.float32))   # |x| < 9 elsewhere (N(0,1))
    tables = np.array([[2]], dtype=np.int32)
    one = oracle.kv_append_fp8(kp, vp, ks, vs, x, x, tables, np.array([0]), BS)
    state = (kp, vp, ks, vs)
    for t in range(BS):
        state = oracle.kv_append_fp8(*state, x[:, t:t + 1], x[:, t:t + 1], tables,
                                     np.array([t]), BS)
    for a, b in zip(one, state):
        assert np.array_equal(a, b)
    assert state[2][2, 0] == np.float32(2.0 ** -5)            # 9 / 448 rounded up


def test_growing_scale_requantises_older_tokens():
    """Tokens of rising magnitude, one per call: the scale never shrinks and ends at
    what one call gives; older tokens re-encoded after each growth hold exactly the
    one-call codes wherever those are normal E4M3 values, and elsewhere stay within
    the rounding error of each scale they were written or re-encoded at."""
    rng = np.random.default_rng(3)
    nb, H, BS, D = 2, 2, 16, 64
    kp, vp, ks, vs = _pool(rng, nb, H, BS, D)
    x = np.stack([_bf16_rows(rng, (H, D), 1.3 ** t) for t in range(BS)])[None]   # [1][BS][H][D]
    tables = np.array([[1]], dtype=np.int32)
    state, scales = (kp, vp, ks, vs), []
    for t in range(BS):
        state = oracle.kv_append_fp8(*state, x[:, t:t + 1], x[:, t:t + 1], tables,
                                     np.array([t]), BS)
        scales.append(state[2][1].copy())
        if t:
            assert np.all(scales[t] >= scales[t - 1])
    assert np.any(scales[-1] > scales[0])                     # the scale did grow
    one = oracle.kv_append_fp8(kp, vp, ks, vs, x, x, tables, np.array([0]), BS)
    assert np.array_equal(state[2], one[2])
    xf = _f32(x[0])
    for h in range(H):
        normal = (one[0][1, h] & 0x78) != 0                   # exponent field > 0
        got, ref = state[0][1, h], one[0][1, h]
        assert np.array_equal(got[normal], ref[normal])
        deq = oracle.decode_e4m3fn(got) * np.float64(scales[-1][h])
        for t in range(BS):
            err = np.zeros(D)
            for u in range(t, BS):                            # each rounding it went through
                err += np.maximum((np.abs(xf[t, h]) + err) * 2.0 ** -4,
                                  np.float64(scales[u][h]) * 2.0 ** -10)
            assert np.all(np.abs(deq[t] - xf[t, h]) <= err * (1 + 1e-6))


def test_older_codes_are_untouched_without_growth_and_a_new_block_resets():
    rng = np.random.default_rng(4)
    tile = rng.integers(0, 0x7E, (16, 8), dtype=np.uint8)
    rows = np.full((2, 8), 0.5, np.float32)
    out, s = append_tile(tile, np.float32(1.0), 5, rows)          # 0.5/448 < 1: no growth
    assert s == np.float32(1.0)
    assert np.array_equal(out[:5], tile[:5]) and np.array_equal(out[7:], tile[7:])
    assert np.array_equal(out[5:7], oracle.encode_e4m3fn(rows))
    out, s = append_tile(tile, np.float32(1.0), 0, rows)          # the block opens: reset
    assert s == np.float32(2.0 ** -9) and np.all(out[:2] == oracle.encode_e4m3fn([256.0]))
    out, s = append_tile(tile, np.float32(2.0 ** -9), 3, rows * 4)  # grows by 4: exact shift
    assert s == np.float32(2.0 ** -7)
    big = (tile[:3] & 0x78) >= 0x18                               # stays normal after / 4
    assert np.array_equal(oracle.decode_e4m3fn(out[:3])[big] * 4,
                          oracle.decode_e4m3fn(tile[:3])[big])
    out, s = append_tile(tile, np.float32(0.0), 0, np.zeros((1, 8), np.float32))
    assert s == 0 and np.all(out[0] == 0) and np.array_equal(out[1:], tile[1:])


def test_calls_that_span_blocks_and_skips():
    """T tokens that cross a block boundary touch each block with its own first
    slot; negative starts, rows past the table and invalid table entries write
    nothing."""
    rng = np.random.default_rng(5)
    nb, H, BS, D = 8, 2, 16, 32
    kp, vp, ks, vs = _pool(rng, nb, H, BS, D)
    x = _bf16_rows(rng, (4, 5, H, D))
    tables = np.array([[3, 6], [2, -1], [1, 7], [0, 4]], dtype=np.int32)
    start = np.array([13, 14, -1, 30], dtype=np.int64)
    k2, v2, ks2, vs2 = oracle.kv_append_fp8(kp, vp, ks, vs, x, x, tables, start, BS)
    xf = _f32(x)
    # sequence 0: slots 13..15 of block 3 (older tokens in 0..12), slots 0..1 of block 6
    exp3, s3 = append_tile(kp[3, 0], ks[3, 0], 13, xf[0, 0:3, 0])
    exp6, s6 = append_tile(kp[6, 0], ks[6, 0], 0, xf[0, 3:5, 0])
    assert np.array_equal(k2[3, 0], exp3) and ks2[3, 0] == s3
    assert np.array_equal(k2[6, 0], exp6) and ks2[6, 0] == s6
    # sequence 1: block 2 written, logical block 1 is -1; sequence 3: block 4 slots 14, 15 only
    exp2, _ = append_tile(kp[2, 1], ks[2, 1], 14, xf[1, 0:2, 1])
    assert np.array_equal(k2[2, 1], exp2)
    exp4, _ = append_tile(kp[4, 1], ks[4, 1], 14, xf[3, 0:2, 1])
    assert np.array_equal(k2[4, 1], exp4)
    for blk in (1, 5, 7, 0):
        assert np.array_equal(k2[blk], kp[blk]) and np.array_equal(ks2[blk], ks[blk])
    assert np.array_equal(v2[3, 0], append_tile(vp[3, 0], vs[3, 0], 13, xf[0, 0:3, 0])[0])


def test_attention_over_the_appended_cache_tracks_the_bf16_values():
    """Attention over a cache written by the quantised append stays close to
    attention over the bf16 values themselves (fp8 error, not a mistake)."""
    rng = np.random.default_rng(6)
    B, Hq, H, BS, D, L = 2, 8, 2, 16, 64, 100
    nblk = -(-L // BS)
    tables = np.arange(B * nblk, dtype=np.int32).reshape(B, nblk)
    kp = np.zeros((B * nblk, H, BS, D), np.uint8)
    vp, ks, vs = kp.copy(), np.zeros((B * nblk, H), np.float32), np.zeros((B * nblk, H), np.float32)
    k_rows, v_rows = _bf16_rows(rng, (B, L, H, D)), _bf16_rows(rng, (B, L, H, D))
    state = (kp, vp, ks, vs)
    for t0 in range(0, L, 7):                                  # calls of 7 tokens
        t1 = min(L, t0 + 7)
        state = oracle.kv_append_fp8(*state, k_rows[:, t0:t1], v_rows[:, t0:t1], tables,
                                     np.array([t0, t0]), BS)
    q = _bf16_rows(rng, (B, Hq, D))
    ctx = np.array([L, L], dtype=np.int32)
    out8, _ = oracle.paged_decode_attention(q, state[0], state[1], tables, ctx, BS, D ** -0.5,
                                            "fp8", state[2], state[3])
    kb = np.zeros((B * nblk, H, BS, D), np.uint16)
    vb = kb.copy()
    kb, vb = oracle.kv_append_tokens(kb, vb, k_rows, v_rows, tables,
                                     np.tile(np.arange(L), (B, 1)), BS)
    out16, _ = oracle.paged_decode_attention(q, kb, vb, tables, ctx, BS, D ** -0.5)
    rel = np.linalg.norm(out8 - out16) / np.linalg.norm(out16)
    assert rel < 0.08, rel
