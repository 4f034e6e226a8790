"""Pins of the KIVI scale layout (keys scaled per channel of each (block, KV
head), values per token): attention by brute force, reduction to the
per-(block, head) layout, the append's per-channel and per-token scales, and the
layout's purpose, smaller key error when a few channels carry outliers."""
import math

import numpy as np
import torch

import oracle
from oracle.quant_cache import append_tile
from workloads import bf16_round, make_case, small_spec


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _bf16(rng, shape, scale=1.0):
    return bf16_round((rng.standard_normal(shape) * scale).astype(np.float32))


def _f32(bits):
    return oracle.bf16_to_float64(bits).astype(np.float32)


def test_kivi_attention_by_brute_force():
    """Scalar loops: every key element decoded times its channel's scale, every
    value element times its token's scale, then softmax-weighted sums."""
    spec = small_spec(num_seqs=2, num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=4,
                      kv_dtype="fp8_kivi", context=9, case_id=9900)
    case = make_case(spec, seed=1, context_lens=[9, 6])
    out, lse = oracle.paged_decode_attention(case["q"], case["k_pool_full"], case["v_pool_full"],
                                             case["block_tables"], case["context_lens"], 4,
                                             0.5, "fp8_kivi", case["k_scale"], case["v_scale"])
    dec = oracle.decode_e4m3fn
    for b in range(2):
        ctx = int(case["context_lens"][b])
        for h in range(4):
            g = h // 2
            qv = [float(x) for x in oracle.bf16_to_float64(case["q"][b, h])]
            scores, vals = [], []
            for t in range(ctx):
                blk, slot = int(case["block_tables"][b, t // 4]), t % 4
                kt = [float(dec(case["k_pool_full"][blk, g, slot, d])) * float(case["k_scale"][blk, g, d])
                      for d in range(8)]
                vt = [float(dec(case["v_pool_full"][blk, g, slot, d])) * float(case["v_scale"][blk, g, slot])
                      for d in range(8)]
                scores.append(0.5 * sum(a * c for a, c in zip(qv, kt)))
                vals.append(vt)
            m = max(scores)
            e = [math.exp(x - m) for x in scores]
            z = sum(e)
            ref = [sum(e[t] * vals[t][d] for t in range(ctx)) / z for d in range(8)]
            assert np.allclose(out[b, h], ref, rtol=0, atol=1e-12)
            assert abs(lse[b, h] - (m + math.log(z))) < 1e-12


def test_uniform_kivi_scales_reduce_to_block_scales():
    spec = small_spec(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=16, block_size=8,
                      kv_dtype="fp8", context=40, case_id=9901)
    case = make_case(spec, seed=2, context_lens=[40, 23])
    ks, vs = case["k_scale"], case["v_scale"]
    ks_kivi = np.repeat(ks[:, :, None], 16, axis=2)
    vs_kivi = np.repeat(vs[:, :, None], 8, axis=2)
    args = (case["q"], case["k_pool_full"], case["v_pool_full"], case["block_tables"],
            case["context_lens"], 8, 0.25)
    a = oracle.paged_decode_attention(*args, "fp8", ks, vs)
    b = oracle.paged_decode_attention(*args, "fp8_kivi", ks_kivi, vs_kivi)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    mq = oracle.paged_multi_query_attention(case["q"][:, None], *args[1:], "fp8_kivi", ks_kivi,
                                            vs_kivi)
    assert np.array_equal(mq[0][:, 0], b[0])


def _kivi_pool(rng, nb, h, bs, d):
    k = rng.integers(0, 0x7E, (nb, h, bs, d), dtype=np.uint8)
    return (k, k[::-1].copy(), rng.uniform(1, 5, (nb, h, d)).astype(np.float32),
            rng.uniform(1, 5, (nb, h, bs)).astype(np.float32))


def test_kivi_append_one_call_scales_and_codes():
    """A block filled in one call: each key channel's scale is the power of two
    with 224 < amax_d / s_d <= 448, each value token's likewise over its row, and
    every code is torch's conversion of x / its scale."""
    rng = np.random.default_rng(3)
    nb, H, BS, D = 4, 2, 16, 32
    kp, vp, ks, vs = _kivi_pool(rng, nb, H, BS, D)
    k_new = _bf16(rng, (1, BS, H, D)) * 1
    k_new = bf16_round((_f32(k_new) * np.float32(3.0) ** np.arange(D, dtype=np.float32) % 7 + 0.1)
                       .astype(np.float32))
    v_new = _bf16(rng, (1, BS, H, D), 2.0)
    tables = np.array([[2]], dtype=np.int32)
    k2, v2, ks2, vs2 = oracle.kv_append_fp8(kp, vp, ks, vs, k_new, v_new, tables, np.array([0]),
                                            BS, layout="kivi")
    xk, xv = _f32(k_new[0]), _f32(v_new[0])
    for h in range(H):
        for d in range(D):
            s = ks2[2, h, d]
            amax = np.max(np.abs(xk[:, h, d]))
            assert np.log2(s) == round(np.log2(s)) and 224 < amax / s <= 448
            assert np.array_equal(k2[2, h, :, d], _torch_e4m3(np.clip(xk[:, h, d] / s, -448, 448)))
        for t in range(BS):
            s = vs2[2, h, t]
            amax = np.max(np.abs(xv[t, h]))
            assert np.log2(s) == round(np.log2(s)) and 224 < amax / s <= 448
            assert np.array_equal(v2[2, h, t], _torch_e4m3(np.clip(xv[t, h] / s, -448, 448)))
    others = [0, 1, 3]
    assert np.array_equal(k2[others], kp[others]) and np.array_equal(ks2[others], ks[others])
    assert np.array_equal(vs2[others], vs[others])


def test_kivi_key_channels_grow_independently():
    """Tokens one per call where only channel 0 grows: channel 0's scale grows and
    its older codes are re-encoded; every other channel keeps its first scale and
    codes; the result equals filling the block in one call."""
    rng = np.random.default_rng(4)
    nb, H, BS, D = 2, 1, 16, 16
    kp, vp, ks, vs = _kivi_pool(rng, nb, H, BS, D)
    x = _f32(_bf16(rng, (1, BS, H, D)))
    x[0, :, 0, 1:] = np.clip(x[0, :, 0, 1:], -1, 1)
    x[0, 0, 0, 1:] = 4.0                                      # largest of channels 1.. at token 0
    x[0, :, 0, 0] = (2.0 ** np.arange(BS)).astype(np.float32) / 64   # channel 0 keeps rising
    bits = bf16_round(x)
    tables = np.array([[1]], dtype=np.int32)
    state = (kp, vp, ks, vs)
    firsts = None
    for t in range(BS):
        state = oracle.kv_append_fp8(*state, bits[:, t:t + 1], bits[:, t:t + 1], tables,
                                     np.array([t]), BS, layout="kivi")
        if t == 0:
            firsts = state[2][1, 0].copy()
        assert np.array_equal(state[2][1, 0, 1:], firsts[1:])
    assert state[2][1, 0, 0] > firsts[0]
    one = oracle.kv_append_fp8(kp, vp, ks, vs, bits, bits, tables, np.array([0]), BS,
                               layout="kivi")
    for a, b in zip(one, state):
        assert np.array_equal(a, b)


def test_kivi_tile_rule_is_the_block_rule_per_column_and_row():
    """The KIVI append of one tile equals the per-(block, head) rule applied to each
    key column and to each value row on its own (written with explicit slicing)."""
    rng = np.random.default_rng(5)
    BS, D = 16, 8
    tile = rng.integers(0, 0x7E, (BS, D), dtype=np.uint8)
    kscale = (2.0 ** rng.integers(-8, -2, D)).astype(np.float32)
    rows = _f32(_bf16(rng, (5, D), 0.5))
    first = 6
    state = oracle.kv_append_fp8(tile[None, None], tile[None, None], kscale[None, None],
                                 np.ones((1, 1, BS), np.float32), bf16_round(rows)[None, :, None],
                                 bf16_round(rows)[None, :, None], np.array([[0]]),
                                 np.array([first]), BS, layout="kivi")
    for d in range(D):
        col, s = append_tile(tile[:, [d]], kscale[d], first, rows[:, [d]])
        assert np.array_equal(state[0][0, 0, :, d], col[:, 0]) and state[2][0, 0, d] == s
    for j in range(5):
        row, s = append_tile(tile[[first + j]], np.float32(1), 0, rows[[j]])
        assert np.array_equal(state[1][0, 0, first + j], row[0]) and state[3][0, 0, first + j] == s
    assert np.array_equal(state[1][0, 0, :first], tile[:first])


def test_kivi_keys_hold_outlier_channels_better():
    """Keys whose few channels carry outliers (as the page's KIVI remark says key
    statistics do).  E4M3 is a floating-point code: its relative precision does
    not depend on the scale, so one scale per block loses accuracy only when the
    channels span more than its normal range (about 2^15) and the small ones fall
    to subnormals.  With outliers 2^14 times larger, per-channel scales keep the
    other channels' error far smaller, and attention over the KIVI cache is
    closer to attention over the bf16 values; with outliers 40 times larger the
    two layouts are equally accurate."""
    rng = np.random.default_rng(6)
    B, Hq, H, BS, D, L = 1, 4, 1, 16, 64, 96
    nblk = L // BS
    tables = np.arange(nblk, dtype=np.int32)[None]
    base = _f32(_bf16(rng, (B, L, H, D)))
    v_bits = _bf16(rng, (B, L, H, D))
    err_b, err_k = _key_errors(base, 40.0, v_bits, L, BS, D, H)
    assert abs(err_k - err_b) < 0.05 * err_b, (err_k, err_b)   # moderate outliers: no gain
    k = base.copy()
    k[..., :3] *= np.float32(2.0 ** 14)                       # three extreme outlier channels
    k_bits = bf16_round(k)
    zeros8 = np.zeros((nblk, H, BS, D), np.uint8)
    blk = oracle.kv_append_fp8(zeros8, zeros8, np.zeros((nblk, H), np.float32),
                               np.zeros((nblk, H), np.float32), k_bits, v_bits, tables,
                               np.array([0]), BS)
    kiv = oracle.kv_append_fp8(zeros8, zeros8, np.zeros((nblk, H, D), np.float32),
                               np.zeros((nblk, H, BS), np.float32), k_bits, v_bits, tables,
                               np.array([0]), BS, layout="kivi")
    ctx = np.array([L], np.int32)
    err_b, err_k = _key_errors(base, 2.0 ** 14, v_bits, L, BS, D, H)
    assert err_k < 0.5 * err_b, (err_k, err_b)
    q = _bf16(rng, (B, Hq, D), 0.1)
    zb = np.zeros((nblk, H, BS, D), np.uint16)
    kr, vr = oracle.kv_append_tokens(zb, zb, k_bits, v_bits, tables, np.arange(L)[None], BS)
    ref, _ = oracle.paged_decode_attention(q, kr, vr, tables, ctx, BS, D ** -0.5)
    ob, _ = oracle.paged_decode_attention(q, blk[0], blk[1], tables, ctx, BS, D ** -0.5, "fp8",
                                          blk[2], blk[3])
    ok, _ = oracle.paged_decode_attention(q, kiv[0], kiv[1], tables, ctx, BS, D ** -0.5,
                                          "fp8_kivi", kiv[2], kiv[3])
    assert np.linalg.norm(ok - ref) < np.linalg.norm(ob - ref)


def _key_errors(base, factor, v_bits, L, BS, D, H):
    """Mean |dequantised - true| over the non-outlier key channels, per-(block,
    head) scales against KIVI scales, with channels 0..2 multiplied by factor."""
    k = base.copy()
    k[..., :3] *= np.float32(factor)
    k_bits = bf16_round(k)
    kx = np.transpose(_f32(k_bits)[0], (1, 0, 2)).astype(np.float64)
    nblk = L // BS
    tables = np.arange(nblk, dtype=np.int32)[None]
    zeros8 = np.zeros((nblk, H, BS, D), np.uint8)
    blk = oracle.kv_append_fp8(zeros8, zeros8, np.zeros((nblk, H), np.float32),
                               np.zeros((nblk, H), np.float32), k_bits, v_bits, tables,
                               np.array([0]), BS)
    kiv = oracle.kv_append_fp8(zeros8, zeros8, np.zeros((nblk, H, D), np.float32),
                               np.zeros((nblk, H, BS), np.float32), k_bits, v_bits, tables,
                               np.array([0]), BS, layout="kivi")
    kb = oracle.attention.dequantized_rows(blk[0], tables[0], L, BS, "fp8", blk[2], "k")
    kk = oracle.attention.dequantized_rows(kiv[0], tables[0], L, BS, "fp8_kivi", kiv[2], "k")
    return np.abs(kb - kx)[..., 3:].mean(), np.abs(kk - kx)[..., 3:].mean()
