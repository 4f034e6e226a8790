"""GPU checks of the fp8 KV append (E4M3 codes with one power-of-two scale per
(block, KV head), grown and re-encoded as a block fills): codes and scales
bit-exact against the oracle, every bf16 value's encoding, and decode steps
that append then attend over the fp8 cache."""
import numpy as np
import pytest
import torch

import oracle
from tests._dev import assert_parity
from workloads import bf16_round, make_case, small_spec

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _rows(rng, shape, scales):
    x = rng.standard_normal(shape).astype(np.float32) * np.asarray(scales, np.float32)
    return bf16_round(x)


def _bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def _u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def _i32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _run(gpu, kp, vp, ks, vs, k_new, v_new, tables, start):
    kd, vd, ksd, vsd = _u8_dev(kp), _u8_dev(vp), _f32_dev(ks), _f32_dev(vs)
    gpu.kv_append_fp8(_bf16_dev(k_new), _bf16_dev(v_new), kd, vd, ksd, vsd, _i32_dev(tables),
                      _i32_dev(start))
    torch.cuda.synchronize()
    return kd.cpu().numpy(), vd.cpu().numpy(), ksd.cpu().numpy(), vsd.cpu().numpy()


def _assert_same(got, ref, label):
    names = ("k codes", "v codes", "k scales", "v scales")
    for g, r, n in zip(got, ref, names):
        if n.endswith("scales"):
            assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"{label}: {n}"
        else:
            bad = np.argwhere(g != r)
            assert bad.size == 0, f"{label}: {n} differ at {bad[:5].tolist()} ({len(bad)} total)"


@pytest.mark.parametrize("hkv,d,bs,T,seed", [
    (8, 128, 16, 1, 0), (8, 128, 16, 4, 1), (2, 64, 32, 7, 2), (40, 128, 16, 1, 3),
    (1, 64, 16, 40, 4), (8, 128, 32, 33, 5),
])
def test_fp8_append_is_bit_exact(gpu, hkv, d, bs, T, seed):
    """Garbage pools and scales (recycled blocks), ragged starts: opening blocks,
    appending into partial blocks with and without growth, crossing blocks,
    skipped sequences and positions past the table."""
    rng = np.random.default_rng(seed)
    B, max_blocks = 9, 6
    nb = B * max_blocks + 3
    kp = rng.integers(0, 0x7E, (nb, hkv, bs, d), dtype=np.uint8)
    vp = rng.integers(0, 0x7E, (nb, hkv, bs, d), dtype=np.uint8)
    ks = (2.0 ** rng.integers(-9, -2, (nb, hkv))).astype(np.float32)
    vs = rng.uniform(0.001, 0.02, (nb, hkv)).astype(np.float32)        # not powers of two
    tables = rng.permutation(nb)[:B * max_blocks].astype(np.int32).reshape(B, max_blocks)
    tables[3, 1] = -1
    cap = max_blocks * bs
    start = rng.integers(0, cap - T + 1, B).astype(np.int32)
    start[0], start[1], start[2] = 0, -1, bs - 1
    start[4] = cap - 1                                                 # tail past the table
    mags = 2.0 ** rng.uniform(-3, 4, (B, T, hkv, 1))                   # growth in some tiles
    k_new, v_new = _rows(rng, (B, T, hkv, d), mags), _rows(rng, (B, T, hkv, d), mags[::-1])
    ref = oracle.kv_append_fp8(kp, vp, ks, vs, k_new, v_new, tables, start, bs)
    got = _run(gpu, kp, vp, ks, vs, k_new, v_new, tables, start)
    _assert_same(got, ref, f"hkv={hkv} d={d} bs={bs} T={T}")


def test_every_bf16_value_encodes_as_the_oracle_does(gpu):
    """Blocks whose largest |x| is 448 get scale 1, so each code is the E4M3
    encoding of the bf16 value itself: every bf16 value of magnitude <= 448."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    keep = np.isfinite(x) & (np.abs(x) <= 448)
    vals = bits[keep].astype(np.uint16)
    bs, d = 16, 128
    per_block = bs * d - 1
    nblk = -(-len(vals) // per_block)
    rows = np.zeros((nblk, per_block + 1), dtype=np.uint16)
    flat = np.zeros(nblk * per_block, dtype=np.uint16)
    flat[:len(vals)] = vals
    rows[:, 1:] = flat.reshape(nblk, per_block)
    rows[:, 0] = bf16_round(np.array([448.0], np.float32))[0]
    new = rows.reshape(1, nblk * bs, 1, d)
    tables = np.arange(nblk, dtype=np.int32)[None]
    kp = np.zeros((nblk, 1, bs, d), np.uint8)
    ks = np.zeros((nblk, 1), np.float32)
    got = _run(gpu, kp, kp, ks, ks, new, new, tables, np.array([0]))
    assert np.all(got[2] == 1.0)
    expect = oracle.encode_e4m3fn(oracle.bf16_to_float64(new).astype(np.float32)).reshape(
        nblk, 1, bs, d)
    bad = np.argwhere(got[0] != expect)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:3].tolist()}"
    assert np.array_equal(got[1], got[0])


@pytest.mark.parametrize("hq,hkv,d,bs", [(40, 40, 128, 16), (32, 8, 128, 16), (16, 4, 64, 32)])
def test_decode_steps_append_then_attend(gpu, hq, hkv, d, bs):
    """Twenty decode steps on an fp8 cache that starts as a quantised prefix (scales
    amax / 448 from the workload generator): each step appends one token per
    sequence and attends; pools match the oracle bit for bit after every append
    and attention matches the oracle on them."""
    lens = [300, 17, 64, 1000]
    spec = small_spec(num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                      block_size=bs, kv_dtype="fp8", context=1100, pool="oversized2x",
                      case_id=9500 + hq + bs)
    case = make_case(spec, seed=7, context_lens=lens)
    steps = 20
    B = len(lens)
    nb = case["k_pool_full"].shape[0]
    tables = case["block_tables"]
    # give every sequence room for the new tokens from the pool's free blocks
    used = set(tables[tables >= 0].tolist())
    free = [i for i in range(nb) if i not in used]
    extra = -(-(max(lens) + steps) // bs)
    grown = np.full((B, extra), -1, dtype=np.int32)
    grown[:, :tables.shape[1]] = tables
    for b in range(B):
        for i in range(-(-lens[b] // bs), -(-(lens[b] + steps) // bs)):
            grown[b, i] = free.pop()
    state = (case["k_pool_full"], case["v_pool_full"], case["k_scale"], case["v_scale"])
    dev = [_u8_dev(state[0]), _u8_dev(state[1]), _f32_dev(state[2]), _f32_dev(state[3])]
    td = _i32_dev(grown)
    rng = np.random.default_rng(hq + bs)
    ctx = np.array(lens, dtype=np.int32)
    for step in range(steps):
        mags = 2.0 ** rng.uniform(-1, 2, (B, 1, hkv, 1))
        k_new, v_new = _rows(rng, (B, 1, hkv, d), mags), _rows(rng, (B, 1, hkv, d), mags)
        q = _rows(rng, (B, hq, d), 1.0)
        state = oracle.kv_append_fp8(*state, k_new, v_new, grown, ctx, bs)
        gpu.kv_append_fp8(_bf16_dev(k_new), _bf16_dev(v_new), *dev, td, _i32_dev(ctx))
        ctx = ctx + 1
        out, lse = gpu.paged_decode_attention(_bf16_dev(q), dev[0], dev[1], td, _i32_dev(ctx),
                                              int(ctx.max()), d ** -0.5, dev[2], dev[3])
        torch.cuda.synchronize()
        got = tuple(t.cpu().numpy() for t in dev)
        _assert_same(got, state, f"step {step}")
        ref, ref_lse = oracle.paged_decode_attention(q, state[0], state[1], grown, ctx, bs,
                                                     d ** -0.5, "fp8", state[2], state[3])
        assert_parity(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                      ref, ref_lse, f"step {step}")


def _fp8_case_with_room(hq, hkv, d, bs, lens, extra_tokens, case_id, seed=7):
    """An fp8 workload (quantised prefix, scales amax / 448) whose tables also name
    free pool blocks for the next extra_tokens tokens of every sequence."""
    spec = small_spec(num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                      block_size=bs, kv_dtype="fp8", context=max(lens), pool="oversized2x",
                      case_id=case_id)
    case = make_case(spec, seed=seed, context_lens=lens)
    nb = case["k_pool_full"].shape[0]
    tables = case["block_tables"]
    used = set(tables[tables >= 0].tolist())
    free = [i for i in range(nb) if i not in used]
    grown = np.full((len(lens), -(-(max(lens) + extra_tokens) // bs)), -1, dtype=np.int32)
    grown[:, :tables.shape[1]] = tables
    for b, n in enumerate(lens):
        for i in range(-(-n // bs), -(-(n + extra_tokens) // bs)):
            grown[b, i] = free.pop()
    state = (case["k_pool_full"], case["v_pool_full"], case["k_scale"], case["v_scale"])
    return state, grown


@pytest.mark.parametrize("hq,hkv,d,bs", [(40, 40, 128, 16), (32, 8, 128, 16), (16, 4, 64, 32),
                                         (8, 1, 128, 16), (64, 8, 128, 32), (64, 8, 64, 16)])
def test_fused_fp8_append_attention(gpu, hq, hkv, d, bs):
    """Twelve fused steps (quantise the new token into the cache and attend, one
    kernel) with ragged lengths: codes and scales bit-exact against the oracle's
    append after every step, attention within the parity bar over them."""
    lens = [700, 17, 63, 4000, 1]
    steps = 12
    state, grown = _fp8_case_with_room(hq, hkv, d, bs, lens, steps, 9600 + hq + bs)
    dev = [_u8_dev(state[0]), _u8_dev(state[1]), _f32_dev(state[2]), _f32_dev(state[3])]
    td = _i32_dev(grown)
    rng = np.random.default_rng(hq * 3 + bs)
    B = len(lens)
    ctx = np.array(lens, dtype=np.int32)
    for step in range(steps):
        mags = 2.0 ** rng.uniform(-2, 3, (B, 1, hkv, 1))
        k_new, v_new = _rows(rng, (B, 1, hkv, d), mags), _rows(rng, (B, 1, hkv, d), mags)
        q = _rows(rng, (B, hq, d), 1.0)
        state = oracle.kv_append_fp8(*state, k_new, v_new, grown, ctx, bs)
        pos = ctx.copy()
        ctx = ctx + 1
        out, lse = gpu.paged_decode_append_attention(
            _bf16_dev(q), _bf16_dev(k_new[:, 0]), _bf16_dev(v_new[:, 0]), _i32_dev(pos),
            dev[0], dev[1], td, _i32_dev(ctx), int(ctx.max()), d ** -0.5,
            k_scale=dev[2], v_scale=dev[3])
        torch.cuda.synchronize()
        _assert_same(tuple(t.cpu().numpy() for t in dev), state, f"fused step {step}")
        ref, ref_lse = oracle.paged_decode_attention(q, state[0], state[1], grown, ctx, bs,
                                                     d ** -0.5, "fp8", state[2], state[3])
        assert_parity(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                      ref, ref_lse, f"fused step {step}")


@pytest.mark.parametrize("hq,hkv,d,bs,nq", [(32, 8, 128, 16, 2), (16, 4, 64, 32, 2),
                                            (8, 8, 128, 16, 8), (40, 40, 128, 16, 4),
                                            (8, 8, 128, 32, 8), (16, 8, 64, 32, 3),
                                            (64, 8, 128, 32, 4), (32, 8, 128, 16, 4)])
def test_fused_fp8_multi_query_append(gpu, hq, hkv, d, bs, nq):
    """Verification steps on an fp8 cache: Q new tokens per sequence quantised into
    the cache (possibly across a block boundary) and attended for all Q positions in
    one kernel; bit-exact pools, parity on every position.  With 8 rows a wave
    chunk is 16 tokens, so a 32-token block is read by two waves."""
    lens = [500, 30, 4100, 9]
    steps = 5
    state, grown = _fp8_case_with_room(hq, hkv, d, bs, lens, steps * nq, 9700 + hq + nq)
    dev = [_u8_dev(state[0]), _u8_dev(state[1]), _f32_dev(state[2]), _f32_dev(state[3])]
    td = _i32_dev(grown)
    rng = np.random.default_rng(hq + nq)
    B = len(lens)
    ctx = np.array(lens, dtype=np.int32)
    for step in range(steps):
        mags = 2.0 ** rng.uniform(-2, 3, (B, nq, hkv, 1))
        k_new, v_new = _rows(rng, (B, nq, hkv, d), mags), _rows(rng, (B, nq, hkv, d), mags)
        q = _rows(rng, (B, nq, hq, d), 1.0)
        state = oracle.kv_append_fp8(*state, k_new, v_new, grown, ctx, bs)
        ctx = ctx + nq
        out, lse = gpu.paged_decode_multi_query_append(
            _bf16_dev(q), _bf16_dev(k_new), _bf16_dev(v_new), dev[0], dev[1], td, _i32_dev(ctx),
            int(ctx.max()), d ** -0.5, k_scale=dev[2], v_scale=dev[3])
        torch.cuda.synchronize()
        _assert_same(tuple(t.cpu().numpy() for t in dev), state, f"verify step {step}")
        ref, ref_lse = oracle.paged_multi_query_attention(q, state[0], state[1], grown, ctx, bs,
                                                          d ** -0.5, "fp8", state[2], state[3])
        assert_parity(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                      ref, ref_lse, f"verify step {step}")


def test_fused_fp8_append_outside_the_attended_tokens(gpu):
    """A position at context_lens (the next token) is written (quantised) but not
    attended; negative positions write nothing."""
    hq, hkv, d, bs = 16, 4, 128, 16
    lens = [300, 40, 1000]
    state, grown = _fp8_case_with_room(hq, hkv, d, bs, lens, 4, 9800)
    rng = np.random.default_rng(11)
    k_new, v_new = _rows(rng, (3, 1, hkv, d), 2.0), _rows(rng, (3, 1, hkv, d), 0.5)
    pos = np.array([300, -1, 1000], dtype=np.int32)     # == ctx, none, == ctx
    ctx = np.array(lens, dtype=np.int32)
    ref_state = oracle.kv_append_fp8(*state, k_new, v_new, grown, pos, bs)
    dev = [_u8_dev(state[0]), _u8_dev(state[1]), _f32_dev(state[2]), _f32_dev(state[3])]
    q = _rows(rng, (3, hq, d), 1.0)
    out, lse = gpu.paged_decode_append_attention(
        _bf16_dev(q), _bf16_dev(k_new[:, 0]), _bf16_dev(v_new[:, 0]), _i32_dev(pos), dev[0],
        dev[1], _i32_dev(grown), _i32_dev(ctx), int(ctx.max()), d ** -0.5,
        k_scale=dev[2], v_scale=dev[3])
    torch.cuda.synchronize()
    _assert_same(tuple(t.cpu().numpy() for t in dev), ref_state, "outside")
    ref, ref_lse = oracle.paged_decode_attention(q, state[0], state[1], grown, ctx, bs, d ** -0.5,
                                                 "fp8", state[2], state[3])
    assert_parity(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                  ref, ref_lse, "outside")
