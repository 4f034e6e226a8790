"""GPU checks of the KIVI fp8 layout (keys scaled per channel of each (block, KV
head), values per token): attention parity against the float64 oracle over the
same stored codes and scales, the quantising append bit for bit, append-then-
attend steps (separate and fused), and the block copy."""
import numpy as np
import pytest
import torch

import oracle
from tests._dev import assert_parity, to_device
from workloads import bf16_round, make_case, make_multi_query_case, small_spec

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ref(case, w=0):
    s = case["spec"]
    args = (case["q"], case["k_pool_full"], case["v_pool_full"], case["block_tables"],
            case["context_lens"], s.block_size, case["softmax_scale"], s.kv_dtype,
            case["k_scale"], case["v_scale"])
    if case.get("num_queries"):
        return oracle.paged_multi_query_attention(*args, sliding_window=w)
    return oracle.paged_decode_attention(*args, sliding_window=w)


def _run(gpu, case, w=0, batch_invariant=False):
    dev = to_device(case)
    mx = int(case["context_lens"].max())
    fn = gpu.paged_decode_multi_query if case.get("num_queries") else gpu.paged_decode_attention
    out, lse = fn(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                  dev["context_lens"], mx, case["softmax_scale"], dev["k_scale"], dev["v_scale"],
                  sliding_window=w, batch_invariant=batch_invariant)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d,bs,hq,hkv", [(128, 16, 40, 40), (128, 16, 8, 2), (64, 32, 8, 2),
                                         (128, 32, 16, 2), (64, 16, 16, 4), (128, 16, 32, 4)])
def test_kivi_attention_parity(gpu, d, bs, hq, hkv):
    """Ragged lengths over several splits, partial last blocks, a shared pool;
    G = 1 .. 8 (8 rows: 16-token wave chunks, so a 32-token block spans two)."""
    lens = [3000, 1, 700, 129, 4097]
    spec = small_spec(num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                      block_size=bs, kv_dtype="fp8_kivi", context=4097, case_id=9950 + d + bs + hq)
    case = make_case(spec, seed=1, context_lens=lens)
    ref, ref_lse = _ref(case)
    out, lse = _run(gpu, case)
    assert_parity(out, lse, ref, ref_lse, f"kivi d={d} bs={bs} G={hq // hkv}")
    out2, lse2 = _run(gpu, case, batch_invariant=True)
    assert_parity(out2, lse2, ref, ref_lse, "kivi batch-invariant")


@pytest.mark.parametrize("nq,w", [(2, 0), (4, 0), (2, 300), (1, 64)])
def test_kivi_multi_query_and_window(gpu, nq, w):
    lens = [2000, 40, 900]
    spec = small_spec(num_seqs=3, num_q_heads=8, num_kv_heads=4, head_dim=128, block_size=16,
                      kv_dtype="fp8_kivi", context=2000, case_id=9960 + nq + w)
    case = (make_multi_query_case(spec, nq, seed=2, context_lens=lens, append=False) if nq > 1
            else make_case(spec, seed=2, context_lens=lens))
    ref, ref_lse = _ref(case, w)
    out, lse = _run(gpu, case, w)
    assert_parity(out, lse, ref, ref_lse, f"kivi Q={nq} w={w}")


def test_kivi_full_size_mha(gpu):
    """The 40-head MHA shape at ctx 8192 with KIVI scales, every output checked."""
    case = make_case("mha_fp8_kivi", seed=0)
    ref, ref_lse = _ref(case)
    out, lse = _run(gpu, case)
    assert_parity(out, lse, ref, ref_lse, "mha_fp8_kivi")


def _rows(rng, shape, scales):
    return bf16_round((rng.standard_normal(shape) * np.asarray(scales)).astype(np.float32))


def _t(a, dtype=None):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _same(got, ref, label):
    for g, r, n in zip(got, ref, ("k codes", "v codes", "k scales", "v scales")):
        if n.endswith("scales"):
            assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"{label}: {n}"
        else:
            bad = np.argwhere(g != r)
            assert bad.size == 0, f"{label}: {n} differ at {bad[:5].tolist()} ({len(bad)})"


@pytest.mark.parametrize("hkv,d,bs,T,seed", [(8, 128, 16, 1, 0), (8, 128, 16, 5, 1),
                                             (2, 64, 32, 9, 2), (40, 128, 16, 1, 3),
                                             (1, 128, 32, 40, 4)])
def test_kivi_append_is_bit_exact(gpu, hkv, d, bs, T, seed):
    rng = np.random.default_rng(50 + seed)
    B, max_blocks = 7, 5
    nb = B * max_blocks + 2
    kp = rng.integers(0, 0x7E, (nb, hkv, bs, d), dtype=np.uint8)
    vp = rng.integers(0, 0x7E, (nb, hkv, bs, d), dtype=np.uint8)
    ks = (2.0 ** rng.integers(-9, -2, (nb, hkv, d))).astype(np.float32)
    vs = rng.uniform(0.001, 0.02, (nb, hkv, bs)).astype(np.float32)
    tables = rng.permutation(nb)[:B * max_blocks].astype(np.int32).reshape(B, max_blocks)
    tables[2, 1] = -1
    cap = max_blocks * bs
    start = rng.integers(0, cap - T + 1, B).astype(np.int32)
    start[0], start[1], start[3] = 0, -1, bs - 1
    start[4] = cap - 1
    mags = 2.0 ** rng.uniform(-3, 4, (B, T, hkv, d))          # per-channel growth varies
    k_new, v_new = _rows(rng, (B, T, hkv, d), mags), _rows(rng, (B, T, hkv, d), mags[::-1])
    ref = oracle.kv_append_fp8(kp, vp, ks, vs, k_new, v_new, tables, start, bs, layout="kivi")
    dev = [_t(kp), _t(vp), _t(ks), _t(vs)]
    gpu.kv_append_fp8(_t(k_new), _t(v_new), *dev, _t(tables), _t(start))
    torch.cuda.synchronize()
    _same(tuple(x.cpu().numpy() for x in dev), ref, f"kivi append hkv={hkv} T={T}")


def test_kivi_decode_steps_append_then_attend(gpu):
    hq, hkv, d, bs = 16, 4, 128, 16
    lens = [500, 17, 64]
    steps = 12
    spec = small_spec(num_seqs=3, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                      kv_dtype="fp8_kivi", context=600, pool="oversized2x", case_id=9970)
    case = make_case(spec, seed=3, context_lens=lens)
    nb = case["k_pool_full"].shape[0]
    tables = case["block_tables"]
    used = set(tables[tables >= 0].tolist())
    free = [i for i in range(nb) if i not in used]
    grown = np.full((3, -(-(max(lens) + steps) // bs)), -1, dtype=np.int32)
    grown[:, :tables.shape[1]] = tables
    for b, n in enumerate(lens):
        for i in range(-(-n // bs), -(-(n + steps) // bs)):
            grown[b, i] = free.pop()
    state = (case["k_pool_full"], case["v_pool_full"], case["k_scale"], case["v_scale"])
    dev = [_t(x) for x in state]
    rng = np.random.default_rng(9)
    ctx = np.array(lens, dtype=np.int32)
    for step in range(steps):
        mags = 2.0 ** rng.uniform(-1, 2, (3, 1, hkv, d))
        k_new, v_new = _rows(rng, (3, 1, hkv, d), mags), _rows(rng, (3, 1, hkv, d), mags)
        q = _rows(rng, (3, hq, d), 1.0)
        state = oracle.kv_append_fp8(*state, k_new, v_new, grown, ctx, bs, layout="kivi")
        gpu.kv_append_fp8(_t(k_new), _t(v_new), *dev, _t(grown), _t(ctx))
        ctx = ctx + 1
        out, lse = gpu.paged_decode_attention(_t(q), dev[0], dev[1], _t(grown), _t(ctx),
                                              int(ctx.max()), d ** -0.5, dev[2], dev[3])
        torch.cuda.synchronize()
        _same(tuple(x.cpu().numpy() for x in dev), state, f"step {step}")
        ref, ref_lse = oracle.paged_decode_attention(q, state[0], state[1], grown, ctx, bs,
                                                     d ** -0.5, "fp8_kivi", state[2], state[3])
        assert_parity(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                      ref, ref_lse, f"kivi step {step}")


def test_kivi_block_copy(gpu):
    rng = np.random.default_rng(11)
    nb, hkv, bs, d = 40, 4, 16, 64
    kp = rng.integers(0, 256, (nb, hkv, bs, d), dtype=np.uint8)
    vp = rng.integers(0, 256, (nb, hkv, bs, d), dtype=np.uint8)
    ks = rng.random((nb, hkv, d), dtype=np.float32)
    vs = rng.random((nb, hkv, bs), dtype=np.float32)
    src = np.array([3, 3, 7, -1, 9], np.int32)
    dst = np.array([10, 11, 12, 13, 9], np.int32)
    ref = oracle.copy_blocks(kp, vp, src, dst, ks, vs)
    dev = [_t(kp), _t(vp), _t(ks), _t(vs)]
    gpu.kv_copy_blocks(dev[0], dev[1], _t(src), _t(dst), dev[2], dev[3])
    torch.cuda.synchronize()
    _same(tuple(x.cpu().numpy() for x in dev), ref, "kivi copy")


def _kivi_room(hq, hkv, d, bs, lens, extra, case_id):
    spec = small_spec(num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                      block_size=bs, kv_dtype="fp8_kivi", context=max(lens),
                      pool="oversized2x", case_id=case_id)
    case = make_case(spec, seed=4, context_lens=lens)
    nb = case["k_pool_full"].shape[0]
    tables = case["block_tables"]
    used = set(tables[tables >= 0].tolist())
    free = [i for i in range(nb) if i not in used]
    grown = np.full((len(lens), -(-(max(lens) + extra) // bs)), -1, dtype=np.int32)
    grown[:, :tables.shape[1]] = tables
    for b, n in enumerate(lens):
        for i in range(-(-n // bs), -(-(n + extra) // bs)):
            grown[b, i] = free.pop()
    return (case["k_pool_full"], case["v_pool_full"], case["k_scale"], case["v_scale"]), grown


@pytest.mark.parametrize("hq,hkv,d,bs,nq", [(16, 4, 128, 16, 1), (64, 8, 128, 32, 1),
                                            (8, 8, 64, 16, 1), (16, 8, 128, 32, 4),
                                            (8, 8, 128, 16, 8)])
def test_kivi_fused_append_and_attend(gpu, hq, hkv, d, bs, nq):
    """Fused steps on a KIVI pool: the new tokens quantised with per-channel key and
    per-token value scales inside the attention kernel (blocks spanning two wave
    chunks included), codes and scales bit-exact after every step, parity on every
    query position."""
    lens = [700, 17, 2100]
    steps = 6
    state, grown = _kivi_room(hq, hkv, d, bs, lens, steps * nq, 9980 + hq + bs + nq)
    dev = [_t(x) for x in state]
    td = _t(grown)
    rng = np.random.default_rng(hq + nq)
    ctx = np.array(lens, dtype=np.int32)
    for step in range(steps):
        mags = 2.0 ** rng.uniform(-2, 3, (3, nq, hkv, d))
        k_new, v_new = _rows(rng, (3, nq, hkv, d), mags), _rows(rng, (3, nq, hkv, d), mags)
        state = oracle.kv_append_fp8(*state, k_new, v_new, grown, ctx, bs, layout="kivi")
        start = ctx.copy()
        ctx = ctx + nq
        if nq == 1:
            q = _rows(rng, (3, hq, d), 1.0)
            out, lse = gpu.paged_decode_append_attention(
                _t(q), _t(k_new[:, 0]), _t(v_new[:, 0]), _t(start), dev[0], dev[1], td, _t(ctx),
                int(ctx.max()), d ** -0.5, k_scale=dev[2], v_scale=dev[3])
            ref, ref_lse = oracle.paged_decode_attention(q, state[0], state[1], grown, ctx, bs,
                                                         d ** -0.5, "fp8_kivi", state[2], state[3])
        else:
            q = _rows(rng, (3, nq, hq, d), 1.0)
            out, lse = gpu.paged_decode_multi_query_append(
                _t(q), _t(k_new), _t(v_new), dev[0], dev[1], td, _t(ctx), int(ctx.max()),
                d ** -0.5, k_scale=dev[2], v_scale=dev[3])
            ref, ref_lse = oracle.paged_multi_query_attention(q, state[0], state[1], grown, ctx, bs,
                                                              d ** -0.5, "fp8_kivi", state[2],
                                                              state[3])
        torch.cuda.synchronize()
        _same(tuple(x.cpu().numpy() for x in dev), state, f"kivi fused step {step}")
        assert_parity(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                      ref, ref_lse, f"kivi fused step {step}")
