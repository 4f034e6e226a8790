"""Pins the float64 oracle (attention, gather, online softmax, merge) to things
other than itself: brute force, a float64 library routine, closed forms and
invariants.  Several tests plant a plausible mistake in the oracle (on the CPU)
and check that a pin catches it."""
import math
import struct

import numpy as np
import pytest
import torch

import oracle
import oracle.attention
import oracle.cache
from oracle import (paged_decode_attention, dense_decode_attention, chunked_attention,
                    merge_partials, gather_sequence, bf16_to_float64)
from workloads import make_case, small_spec, bf16_round


# ---------------------------------------------------------------- brute force
def _bf16_bits_to_float_py(bits):
    """Independent widening for the brute-force side: bytes through struct."""
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _brute(case):
    """Pure-Python loops: place every logical token through a dict built from the
    table, then textbook softmax attention in Python floats."""
    spec = case["spec"]
    BS, G = spec.block_size, spec.group
    q, kp, vp, bt, ctxs = (case["q"], case["k_pool_full"], case["v_pool_full"],
                           case["block_tables"], case["context_lens"])
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -math.inf)
    for b in range(B):
        where = {}
        for i, phys in enumerate(bt[b]):
            for slot in range(BS):
                where[i * BS + slot] = (int(phys), slot)
        for h in range(Hq):
            kvh = h // G
            qv = [_bf16_bits_to_float_py(x) for x in q[b, h]]
            scores = []
            for t in range(int(ctxs[b])):
                p, s = where[t]
                kv = [_bf16_bits_to_float_py(x) for x in kp[p, kvh, s]]
                scores.append(spec_scale(case) * sum(a * c for a, c in zip(qv, kv)))
            if not scores:
                continue
            mx = max(scores)
            ex = [math.exp(s - mx) for s in scores]
            z = sum(ex)
            acc = [0.0] * D
            for t, e in enumerate(ex):
                p, s = where[t]
                vv = [_bf16_bits_to_float_py(x) for x in vp[p, kvh, s]]
                for d in range(D):
                    acc[d] += e / z * vv[d]
            out[b, h] = acc
            lse[b, h] = mx + math.log(z)
    return out, lse


def spec_scale(case):
    return case["softmax_scale"]


def _run(case):
    s = case["spec"]
    return paged_decode_attention(case["q"], case["k_pool_full"], case["v_pool_full"],
                                  case["block_tables"], case["context_lens"], s.block_size,
                                  case["softmax_scale"], s.kv_dtype, case["k_scale"], case["v_scale"])


TINY_SPECS = [
    small_spec(num_seqs=2, num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=4, context=13, case_id=201),
    small_spec(num_seqs=3, num_q_heads=4, num_kv_heads=1, head_dim=8, block_size=1, context=5, case_id=202),
    small_spec(num_seqs=1, num_q_heads=2, num_kv_heads=2, head_dim=16, block_size=16, context=40, case_id=203),
    small_spec(num_seqs=2, num_q_heads=4, num_kv_heads=1, head_dim=4, block_size=2, context=("uniform", 1, 40),
               case_id=204, pool="exact"),
]


@pytest.mark.parametrize("spec", TINY_SPECS, ids=lambda s: f"cid{s.case_id}")
def test_oracle_matches_brute_force(spec):
    case = make_case(spec, seed=3)
    out, lse = _run(case)
    bo, bl = _brute(case)
    assert np.max(np.abs(out - bo)) <= 1e-12
    assert np.max(np.abs(lse - bl)) <= 1e-12


def test_brute_force_catches_wrong_head_group(monkeypatch):
    """Planted mistake: query head h reads KV head h % H_kv instead of h // G."""
    case = make_case(TINY_SPECS[0], seed=3)

    def wrong(q, k, v, scale):
        Hq, D = q.shape
        Hkv = k.shape[0]
        out = np.zeros((Hq, D))
        lse = np.zeros(Hq)
        for h in range(Hq):
            s = scale * (k[h % Hkv] @ q[h])
            w = np.exp(s - s.max())
            out[h] = (w / w.sum()) @ v[h % Hkv]
            lse[h] = s.max() + np.log(w.sum())
        return out, lse

    monkeypatch.setattr(oracle.attention, "dense_decode_attention", wrong)
    out, _ = _run(case)
    bo, _ = _brute(case)
    assert np.max(np.abs(out - bo)) > 1e-3


def test_brute_force_catches_transposed_block_index(monkeypatch):
    """Planted mistake: physical block from t % BS and slot from t // BS."""
    case = make_case(TINY_SPECS[0], seed=3)

    def wrong(pool, row, ctx, bs):
        t = np.arange(ctx)
        nb = (ctx + bs - 1) // bs
        phys = np.asarray(row)[(t % bs) % nb]
        rows = pool[phys, :, (t // bs) % bs, :]
        return np.transpose(rows, (1, 0, 2))

    monkeypatch.setattr(oracle.attention, "gather_sequence", wrong)
    out, _ = _run(case)
    bo, _ = _brute(case)
    assert not np.allclose(out, bo, atol=1e-6)


# ---------------------------------------------------------------- library routine
@pytest.mark.parametrize("hq,hkv,d,ctx", [(8, 2, 64, 100), (4, 4, 32, 17), (8, 1, 16, 1), (16, 2, 128, 333)])
def test_identity_table_equals_float64_sdpa(hq, hkv, d, ctx):
    """With an identity block table the paged oracle is torch SDPA (float64, CPU)
    over K/V whose heads are repeated G times (the pages' Lab 2 uses this pattern)."""
    rng = np.random.default_rng(hq * 1000 + ctx)
    BS = 16
    nb = (ctx + BS - 1) // BS
    q = bf16_round(rng.standard_normal((1, hq, d)).astype(np.float32))
    kp = bf16_round(rng.standard_normal((nb, hkv, BS, d)).astype(np.float32))
    vp = bf16_round(rng.standard_normal((nb, hkv, BS, d)).astype(np.float32))
    bt = np.arange(nb, dtype=np.int32)[None, :]
    scale = 1 / math.sqrt(d)
    out, lse = paged_decode_attention(q, kp, vp, bt, np.array([ctx]), BS, scale)

    def dense(pool):   # contiguous [1][H_kv][T][d] through plain reshape of the identity layout
        x = bf16_to_float64(pool).transpose(1, 0, 2, 3).reshape(hkv, nb * BS, d)[:, :ctx]
        return torch.from_numpy(np.ascontiguousarray(x))[None]

    G = hq // hkv
    K = dense(kp).repeat_interleave(G, dim=1)
    V = dense(vp).repeat_interleave(G, dim=1)
    Q = torch.from_numpy(bf16_to_float64(q))[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[0, :, 0].numpy()
    assert np.max(np.abs(out[0] - ref)) <= 1e-12
    s = scale * torch.einsum("hd,htd->ht", Q[0, :, 0], K[0])
    assert np.max(np.abs(lse[0] - torch.logsumexp(s, dim=-1).numpy())) <= 1e-12


# ---------------------------------------------------------------- closed forms
def _random_case(ctx, hq=4, hkv=2, d=16, bs=4, seed=0):
    return make_case(small_spec(num_seqs=1, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                block_size=bs, context=ctx, case_id=300 + ctx), seed=seed)


def test_ctx1_returns_the_single_value_exactly():
    case = _random_case(1)
    out, lse = _run(case)
    v0 = bf16_to_float64(gather_sequence(case["v_pool_full"], case["block_tables"][0], 1, 4))
    k0 = bf16_to_float64(gather_sequence(case["k_pool_full"], case["block_tables"][0], 1, 4))
    q = bf16_to_float64(case["q"][0])
    for h in range(4):
        assert np.array_equal(out[0, h], v0[h // 2, 0])
        assert lse[0, h] == case["softmax_scale"] * (k0[h // 2, 0] @ q[h])


def test_zero_query_gives_mean_of_values_and_log_ctx():
    case = _random_case(37)
    case["q"][:] = 0
    out, lse = _run(case)
    v = bf16_to_float64(gather_sequence(case["v_pool_full"], case["block_tables"][0], 37, 4))
    for h in range(4):
        assert np.max(np.abs(out[0, h] - v[h // 2].mean(axis=0))) <= 1e-14
        assert abs(lse[0, h] - math.log(37)) <= 1e-14


def test_weights_sum_to_one():
    case = _random_case(29)
    one = np.uint16(0x3F80)        # bf16 1.0
    case["v_pool_full"] = np.where(np.isnan(bf16_to_float64(case["v_pool_full"])),
                                   case["v_pool_full"], one).astype(np.uint16)
    out, _ = _run(case)
    assert np.max(np.abs(out - 1.0)) <= 1e-14


def test_dominant_key_selects_its_value():
    case = _random_case(20)
    k = bf16_to_float64(gather_sequence(case["k_pool_full"], case["block_tables"][0], 20, 4))
    q = np.zeros(16)
    q[:] = k[0, 7] * 1000.0                       # head 0 aligns with token 7 of KV head 0
    case["q"][0, 0] = bf16_round(q.astype(np.float32))
    out, _ = _run(case)
    v = bf16_to_float64(gather_sequence(case["v_pool_full"], case["block_tables"][0], 20, 4))
    assert np.max(np.abs(out[0, 0] - v[0, 7])) < 1e-6


def test_empty_context():
    case = make_case(small_spec(num_seqs=2, context=5, case_id=310), seed=1, context_lens=[0, 5])
    out, lse = _run(case)
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(out[1]))


# ---------------------------------------------------------------- invariants
def test_physical_block_permutation_is_bit_identical():
    case = make_case(small_spec(num_seqs=3, context=("uniform", 10, 70), case_id=320), seed=2)
    out, lse = _run(case)
    rng = np.random.default_rng(5)
    nbk = case["k_pool_full"].shape[0]
    perm = rng.permutation(nbk)
    moved = dict(case)
    moved["k_pool_full"] = np.empty_like(case["k_pool_full"])
    moved["v_pool_full"] = np.empty_like(case["v_pool_full"])
    moved["k_pool_full"][perm] = case["k_pool_full"]
    moved["v_pool_full"][perm] = case["v_pool_full"]
    bt = case["block_tables"].copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    moved["block_tables"] = bt
    out2, lse2 = _run(moved)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_batch_invariance():
    case = make_case(small_spec(num_seqs=4, context=("uniform", 1, 90), case_id=330), seed=4)
    out, lse = _run(case)
    for b in range(4):
        one = dict(case)
        one["q"] = case["q"][b:b + 1]
        one["block_tables"] = case["block_tables"][b:b + 1]
        one["context_lens"] = case["context_lens"][b:b + 1]
        o1, l1 = _run(one)
        assert np.array_equal(o1[0], out[b]) and np.array_equal(l1[0], lse[b])


def test_gqa_equals_mha_with_repeated_kv_heads():
    case = make_case(small_spec(num_seqs=2, num_q_heads=8, num_kv_heads=2, context=50, case_id=340), seed=6)
    out, lse = _run(case)
    mha = dict(case)
    mha["k_pool_full"] = np.repeat(case["k_pool_full"], 4, axis=1)
    mha["v_pool_full"] = np.repeat(case["v_pool_full"], 4, axis=1)
    mha["spec"] = small_spec(num_seqs=2, num_q_heads=8, num_kv_heads=8, context=50, case_id=340)
    o2, l2 = _run(mha)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def test_poisoned_slots_never_reach_the_result():
    case = make_case(small_spec(num_seqs=3, context=("uniform", 1, 60), case_id=350), seed=8)
    out, lse = _run(case)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_fp8_pool_equals_bf16_oracle_on_dequantised_values():
    """The fp8 path is decode(code) * scale; feeding those values through the float64
    definition directly must give the same result."""
    case = make_case(small_spec(num_seqs=2, num_q_heads=4, num_kv_heads=4, head_dim=32,
                                kv_dtype="fp8", context=("uniform", 5, 60), case_id=360), seed=9)
    out, lse = _run(case)
    from oracle import decode_e4m3fn
    for b in range(2):
        ctx = int(case["context_lens"][b])
        t = np.arange(ctx)
        phys = case["block_tables"][b][t // 16]
        k = decode_e4m3fn(case["k_pool_full"][phys, :, t % 16, :]) * case["k_scale"][phys][:, :, None].astype(np.float64)
        v = decode_e4m3fn(case["v_pool_full"][phys, :, t % 16, :]) * case["v_scale"][phys][:, :, None].astype(np.float64)
        o, l = dense_decode_attention(bf16_to_float64(case["q"][b]), k.transpose(1, 0, 2),
                                      v.transpose(1, 0, 2), case["softmax_scale"])
        assert np.max(np.abs(o - out[b])) <= 1e-13 and np.max(np.abs(l - lse[b])) <= 1e-13


# ---------------------------------------------------------------- online softmax / merge
@pytest.mark.parametrize("chunk", [1, 3, 7, 16, 64, 1000])
def test_chunked_online_softmax_equals_direct(chunk):
    rng = np.random.default_rng(chunk)
    q = rng.standard_normal(32)
    k = rng.standard_normal((200, 32)) * 3
    v = rng.standard_normal((200, 32))
    o, l = chunked_attention(q, k, v, 0.3, chunk)
    od, ld = dense_decode_attention(q[None], k[None], v[None], 0.3)
    assert np.max(np.abs(o - od[0])) <= 1e-12 and abs(l - ld[0]) <= 1e-12


@pytest.mark.parametrize("cuts", [[0, 200], [0, 1, 200], [0, 50, 100, 150, 200], [0, 0, 64, 64, 200]])
def test_lse_merge_of_shards_equals_direct(cuts):
    rng = np.random.default_rng(len(cuts))
    q = rng.standard_normal(16)
    k = rng.standard_normal((200, 16)) * 4
    v = rng.standard_normal((200, 16))
    outs, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = chunked_attention(q, k[a:b], v[a:b], 0.5, 13)
        outs.append(o)
        lses.append(l)
    o, l = merge_partials(np.array(outs), np.array(lses))
    od, ld = dense_decode_attention(q[None], k[None], v[None], 0.5)
    assert np.max(np.abs(o - od[0])) <= 1e-12 and abs(l - ld[0]) <= 1e-12


def test_merge_catches_missing_rescale():
    """Planted mistake: merging shards with equal weights instead of exp(lse_j - M)."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal(16)
    k = rng.standard_normal((100, 16)) * 4
    v = rng.standard_normal((100, 16))
    o1, l1 = chunked_attention(q, k[:30], v[:30], 0.5, 8)
    o2, l2 = chunked_attention(q, k[30:], v[30:], 0.5, 8)
    wrong = (o1 + o2) / 2
    od, _ = dense_decode_attention(q[None], k[None], v[None], 0.5)
    assert np.max(np.abs(wrong - od[0])) > 1e-3


def test_merge_all_empty():
    o, l = merge_partials(np.zeros((3, 4)), np.array([-np.inf] * 3))
    assert np.all(o == 0) and l == -np.inf
