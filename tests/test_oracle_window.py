"""Pins the sliding-window reading of the oracle (each query attends to its w most
recent tokens, itself included) to a brute force, closed forms, the no-window
oracle and float64 SDPA with a band mask."""
import math
import struct

import numpy as np
import pytest
import torch

import oracle
import oracle.attention
from oracle import paged_decode_attention, paged_multi_query_attention, bf16_to_float64
from workloads import make_case, make_multi_query_case, small_spec


def _f(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _brute(case, w, nq):
    """Python loops over positions: query i (at ctx - nq + i) sees positions p with
    ctx - nq + i - w < p <= ctx - nq + i."""
    spec = case["spec"]
    BS, G = spec.block_size, spec.group
    q = case["q"] if nq > 1 else case["q"][:, None]
    kp, vp, bt, ctxs = case["k_pool_full"], case["v_pool_full"], case["block_tables"], case["context_lens"]
    B, _, Hq, D = q.shape
    out = np.zeros((B, nq, Hq, D))
    for b in range(B):
        where = {i * BS + s: (int(p), s) for i, p in enumerate(bt[b]) for s in range(BS)}
        for i in range(nq):
            me = int(ctxs[b]) - nq + i
            for h in range(Hq):
                qv = [_f(x) for x in q[b, i, h]]
                toks = [t for t in range(me + 1) if t > me - w]
                sc = []
                for t in toks:
                    p, s = where[t]
                    sc.append(case["softmax_scale"] * sum(a * _f(c) for a, c in zip(qv, kp[p, h // G, s])))
                mx = max(sc)
                ex = [math.exp(x - mx) for x in sc]
                z = sum(ex)
                acc = [0.0] * D
                for t, e in zip(toks, ex):
                    p, s = where[t]
                    for d, x in enumerate(vp[p, h // G, s]):
                        acc[d] += e / z * _f(x)
                out[b, i, h] = acc
    return out if nq > 1 else out[:, 0]


def _single(case, w):
    s = case["spec"]
    return paged_decode_attention(case["q"], case["k_pool_full"], case["v_pool_full"],
                                  case["block_tables"], case["context_lens"], s.block_size,
                                  case["softmax_scale"], sliding_window=w)


def _multi(case, w):
    s = case["spec"]
    return paged_multi_query_attention(case["q"], case["k_pool_full"], case["v_pool_full"],
                                       case["block_tables"], case["context_lens"], s.block_size,
                                       case["softmax_scale"], sliding_window=w)


def _spec(lens, case_id):
    return small_spec(num_seqs=len(lens), num_q_heads=4, num_kv_heads=2, head_dim=16,
                      block_size=16, context=max(lens), case_id=case_id)


@pytest.mark.parametrize("w", [1, 5, 17, 40])
def test_window_matches_brute_force(w):
    lens = [30, 7, 41]
    case = make_case(_spec(lens, 7000 + w), seed=1, context_lens=lens)
    out, _ = _single(case, w)
    assert np.max(np.abs(out - _brute(case, w, 1))) < 1e-12
    mcase = make_multi_query_case(_spec(lens, 7100 + w), 3, seed=1, context_lens=lens)
    mout, _ = _multi(mcase, w)
    assert np.max(np.abs(mout - _brute(mcase, w, 3))) < 1e-12


def test_brute_force_catches_a_window_one_token_short(monkeypatch):
    lens = [30, 41]
    case = make_case(_spec(lens, 7200), seed=2, context_lens=lens)
    real = oracle.attention.dense_decode_attention
    monkeypatch.setattr(oracle.attention, "dense_decode_attention",
                        lambda q, k, v, s: real(q, k[:, 1:], v[:, 1:], s))
    out, _ = _single(case, 9)
    assert np.max(np.abs(out - _brute(case, 9, 1))) > 1e-3


def test_window_covering_the_context_changes_nothing():
    lens = [30, 7, 41]
    case = make_case(_spec(lens, 7300), seed=3, context_lens=lens)
    o1, l1 = _single(case, 41)
    o2, l2 = _single(case, 0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    mcase = make_multi_query_case(_spec(lens, 7301), 4, seed=3, context_lens=lens)
    o1, l1 = _multi(mcase, 10 ** 6)
    o2, l2 = _multi(mcase, 0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_window_of_one_returns_the_own_value_and_zero_lse_offset():
    """w = 1: each query sees only its own token: out = that token's value row and
    lse = its score."""
    lens = [30, 41]
    case = make_multi_query_case(_spec(lens, 7400), 3, seed=4, context_lens=lens)
    out, lse = _multi(case, 1)
    bt = case["block_tables"]
    for b, ctx in enumerate(lens):
        for i in range(3):
            pos = ctx - 3 + i
            blk, slot = bt[b, pos // 16], pos % 16
            v = bf16_to_float64(case["v_pool_full"][blk, :, slot, :])          # [H_kv][d]
            assert np.array_equal(out[b, i], np.repeat(v, 2, axis=0))
            k = bf16_to_float64(case["k_pool_full"][blk, :, slot, :])
            qv = bf16_to_float64(case["q"][b, i])
            s = case["softmax_scale"] * np.sum(qv * np.repeat(k, 2, axis=0), axis=1)
            assert np.max(np.abs(lse[b, i] - s)) < 1e-12


def test_window_equals_float64_sdpa_with_a_band_mask():
    ctx, nq, w = 50, 4, 13
    spec = small_spec(num_seqs=1, num_q_heads=8, num_kv_heads=2, head_dim=32, block_size=16,
                      context=ctx, pool="exact", case_id=7500)
    case = make_multi_query_case(spec, nq, seed=5, poison=False)
    nb = -(-ctx // 16)
    case["block_tables"][0, :nb] = np.arange(nb)
    out, lse = _multi(case, w)
    k = torch.from_numpy(bf16_to_float64(case["k_pool_full"][:nb])).permute(1, 0, 2, 3)
    v = torch.from_numpy(bf16_to_float64(case["v_pool_full"][:nb])).permute(1, 0, 2, 3)
    k = k.reshape(2, nb * 16, 32)[:, :ctx].repeat_interleave(4, 0)
    v = v.reshape(2, nb * 16, 32)[:, :ctx].repeat_interleave(4, 0)
    qq = torch.from_numpy(bf16_to_float64(case["q"][0])).permute(1, 0, 2)
    pos = torch.arange(ctx - nq, ctx)[:, None]
    t = torch.arange(ctx)[None, :]
    mask = (t <= pos) & (t > pos - w)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v, attn_mask=mask,
                                                           scale=case["softmax_scale"])
    sc = (qq @ k.transpose(1, 2)) * case["softmax_scale"]
    ref_lse = torch.logsumexp(sc.masked_fill(~mask, -math.inf), dim=-1)
    assert np.max(np.abs(out[0] - ref.permute(1, 0, 2).numpy())) < 1e-12
    assert np.max(np.abs(lse[0] - ref_lse.T.numpy())) < 1e-12
