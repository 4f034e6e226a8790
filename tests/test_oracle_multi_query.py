"""Pins the multi-position oracle (speculative verification: Q consecutive query
positions per sequence, each attending causally) to things other than itself: a
pure-Python brute force, float64 SDPA with an explicit causal mask, the
single-position oracle it must reduce to, and a planted off-by-one."""
import math
import struct

import numpy as np
import pytest
import torch

import oracle
import oracle.multi_query
from oracle import (paged_multi_query_attention, paged_decode_attention, kv_append,
                    kv_append_tokens, bf16_to_float64)
from workloads import make_multi_query_case, small_spec


def _f(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _brute(case):
    """Python loops: token positions through a dict built from the table; query i
    of sequence b sees positions 0 .. ctx - Q + i."""
    spec = case["spec"]
    BS, G, Q = spec.block_size, spec.group, case["num_queries"]
    q, kp, vp, bt, ctxs = (case["q"], case["k_pool_full"], case["v_pool_full"],
                           case["block_tables"], case["context_lens"])
    B, _, Hq, D = q.shape
    out = np.zeros((B, Q, Hq, D))
    lse = np.full((B, Q, Hq), -math.inf)
    for b in range(B):
        ctx = int(ctxs[b])
        where = {i * BS + s: (int(p), s) for i, p in enumerate(bt[b]) for s in range(BS)}
        for i in range(Q):
            last = ctx - Q + i                        # the query's own position
            for h in range(Hq):
                kvh = h // G
                qv = [_f(x) for x in q[b, i, h]]
                sc = []
                for t in range(last + 1):
                    p, s = where[t]
                    sc.append(case["softmax_scale"] * sum(a * _f(c) for a, c in zip(qv, kp[p, kvh, s])))
                if not sc:
                    continue
                mx = max(sc)
                ex = [math.exp(x - mx) for x in sc]
                z = sum(ex)
                acc = [0.0] * D
                for t, e in enumerate(ex):
                    p, s = where[t]
                    for d, x in enumerate(vp[p, kvh, s]):
                        acc[d] += e / z * _f(x)
                out[b, i, h] = acc
                lse[b, i, h] = mx + math.log(z)
    return out, lse


def _run(case):
    s = case["spec"]
    return paged_multi_query_attention(case["q"], case["k_pool_full"], case["v_pool_full"],
                                       case["block_tables"], case["context_lens"], s.block_size,
                                       case["softmax_scale"])


def _tiny(q=3, lens=(7, 19, 3), hq=4, hkv=2, case_id=5000):
    spec = small_spec(num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=16,
                      block_size=16, context=max(lens), case_id=case_id)
    return make_multi_query_case(spec, q, seed=1, context_lens=list(lens))


@pytest.mark.parametrize("q,lens", [(3, (7, 19, 3)), (1, (5, 33)), (5, (5, 40, 17))])
def test_multi_query_matches_brute_force(q, lens):
    case = _tiny(q, lens)
    out, lse = _run(case)
    ref, ref_lse = _brute(case)
    assert np.max(np.abs(out - ref)) < 1e-12 and np.max(np.abs(lse - ref_lse)) < 1e-12


def test_brute_force_catches_off_by_one_causal_limit(monkeypatch):
    """Planted in the oracle: each query drops its own token (limit one short)."""
    case = _tiny()
    real = oracle.multi_query.dense_decode_attention
    monkeypatch.setattr(oracle.multi_query, "dense_decode_attention",
                        lambda q, k, v, s: real(q, k[:, :-1], v[:, :-1], s))
    out, _ = _run(case)
    ref, _ = _brute(case)
    assert np.max(np.abs(out - ref)) > 1e-3


@pytest.mark.parametrize("hq,hkv,q,ctx", [(8, 2, 4, 40), (4, 4, 3, 17), (8, 1, 2, 64)])
def test_identity_table_equals_float64_causal_sdpa(hq, hkv, q, ctx):
    """Contiguous cache (identity table): the Q queries are the last Q rows of a causal
    attention over the sequence, computed by float64 torch SDPA with an explicit mask."""
    spec = small_spec(num_seqs=1, num_q_heads=hq, num_kv_heads=hkv, head_dim=32, block_size=16,
                      context=ctx, pool="exact", case_id=5100 + ctx)
    case = make_multi_query_case(spec, q, seed=2, poison=False)   # every slot a real value
    nb = -(-ctx // 16)
    case["block_tables"][0, :nb] = np.arange(nb)             # identity placement
    out, lse = _run(case)
    G = hq // hkv
    k = torch.from_numpy(bf16_to_float64(case["k_pool_full"][:nb])).permute(1, 0, 2, 3)
    v = torch.from_numpy(bf16_to_float64(case["v_pool_full"][:nb])).permute(1, 0, 2, 3)
    k = k.reshape(hkv, nb * 16, 32)[:, :ctx].repeat_interleave(G, 0)       # [H_q][ctx][d]
    v = v.reshape(hkv, nb * 16, 32)[:, :ctx].repeat_interleave(G, 0)
    qq = torch.from_numpy(bf16_to_float64(case["q"][0])).permute(1, 0, 2)    # [H_q][Q][d]
    pos = torch.arange(ctx - q, ctx)[:, None]
    mask = torch.arange(ctx)[None, :] <= pos                                  # [Q][ctx]
    sc = case["softmax_scale"]
    ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v, attn_mask=mask, scale=sc)
    scores = (qq @ k.transpose(1, 2)) * sc
    ref_lse = torch.logsumexp(scores.masked_fill(~mask, -math.inf), dim=-1)   # [H_q][Q]
    assert np.max(np.abs(out[0] - ref.permute(1, 0, 2).numpy())) < 1e-12
    assert np.max(np.abs(lse[0] - ref_lse.T.numpy())) < 1e-12


def test_single_query_is_the_single_position_oracle():
    case = _tiny(q=1, lens=(9, 30))
    out, lse = _run(case)
    s = case["spec"]
    ref, ref_lse = paged_decode_attention(case["q"][:, 0], case["k_pool_full"], case["v_pool_full"],
                                          case["block_tables"], case["context_lens"], s.block_size,
                                          case["softmax_scale"])
    assert np.array_equal(out[:, 0], ref) and np.array_equal(lse[:, 0], ref_lse)


def test_each_query_is_single_position_attention_over_its_prefix():
    """Query i equals one-position attention with the context cut after its position."""
    case = _tiny(q=4, lens=(11, 26, 4))
    out, lse = _run(case)
    s = case["spec"]
    for i in range(4):
        cut = case["context_lens"] - 4 + 1 + i
        ref, ref_lse = paged_decode_attention(case["q"][:, i], case["k_pool_full"],
                                              case["v_pool_full"], case["block_tables"], cut,
                                              s.block_size, case["softmax_scale"])
        assert np.array_equal(out[:, i], ref) and np.array_equal(lse[:, i], ref_lse)


def test_malformed_and_empty_contexts():
    case = _tiny(q=3, lens=(2, 0, 8))
    out, lse = _run(case)
    assert np.all(np.isnan(out[0])) and np.all(np.isnan(lse[0]))
    assert np.all(out[1] == 0) and np.all(lse[1] == -np.inf)
    assert np.all(np.isfinite(out[2]))


def test_first_query_of_a_full_context_sees_one_token_less():
    """ctx = Q: query 0 sits at position 0 and attends only to token 0, so its output is
    that token's value row exactly."""
    case = _tiny(q=3, lens=(3,), hq=2, hkv=2)
    out, _ = _run(case)
    bt, BS = case["block_tables"], 16
    v0 = bf16_to_float64(case["v_pool_full"][bt[0, 0], :, 0, :])              # [H_kv][d]
    assert np.array_equal(out[0, 0], v0)


def test_append_tokens_single_is_append():
    case = _tiny(q=1, lens=(9, 30))
    k1, v1 = kv_append_tokens(case["k_pool"], case["v_pool"], case["k_new"], case["v_new"],
                              case["block_tables"], case["positions"], 16)
    k2, v2 = kv_append(case["k_pool"], case["v_pool"], case["k_new"][:, 0], case["v_new"][:, 0],
                       case["block_tables"], case["positions"][:, 0], 16)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_append_tokens_restores_the_full_pools_and_skips_out_of_range():
    case = _tiny(q=4, lens=(7, 19, 3))
    k, v = kv_append_tokens(case["k_pool"], case["v_pool"], case["k_new"], case["v_new"],
                            case["block_tables"], case["positions"], 16)
    assert np.array_equal(k, case["k_pool_full"]) and np.array_equal(v, case["v_pool_full"])
    pos = case["positions"].copy()
    pos[0, 0] = case["block_tables"].shape[1] * 16          # past the table: skipped
    k3, _ = kv_append_tokens(case["k_pool"], case["v_pool"], case["k_new"], case["v_new"],
                             case["block_tables"], pos, 16)
    blk, slot = case["block_tables"][0, 3 // 16], 3 % 16    # sequence 0's first new slot
    assert np.array_equal(k3[blk, :, slot], case["k_pool"][blk, :, slot])
