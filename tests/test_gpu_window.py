"""GPU parity of sliding-window attention (each query attends to its w most recent
tokens) against the float64 oracle, for single and several query positions,
both compute paths, and the fused steps; blocks wholly before every window are
never read.  Also regressions for launches whose hint plan rounds to fewer
splits than a shorter sequence needs."""
import numpy as np
import pytest
import torch

import oracle
from tests._dev import to_device, assert_parity, run_step
from workloads import make_case, make_multi_query_case, small_spec

pytestmark = pytest.mark.gpu


def _ref(case, w):
    s = case["spec"]
    args = (case["q"], case["k_pool_full"], case["v_pool_full"], case["block_tables"],
            case["context_lens"], s.block_size, case["softmax_scale"], s.kv_dtype,
            case["k_scale"], case["v_scale"])
    if case.get("num_queries"):
        return oracle.paged_multi_query_attention(*args, sliding_window=w)
    return oracle.paged_decode_attention(*args, sliding_window=w)


def _run(gqa, case, dev, w, max_ctx=None, fused=False):
    if max_ctx is None:
        max_ctx = int(case["context_lens"].max())
    args = dict(softmax_scale=case["softmax_scale"], sliding_window=w)
    if case.get("num_queries"):
        if fused:
            out, lse = gqa.paged_decode_multi_query_append(
                dev["q"], dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                dev["block_tables"], dev["context_lens"], max_ctx, **args)
        else:
            out, lse = gqa.paged_decode_multi_query(
                dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                dev["context_lens"], max_ctx, k_scale=dev["k_scale"], v_scale=dev["v_scale"], **args)
    elif fused:
        out, lse = gqa.paged_decode_append_attention(
            dev["q"], dev["k_new"], dev["v_new"], dev["positions"], dev["k_cache"], dev["v_cache"],
            dev["block_tables"], dev["context_lens"], max_ctx, **args)
    else:
        out, lse = gqa.paged_decode_attention(
            dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
            max_ctx, k_scale=dev["k_scale"], v_scale=dev["v_scale"], **args)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("hq,hkv,d,bs,dt,nq,w", [
    (32, 8, 128, 16, "bf16", 1, 4096),
    (32, 8, 128, 16, "bf16", 1, 1),
    (32, 8, 128, 16, "bf16", 1, 33),
    (64, 8, 128, 32, "bf16", 1, 1000),
    (8, 8, 128, 16, "bf16", 1, 500),
    (40, 40, 128, 16, "fp8", 1, 700),
    (32, 8, 128, 16, "bf16", 4, 100),
    (16, 4, 64, 32, "fp8", 2, 50),
    (64, 8, 128, 32, "bf16", 4, 1000),   # 32 rows: two row tiles
    (64, 8, 128, 32, "fp8", 4, 300),     # fp8 on the matrix path, 32 rows
])
def test_window_parity(gpu, hq, hkv, d, bs, dt, nq, w):
    lens = [8192, 3000, 100, 4097, nq]
    spec = small_spec(num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                      block_size=bs, kv_dtype=dt, context=8192, case_id=8000 + w + nq)
    case = (make_multi_query_case(spec, nq, seed=1, context_lens=lens, append=False) if nq > 1
            else make_case(spec, seed=1, context_lens=lens))
    ref, ref_lse = _ref(case, w)
    out, lse = _run(gpu, case, to_device(case), w)
    assert_parity(out, lse, ref, ref_lse, f"w={w} Q={nq} G={hq // hkv} {dt}")


def test_window_on_four_wave_workgroups(gpu):
    """A window over 24 ragged sequences x 8 KV heads (4-wave workgroups sharing
    slots out by each sequence's attended span)."""
    lens = [int(n) for n in np.random.default_rng(77).integers(1, 3000, 24)]
    spec = small_spec(num_seqs=24, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=3000, case_id=8077)
    case = make_case(spec, seed=2, context_lens=lens)
    ref, ref_lse = _ref(case, 300)
    out, lse = _run(gpu, case, to_device(case), 300)
    assert_parity(out, lse, ref, ref_lse, "w=300, 24 ragged sequences")


@pytest.mark.parametrize("nq", [1, 3])
def test_blocks_before_the_window_are_never_read(gpu, nq):
    """Table entries of blocks wholly before every query's window are set to -1 and
    those blocks filled with NaN codes: results are unchanged."""
    w, lens = 300, [5000, 2000, 310]
    spec = small_spec(num_seqs=3, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=5000, case_id=8100 + nq)
    case = (make_multi_query_case(spec, nq, seed=2, context_lens=lens, append=False) if nq > 1
            else make_case(spec, seed=2, context_lens=lens))
    ref, ref_lse = _ref(case, w)
    bt = case["block_tables"].copy()
    kp, vp = case["k_pool"].copy(), case["v_pool"].copy()
    for b, ctx in enumerate(lens):
        first = ctx - nq + 1 - w                         # query 0's first attended token
        for blk in range(max(0, first) // 16):           # blocks wholly before it
            kp[bt[b, blk]] = 0x7FC0
            vp[bt[b, blk]] = 0x7FC0
            bt[b, blk] = -1
    moved = dict(case, block_tables=bt, k_pool=kp, v_pool=vp)
    out, lse = _run(gpu, moved, to_device(moved), w)
    assert_parity(out, lse, ref, ref_lse, "released blocks")


def test_fused_steps_with_a_window(gpu):
    lens = [4096, 900, 40]
    spec = small_spec(num_seqs=3, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=4096, append=True, case_id=8200)
    case = make_case(spec, seed=3, context_lens=lens)
    ref, ref_lse = _ref(case, 257)
    dev = to_device(case)
    out, lse = _run(gpu, case, dev, 257, fused=True)
    assert_parity(out, lse, ref, ref_lse, "fused single, window")
    k = dev["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(k, case["k_pool_full"])
    mcase = make_multi_query_case(spec, 4, seed=4, context_lens=lens)
    mref, mref_lse = _ref(mcase, 257)
    mdev = to_device(mcase)
    out, lse = _run(gpu, mcase, mdev, 257, fused=True)
    assert_parity(out, lse, mref, mref_lse, "fused verify, window")
    k = mdev["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(k, mcase["k_pool_full"])


def test_window_covering_the_context_is_bitwise_the_full_attention(gpu):
    lens = [3000, 700]
    spec = small_spec(num_seqs=2, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=3000, case_id=8300)
    case = make_case(spec, seed=5, context_lens=lens)
    dev = to_device(case)
    o1, l1 = _run(gpu, case, dev, 3000)
    o2, l2 = _run(gpu, case, dev, 0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("hint,ctx,invariant", [(4100, 4000, False), (10000, 8192, True),
                                                (10000, 8192, False)])
def test_shorter_sequence_under_a_rounding_hint(gpu, hint, ctx, invariant):
    """The hint's own split plan can round to fewer splits than a shorter sequence
    needs (4100 tokens at target 32: 26 splits; 4000 tokens: 32); the launch covers
    every length up to the hint."""
    spec = small_spec(num_seqs=1, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=hint, case_id=8400 + ctx)
    case = make_case(spec, seed=6, context_lens=[hint])
    case["context_lens"] = np.array([ctx], dtype=np.int32)
    ref, ref_lse = oracle.paged_decode_attention(case["q"], case["k_pool_full"],
                                                 case["v_pool_full"], case["block_tables"],
                                                 case["context_lens"], 16, case["softmax_scale"])
    out, lse = run_step(gpu, to_device(case), case, max_context_len=hint,
                        batch_invariant=invariant)
    assert_parity(out, lse, ref, ref_lse, f"hint {hint} ctx {ctx}")
