"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Bar: max-abs <= 1e-2 and relative L2 <= 2e-3 on the attention output, lse within
1e-3; fp8 pools are compared with the oracle run on the same stored codes and
scales (so quantisation error is excluded)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from tests._dev import (to_device, run_step, run_fused_step, run_oracle, assert_parity,
                        named_case, named_reference)
from workloads import make_case, small_spec

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "llama8b", "batched", "long", "mha_fp8", "long_fp8"])
def test_named_workload_full_size(gpu, name):
    case = named_case(name)
    ref, ref_lse = named_reference(name)
    out, lse = run_step(gpu, to_device(case), case)
    max_abs, rel = assert_parity(out, lse, ref, ref_lse, name)
    print(f"{name}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    log_dir = os.environ.get("GQA_PARITY_LOG_DIR")
    if log_dir:
        os.makedirs(log_dir, exist_ok=True)
        with open(os.path.join(log_dir, f"parity_{name}.json"), "w") as f:
            json.dump({"workload": name, "max_abs": max_abs, "rel_l2": rel,
                       "lse_max_abs": float(np.max(np.abs(lse - ref_lse)))}, f)


SHAPES = [
    # (D, BS, H_q, H_kv, dtype)
    (d, bs, hq, hkv, dt)
    for d in (64, 128) for bs in (16, 32) for (hq, hkv) in ((4, 4), (8, 4), (8, 2), (16, 2))
    for dt in ("bf16", "fp8")
]


@pytest.mark.parametrize("d,bs,hq,hkv,dt", SHAPES, ids=lambda v: str(v))
def test_shape_sweep_ragged(gpu, d, bs, hq, hkv, dt):
    """Every supported (head_dim, block, group, dtype) with ragged lengths that span
    several splits, partial last blocks and a shared interleaved pool."""
    spec = small_spec(num_seqs=5, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                      kv_dtype=dt, context=("uniform", 1, 700), pool="oversized2x",
                      case_id=1000 + d + bs + hq * 7 + hkv * 3 + (dt == "fp8"))
    case = make_case(spec, seed=1)
    ref, ref_lse = run_oracle(case)
    out, lse = run_step(gpu, to_device(case), case)
    assert_parity(out, lse, ref, ref_lse, str((d, bs, hq, hkv, dt)))


@pytest.mark.parametrize("ctx", [1, 2, 15, 16, 17, 31, 32, 33, 127, 128, 129, 4095, 4096, 4097,
                                 8191, 8193, 9000])
def test_context_edges(gpu, ctx):
    """Lengths at block, chunk and split boundaries."""
    spec = small_spec(num_seqs=1, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                      context=ctx, case_id=2000 + ctx)
    case = make_case(spec, seed=2)
    ref, ref_lse = run_oracle(case)
    out, lse = run_step(gpu, to_device(case), case)
    assert_parity(out, lse, ref, ref_lse, f"ctx={ctx}")


def test_ctx1_is_exact(gpu):
    """With one token the softmax weight is exactly 1: out equals v_0 bit for bit."""
    spec = small_spec(num_seqs=3, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                      context=1, case_id=2100)
    case = make_case(spec, seed=3)
    ref, _ = run_oracle(case)
    out, _ = run_step(gpu, to_device(case), case)
    assert np.array_equal(out, ref)


def test_empty_and_mixed_batch(gpu):
    spec = small_spec(num_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                      context=50, case_id=2200)
    case = make_case(spec, seed=4, context_lens=[0, 50, 0, 300])
    ref, ref_lse = run_oracle(case)
    out, lse = run_step(gpu, to_device(case), case)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(lse[0] == -np.inf) and np.all(lse[2] == -np.inf)
    assert_parity(out, lse, ref, ref_lse, "mixed")


@pytest.mark.parametrize("lens", [
    [9000] + [3] * 19,                                       # one long among many tiny
    [1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987, 1597, 2584, 4181],
])
def test_ragged_batch_shares_workgroups(gpu, lens):
    """Ragged batches share each KV head's workgroups out by length; every sequence
    still matches the oracle."""
    spec = small_spec(num_seqs=len(lens), num_q_heads=16, num_kv_heads=4, head_dim=128,
                      block_size=16, context=max(lens), case_id=2800 + len(lens))
    case = make_case(spec, seed=10, context_lens=lens)
    ref, ref_lse = run_oracle(case)
    out, lse = run_step(gpu, to_device(case), case)
    assert_parity(out, lse, ref, ref_lse, f"ragged {len(lens)}")


@pytest.mark.parametrize("nseq", [64, 65])
def test_ragged_batch_at_the_lane_limit(gpu, nseq):
    """64 sequences (the most one wave shares out) and 65 (the uniform plan)."""
    lens = np.random.default_rng(nseq).integers(1, 1500, nseq).tolist()
    spec = small_spec(num_seqs=nseq, num_q_heads=8, num_kv_heads=1, head_dim=64,
                      block_size=16, context=1500, case_id=2900 + nseq)
    case = make_case(spec, seed=11, context_lens=lens)
    ref, ref_lse = run_oracle(case)
    out, lse = run_step(gpu, to_device(case), case)
    assert_parity(out, lse, ref, ref_lse, f"{nseq} sequences")


@pytest.mark.parametrize("dt,hq", [("bf16", 32), ("bf16", 8), ("fp8", 8), ("fp8_kivi", 8)])
def test_ragged_batch_on_four_wave_workgroups(gpu, dt, hq):
    """Ragged batches whose 8-wave plan gives each sequence at most two splits run
    on 4-wave workgroups (twice the slots to share out by length): the matrix path
    (G = 4) and the vector path (G = 1) on bf16, fp8 and KIVI pools."""
    lens = np.random.default_rng(24).integers(1, 1500, 24).tolist()
    spec = small_spec(num_seqs=24, num_q_heads=hq, num_kv_heads=8, head_dim=128, block_size=16,
                      kv_dtype=dt, context=1500, case_id=2950 + hq + len(dt))
    case = make_case(spec, seed=12, context_lens=lens)
    ref, ref_lse = run_oracle(case)
    out, lse = run_step(gpu, to_device(case), case)
    assert_parity(out, lse, ref, ref_lse, f"24 ragged sequences, {dt}, H_q {hq}")


def test_ragged_batch_with_invalid_lengths(gpu):
    """Invalid lengths inside a ragged batch: those sequences get NaN (negative, or
    longer than the launch hint), an empty one gets zeros, the rest match the oracle."""
    spec = small_spec(num_seqs=6, num_q_heads=8, num_kv_heads=2, head_dim=128,
                      block_size=16, context=2000, case_id=3000)
    case = make_case(spec, seed=12, context_lens=[500, 10, 1200, 1500, 0, 70])
    ref, ref_lse = run_oracle(case)
    bad = dict(case)
    bad["context_lens"] = case["context_lens"].copy()
    bad["context_lens"][1] = -3
    out, lse = run_step(gpu, to_device(bad), bad, max_context_len=1400)   # 1500 > hint
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(lse[1]))
    assert np.all(np.isnan(out[3])) and np.all(np.isnan(lse[3]))
    assert np.all(out[4] == 0) and np.all(lse[4] == -np.inf)
    keep = [0, 2, 5]
    assert_parity(out[keep], lse[keep], ref[keep], ref_lse[keep], "valid sequences")


@pytest.mark.parametrize("lens", [
    [3000, 17, 700, 1, 2048, 129],
    [int(n) for n in np.random.default_rng(31).integers(1, 2000, 24)],   # 4-wave workgroups
], ids=["6 sequences", "24 sequences"])
def test_fused_append_ragged_batch(gpu, lens):
    """The fused append with a ragged batch: each sequence's new token is committed by
    the workgroup that owns its slot, and attention matches the oracle."""
    spec = small_spec(num_seqs=len(lens), num_q_heads=32, num_kv_heads=8, head_dim=128,
                      block_size=16, context=max(lens), append=True, case_id=3100 + len(lens))
    case = make_case(spec, seed=13, context_lens=lens)
    ref, ref_lse = run_oracle(case)
    dev = to_device(case)
    out, lse = run_fused_step(gpu, dev, case)
    assert_parity(out, lse, ref, ref_lse, "fused ragged")
    k = dev["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    v = dev["v_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(k, case["k_pool_full"]) and np.array_equal(v, case["v_pool_full"])


def test_zero_sequences_is_a_no_op(gpu):
    import torch
    spec = small_spec(num_seqs=1, context=20, case_id=2300)
    case = make_case(spec, seed=5)
    dev = to_device(case)
    q = dev["q"][:0]
    out, lse = gpu.paged_decode_attention(q, dev["k_cache"], dev["v_cache"], dev["block_tables"][:0],
                                          dev["context_lens"][:0], 20)
    torch.cuda.synchronize()
    assert out.shape[0] == 0


def test_long_context_beyond_hint_gives_nan(gpu):
    """A sequence longer than max_context_len is flagged with NaN, not truncated."""
    spec = small_spec(num_seqs=2, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                      context=3000, case_id=2400)
    case = make_case(spec, seed=6, context_lens=[3000, 100])
    ref, ref_lse = run_oracle(case)
    out, lse = run_step(gpu, to_device(case), case, max_context_len=200)
    assert np.all(np.isnan(out[0])) and np.all(np.isnan(lse[0]))
    assert_parity(out[1:], lse[1:], ref[1:], ref_lse[1:], "in-range sequence")


def test_bad_block_id_gives_nan(gpu):
    spec = small_spec(num_seqs=2, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                      context=100, case_id=2500)
    case = make_case(spec, seed=7)
    ref, ref_lse = run_oracle(case)
    case["block_tables"][0, 3] = case["k_pool"].shape[0] + 5      # out of range
    out, lse = run_step(gpu, to_device(case), case)
    assert np.all(np.isnan(out[0])) and np.all(np.isnan(lse[0]))
    assert_parity(out[1:], lse[1:], ref[1:], ref_lse[1:], "other sequence")


def test_large_scores_stay_finite(gpu):
    """Scores spread over hundreds of nats exercise the lazy max update."""
    spec = small_spec(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                      context=2000, case_id=2600)
    case = make_case(spec, seed=8)
    case["softmax_scale"] = 4.0          # scores ~ N(0, 16 * 128)
    ref, ref_lse = run_oracle(case)
    out, lse = run_step(gpu, to_device(case), case)
    assert_parity(out, lse, ref, ref_lse, "large scores")


@pytest.mark.parametrize("name", ["llama8b", "long"])
def test_fused_append_attention_full_size(gpu, name):
    """The fused step (append + attention in one kernel) matches the oracle, and leaves
    the cache bit-identical to the oracle's append."""
    case = named_case(name)
    ref, ref_lse = named_reference(name)
    dev = to_device(case)
    out, lse = run_fused_step(gpu, dev, case)
    assert_parity(out, lse, ref, ref_lse, f"fused {name}")
    k = dev["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    v = dev["v_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(k, case["k_pool_full"]) and np.array_equal(v, case["v_pool_full"])


@pytest.mark.parametrize("hq,hkv", [(16, 4), (8, 8), (64, 8)])   # matrix G=4, vector G=1, G=8
@pytest.mark.parametrize("ctx", [1, 17, 129, 700, 4097])
def test_fused_append_matches_two_calls_bitwise(gpu, ctx, hq, hkv):
    """The fused step equals the append followed by attention, bit for bit: the new
    row sits in a wave's first chunk (ctx 1, 17) or in a later one."""
    spec = small_spec(num_seqs=3, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=16,
                      context=ctx, append=True, case_id=2700 + ctx + hq)
    case = make_case(spec, seed=9)
    o1, l1 = run_step(gpu, to_device(case), case)
    o2, l2 = run_fused_step(gpu, to_device(case), case)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_workspace_reused_across_calls(gpu):
    """Arrival counters return to zero: a workspace serves consecutive calls, including
    a call with a smaller batch and shorter contexts."""
    spec = small_spec(num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=("uniform", 500, 6000), append=True, case_id=2800)
    case = make_case(spec, seed=10)
    hint = case["block_tables"].shape[1] * 16
    dev = to_device(case)
    shape = gpu.make_shape(4, 32, dev["k_cache"], dev["block_tables"])
    ws = torch.full((gpu.workspace_size(shape, hint),), 0xAB, dtype=torch.uint8, device="cuda:0")
    gpu.workspace_init(shape, hint, ws)
    ref, ref_lse = run_oracle(case)
    for _ in range(3):
        fresh = to_device(case)
        out, lse = run_fused_step(gpu, fresh, case, max_context_len=hint, workspace=ws)
        assert_parity(out, lse, ref, ref_lse, "reused workspace")
    small = dict(case)
    for key in ("q", "block_tables", "context_lens", "positions", "k_new", "v_new"):
        small[key] = case[key][:2]
    out2, lse2 = run_fused_step(gpu, to_device(small), small, max_context_len=hint, workspace=ws)
    assert_parity(out2, lse2, ref[:2], ref_lse[:2], "smaller call")


def test_fp8_grouped_long_context_on_the_matrix_path(gpu):
    """fp8 KV at the 32K workload's head geometry (64/8 heads, G = 8, d 128, block 32)
    on the matrix path: codes widened to bf16, block scales folded into scores and
    weights.  Two ragged sequences of 16385 and 9000 tokens."""
    spec = small_spec(num_seqs=2, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=32,
                      kv_dtype="fp8", context=16385, case_id=7600)
    case = make_case(spec, seed=0, context_lens=[16385, 9000])
    ref, ref_lse = run_oracle(case)
    out, lse = run_step(gpu, to_device(case), case)
    assert_parity(out, lse, ref, ref_lse, "fp8 G=8 long context")


@pytest.mark.parametrize("hq,hkv,dt", [(4, 4, "fp8"), (16, 4, "fp8"), (16, 4, "fp8_kivi"),
                                       (8, 8, "fp8_kivi")])
def test_unused_block_scales_are_never_used(gpu, hq, hkv, dt):
    """Regression: the part of a split's last chunk past its end reads a stand-in
    block (block 0) and multiplies weights of 0 by that block's scales.  Block 0 is
    made unused here and its scales are NaN; the outputs must still match the
    oracle, which never reads it.  The lengths end 16 or 8 tokens into a 32-token
    chunk; G = 1 runs the vector path, G = 4 the matrix path, and KIVI the vector
    path with per-channel and per-token scales."""
    lens = [48, 1000, 2064, 7]
    spec = small_spec(num_seqs=4, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=16,
                      kv_dtype=dt, context=2064, pool="oversized2x", case_id=7800 + hq)
    case = make_case(spec, seed=3, context_lens=lens)
    tab = case["block_tables"]
    used = set(int(x) for x in tab.ravel() if x >= 0)
    u = next(i for i in range(case["k_pool"].shape[0]) if i not in used)
    # without an append the pool before and after it is one array: swap each once
    arrays = {id(case[key]): case[key] for key in
              ("k_pool", "v_pool", "k_pool_full", "v_pool_full", "k_scale", "v_scale")}
    for a in arrays.values():
        a[[0, u]] = a[[u, 0]]
    tab[tab == 0] = u
    assert 0 not in set(int(x) for x in tab.ravel())
    case["k_scale"][0] = np.nan
    case["v_scale"][0] = np.nan
    ref, ref_lse = run_oracle(case)
    out, lse = run_step(gpu, to_device(case), case)
    assert_parity(out, lse, ref, ref_lse, f"NaN scales in unused block 0, G={hq // hkv} {dt}")


@pytest.mark.parametrize("hq,hkv,dt", [(128, 8, "bf16"), (32, 1, "bf16"), (64, 4, "fp8"),
                                       (32, 1, "fp8")])
def test_sixteen_or_more_query_heads_per_kv_head(gpu, hq, hkv, dt):
    """One position with G = 16 or 32 (multi-query attention at G = 32): 16 or more
    rows per KV head, so K is staged through LDS and the splits merge in a launch
    of their own.  Ragged lengths with an empty sequence; bf16 also through the
    fused append-and-attend entry point."""
    lens = [2500, 37, 0, 1200, 640]
    spec = small_spec(num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                      block_size=16, kv_dtype=dt, context=2500, append=(dt == "bf16"),
                      case_id=5300 + hq + hkv + (dt == "fp8"))
    case = make_case(spec, seed=2, context_lens=lens)
    ref, ref_lse = run_oracle(case)
    out, lse = run_step(gpu, to_device(case), case)
    assert_parity(out, lse, ref, ref_lse, f"G={hq // hkv} {dt}")
    if dt == "bf16":
        out, lse = run_fused_step(gpu, to_device(case), case)
        assert_parity(out, lse, ref, ref_lse, f"fused, G={hq // hkv}")
