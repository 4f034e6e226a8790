"""GPU parity of multi-position queries (speculative verification): the new
tokens are committed with gqa_kv_append_tokens, then gqa_paged_decode_multi_query
attends for every query position, compared with the float64 oracle.  Same bar
as the single-query path: max-abs <= 1e-2, relative L2 <= 2e-3, lse within 1e-3."""
import numpy as np
import pytest
import torch

import oracle
from tests._dev import to_device, assert_parity
from workloads import make_multi_query_case, small_spec

pytestmark = pytest.mark.gpu


def _reference(case):
    s = case["spec"]
    return oracle.paged_multi_query_attention(case["q"], case["k_pool_full"], case["v_pool_full"],
                                              case["block_tables"], case["context_lens"],
                                              s.block_size, case["softmax_scale"], s.kv_dtype,
                                              case["k_scale"], case["v_scale"])


def _verify_step(gqa, case, dev, max_context_len=None, batch_invariant=False):
    """Commit the Q new tokens (bf16 pools), then attend for all Q positions."""
    if case["k_new"] is not None:
        gqa.kv_append_tokens(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                             dev["block_tables"], dev["positions"])
    if max_context_len is None:
        max_context_len = int(case["context_lens"].max())
    out, lse = gqa.paged_decode_multi_query(dev["q"], dev["k_cache"], dev["v_cache"],
                                            dev["block_tables"], dev["context_lens"],
                                            max_context_len, case["softmax_scale"],
                                            dev["k_scale"], dev["v_scale"],
                                            batch_invariant=batch_invariant)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("hq,hkv,nq,d,bs,dt", [
    (32, 8, 4, 128, 16, "bf16"),     # G=4, 4 positions: 16 rows, a full MFMA tile
    (64, 8, 2, 128, 32, "bf16"),     # G=8, 2 positions
    (8, 8, 16, 128, 16, "bf16"),     # MHA, 16 positions
    (16, 8, 3, 64, 16, "bf16"),      # 6 rows in an 8-row tile
    (32, 8, 3, 128, 16, "bf16"),     # 12 rows in a 16-row tile
    (8, 8, 1, 128, 32, "bf16"),      # one row: the vector path
    (64, 8, 4, 128, 32, "bf16"),     # G=8, 4 positions: 32 rows, two row tiles (the 32K shape)
    (32, 8, 8, 128, 16, "bf16"),     # G=4, 8 positions: 32 rows
    (64, 8, 3, 64, 16, "bf16"),      # 24 rows in a 32-row capacity, d=64
    (4, 4, 2, 128, 16, "fp8"),
    (16, 4, 2, 64, 32, "fp8"),
    (8, 8, 8, 128, 16, "fp8"),
    (64, 8, 4, 128, 32, "fp8"),      # fp8, G=8, 4 positions: 32 rows (matrix path)
    (32, 8, 4, 128, 16, "fp8"),      # fp8, 16 rows
    (16, 8, 3, 64, 16, "fp8"),       # fp8, 6 rows, d=64
    (128, 8, 2, 128, 16, "bf16"),    # G=16, 2 positions: 32 rows
    (32, 1, 1, 64, 32, "fp8"),       # G=32 (multi-query attention), one position
])
def test_multi_query_parity(gpu, hq, hkv, nq, d, bs, dt):
    lens = [nq, nq + 1, 100, 1000, 3000]
    spec = small_spec(num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                      block_size=bs, kv_dtype=dt, context=3000, case_id=6000 + hq * 10 + nq)
    case = make_multi_query_case(spec, nq, seed=3, context_lens=lens, append=(dt == "bf16"))
    ref, ref_lse = _reference(case)
    dev = to_device(case)
    out, lse = _verify_step(gpu, case, dev)
    assert_parity(out, lse, ref, ref_lse, f"G={hq // hkv} Q={nq} d={d} bs={bs} {dt}")
    if dt == "bf16":
        k = dev["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(k, case["k_pool_full"])


@pytest.mark.parametrize("hq,nq,dt", [(32, 4, "bf16"), (8, 2, "bf16"), (8, 4, "fp8")])
def test_multi_query_ragged_on_four_wave_workgroups(gpu, hq, nq, dt):
    """24 ragged sequences x 8 KV heads: the 8-wave plan gives each at most two
    splits, so the call runs on 4-wave workgroups sharing slots out by length."""
    lens = [int(n) for n in np.random.default_rng(nq).integers(nq, 1500, 24)]
    spec = small_spec(num_seqs=24, num_q_heads=hq, num_kv_heads=8, head_dim=128,
                      block_size=16, kv_dtype=dt, context=1500, case_id=6700 + hq + nq)
    case = make_multi_query_case(spec, nq, seed=5, context_lens=lens, append=(dt == "bf16"))
    ref, ref_lse = _reference(case)
    out, lse = _verify_step(gpu, case, to_device(case))
    assert_parity(out, lse, ref, ref_lse, f"24 ragged sequences, G={hq // 8} Q={nq} {dt}")


@pytest.mark.parametrize("nq,dt", [(4, "bf16"), (2, "fp8")])
def test_one_long_sequence_among_short_ones_merged_in_second_launch(gpu, nq, dt):
    """16 or more rows merge in a launch of their own, which loads the splits
    below the launch's per-sequence split count S together with the count.  The
    length-proportional sharing gives the long sequence about 0.87 of the 8 S
    slots of each KV head (capped at 7000 / 128 splits), far more than S, so the
    merge also loads the rest."""
    lens = [7000] + [nq + 37 * i for i in range(1, 8)]
    spec = small_spec(num_seqs=8, num_q_heads=32 if dt == "bf16" else 64, num_kv_heads=8,
                      head_dim=128, block_size=16, kv_dtype=dt, context=7000,
                      case_id=6750 + nq)
    case = make_multi_query_case(spec, nq, seed=9, context_lens=lens, append=(dt == "bf16"))
    ref, ref_lse = _reference(case)
    out, lse = _verify_step(gpu, case, to_device(case))
    assert_parity(out, lse, ref, ref_lse, f"one long sequence, Q={nq} {dt}")


@pytest.mark.parametrize("batch_invariant", [False, True])
@pytest.mark.parametrize("hq,hkv,nq,dt", [(32, 8, 2, "bf16"), (32, 8, 4, "bf16"),
                                          (8, 4, 2, "fp8"), (8, 4, 4, "fp8")])
def test_rows_that_see_no_token_of_a_split(gpu, hq, hkv, nq, dt, batch_invariant):
    """Regression: at 385, 386 and 513 tokens the last 128-token split holds fewer
    tokens than the Q query positions, so some rows see none of its tokens; their
    partial must weigh zero in the merge rather than turn the output into NaN.
    Uniform batches of each length, then one ragged batch of all of them."""
    batches = [[385] * 3, [386] * 3, [513] * 3, [385, 386, 513, 1000]]
    for n, lens in enumerate(batches):
        spec = small_spec(num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                          block_size=16, kv_dtype=dt, context=1000,
                          case_id=6800 + 10 * n + hq + nq)
        case = make_multi_query_case(spec, nq, seed=11, context_lens=lens,
                                     append=(dt == "bf16"))
        ref, ref_lse = _reference(case)
        out, lse = _verify_step(gpu, case, to_device(case), batch_invariant=batch_invariant)
        assert_parity(out, lse, ref, ref_lse, f"lens={lens} G={hq // hkv} Q={nq} {dt}")
        if dt == "bf16":            # the fused verification step on the same lengths
            d = to_device(case)
            o2, l2 = gpu.paged_decode_multi_query_append(
                d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["block_tables"],
                d["context_lens"], max(lens), batch_invariant=batch_invariant)
            torch.cuda.synchronize()
            assert_parity(o2.cpu().numpy().astype(np.float64),
                          l2.cpu().numpy().astype(np.float64), ref, ref_lse,
                          f"fused, lens={lens} G={hq // hkv} Q={nq}")


def test_single_position_matches_the_decode_entry_point_bitwise(gpu):
    spec = small_spec(num_seqs=3, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=2000, case_id=6100)
    case = make_multi_query_case(spec, 1, seed=4, context_lens=[2000, 700, 33], append=False)
    dev = to_device(case)
    o1, l1 = gpu.paged_decode_multi_query(dev["q"], dev["k_cache"], dev["v_cache"],
                                          dev["block_tables"], dev["context_lens"], 2000)
    o2, l2 = gpu.paged_decode_attention(dev["q"][:, 0].contiguous(), dev["k_cache"],
                                        dev["v_cache"], dev["block_tables"],
                                        dev["context_lens"], 2000)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, 0], o2) and torch.equal(l1[:, 0], l2)


def test_malformed_and_empty_contexts(gpu):
    spec = small_spec(num_seqs=4, num_q_heads=16, num_kv_heads=4, head_dim=64, block_size=16,
                      context=300, case_id=6200)
    case = make_multi_query_case(spec, 4, seed=5, context_lens=[300, 2, 0, 4], append=False)
    ref, ref_lse = _reference(case)
    out, lse = _verify_step(gpu, case, to_device(case))
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(lse[1]))
    assert np.all(out[2] == 0) and np.all(lse[2] == -np.inf)
    keep = [0, 3]
    assert_parity(out[keep], lse[keep], ref[keep], ref_lse[keep], "valid sequences")


@pytest.mark.parametrize("hq,hkv,nq,dt", [(32, 8, 9, "bf16"), (32, 8, 9, "fp8"),
                                          (16, 8, 5, "fp8_kivi")])
def test_too_many_rows_is_unsupported(gpu, hq, hkv, nq, dt):
    """More than 32 rows (G * Q), or 8 for KIVI pools, is refused."""
    spec = small_spec(num_seqs=1, num_q_heads=hq, num_kv_heads=hkv, head_dim=64, block_size=16,
                      kv_dtype=dt, context=64, case_id=6300)
    case = make_multi_query_case(spec, nq, seed=6, append=False)
    dev = to_device(case)
    with pytest.raises(gpu.GqaError) as e:
        gpu.paged_decode_multi_query(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                     dev["context_lens"], 64, None, dev["k_scale"], dev["v_scale"])
    assert e.value.status == 2


def test_batch_invariant_mode(gpu):
    """With the flag, each sequence's bits do not depend on the rest of the batch."""
    spec = small_spec(num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=5000, case_id=6400)
    case = make_multi_query_case(spec, 4, seed=7, context_lens=[5000, 64, 1500, 4096],
                                 append=False)
    ref, ref_lse = _reference(case)
    hint = case["block_tables"].shape[1] * 16
    out, lse = _verify_step(gpu, case, to_device(case), max_context_len=hint,
                            batch_invariant=True)
    assert_parity(out, lse, ref, ref_lse, "batch-invariant")
    one = dict(case)
    for key in ("q", "block_tables", "context_lens", "positions"):
        one[key] = case[key][2:3]
    o1, l1 = _verify_step(gpu, one, to_device(one), batch_invariant=True)
    assert np.array_equal(o1[0], out[2]) and np.array_equal(l1[0], lse[2])


def test_speculative_verify_long_context_g8(gpu):
    """The 32K long-context shape (B=4, 64/8 heads, d=128, block 32) verifying 3
    drafts plus the pending token: 32 rows per (sequence, KV head), fused append."""
    spec = small_spec(num_seqs=4, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=32,
                      context=32772, case_id=6550)
    case = make_multi_query_case(spec, 4, seed=8)
    ref, ref_lse = _reference(case)
    d = to_device(case)
    out, lse = gpu.paged_decode_multi_query_append(d["q"], d["k_new"], d["v_new"], d["k_cache"],
                                                   d["v_cache"], d["block_tables"],
                                                   d["context_lens"], 32772)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                  ref, ref_lse, "verify 32K G=8")


def test_speculative_verify_full_size(gpu):
    """The 8K grouped-query shape (B=1, 32/8 heads, d=128) verifying 3 drafts plus the
    pending token: 4 positions appended, then attended."""
    spec = small_spec(num_seqs=1, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=8192, case_id=6500)
    case = make_multi_query_case(spec, 4, seed=8)
    ref, ref_lse = _reference(case)
    out, lse = _verify_step(gpu, case, to_device(case))
    assert_parity(out, lse, ref, ref_lse, "verify 8K")


@pytest.mark.parametrize("hq,hkv,nq,bs", [(32, 8, 4, 16), (64, 8, 2, 32), (8, 8, 16, 16),
                                          (16, 8, 3, 16), (64, 8, 4, 32)])
def test_fused_verify_step_matches_two_calls_bitwise(gpu, hq, hkv, nq, bs):
    """Fused append + multi-position attention equals the append followed by the
    attention call, bit for bit, and leaves the same cache."""
    lens = [nq, 40, 1000, 3333]
    spec = small_spec(num_seqs=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                      block_size=bs, context=3333, case_id=6600 + hq + nq)
    case = make_multi_query_case(spec, nq, seed=9, context_lens=lens)
    ref, ref_lse = _reference(case)
    d1, d2 = to_device(case), to_device(case)
    o1, l1 = _verify_step(gpu, case, d1)
    o2, l2 = gpu.paged_decode_multi_query_append(d2["q"], d2["k_new"], d2["v_new"], d2["k_cache"],
                                                 d2["v_cache"], d2["block_tables"],
                                                 d2["context_lens"], max(lens))
    torch.cuda.synchronize()
    o2, l2 = o2.cpu().numpy().astype(np.float64), l2.cpu().numpy().astype(np.float64)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    bits = lambda t: t.view(torch.int16)                 # NaN-poisoned slots compare by bits
    assert torch.equal(bits(d1["k_cache"]), bits(d2["k_cache"]))
    assert torch.equal(bits(d1["v_cache"]), bits(d2["v_cache"]))
    assert_parity(o2, l2, ref, ref_lse, "fused verify")


@pytest.mark.parametrize("hq,hkv,nq", [(32, 8, 4), (64, 8, 4)])
def test_unused_block_scales_are_never_used_staged(gpu, hq, hkv, nq):
    """Regression for the variants that stage K through LDS (16 and 32 rows, fp8):
    whole blocks past a split's end read block 0 as a stand-in, and its K scale
    multiplies the scores of a masked tile.  Block 0 is made unused here with NaN
    scales; the outputs must still match the oracle, which never reads it."""
    lens = [48, 1000, 2064, 7]
    spec = small_spec(num_seqs=4, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=16,
                      kv_dtype="fp8", context=2064, pool="oversized2x", case_id=7900 + hq)
    case = make_multi_query_case(spec, nq, seed=3, context_lens=lens, append=False)
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
    ref, ref_lse = _reference(case)
    out, lse = _verify_step(gpu, case, to_device(case))
    assert_parity(out, lse, ref, ref_lse, f"NaN scales in unused block 0, {hq // hkv * nq} rows")


def test_split_length_override_multi_query_fp8(gpu):
    """The split-length override on the staged fp8 path (16 rows): parity, and the
    same bits for a sequence alone and in the batch."""
    spec = small_spec(num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      kv_dtype="fp8", context=3000, case_id=7950)
    case = make_multi_query_case(spec, 4, seed=5, context_lens=[4, 700, 3000, 1500],
                                 append=False)
    ref, ref_lse = _reference(case)
    try:
        gpu.set_split_tokens(256)
        out, lse = _verify_step(gpu, case, to_device(case), max_context_len=3000)
        one = dict(case)
        for key in ("q", "block_tables", "context_lens", "positions"):
            one[key] = case[key][2:3]
        o1, l1 = _verify_step(gpu, one, to_device(one))
    finally:
        gpu.set_split_tokens(0)
    assert_parity(out, lse, ref, ref_lse, "split length 256, fp8, 16 rows")
    assert np.array_equal(o1[0], out[2]) and np.array_equal(l1[0], lse[2])
