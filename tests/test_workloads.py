"""Properties of the seeded input generators (shapes, placement, poison, fp8 scales)."""
import numpy as np
import pytest

from oracle import decode_e4m3fn, bf16_to_float64
from workloads import make_case, small_spec, SPECS


def test_deterministic():
    a = make_case("tiny", seed=0)
    b = make_case("tiny", seed=0)
    c = make_case("tiny", seed=1)
    assert np.array_equal(a["k_pool"], b["k_pool"]) and np.array_equal(a["q"], b["q"])
    assert not np.array_equal(a["q"], c["q"])


def test_tiny_is_a_permutation_of_eight_blocks():
    c = make_case("tiny")
    assert c["k_pool"].shape == (8, 1, 16, 64)
    assert sorted(c["block_tables"][0].tolist()) == list(range(8))
    assert c["block_tables"][0].tolist() != list(range(8))
    assert c["context_lens"].tolist() == [128]
    assert c["q"].shape == (1, 4, 64)


def test_values_are_standard_normal_bf16():
    c = make_case("tiny")
    x = bf16_to_float64(c["k_pool"]).ravel()
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05


def test_ragged_uniform_lengths_and_shared_interleaved_pool():
    spec = small_spec(num_seqs=16, context=("uniform", 512, 8192), pool="exact", head_dim=8,
                      num_q_heads=4, num_kv_heads=2, case_id=2)
    c = make_case(spec)
    ctx = c["context_lens"]
    assert ctx.min() >= 512 and ctx.max() <= 8192 and np.any(ctx % 16 != 0)
    nb = (ctx + 15) // 16
    assert c["k_pool"].shape[0] == nb.sum()
    owned = np.concatenate([c["block_tables"][b, :nb[b]] for b in range(16)])
    assert sorted(owned.tolist()) == list(range(nb.sum()))


def test_poison_marks_exactly_the_invalid_slots():
    c = make_case(small_spec(num_seqs=2, block_size=16, context=("uniform", 3, 40), case_id=9), seed=4)
    x = bf16_to_float64(c["k_pool_full"])
    valid = np.zeros(x.shape[0] * 16, bool).reshape(-1, 16)
    for b in range(2):
        for t in range(int(c["context_lens"][b])):
            valid[c["block_tables"][b][t // 16], t % 16] = True
    nanslot = np.isnan(x).all(axis=(1, 3))
    assert np.array_equal(nanslot, ~valid)


def test_append_case_poisons_the_target_slot_before_the_append():
    c = make_case(small_spec(num_seqs=2, context=20, append=True, case_id=10), seed=1)
    assert c["positions"].tolist() == [19, 19]
    for b in range(2):
        blk = c["block_tables"][b][1]
        assert np.isnan(bf16_to_float64(c["k_pool"][blk, :, 3])).all()
        assert np.array_equal(c["k_pool_full"][blk, :, 3], c["k_new"][b])


def test_fp8_scale_is_amax_over_448():
    spec = small_spec(num_seqs=2, num_q_heads=4, num_kv_heads=4, head_dim=32, kv_dtype="fp8",
                      context=("uniform", 5, 60), case_id=11)
    c = make_case(spec, seed=2)
    codes = c["k_pool_full"]
    vals = decode_e4m3fn(codes)
    nb = (c["context_lens"] + 15) // 16
    for b in range(2):
        for i in range(nb[b]):
            blk = c["block_tables"][b][i]
            for h in range(4):
                # the block's largest source magnitude maps exactly to 448
                assert np.nanmax(np.abs(vals[blk, h])) == 448.0
                assert c["k_scale"][blk, h] > 0


def test_spec_table():
    assert SPECS["llama8b"].group == 4 and SPECS["long"].group == 8 and SPECS["mha_fp8"].group == 1
    assert SPECS["long"].context == 32769 and SPECS["long"].block_size == 32
