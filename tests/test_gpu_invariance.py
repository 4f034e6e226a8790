"""GPU invariants: physical placement, batch composition, fp8 code decoding."""
import numpy as np
import pytest

import oracle
from tests._dev import assert_parity, run_fused_step, run_oracle, to_device, run_step
from workloads import make_case, small_spec

pytestmark = pytest.mark.gpu


def test_block_permutation_is_bit_identical(gpu):
    """Results follow logical positions, not where blocks sit in the pool."""
    spec = small_spec(num_seqs=3, num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                      context=("uniform", 100, 3000), case_id=4000)
    case = make_case(spec, seed=1)
    out, lse = run_step(gpu, to_device(case), case)
    rng = np.random.default_rng(9)
    perm = rng.permutation(case["k_pool"].shape[0])
    moved = dict(case)
    for key in ("k_pool", "v_pool"):
        moved[key] = np.empty_like(case[key])
        moved[key][perm] = case[key]
    bt = case["block_tables"].copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    moved["block_tables"] = bt
    out2, lse2 = run_step(gpu, to_device(moved), moved)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def _batch_case():
    spec = small_spec(num_seqs=6, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=("uniform", 1, 9000), case_id=4001)
    return make_case(spec, seed=2)


def _one(case, b):
    one = dict(case)
    for key in ("q", "block_tables", "context_lens", "positions"):
        one[key] = case[key][b:b + 1]
    return one


def test_batch_invariant_mode_bitwise(gpu):
    """With the batch-invariant flag a sequence gives the same bits alone and in a
    batch, whatever the launch hint."""
    case = _batch_case()
    hint = case["block_tables"].shape[1] * 16          # the largest length the tables allow
    out, lse = run_step(gpu, to_device(case), case, max_context_len=hint, batch_invariant=True)
    for b in (0, 3, 5):
        one = _one(case, b)
        o1, l1 = run_step(gpu, to_device(one), one, batch_invariant=True)   # smaller hint
        assert np.array_equal(o1[0], out[b]) and np.array_equal(l1[0], lse[b])


def test_default_mode_order_invariant_and_batch_consistent(gpu):
    """Default mode: reordering the batch changes no bit; a sequence alone agrees with
    its batched result to fp32 rounding (the split count follows the batch size)."""
    case = _batch_case()
    hint = case["block_tables"].shape[1] * 16
    out, lse = run_step(gpu, to_device(case), case, max_context_len=hint)
    rev = dict(case)
    for key in ("q", "block_tables", "context_lens", "positions"):
        rev[key] = np.ascontiguousarray(case[key][::-1])
    o2, l2 = run_step(gpu, to_device(rev), rev, max_context_len=hint)
    assert np.array_equal(o2[::-1], out) and np.array_equal(l2[::-1], lse)
    for b in (0, 3, 5):
        one = _one(case, b)
        o1, l1 = run_step(gpu, to_device(one), one)
        assert np.max(np.abs(o1[0] - out[b])) <= 1e-5 and np.max(np.abs(l1[0] - lse[b])) <= 1e-5


@pytest.fixture
def split_override(gpu):
    """The binding, with the split-length override cleared again afterwards."""
    yield gpu
    gpu.set_split_tokens(0)


@pytest.mark.parametrize("tokens", [256, 1024, 4128])   # 4128: T / 32 needs the high plan bits
def test_split_length_override_is_batch_invariant(split_override, tokens):
    """With a split-length override the results match the oracle, and a sequence
    gives the same bits alone (small hint) and in the batch (large hint)."""
    gpu = split_override
    case = _batch_case()
    hint = case["block_tables"].shape[1] * 16
    ref, ref_lse = run_oracle(case)
    gpu.set_split_tokens(tokens)
    out, lse = run_step(gpu, to_device(case), case, max_context_len=hint)
    assert_parity(out, lse, ref, ref_lse, f"split length {tokens}")
    for b in (0, 3, 5):
        one = _one(case, b)
        o1, l1 = run_step(gpu, to_device(one), one)
        assert np.array_equal(o1[0], out[b]) and np.array_equal(l1[0], lse[b]), b


def test_split_length_128_is_the_batch_invariant_plan(split_override):
    """An override of 128 tokens is the batch-invariant flag's own plan: same bits."""
    gpu = split_override
    case = _batch_case()
    o_flag, l_flag = run_step(gpu, to_device(case), case, batch_invariant=True)
    gpu.set_split_tokens(128)
    o_t, l_t = run_step(gpu, to_device(case), case)
    assert np.array_equal(o_flag, o_t) and np.array_equal(l_flag, l_t)


def test_split_length_override_fused_append(split_override):
    """The fused append step under an override (G = 8, block 32, a split boundary
    inside the sequences): cache bits and attention against the oracle."""
    gpu = split_override
    spec = small_spec(num_seqs=3, num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=32,
                      context=("uniform", 700, 3000), append=True, case_id=4002)
    case = make_case(spec, seed=4)
    ref, ref_lse = run_oracle(case)
    gpu.set_split_tokens(512)
    dev = to_device(case)
    out, lse = run_fused_step(gpu, dev, case)
    assert_parity(out, lse, ref, ref_lse, "fused append, split length 512")
    import torch
    k = dev["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    v = dev["v_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(k, case["k_pool_full"]) and np.array_equal(v, case["v_pool_full"])


def test_fp8_codes_decode_exactly(gpu):
    """ctx = 1 makes out = decode(code) * scale exactly: all 254 finite codes."""
    spec = small_spec(num_seqs=1, num_q_heads=2, num_kv_heads=2, head_dim=128, block_size=16,
                      kv_dtype="fp8", context=1, pool="exact", case_id=4002)
    case = make_case(spec, seed=3)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = np.concatenate([codes, codes[:2]])                   # 256 values, 2 heads x 128
    blk = case["block_tables"][0, 0]
    for pool in ("v_pool", "v_pool_full"):
        case[pool][blk, :, 0, :] = codes.reshape(2, 128)
    case["v_scale"][blk, :] = np.float32(1.0)
    out, _ = run_step(gpu, to_device(case), case)
    want = oracle.decode_e4m3fn(codes).reshape(2, 128)
    assert np.array_equal(out[0], want)
