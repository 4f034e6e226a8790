"""The Python binding rejects tensors the kernels would read out of bounds (another
dtype, size or layout, or host memory) before any pointer crosses the boundary.
Runs on the CPU: every case fails in the binding's checks, so no kernel launches."""
import pytest
import torch

import gqa_decode_attention_paged_amd as gqa

NB, HKV, BS, D, B, HQ, MB = 12, 2, 16, 64, 2, 8, 6


def _case(dtype=torch.bfloat16):
    pools = torch.zeros((NB, HKV, BS, D), dtype=dtype)
    return dict(q=torch.zeros((B, HQ, D), dtype=torch.bfloat16), k_cache=pools,
                v_cache=pools.clone(), block_tables=torch.zeros((B, MB), dtype=torch.int32),
                context_lens=torch.full((B,), 40, dtype=torch.int32))


def _attend(c, **over):
    args = {**c, **over}
    return gqa.paged_decode_attention(args["q"], args["k_cache"], args["v_cache"],
                                      args["block_tables"], args["context_lens"], 96,
                                      k_scale=args.get("k_scale"), v_scale=args.get("v_scale"))


def test_host_tensors_are_rejected():
    with pytest.raises(ValueError, match="GPU memory"):
        _attend(_case())


def test_int64_tables_are_rejected():
    c = _case()
    with pytest.raises(TypeError, match="block_tables"):
        _attend(c, block_tables=c["block_tables"].long())
    with pytest.raises(TypeError, match="context_lens"):
        _attend(c, context_lens=c["context_lens"].long())


def test_float32_query_is_rejected():
    c = _case()
    with pytest.raises(TypeError, match="q:"):
        _attend(c, q=c["q"].float())


def test_strided_query_is_rejected():
    c = _case()
    wide = torch.zeros((B, HQ, 2 * D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="contiguous"):
        _attend(c, q=wide[:, :, ::2])


def test_head_dim_mismatch_is_rejected():
    c = _case()
    with pytest.raises(ValueError, match="head dim"):
        _attend(c, q=torch.zeros((B, HQ, 2 * D), dtype=torch.bfloat16))


def test_short_tables_and_lengths_are_rejected():
    c = _case()
    with pytest.raises(ValueError, match="block_tables"):
        _attend(c, block_tables=c["block_tables"][:1])
    with pytest.raises(ValueError, match="context_lens"):
        _attend(c, context_lens=c["context_lens"][:1])


def test_pools_must_match():
    c = _case()
    with pytest.raises(ValueError, match="v_cache"):
        _attend(c, v_cache=torch.zeros((NB, HKV, BS // 2, D), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="v_cache"):
        _attend(c, v_cache=torch.zeros((NB, HKV, BS, D), dtype=torch.uint8))


def test_fp8_scale_layouts_are_checked():
    c = _case(torch.uint8)
    good = torch.ones((NB, HKV), dtype=torch.float32)
    with pytest.raises(ValueError, match="v_scale"):
        _attend(c, k_scale=good, v_scale=torch.ones((NB, HKV + 1), dtype=torch.float32))
    # KIVI: keys per channel [NB][H_kv][d_h], values per token [NB][H_kv][BS]
    with pytest.raises(ValueError, match="v_scale"):
        _attend(c, k_scale=torch.ones((NB, HKV, D), dtype=torch.float32), v_scale=good)
    with pytest.raises(TypeError, match="k_scale"):
        _attend(c, k_scale=good.double(), v_scale=good)


def test_append_rows_must_match_the_pools():
    c = _case()
    k_new = torch.zeros((B, HKV, D + 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k_new"):
        gqa.kv_append(k_new, k_new.clone(), c["k_cache"], c["v_cache"], c["block_tables"],
                      torch.zeros(B, dtype=torch.int32))


def test_copy_lists_must_pair_up():
    c = _case()
    with pytest.raises(ValueError, match="dst_blocks"):
        gqa.kv_copy_blocks(c["k_cache"], c["v_cache"], torch.zeros(3, dtype=torch.int32),
                           torch.zeros(2, dtype=torch.int32))
    with pytest.raises(TypeError, match="src_blocks"):
        gqa.kv_copy_blocks(c["k_cache"], c["v_cache"], torch.zeros(3, dtype=torch.int64),
                           torch.zeros(3, dtype=torch.int32))


def test_fused_step_rows_and_positions_are_checked():
    c = _case()
    k_new = torch.zeros((B, HKV, D), dtype=torch.bfloat16)
    pos = torch.zeros(B, dtype=torch.int32)

    def fused(**over):
        a = {**c, "k_new": k_new, "v_new": k_new.clone(), "positions": pos, **over}
        return gqa.paged_decode_append_attention(a["q"], a["k_new"], a["v_new"], a["positions"],
                                                 a["k_cache"], a["v_cache"], a["block_tables"],
                                                 a["context_lens"], 96)
    with pytest.raises(ValueError, match="k_new"):
        fused(k_new=torch.zeros((B, HKV + 1, D), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="positions"):
        fused(positions=pos.long())
    with pytest.raises(ValueError, match="GPU memory"):
        fused()


def test_multi_position_outputs_are_checked():
    c = _case()
    Q = 3
    q = torch.zeros((B, Q, HQ, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out:"):
        gqa.paged_decode_multi_query(q, c["k_cache"], c["v_cache"], c["block_tables"],
                                     c["context_lens"], 96,
                                     out=torch.zeros((B, HQ, D), dtype=torch.float32))
    with pytest.raises(ValueError, match="out_lse"):
        gqa.paged_decode_multi_query(q, c["k_cache"], c["v_cache"], c["block_tables"],
                                     c["context_lens"], 96,
                                     out_lse=torch.zeros((B, HQ), dtype=torch.float32))
