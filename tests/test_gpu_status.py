"""GPU checks of the workspace status word: a clean call leaves it zero, and each
kind of bad device-resident input (table entry, context length, launch hint,
append position) sets its bit while the outputs follow the NaN contract.  The
contract checked is the paged table's: every logical block a sequence attends
maps to a physical block of the pool (*Module 10*, "Mapping logical positions
to physical blocks"; *The Mathematics of Transformer Inference* §9)."""
import numpy as np
import pytest
import torch

from tests._dev import to_device, run_oracle, assert_parity
from workloads import make_case, make_multi_query_case, small_spec

pytestmark = pytest.mark.gpu


def _attend(gqa, case, dev, ws, hint=None, fused=False, kv="bf16"):
    hint = int(case["context_lens"].max()) if hint is None else hint
    if fused:
        out, lse = gqa.paged_decode_append_attention(
            dev["q"], dev["k_new"], dev["v_new"], dev["positions"], dev["k_cache"],
            dev["v_cache"], dev["block_tables"], dev["context_lens"], hint,
            case["softmax_scale"], workspace=ws, k_scale=dev["k_scale"], v_scale=dev["v_scale"])
    else:
        out, lse = gqa.paged_decode_attention(dev["q"], dev["k_cache"], dev["v_cache"],
                                              dev["block_tables"], dev["context_lens"], hint,
                                              case["softmax_scale"], dev["k_scale"],
                                              dev["v_scale"], workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _workspace(gqa, case, dev, hint, nq=1):
    shape = gqa.make_shape(case["q"].shape[0], case["spec"].num_q_heads, dev["k_cache"],
                           dev["block_tables"], k_scale=dev["k_scale"])
    n = gqa.multi_query_workspace_size(shape, nq, hint)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device="cuda:0")


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_clean_calls_leave_the_status_zero(gpu, dt):
    spec = small_spec(num_seqs=3, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                      kv_dtype=dt, context=("uniform", 1, 900), case_id=7100)
    case = make_case(spec, seed=1)
    dev = to_device(case)
    hint = int(case["context_lens"].max())
    ws = _workspace(gpu, case, dev, hint)
    for _ in range(2):
        _attend(gpu, case, dev, ws, hint=hint)
    assert gpu.workspace_status(ws) == 0


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_bad_block_id_sets_its_bit(gpu, dt):
    spec = small_spec(num_seqs=2, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                      kv_dtype=dt, context=100, case_id=2500)
    case = make_case(spec, seed=7)
    ref, ref_lse = run_oracle(case)
    case["block_tables"][0, 3] = case["k_pool"].shape[0] + 5      # out of range
    dev = to_device(case)
    ws = _workspace(gpu, case, dev, 100)
    out, lse = _attend(gpu, case, dev, ws)
    assert np.all(np.isnan(out[0])) and np.all(np.isnan(lse[0]))
    assert_parity(out[1:], lse[1:], ref[1:], ref_lse[1:], "other sequence")
    assert gpu.workspace_status(ws, clear=True) == gpu.STATUS_BAD_BLOCK_ID
    assert gpu.workspace_status(ws) == 0                          # cleared
    case["block_tables"][0, 3] = -1                               # negative is out of range too
    dev = to_device(case)
    _attend(gpu, case, dev, ws)
    assert gpu.workspace_status(ws) == gpu.STATUS_BAD_BLOCK_ID


def test_bad_lengths_set_their_bits(gpu):
    spec = small_spec(num_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                      context=300, case_id=7200)
    case = make_case(spec, seed=2, context_lens=[300, 250, 200, 100])
    ref, ref_lse = run_oracle(case)
    dev = to_device(case)
    ws = _workspace(gpu, case, dev, 300)
    table_tokens = case["block_tables"].shape[1] * 16
    dev["context_lens"][1] = table_tokens + 1                     # beyond the table
    _attend(gpu, case, dev, ws, hint=300)
    assert gpu.workspace_status(ws, clear=True) == gpu.STATUS_BAD_CONTEXT_LEN
    dev["context_lens"][1] = -3
    _attend(gpu, case, dev, ws, hint=300)
    assert gpu.workspace_status(ws, clear=True) == gpu.STATUS_BAD_CONTEXT_LEN
    dev["context_lens"][1] = 250
    out, lse = _attend(gpu, case, dev, ws, hint=260)              # sequence 0 exceeds the hint
    assert np.all(np.isnan(out[0]))
    assert_parity(out[1:], lse[1:], ref[1:], ref_lse[1:], "within the hint")
    assert gpu.workspace_status(ws, clear=True) == gpu.STATUS_CONTEXT_OVER_HINT


def test_multi_query_short_context_sets_the_length_bit(gpu):
    spec = small_spec(num_seqs=2, num_q_heads=16, num_kv_heads=4, head_dim=64, block_size=16,
                      context=300, case_id=6200)
    case = make_multi_query_case(spec, 4, seed=5, context_lens=[300, 2], append=False)
    dev = to_device(case)
    ws = _workspace(gpu, case, dev, 300, nq=4)
    out, _ = gpu.paged_decode_multi_query(dev["q"], dev["k_cache"], dev["v_cache"],
                                          dev["block_tables"], dev["context_lens"], 300,
                                          workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(out[1]).all()
    assert gpu.workspace_status(ws) == gpu.STATUS_BAD_CONTEXT_LEN


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_bad_append_sets_its_bit(gpu, dt):
    """A fused append whose position is past the table, or whose table entry is no
    block of the pool, writes nothing and sets the append bit; attention over the
    sequence's valid tokens is unaffected."""
    lens = [150, 200]
    spec = small_spec(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                      context=200, append=True, case_id=7300)
    case = make_case(spec, seed=3, context_lens=lens)
    if dt == "fp8":          # the fused fp8 step quantises the bf16 rows into an fp8 pool
        fspec = small_spec(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                           block_size=16, kv_dtype="fp8", context=200, case_id=7300)
        f = make_case(fspec, seed=3, context_lens=lens)
        for key in ("k_pool", "v_pool", "k_scale", "v_scale", "block_tables"):
            case[key] = f[key]
    dev = to_device(case)
    ws = _workspace(gpu, case, dev, 200)
    out0, _ = _attend(gpu, case, dev, ws, fused=True)       # a valid step fills the new slots
    assert np.all(np.isfinite(out0))
    assert gpu.workspace_status(ws) == 0
    table_tokens = case["block_tables"].shape[1] * 16
    assert table_tokens >= 12 * 16
    for bad in ("past the table", "not a block"):
        before = [dev[k].clone() for k in ("k_cache", "v_cache")]
        pos = dev["positions"].clone()
        if bad == "past the table":
            dev["positions"][0] = table_tokens + 7
        else:                                               # block 11: beyond sequence 0's 150 tokens
            dev["positions"][0] = 11 * 16 + 3
            dev["block_tables"][0, 11] = case["k_pool"].shape[0] + 3
        dev["positions"][1] = -1                            # sequence 1 appends nothing
        out, _ = _attend(gpu, case, dev, ws, fused=True)
        assert gpu.workspace_status(ws, clear=True) == gpu.STATUS_BAD_APPEND, bad
        assert np.array_equal(out, out0), bad               # the same tokens are attended
        for t, b in zip((dev["k_cache"], dev["v_cache"]), before):
            assert torch.equal(t.view(torch.uint8), b.view(torch.uint8)), bad
        dev["positions"].copy_(pos)
        dev["block_tables"].copy_(torch.from_numpy(case["block_tables"]))
