"""The entry point that allocates nothing (gqa_paged_decode_attention_noalloc):
its results equal gqa_paged_decode_attention's with a caller workspace, on two
calls in a row, the second with a smaller batch; it matches the float64 oracle
within the usual bar; and a call too large for its static scratch is refused."""
import numpy as np
import pytest
import torch

from tests._dev import to_device, run_oracle, assert_parity
from workloads import make_case, small_spec, SPECS

pytestmark = pytest.mark.gpu


def _both(gqa, case, dev, hint=None):
    hint = int(case["context_lens"].max()) if hint is None else hint
    a = gqa.paged_decode_attention(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                   dev["context_lens"], hint, case["softmax_scale"],
                                   dev["k_scale"], dev["v_scale"])
    b = gqa.paged_decode_attention_noalloc(dev["q"], dev["k_cache"], dev["v_cache"],
                                           dev["block_tables"], dev["context_lens"], hint,
                                           case["softmax_scale"], dev["k_scale"], dev["v_scale"])
    torch.cuda.synchronize()
    return [t.cpu().numpy().astype(np.float64) for t in (*a, *b)]


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_noalloc_matches_the_workspace_entry_point(gpu, dt):
    big = small_spec(num_seqs=6, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                     kv_dtype=dt, context=("uniform", 200, 3000), case_id=7400)
    small = small_spec(num_seqs=2, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                       kv_dtype=dt, context=("uniform", 50, 900), case_id=7401)
    for spec in (big, small):                       # the second call is the smaller one
        case = make_case(spec, seed=4)
        ref, ref_lse = run_oracle(case)
        o1, l1, o2, l2 = _both(gpu, case, to_device(case))
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), spec.name
        assert_parity(o2, l2, ref, ref_lse, f"noalloc {dt} B={spec.num_seqs}")


def test_noalloc_full_size_long_context(gpu):
    """The 32K workload's shape (B=4, 64/8 heads, ctx 32769, block 32) fits the scratch."""
    case = make_case(SPECS["long"], seed=0)
    dev = to_device(case)
    gpu.kv_append(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                  dev["block_tables"], dev["positions"])
    o1, l1, o2, l2 = _both(gpu, case, dev)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_noalloc_refuses_calls_beyond_its_scratch(gpu):
    spec = small_spec(num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=100, case_id=7402)
    case = make_case(spec, seed=1)
    dev = to_device(case)
    big_hint = 200000
    bt = torch.zeros((64, big_hint // 16 + 1), dtype=torch.int32, device="cuda:0")
    shape = gpu.make_shape(64, 32, dev["k_cache"], bt)
    assert gpu.workspace_size(shape, big_hint) > gpu.NOALLOC_SCRATCH_BYTES
    with pytest.raises(gpu.GqaError) as e:
        gpu.paged_decode_attention_noalloc(dev["q"], dev["k_cache"], dev["v_cache"], bt,
                                           dev["context_lens"], big_hint)
    assert e.value.status == 3
