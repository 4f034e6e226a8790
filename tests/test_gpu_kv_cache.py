"""GPU: KV append and block-table gather are bit-exact against the oracle's scatter/gather."""
import numpy as np
import pytest

import oracle
from tests._dev import to_device, named_case
from workloads import make_case, small_spec

pytestmark = pytest.mark.gpu


def _pool_bits(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("spec", [
    small_spec(num_seqs=5, num_kv_heads=2, head_dim=64, block_size=16, context=("uniform", 1, 300),
               append=True, case_id=3000),
    small_spec(num_seqs=3, num_kv_heads=8, head_dim=128, block_size=32, context=("uniform", 1, 300),
               append=True, case_id=3001),
], ids=["d64bs16", "d128bs32"])
def test_append_bit_exact(gpu, spec):
    import torch
    case = make_case(spec, seed=1)
    dev = to_device(case)
    gpu.kv_append(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                  dev["block_tables"], dev["positions"])
    torch.cuda.synchronize()
    kp, vp = oracle.kv_append(case["k_pool"], case["v_pool"], case["k_new"], case["v_new"],
                              case["block_tables"], case["positions"], spec.block_size)
    assert np.array_equal(_pool_bits(dev["k_cache"]), kp)
    assert np.array_equal(_pool_bits(dev["v_cache"]), vp)


def test_append_long_workload_bit_exact(gpu):
    import torch
    case = named_case("long")
    dev = to_device(case)
    gpu.kv_append(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                  dev["block_tables"], dev["positions"])
    torch.cuda.synchronize()
    assert np.array_equal(_pool_bits(dev["k_cache"]), case["k_pool_full"])
    assert np.array_equal(_pool_bits(dev["v_cache"]), case["v_pool_full"])


def test_append_skips_negative_and_out_of_range(gpu):
    import torch
    spec = small_spec(num_seqs=3, num_kv_heads=2, head_dim=64, block_size=16, context=40,
                      append=True, case_id=3002)
    case = make_case(spec, seed=2)
    case["positions"][:] = [-1, 10 ** 6, 39]
    dev = to_device(case)
    gpu.kv_append(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                  dev["block_tables"], dev["positions"])
    torch.cuda.synchronize()
    kp, _ = oracle.kv_append(case["k_pool"], case["v_pool"], case["k_new"], case["v_new"],
                             case["block_tables"], np.array([-1, -1, 39]), 16)
    assert np.array_equal(_pool_bits(dev["k_cache"]), kp)


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_gather_bit_exact(gpu, dt):
    spec = small_spec(num_seqs=4, num_kv_heads=4, num_q_heads=8, head_dim=128, block_size=16,
                      kv_dtype=dt, context=("uniform", 1, 500), case_id=3010 + (dt == "fp8"))
    case = make_case(spec, seed=3)
    dev = to_device(case)
    for b in range(4):
        ctx = int(case["context_lens"][b])
        got = _pool_bits(gpu.kv_gather(dev["k_cache"], dev["block_tables"], b, ctx))
        want = oracle.gather_sequence(case["k_pool"], case["block_tables"][b], ctx, 16)
        assert np.array_equal(got, want)
