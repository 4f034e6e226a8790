"""GPU parity at the limits of the boundary: pools beyond 4 GiB (blocks addressed
past 32-bit byte offsets), batches of hundreds of sequences (the uniform split
plan), and a 65,536-token context (the 64-split maximum)."""
import numpy as np
import pytest
import torch

import oracle
from tests._dev import assert_parity, to_device
from workloads import make_case, small_spec

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(gpu, dev, case, tables=None, kc=None, vc=None, ks=None, vs=None):
    out, lse = gpu.paged_decode_attention(
        dev["q"], dev["k_cache"] if kc is None else kc, dev["v_cache"] if vc is None else vc,
        dev["block_tables"] if tables is None else tables, dev["context_lens"],
        int(case["context_lens"].max()), case["softmax_scale"],
        dev["k_scale"] if ks is None else ks, dev["v_scale"] if vs is None else vs)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _ref(case):
    s = case["spec"]
    return oracle.paged_decode_attention(case["q"], case["k_pool_full"], case["v_pool_full"],
                                         case["block_tables"], case["context_lens"], s.block_size,
                                         case["softmax_scale"], s.kv_dtype, case["k_scale"],
                                         case["v_scale"])


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_pool_beyond_4gib(gpu, dt):
    """The case's blocks moved to the top of a pool of more than 4 GiB per pool
    (unused blocks left uninitialised): same results as the small pool."""
    lens = [3000, 700]
    spec = small_spec(num_seqs=2, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=16,
                      kv_dtype=dt, context=3000, case_id=9990 + (dt == "fp8"))
    case = make_case(spec, seed=1, context_lens=lens)
    dev = to_device(case)
    nb_small = dev["k_cache"].shape[0]
    tile = 8 * 16 * 128 * (1 if dt == "fp8" else 2)          # bytes per block per pool
    nb_big = (5 << 30) // tile + nb_small                    # > 4 GiB per pool
    big_k = torch.empty((nb_big,) + tuple(dev["k_cache"].shape[1:]), dtype=dev["k_cache"].dtype,
                        device=DEV)
    big_v = torch.empty_like(big_k)
    shift = nb_big - nb_small                                # the case's blocks start past 5 GiB
    big_k[shift:] = dev["k_cache"]
    big_v[shift:] = dev["v_cache"]
    tables = dev["block_tables"].clone()
    tables[tables >= 0] += shift
    ks = vs = None
    if dt == "fp8":
        ks = torch.zeros((nb_big, 8), dtype=torch.float32, device=DEV)
        vs = torch.zeros_like(ks)
        ks[shift:] = dev["k_scale"]
        vs[shift:] = dev["v_scale"]
    assert shift * tile > (1 << 32)
    ref, ref_lse = _ref(case)
    out, lse = _run(gpu, dev, case, tables, big_k, big_v, ks, vs)
    assert_parity(out, lse, ref, ref_lse, f"pool > 4 GiB {dt}")
    del big_k, big_v
    torch.cuda.empty_cache()


def test_two_hundred_sequences(gpu):
    """More sequences than one wave shares out by length: the uniform split plan
    over a ragged batch of 200."""
    rng = np.random.default_rng(12)
    lens = rng.integers(1, 1200, 200).tolist()
    lens[7] = 0
    spec = small_spec(num_seqs=200, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                      context=1200, case_id=9995)
    case = make_case(spec, seed=2, context_lens=lens)
    ref, ref_lse = _ref(case)
    out, lse = _run(gpu, to_device(case), case)
    assert_parity(out, lse, ref, ref_lse, "200 sequences")


def test_sixty_five_thousand_tokens(gpu):
    """One sequence of 65,536 tokens: 64 splits of 1,024 tokens, the most a plan uses."""
    spec = small_spec(num_seqs=1, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=32,
                      context=65536, case_id=9996)
    case = make_case(spec, seed=3)
    assert gpu.num_splits(65536) == 64
    ref, ref_lse = _ref(case)
    out, lse = _run(gpu, to_device(case), case)
    assert_parity(out, lse, ref, ref_lse, "65536 tokens")
    out2, lse2 = gpu.paged_decode_attention(*[to_device(case)[k] for k in
                                              ("q", "k_cache", "v_cache", "block_tables",
                                               "context_lens")], 65536, case["softmax_scale"],
                                            batch_invariant=True)
    torch.cuda.synchronize()
    assert_parity(out2.cpu().numpy().astype(np.float64), lse2.cpu().numpy().astype(np.float64),
                  ref, ref_lse, "65536 tokens, batch-invariant")
