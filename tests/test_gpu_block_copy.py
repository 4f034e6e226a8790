"""GPU checks of the copy-on-write block copy: bit-exact against the oracle's
copy for both pool dtypes (fp8 scales included), and the fork flow in which two
sequences share a partially filled block, one of them gets a private copy, and
both then commit new tokens and attend in one fused step."""
import numpy as np
import pytest
import torch

import oracle
from tests._dev import assert_parity
from workloads import make_case, small_spec

pytestmark = pytest.mark.gpu


def _random_pool(rng, nb, hkv, bs, d, dt):
    if dt == "fp8":
        shape = (nb, hkv, bs, d)
        k = rng.integers(0, 256, shape, dtype=np.uint8)
        v = rng.integers(0, 256, shape, dtype=np.uint8)
        ks = rng.random((nb, hkv), dtype=np.float32) + 0.01
        vs = rng.random((nb, hkv), dtype=np.float32) + 0.01
        return k, v, ks, vs
    k = rng.integers(0, 1 << 16, (nb, hkv, bs, d), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, (nb, hkv, bs, d), dtype=np.uint16)
    return k, v, None, None


def _dev_pool(a):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if a.dtype == np.uint16 else np.uint8))
    return t.to("cuda:0")


def _host_pool(t, dtype):
    return t.cpu().numpy().view(dtype)


def _pairs(rng, nb, n, invalid=True):
    """n pairs with distinct destinations that are never sources; with ``invalid``
    a few pairs name ids outside the pool or copy a block onto itself."""
    perm = rng.permutation(nb)
    src = perm[:n].astype(np.int32)
    dst = perm[n:2 * n].astype(np.int32)
    if invalid and n >= 4:
        src[0] = -1
        dst[1] = nb
        src[2] = dst[2]
        dst[3] = -7
    return src, dst


@pytest.mark.parametrize("dt,hkv,bs,d,nb,n", [
    ("bf16", 8, 16, 128, 300, 100),
    ("bf16", 1, 32, 64, 64, 30),
    ("bf16", 40, 16, 128, 80, 7),
    ("fp8", 8, 16, 128, 300, 100),
    ("fp8", 40, 32, 64, 50, 20),
    ("bf16", 8, 16, 128, 9000, 4096),
    ("bf16", 5, 16, 64, 60, 13),          # 10 KiB blocks: a partial last slice, 39 work items
])
def test_copy_blocks_is_bit_exact(gpu, dt, hkv, bs, d, nb, n):
    rng = np.random.default_rng(nb + n + hkv)
    k, v, ks, vs = _random_pool(rng, nb, hkv, bs, d, dt)
    src, dst = _pairs(rng, nb, n)
    ref = oracle.copy_blocks(k, v, src, dst, ks, vs)
    kd, vd = _dev_pool(k), _dev_pool(v)
    ksd = None if ks is None else torch.from_numpy(ks).to("cuda:0")
    vsd = None if vs is None else torch.from_numpy(vs).to("cuda:0")
    gpu.kv_copy_blocks(kd, vd, torch.from_numpy(src).to("cuda:0"),
                       torch.from_numpy(dst).to("cuda:0"), ksd, vsd)
    torch.cuda.synchronize()
    assert np.array_equal(_host_pool(kd, k.dtype), ref[0])
    assert np.array_equal(_host_pool(vd, v.dtype), ref[1])
    if ks is not None:
        assert np.array_equal(ksd.cpu().numpy(), ref[2])
        assert np.array_equal(vsd.cpu().numpy(), ref[3])


@pytest.mark.parametrize("dt,seed", [("bf16", 0), ("bf16", 1), ("fp8", 2)])
def test_copy_blocks_with_shared_sources(gpu, dt, seed):
    """Forks list one source several times in a row (runs of 1 to 20 copies), with
    invalid ids inside runs: every copy is made."""
    rng = np.random.default_rng(100 + seed)
    nb, hkv, bs, d = 400, 8, 16, 128
    k, v, ks, vs = _random_pool(rng, nb, hkv, bs, d, dt)
    runs = rng.integers(1, 21, 20)
    perm = rng.permutation(nb).astype(np.int32)
    src = np.repeat(perm[:len(runs)], runs).astype(np.int32)
    dst = perm[len(runs):len(runs) + len(src)].copy()
    src[5], dst[9], dst[17] = -1, nb + 3, src[17]
    ref = oracle.copy_blocks(k, v, src, dst, ks, vs)
    kd, vd = _dev_pool(k), _dev_pool(v)
    ksd = None if ks is None else torch.from_numpy(ks).to("cuda:0")
    vsd = None if vs is None else torch.from_numpy(vs).to("cuda:0")
    gpu.kv_copy_blocks(kd, vd, torch.from_numpy(src).to("cuda:0"),
                       torch.from_numpy(dst).to("cuda:0"), ksd, vsd)
    torch.cuda.synchronize()
    assert np.array_equal(_host_pool(kd, k.dtype), ref[0])
    assert np.array_equal(_host_pool(vd, v.dtype), ref[1])
    if ks is not None:
        assert np.array_equal(ksd.cpu().numpy(), ref[2])
        assert np.array_equal(vsd.cpu().numpy(), ref[3])


def test_copy_no_pairs_changes_nothing(gpu):
    rng = np.random.default_rng(5)
    k, v, _, _ = _random_pool(rng, 10, 2, 16, 64, "bf16")
    kd, vd = _dev_pool(k), _dev_pool(v)
    empty = torch.empty(0, dtype=torch.int32, device="cuda:0")
    gpu.kv_copy_blocks(kd, vd, empty, empty)
    torch.cuda.synchronize()
    assert np.array_equal(_host_pool(kd, np.uint16), k)
    assert np.array_equal(_host_pool(vd, np.uint16), v)


def _bf16_bits(rng, shape):
    return (rng.standard_normal(shape, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")


@pytest.mark.parametrize("prefix,nq", [(1000, 1), (1006, 4), (992, 1), (5, 3)])
def test_fork_copies_the_shared_partial_block(gpu, prefix, nq):
    """Sequence B is a fork of A: both tables name the same blocks.  Before they
    write their own next tokens, B's copy of the shared last block (if it is not
    full) is made private with the block copy and fresh blocks take any tokens
    past it; then one fused step commits each sequence's new tokens and attends.
    Pools and attention match the oracle; A's blocks hold A's tokens only."""
    hq, hkv, d, bs = 32, 8, 128, 16
    spec = small_spec(num_seqs=1, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                      context=prefix, pool="oversized2x", case_id=9000 + prefix + nq)
    case = make_case(spec, seed=3, context_lens=[prefix])
    k0, v0 = case["k_pool_full"], case["v_pool_full"]
    nb = k0.shape[0]
    table_a = case["block_tables"][0]
    owned = table_a[table_a >= 0].tolist()
    free = [i for i in range(nb) if i not in set(owned)]

    total = prefix + nq
    nblk = -(-total // bs)
    tables = np.full((2, nblk), -1, dtype=np.int32)
    tables[0, :len(owned)] = owned
    tables[1, :len(owned)] = owned
    src, dst = [], []
    if prefix % bs:                          # shared last block is partial: B copies it
        last = len(owned) - 1
        src.append(owned[last])
        dst.append(free.pop())
        tables[1, last] = dst[-1]
    for j in range(len(owned), nblk):        # blocks past the prefix are private
        tables[0, j] = free.pop()
        tables[1, j] = free.pop()

    rng = np.random.default_rng(prefix * 10 + nq)
    q = _bf16_bits(rng, (2, nq, hq, d))
    k_new = _bf16_bits(rng, (2, nq, hkv, d))
    v_new = _bf16_bits(rng, (2, nq, hkv, d))
    ctx = np.array([total, total], dtype=np.int32)
    positions = np.tile(np.arange(prefix, total, dtype=np.int32), (2, 1))

    kr, vr = oracle.copy_blocks(k0, v0, np.array(src, dtype=np.int32),
                                np.array(dst, dtype=np.int32))
    kr, vr = oracle.kv_append_tokens(kr, vr, k_new, v_new, tables, positions, bs)
    scale = 1.0 / np.sqrt(d)
    ref, ref_lse = oracle.paged_multi_query_attention(q, kr, vr, tables, ctx, bs, scale)

    kd, vd = _dev_pool(k0), _dev_pool(v0)
    if src:
        gpu.kv_copy_blocks(kd, vd, torch.tensor(src, dtype=torch.int32, device="cuda:0"),
                           torch.tensor(dst, dtype=torch.int32, device="cuda:0"))
    kd, vd = kd.view(torch.bfloat16), vd.view(torch.bfloat16)
    td = torch.from_numpy(tables).to("cuda:0")
    cd = torch.from_numpy(ctx).to("cuda:0")
    out, lse = gpu.paged_decode_multi_query_append(_bf16_dev(q), _bf16_dev(k_new),
                                                   _bf16_dev(v_new), kd, vd, td, cd, total,
                                                   float(scale))
    torch.cuda.synchronize()
    assert np.array_equal(_host_pool(kd.view(torch.int16), np.uint16), kr)
    assert np.array_equal(_host_pool(vd.view(torch.int16), np.uint16), vr)
    assert_parity(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                  ref, ref_lse, f"fork prefix={prefix} Q={nq}")
    # A's own blocks never hold B's tokens
    for t in range(prefix, total):
        blk = tables[0, t // bs]
        assert np.array_equal(kr[blk, :, t % bs], k_new[0, t - prefix])
