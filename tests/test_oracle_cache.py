"""Pins the oracle's block-table gather and KV append with brute-force indexing."""
import numpy as np

from oracle import gather_sequence, kv_append
from workloads import make_case, small_spec, SPECS


def test_gather_by_loops():
    case = make_case(small_spec(num_seqs=3, block_size=4, context=("uniform", 1, 30), case_id=400), seed=1)
    pool = case["k_pool_full"]
    for b in range(3):
        ctx = int(case["context_lens"][b])
        g = gather_sequence(pool, case["block_tables"][b], ctx, 4)
        assert g.shape == (pool.shape[1], ctx, pool.shape[3])
        for t in range(ctx):
            blk = case["block_tables"][b][t // 4]
            for h in range(pool.shape[1]):
                assert np.array_equal(g[h, t], pool[blk, h, t % 4])


def test_gather_never_reads_beyond_context():
    case = make_case(small_spec(num_seqs=1, block_size=16, context=17, case_id=401), seed=1)
    row = case["block_tables"][0].copy()
    row[2:] = 10 ** 6            # entries beyond ceil(17/16) = 2 are garbage
    g = gather_sequence(case["k_pool_full"], row, 17, 16)
    assert g.shape[1] == 17


def test_append_writes_exactly_one_slot_per_sequence_and_head():
    spec = SPECS["llama8b"]
    case = make_case(small_spec(num_seqs=3, num_kv_heads=2, block_size=16, context=("uniform", 1, 50),
                                append=True, case_id=402), seed=2)
    kp, vp = kv_append(case["k_pool"], case["v_pool"], case["k_new"], case["v_new"],
                       case["block_tables"], case["positions"], 16)
    changed = np.argwhere(np.any(kp.view(np.uint16) != case["k_pool"].view(np.uint16), axis=-1))
    assert len(changed) == 3 * 2
    # the appended pool is the full pool: the poisoned slot now holds the new token
    assert np.array_equal(kp, case["k_pool_full"]) and np.array_equal(vp, case["v_pool_full"])
    # inputs untouched
    assert not np.array_equal(case["k_pool"], case["k_pool_full"])
    assert spec.append


def test_append_negative_position_is_a_no_op():
    case = make_case(small_spec(num_seqs=2, context=20, append=True, case_id=403), seed=3)
    pos = case["positions"].copy()
    pos[1] = -1
    kp, _ = kv_append(case["k_pool"], case["v_pool"], case["k_new"], case["v_new"],
                      case["block_tables"], pos, 16)
    blk = case["block_tables"][1][19 // 16]
    assert np.array_equal(kp[blk], case["k_pool"][blk])


def test_copy_blocks_by_loops_and_the_copy_on_write_flow():
    """copy_blocks checked element by element, then the copy-on-write use: two
    sequences share a partial last block; before one of them appends, the block is
    copied to a fresh one and its table remapped, which leaves the other sequence's
    gathered rows unchanged and gives the writer the shared rows plus its own token."""
    from oracle import copy_blocks, kv_append, gather_sequence
    rng = np.random.default_rng(3)
    NB, H, BS, D = 8, 2, 4, 3
    k = rng.integers(0, 60000, (NB, H, BS, D)).astype(np.uint16)
    v = rng.integers(0, 60000, (NB, H, BS, D)).astype(np.uint16)
    ks = rng.random((NB, H)).astype(np.float32)
    vs = rng.random((NB, H)).astype(np.float32)
    k2, v2, ks2, vs2 = copy_blocks(k, v, [1, 5, 9, 3], [6, 0, 2, 3], ks, vs)
    for blk in range(NB):
        src = {6: 1, 0: 5}.get(blk, blk)          # 9 is out of range: skipped; 3 -> 3
        for h in range(H):
            assert ks2[blk, h] == ks[src, h] and vs2[blk, h] == vs[src, h]
            for s_ in range(BS):
                for d in range(D):
                    assert k2[blk, h, s_, d] == k[src, h, s_, d]
                    assert v2[blk, h, s_, d] == v[src, h, s_, d]
    # copy-on-write: blocks [4, 7] hold 6 tokens shared by sequences A and B
    tables = np.array([[4, 7], [4, 7]])
    ka, _ = copy_blocks(k, v, [7], [1])               # B's private copy of the partial block
    tables[1, 1] = 1
    new = rng.integers(0, 60000, (2, H, D)).astype(np.uint16)
    kb, _ = kv_append(ka, ka, new, new, tables, np.array([-1, 6]), BS)
    assert np.array_equal(gather_sequence(kb, tables[0], 6, BS), gather_sequence(k, [4, 7], 6, BS))
    rows_b = gather_sequence(kb, tables[1], 7, BS)
    assert np.array_equal(rows_b[:, :6], gather_sequence(k, [4, 7], 6, BS))
    assert np.array_equal(rows_b[:, 6], new[1])
