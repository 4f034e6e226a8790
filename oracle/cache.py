"""Paged KV cache: block-table gather and single-token append (oracle side).

Cites:
* *Module 10: Inference and Deployment Serving* (wrwei.github.io), "Mapping
  logical positions to physical blocks": the cache is cut into fixed-size
  blocks in one shared pool; a per-sequence block table maps logical block i
  to a physical block; a sequence's blocks need not be adjacent; with 16-token
  blocks at most 15 tail slots are wasted.
* *Ch. 6 Inference Efficiency and Model Serving* (Stochastic Parrot vol. 1),
  §6.4: logical positions split into fixed blocks, mapped to non-contiguous
  physical blocks; the last block has at most one block of internal waste.
* *LLM Inference Systems Engineering* (jasonzhang109), §2.1.3: the cache only
  holds positions already forwarded; each step first commits the pending
  token's K/V, then attends.
* *The Mathematics of Transformer Inference* (hs-black), §1: decode reads the
  cache for attention and appends the new token's own K and V; §9: sequences
  may share physical blocks, with reference counts and copy-on-write.
* Copy-on-write: *Module 10*, "Share only state with the same identity" (a
  sequence about to write into a shared, not yet full block first gets a
  private copy, so the other sequence's state is unchanged; full prefix blocks
  stay shared); *Stochastic Parrot* §6.4 (branches point at the same read-only
  block and get a new one on a divergent write).

Pool layout (a reading; the pages fix no layout): ``pool[num_blocks][H_kv][BS][d_h]``;
token t of sequence b lives in physical block ``block_table[b][t // BS]`` at
slot ``t % BS``.
"""
import numpy as np


def gather_sequence(pool: np.ndarray, block_table_row: np.ndarray, ctx: int,
                    block_size: int) -> np.ndarray:
    """Return the sequence's cached rows in logical order: ``[H_kv][ctx][d_h]``.

    Only the first ceil(ctx / BS) table entries are read, and only the first
    ``ctx`` slots of the logical stream are returned.
    """
    ctx = int(ctx)
    t = np.arange(ctx)
    phys = np.asarray(block_table_row)[t // block_size]
    slot = t % block_size
    rows = pool[phys, :, slot, :]            # [ctx][H_kv][d_h]
    return np.ascontiguousarray(np.transpose(rows, (1, 0, 2)))


def kv_append(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              block_tables: np.ndarray, positions: np.ndarray, block_size: int):
    """Write token ``positions[b]`` of every sequence b into the pools.

    ``k_new/v_new`` are ``[B][H_kv][d_h]``.  A negative position means "no
    append for this sequence".  Returns new pools; inputs are not modified.
    Only the one slot per (sequence, KV head) changes.
    """
    k_out, v_out = k_pool.copy(), v_pool.copy()
    for b, pos in enumerate(np.asarray(positions)):
        pos = int(pos)
        if pos < 0:
            continue
        blk = int(block_tables[b][pos // block_size])
        slot = pos % block_size
        k_out[blk, :, slot, :] = k_new[b]
        v_out[blk, :, slot, :] = v_new[b]
    return k_out, v_out


def kv_append_tokens(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
                     v_new: np.ndarray, block_tables: np.ndarray, positions: np.ndarray,
                     block_size: int):
    """Write T tokens per sequence: ``k_new/v_new`` ``[B][T][H_kv][d_h]`` at logical
    positions ``[B][T]``.  A position outside the table's range, or whose table
    entry is not a block of the pool, writes nothing.  Returns new pools."""
    k_out, v_out = k_pool.copy(), v_pool.copy()
    capacity = block_tables.shape[1] * block_size
    for b in range(positions.shape[0]):
        for j in range(positions.shape[1]):
            pos = int(positions[b, j])
            if pos < 0 or pos >= capacity:
                continue
            blk = int(block_tables[b][pos // block_size])
            if blk < 0 or blk >= k_pool.shape[0]:
                continue
            k_out[blk, :, pos % block_size, :] = k_new[b, j]
            v_out[blk, :, pos % block_size, :] = v_new[b, j]
    return k_out, v_out


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, src_blocks, dst_blocks,
                k_scale=None, v_scale=None):
    """Copy whole physical blocks (every KV head, every slot, K and V, and the
    fp8 scales when given): block ``dst_blocks[j]`` becomes a copy of
    ``src_blocks[j]``, as taken before the call.  A pair with an id outside the
    pool is skipped.  Returns new pools (and scales); inputs are not modified."""
    nb = k_pool.shape[0]
    k_out, v_out = k_pool.copy(), v_pool.copy()
    ks_out = None if k_scale is None else np.array(k_scale, copy=True)
    vs_out = None if v_scale is None else np.array(v_scale, copy=True)
    for src, dst in zip(np.asarray(src_blocks), np.asarray(dst_blocks)):
        src, dst = int(src), int(dst)
        if not (0 <= src < nb and 0 <= dst < nb):
            continue
        k_out[dst] = k_pool[src]
        v_out[dst] = v_pool[src]
        if ks_out is not None:
            ks_out[dst] = k_scale[src]
            vs_out[dst] = v_scale[src]
    if ks_out is None:
        return k_out, v_out
    return k_out, v_out, ks_out, vs_out
