"""Appending new tokens to an fp8 (E4M3) paged KV cache with per-(block, KV head)
scales, in float32 where the result is a code (test infrastructure only).

Cites:
* *The Mathematics of Transformer Inference* (hs-black), §11: quantising is
  x ~ s * round(x / s); what matters is the granularity of the scale s, and KV
  caches usually take one per head and per token; dequantisation is fused into
  the attention kernel, so the halved KV bytes are real.
* *Module 10: Inference and Deployment Serving* (wrwei.github.io), "Quantise
  the cache, evaluate the artifact": a one-byte cache halves memory and
  traffic, before the cost of scale metadata and of (de)quantisation.
* The E4M3 code and its largest value 448: ``oracle.fp8``.

Reading (the pages fix neither the granularity nor how a scale follows a block
that fills token by token): every (block, KV head) tile has one fp32 scale, as
the pool's scales are laid out, and a scale this append sets is a power of two.
For each tile a call writes into, with ``first`` the lowest slot it writes,
amax the largest |x| over the call's new rows of that tile and
``t = amax / 448`` (float32), ``p(t)`` = the smallest power of two >= t:
  * ``first == 0``: the block opens with this call; its scale becomes p(t).
  * ``first > 0`` (older tokens of the sequence sit in slots < first): the scale
    stays s_old when s_old >= t; otherwise it becomes p(t) and the older codes
    are re-encoded as encode(decode(c) * s_old / p(t)).
  * the new rows become encode(clamp(x / s, -448, 448)); with s == 0 (every new
    value zero and no older scale) they become code 0x00.
Why powers of two: E4M3 is a floating-point code, so its relative precision does
not depend on s and the scale only has to keep amax / s <= 448; scaling by a
power of two commutes with rounding to E4M3 (outside its subnormal range), so
re-encoding older tokens after a growth is exact for every value that stays
normal, where a growth to amax / 448 itself would round the older tokens once
more at every growth.  The price is at most one binade of headroom.  A scale
never shrinks while its block is open, and a block filled over many calls ends
with the scale that filling it in one call gives.
Each division and product is one float32 operation, as the kernel computes it,
so the codes (integers decided in floating point) match bit for bit.

KIVI layout (``layout="kivi"``, the pool's ``fp8_kivi`` scales, see
``oracle.attention``): keys keep one scale per channel of each (block, KV
head) tile and follow the rule above channel by channel (t, the old scale and
the re-encoding are per channel d, over the column x[:, d] of the new rows);
values keep one scale per token, p(max|row| / 448) for each new row, set once
when the row is written.  *Module 10*, "Quantize the cache" (KIVI: per-channel
keys, per-token values).

Positions of sequence b are start[b] .. start[b] + T - 1 (start < 0: none);
rows past the block table, or whose table entry is not a block of the pool,
write nothing.
"""
import numpy as np

from .bf16 import bf16_to_float64
from .fp8 import FP8_MAX, decode_e4m3fn, encode_e4m3fn

_F32_MAX = np.float32(FP8_MAX)


def _encode_scaled(x32: np.ndarray, s: np.float32) -> np.ndarray:
    if s == 0:
        return np.zeros(x32.shape, dtype=np.uint8)
    q = np.clip(x32 / s, -_F32_MAX, _F32_MAX)          # one float32 division per element
    return encode_e4m3fn(q)


def pow2_ceil(t: np.float32) -> np.float32:
    """The smallest power of two >= t (t >= 0; 0 stays 0)."""
    if t == 0:
        return np.float32(0)
    m, e = np.frexp(np.float64(t))          # t = m * 2^e, 0.5 <= m < 1
    return np.float32(np.ldexp(1.0, int(e) - 1 if m == 0.5 else int(e)))


def append_tile(tile: np.ndarray, scale: np.float32, first: int, rows32: np.ndarray):
    """One (block, KV head) tile [BS][d] of codes, its scale, the lowest slot written
    and the new rows [n][d] (float32).  Returns (new tile, new scale)."""
    tile = tile.copy()
    amax = np.float32(np.max(np.abs(rows32))) if rows32.size else np.float32(0)
    t = np.float32(amax / _F32_MAX)
    old = np.float32(scale)
    if first > 0 and old >= t:
        s = old
    else:
        s = pow2_ceil(t)
    if first > 0 and t > old:
        older = decode_e4m3fn(tile[:first]).astype(np.float32) * old
        tile[:first] = _encode_scaled(older, s)
    tile[first:first + rows32.shape[0]] = _encode_scaled(rows32, s)
    return tile, s


def _append_tile_kivi(tile, scale, first, rows32, is_key):
    """KIVI: keys column by column (scale [d]), values row by row (scale [BS])."""
    tile, scale = tile.copy(), np.array(scale, dtype=np.float32, copy=True)
    if is_key:
        for d in range(tile.shape[1]):
            col, scale[d] = append_tile(tile[:, d:d + 1], scale[d], first, rows32[:, d:d + 1])
            tile[:, d] = col[:, 0]
    else:
        for j in range(rows32.shape[0]):
            slot = first + j
            row, scale[slot] = append_tile(tile[slot:slot + 1], scale[slot], 0, rows32[j:j + 1])
            tile[slot] = row[0]
    return tile, scale


def kv_append_fp8(k_pool, v_pool, k_scale, v_scale, k_new_bits, v_new_bits, block_tables,
                  start_positions, block_size, layout="block"):
    """k_pool/v_pool uint8 [NB][H_kv][BS][d]; k_scale/v_scale float32 [NB][H_kv]
    (layout "kivi": k_scale [NB][H_kv][d], v_scale [NB][H_kv][BS]);
    k_new_bits/v_new_bits uint16 bf16 [B][T][H_kv][d]; start_positions int [B].
    Returns new (k_pool, v_pool, k_scale, v_scale); inputs are not modified."""
    out = []
    for is_key, pool, scale, new in ((True, k_pool, k_scale, k_new_bits),
                                     (False, v_pool, v_scale, v_new_bits)):
        pool = pool.copy()
        scale = np.array(scale, dtype=np.float32, copy=True)
        x = bf16_to_float64(new).astype(np.float32)          # exact
        B, T, H, _ = x.shape
        nb, max_blocks = pool.shape[0], block_tables.shape[1]
        for b in range(B):
            st = int(start_positions[b])
            if st < 0:
                continue
            pos = st
            while pos < st + T:
                bi, first = pos // block_size, pos % block_size
                n = min(block_size - first, st + T - pos)
                if bi >= max_blocks:
                    break
                blk = int(block_tables[b, bi])
                if 0 <= blk < nb:
                    for h in range(H):
                        rows = x[b, pos - st:pos - st + n, h]
                        if layout == "kivi":
                            pool[blk, h], scale[blk, h] = _append_tile_kivi(
                                pool[blk, h], scale[blk, h], first, rows, is_key)
                        else:
                            pool[blk, h], scale[blk, h] = append_tile(
                                pool[blk, h], scale[blk, h], first, rows)
                pos += n
        out += [pool, scale]
    return out[0], out[2], out[1], out[3]
