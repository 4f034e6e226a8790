"""Seeded synthetic inputs for paged GQA decode attention.

This module only *makes inputs*: random query/key/value values, a paged KV
pool, block tables, context lengths and the new token of a KV append.  It holds
none of the attention arithmetic; both the float64 oracle and the HIP path
consume what it returns, and neither imports the other.

Workloads (sizes are those of the five named decode cases):

* ``tiny``      B=1, H_q=4, H_kv=1, d_h=64, ctx 128, block 16, pool = a random
                permutation of exactly 8 physical blocks.
* ``llama8b``   B=1, H_q=32, H_kv=8, d_h=128, ctx 8192 (8191 cached + 1
                appended), block 16, random placement in a 2x oversized pool.
* ``batched``   B=16, H_q=32, H_kv=8, d_h=128, ctx uniform in [512, 8192],
                block 16, all sequences' blocks interleaved in one shared pool
                of exactly the blocks needed.
* ``long``      B=4, H_q=64, H_kv=8, d_h=128, 32768 cached + 1 appended
                (ctx 32769), block 32, 2x oversized pool.
* ``mha_fp8``   B=4, H_q=H_kv=40, d_h=128, ctx 8192, block 16, K/V stored as
                OCP FP8 E4M3 (finite-only, max 448) with one fp32 scale per
                (physical block, KV head) equal to amax/448 of that block's
                valid source values.

Two more workloads share these recipes: ``mha_fp8_kivi`` (the mha_fp8 shape with
per-channel key and per-token value scales) and ``long_fp8`` (the long shape,
32768 tokens, with K/V stored as fp8 like mha_fp8 and no append: grouped queries
over an fp8 pool).

Recipe: q, k, v source values are i.i.d. N(0, 1) float32 rounded to bf16 by
round-to-nearest-even (for fp8, the float32 values are scaled and encoded
instead).  Because the values are i.i.d., they are drawn directly in pool
layout ``[num_blocks][H_kv][block][d_h]``; the block table decides which pool
slots a sequence owns.  Pool slots that hold no valid token (the tail of a
partially filled last block, blocks no sequence owns, and the slot an append
is about to fill) are poisoned with NaN codes so that any read of them shows
up in the result.  Generators are numpy PCG64 streams seeded by
``SeedSequence([seed, case_id])``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)
FP8_E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape of one decode-attention workload."""

    name: str
    case_id: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str = "bf16"          # "bf16", "fp8" or "fp8_kivi"
    context: int | tuple = 128       # fixed length, or ("uniform", lo, hi)
    append: bool = False             # last token of each sequence arrives via kv_append
    pool: str = "exact"              # "exact" or "oversized2x"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


SPECS = {
    "tiny": Spec("tiny", 0, 1, 4, 1, 64, 16, context=128, pool="exact"),
    "llama8b": Spec("llama8b", 1, 1, 32, 8, 128, 16, context=8192, append=True,
                    pool="oversized2x"),
    "batched": Spec("batched", 2, 16, 32, 8, 128, 16, context=("uniform", 512, 8192),
                    pool="exact"),
    "long": Spec("long", 3, 4, 64, 8, 128, 32, context=32769, append=True,
                 pool="oversized2x"),
    "mha_fp8": Spec("mha_fp8", 4, 4, 40, 40, 128, 16, kv_dtype="fp8", context=8192,
                    pool="exact"),
    "mha_fp8_kivi": Spec("mha_fp8_kivi", 5, 4, 40, 40, 128, 16, kv_dtype="fp8_kivi",
                         context=8192, pool="exact"),
    "long_fp8": Spec("long_fp8", 6, 4, 64, 8, 128, 32, kv_dtype="fp8", context=32768,
                     pool="oversized2x"),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite N(0,1) draws; NaN/Inf handling is not needed here.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP FP8 E4M3 codes (uint8), round to nearest even, saturating at +-448.

    Format: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0
    holds subnormals m/8 * 2^-6; code 0x7F/0xFF is NaN; there is no infinity.
    Used only to build fp8 cache contents from source values.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), FP8_E4M3_MAX)
    # exponent of the representable binade (subnormals share the 2^-6 step)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))   # a = m * 2^ex, m in [0.5, 1)
    e = np.clip(ex - 1, -6, 8).astype(np.float64)
    step = 2.0 ** (e - 3)                      # spacing of 3-bit mantissa in binade e
    q = np.round(a / step)                    # numpy rounds half to even
    v = q * step
    # mantissa overflow (q == 16) moves to the next binade: still exact as v
    e2 = np.where(v >= 2.0 ** (e + 1), e + 1, e)
    v = np.minimum(v, FP8_E4M3_MAX)
    normal = v >= 2.0 ** -6
    exp_field = np.where(normal, e2 + 7, 0).astype(np.int64)
    man = np.where(normal, np.round(v / 2.0 ** (e2 - 3)) - 8, np.round(v / 2.0 ** -9))
    man = man.astype(np.int64)
    code = (exp_field << 3) | man
    code = np.where(v == 0, 0, code)
    code = code | (sign.astype(np.int64) << 7)
    return code.astype(np.uint8)


def _context_lengths(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    if isinstance(spec.context, tuple):
        _, lo, hi = spec.context
        while True:
            ctx = rng.integers(lo, hi + 1, size=spec.num_seqs, dtype=np.int64)
            if np.any(ctx % spec.block_size != 0):
                return ctx.astype(np.int32)
    return np.full(spec.num_seqs, spec.context, dtype=np.int32)


def _normal_bf16(rng, shape, chunk=1 << 24):
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    n = out.size
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = bf16_round(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def _normal_f32(rng, shape, chunk=1 << 24):
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    n = out.size
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def make_case(spec: Spec | str, seed: int = 0, *, context_lens=None,
              poison: bool = True) -> dict:
    """Build one seeded decode-attention input set.

    Returns a dict of numpy arrays:
      q            uint16 [B][H_q][d_h]              bf16 bits
      k_pool/v_pool uint16 or uint8 [NB][H_kv][BS][d_h]  pool *before* the append
      k_scale/v_scale float32 [NB][H_kv] (fp8 only, else None)
      block_tables int32 [B][max_blocks]  (-1 beyond each sequence's blocks)
      context_lens int32 [B]   tokens attended per sequence, after the append
      positions    int32 [B]   slot index the append writes (ctx-1), or -1
      k_new/v_new  uint16 [B][H_kv][d_h]  appended token (bf16 only)
      k_pool_full/v_pool_full: pool after the append (what attention reads)
    ``context_lens`` overrides the spec's lengths (used for edge cases).
    """
    if isinstance(spec, str):
        spec = SPECS[spec]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, spec.case_id])))
    B, Hq, Hkv, D, BS = (spec.num_seqs, spec.num_q_heads, spec.num_kv_heads,
                         spec.head_dim, spec.block_size)
    if context_lens is None:
        ctx = _context_lengths(spec, rng)
    else:
        ctx = np.asarray(context_lens, dtype=np.int32)
        B = ctx.shape[0]
    nb = [(int(c) + BS - 1) // BS for c in ctx]
    used = int(sum(nb))
    max_blocks = max(1, max(nb) if nb else 1)
    num_blocks = max(1, used if spec.pool == "exact" else 2 * used)

    q = _normal_bf16(rng, (B, Hq, D))
    # random placement: a permutation of the pool, first `used` entries owned
    perm = rng.permutation(num_blocks).astype(np.int32)
    block_tables = np.full((B, max_blocks), -1, dtype=np.int32)
    owner = perm[:used]
    # interleave sequences' blocks: assign owned physical ids in random order
    off = 0
    for b in range(B):
        block_tables[b, : nb[b]] = owner[off: off + nb[b]]
        off += nb[b]

    valid = np.zeros((num_blocks, BS), dtype=bool)   # slot holds a valid token
    for b in range(B):
        for i in range(nb[b]):
            n_in = min(BS, int(ctx[b]) - i * BS)
            valid[block_tables[b, i], :n_in] = True

    positions = np.full(B, -1, dtype=np.int32)
    if spec.append:
        positions = np.where(ctx > 0, ctx - 1, -1).astype(np.int32)

    out = dict(spec=spec, q=q, block_tables=block_tables, context_lens=ctx.astype(np.int32),
               positions=positions, num_blocks=num_blocks, max_blocks=max_blocks,
               k_scale=None, v_scale=None, k_new=None, v_new=None)

    if spec.kv_dtype == "bf16":
        kf = _normal_bf16(rng, (num_blocks, Hkv, BS, D))
        vf = _normal_bf16(rng, (num_blocks, Hkv, BS, D))
        nan = BF16_NAN
    elif spec.kv_dtype == "fp8":
        kf, ks = _fp8_pool(rng, (num_blocks, Hkv, BS, D), valid)
        vf, vs = _fp8_pool(rng, (num_blocks, Hkv, BS, D), valid)
        out["k_scale"], out["v_scale"] = ks, vs
        nan = FP8_NAN
    elif spec.kv_dtype == "fp8_kivi":
        kf, ks = _fp8_pool(rng, (num_blocks, Hkv, BS, D), valid, per="channel")
        vf, vs = _fp8_pool(rng, (num_blocks, Hkv, BS, D), valid, per="token")
        out["k_scale"], out["v_scale"] = ks, vs
        nan = FP8_NAN
    else:
        raise ValueError(spec.kv_dtype)

    if poison:
        inval = ~valid
        kf[np.broadcast_to(inval[:, None, :, None], kf.shape)] = nan
        vf[np.broadcast_to(inval[:, None, :, None], vf.shape)] = nan
    out["k_pool_full"], out["v_pool_full"] = kf, vf

    k_pool, v_pool = kf, vf
    if spec.append:
        if spec.kv_dtype != "bf16":
            raise ValueError("append workloads are bf16")
        k_new = np.zeros((B, Hkv, D), dtype=np.uint16)
        v_new = np.zeros((B, Hkv, D), dtype=np.uint16)
        k_pool, v_pool = kf.copy(), vf.copy()
        for b in range(B):
            p = int(positions[b])
            if p < 0:
                continue
            blk, slot = block_tables[b, p // BS], p % BS
            k_new[b] = kf[blk, :, slot, :]
            v_new[b] = vf[blk, :, slot, :]
            if poison:
                k_pool[blk, :, slot, :] = nan
                v_pool[blk, :, slot, :] = nan
        out["k_new"], out["v_new"] = k_new, v_new
    out["k_pool"], out["v_pool"] = k_pool, v_pool
    out["softmax_scale"] = 1.0 / math.sqrt(D)
    return out


def make_multi_query_case(spec: Spec | str, num_queries: int, seed: int = 0, *,
                          context_lens=None, append: bool = True, poison: bool = True) -> dict:
    """A case with ``num_queries`` consecutive query positions per sequence.

    The base pools, tables and lengths are ``make_case`` of ``spec`` without its
    single-token append.  ``q`` is ``[B][Q][H_q][d]`` bf16 from its own seeded
    stream; query i of sequence b sits at position ``ctx_b - Q + i``.  With
    ``append`` the last Q tokens of every sequence are the step's new tokens:
    ``k_new``/``v_new`` are ``[B][Q][H_kv][d]``, ``positions`` ``[B][Q]`` (-1 where
    ``ctx_b - Q + i < 0``), and ``k_pool``/``v_pool`` hold NaN codes in those
    slots until the append fills them (``k_pool_full``/``v_pool_full`` hold them).
    """
    if isinstance(spec, str):
        spec = SPECS[spec]
    base = Spec(spec.name, spec.case_id, spec.num_seqs, spec.num_q_heads, spec.num_kv_heads,
                spec.head_dim, spec.block_size, kv_dtype=spec.kv_dtype, context=spec.context,
                append=False, pool=spec.pool)
    case = make_case(base, seed, context_lens=context_lens, poison=poison)
    Q = int(num_queries)
    B = case["context_lens"].shape[0]
    Hq, Hkv, D, BS = spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, spec.case_id, 1])))
    case["q"] = _normal_bf16(rng, (B, Q, Hq, D))
    case["num_queries"] = Q
    ctx = case["context_lens"].astype(np.int64)
    positions = (ctx[:, None] - Q + np.arange(Q)[None, :]).astype(np.int32)
    positions[positions < 0] = -1
    case["positions"] = positions
    if append:
        if spec.kv_dtype != "bf16":
            raise ValueError("append workloads are bf16")
        kf, vf = case["k_pool_full"], case["v_pool_full"]
        k_new = np.zeros((B, Q, Hkv, D), dtype=np.uint16)
        v_new = np.zeros((B, Q, Hkv, D), dtype=np.uint16)
        k_pool, v_pool = kf.copy(), vf.copy()
        for b in range(B):
            for i in range(Q):
                p = int(positions[b, i])
                if p < 0:
                    continue
                blk, slot = case["block_tables"][b, p // BS], p % BS
                k_new[b, i] = kf[blk, :, slot, :]
                v_new[b, i] = vf[blk, :, slot, :]
                if poison:
                    k_pool[blk, :, slot, :] = BF16_NAN
                    v_pool[blk, :, slot, :] = BF16_NAN
        case["k_new"], case["v_new"] = k_new, v_new
        case["k_pool"], case["v_pool"] = k_pool, v_pool
    return case


def new_token_rows(spec: Spec | str, num_tokens: int = 1, seed: int = 0) -> np.ndarray:
    """Seeded bf16 K or V rows of new tokens, [B][T][H_kv][d] (N(0,1) draws), for
    appends that quantise (fp8 pools), where the pool after the append is not
    built here."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, spec.case_id, 2])))
    return _normal_bf16(rng, (spec.num_seqs, num_tokens, spec.num_kv_heads, spec.head_dim))


def _fp8_pool(rng, shape, valid, per="block"):
    """N(0,1) float32 source values -> fp8 codes + scales amax/448 over the valid
    values of each scale's group: per="block" one per (block, head) [NB][H];
    "channel" one per (block, head, channel) [NB][H][D]; "token" one per
    (block, head, slot) [NB][H][BS].  A group with no valid value gets scale 1."""
    NB, H, BS, D = shape
    codes = np.empty(shape, dtype=np.uint8)
    axes = {"block": (2, 3), "channel": (2,), "token": (3,)}[per]
    scales = np.ones({"block": (NB, H), "channel": (NB, H, D), "token": (NB, H, BS)}[per],
                     dtype=np.float32)
    for b0 in range(0, NB, 256):
        b1 = min(NB, b0 + 256)
        x = _normal_f32(rng, (b1 - b0, H, BS, D))
        m = valid[b0:b1][:, None, :, None]
        amax = np.max(np.where(m, np.abs(x), 0.0), axis=axes, keepdims=True).astype(np.float32)
        sc = np.where(amax > 0, amax / np.float32(FP8_E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scales[b0:b1] = sc.reshape(scales[b0:b1].shape)
        codes[b0:b1] = encode_e4m3fn((x / sc).astype(np.float32))
    return codes, scales


def small_spec(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
               kv_dtype="bf16", context=100, append=False, pool="oversized2x",
               case_id=100, name="small") -> Spec:
    """A custom small workload (tests use these for many shapes)."""
    return Spec(name, case_id, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                kv_dtype=kv_dtype, context=context, append=append, pool=pool)
