"""Single-token decode attention over a paged KV cache, in float64 (the definition).

Cites:
* *The Mathematics of Transformer Inference* (hs-black), §1 and §4: at decode
  the one new query of each head takes a dot product with every cached key and
  forms the softmax-weighted sum of the cached values; with grouped-query
  attention G = N/K query heads read the same KV head (§5).
* *Module 10: Inference and Deployment Serving* (wrwei.github.io), "Attention
  reads a different cache per sequence": one layer and one decode position cost
  about 4 n_h d_head t FLOPs and read 2 n_kv d_head t b bytes; Lab 2 shares KV
  heads by repeating each KV head over its consecutive query heads, i.e. query
  head h reads KV head floor(h / G).
* *Ch. 6 Inference Efficiency and Model Serving* (Stochastic Parrot vol. 1),
  §6.2.2: the decode query dots all history keys and aggregates the values.
* Paged addressing: see ``oracle.cache``.

For every sequence b and query head h (g = h // G, ctx = context_lens[b]):
  k_t, v_t = rows of logical token t (t < ctx), read through the block table
  (fp8: code decoded exactly, times the (block, head) scale)
  s_t = softmax_scale * <q[b, h], k_t>
  w   = exp(s - max s) / sum exp(s - max s)
  out[b, h] = sum_t w_t v_t ;  lse[b, h] = max s + ln sum exp(s - max s)
An empty context (ctx = 0) gives out = 0 and lse = -inf (a reading: the pages
do not treat it).

Scale layouts of fp8 pools (``kv_dtype``):
* ``"fp8"``: one scale per (block, KV head), k_scale/v_scale [NB][H_kv].
* ``"fp8_kivi"``: keys scaled per channel and values per token, as KIVI does
  (*Module 10*, "Quantize the cache": key outliers and value statistics
  differ; KIVI studies per-channel keys and per-token values; *The Mathematics
  of Transformer Inference* §11: KV scales per head and per token).  k_scale is
  [NB][H_kv][d] (one scale per channel of each (block, KV head)), v_scale
  [NB][H_kv][BS] (one per slot).  value = decode(code) * the element's scale.

Sliding window (``sliding_window = w > 0``): the query, at position ctx - 1,
attends only to the w most recent tokens, ctx - w .. ctx - 1 (all of them when
ctx <= w).  *Module 10*, "Parameter count alone does not determine cache size"
(sliding-window attention keeps a bounded recent context; Mistral 7B uses a
4,096-token window); *The Mathematics of Transformer Inference* §5 (local
layers see only the most recent w tokens, so their cache is bounded by w).
"""
import numpy as np

from .bf16 import bf16_to_float64
from .cache import gather_sequence
from .fp8 import decode_e4m3fn


def _widen(pool_rows: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "bf16":
        return bf16_to_float64(pool_rows)
    if kv_dtype in ("fp8", "fp8_kivi"):
        return decode_e4m3fn(pool_rows)
    raise ValueError(kv_dtype)


def dequantized_rows(pool, table_row, ctx, block_size, kv_dtype, scale=None, which="k"):
    """The first ctx K (``which="k"``) or V rows of one sequence, widened to float64
    [H_kv][ctx][d] (fp8: decoded and multiplied by each element's scale)."""
    rows = _widen(gather_sequence(pool, table_row, ctx, block_size), kv_dtype)
    if kv_dtype == "bf16":
        return rows
    t = np.arange(ctx)
    phys = np.asarray(table_row)[t // block_size]
    sc = np.asarray(scale, dtype=np.float64)
    if kv_dtype == "fp8":
        return rows * sc[phys, :].T[:, :, None]                     # [H_kv][ctx] per token's block
    if kv_dtype == "fp8_kivi" and which == "k":
        return rows * np.transpose(sc[phys], (1, 0, 2))              # per channel: [H_kv][ctx][d]
    if kv_dtype == "fp8_kivi":
        return rows * sc[phys, :, t % block_size].T[:, :, None]     # per slot (token)
    raise ValueError(kv_dtype)


def dense_decode_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, softmax_scale: float):
    """One sequence: q [H_q][d] float64, k/v [H_kv][ctx][d] float64 -> (out [H_q][d], lse [H_q])."""
    Hq, D = q.shape
    Hkv, ctx, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    lse = np.full(Hq, -np.inf, dtype=np.float64)
    if ctx == 0:
        return out, lse
    for h in range(Hq):
        g = h // G
        s = softmax_scale * (k[g] @ q[h])            # [ctx]
        mx = np.max(s)
        e = np.exp(s - mx)
        z = np.sum(e)
        out[h] = (e / z) @ v[g]
        lse[h] = mx + np.log(z)
    return out, lse


def paged_decode_attention(q_bits, k_pool, v_pool, block_tables, context_lens, block_size,
                           softmax_scale, kv_dtype="bf16", k_scale=None, v_scale=None,
                           sliding_window=0):
    """Paged decode attention for a batch.

    q_bits      uint16 [B][H_q][d] (bf16 bit patterns)
    k_pool/v_pool uint16 (bf16) or uint8 (fp8 codes) [NB][H_kv][BS][d]
    block_tables int [B][max_blocks]; context_lens int [B]
    k_scale/v_scale float32 [NB][H_kv] for fp8 (dequantised value = decode(code) * scale);
                for fp8_kivi k_scale [NB][H_kv][d] and v_scale [NB][H_kv][BS]
    sliding_window  w > 0 restricts each query to its w most recent tokens (0: all)
    Returns (out float64 [B][H_q][d], lse float64 [B][H_q]).
    """
    q = bf16_to_float64(q_bits)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        ctx = int(context_lens[b])
        if ctx == 0:
            continue
        kr = dequantized_rows(k_pool, block_tables[b], ctx, block_size, kv_dtype, k_scale, "k")
        vr = dequantized_rows(v_pool, block_tables[b], ctx, block_size, kv_dtype, v_scale, "v")
        lo = max(0, ctx - sliding_window) if sliding_window > 0 else 0
        out[b], lse[b] = dense_decode_attention(q[b], kr[:, lo:], vr[:, lo:], softmax_scale)
    return out, lse
