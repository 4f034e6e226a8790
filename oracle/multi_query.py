"""Attention for several consecutive query positions per sequence over the paged
cache, in float64 (the definition).  Test infrastructure only.

Cites:
* *LLM Inference Systems Engineering* (jasonzhang109), §2.1.3: the
  verification step of speculative decoding runs the target over the pending
  token and the drafted ones in one pass against the committed cache; the
  provisional cache holds those positions.
* *The Mathematics of Transformer Inference* (hs-black), §10: the target model
  runs one forward over the prefix plus the k drafted tokens and obtains the
  k + 1 positions' outputs; each position sees the prefix and the earlier new
  positions (the causal rule of §1: a position attends to itself and what came
  before it).
* Paged addressing, fp8 decoding and the single-position definition: see
  ``oracle.attention`` and ``oracle.cache``.

For sequence b with ctx = context_lens[b] cached tokens (the Q new ones are the
last Q of them), query i (0 <= i < Q) sits at position ctx - Q + i and attends
to the tokens 0 .. ctx - Q + i, i.e. to the first n_i = ctx - Q + 1 + i rows:
  out[b, i, h], lse[b, i, h] = single-position attention of q[b, i, h] over those
  n_i tokens.
Readings (the pages do not treat them): ctx = 0 gives out = 0 and lse = -inf
for every query; 0 < ctx < Q is malformed (a query would sit before position 0)
and gives NaN.  With a sliding window w > 0, query i also drops the tokens
before position ctx - Q + i - w + 1 (see ``oracle.attention``).
"""
import numpy as np

from .attention import dense_decode_attention, dequantized_rows
from .bf16 import bf16_to_float64


def paged_multi_query_attention(q_bits, k_pool, v_pool, block_tables, context_lens, block_size,
                                softmax_scale, kv_dtype="bf16", k_scale=None, v_scale=None,
                                sliding_window=0):
    """q_bits uint16 [B][Q][H_q][d]; pools, tables, scales as ``paged_decode_attention``.

    Returns (out float64 [B][Q][H_q][d], lse float64 [B][Q][H_q]).
    """
    q = bf16_to_float64(q_bits)
    B, Q, Hq, D = q.shape
    out = np.zeros((B, Q, Hq, D), dtype=np.float64)
    lse = np.full((B, Q, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        ctx = int(context_lens[b])
        if ctx == 0:
            continue
        if ctx < Q:
            out[b] = np.nan
            lse[b] = np.nan
            continue
        kr = dequantized_rows(k_pool, block_tables[b], ctx, block_size, kv_dtype, k_scale, "k")
        vr = dequantized_rows(v_pool, block_tables[b], ctx, block_size, kv_dtype, v_scale, "v")
        for i in range(Q):
            n = ctx - Q + 1 + i                        # tokens up to and including position ctx-Q+i
            lo = max(0, n - sliding_window) if sliding_window > 0 else 0
            out[b, i], lse[b, i] = dense_decode_attention(q[b, i], kr[:, lo:n], vr[:, lo:n],
                                                          softmax_scale)
    return out, lse
