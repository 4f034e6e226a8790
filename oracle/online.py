"""Block-wise (online) softmax and log-sum-exp merge of partial attentions, float64.

These are the two algorithmic steps the split decode path is built from.  They
are kept in the oracle so that tests can pin the decomposition itself: for any
chunking, the chunked form must equal ``dense_decode_attention`` up to float64
rounding.

Cites:
* *LLM Inference Systems Engineering* (jasonzhang109), §2.8.3 (FlashAttention):
  for one score row keep the running max m, the exponential sum l and the
  unnormalised weighted value sum o.  A new chunk with scores s and values V
  updates them as
      m' = max(m, max s)
      l' = e^(m - m') l + sum e^(s - m')
      o' = e^(m - m') o + sum e^(s - m') V
  and the output is o' / l'.  Only these three reductions survive between
  chunks, and the softmax result is unchanged.
* *The Mathematics of Transformer Inference* (hs-black), §8: when the KV cache
  is sharded along the sequence, each shard computes local attention and the
  shards are combined by a log-sum-exp merge, as in FlashAttention.

The merge written out: shard j returns its normalised output o_j and its
log-sum-exp lse_j = m_j + ln l_j.  With M = max_j lse_j and
w_j = exp(lse_j - M), the merged output is sum_j w_j o_j / sum_j w_j and the
merged log-sum-exp is M + ln sum_j w_j.  Shards with lse_j = -inf (no tokens)
carry zero weight.
"""
import numpy as np


def chunked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, softmax_scale: float,
                      chunk: int):
    """One query row over one KV stream, processed ``chunk`` tokens at a time.

    q [d], k/v [T][d] float64.  Returns (out [d], lse scalar).
    """
    T, D = k.shape
    m = -np.inf
    l = 0.0
    o = np.zeros(D, dtype=np.float64)
    for c0 in range(0, T, chunk):
        s = softmax_scale * (k[c0:c0 + chunk] @ q)
        m_new = max(m, float(np.max(s)))
        alpha = np.exp(m - m_new) if m != -np.inf else 0.0
        p = np.exp(s - m_new)
        l = alpha * l + np.sum(p)
        o = alpha * o + p @ v[c0:c0 + chunk]
        m = m_new
    if T == 0:
        return o, -np.inf
    return o / l, m + np.log(l)


def merge_partials(outs: np.ndarray, lses: np.ndarray):
    """Merge shard results: outs [S][d] (each normalised), lses [S] -> (out [d], lse)."""
    lses = np.asarray(lses, dtype=np.float64)
    outs = np.asarray(outs, dtype=np.float64)
    if lses.size == 0 or np.all(lses == -np.inf):
        return np.zeros(outs.shape[-1]), -np.inf
    M = np.max(lses)
    w = np.exp(lses - M)
    z = np.sum(w)
    return (w @ outs) / z, M + np.log(z)
