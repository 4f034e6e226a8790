"""KV-cache byte count and decode-attention work, as the pages state them.

Cites:
* *Ch. 6 Inference Efficiency and Model Serving* (Stochastic Parrot vol. 1),
  §6.3: the KV cache holds about 2 L B T H_kv d_h b bytes (2 for K and V,
  L layers, B sequences, T cached tokens, H_kv KV heads, d_h per-head width,
  b bytes per element); its worked example L=32, B=1, T=8192, H_kv=8,
  d_h=128, bf16 is exactly 2^30 bytes.
* *LLM Inference Systems Engineering* (jasonzhang109), §2.2.3: per token
  2 h_kv d_head L b bytes, 131072 B for h_kv=8, d_head=128, L=32, BF16.
* *Module 10: Inference and Deployment Serving* (wrwei.github.io), "Attention
  reads a different cache per sequence": per layer and decode position about
  4 n_h d_head t FLOPs against 2 n_kv d_head t b bytes, so the intensity is
  2 (n_h / n_kv) / b FLOP per byte — four for G = 4 with bf16, whatever the batch.
* *The Mathematics of Transformer Inference* (hs-black), §4: decode attention
  intensity is about 1 for MHA and about G with grouped queries.
"""


def kv_cache_bytes(layers: int, batch: int, tokens: int, kv_heads: int, head_dim: int,
                   bytes_per_elem: float) -> float:
    return 2 * layers * batch * tokens * kv_heads * head_dim * bytes_per_elem


def decode_attention_flops(q_heads: int, head_dim: int, tokens: int) -> int:
    """FLOPs of one layer, one sequence, one decode position (QK and PV, 2 per MAC)."""
    return 4 * q_heads * head_dim * tokens


def decode_attention_intensity(q_heads: int, kv_heads: int, bytes_per_elem: float) -> float:
    """FLOP per KV byte read; independent of batch and context length."""
    flops = decode_attention_flops(q_heads, 1, 1)
    bytes_read = kv_cache_bytes(1, 1, 1, kv_heads, 1, bytes_per_elem)
    return flops / bytes_read
