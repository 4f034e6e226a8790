"""Float64 CPU oracle for paged GQA decode attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or links anything here, and this
package never imports the product path.  It is plain, slow and meant to be
checked by eye against the pages it cites:

* ``attention.paged_decode_attention`` — the definition of single-token decode
  attention over a paged KV cache, written out in float64.
* ``cache.kv_append`` / ``cache.kv_append_tokens`` / ``cache.gather_sequence`` /
  ``cache.copy_blocks`` — the block-table scatter, gather and copy-on-write
  block copy, as integer indexing.
* ``multi_query.paged_multi_query_attention`` — several consecutive query
  positions per sequence (speculative verification), each attending causally.
* ``fp8.decode_e4m3fn`` / ``fp8.encode_e4m3fn`` — OCP FP8 E4M3 (finite-only,
  max 448) decoding from the format definition, and encoding as a nearest-value
  search with ties to even.
* ``quant_cache.kv_append_fp8`` — appending tokens to an fp8 cache with one
  scale per (block, KV head), the scale growing (and older codes re-encoded)
  when new tokens exceed it.
* ``online.chunked_attention`` / ``online.merge_partials`` — the online-softmax
  block update and the log-sum-exp merge of partial results, in the pages' own
  steps, to pin the split decomposition against the direct form.
* ``formulas`` — KV-cache byte count and decode-attention arithmetic intensity.

Every function is pinned by ``-m "not gpu"`` tests to something other than
itself (brute force, a float64 library routine, closed forms, invariants and
values printed on the pages).  No function here is "parity unpinned".
"""
from .attention import paged_decode_attention, dense_decode_attention
from .cache import kv_append, kv_append_tokens, gather_sequence, copy_blocks
from .multi_query import paged_multi_query_attention
from .fp8 import decode_e4m3fn, encode_e4m3fn
from .quant_cache import kv_append_fp8
from .bf16 import bf16_to_float64
from .online import chunked_attention, merge_partials
from .formulas import kv_cache_bytes, decode_attention_flops, decode_attention_intensity

__all__ = [
    "paged_decode_attention", "dense_decode_attention", "kv_append", "kv_append_tokens",
    "gather_sequence", "copy_blocks", "paged_multi_query_attention",
    "decode_e4m3fn", "encode_e4m3fn", "kv_append_fp8", "bf16_to_float64", "chunked_attention", "merge_partials",
    "kv_cache_bytes", "decode_attention_flops", "decode_attention_intensity",
]
