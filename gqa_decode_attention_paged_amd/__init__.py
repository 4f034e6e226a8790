"""Python binding of the paged GQA decode-attention library (libgqa_paged.so).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI declared in ``include/gqa_paged.h``.  PyTorch supplies
device memory and the stream; there is no CPU fallback — if the shared library
is missing, ``load()`` raises.

Tensor conventions (all on the same CUDA/HIP device):
  q             [B][H_q][d_h]    torch.bfloat16
  k_cache/v_cache [num_blocks][H_kv][block_size][d_h]  torch.bfloat16, or
                torch.uint8 / torch.float8_e4m3fn holding OCP E4M3 codes
  k_scale/v_scale [num_blocks][H_kv] torch.float32 (fp8 pools only)
  block_tables  [B][max_blocks_per_seq] torch.int32
  context_lens, positions [B] torch.int32
  out           [B][H_q][d_h] torch.float32; out_lse [B][H_q] torch.float32
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "load", "GqaError", "PagedShape", "kv_append", "paged_decode_attention",
    "workspace_size", "num_splits", "kv_gather", "last_error", "version", "LIB_PATH",
    "paged_decode_append_attention", "make_workspace", "workspace_init", "make_shape",
    "workspace_status", "STATUS_BAD_CONTEXT_LEN", "STATUS_CONTEXT_OVER_HINT",
    "STATUS_BAD_BLOCK_ID", "STATUS_BAD_APPEND", "set_split_tokens", "split_tokens",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_paged.so")

GQA_KV_BF16 = 0
GQA_KV_FP8_E4M3 = 1
GQA_KV_FP8_E4M3_KIVI = 2
GQA_FLAG_BATCH_INVARIANT = 1
# Device status bits recorded in a workspace by the attention calls (gqa_paged.h).
STATUS_BAD_CONTEXT_LEN = 1
STATUS_CONTEXT_OVER_HINT = 2
STATUS_BAD_BLOCK_ID = 4
STATUS_BAD_APPEND = 8
STATUS_NAMES = {0: "GQA_OK", 1: "GQA_ERR_INVALID_ARG", 2: "GQA_ERR_UNSUPPORTED",
                3: "GQA_ERR_WORKSPACE", 4: "GQA_ERR_HIP"}


class PagedShape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("sliding_window", ctypes.c_int32)]


class GqaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None
_P = ctypes.c_void_p


def load():
    """Load libgqa_paged.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m gqa_decode_attention_paged_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    S = ctypes.POINTER(PagedShape)
    lib.gqa_kv_append.argtypes = [S, _P, _P, _P, _P, _P, _P, _P]
    lib.gqa_kv_append.restype = ctypes.c_int
    lib.gqa_kv_append_tokens.argtypes = [S, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P]
    lib.gqa_kv_append_tokens.restype = ctypes.c_int
    lib.gqa_paged_multi_query_workspace_size.argtypes = [S, ctypes.c_int32, ctypes.c_int32]
    lib.gqa_paged_multi_query_workspace_size.restype = ctypes.c_size_t
    lib.gqa_paged_decode_multi_query.argtypes = [S, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P,
                                                 ctypes.c_int32, ctypes.c_float, _P, _P, _P,
                                                 ctypes.c_size_t, _P]
    lib.gqa_paged_decode_multi_query.restype = ctypes.c_int
    lib.gqa_paged_decode_multi_query_append.argtypes = [S, ctypes.c_int32, _P, _P, _P, _P, _P,
                                                        _P, _P, _P, _P, ctypes.c_int32,
                                                        ctypes.c_float, _P, _P, _P,
                                                        ctypes.c_size_t, _P]
    lib.gqa_paged_decode_multi_query_append.restype = ctypes.c_int
    lib.gqa_decode_num_splits.argtypes = [ctypes.c_int32]
    lib.gqa_decode_num_splits.restype = ctypes.c_int32
    lib.gqa_set_split_tokens.argtypes = [ctypes.c_int32]
    lib.gqa_set_split_tokens.restype = ctypes.c_int
    lib.gqa_split_tokens.argtypes = []
    lib.gqa_split_tokens.restype = ctypes.c_int32
    lib.gqa_paged_decode_workspace_size.argtypes = [S, ctypes.c_int32]
    lib.gqa_paged_decode_workspace_size.restype = ctypes.c_size_t
    lib.gqa_paged_decode_attention.argtypes = [S, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                               ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]
    lib.gqa_paged_decode_attention.restype = ctypes.c_int
    lib.gqa_paged_decode_append_attention.argtypes = [S, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                      _P, ctypes.c_int32, ctypes.c_float, _P,
                                                      _P, _P, ctypes.c_size_t, _P]
    lib.gqa_paged_decode_append_attention.restype = ctypes.c_int
    lib.gqa_paged_decode_attention_noalloc.argtypes = [S, _P, _P, _P, _P, _P, _P, _P,
                                                       ctypes.c_int32, ctypes.c_float, _P, _P, _P]
    lib.gqa_paged_decode_attention_noalloc.restype = ctypes.c_int
    lib.gqa_paged_decode_workspace_init.argtypes = [S, ctypes.c_int32, _P, ctypes.c_size_t, _P]
    lib.gqa_paged_decode_workspace_init.restype = ctypes.c_int
    lib.gqa_kv_append_fp8.argtypes = [S, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.gqa_kv_append_fp8.restype = ctypes.c_int
    lib.gqa_probe_read.argtypes = [_P, ctypes.c_int64, _P, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32, _P, _P]
    lib.gqa_probe_read.restype = ctypes.c_int
    lib.gqa_probe_read_pattern.argtypes = [_P, ctypes.c_int64, _P, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]
    lib.gqa_probe_read_pattern.restype = ctypes.c_int
    lib.gqa_workspace_read_status.argtypes = [_P, ctypes.c_size_t, ctypes.c_int32,
                                              ctypes.POINTER(ctypes.c_uint32), _P]
    lib.gqa_workspace_read_status.restype = ctypes.c_int
    lib.gqa_kv_copy_blocks.argtypes = [S, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P]
    lib.gqa_kv_copy_blocks.restype = ctypes.c_int
    lib.gqa_kv_gather.argtypes = [S, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P]
    lib.gqa_kv_gather.restype = ctypes.c_int
    lib.gqa_last_error.argtypes = []
    lib.gqa_last_error.restype = ctypes.c_char_p
    lib.gqa_version.argtypes = []
    lib.gqa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load().gqa_last_error().decode()


def version() -> str:
    return load().gqa_version().decode()


def _check(status: int):
    if status != 0:
        raise GqaError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtypes(kind):
    import torch
    bf16 = (torch.bfloat16, torch.int16, torch.uint16)
    return {"bf16": bf16, "pool": bf16 + (torch.uint8, torch.float8_e4m3fn),
            "i32": (torch.int32,), "f32": (torch.float32,)}[kind]


class _Checks:
    """Checks of the tensor arguments of one call, before any pointer crosses the
    boundary.  The kernels index raw device memory by the sizes they are given,
    so a tensor of another dtype, size or layout, or one in host memory, would
    be read out of bounds instead of rejected.  Each call checks dtype, shape
    and layout per tensor, then (``on_gpu``) that all of them are in GPU memory."""

    def __init__(self):
        self.seen = []

    def __call__(self, t, name, kind=None, shape=None, min_rows=None):
        """``shape`` is the exact shape; ``min_rows`` a lower bound on the first
        dimension (tables and lengths may cover more sequences than the call uses)."""
        if t is None:
            raise ValueError(f"{name} is required")
        if kind is not None and t.dtype not in _dtypes(kind):
            names = " or ".join(str(d).replace("torch.", "") for d in _dtypes(kind))
            raise TypeError(f"{name}: expected {names}, got {str(t.dtype).replace('torch.', '')}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
        if min_rows is not None and (t.dim() == 0 or t.shape[0] < min_rows):
            raise ValueError(f"{name}: needs at least {min_rows} rows, got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        self.seen.append((name, t))
        return t

    def on_gpu(self):
        for name, t in self.seen:
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be in GPU memory, got {t.device}")


def _pools(chk, k_cache, v_cache, k_scale=None, v_scale=None):
    """The two pools: same dtype and [NB][H_kv][BS][d_h] shape; fp8 scales, when
    given, float32 in the per-(block, head) or KIVI layout."""
    chk(k_cache, "k_cache", "pool")
    if k_cache.dim() != 4:
        raise ValueError(f"k_cache: expected [num_blocks][H_kv][block_size][d_h], got "
                         f"shape {tuple(k_cache.shape)}")
    if v_cache.dtype != k_cache.dtype:
        raise TypeError(f"v_cache: expected {k_cache.dtype} like k_cache, got {v_cache.dtype}")
    chk(v_cache, "v_cache", shape=k_cache.shape)
    nb, hkv, bs, d = k_cache.shape
    kivi = _kv_dtype(k_cache, k_scale) == GQA_KV_FP8_E4M3_KIVI
    if k_scale is not None:
        chk(k_scale, "k_scale", "f32", (nb, hkv, d) if kivi else (nb, hkv))
    if v_scale is not None:
        chk(v_scale, "v_scale", "f32", (nb, hkv, bs) if kivi else (nb, hkv))
    return nb, hkv, bs, d


def _attention_args(chk, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                    out, out_lse, workspace):
    """Common checks of the attention entry points; q is [B](Q)[H_q][d_h]."""
    chk(q, "q", "bf16")
    _, _, _, d = _pools(chk, k_cache, v_cache, k_scale, v_scale)
    if q.shape[-1] != d:
        raise ValueError(f"q: head dim {q.shape[-1]} differs from the pools' {d}")
    B = q.shape[0]
    chk(block_tables, "block_tables", "i32", min_rows=B)
    if block_tables.dim() != 2:
        raise ValueError(f"block_tables: expected [B][max_blocks], got {tuple(block_tables.shape)}")
    chk(context_lens, "context_lens", "i32", min_rows=B)
    chk(out, "out", "f32", tuple(q.shape))
    if out_lse is not None:
        chk(out_lse, "out_lse", "f32", tuple(q.shape[:-1]))
    chk(workspace, "workspace")


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _kv_dtype(cache, k_scale=None) -> int:
    import torch
    if cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        if k_scale is not None and k_scale.dim() == 3:
            return GQA_KV_FP8_E4M3_KIVI
        return GQA_KV_FP8_E4M3
    if cache.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return GQA_KV_BF16
    raise TypeError(f"unsupported KV cache dtype {cache.dtype}")


def make_shape(num_seqs, num_q_heads, k_cache, block_tables, batch_invariant=False,
               sliding_window=0, k_scale=None) -> PagedShape:
    """The shape of a call.  An fp8 pool whose k_scale is [NB][H_kv][d_h] (one scale
    per channel) has the KIVI layout."""
    nb, hkv, bs, d = k_cache.shape
    return PagedShape(num_seqs, num_q_heads, hkv, d, bs, nb, block_tables.shape[1],
                      _kv_dtype(k_cache, k_scale),
                      GQA_FLAG_BATCH_INVARIANT if batch_invariant else 0, int(sliding_window))


def num_splits(context_len: int) -> int:
    """Partial attentions a sequence of this length is split into under the
    batch-invariant plan (with the split-length override, if one is set)."""
    return int(load().gqa_decode_num_splits(int(context_len)))


def set_split_tokens(tokens: int) -> None:
    """Set (a multiple of 32 in [128, 2^19]) or clear (0) the process-wide
    split-length override; while set, attention calls split each sequence by its
    own length into about one split per that many tokens (at most 64 splits)."""
    _check(load().gqa_set_split_tokens(int(tokens)))


def split_tokens() -> int:
    """The current split-length override (0: none)."""
    return int(load().gqa_split_tokens())


def workspace_size(shape: PagedShape, max_context_len: int) -> int:
    return int(load().gqa_paged_decode_workspace_size(ctypes.byref(shape), int(max_context_len)))


def kv_append(k_new, v_new, k_cache, v_cache, block_tables, positions):
    """Write one new token per sequence into the paged pools (in place)."""
    chk = _Checks()
    lib = load()
    _, hkv, _, d = _pools(chk, k_cache, v_cache)
    B = k_new.shape[0]
    chk(k_new, "k_new", "bf16", (B, hkv, d))
    chk(v_new, "v_new", "bf16", (B, hkv, d))
    chk(block_tables, "block_tables", "i32", min_rows=B)
    chk(positions, "positions", "i32", min_rows=B)
    shape = make_shape(B, hkv, k_cache, block_tables)
    chk.on_gpu()
    _check(lib.gqa_kv_append(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                             _ptr(v_cache), _ptr(block_tables), _ptr(positions),
                             _stream(k_cache)))


def kv_append_tokens(k_new, v_new, k_cache, v_cache, block_tables, positions):
    """Write T new tokens per sequence ([B][T][H_kv][d_h] rows at positions [B][T])."""
    chk = _Checks()
    lib = load()
    _, hkv, _, d = _pools(chk, k_cache, v_cache)
    B, T = k_new.shape[0], k_new.shape[1]
    chk(k_new, "k_new", "bf16", (B, T, hkv, d))
    chk(v_new, "v_new", "bf16", (B, T, hkv, d))
    chk(block_tables, "block_tables", "i32", min_rows=B)
    chk(positions, "positions", "i32", (B, T))
    shape = make_shape(B, hkv, k_cache, block_tables)
    chk.on_gpu()
    _check(lib.gqa_kv_append_tokens(ctypes.byref(shape), int(T), _ptr(k_new), _ptr(v_new),
                                    _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                    _ptr(positions), _stream(k_cache)))


def multi_query_workspace_size(shape: PagedShape, num_queries: int, max_context_len: int) -> int:
    return int(load().gqa_paged_multi_query_workspace_size(ctypes.byref(shape), int(num_queries),
                                                           int(max_context_len)))


def paged_decode_multi_query(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                             softmax_scale=None, k_scale=None, v_scale=None, out=None,
                             out_lse=None, workspace=None, return_lse=True,
                             batch_invariant=False, sliding_window=0):
    """Attention for Q consecutive query positions per sequence, q [B][Q][H_q][d_h]: query i
    sits at position context_lens[b] - Q + i and attends causally.  Returns (out, lse)."""
    import torch
    chk = _Checks()
    lib = load()
    B, Q, Hq, D = q.shape
    shape = make_shape(B, Hq, k_cache, block_tables, batch_invariant, sliding_window, k_scale)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Q, Hq, D), dtype=torch.float32, device=q.device)
    if out_lse is None and return_lse:
        out_lse = torch.empty((B, Q, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = multi_query_workspace_size(shape, Q, max_context_len)
        workspace = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _attention_args(chk, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, out,
                    out_lse, workspace)
    chk.on_gpu()
    _check(lib.gqa_paged_decode_multi_query(
        ctypes.byref(shape), int(Q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(block_tables), _ptr(context_lens), int(max_context_len),
        float(softmax_scale), _ptr(out), _ptr(out_lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q)))
    return out, out_lse


def paged_decode_attention(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                           softmax_scale=None, k_scale=None, v_scale=None, out=None,
                           out_lse=None, workspace=None, return_lse=True, batch_invariant=False, sliding_window=0):
    """Decode attention for a batch; returns (out, lse) (lse None if not requested)."""
    import torch
    chk = _Checks()
    lib = load()
    B, Hq, D = q.shape
    shape = make_shape(B, Hq, k_cache, block_tables, batch_invariant, sliding_window, k_scale)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if out_lse is None and return_lse:
        out_lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = make_workspace(shape, max_context_len, q.device)
    _attention_args(chk, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, out,
                    out_lse, workspace)
    chk.on_gpu()
    _check(lib.gqa_paged_decode_attention(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(block_tables), _ptr(context_lens), int(max_context_len),
        float(softmax_scale), _ptr(out), _ptr(out_lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q)))
    return out, out_lse


NOALLOC_SCRATCH_BYTES = 32 << 20      # GQA_NOALLOC_SCRATCH_BYTES


def paged_decode_attention_noalloc(q, k_cache, v_cache, block_tables, context_lens,
                                   max_context_len, softmax_scale=None, k_scale=None,
                                   v_scale=None, out=None, out_lse=None, return_lse=True,
                                   batch_invariant=False, sliding_window=0):
    """paged_decode_attention with the library's static per-device workspace instead of
    a caller-supplied one (the C call allocates nothing).  Calls that overlap on one
    device race; order them on one stream."""
    import torch
    chk = _Checks()
    lib = load()
    B, Hq, D = q.shape
    shape = make_shape(B, Hq, k_cache, block_tables, batch_invariant, sliding_window, k_scale)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if out_lse is None and return_lse:
        out_lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    chk(q, "q", "bf16")
    _, _, _, d = _pools(chk, k_cache, v_cache, k_scale, v_scale)
    if d != D:
        raise ValueError(f"q: head dim {D} differs from the pools' {d}")
    chk(block_tables, "block_tables", "i32", min_rows=B)
    chk(context_lens, "context_lens", "i32", min_rows=B)
    chk(out, "out", "f32", (B, Hq, D))
    if out_lse is not None:
        chk(out_lse, "out_lse", "f32", (B, Hq))
    chk.on_gpu()
    _check(lib.gqa_paged_decode_attention_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
        _ptr(v_scale), _ptr(block_tables), _ptr(context_lens), int(max_context_len),
        float(softmax_scale), _ptr(out), _ptr(out_lse), _stream(q)))
    return out, out_lse


def paged_decode_multi_query_append(q, k_new, v_new, k_cache, v_cache, block_tables,
                                    context_lens, max_context_len, softmax_scale=None, out=None,
                                    out_lse=None, workspace=None, return_lse=True,
                                    batch_invariant=False, sliding_window=0, k_scale=None,
                                    v_scale=None):
    """Fused verification step: commit k_new/v_new [B][Q][H_kv][d_h] at positions
    context_lens[b] - Q + i, then attend for the Q positions (one kernel).  fp8
    pools: the rows are quantised into them and k_scale/v_scale updated."""
    import torch
    chk = _Checks()
    lib = load()
    B, Q, Hq, D = q.shape
    shape = make_shape(B, Hq, k_cache, block_tables, batch_invariant, sliding_window, k_scale)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Q, Hq, D), dtype=torch.float32, device=q.device)
    if out_lse is None and return_lse:
        out_lse = torch.empty((B, Q, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = multi_query_workspace_size(shape, Q, max_context_len)
        workspace = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _attention_args(chk, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, out,
                    out_lse, workspace)
    chk(k_new, "k_new", "bf16", (B, Q, k_cache.shape[1], D))
    chk(v_new, "v_new", "bf16", (B, Q, k_cache.shape[1], D))
    chk.on_gpu()
    _check(lib.gqa_paged_decode_multi_query_append(
        ctypes.byref(shape), int(Q), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
        _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), _ptr(context_lens),
        int(max_context_len),
        float(softmax_scale), _ptr(out), _ptr(out_lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q)))
    return out, out_lse


def make_workspace(shape: PagedShape, max_context_len: int, device):
    """A zero-filled workspace (its split arrival counters must start at zero)."""
    import torch
    nbytes = workspace_size(shape, max_context_len)
    return torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)


def paged_decode_append_attention(q, k_new, v_new, positions, k_cache, v_cache, block_tables,
                                  context_lens, max_context_len, softmax_scale=None, out=None,
                                  out_lse=None, workspace=None, return_lse=True,
                                  batch_invariant=False, sliding_window=0, k_scale=None,
                                  v_scale=None):
    """Fused decode step: commit the new token at positions[b], then attend (one kernel).
    fp8 pools: the row is quantised into them and k_scale/v_scale updated."""
    import torch
    chk = _Checks()
    lib = load()
    B, Hq, D = q.shape
    shape = make_shape(B, Hq, k_cache, block_tables, batch_invariant, sliding_window, k_scale)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if out_lse is None and return_lse:
        out_lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = make_workspace(shape, max_context_len, q.device)
    _attention_args(chk, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, out,
                    out_lse, workspace)
    chk(k_new, "k_new", "bf16", (B, k_cache.shape[1], D))
    chk(v_new, "v_new", "bf16", (B, k_cache.shape[1], D))
    chk(positions, "positions", "i32", min_rows=B)
    chk.on_gpu()
    _check(lib.gqa_paged_decode_append_attention(
        ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(positions), _ptr(k_cache),
        _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), _ptr(context_lens),
        int(max_context_len),
        float(softmax_scale), _ptr(out), _ptr(out_lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q)))
    return out, out_lse


def workspace_init(shape: PagedShape, max_context_len: int, workspace):
    """Zero a workspace's arrival counters on the current stream."""
    chk = _Checks()
    chk(workspace, "workspace")
    chk.on_gpu()
    _check(load().gqa_paged_decode_workspace_init(
        ctypes.byref(shape), int(max_context_len), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(workspace)))


def workspace_status(workspace, clear=False) -> int:
    """The STATUS_* bits the attention calls recorded in this workspace (blocking:
    waits for the current stream); ``clear`` zeroes them afterwards."""
    chk = _Checks()
    chk(workspace, "workspace")
    chk.on_gpu()
    word = ctypes.c_uint32(0)
    _check(load().gqa_workspace_read_status(
        _ptr(workspace), workspace.numel() * workspace.element_size(), 1 if clear else 0,
        ctypes.byref(word), _stream(workspace)))
    return int(word.value)


def kv_append_fp8(k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables,
                  start_positions):
    """Quantise and write new tokens into an fp8 pool: k_new/v_new bf16 [B][H_kv][d_h]
    (one token) or [B][T][H_kv][d_h] at positions start_positions[b] + j (in place,
    scales included).  Scales [NB][H_kv] (per (block, head)) or the KIVI layout
    (k_scale [NB][H_kv][d_h], v_scale [NB][H_kv][BS])."""
    chk = _Checks()
    lib = load()
    if k_new.dim() == 3:
        k_new, v_new = k_new.unsqueeze(1), v_new.unsqueeze(1)
    B, T = k_new.shape[0], k_new.shape[1]
    _, hkv, _, d = _pools(chk, k_cache, v_cache, k_scale, v_scale)
    chk(k_new, "k_new", "bf16", (B, T, hkv, d))
    chk(v_new, "v_new", "bf16", (B, T, hkv, d))
    chk(block_tables, "block_tables", "i32", min_rows=B)
    chk(start_positions, "start_positions", "i32", min_rows=B)
    shape = make_shape(B, hkv, k_cache, block_tables, k_scale=k_scale)
    chk.on_gpu()
    _check(lib.gqa_kv_append_fp8(ctypes.byref(shape), int(T), _ptr(k_new), _ptr(v_new),
                                 _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                 _ptr(block_tables), _ptr(start_positions), _stream(k_cache)))


def kv_copy_blocks(k_cache, v_cache, src_blocks, dst_blocks, k_scale=None, v_scale=None):
    """Copy-on-write block copy: block dst_blocks[j] of both pools (and the fp8 scales)
    becomes a copy of src_blocks[j], in place."""
    chk = _Checks()
    nb, hkv, bs, d = _pools(chk, k_cache, v_cache, k_scale, v_scale)
    chk(src_blocks, "src_blocks", "i32")
    chk(dst_blocks, "dst_blocks", "i32", shape=src_blocks.shape)
    shape = PagedShape(1, hkv, hkv, d, bs, nb, 1, _kv_dtype(k_cache, k_scale), 0, 0)
    chk.on_gpu()
    _check(load().gqa_kv_copy_blocks(ctypes.byref(shape), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(k_scale), _ptr(v_scale), _ptr(src_blocks),
                                     _ptr(dst_blocks), int(src_blocks.numel()),
                                     _stream(k_cache)))


# Per-instruction load patterns of the read probe (include/gqa_probe.h).
PROBE_WHOLE_ROWS = 0
PROBE_OPERAND_ROWS_256 = 1
PROBE_OPERAND_ROWS_128 = 2
PROBE_OPERAND_ROWS_128_NARROW = 3
PROBE_MIXED_256 = 4


def probe_read(pool_address, pool_tiles, tile_ids, num_tiles, tile_bytes, non_temporal,
               num_workgroups, sink, pattern=PROBE_WHOLE_ROWS):
    """One read-probe launch (measurement only): num_tiles tiles of tile_bytes bytes from
    the device buffer at pool_address (an address inside a tensor the caller keeps,
    holding pool_tiles tiles), through tile_ids (int32 [num_tiles]) or contiguously,
    each wave instruction covering a tile as `pattern` (PROBE_*) says."""
    chk = _Checks()
    if tile_ids is not None:
        chk(tile_ids, "tile_ids", "i32", min_rows=num_tiles)
    chk(sink, "sink", min_rows=num_workgroups * 8)
    if sink.dtype not in (__import__("torch").int32, __import__("torch").uint32):
        raise TypeError("sink: expected int32 or uint32")
    chk.on_gpu()
    _check(load().gqa_probe_read_pattern(ctypes.c_void_p(int(pool_address)), int(pool_tiles),
                                         _ptr(tile_ids), int(num_tiles), int(tile_bytes),
                                         int(pattern), 1 if non_temporal else 0,
                                         int(num_workgroups), _ptr(sink), _stream(sink)))


def kv_gather(cache, block_tables, seq, num_tokens):
    """Copy sequence ``seq``'s first ``num_tokens`` rows out of a pool: [H_kv][T][d_h]."""
    chk = _Checks()
    import torch
    lib = load()
    chk(cache, "cache", "pool")
    chk(block_tables, "block_tables", "i32")
    nb, hkv, bs, d = cache.shape
    shape = PagedShape(block_tables.shape[0], hkv, hkv, d, bs, nb, block_tables.shape[1],
                       _kv_dtype(cache), 0, 0)
    out = torch.empty((hkv, num_tokens, d), dtype=cache.dtype, device=cache.device)
    chk.on_gpu()
    _check(lib.gqa_kv_gather(ctypes.byref(shape), _ptr(cache), _ptr(block_tables), int(seq),
                             int(num_tokens), _ptr(out), _stream(cache)))
    return out
