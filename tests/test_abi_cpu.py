"""CPU-only checks of the C ABI: the library loads, exports every declared symbol,
and its host-side logic (split policy, workspace size, argument validation)
behaves as documented.  No call here launches a kernel."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_paged.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def lib():
    import gqa_decode_attention_paged_amd as gqa
    from gqa_decode_attention_paged_amd import build
    if not os.path.exists(gqa.LIB_PATH):
        build.build()
    return gqa.load()


def declared_functions():
    """Every function the headers under include/ declare."""
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names.update(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("gqa_kv_append", "gqa_paged_decode_attention",
                     "gqa_paged_decode_workspace_size", "gqa_last_error"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def _shape(**kw):
    from gqa_decode_attention_paged_amd import PagedShape
    base = dict(num_seqs=2, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                num_blocks=1024, max_blocks_per_seq=3000, kv_dtype=0, flags=0, sliding_window=0)
    base.update(kw)
    return PagedShape(**base)


def test_split_policy(lib):
    import gqa_decode_attention_paged_amd as gqa
    assert gqa.num_splits(0) == 0 and gqa.num_splits(-5) == 0
    assert gqa.num_splits(1) == 1 and gqa.num_splits(128) == 1 and gqa.num_splits(129) == 2
    assert gqa.num_splits(8192) == 64
    assert gqa.num_splits(32769) <= 64
    prev = 0
    for ctx in range(0, 20000, 37):
        n = gqa.num_splits(ctx)
        assert 0 <= n <= 64
        assert n >= (1 if ctx > 0 else 0)
        prev = n
    assert prev > 0


def test_workspace_size_formula(lib):
    import gqa_decode_attention_paged_amd as gqa
    s = _shape()
    ms = gqa.num_splits(8192)
    rows = 2 * 32 * ms
    o_off = (2 * 8 * 64 * 4 + 255) // 256 * 256     # counters come first, 256 B apart
    lse_off = (o_off + rows * 128 * 4 + 255) // 256 * 256
    assert gqa.workspace_size(s, 8192) == lse_off + rows * 4
    assert gqa.workspace_size(_shape(head_dim=96), 8192) == 0      # unsupported
    assert gqa.workspace_size(s, -1) == 0


def test_workspace_covers_every_plan_up_to_the_hint(lib):
    """The plan of a 10000-token hint rounds to 63 splits while an 8192-token sequence
    under it needs 64: the workspace provides min(64, ceil(len / 128)) splits."""
    import gqa_decode_attention_paged_amd as gqa
    assert gqa.num_splits(10000) == 63 and gqa.num_splits(8192) == 64
    s = _shape()
    rows = 2 * 32 * 64
    o_off = (2 * 8 * 64 * 4 + 255) // 256 * 256
    lse_off = (o_off + rows * 128 * 4 + 255) // 256 * 256
    assert gqa.workspace_size(s, 10000) == lse_off + rows * 4


def test_sliding_window_bounds_the_workspace(lib):
    """With a window the split partials cover the window's span, not the hint."""
    import gqa_decode_attention_paged_amd as gqa
    full = gqa.workspace_size(_shape(), 32768)
    win = gqa.workspace_size(_shape(sliding_window=1000), 32768)
    span = 1000 + 16 - 1                           # window + partial first block
    rows = 2 * 32 * -(-span // 128)
    o_off = (2 * 8 * 64 * 4 + 255) // 256 * 256
    lse_off = (o_off + rows * 128 * 4 + 255) // 256 * 256
    assert win == lse_off + rows * 4 and win < full
    assert _call_decode(lib, _shape(sliding_window=-1)) == 1


def _call_decode(lib, shape, ws_bytes=1 << 30, ptr=16, **over):
    args = dict(q=ptr, k=ptr, v=ptr, ks=None, vs=None, bt=ptr, ctx=ptr, max_ctx=100,
                scale=0.1, out=ptr, lse=None, ws=ptr, ws_bytes=ws_bytes)
    args.update(over)
    P = ctypes.c_void_p
    return lib.gqa_paged_decode_attention(
        ctypes.byref(shape), P(args["q"]), P(args["k"]), P(args["v"]), P(args["ks"]),
        P(args["vs"]), P(args["bt"]), P(args["ctx"]), args["max_ctx"], args["scale"],
        P(args["out"]), P(args["lse"]), P(args["ws"]), args["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=96), 2), (dict(block_size=8), 2), (dict(num_q_heads=24), 2),
    (dict(num_q_heads=512), 2), (dict(num_q_heads=96), 2),   # G = 64; G = 12
    (dict(num_q_heads=30), 1), (dict(num_seqs=-1), 1), (dict(kv_dtype=7), 2),
    (dict(num_blocks=0), 1), (dict(flags=6), 1),
])
def test_decode_rejects_bad_shapes(lib, over, status):
    assert _call_decode(lib, _shape(**over)) == status
    assert lib.gqa_last_error().decode() != ""


@pytest.mark.parametrize("over,status", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(ws=None), 3), (dict(ws_bytes=10), 3),
    (dict(q=17), 1), (dict(max_ctx=-1), 1), (dict(max_ctx=10 ** 6), 1),
    (dict(scale=float("nan")), 1), (dict(ks=16), 1),
])
def test_decode_rejects_bad_arguments(lib, over, status):
    assert _call_decode(lib, _shape(), **over) == status


def test_fp8_needs_scales(lib):
    assert _call_decode(lib, _shape(kv_dtype=1)) == 1


def test_zero_sequences_return_ok_without_launching(lib):
    assert _call_decode(lib, _shape(num_seqs=0)) == 0


@pytest.mark.parametrize("hq,status", [(128, 0), (256, 0), (512, 2)])
def test_group_sizes_up_to_32_are_accepted(lib, hq, status):
    """G = 16 and 32 (8 KV heads) pass the shape checks; G = 64 is more rows than
    a kernel takes.  No sequences, so nothing launches."""
    assert _call_decode(lib, _shape(num_seqs=0, num_q_heads=hq)) == status


def test_fused_append_validation(lib):
    P = ctypes.c_void_p
    s = _shape()
    call = lambda shape, pos, kn, sc=None: lib.gqa_paged_decode_append_attention(
        ctypes.byref(shape), P(16), P(kn), P(16), P(pos), P(16), P(16), P(sc), P(sc), P(16),
        P(16), 100, 0.1, P(16), None, P(16), 1 << 30, None)
    assert call(s, None, 16) == 1                     # positions required
    assert call(s, 16, None) == 1                     # new rows required
    assert call(s, 16, 16, 16) == 1                   # bf16 pools take no scales
    assert call(_shape(kv_dtype=1), 16, 16) == 1      # fp8 pools need their scales
    assert call(_shape(num_seqs=0), None, None) == 0
    mq = lambda shape, nq: lib.gqa_paged_decode_multi_query_append(
        ctypes.byref(shape), nq, P(16), P(16), P(16), P(16), P(16), P(16), P(16), P(16), P(16),
        100, 0.1, P(16), None, P(16), 1 << 30, None)
    assert mq(_shape(kv_dtype=1, num_q_heads=8, block_size=16), 17) == 2   # > block size


def test_probe_validation(lib):
    P = ctypes.c_void_p
    pr = lib.gqa_probe_read
    assert pr(P(16), 8, None, 8, 3000, 1, 1, P(16), None) == 2          # tile size
    assert pr(None, 8, None, 8, 4096, 1, 1, P(16), None) == 1
    assert pr(P(16), 8, None, 8, 4096, 1, 0, P(16), None) == 1          # no workgroups
    assert pr(P(16), 8, None, 9, 4096, 1, 1, P(16), None) == 1          # stream past the pool
    assert pr(P(8), 8, None, 8, 4096, 1, 1, P(16), None) == 1           # misaligned
    assert pr(P(16), 8, None, 0, 4096, 1, 1, P(16), None) == 0          # nothing to read


def test_probe_pattern_validation(lib):
    P = ctypes.c_void_p
    pp = lib.gqa_probe_read_pattern
    call = lambda tile, pattern, pool=P(16): pp(pool, 8, None, 8, tile, pattern, 1, 1, P(16), None)
    assert call(4096, 5) == 2 and call(4096, -1) == 2                   # no such pattern
    assert call(2048, 1) == 2 and call(2048, 4) == 2                    # 256-byte rows: 4 KiB tiles
    assert call(1024, 2) == 2 and call(1024, 3) == 2                    # 128-byte rows: 2 KiB tiles
    for tile, pattern in ((1024, 0), (4096, 1), (2048, 2), (2048, 3), (8192, 4)):
        assert call(tile, pattern, None) == 1                           # accepted; NULL pool refused
        assert pp(P(16), 8, None, 0, tile, pattern, 1, 1, P(16), None) == 0   # nothing to read


def test_read_status_validation(lib):
    P = ctypes.c_void_p
    word = ctypes.c_uint32(7)
    rd = lib.gqa_workspace_read_status
    assert rd(None, 1 << 20, 0, ctypes.byref(word), None) == 1
    assert rd(P(16), 1 << 20, 0, None, None) == 1
    assert rd(P(16), 4, 0, ctypes.byref(word), None) == 3        # the word sits at bytes 4..7
    assert word.value == 7


def test_workspace_init_validation(lib):
    P = ctypes.c_void_p
    s = _shape()
    assert lib.gqa_paged_decode_workspace_init(ctypes.byref(s), 100, None, 0, None) == 3
    assert lib.gqa_paged_decode_workspace_init(ctypes.byref(s), -1, P(16), 1 << 20, None) == 1


def test_append_validation(lib):
    P = ctypes.c_void_p
    s = _shape(kv_dtype=1)
    assert lib.gqa_kv_append(ctypes.byref(s), P(16), P(16), P(16), P(16), P(16), P(16), None) == 2
    s = _shape()
    assert lib.gqa_kv_append(ctypes.byref(s), None, P(16), P(16), P(16), P(16), P(16), None) == 1
    assert lib.gqa_kv_append(None, P(16), P(16), P(16), P(16), P(16), P(16), None) == 1


def test_gather_validation(lib):
    P = ctypes.c_void_p
    s = _shape()
    assert lib.gqa_kv_gather(ctypes.byref(s), P(16), P(16), 5, 10, P(16), None) == 1
    assert lib.gqa_kv_gather(ctypes.byref(s), P(16), P(16), 0, -1, P(16), None) == 1
    assert lib.gqa_kv_gather(ctypes.byref(s), P(16), P(16), 0, 0, P(16), None) == 0


def test_version(lib):
    assert b"gfx950" in lib.gqa_version()


def test_copy_blocks_validation(lib):
    P = ctypes.c_void_p
    s = _shape()
    cb = lib.gqa_kv_copy_blocks
    assert cb(ctypes.byref(s), P(16), P(16), None, None, P(16), P(16), -1, None) == 1
    assert cb(ctypes.byref(s), P(16), P(16), P(16), P(16), P(16), P(16), 1, None) == 1
    assert cb(ctypes.byref(s), None, P(16), None, None, P(16), P(16), 3, None) == 1
    assert cb(ctypes.byref(s), P(16), P(16), None, None, None, None, 0, None) == 0
    f = _shape(kv_dtype=1)
    assert cb(ctypes.byref(f), P(16), P(16), None, None, P(16), P(16), 1, None) == 1
    assert cb(ctypes.byref(f), P(16), P(16), P(16), None, P(16), P(16), 1, None) == 1
    # one launch covers pairs x 4 KiB slices of 256 threads each, and the dispatch
    # counts threads in 32 bits: at most 2^24 - 1 work items
    big = _shape(num_kv_heads=256, num_q_heads=256, block_size=32)
    assert cb(ctypes.byref(big), P(16), P(16), None, None, P(16), P(16), 1 << 23, None) == 1
    assert "exceed one launch" in lib.gqa_last_error().decode()
    one = _shape(num_kv_heads=1, num_q_heads=1, head_dim=128, block_size=16)   # 4 KiB blocks
    assert cb(ctypes.byref(one), P(16), P(16), None, None, P(16), P(16), 1 << 24, None) == 1
    assert "exceed one launch" in lib.gqa_last_error().decode()
    if not os.path.exists("/dev/kfd"):
        # no GPU: one item fewer passes validation and fails only at the launch
        assert cb(ctypes.byref(one), P(16), P(16), None, None, P(16), P(16), (1 << 24) - 1,
                  None) == 4


def test_append_fp8_validation(lib):
    P = ctypes.c_void_p
    ap = lib.gqa_kv_append_fp8
    f = _shape(kv_dtype=1)
    args = [P(16)] * 8
    assert ap(ctypes.byref(_shape()), 1, *args, None) == 1            # bf16 pool
    assert ap(ctypes.byref(f), -1, *args, None) == 1
    assert ap(ctypes.byref(f), 70000, *args, None) == 1
    assert ap(ctypes.byref(f), 0, *args, None) == 0                   # nothing to write
    assert ap(ctypes.byref(f), 1, *([P(16)] * 4), None, P(16), P(16), P(16), None) == 1
    assert ap(ctypes.byref(f), 1, P(8), *([P(16)] * 7), None) == 1      # misaligned rows


def test_kivi_dtype_is_accepted(lib):
    P = ctypes.c_void_p
    k = _shape(kv_dtype=2)
    assert lib.gqa_paged_decode_workspace_size(ctypes.byref(k), 1000) > 0
    # validation only (no launch): the fused step needs its new rows and the scales
    call = lambda shape, kn, sc: lib.gqa_paged_decode_append_attention(
        ctypes.byref(shape), P(16), P(kn), P(16), P(16), P(16), P(16), P(sc), P(sc), P(16),
        P(16), 100, 0.1, P(16), None, P(16), 1 << 30, None)
    assert call(k, None, 16) == 1
    assert call(k, 16, None) == 1
    assert lib.gqa_paged_decode_workspace_size(ctypes.byref(_shape(kv_dtype=3)), 1000) == 0


def _split_plan(ctx, target=64, min_tokens=128):
    """The split plan as the kernels apply it: at most `target` splits of a whole
    number of 32-token chunks, none under `min_tokens` tokens unless the context is."""
    if ctx <= 0:
        return 0, 0
    n = min(max(-(-ctx // min_tokens), 1), target)
    st = -(-ctx // n)
    st = -(-st // 32) * 32
    return -(-ctx // st), st


# Lengths at which the last split holds fewer tokens than query positions, so
# that some query row (position ctx - Q + i) sees none of that split's tokens.
SHORT_LAST_SPLIT = {2: (385, 513), 4: (385, 386, 513)}


def test_split_mirror_matches_the_library(lib):
    import gqa_decode_attention_paged_amd as gqa
    for ctx in list(range(0, 3000)) + [8192, 32769]:
        assert _split_plan(ctx)[0] == gqa.num_splits(ctx), ctx


@pytest.mark.parametrize("nq", sorted(SHORT_LAST_SPLIT))
def test_regression_lengths_give_a_row_no_token_of_the_last_split(lib, nq):
    """The GPU regression for rows that see nothing of a split uses these lengths;
    check that they really produce that case under the batch-invariant plan (and
    under any target of at least 5 splits, the plan every small test batch gets)."""
    for ctx in SHORT_LAST_SPLIT[nq]:
        for target in (5, 8, 16, 64):
            n, st = _split_plan(ctx, target)
            last_start = (n - 1) * st
            assert last_start > ctx - nq, (ctx, nq, target)   # query 0 sits at ctx - nq
            assert last_start < ctx


def test_split_tokens_override(lib):
    """The split-length override: set, read back, cleared; bad values refused with
    the old value kept; the host split plan follows it."""
    import gqa_decode_attention_paged_amd as gqa
    assert gqa.split_tokens() == 0
    try:
        for t in (128, 160, 2080, 4128, 1 << 19):
            gqa.set_split_tokens(t)
            assert gqa.split_tokens() == t
            for ctx in list(range(0, 700, 7)) + [2047, 2048, 2049, 8192, 32769, 1 << 22]:
                assert gqa.num_splits(ctx) == _split_plan(ctx, 64, t)[0], (t, ctx)
        gqa.set_split_tokens(2080)
        for bad in (-32, 1, 96, 127, 130, 2081, (1 << 19) + 32, 1 << 20):
            with pytest.raises(gqa.GqaError):
                gqa.set_split_tokens(bad)
            assert gqa.split_tokens() == 2080
        assert gqa.num_splits(32769) == 16                 # 16 splits of 2080 tokens
    finally:
        gqa.set_split_tokens(0)
    assert gqa.split_tokens() == 0 and gqa.num_splits(32769) == _split_plan(32769)[0]


@pytest.mark.parametrize("value,expect", [("512", 512), ("2080", 2080), ("100", 0),
                                          ("130", 0), ("4096x", 0), ("", 0)])
def test_split_tokens_environment(lib, value, expect):
    """GQA_SPLIT_TOKENS is read once at start-up; invalid values leave no override."""
    import subprocess
    import sys
    code = ("import gqa_decode_attention_paged_amd as g; "
            "print(g.split_tokens(), g.num_splits(32769))")
    env = dict(os.environ, GQA_SPLIT_TOKENS=value)
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, check=True,
                         capture_output=True, text=True).stdout.split()
    assert int(out[0]) == expect
    assert int(out[1]) == _split_plan(32769, 64, expect or 128)[0]
