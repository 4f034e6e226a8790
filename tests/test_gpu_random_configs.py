"""Seeded random configurations against the float64 oracle.

Each case draws a combination the other tests cover one axis at a time: head
dim, block size, grouping G, query positions Q, KV dtype (bf16, fp8 with block
scales, fp8 KIVI), sliding window, batch size with ragged (and empty) lengths,
pool placement, split plan (default, batch-invariant flag, split-length
override) and, for bf16, the fused append.  Sizes stay small enough for the
oracle; rows per KV head stay within the library's limits (G*Q <= 32, <= 8 for
KIVI), and lengths are 0 or at least Q (0 < ctx < Q is malformed by definition).
"""
import numpy as np
import pytest
import torch

from tests._dev import to_device, assert_parity
from tests.test_gpu_window import _ref, _run
from workloads import make_case, make_multi_query_case, small_spec

pytestmark = pytest.mark.gpu
CASES = 96


def _draw(i):
    rng = np.random.default_rng([2024, 12, i])
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32]))
    dt = str(rng.choice(["bf16", "bf16", "fp8", "fp8_kivi"]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    cap = 8 if dt == "fp8_kivi" else 32
    nq = min(int(rng.choice([1, 1, 1, 2, 3, 4, 8])), cap // g)
    b = int(rng.integers(1, 7))
    lens = rng.integers(nq, 2600, b)
    lens[rng.random(b) < 0.1] = 0                     # an empty sequence now and then
    window = 0 if rng.random() < 0.6 else int(rng.integers(1, 1500))
    plan = str(rng.choice(["default", "default", "invariant", "override"]))
    tokens = int(rng.choice([128, 256, 512, 1024, 4128]))
    fused = dt == "bf16" and plan != "invariant" and rng.random() < 0.5
    pool = str(rng.choice(["exact", "oversized2x"]))
    return dict(d=d, bs=bs, dt=dt, hkv=hkv, g=g, nq=nq, lens=[int(x) for x in lens], w=window,
                plan=plan, tokens=tokens, fused=fused, pool=pool)


@pytest.mark.parametrize("i", range(CASES))
def test_random_configuration(gpu, i):
    c = _draw(i)
    label = str(c)
    spec = small_spec(num_seqs=len(c["lens"]), num_q_heads=c["hkv"] * c["g"],
                      num_kv_heads=c["hkv"], head_dim=c["d"], block_size=c["bs"],
                      kv_dtype=c["dt"], context=max(c["lens"] + [1]), append=c["fused"],
                      pool=c["pool"], case_id=9000 + i)
    if c["nq"] > 1:
        case = make_multi_query_case(spec, c["nq"], seed=i, context_lens=c["lens"],
                                     append=c["fused"])
    else:
        case = make_case(spec, seed=i, context_lens=c["lens"])
    ref, ref_lse = _ref(case, c["w"])
    dev = to_device(case)
    try:
        if c["plan"] == "override":
            gpu.set_split_tokens(c["tokens"])
        if c["plan"] == "invariant":
            # the flag is a field of the shape; the binding passes it per call
            out, lse = _run_invariant(gpu, case, dev, c["w"])
        else:
            out, lse = _run(gpu, case, dev, c["w"], fused=c["fused"])
    finally:
        gpu.set_split_tokens(0)
    assert_parity(out, lse, ref, ref_lse, label)
    if c["fused"]:
        k = dev["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(k, case["k_pool_full"]), label


def _run_invariant(gqa, case, dev, w):
    max_ctx = int(case["context_lens"].max())
    args = dict(softmax_scale=case["softmax_scale"], sliding_window=w, batch_invariant=True,
                k_scale=dev["k_scale"], v_scale=dev["v_scale"])
    if case.get("num_queries"):
        out, lse = gqa.paged_decode_multi_query(dev["q"], dev["k_cache"], dev["v_cache"],
                                                dev["block_tables"], dev["context_lens"],
                                                max_ctx, **args)
    else:
        out, lse = gqa.paged_decode_attention(dev["q"], dev["k_cache"], dev["v_cache"],
                                              dev["block_tables"], dev["context_lens"],
                                              max_ctx, **args)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _draw_fp8_append(i):
    rng = np.random.default_rng([2024, 13, i])
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    nq = min(int(rng.choice([1, 1, 2, 4])), 32 // g)
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32]))
    lens = [int(x) for x in rng.integers(1, 3000, int(rng.integers(1, 5)))]
    plan = str(rng.choice(["default", "invariant", "override"]))
    tokens = int(rng.choice([128, 512, 2080]))
    window = 0 if rng.random() < 0.7 else int(rng.integers(8, 1000))
    return dict(hkv=hkv, g=g, nq=nq, d=d, bs=bs, lens=lens, plan=plan, tokens=tokens, w=window)


@pytest.mark.parametrize("i", range(24))
def test_random_fused_fp8_append(gpu, i):
    """Fused steps that quantise the new tokens into an fp8 cache (power-of-two
    block scales, grown and re-encoded as blocks fill) and attend, over random
    shapes, query positions, windows and split plans: codes and scales bit-exact
    against the oracle's append after every step, attention within the parity bar."""
    from tests.test_gpu_fp8_append import (_assert_same, _bf16_dev, _f32_dev, _fp8_case_with_room,
                                           _i32_dev, _rows, _u8_dev)
    import oracle
    c = _draw_fp8_append(i)
    label = str(c)
    hq, hkv, d, bs, nq = c["hkv"] * c["g"], c["hkv"], c["d"], c["bs"], c["nq"]
    steps = 3
    state, grown = _fp8_case_with_room(hq, hkv, d, bs, c["lens"], steps * nq, 9800 + i, seed=i)
    dev = [_u8_dev(state[0]), _u8_dev(state[1]), _f32_dev(state[2]), _f32_dev(state[3])]
    td = _i32_dev(grown)
    rng = np.random.default_rng([7, i])
    B = len(c["lens"])
    ctx = np.array(c["lens"], dtype=np.int32)
    kw = dict(k_scale=dev[2], v_scale=dev[3], batch_invariant=c["plan"] == "invariant",
              sliding_window=c["w"])
    try:
        if c["plan"] == "override":
            gpu.set_split_tokens(c["tokens"])
        for step in range(steps):
            mags = 2.0 ** rng.uniform(-2, 3, (B, nq, hkv, 1))
            k_new, v_new = _rows(rng, (B, nq, hkv, d), mags), _rows(rng, (B, nq, hkv, d), mags)
            q = _rows(rng, (B, nq, hq, d), 1.0)
            state = oracle.kv_append_fp8(*state, k_new, v_new, grown, ctx, bs)
            pos = ctx.copy()
            ctx = ctx + nq
            if nq == 1:
                out, lse = gpu.paged_decode_append_attention(
                    _bf16_dev(q[:, 0]), _bf16_dev(k_new[:, 0]), _bf16_dev(v_new[:, 0]),
                    _i32_dev(pos), dev[0], dev[1], td, _i32_dev(ctx), int(ctx.max()), d ** -0.5,
                    **kw)
                ref, ref_lse = oracle.paged_decode_attention(
                    q[:, 0], state[0], state[1], grown, ctx, bs, d ** -0.5, "fp8", state[2],
                    state[3], sliding_window=c["w"])
            else:
                out, lse = gpu.paged_decode_multi_query_append(
                    _bf16_dev(q), _bf16_dev(k_new), _bf16_dev(v_new), dev[0], dev[1], td,
                    _i32_dev(ctx), int(ctx.max()), d ** -0.5, **kw)
                ref, ref_lse = oracle.paged_multi_query_attention(
                    q, state[0], state[1], grown, ctx, bs, d ** -0.5, "fp8", state[2], state[3],
                    sliding_window=c["w"])
            torch.cuda.synchronize()
            _assert_same(tuple(t.cpu().numpy() for t in dev), state, f"{label} step {step}")
            assert_parity(out.cpu().numpy().astype(np.float64),
                          lse.cpu().numpy().astype(np.float64), ref, ref_lse,
                          f"{label} step {step}")
    finally:
        gpu.set_split_tokens(0)


@pytest.mark.parametrize("i", range(16))
def test_random_fused_kivi_append(gpu, i):
    """The same on KIVI pools (keys scaled per channel, values per token; at most 8
    rows per KV head): fused quantising steps over random shapes, query positions,
    windows and split plans, bit-exact codes and scales, attention within the bar."""
    from tests.test_gpu_kivi import _kivi_room, _rows, _same, _t
    import oracle
    rng = np.random.default_rng([2024, 14, i])
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    nq = min(int(rng.choice([1, 1, 2, 4])), 8 // g)
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32]))
    lens = [int(x) for x in rng.integers(1, 2500, int(rng.integers(1, 5)))]
    plan = str(rng.choice(["default", "invariant", "override"]))
    window = 0 if rng.random() < 0.7 else int(rng.integers(8, 1000))
    label = str(dict(hkv=hkv, g=g, nq=nq, d=d, bs=bs, lens=lens, plan=plan, w=window))
    hq = hkv * g
    steps = 3
    state, grown = _kivi_room(hq, hkv, d, bs, lens, steps * nq, 9900 + i)
    dev = [_t(x) for x in state]
    td = _t(grown)
    B = len(lens)
    ctx = np.array(lens, dtype=np.int32)
    kw = dict(k_scale=dev[2], v_scale=dev[3], batch_invariant=plan == "invariant",
              sliding_window=window)
    try:
        if plan == "override":
            gpu.set_split_tokens(256)
        for step in range(steps):
            mags = 2.0 ** rng.uniform(-2, 3, (B, nq, hkv, d))
            k_new, v_new = _rows(rng, (B, nq, hkv, d), mags), _rows(rng, (B, nq, hkv, d), mags)
            q = _rows(rng, (B, nq, hq, d), 1.0)
            state = oracle.kv_append_fp8(*state, k_new, v_new, grown, ctx, bs, layout="kivi")
            start = ctx.copy()
            ctx = ctx + nq
            if nq == 1:
                out, lse = gpu.paged_decode_append_attention(
                    _t(q[:, 0]), _t(k_new[:, 0]), _t(v_new[:, 0]), _t(start), dev[0], dev[1], td,
                    _t(ctx), int(ctx.max()), d ** -0.5, **kw)
                ref, ref_lse = oracle.paged_decode_attention(
                    q[:, 0], state[0], state[1], grown, ctx, bs, d ** -0.5, "fp8_kivi", state[2],
                    state[3], sliding_window=window)
            else:
                out, lse = gpu.paged_decode_multi_query_append(
                    _t(q), _t(k_new), _t(v_new), dev[0], dev[1], td, _t(ctx), int(ctx.max()),
                    d ** -0.5, **kw)
                ref, ref_lse = oracle.paged_multi_query_attention(
                    q, state[0], state[1], grown, ctx, bs, d ** -0.5, "fp8_kivi", state[2],
                    state[3], sliding_window=window)
            torch.cuda.synchronize()
            _same(tuple(x.cpu().numpy() for x in dev), state, f"{label} step {step}")
            assert_parity(out.cpu().numpy().astype(np.float64),
                          lse.cpu().numpy().astype(np.float64), ref, ref_lse,
                          f"{label} step {step}")
    finally:
        gpu.set_split_tokens(0)
