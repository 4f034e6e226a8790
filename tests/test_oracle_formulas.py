"""Pins the oracle's KV byte formula and intensity to the values printed on the pages."""
import json
import math
import os

import pytest

from oracle import kv_cache_bytes, decode_attention_intensity, decode_attention_flops

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_bytes.json")))


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=lambda c: c["printed"][:40])
def test_kv_bytes_printed_values(case):
    got = kv_cache_bytes(*case["args"])
    if "rel_tol" in case:
        assert math.isclose(got, case["bytes"], rel_tol=case["rel_tol"]), (got, case)
    else:
        assert got == case["bytes"], (got, case)


@pytest.mark.parametrize("case", GOLDEN["intensity"], ids=lambda c: f"{c['q_heads']}/{c['kv_heads']}")
def test_intensity_printed_values(case):
    got = decode_attention_intensity(case["q_heads"], case["kv_heads"], case["bytes_per_elem"])
    assert got == case["flop_per_byte"]


def test_intensity_is_batch_and_length_free():
    # FLOPs and bytes both scale with t and B: the ratio does not move
    for t in (1, 128, 8192):
        f = decode_attention_flops(32, 128, t)
        b = kv_cache_bytes(1, 1, t, 8, 128, 2)
        assert f / b == 4


def test_flops_count_small_case_by_enumeration():
    # 2 FLOPs per multiply-add, QK and PV each do H_q * d * t MACs
    hq, d, t = 3, 5, 7
    macs = 0
    for _h in range(hq):
        for _t in range(t):
            for _d in range(d):
                macs += 2          # one MAC in q.k, one in p.v
    assert decode_attention_flops(hq, d, t) == 2 * macs
