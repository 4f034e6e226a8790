"""Helpers for GPU tests: move a seeded workload to the device, run the HIP path
through the C ABI, and compare with the float64 oracle."""
import functools

import numpy as np

import oracle
from workloads import make_case, SPECS

# Acceptance bar for attention outputs against the float64 oracle.
MAX_ABS = 1e-2
REL_L2 = 2e-3
LSE_ABS = 1e-3        # natural-log lse; fp32 sums over <= 33K terms


def to_device(case, device="cuda:0"):
    import torch

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    def pool(a):
        if a.dtype == np.uint8:
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return bf16(a)

    d = dict(
        q=bf16(case["q"]),
        k_cache=pool(case["k_pool"]), v_cache=pool(case["v_pool"]),
        block_tables=torch.from_numpy(case["block_tables"]).to(device),
        context_lens=torch.from_numpy(case["context_lens"]).to(device),
        positions=torch.from_numpy(case["positions"]).to(device),
        k_scale=None, v_scale=None, k_new=None, v_new=None,
    )
    if case["k_scale"] is not None:
        d["k_scale"] = torch.from_numpy(case["k_scale"]).to(device)
        d["v_scale"] = torch.from_numpy(case["v_scale"]).to(device)
    if case["k_new"] is not None:
        d["k_new"] = bf16(case["k_new"])
        d["v_new"] = bf16(case["v_new"])
    return d


def run_step(gqa, dev, case, max_context_len=None, batch_invariant=False):
    """One decode step through the C ABI: append (if the workload has one), then attention."""
    import torch
    if case["k_new"] is not None:
        gqa.kv_append(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                      dev["block_tables"], dev["positions"])
    if max_context_len is None:
        max_context_len = int(case["context_lens"].max()) if case["context_lens"].size else 0
    out, lse = gqa.paged_decode_attention(dev["q"], dev["k_cache"], dev["v_cache"],
                                          dev["block_tables"], dev["context_lens"],
                                          max_context_len, case["softmax_scale"],
                                          dev["k_scale"], dev["v_scale"],
                                          batch_invariant=batch_invariant)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def run_fused_step(gqa, dev, case, max_context_len=None, workspace=None):
    """One decode step through the fused entry point (append + attention, one kernel)."""
    import torch
    if max_context_len is None:
        max_context_len = int(case["context_lens"].max()) if case["context_lens"].size else 0
    out, lse = gqa.paged_decode_append_attention(dev["q"], dev["k_new"], dev["v_new"],
                                                 dev["positions"], dev["k_cache"], dev["v_cache"],
                                                 dev["block_tables"], dev["context_lens"],
                                                 max_context_len, case["softmax_scale"],
                                                 workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def run_oracle(case):
    s = case["spec"]
    return oracle.paged_decode_attention(case["q"], case["k_pool_full"], case["v_pool_full"],
                                         case["block_tables"], case["context_lens"],
                                         s.block_size, case["softmax_scale"], s.kv_dtype,
                                         case["k_scale"], case["v_scale"])


def parity(out, ref):
    """(max abs error, relative L2 error) of out against ref."""
    err = out - ref
    max_abs = float(np.max(np.abs(err))) if err.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(err) / den) if den > 0 else float(np.linalg.norm(err))
    return max_abs, rel


def assert_parity(out, lse, ref, ref_lse, label=""):
    assert np.all(np.isfinite(out)), f"{label}: non-finite output"
    max_abs, rel = parity(out, ref)
    assert max_abs <= MAX_ABS and rel <= REL_L2, f"{label}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{label}: lse finiteness differs"
    if fin.any():
        lerr = float(np.max(np.abs(lse[fin] - ref_lse[fin])))
        assert lerr <= LSE_ABS, f"{label}: lse err {lerr:.3e}"
    return max_abs, rel


@functools.lru_cache(maxsize=None)
def named_case(name, seed=0):
    return make_case(SPECS[name], seed=seed)


@functools.lru_cache(maxsize=None)
def named_reference(name, seed=0):
    return run_oracle(named_case(name, seed))
