"""The entry points inside a captured HIP graph, as the benchmark runs them: every
replay (with eager work and synchronisation between replays) gives the same bits
as the eager call, for the fused steps on bf16, fp8 and KIVI pools, plain and
multi-position attention, and the block copy.  The split-merge counters reset
themselves, so a graph can be replayed without clearing the workspace."""
import numpy as np
import pytest
import torch

from tests._dev import to_device
from workloads import bf16_round, make_case, make_multi_query_case, small_spec

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    """Bit patterns (pools hold NaN poison, which compares unequal as a value)."""
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t


def _replays_match(fn, outputs, state=(), replays=4):
    """Run fn eagerly twice (the second from the state the first leaves, as every
    replay sees it), capture it, and check each replay against the second eager
    run: `outputs` are poisoned before every replay, `state` (pools, scales) is
    left as it is and must also come out the same."""
    fn()
    fn()
    torch.cuda.synchronize()
    want = [t.clone() for t in list(outputs) + list(state)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        fn()
    torch.cuda.synchronize()
    scratch = torch.ones(1 << 20, device=DEV)
    for r in range(replays):
        for o in outputs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        scratch.mul_(1.0001).add_(r)            # eager work between replays
        torch.cuda.synchronize()
        for i, (t, w) in enumerate(zip(list(outputs) + list(state), want)):
            assert torch.equal(_bits(t), _bits(w)), f"replay {r}, tensor {i}"


def _bf16(rng, shape, scale=1.0):
    a = bf16_round((rng.standard_normal(shape) * scale).astype(np.float32))
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("lens", [[8192], [700, 3000, 64, 9]])
def test_fused_bf16_step_replays(gpu, lens):
    spec = small_spec(num_seqs=len(lens), num_q_heads=32, num_kv_heads=8, head_dim=128,
                      block_size=16, context=max(lens), append=True, case_id=9700 + len(lens))
    case = make_case(spec, seed=1, context_lens=lens)
    d = to_device(case)
    mx = max(lens)
    shape = gpu.make_shape(len(lens), 32, d["k_cache"], d["block_tables"])
    ws = torch.zeros(gpu.workspace_size(shape, mx), dtype=torch.uint8, device=DEV)
    out = torch.empty((len(lens), 32, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((len(lens), 32), dtype=torch.float32, device=DEV)

    def step():
        gpu.paged_decode_append_attention(d["q"], d["k_new"], d["v_new"], d["positions"],
                                          d["k_cache"], d["v_cache"], d["block_tables"],
                                          d["context_lens"], mx, case["softmax_scale"], out=out,
                                          out_lse=lse, workspace=ws)
    _replays_match(step, [out, lse], [d["k_cache"], d["v_cache"]])
    assert int(ws[:4].view(torch.int32).item()) == 0          # counters back to zero


@pytest.mark.parametrize("kivi", [False, True])
def test_fused_fp8_step_replays(gpu, kivi):
    lens = [900, 33, 4096]
    spec = small_spec(num_seqs=3, num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                      kv_dtype="fp8_kivi" if kivi else "fp8", context=4096, case_id=9710 + kivi)
    case = make_case(spec, seed=2, context_lens=lens)
    d = to_device(case)
    rng = np.random.default_rng(3)
    k_new, v_new = _bf16(rng, (3, 4, 128), 2.0), _bf16(rng, (3, 4, 128), 2.0)
    # the new token goes to position ctx - 1 (the pool's last valid slot is overwritten)
    pos = torch.tensor([n - 1 for n in lens], dtype=torch.int32, device=DEV)
    shape = gpu.make_shape(3, 16, d["k_cache"], d["block_tables"], k_scale=d["k_scale"])
    ws = torch.zeros(gpu.workspace_size(shape, 4096), dtype=torch.uint8, device=DEV)
    out = torch.empty((3, 16, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((3, 16), dtype=torch.float32, device=DEV)

    def step():
        gpu.paged_decode_append_attention(d["q"], k_new, v_new, pos, d["k_cache"], d["v_cache"],
                                          d["block_tables"], d["context_lens"], 4096,
                                          case["softmax_scale"], out=out, out_lse=lse,
                                          workspace=ws, k_scale=d["k_scale"], v_scale=d["v_scale"])
    _replays_match(step, [out, lse], [d["k_scale"], d["v_scale"], d["k_cache"], d["v_cache"]])


def test_fused_verify_step_replays(gpu):
    lens = [2000, 10, 700]
    spec = small_spec(num_seqs=3, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=2000, case_id=9720)
    case = make_multi_query_case(spec, 4, seed=4, context_lens=lens)
    d = to_device(case)
    shape = gpu.make_shape(3, 32, d["k_cache"], d["block_tables"])
    ws = torch.zeros(gpu.multi_query_workspace_size(shape, 4, 2000), dtype=torch.uint8, device=DEV)
    out = torch.empty((3, 4, 32, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((3, 4, 32), dtype=torch.float32, device=DEV)

    def step():
        gpu.paged_decode_multi_query_append(d["q"], d["k_new"], d["v_new"], d["k_cache"],
                                            d["v_cache"], d["block_tables"], d["context_lens"],
                                            2000, case["softmax_scale"], out=out, out_lse=lse,
                                            workspace=ws)
    _replays_match(step, [out, lse], [d["k_cache"], d["v_cache"]])


def test_kivi_attention_and_block_copy_replay(gpu):
    spec = small_spec(num_seqs=2, num_q_heads=8, num_kv_heads=8, head_dim=128, block_size=32,
                      kv_dtype="fp8_kivi", context=3000, case_id=9730)
    case = make_case(spec, seed=5, context_lens=[3000, 129])
    d = to_device(case)
    nb = d["k_cache"].shape[0]
    shape = gpu.make_shape(2, 8, d["k_cache"], d["block_tables"], k_scale=d["k_scale"])
    ws = torch.zeros(gpu.workspace_size(shape, 3000), dtype=torch.uint8, device=DEV)
    out = torch.empty((2, 8, 128), dtype=torch.float32, device=DEV)
    used = set(case["block_tables"][case["block_tables"] >= 0].tolist())
    free = [i for i in range(nb) if i not in used][:3]
    src = torch.tensor(sorted(used)[:3], dtype=torch.int32, device=DEV)
    dst = torch.tensor(free, dtype=torch.int32, device=DEV)

    def step():
        gpu.kv_copy_blocks(d["k_cache"], d["v_cache"], src, dst, d["k_scale"], d["v_scale"])
        gpu.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                   d["context_lens"], 3000, case["softmax_scale"], d["k_scale"],
                                   d["v_scale"], out=out, workspace=ws, return_lse=False)
    _replays_match(step, [out], [d["k_cache"], d["k_scale"], d["v_scale"]])


def test_noalloc_attention_replays(gpu):
    """The entry point with the static workspace is two kernels (a fill of the
    scratch's counters, then the decode kernel); both go into the graph, and every
    replay gives the eager bits."""
    spec = small_spec(num_seqs=3, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context=("uniform", 200, 3000), case_id=7500)
    case = make_case(spec, seed=2)
    dev = to_device(case)
    hint = int(case["context_lens"].max())
    out = torch.empty((3, 32, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((3, 32), dtype=torch.float32, device=DEV)

    def fn():
        gpu.paged_decode_attention_noalloc(dev["q"], dev["k_cache"], dev["v_cache"],
                                           dev["block_tables"], dev["context_lens"], hint,
                                           case["softmax_scale"], out=out, out_lse=lse)

    _replays_match(fn, [out, lse])
