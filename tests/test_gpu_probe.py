"""GPU check of the read probe: every load pattern reads each 32-bit word of each
listed tile exactly once (the probe folds what it reads into per-wave XOR
checksums, and their XOR must equal the XOR of the listed tiles' words)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

# (pattern, tile bytes) pairs the probe accepts
CASES = [(0, 1024), (0, 2048), (0, 4096), (0, 8192), (0, 16384), (1, 4096), (1, 8192),
         (2, 2048), (2, 4096), (3, 2048), (3, 4096), (4, 4096), (4, 8192)]


@pytest.mark.parametrize("non_temporal", [1, 0])
@pytest.mark.parametrize("pattern,tile", CASES)
def test_probe_reads_every_word_once(gpu, pattern, tile, non_temporal):
    rng = np.random.default_rng([pattern, tile, non_temporal])
    pool_tiles = 64
    words = rng.integers(0, 2**32, size=pool_tiles * tile // 4, dtype=np.uint64).astype(np.uint32)
    ids = rng.integers(0, pool_tiles, size=41).astype(np.int32)
    ids[7] = pool_tiles + 5                  # out of range: the probe reads tile 0
    dev = torch.device("cuda:0")
    pool = torch.from_numpy(words.view(np.int32)).to(dev)
    tids = torch.from_numpy(ids).to(dev)
    workgroups = 3
    sink = torch.full((workgroups * 8,), -1, dtype=torch.int32, device=dev)
    gpu.probe_read(pool.data_ptr(), pool_tiles, tids, len(ids), tile, non_temporal, workgroups,
                   sink, pattern=pattern)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    per_tile = words.reshape(pool_tiles, -1)
    want = np.uint32(0)
    for t in np.where((ids >= 0) & (ids < pool_tiles), ids, 0):
        want ^= np.bitwise_xor.reduce(per_tile[t])
    assert got == want


def test_probe_stream_without_table(gpu):
    """No table: tiles 0 .. num_tiles-1 in order."""
    rng = np.random.default_rng(5)
    words = rng.integers(0, 2**32, size=20 * 4096 // 4, dtype=np.uint64).astype(np.uint32)
    pool = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    sink = torch.zeros(2 * 8, dtype=torch.int32, device="cuda:0")
    gpu.probe_read(pool.data_ptr(), 20, None, 13, 4096, 1, 2, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words[:13 * 1024])
