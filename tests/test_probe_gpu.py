"""The measurement probes (include/hpc_probe.h) on the GPU.

The read probe reads every 16-byte word of its buffer exactly once: each
workgroup writes the XOR fold of the words it read (low 16 bits, as a float)
to its sink entry, and that equals the same fold computed here on the host
from the probe's stated split (contiguous chunks of 2048-word blocks, the rest
grid-stride).  The timed form writes the same sink and returns a positive
duration.  The copy is bitwise and writes nothing past its bytes."""
import numpy as np
import pytest
import torch

import load_balanced_paged_step_amd as hd
from decode_harness import announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def _expected_sink(words: np.ndarray, grid: int) -> np.ndarray:
    """Per-workgroup XOR fold of the probe's words; `words` is uint32 [n16, 4]."""
    n16 = words.shape[0]
    block = 256 * 8
    per = n16 // grid // block * block
    x = np.bitwise_xor.reduce(words, axis=1)
    out = np.zeros(grid, dtype=np.float32)
    tail = np.arange(per * grid, n16)
    owner = ((tail - per * grid) // 256) % grid
    for g in range(grid):
        acc = np.uint32(0)
        if per:
            acc ^= np.bitwise_xor.reduce(x[g * per:(g + 1) * per])
        mine = tail[owner == g]
        if mine.size:
            acc ^= np.bitwise_xor.reduce(x[mine])
        out[g] = float(int(acc) & 0xFFFF)
    return out


@pytest.mark.parametrize("n16,grid", [(4 * 2048 * 3 + 1000, 4), (5000, 7), (2048 * 16, 16), (1, 1)])
def test_read_probe_reads_every_word_once(n16, grid):
    announce(f"read probe, {n16} words, {grid} workgroups")
    rng = np.random.default_rng(n16 + grid)
    host = rng.integers(0, 2**32, size=(n16, 4), dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.uint8).reshape(-1).copy()).cuda()
    want = _expected_sink(host, grid)
    sink = torch.full((grid + 8,), -1.0, dtype=torch.float32, device="cuda")
    hd.hpc_probe_read(buf, sink, grid)
    torch.cuda.synchronize()
    got = sink.cpu().numpy()
    assert np.array_equal(got[:grid], want)
    assert np.all(got[grid:] == -1.0)          # nothing written past the grid's entries
    sink.fill_(-1.0)
    ms = hd.hpc_probe_read_timed(buf, sink, grid)
    assert ms > 0.0
    assert np.array_equal(sink.cpu().numpy()[:grid], want)


@pytest.mark.parametrize("nbytes", [16, 4096, 256 * 16 * 8192 + 48])
def test_copy_probe_is_bitwise(nbytes):
    announce(f"copy probe, {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    src = torch.from_numpy(rng.integers(0, 256, size=nbytes, dtype=np.uint8)).cuda()
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    hd.hpc_probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].count_nonzero()) == 0
