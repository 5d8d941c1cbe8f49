"""The streaming-read measurement reference (include/bdiff_probe.h) reads
every byte: its XOR checksum equals the one computed on the host, for sizes
that end inside the unrolled loop, in its tail, and below one wave."""
import numpy as np
import pytest
import torch

from block_diffusion_vlm_amd import bdiff as bd

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words,grid", [(4, 1), (4 * 1000, 3), (4 * 256 * 1024 * 16 + 12, 1024),
                                         ((1 << 26) + 4 * 37, 512)])
def test_stream_read_checksum(n_words, grid):
    assert torch.cuda.is_available() and bd.bd_device_check(0) == bd.BD_OK
    rng = np.random.default_rng(n_words)
    host = rng.integers(0, 2 ** 32, n_words, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    bd.bd_probe_stream_read(src, n_words * 4, grid, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(np.bitwise_xor.reduce(host))
