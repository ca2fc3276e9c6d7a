"""The read-stream probe (include/skinny_stream_probe.h) reads every byte once: the
XOR of its sink words equals the XOR of the buffer's 32-bit words (host side)."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,grid,nt", [(0, 4, 1), (16, 1, 0), (4096, 8, 1),
                                            ((1 << 20) + 48, 3, 0), (1 << 20, 7, 1),
                                            (64 << 20, 1024, 1), (64 << 20, 2048, 0)])
def test_probe_reads_every_byte(nbytes, grid, nt):
    from bf16_skinny_gemm_amd import probe

    host = np.random.default_rng([nbytes, grid]).integers(0, 1 << 32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda")
    sink = torch.full((probe.sink_words(grid) + 64,), -1, dtype=torch.int32, device="cuda")
    probe.read(buf, sink, nontemporal=bool(nt), grid_blocks=grid)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(host) if nbytes else np.uint32(0)
    assert np.bitwise_xor.reduce(got[:probe.sink_words(grid)]) == want
    assert np.all(got[probe.sink_words(grid):] == 0xFFFFFFFF)   # nothing written past the sink


@pytest.mark.parametrize("nbytes,loads,threads,nt", [(16, 2, 64, 1), (4096, 4, 256, 0),
                                                     ((1 << 20) + 48, 4, 256, 1),
                                                     ((3 << 20) + 1024, 8, 512, 0),
                                                     (64 << 20, 16, 128, 1), (64 << 20, 4, 1024, 1)])
def test_tile_probe_reads_every_byte(nbytes, loads, threads, nt):
    from bf16_skinny_gemm_amd import probe

    host = np.random.default_rng([nbytes, loads, threads]).integers(0, 1 << 32, nbytes // 4,
                                                                   dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda")
    words = probe.tiles_sink_words(nbytes, loads, threads)
    sink = torch.full((words + 64,), -1, dtype=torch.int32, device="cuda")
    probe.read_tiles(buf, sink, loads=loads, threads=threads, nontemporal=bool(nt))
    probe.empty(64, 256)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert np.bitwise_xor.reduce(got[:words]) == np.bitwise_xor.reduce(host)
    assert np.all(got[words:] == 0xFFFFFFFF)   # nothing written past the sink


def test_probe_rejects_bad_sink():
    from bf16_skinny_gemm_amd import probe

    buf = torch.zeros(1024, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        probe.read(buf, torch.zeros(10, dtype=torch.int32, device="cuda"), grid_blocks=1)
    with pytest.raises(ValueError):
        probe.read(buf, torch.zeros(256, dtype=torch.int64, device="cuda"), grid_blocks=1)
