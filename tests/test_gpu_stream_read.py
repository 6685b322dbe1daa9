"""The streaming-read measurement kernel reads every 16-byte chunk exactly
once: the xor of its per-thread checksums equals the xor of the data, for
sizes that leave a ragged tail, every unroll and an odd grid (a chunk read
twice or skipped changes the xor)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from bit_moe_expert_02_amd import _lib as L          # noqa: E402


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (3 << 20) + 16 * 37 + 5])
@pytest.mark.parametrize("grid,unroll", [(1, 1), (37, 2), (64, 4), (129, 8)])
def test_stream_read_reads_every_chunk_once(nbytes, grid, unroll):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    rng = np.random.default_rng(nbytes * 131 + grid)
    host = rng.integers(0, 2**32, size=(nbytes + 15) // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32).copy()).cuda()
    sink = torch.zeros(grid * 256, dtype=torch.int32, device="cuda")
    L.moe_stream_read(buf, nbytes, sink, grid, unroll)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    whole = (nbytes // 16) * 4                         # 32-bit words in whole chunks
    want = np.bitwise_xor.reduce(host[:whole]) if whole else np.uint32(0)
    assert got == want


def test_stream_read_rejects_bad_arguments():
    buf = torch.zeros(64, dtype=torch.int32, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    for grid, unroll in ((0, 1), (1, 3), (70000, 1)):
        with pytest.raises(L.MoeError):
            L.moe_stream_read(buf, 256, sink, grid, unroll)
