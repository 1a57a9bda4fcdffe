"""The achievable-bandwidth reference kernel (moe_stream_read) reads every byte once: each
workgroup's XOR word equals the XOR of the 16-byte pieces it strides over, computed on the host."""
import numpy as np
import pytest
import torch

from moe_routed_expert_route_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16,grid", [(1, 1), (4096 + 37, 7), (65536 * 9 + 5, 300)])
def test_stream_read_checksums(n16, grid):
    rng = np.random.default_rng(n16 + grid)
    words = rng.integers(0, 2 ** 32, size=4 * n16, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.full((grid + 3,), -1, dtype=torch.int32, device="cuda")
    B.moe_stream_read(buf, out, grid)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    piece = np.bitwise_xor.reduce(words.reshape(n16, 4), axis=1)
    owner = (np.arange(n16) % (grid * 256)) // 256       # workgroup of each 16-byte piece
    want = np.zeros(grid, np.uint32)
    np.bitwise_xor.at(want, owner, piece)
    assert np.array_equal(got[:grid], want)
    assert np.all(got[grid:] == np.uint32(0xFFFFFFFF))   # nothing past the grid's words
