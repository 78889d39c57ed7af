"""The read calibration kernel behind bench.py's ceiling figures
(q4k_read_calibrate): every 16-byte word of the buffer is read exactly once.

Each workgroup's checksum is the xor of the words its lanes read; the whole
grid sweeps the buffer in address order, one word per lane and pass, so word
i belongs to workgroup (i mod (grid x 512)) / 512.  The expected checksums
are computed here with numpy from that assignment.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_quantized_decode_q4_amd import q4k  # noqa: E402

pytestmark = pytest.mark.gpu

LANES = 512     # lanes per workgroup of the calibration kernel


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4k.load_library()
    yield


@pytest.mark.parametrize("nbytes", [16, 16 * 1000, 16 * (1024 * 512 * 2 + 12345)])
def test_read_calibrate_covers_every_word_once(nbytes):
    grid = q4k.q4k_read_calibrate_blocks()
    rng = np.random.default_rng(77 + nbytes)
    words = rng.integers(0, 1 << 32, size=(nbytes // 16, 4), dtype=np.uint64).astype(np.uint32)
    folded = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
    owner = (np.arange(words.shape[0]) % (grid * LANES)) // LANES
    acc = np.zeros(grid, dtype=np.uint32)
    np.bitwise_xor.at(acc, owner, folded)
    expect = (acc & 0xFFFF).astype(np.float32)
    print("read calibration: %d bytes, %d workgroups" % (nbytes, grid), flush=True)
    buf = torch.from_numpy(words.view(np.uint8).reshape(-1)).cuda()
    out = torch.full((grid,), -1.0, dtype=torch.float32, device="cuda")
    q4k.q4k_read_calibrate(buf, nbytes, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), expect)
