"""The read-stream probe (measurement support): every launch shape reads every byte once.
Each lane folds (XOR) the 16-byte words it loaded, so the fold of all lanes' outputs must equal
the XOR of the whole buffer's 32-bit words, computed here on the CPU."""
import numpy as np
import pytest
import torch

from weight_only_quant_amd import probe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [1024, 5 * 1024, 1 << 20, (1 << 20) + 7 * 1024])
@pytest.mark.parametrize("shape", [(1, 0, 1, 4, 0), (3, 0, 2, 1, 0), (16, 0, 4, 8, 0), (64, 0, 16, 1, 40960),
                                   (7, 0, 8, 2, 0), (0, 5, 4, 8, 0), (0, 2048, 4, 8, 0), (0, 3, 16, 1, 20480),
                                   (1, -1, 1, 1, 0), (3, -1, 2, 4, 0), (5, -1, 16, 2, 0), (240, -1, 8, 4, 65536)])
def test_probe_reads_every_byte_once(nbytes, shape):
    print(f"probe nbytes={nbytes} shape={shape}", flush=True)
    rng = np.random.default_rng(nbytes + 131 * shape[0] + 7 * shape[1] + shape[2])
    host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.full((probe.read_out_words(nbytes, shape),), -1, dtype=torch.int32, device="cuda")
    probe.read(buf, nbytes, shape, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host)
    assert got == want


def test_best_read_reports_every_shape():
    shapes = ((8, 0, 4, 4, 0), (0, 512, 8, 8, 0))
    best, res = probe.best_read_gbs(64 << 20, reps=3, shapes=shapes)
    assert set(res) == {probe.shape_name(s) for s in shapes} and best == max(res.values()) and best > 0
    best, res = probe.best_read_gbs(64 << 20, window=20 << 20, reps=5, shapes=shapes[:1])
    assert len(res) == 1 and best > 0
