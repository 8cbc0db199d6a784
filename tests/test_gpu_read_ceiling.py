"""The read-ceiling measurement helper really reads every byte it is given:
the XOR of its per-workgroup words equals the XOR of all 32-bit words of the
buffer (exact integer check), for sizes with a ragged last pass and sizes
that need several grid-stride passes."""
import numpy as np
import pytest

import bit_gemv_amd as rf
from _gpu import announce, empty, host, to_dev, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 1_000_000, 16 * 2048 * 256 * 3 + 48])
def test_read_ceiling_reads_every_word(nbytes):
    announce("read_ceiling", nbytes)
    data = np.random.default_rng(nbytes).integers(0, 256, nbytes + 64, dtype=np.uint8)
    buf = to_dev(data)
    out = empty(rf.READ_CEILING_OUTPUTS, torch.int32)
    out.fill_(0)
    rf.rfp2_read_ceiling(buf, nbytes, out)
    grid = min(rf.READ_CEILING_OUTPUTS, -(-(nbytes // 16) // 256))
    got = np.bitwise_xor.reduce(host(out)[:grid].view(np.uint32))
    want = np.bitwise_xor.reduce(data[:nbytes].view(np.uint32))
    assert got == want


def test_read_ceiling_rejects_bad_sizes():
    buf = empty(64, torch.uint8)
    out = empty(rf.READ_CEILING_OUTPUTS, torch.int32)
    with pytest.raises(rf.Rfp2Error):
        rf.rfp2_read_ceiling(buf, 40, out)
