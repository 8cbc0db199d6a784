"""The read-ceiling measurement helper really reads every piece it is given:
in a zero buffer, pieces planted with one value V are each the only non-zero
piece their thread visits, so exactly the threads that own them (thread
p mod T for piece p, T threads in the grid-stride grid) find XOR == magic and
write; every other entry stays untouched.  The planted pieces include the
first and the last piece, a piece in the ragged last pass, and one per
grid-stride pass."""
import numpy as np
import pytest

import bit_gemv_amd as rf
from _gpu import announce, empty, host, to_dev, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 1_000_000, 16 * 2048 * 256 * 3 + 48])
def test_read_ceiling_reads_every_planted_piece(nbytes):
    announce("read_ceiling", nbytes)
    pieces = nbytes // 16
    T = rf.read_ceiling_threads(nbytes)
    rng = np.random.default_rng(nbytes)
    passes = -(-pieces // T)
    # one piece per grid-stride pass, each owned by a distinct thread, plus the
    # first and the last piece
    owners = {}
    for p in [0, pieces - 1] + [int(rng.integers(k * T, min((k + 1) * T, pieces)))
                                for k in range(passes)]:
        owners.setdefault(p % T, p)          # one planted piece per thread
    planted = sorted(owners.values())
    assert 0 in planted and pieces - 1 in planted
    data = np.zeros(nbytes + 64, dtype=np.uint8)
    V = np.array([0x11223344, 0x0A0B0C0D, 0x55667788, 0x01020304], dtype=np.uint32)
    magic = int(np.bitwise_xor.reduce(V))
    for p in planted:
        data[16 * p:16 * p + 16] = V.view(np.uint8)
    out = empty(rf.READ_CEILING_OUTPUTS, torch.int32)
    out.fill_(-1)
    rf.rfp2_read_ceiling(to_dev(data), nbytes, out, magic=magic)
    got = host(out)[:T].view(np.uint32)
    written = np.flatnonzero(got != 0xFFFFFFFF)
    assert sorted(written.tolist()) == sorted(p % T for p in planted)
    assert (got[written] == magic).all()
    # a magic nothing matches: no thread writes
    out.fill_(-1)
    rf.rfp2_read_ceiling(to_dev(data), nbytes, out, magic=magic ^ 1)
    assert (host(out)[:T].view(np.uint32) == 0xFFFFFFFF).all()


def test_read_ceiling_rejects_bad_sizes():
    buf = empty(64, torch.uint8)
    out = empty(rf.READ_CEILING_OUTPUTS, torch.int32)
    with pytest.raises(rf.Rfp2Error):
        rf.rfp2_read_ceiling(buf, 40, out)
