"""The library's calls captured in a HIP graph and replayed: every replay,
with eager work and synchronisation in between, must equal the eager result
bit for bit (no call enqueues memsets or allocations)."""
import numpy as np
import pytest

import bit_gemv_amd as rf
import oracle
import synth
from _gpu import announce, device, empty, to_dev, torch
from test_gpu_decode import random_blocks

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    dev = device()
    announce("graph replay")
    N, K, M, E = 512, 2048, 3, 4
    w = to_dev(random_blocks(N, K, seed=21, scale_hi=0x30).reshape(-1))
    bank = to_dev(np.stack([random_blocks(N, K, seed=30 + e, scale_hi=0x30)
                            for e in range(E)]).reshape(-1))
    ids = torch.tensor([2, 0, 3], dtype=torch.int32, device=dev)
    a = to_dev(synth.activations(M, K))
    q = empty((M, K), torch.int8)
    d = empty((M, K // 32), torch.float32)
    y1 = empty((M, N), torch.float32)
    y2 = empty((M, N), torch.float32)
    y3 = empty((3, N), torch.float32)
    torch.cuda.synchronize()          # the inputs were written on the default stream
    s = torch.cuda.Stream(device=dev)

    def run():
        rf.rfp2_quantize_acts(a, M, K, q, d, s)
        rf.rfp2_gemv(w, N, K, q, d, M, y1, s)
        rf.rfp2_gemm(w, N, K, q, d, M, y2, s)
        rf.rfp2_moe_gemv(bank, E, N, K, ids, 3, q, d, y3, None, s)

    with torch.cuda.stream(s):
        run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (q, d, y1, y2, y3)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    for _ in range(4):
        for t in (q, d, y1, y2, y3):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip((q, d, y1, y2, y3), ref):
            assert torch.equal(t, r)
    q_ref, d_ref = oracle.quantize_acts(synth.activations(M, K))
    assert np.array_equal(q.cpu().numpy(), q_ref)
