"""GPU parity of the one-token entry points that quantize the activations
inside the product launch (rfp2_quant_gemv, rfp2_quant_moe_gemv).

They must reproduce rfp2_quantize_acts followed by rfp2_gemv / rfp2_moe_gemv
(q and d bit for bit, and q, d must equal the oracle's quantization; y bit for
bit where both launches split K the same way, else within the fp32 bound of
the oracle's product), and the oracle's product within the fp32 bound.
The activations include blocks built to sit on the rounding boundaries of
q = round(a / d): with max |a| = 127 the scale is exactly 1, so values
k + 0.5 are exact ties (halves go away from zero) and their neighbours one
ulp away must fall on either side.
"""
import numpy as np
import pytest

import bit_gemv_amd as rf
import oracle
import synth
from _gpu import announce, assert_within_bound, empty, host, to_dev, torch
from test_gpu_decode import random_blocks
from test_oracle_acts import deep_subnormal_block

pytestmark = pytest.mark.gpu


def boundary_activations(K: int, seed: int) -> np.ndarray:
    """fp32 [K]: normal draws, with blocks of ties, near-ties, zeros, a NaN,
    an infinity and subnormal scales (some of them clamping) scattered over
    it."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(K).astype(np.float32)
    nb = K // 32
    ties = (np.arange(-126, 127, 8) + 0.5).astype(np.float32)
    for b in range(0, nb, 7):
        blk = a[32 * b:32 * b + 32]
        kind = (b // 7) % 6
        if kind == 0:     # exact ties at scale 1
            blk[:] = ties[rng.integers(0, len(ties), 32)]
            blk[0] = 127.0
        elif kind == 1:   # one ulp either side of the ties
            t = ties[rng.integers(0, len(ties), 32)]
            blk[:] = np.where(rng.random(32) < 0.5, np.nextafter(t, np.float32(np.inf)),
                              np.nextafter(t, np.float32(-np.inf)))
            blk[0] = -127.0
        elif kind == 2:   # all zeros: d = 0, q = 0
            blk[:] = 0.0
        elif kind == 3:   # tiny values: the scale is a subnormal number
            if (b // 42) % 2:   # so small that only the clamp keeps q at 127
                blk[:] = deep_subnormal_block()
            else:
                blk[:] = (rng.standard_normal(32) * 1e-37).astype(np.float32)
        elif kind == 4:   # a NaN poisons the block
            blk[rng.integers(0, 32)] = np.nan
        else:             # an infinity too
            blk[rng.integers(0, 32)] = -np.inf
    return a


# K whose one-column split puts 8 groups (6144, 8192) or 16 groups (12288,
# 16384) on each wave: at the sizes here the quantizing launch takes a split
# with at most 4 or 8 groups per wave (more waves), so its y sums in another
# order than rfp2_gemv's.  At K = 10240 and 14336 with fewer rows than 16 per
# compute unit it keeps the one-column split (8 groups, two halves per lane)
# and y is bit-identical; with more rows it takes a 16-row split (below).
OWN_SPLIT_K = (6144, 8192, 12288, 16384)


def same_y(y1, y2, K, ref, absref, what):
    """y of the quantizing call against the two-call y: bit for bit when both
    split K alike, else both within the fp32 bound of the oracle."""
    if K in OWN_SPLIT_K:
        assert_within_bound(y1, ref, absref, what + " (quantizing call)")
        assert_within_bound(y2, ref, absref, what + " (two calls)")
    else:
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), what


def run_both(packed, N, K, a):
    """(y, q, d) of the quantizing call and of the two-call sequence."""
    w = to_dev(packed.reshape(-1))
    a_g = to_dev(a)
    q1, d1, y1 = empty(K, torch.int8), empty(K // 32, torch.float32), empty(N, torch.float32)
    rf.rfp2_quant_gemv(w, N, K, a_g, q1, d1, y1)
    q2, d2, y2 = empty(K, torch.int8), empty(K // 32, torch.float32), empty(N, torch.float32)
    rf.rfp2_quantize_acts(a_g, 1, K, q2, d2)
    rf.rfp2_gemv(w, N, K, q2, d2, 1, y2)
    return (host(y1), host(q1), host(d1)), (host(y2), host(q2), host(d2))


# K/256 = 1, 3, 5, 8, 16, 20, 24, 28, 32 groups (one half per lane), 40, 48,
# 56, 64 (two halves per lane) and 128 (quantization kernel + product);
# ragged row counts
SHAPES = [(300, 256), (257, 768), (123, 1280), (513, 2048), (96, 4096), (1000, 5120),
          (300, 6144), (130, 7168), (129, 8192), (77, 10240), (90, 12288), (50, 14336),
          (64, 16384), (37, 32768)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_quant_gemv_matches_two_calls(N, K):
    announce("quant_gemv", N, K)
    packed = random_blocks(N, K, seed=N + 3 * K, scale_lo=0x00, scale_hi=0x30)
    a = synth.activations(1, K, seed=K)[0]
    (y1, q1, d1), (y2, q2, d2) = run_both(packed, N, K, a)
    q_ref, d_ref = oracle.quantize_acts(a[None, :])
    assert np.array_equal(q1, q_ref[0]) and np.array_equal(q1, q2)
    assert np.array_equal(d1.view(np.uint32), d_ref[0].view(np.uint32))
    assert np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
    ref = oracle.ref_gemv(packed, N, K, q_ref, d_ref)[0]
    absref = oracle.abs_product_sums(packed, N, K, q_ref, d_ref)[0]
    same_y(y1, y2, K, ref, absref, f"quant_gemv {N}x{K}")
    assert_within_bound(y1, ref, absref, f"quant_gemv {N}x{K}")


@pytest.mark.parametrize("N,K", [(4100, 10240), (4096, 14336)])
def test_quant_gemv_sixteen_row_split(N, K):
    # enough rows for a 16-row workgroup on every compute unit: two halves per
    # lane, two groups per lane; q and d bit for bit, y within the fp32 bound
    # of the oracle on sampled rows (and so is the two-call y)
    announce("quant_gemv 16-row split", N, K)
    packed = random_blocks(N, K, seed=N + K, scale_lo=0x00, scale_hi=0x30)
    a = synth.activations(1, K, seed=K + 1)[0]
    (y1, q1, d1), (y2, q2, d2) = run_both(packed, N, K, a)
    q_ref, d_ref = oracle.quantize_acts(a[None, :])
    assert np.array_equal(q1, q_ref[0]) and np.array_equal(q1, q2)
    assert np.array_equal(d1.view(np.uint32), d_ref[0].view(np.uint32))
    assert np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
    rows = np.unique(np.concatenate([np.arange(0, 16), np.arange(N - 20, N),
                                     np.random.default_rng(K).choice(N, 48, replace=False)]))
    ref = oracle.ref_gemv(packed[rows], len(rows), K, q_ref, d_ref)[0]
    absref = oracle.abs_product_sums(packed[rows], len(rows), K, q_ref, d_ref)[0]
    assert_within_bound(y1[rows], ref, absref, f"quant_gemv {N}x{K}")
    assert_within_bound(y2[rows], ref, absref, f"two calls {N}x{K}")


@pytest.mark.parametrize("K", [2048, 5120, 8192, 14336])
def test_quant_gemv_rounding_boundaries_and_special_blocks(K):
    announce("quant_gemv boundaries", K)
    N = 200
    packed = random_blocks(N, K, seed=K + 11, scale_hi=0x28)
    a = boundary_activations(K, seed=K)
    (y1, q1, d1), (y2, q2, d2) = run_both(packed, N, K, a)
    assert np.array_equal(q1, q2)
    assert np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
    assert np.array_equal(np.isnan(y1), np.isnan(y2))
    if K not in OWN_SPLIT_K:
        assert np.array_equal(y1[~np.isnan(y1)].view(np.uint32),
                              y2[~np.isnan(y2)].view(np.uint32))
    # the oracle refuses non-finite activations: compare q, d on the finite blocks
    nb = K // 32
    fin = np.isfinite(a.reshape(nb, 32)).all(axis=1)
    a_fin = np.where(np.repeat(fin, 32), a, 0.0).astype(np.float32)
    q_ref, d_ref = oracle.quantize_acts(a_fin[None, :])
    qb = q1.reshape(nb, 32)
    assert np.array_equal(qb[fin], q_ref[0].reshape(nb, 32)[fin])
    assert np.array_equal(d1[fin].view(np.uint32), d_ref[0][fin].view(np.uint32))
    assert np.isnan(d1[~fin]).all() and (qb[~fin] == 0).all()
    # the ties blocks really hold ties, and they went away from zero
    tie_blk = np.arange(0, nb, 7)[(np.arange(0, nb, 7) // 7) % 6 == 0]
    for b in tie_blk:
        vals = a[32 * b:32 * b + 32]
        assert d1[b] == 1.0
        assert np.array_equal(qb[b], np.clip(np.sign(vals) * np.floor(np.abs(vals) + 0.5),
                                             -127, 127).astype(np.int8))
    assert not fin.all() and np.isnan(y1).all()   # a NaN scale poisons every row


def test_quant_gemv_full_size_matches_two_calls():
    # the 16384x5120 layer with GPU-quantized weights of the workload
    announce("quant_gemv 16384x5120")
    N, K = 16384, 5120
    W = torch.from_numpy(synth.weights(N, K, 0.015, seed=0)).to(torch.device("cuda:0"))
    w = empty(N * K // 32 * 10, torch.uint8)
    rf.rfp2_quantize_weights(W, N, K, w)
    a = synth.activations(1, K)[0]
    (y1, q1, d1), (y2, q2, d2) = run_both(host(w).reshape(N, -1), N, K, a)
    assert np.array_equal(q1, q2) and np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("K", [4096, 8192, 14336])
def test_quant_moe_gemv_matches_two_calls(K):
    announce("quant_moe_gemv", K)
    E, N = 6, 300
    bank = np.stack([random_blocks(N, K, seed=90 + e, scale_hi=0x28) for e in range(E)])
    ids = to_dev(np.array([4, 0, 4, 2, 7, 1], np.int32))     # 7 is out of range
    top_k = 6
    w = to_dev(bank.reshape(-1))
    a = to_dev(synth.activations(1, K, seed=5)[0])
    out = []
    for fused in (True, False):
        q, d = empty(K, torch.int8), empty(K // 32, torch.float32)
        y = empty((top_k, N), torch.float32)
        err = torch.zeros(1, dtype=torch.int32, device=y.device)
        if fused:
            rf.rfp2_quant_moe_gemv(w, E, N, K, ids, top_k, a, q, d, y, err)
        else:
            rf.rfp2_quantize_acts(a, 1, K, q, d)
            rf.rfp2_moe_gemv(w, E, N, K, ids, top_k, q, d, y, err)
        out.append((host(y), host(q), host(d), int(host(err)[0])))
    (y1, q1, d1, e1), (y2, q2, d2, e2) = out
    assert e1 == e2 == 1
    assert np.array_equal(q1, q2) and np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
    assert np.isnan(y1[4]).all() and np.isnan(y2[4]).all()
    ok = [0, 1, 2, 3, 5]
    ids_h = [4, 0, 4, 2, 7, 1]
    ref = oracle.ref_moe_gemv(bank, E, N, K, ids_h, q1[None, :], d1[None, :])
    absref = np.stack([oracle.abs_product_sums(bank[ids_h[j]], N, K, q1[None, :],
                                               d1[None, :])[0] for j in ok])
    same_y(y1[ok], y2[ok], K, ref[ok], absref, f"quant_moe_gemv K={K}")
    assert_within_bound(y1[ok], ref[ok], absref, f"quant_moe_gemv K={K}")


# one and two halves per lane
@pytest.mark.parametrize("N,K", [(4096, 4096), (1024, 14336)])
def test_quant_gemv_graph_replays_match_eager(N, K):
    announce("quant_gemv graph", N, K)
    packed = random_blocks(N, K, seed=123, scale_hi=0x28)
    w = to_dev(packed.reshape(-1))
    a = to_dev(synth.activations(1, K, seed=9)[0])
    q, d, y = empty(K, torch.int8), empty(K // 32, torch.float32), empty(N, torch.float32)
    torch.cuda.synchronize()          # the inputs were written on the default stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        rf.rfp2_quant_gemv(w, N, K, a, q, d, y, s)
        torch.cuda.synchronize()
        y_eager = y.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            rf.rfp2_quant_gemv(w, N, K, a, q, d, y, s)
        for _ in range(3):
            y.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, y_eager)


@pytest.mark.parametrize("N", [83886, 83887])
def test_quant_gemv_either_side_of_the_two_launch_size(N):
    # 128 MiB of weights is the largest one-token call done as one quantizing
    # launch (83886 rows of K = 5120, 1600 bytes each, are just under it,
    # 83887 just over): on
    # both sides q, d and y equal the two-call sequence bit for bit, and q, d
    # the oracle's quantization
    K = 5120
    announce("quant_gemv size switch", N, K)
    packed = random_blocks(N, K, seed=N, scale_hi=0x28)
    a = synth.activations(1, K, seed=9)[0]
    (y1, q1, d1), (y2, q2, d2) = run_both(packed, N, K, a)
    q, d = oracle.quantize_acts(a[None, :])
    assert np.array_equal(q1, q[0]) and np.array_equal(d1.view(np.uint32), d[0].view(np.uint32))
    assert np.array_equal(q1, q2) and np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_quant_moe_gemv_above_the_two_launch_size():
    # 8 routed experts of 16384 x 1024 are 8 * 16384 * 320 = 40 MiB; 7 of
    # 65536 x 1024 = 140 MiB goes as two launches: both match the two calls
    announce("quant_moe_gemv size switch")
    K = 1024
    a = to_dev(synth.activations(1, K, seed=6)[0])
    for E, N, ids in ((8, 16384, [3, 1, 7, 0, 2, 6, 5, 4]), (7, 65536, [6, 0, 3, 1, 5, 2, 4])):
        top_k = len(ids)
        bank = np.stack([random_blocks(N, K, seed=e, scale_hi=0x28) for e in range(E)])
        w = to_dev(bank.reshape(-1))
        ids_g = to_dev(np.array(ids, np.int32))
        out = []
        for fused in (True, False):
            q, d = empty(K, torch.int8), empty(K // 32, torch.float32)
            y = empty((top_k, N), torch.float32)
            if fused:
                rf.rfp2_quant_moe_gemv(w, E, N, K, ids_g, top_k, a, q, d, y)
            else:
                rf.rfp2_quantize_acts(a, 1, K, q, d)
                rf.rfp2_moe_gemv(w, E, N, K, ids_g, top_k, q, d, y)
            out.append((host(y), host(q), host(d)))
        (y1, q1, d1), (y2, q2, d2) = out
        assert np.array_equal(q1, q2) and np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), (E, N)
        del w
