"""GPU parity of rfp2_gemv (1..8 activation columns) against the fp64 oracle.

Bound per output (fp32 result): |y_gpu - y_ref| <= 1e-5 * sum_k |w_k a_k| + 1e-6.
"""
import numpy as np
import pytest

import bit_gemv_amd as rf
import oracle
import synth
from _gpu import announce, assert_within_bound, empty, host, sample_rows, to_dev, torch
from test_gpu_decode import random_blocks

pytestmark = pytest.mark.gpu


def run_gemv(packed, N, K, q, d):
    M = q.shape[0]
    y = empty((M, N), torch.float32)
    rf.rfp2_gemv(to_dev(packed.reshape(-1)), N, K, to_dev(q), to_dev(d), M, y)
    return host(y)


def check(packed, N, K, q, d, what):
    y = run_gemv(packed, N, K, q, d)
    return assert_within_bound(y, oracle.ref_gemv(packed, N, K, q, d),
                               oracle.abs_product_sums(packed, N, K, q, d), what)


def test_gemv_512x2048_full_oracle_weights():
    # small GEMV: every output, oracle-quantized weights and activations
    announce("gemv 512x2048 M=1")
    W = synth.weights(512, 2048, 0.02, seed=0)
    packed = oracle.quantize_weights(W)
    q, d = oracle.quantize_acts(synth.activations(1, 2048))
    check(packed, 512, 2048, q, d, "gemv 512x2048")


# (N, K, M): ragged row counts, every lanes-per-row geometry (K/256 = 1, 3, 5,
# 8, 10, 16, 20, 28, 56, 64, 128 groups), 1..8 columns and column chunking (the
# largest K with eight columns runs as eight one-column launches).  Two to
# four columns run the matrix-core form at 1, 2, 4, 8 and 16 lanes per row
# (257x768, 200x5120, 130x4096, 70x14336, 33x16384) and fall back to the dot
# form at 32 (45x32768 with two columns).
SHAPES = [
    (1, 256, 1), (300, 256, 1), (257, 768, 3), (1000, 1280, 2), (123, 2560, 5),
    (96, 4096, 8), (200, 5120, 4), (130, 7168, 7), (64, 16384, 1), (37, 32768, 1),
    (70, 16384, 8), (513, 2048, 6), (45, 32768, 8), (50, 14336, 1),
    (130, 4096, 2), (70, 14336, 4), (33, 16384, 3), (45, 32768, 2), (5, 256, 4),
]


@pytest.mark.parametrize("N,K,M", SHAPES)
def test_gemv_shapes(N, K, M):
    announce("gemv", N, K, M)
    packed = random_blocks(N, K, seed=N * 7 + K, scale_lo=0x00, scale_hi=0x30)
    q, d = oracle.quantize_acts(synth.activations(M, K, seed=M + K))
    check(packed, N, K, q, d, f"gemv {N}x{K} M={M}")


def test_gemv_columns_are_independent():
    # a column's result does not depend on the other columns of the call: a
    # 4-column call and four 1-column calls agree to within twice the fp32
    # bound (the split of K over lanes and waves, and so the summation order,
    # is chosen per column count); a 4-column call repeated is bit-identical
    announce("gemv column independence")
    N, K = 200, 5120
    packed = random_blocks(N, K, seed=1, scale_hi=0x20)
    q, d = oracle.quantize_acts(synth.activations(4, K))
    y4 = run_gemv(packed, N, K, q, d)
    assert np.array_equal(y4, run_gemv(packed, N, K, q, d))
    absum = oracle.abs_product_sums(packed, N, K, q, d)
    for m in range(4):
        y1 = run_gemv(packed, N, K, q[m:m + 1], d[m:m + 1])
        assert_within_bound(y4[m], y1[0].astype(np.float64), 2 * absum[m],
                            f"column {m} alone vs in a batch of 4")


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_gemv_illegal_scale_gives_nan_row(M):
    # one column: the dot4 form; two to four: the matrix-core form
    announce("gemv illegal scale byte", M)
    N, K = 64, 1024
    packed = random_blocks(N, K, seed=2, scale_hi=0x20)
    packed[5, 10 * 7 + 9] = 0x7F           # e1 of block 7 of row 5
    packed[9, 10 * 30 + 8] = 0x91          # e0 of block 30 of row 9
    q, d = oracle.quantize_acts(synth.activations(M, K))
    y = run_gemv(packed, N, K, q, d)
    assert np.isnan(y[:, 5]).all() and np.isnan(y[:, 9]).all()
    ok = np.ones(N, bool)
    ok[[5, 9]] = False
    good = packed[ok]
    assert_within_bound(y[:, ok], oracle.ref_gemv(good, ok.sum(), K, q, d),
                        oracle.abs_product_sums(good, ok.sum(), K, q, d), "clean rows")


@pytest.mark.parametrize("name", ["gemv_4096x4096", "gemv_16384x5120", "gemv_16384x5120_m4"])
def test_gemv_full_size_sampled_rows(name):
    # full-size workload, same path as the bench: GPU-quantized weights and
    # activations; the oracle quantizes the sampled rows itself
    cfg = synth.WORKLOADS[name]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    announce("gemv full", name)
    W = synth.weights(N, K, cfg["sigma"], seed=cfg["wseed"])
    a = synth.activations(M, K)
    w_g = empty((N * K // 32 * 10,), torch.uint8)
    rf.rfp2_quantize_weights(to_dev(W), N, K, w_g)
    q_g = empty((M, K), torch.int8)
    d_g = empty((M, K // 32), torch.float32)
    rf.rfp2_quantize_acts(to_dev(a), M, K, q_g, d_g)
    y_g = empty((M, N), torch.float32)
    rf.rfp2_gemv(w_g, N, K, q_g, d_g, M, y_g)
    y = host(y_g)
    rows = sample_rows(N, 48, seed=12)
    packed_rows = oracle.quantize_weights(W[rows])
    got_rows = host(w_g).reshape(N, -1)[rows]
    assert np.array_equal(got_rows, packed_rows)
    q, d = oracle.quantize_acts(a)
    assert np.array_equal(host(q_g), q) and np.array_equal(host(d_g), d)
    assert_within_bound(y[:, rows], oracle.ref_gemv(packed_rows, len(rows), K, q, d),
                        oracle.abs_product_sums(packed_rows, len(rows), K, q, d), name)
    assert np.isfinite(y).all()


# Large matrices whose usual split of K would need two rounds of workgroups,
# so the launch takes another: one lane per row over 64-row workgroups
# (32768 x 4096, 18432 x 7168: seven groups per lane) or the one-round split
# nearest two groups per lane (4096 x 14336: 16 lanes per row, seven waves;
# 14336 x 4096 with two and three columns).
@pytest.mark.parametrize("N,K,M", [(32768, 4096, 4), (18432, 7168, 4), (4096, 14336, 4),
                                   (14336, 4096, 3), (14336, 4096, 2)])
def test_gemv_one_round_splits(N, K, M):
    announce("gemv one-round split", N, K, M)
    packed = random_blocks(N, K, seed=N + M, scale_lo=0x00, scale_hi=0x30)
    q, d = oracle.quantize_acts(synth.activations(M, K, seed=60 + M))
    y = run_gemv(packed, N, K, q, d)
    rows = sample_rows(N, 48, seed=N)
    assert_within_bound(y[:, rows], oracle.ref_gemv(packed[rows], len(rows), K, q, d),
                        oracle.abs_product_sums(packed[rows], len(rows), K, q, d),
                        f"gemv {N}x{K} M={M}")
    assert np.isfinite(y).all()


@pytest.mark.parametrize("M", [6, 7, 8])
def test_gemv_many_columns_large_matrix(M):
    # 16384 x 5120 with 6 and 7 columns runs as one launch whose workgroups
    # take more than 64 KiB of LDS each; 8 columns as launches of 5 and 3:
    # sampled rows of every column against the oracle
    N, K = 16384, 5120
    announce("gemv many columns", N, K, M)
    packed = random_blocks(N, K, seed=M, scale_lo=0x00, scale_hi=0x30)
    q, d = oracle.quantize_acts(synth.activations(M, K, seed=40 + M))
    y = run_gemv(packed, N, K, q, d)
    rows = sample_rows(N, 48, seed=M)
    assert_within_bound(y[:, rows], oracle.ref_gemv(packed[rows], len(rows), K, q, d),
                        oracle.abs_product_sums(packed[rows], len(rows), K, q, d),
                        f"gemv {N}x{K} M={M}")
    assert np.isfinite(y).all()
