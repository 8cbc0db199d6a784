"""GPU parity of rfp2_gemm (i8 matrix cores) against the fp64 oracle."""
import numpy as np
import pytest

import bit_gemv_amd as rf
import oracle
import synth
from _gpu import announce, assert_within_bound, empty, host, sample_rows, to_dev, torch
from test_gpu_decode import random_blocks

pytestmark = pytest.mark.gpu


GEMMS = ["rfp2_gemm", "rfp2_gemm_f16"]


def run_gemm(packed, N, K, q, d, fn="rfp2_gemm"):
    M = q.shape[0]
    y = empty((M, N), torch.float32)
    getattr(rf, fn)(to_dev(packed.reshape(-1)), N, K, to_dev(q), to_dev(d), M, y)
    return host(y)


# token counts of the report's multi-column check (1, 4, 32, 128) plus a
# prompt batch, with ragged token and row counts
SHAPES = [(1, 128, 256), (4, 200, 512), (32, 256, 1024), (128, 384, 2048),
          (130, 300, 768), (512, 512, 4096), (257, 129, 5120), (3, 1, 256)]


@pytest.mark.parametrize("fn", GEMMS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_shapes(M, N, K, fn):
    announce(fn, M, N, K)
    packed = random_blocks(N, K, seed=M + N + K, scale_hi=0x30)
    q, d = oracle.quantize_acts(synth.activations(M, K, seed=M))
    y = run_gemm(packed, N, K, q, d, fn)
    assert_within_bound(y, oracle.ref_gemm(packed, N, K, q, d),
                        oracle.abs_product_sums(packed, N, K, q, d), f"gemm {M}x{N}x{K}")


@pytest.mark.parametrize("fn", GEMMS)
def test_gemm_matches_gemv_columns(fn):
    announce(fn, "vs gemv")
    N, K = 256, 2048
    packed = random_blocks(N, K, seed=3, scale_hi=0x30)
    q, d = oracle.quantize_acts(synth.activations(4, K))
    y_mm = run_gemm(packed, N, K, q, d, fn)
    y_mv = empty((4, N), torch.float32)
    rf.rfp2_gemv(to_dev(packed.reshape(-1)), N, K, to_dev(q), to_dev(d), 4, y_mv)
    absum = oracle.abs_product_sums(packed, N, K, q, d)
    assert np.all(np.abs(y_mm - host(y_mv)) <= 2e-5 * absum + 2e-6)


@pytest.mark.parametrize("fn", GEMMS)
def test_gemm_illegal_scale_gives_nan_row(fn):
    announce(fn, "illegal scale byte")
    M, N, K = 40, 150, 512
    packed = random_blocks(N, K, seed=4, scale_hi=0x30)
    packed[77, 10 * 3 + 8] = 0x7F
    q, d = oracle.quantize_acts(synth.activations(M, K))
    y = run_gemm(packed, N, K, q, d, fn)
    assert np.isnan(y[:, 77]).all()
    assert np.isfinite(np.delete(y, 77, axis=1)).all()


@pytest.mark.parametrize("fn", GEMMS)
def test_gemm_full_size_sampled_rows(fn):
    cfg = synth.WORKLOADS["gemm_512x14336x4096"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    announce(fn, "full", M, N, K)
    W = synth.weights(N, K, cfg["sigma"], seed=cfg["wseed"])
    a = synth.activations(M, K)
    w_g = empty((N * K // 32 * 10,), torch.uint8)
    rf.rfp2_quantize_weights(to_dev(W), N, K, w_g)
    q_g = empty((M, K), torch.int8)
    d_g = empty((M, K // 32), torch.float32)
    rf.rfp2_quantize_acts(to_dev(a), M, K, q_g, d_g)
    y_g = empty((M, N), torch.float32)
    getattr(rf, fn)(w_g, N, K, q_g, d_g, M, y_g)
    y = host(y_g)
    rows = sample_rows(N, 24, seed=14)
    packed_rows = oracle.quantize_weights(W[rows])
    assert np.array_equal(host(w_g).reshape(N, -1)[rows], packed_rows)
    q, d = oracle.quantize_acts(a)
    assert_within_bound(y[:, rows], oracle.ref_gemm(packed_rows, len(rows), K, q, d),
                        oracle.abs_product_sums(packed_rows, len(rows), K, q, d), fn + " full")
    assert np.isfinite(y).all()
