"""GPU parity: activation and weight quantizers against the oracle, bit for bit."""
import numpy as np
import pytest

import bit_gemv_amd as rf
import oracle
import synth
from _gpu import announce, empty, host, sample_rows, to_dev, torch
from test_oracle_acts import deep_subnormal_block

pytestmark = pytest.mark.gpu


def _gpu_quantize_acts(a):
    M, K = a.shape
    q = empty((M, K), torch.int8)
    d = empty((M, K // 32), torch.float32)
    rf.rfp2_quantize_acts(to_dev(a), M, K, q, d)
    return host(q), host(d)


@pytest.mark.parametrize("M,K", [(1, 2048), (1, 4096), (4, 5120), (512, 4096), (3, 32), (2, 96)])
def test_quantize_acts_bitexact(M, K):
    announce("quantize_acts", M, K)
    a = synth.activations(M, K)
    if K >= 96:
        a[0, :32] = 0.0                                   # all-zero block
        a[0, 32:64] = np.arange(32, dtype=np.float32) - 15.5  # d = 1: a/d ends in .5
        a[0, 63] = 127.0
        a[-1, 64:96] *= np.float32(1e-30)                  # tiny values
    if K >= 128:
        a[0, 96:128] = deep_subnormal_block()               # clamped quotients
    q_ref, d_ref = oracle.quantize_acts(a)
    q, d = _gpu_quantize_acts(a)
    assert np.array_equal(d.view(np.uint32), d_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)


def test_quantize_acts_nonfinite_blocks_are_loud():
    announce("quantize_acts non-finite")
    a = synth.activations(2, 256)
    a[0, 3] = np.nan
    a[1, 100] = np.inf
    q, d = _gpu_quantize_acts(a)
    assert np.isnan(d[0, 0]) and np.isnan(d[1, 3])
    assert np.all(q[0, :32] == 0) and np.all(q[1, 96:128] == 0)
    clean = a.copy()
    clean[0, :32] = 0
    clean[1, 96:128] = 0
    q_ref, d_ref = oracle.quantize_acts(clean)
    ok = np.ones(d.shape, bool)
    ok[0, 0] = ok[1, 3] = False
    assert np.array_equal(d[ok], d_ref[ok])
    mask = np.repeat(ok, 32, axis=1)
    assert np.array_equal(q[mask], q_ref[mask])


def _gpu_quantize_weights(W):
    N, K = W.shape
    w = empty((N * K // 32 * 10,), torch.uint8)
    rf.rfp2_quantize_weights(to_dev(W), N, K, w)
    return host(w).reshape(N, K // 32 * 10)


def test_quantize_weights_bitexact_full_small():
    announce("quantize_weights 512x2048")
    W = synth.weights(512, 2048, 0.02, seed=0)
    assert np.array_equal(_gpu_quantize_weights(W), oracle.quantize_weights(W))


def test_quantize_weights_edge_halves():
    announce("quantize_weights edge halves")
    halves = [
        [0.0] * 16, [-0.0] * 16, [2.125] * 16, [0.1875] * 16, [2.0 ** -12] * 16,
        [1e4] + [0.0] * 15, [224.0 * 4] * 16, [2.5, -2.5, 1.0, -1.0] * 4,
        [1e-45] * 16, [-1.8, -0.4, 0.7, 2.1] * 4, list(np.linspace(-1, 1, 16)),
        [3.0, -3.0, 0.0, 1e-9] * 4,
    ]
    if len(halves) % 2:
        halves.append([0.25] * 16)
    W = np.array(halves, dtype=np.float32).reshape(-1, 32)
    W = np.concatenate([W, synth.weights(6, 32, 1.0, seed=3)])
    assert np.array_equal(_gpu_quantize_weights(W), oracle.quantize_weights(W))


@pytest.mark.parametrize("name", ["gemv_4096x4096", "gemv_16384x5120", "gemm_512x14336x4096"])
def test_quantize_weights_full_size_sampled_rows(name):
    cfg = synth.WORKLOADS[name]
    N, K = cfg["N"], cfg["K"]
    announce("quantize_weights full", name)
    W = synth.weights(N, K, cfg["sigma"], seed=cfg["wseed"])
    packed = _gpu_quantize_weights(W)
    rows = sample_rows(N, 24, seed=11)
    assert np.array_equal(packed[rows], oracle.quantize_weights(W[rows]))


def _gpu_quantize_weights_imatrix(W, imp):
    N, K = W.shape
    w = empty((N * K // 32 * 10,), torch.uint8)
    rf.rfp2_quantize_weights_imatrix(to_dev(W), N, K, to_dev(imp), w)
    return host(w).reshape(N, K // 32 * 10)


def test_quantize_weights_imatrix_bitexact_full_small():
    # the importance-weighted search ("05 · Completed experiment") on the GPU
    # against the oracle, every block; it must differ from the plain search
    announce("quantize_weights_imatrix 512x2048")
    W = synth.weights(512, 2048, 0.02, seed=0)
    imp = synth.importance(2048)
    got = _gpu_quantize_weights_imatrix(W, imp)
    assert np.array_equal(got, oracle.quantize_weights(W, imp))
    assert not np.array_equal(got, oracle.quantize_weights(W))


def test_quantize_weights_imatrix_special_importances():
    announce("quantize_weights_imatrix special importances")
    W = np.concatenate([synth.weights(8, 256, 0.02, seed=5),
                        synth.weights(8, 256, 1.0, seed=6)])
    K = W.shape[1]
    one_hot = np.zeros(K, np.float32)
    one_hot[::16] = 2.0                                  # one value per half
    for imp in (np.zeros(K, np.float32), np.ones(K, np.float32), one_hot,
                np.linspace(0, 4, K).astype(np.float32)):
        assert np.array_equal(_gpu_quantize_weights_imatrix(W, imp),
                              oracle.quantize_weights(W, imp))


def test_quantize_weights_imatrix_full_size_sampled_rows():
    announce("quantize_weights_imatrix 16384x5120")
    cfg = synth.WORKLOADS["gemv_16384x5120"]
    N, K = cfg["N"], cfg["K"]
    W = synth.weights(N, K, cfg["sigma"], seed=cfg["wseed"])
    imp = synth.importance(K)
    packed = _gpu_quantize_weights_imatrix(W, imp)
    rows = sample_rows(N, 24, seed=12)
    assert np.array_equal(packed[rows], oracle.quantize_weights(W[rows], imp))
