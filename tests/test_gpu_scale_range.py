"""GPU parity of every product over the whole legal scale range ("02 ·
Quantization": one scale byte per 16-weight half, 127 legal values
0x00..0x7E, 2^-10 .. 224).

The other product tests draw their scale bytes from the low end of the range
or from the page's own search on normal weights.  Here the two halves of a
block are as far apart as the format allows (0x00..0x0F next to 0x60..0x7E,
in either order, including 0x01 beside 0x7E), every block sits at the top of
the range, or the bytes are uniform over all 127 values.  Every output is
held to |y - y_ref| <= 1e-5 * sum_k |w_k a_k| + 1e-6 against the fp64
oracle."""
import numpy as np
import pytest

import bit_gemv_amd as rf
import oracle
import synth
from _gpu import announce, assert_within_bound, empty, host, to_dev, torch

pytestmark = pytest.mark.gpu

MODES = ["split", "high", "full"]


def wide_scale_blocks(N, K, seed, mode):
    """uint8 [N, K/32*10]: uniform code bytes (all 256 values when there is
    room) and scale bytes by `mode`."""
    rng = np.random.default_rng(seed)
    B = K // 32
    codes = rng.integers(0, 256, (N, B, 8))
    flat = codes.reshape(-1)
    flat[:min(256, flat.size)] = np.arange(min(256, flat.size))
    if mode == "split":
        lo = rng.integers(0x00, 0x10, (N, B))
        hi = rng.integers(0x60, 0x7F, (N, B))
        swap = rng.random((N, B)) < 0.5
        e0, e1 = np.where(swap, hi, lo), np.where(swap, lo, hi)
        scales = np.stack([e0, e1], axis=2)
        scales[0, 0] = [0x01, 0x7E]
        scales[-1, -1] = [0x7E, 0x01]
    elif mode == "high":
        scales = rng.integers(0x70, 0x7F, (N, B, 2))
        scales[0, 0] = [0x7E, 0x7E]
    else:
        scales = rng.integers(0x00, 0x7F, (N, B, 2))
        sflat = scales.reshape(-1)
        sflat[:min(127, sflat.size)] = np.arange(min(127, sflat.size))
    return np.concatenate([codes, scales], axis=2).astype(np.uint8).reshape(N, B * 10)


def _acts(M, K, seed):
    return oracle.quantize_acts(synth.activations(M, K, seed=seed))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M", [1, 3, 4, 8])
def test_gemv_scale_range(mode, M):
    N, K = 300, 2048
    announce("gemv scale range", mode, M)
    packed = wide_scale_blocks(N, K, seed=M, mode=mode)
    q, d = _acts(M, K, seed=40 + M)
    y = empty((M, N), torch.float32)
    rf.rfp2_gemv(to_dev(packed.reshape(-1)), N, K, to_dev(q), to_dev(d), M, y)
    assert_within_bound(host(y), oracle.ref_gemv(packed, N, K, q, d),
                        oracle.abs_product_sums(packed, N, K, q, d), f"gemv {mode} M={M}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("K", [2048, 8192, 14336])
def test_quant_gemv_scale_range(mode, K):
    N = 200
    announce("quant_gemv scale range", mode, K)
    packed = wide_scale_blocks(N, K, seed=K, mode=mode)
    a = synth.activations(1, K, seed=K + 1)
    q_ref, d_ref = oracle.quantize_acts(a)
    q, d, y = empty(K, torch.int8), empty(K // 32, torch.float32), empty(N, torch.float32)
    rf.rfp2_quant_gemv(to_dev(packed.reshape(-1)), N, K, to_dev(a[0]), q, d, y)
    assert np.array_equal(host(q), q_ref[0]) and np.array_equal(host(d), d_ref[0])
    assert_within_bound(host(y), oracle.ref_gemv(packed, N, K, q_ref, d_ref)[0],
                        oracle.abs_product_sums(packed, N, K, q_ref, d_ref)[0],
                        f"quant_gemv {mode} K={K}")


@pytest.mark.parametrize("mode", MODES)
def test_moe_gemv_and_quant_moe_gemv_scale_range(mode):
    E, N, K, top_k = 6, 200, 2048, 4
    announce("moe_gemv scale range", mode)
    bank = np.stack([wide_scale_blocks(N, K, seed=10 + e, mode=mode) for e in range(E)])
    ids = np.array([5, 0, 3, 0], np.int32)
    a = synth.activations(1, K, seed=3)
    q, d = oracle.quantize_acts(a)
    ref = oracle.ref_moe_gemv(bank.reshape(-1), E, N, K, ids, q, d)
    absum = np.stack([oracle.abs_product_sums(bank[e], N, K, q, d)[0] for e in ids])
    y = empty((top_k, N), torch.float32)
    rf.rfp2_moe_gemv(to_dev(bank.reshape(-1)), E, N, K, to_dev(ids), top_k, to_dev(q),
                     to_dev(d), y)
    assert_within_bound(host(y), ref, absum, f"moe_gemv {mode}")
    qg, dg, y2 = empty(K, torch.int8), empty(K // 32, torch.float32), empty((top_k, N),
                                                                          torch.float32)
    rf.rfp2_quant_moe_gemv(to_dev(bank.reshape(-1)), E, N, K, to_dev(ids), top_k,
                           to_dev(a[0]), qg, dg, y2)
    assert_within_bound(host(y2), ref, absum, f"quant_moe_gemv {mode}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("T", [2, 4, 8])
def test_moe_gemv_tokens_scale_range(mode, T):
    E, N, K, top_k = 8, 200, 2048, 4
    announce("moe_gemv_tokens scale range", mode, T)
    rng = np.random.default_rng(T)
    bank = np.stack([wide_scale_blocks(N, K, seed=20 + e, mode=mode) for e in range(E)])
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[-1] = ids[0]                                   # shared experts between tokens
    q, d = _acts(T, K, seed=50 + T)
    ref = oracle.ref_moe_batch(bank.reshape(-1), E, N, K, ids, q, d)
    absum = np.stack([oracle.abs_product_sums(bank[ids[t, j]], N, K, q[t:t + 1],
                                              d[t:t + 1])[0]
                      for t in range(T) for j in range(top_k)])
    y = empty((T * top_k, N), torch.float32)
    rf.rfp2_moe_gemv_tokens(to_dev(bank.reshape(-1)), E, N, K, to_dev(ids), T, top_k,
                            to_dev(q), to_dev(d), y)
    assert_within_bound(host(y), ref, absum, f"moe_gemv_tokens {mode} T={T}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("call", ["rfp2_gemm", "rfp2_gemm_f16"])
@pytest.mark.parametrize("M", [5, 130])
def test_gemm_scale_range(mode, call, M):
    N, K = 260, 1024
    announce(call, "scale range", mode, M)
    packed = wide_scale_blocks(N, K, seed=M + 7, mode=mode)
    q, d = _acts(M, K, seed=60 + M)
    y = empty((M, N), torch.float32)
    getattr(rf, call)(to_dev(packed.reshape(-1)), N, K, to_dev(q), to_dev(d), M, y)
    assert_within_bound(host(y), oracle.ref_gemm(packed, N, K, q, d),
                        oracle.abs_product_sums(packed, N, K, q, d), f"{call} {mode} M={M}")


@pytest.mark.parametrize("mode", MODES)
def test_moe_gemm_scale_range(mode):
    E, N, K, T, top_k = 6, 200, 1024, 40, 3
    announce("moe_gemm scale range", mode)
    rng = np.random.default_rng(11)
    bank = np.stack([wide_scale_blocks(N, K, seed=30 + e, mode=mode) for e in range(E)])
    ids = np.stack([rng.choice(E, top_k, replace=False) for _ in range(T)]).astype(np.int32)
    q, d = _acts(T, K, seed=70)
    ref = oracle.ref_moe_batch(bank.reshape(-1), E, N, K, ids, q, d)
    absum = np.stack([oracle.abs_product_sums(bank[ids[t, j]], N, K, q[t:t + 1],
                                              d[t:t + 1])[0]
                      for t in range(T) for j in range(top_k)])
    y = empty((T * top_k, N), torch.float32)
    rf.rfp2_moe_gemm(to_dev(bank.reshape(-1)), E, N, K, to_dev(ids), T, top_k, to_dev(q),
                     to_dev(d), y)
    assert_within_bound(host(y), ref, absum, f"moe_gemm {mode}")
