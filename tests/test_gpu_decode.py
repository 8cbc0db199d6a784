"""GPU parity, bit for bit: the int8 lanes and scales a stored block expands
to, and the int32 half sums, as computed by the device functions the product
kernels use."""
import numpy as np
import pytest

import bit_gemv_amd as rf
import oracle
import synth
from _gpu import announce, empty, host, to_dev, torch

pytestmark = pytest.mark.gpu


def random_blocks(N, K, seed, scale_lo=0, scale_hi=0x7E):
    """uint8 [N, K/32*10]: uniform code bytes, scale bytes in [lo, hi]; every
    code byte value and every legal scale byte appears when there is room."""
    B = K // 32
    codes = synth.uniform_bytes(N * B * 8, 0, 255, seed).reshape(N, B, 8)
    scales = synth.uniform_bytes(N * B * 2, scale_lo, scale_hi, seed + 1).reshape(N, B, 2)
    flat = codes.reshape(-1)
    n = min(256, flat.size)
    flat[:n] = np.arange(n, dtype=np.uint8)
    sflat = scales.reshape(-1)
    n = min(scale_hi - scale_lo + 1, sflat.size)
    sflat[:n] = np.arange(scale_lo, scale_lo + n, dtype=np.uint8)
    return np.concatenate([codes, scales], axis=2).reshape(N, B * 10)


def _decode(packed, N, K):
    codes = empty((N, K), torch.int8)
    scales = empty((N, K // 16), torch.float32)
    rf.rfp2_debug_decode(to_dev(packed.reshape(-1)), N, K, codes, scales)
    return host(codes), host(scales)


@pytest.mark.parametrize("N,K", [(16, 256), (33, 96), (7, 4096)])
def test_decode_lanes_and_scales_bitexact(N, K):
    announce("debug_decode", N, K)
    packed = random_blocks(N, K, seed=N + K)
    codes, scales = _decode(packed, N, K)
    assert np.array_equal(codes, oracle.decoded_int8(packed, N, K))
    _, eb = oracle.unpack_matrix(packed, N, K)
    assert np.array_equal(scales, oracle.ue4m3_table()[eb].astype(np.float32))


def test_decode_illegal_scale_bytes_are_nan():
    announce("debug_decode illegal scale bytes")
    N, K = 4, 64
    packed = random_blocks(N, K, seed=5)
    bad = [0x7F, 0x80, 0xFF, 0xC3]
    for i, b in enumerate(bad):
        packed[i, 8] = b                     # e0 of block 0 of row i
    packed[0, 9] = 0x7E                      # a legal partner next to 0x7F
    packed[2, 9] = 0x00                      # a legal partner next to 0xFF
    _, scales = _decode(packed, N, K)
    for i in range(len(bad)):
        assert np.isnan(scales[i, 0])
    assert scales[0, 1] == 224.0 and scales[2, 1] == 0.0
    assert not np.isnan(scales[:, 2:]).any()


@pytest.mark.parametrize("N,K,M", [(8, 256, 1), (5, 96, 3), (3, 1024, 4)])
def test_half_dots_bitexact(N, K, M):
    announce("debug_half_dots", N, K, M)
    packed = random_blocks(N, K, seed=10 * N + M)
    q = synth.uniform_bytes(M * K, 0, 254, seed=M).view(np.int8).reshape(M, K)
    q = np.where(q == -128, 127, q).astype(np.int8)
    q[0, :32] = 127                          # extreme sums
    packed[0, :8] = 0xFF                     # all codes +4 in block 0 of row 0
    sums = empty((M, N, K // 32, 2), torch.int32)
    rf.rfp2_debug_half_dots(to_dev(packed.reshape(-1)), N, K, to_dev(q), M, sums)
    ref = oracle.half_sums(packed, N, K, q)
    got = host(sums)
    assert np.array_equal(got.astype(np.int64), ref)
    assert got[0, 0, 0, 0] == 8128
