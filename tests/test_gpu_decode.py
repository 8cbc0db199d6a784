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


def parity_blocks(pairs=256):
    """Blocks 2t and 2t + 1 identical (t < pairs), so that every byte value
    sits in an even block (starting on a dword of an 80-byte group) and in an
    odd one (starting at byte 2 of a dword): code bytes (8t + j) % 256 cover
    all 256 values at both parities, the scale pair (t % 256, (t + 128) %
    256) every legal and illegal scale byte in both positions.  -> uint8
    [2 * pairs * 10]."""
    t = np.repeat(np.arange(pairs), 2)
    codes = (8 * t[:, None] + np.arange(8)[None, :]) % 256
    scales = np.stack([t % 256, (t + 128) % 256], axis=1)
    return np.concatenate([codes, scales], axis=1).astype(np.uint8).reshape(-1)


def _expected_scales(eb):
    legal = eb <= oracle.UE4M3_MAX_BYTE
    ref = np.full(eb.shape, np.nan, np.float32)
    ref[legal] = oracle.ue4m3_table()[eb[legal]].astype(np.float32)
    return ref


@pytest.mark.parametrize("N,K", [(16, 1024), (4, 4096), (3, 96)])
def test_gemv_group_decode_all_bytes_both_parities(N, K):
    # the GEMV's own decode (decode_block on an 80-byte group), bit for bit:
    # every code byte and every scale byte at even and odd block positions
    announce("debug_decode parity blocks", N, K)
    flat = parity_blocks(256)
    packed = np.resize(flat, N * K // 32 * 10).reshape(N, K // 32 * 10)
    codes, scales = _decode(packed, N, K)
    assert np.array_equal(codes, oracle.decoded_int8(packed, N, K))
    _, eb = oracle.unpack_matrix(packed, N, K)
    ref = _expected_scales(eb)
    assert np.array_equal(np.isnan(scales), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(scales[ok], ref[ok])
    if N * K // 32 >= 512:
        # each legal and illegal byte was seen in both positions, both parities
        blk = np.arange(N * K // 32)
        for pos in (0, 1):
            for par in (0, 1):
                seen = eb.reshape(-1, 2)[(blk % 2 == par), pos]
                assert len(np.unique(seen)) == 256


@pytest.mark.parametrize("N,K,M", [(16, 1024, 2), (3, 96, 1)])
def test_gemv_group_half_dots_all_bytes_both_parities(N, K, M):
    announce("debug_half_dots parity blocks", N, K, M)
    flat = parity_blocks(256)
    packed = np.resize(flat, N * K // 32 * 10).reshape(N, K // 32 * 10)
    q = synth.uniform_bytes(M * K, 0, 254, seed=17 + M).view(np.int8).reshape(M, K)
    q = np.where(q == -128, -127, q).astype(np.int8)
    q[0, :64] = 127                          # extremes on an even and an odd block
    q[-1, 64:128] = -127
    sums = empty((M, N, K // 32, 2), torch.int32)
    rf.rfp2_debug_half_dots(to_dev(packed.reshape(-1)), N, K, to_dev(q), M, sums)
    got = host(sums).astype(np.int64)
    assert np.array_equal(got, oracle.half_sums(packed, N, K, q))


@pytest.mark.parametrize("N,K,M", [(16, 1024, 4), (7, 256, 1), (9, 512, 3), (5, 2048, 6)])
def test_gemv_mf_half_sums_all_bytes_both_parities(N, K, M):
    # the int32 half sums of the GEMV's matrix-core form (4x4x4 int8 products
    # over quads of four rows at one group), bit for bit: every code byte at
    # even and odd block positions, extreme activations, ragged rows and
    # column quads (M = 1, 3 and 6 leave column slots past the end)
    announce("debug_half_sums_mf", N, K, M)
    flat = parity_blocks(256)
    packed = np.resize(flat, N * K // 32 * 10).reshape(N, K // 32 * 10)
    q = synth.uniform_bytes(M * K, 0, 254, seed=29 + M).view(np.int8).reshape(M, K)
    q = np.where(q == -128, -127, q).astype(np.int8)
    q[0, :64] = 127
    q[-1, 64:128] = -127
    ref = oracle.half_sums(packed, N, K, q)
    sums = empty((M, N, K // 32, 2), torch.int32)
    rf.rfp2_debug_half_sums_mf(to_dev(packed.reshape(-1)), N, K, to_dev(q), M, sums)
    assert np.array_equal(host(sums).astype(np.int64), ref)
    if M == 1 and N == 7:
        # the dot4 form of the same sums agrees as well
        dots = empty((M, N, K // 32, 2), torch.int32)
        rf.rfp2_debug_half_dots(to_dev(packed.reshape(-1)), N, K, to_dev(q), M, dots)
        assert np.array_equal(host(dots), host(sums))


@pytest.mark.parametrize("form", [0, 1])
@pytest.mark.parametrize("N,K", [(16, 1024), (3, 96), (5, 32)])
def test_f16_decode_bitexact(form, N, K):
    # the fp16 matrix-core kernels' decode (form 0: rfp2_gemm_f16's staging;
    # form 1: rfp2_moe_gemm's per-lane operand decode), bit for bit against
    # level * scale in IEEE half precision; a block with an illegal scale byte
    # is NaN in both halves
    announce("debug_decode_f16", form, N, K)
    flat = parity_blocks(256)
    packed = np.resize(flat, N * K // 32 * 10).reshape(N, K // 32 * 10)
    h = empty((N, K), torch.int16)
    rf.rfp2_debug_decode_f16(to_dev(packed.reshape(-1)), N, K, form, h)
    got = host(h).view(np.float16)
    codes, eb = oracle.unpack_matrix(packed, N, K)
    eb_blk = eb.reshape(N, K // 32, 2)
    bad_blk = (eb_blk > oracle.UE4M3_MAX_BYTE).any(axis=2)             # [N, B]
    clean = packed.copy().reshape(N, K // 32, 10)
    clean[..., 8:10] = np.where(clean[..., 8:10] > 0x7E, 0x38, clean[..., 8:10])
    ref = oracle.dequantize_weights(clean.reshape(N, -1), N, K).astype(np.float16)
    bad = np.repeat(bad_blk, 32, axis=1)
    assert np.isnan(got[bad]).all()
    assert np.array_equal(got[~bad].view(np.uint16), ref[~bad].view(np.uint16))


def exponent_grid_blocks():
    """Legal blocks for the int8 GEMM's folded decode: blocks 2t and 2t + 1
    identical (both parities of a pair, as parity_blocks); code bytes
    (8t + j) % 256; scale pair t covers the exponent pair (E0, E1) =
    (t // 16, t % 16), every gap 0..15 in both orders, subnormal halves
    (E = 0) included, with mantissas spread over 0..7 (0..6 at E = 15, where
    0x7F is illegal).  -> uint8 [512 * 10]."""
    t = np.repeat(np.arange(256), 2)
    E0, E1 = t // 16, t % 16
    M0, M1 = (3 * E0 + E1) % 8, (5 * E1 + E0 + 1) % 8
    M0 = np.where(E0 == 15, np.minimum(M0, 6), M0)
    M1 = np.where(E1 == 15, np.minimum(M1, 6), M1)
    codes = (8 * t[:, None] + np.arange(8)[None, :]) % 256
    scales = np.stack([8 * E0 + M0, 8 * E1 + M1], axis=1)
    return np.concatenate([codes, scales], axis=1).astype(np.uint8).reshape(-1)


def _decode_i8(packed, N, K):
    wa, wb = empty((N, K), torch.int8), empty((N, K), torch.int8)
    sc = empty((N, K // 32, 6), torch.float32)
    rf.rfp2_debug_decode_i8(to_dev(packed.reshape(-1)), N, K, wa, wb, sc)
    return host(wa).astype(np.int64), host(wb).astype(np.int64), host(sc).astype(np.float64)


@pytest.mark.parametrize("N,K", [(16, 1024), (3, 96), (5, 32)])
def test_gemm_i8_folded_decode_bitexact(N, K):
    # the int8 GEMM's staging decode (pairs of blocks, the second one
    # funnel-shifted; the scale mantissas folded into two int8 operands), bit
    # for bit: every weight's wa * sA + wb * sB is level * scale exactly; a
    # block is folded whole (s = sA = sB > 0) exactly when its exponents
    # (E, 0 counted as 1) differ by at most 2, s then the power of two of the
    # smaller one; otherwise s = -sB and sA, sB are the halves' own powers of
    # two.  The bias constants are -1.5 * 2^23 times their scales.
    announce("debug_decode_i8", N, K)
    packed = np.resize(exponent_grid_blocks(), N * K // 32 * 10).reshape(N, K // 32 * 10)
    wa, wb, sc = _decode_i8(packed, N, K)
    ref = oracle.dequantize_weights(packed, N, K)
    sA = np.repeat(sc[..., 2], 32, axis=1)
    sB = np.repeat(sc[..., 4], 32, axis=1)
    assert np.array_equal(wa * sA + wb * sB, ref)
    _, eb = oracle.unpack_matrix(packed, N, K)
    x = np.maximum(eb.astype(np.int64).reshape(N, K // 32, 2) >> 3, 1)
    whole = np.abs(x[..., 0] - x[..., 1]) <= 2
    assert np.array_equal(sc[..., 0] > 0, whole)
    assert np.array_equal(sc[whole][:, 0], sc[whole][:, 2])
    assert np.array_equal(sc[whole][:, 0], sc[whole][:, 4])
    assert np.array_equal(sc[~whole][:, 0], -sc[~whole][:, 4])
    assert np.array_equal(sc[..., 4], 2.0 ** (x.min(axis=2) - 11))
    assert np.array_equal(sc[~whole][:, 2], 2.0 ** (x[~whole].max(axis=1) - 11))
    for v, s_ in ((1, 4), (3, 2), (5, 4)):
        assert np.array_equal(sc[..., v], -12582912.0 * sc[..., s_])
    # a whole block's sum stays below 2^22 with any int8 activations
    assert np.abs(wa + wb).max() <= 240
    if N * K // 32 >= 512:
        assert whole.any() and (~whole).any()


def test_gemm_i8_decode_illegal_scale_is_nan():
    # a block with an illegal scale byte (0x7F..0xFF in either half, in
    # either block of a pair) gets NaN for all six of its scales
    announce("debug_decode_i8 illegal scale bytes")
    N, K = 16, 1024
    packed = np.resize(parity_blocks(256), N * K // 32 * 10).reshape(N, K // 32 * 10)
    _, _, sc = _decode_i8(packed, N, K)
    assert np.isnan(sc).all()
    packed = packed.reshape(N, K // 32, 10)
    packed[..., 8:10] = np.where(packed[..., 8:10] > 0x7E, 0x38, packed[..., 8:10])
    _, _, sc = _decode_i8(packed.reshape(N, -1), N, K)
    assert not np.isnan(sc).any()
