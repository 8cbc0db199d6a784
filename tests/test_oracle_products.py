"""Pins of the oracle's products (GEMV, multi-column, GEMM, routed experts).

Every quantity in the method is a dyadic rational (UE4M3 scales, fp32
activation scales, integer codes), so on tiny shapes the exact result can be
computed with fractions, straight from the stored bytes, with a per-element
loop that shares nothing with the oracle.  The oracle's fp64 products must
agree to fp64 rounding, and the rescale identity d * (s0*S0 + s1*S1) summed
over blocks must reproduce the exact result with no error at all.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
_SCALES = [Fraction(v) / 2 for v in
           torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn)
           .to(torch.float64).tolist()]
_LEVELS = (-4, -1, 1, 4)


def _exact(packed, N, K, q, d, with_abs=False):
    """Exact y[m][n], exact per-half integer sums and (with_abs) the exact
    sum_k |w[n,k] * a[m,k]|, from the raw bytes."""
    M = q.shape[0]
    B = K // 32
    y = [[Fraction(0)] * N for _ in range(M)]
    ab = [[Fraction(0)] * N for _ in range(M)]
    sums = np.zeros((M, N, B, 2), dtype=np.int64)
    for n in range(N):
        for b in range(B):
            blk = packed[n, 10 * b:10 * b + 10]
            for i in range(32):
                code = (int(blk[i // 4]) >> (2 * (i % 4))) & 3
                level = _LEVELS[code]
                s = _SCALES[int(blk[8 + i // 16])]
                for m in range(M):
                    qa = int(q[m, 32 * b + i])
                    term = level * s * qa * Fraction(float(d[m, b]))
                    y[m][n] += term
                    ab[m][n] += abs(term)
                    sums[m, n, b, i // 16] += level * qa
    return (y, sums, ab) if with_abs else (y, sums)


def _tiny_matrix(N, K, seed, all_bytes=False):
    rng = np.random.default_rng(seed)
    B = K // 32
    blocks = rng.integers(0, 256, (N, B, 10))
    blocks[..., 8:10] = rng.integers(0, 0x7F, (N, B, 2))
    if all_bytes:
        # every one of the 256 code byte values appears
        flat = blocks[..., :8].reshape(-1)
        flat[:256] = np.arange(256)
        blocks[..., :8] = flat.reshape(N, B, 8)
        # and the edge scale bytes
        blocks[0, 0, 8:10] = [0x00, 0x7E]
        blocks[-1, -1, 8:10] = [0x01, 0x07]
    return blocks.reshape(N, B * 10).astype(np.uint8)


CASES = [(1, 32, 1), (4, 64, 1), (3, 256, 3), (2, 256, 2), (4, 1024, 2)]


@pytest.mark.parametrize("N,K,M", CASES)
def test_products_match_exact_rationals(N, K, M):
    packed = _tiny_matrix(N, K, seed=N * 1000 + K, all_bytes=(K == 1024))
    rng = np.random.default_rng(K + M)
    a = rng.standard_normal((M, K)).astype(np.float32)
    q, d = oracle.quantize_acts(a)
    y_exact, sums_exact = _exact(packed, N, K, q, d)
    y = oracle.ref_gemv(packed, N, K, q, d)
    absum = oracle.abs_product_sums(packed, N, K, q, d)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(y[m, n])) - y_exact[m][n]) <= \
                Fraction(1, 10 ** 15) * (Fraction(float(absum[m, n])) + Fraction(1, 10 ** 300))
    assert np.array_equal(oracle.half_sums(packed, N, K, q), sums_exact)
    assert np.array_equal(oracle.ref_gemm(packed, N, K, q, d), y)


@pytest.mark.parametrize("N,K,M", CASES[:3])
def test_rescale_identity_is_exact(N, K, M):
    # y = sum_b d[m,b] * (s0 * S0 + s1 * S1), exactly, from the half sums
    packed = _tiny_matrix(N, K, seed=7 + K)
    a = np.random.default_rng(11).standard_normal((M, K)).astype(np.float32)
    q, d = oracle.quantize_acts(a)
    y_exact, _ = _exact(packed, N, K, q, d)
    S = oracle.half_sums(packed, N, K, q)
    _, eb = oracle.unpack_matrix(packed, N, K)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for b in range(K // 32):
                s0 = Fraction(oracle.ue4m3_decode(eb[n, 2 * b]))
                s1 = Fraction(oracle.ue4m3_decode(eb[n, 2 * b + 1]))
                tot += Fraction(float(d[m, b])) * (s0 * int(S[m, n, b, 0]) + s1 * int(S[m, n, b, 1]))
            assert tot == y_exact[m][n]


def test_half_sums_fit_int32_with_room():
    # |S| <= 16 * 4 * 127 = 8128: int32 accumulation cannot overflow and the
    # conversion to fp32 is exact
    packed = oracle.pack_matrix(np.full((1, 32), 3), np.array([[0x38, 0x38]]))
    q = np.full((1, 32), 127, np.int8)
    S = oracle.half_sums(packed, 1, 32, q)
    assert S.max() == 8128


def test_multi_column_equals_single_columns():
    packed = _tiny_matrix(5, 512, seed=3)
    a = np.random.default_rng(4).standard_normal((4, 512)).astype(np.float32)
    q, d = oracle.quantize_acts(a)
    y4 = oracle.ref_gemv(packed, 5, 512, q, d)
    for m in range(4):
        y1 = oracle.ref_gemv(packed, 5, 512, q[m:m + 1], d[m:m + 1])
        assert np.allclose(y4[m], y1[0], rtol=1e-15, atol=0)


def test_moe_rows_follow_ids_and_bad_ids_are_nan():
    E, N, K = 5, 3, 64
    bank = np.stack([_tiny_matrix(N, K, seed=50 + e) for e in range(E)])
    a = np.random.default_rng(5).standard_normal((1, K)).astype(np.float32)
    q, d = oracle.quantize_acts(a)
    ids = np.array([3, 0, 3, 7, -1, 4], np.int32)
    y = oracle.ref_moe_gemv(bank.reshape(-1), E, N, K, ids, q, d)
    assert y.shape == (6, N)
    for j, e in enumerate(ids):
        if 0 <= e < E:
            assert np.array_equal(y[j], oracle.ref_gemv(bank[e], N, K, q, d)[0])
        else:
            assert np.all(np.isnan(y[j]))
    assert np.array_equal(y[0], y[2])            # duplicates are independent copies


@pytest.mark.parametrize("N,K,M", CASES)
def test_abs_product_sums_match_exact_rationals(N, K, M):
    # The tolerance scale of every GPU comparison, sum_k |w[n,k] * a[m,k]|
    # ("03 · Runtime": the magnitudes of the terms d_a * s * level * q that
    # the integer pipeline sums), pinned to an exact evaluation from the raw
    # bytes.  Every term is exact in fp64 (a level times a UE4M3 scale has at
    # most 4 significant bits, q * d at most 31), so the oracle's only error
    # is the fp64 summation of K non-negative terms: at most (K - 1) * 2^-53
    # relative.  A scaled, shifted, signed or term-dropping variant fails.
    packed = _tiny_matrix(N, K, seed=N * 1000 + K + 1, all_bytes=(K == 1024))
    rng = np.random.default_rng(K + M + 1)
    a = rng.standard_normal((M, K)).astype(np.float32)
    q, d = oracle.quantize_acts(a)
    _, _, ab_exact = _exact(packed, N, K, q, d, with_abs=True)
    absum = oracle.abs_product_sums(packed, N, K, q, d)
    assert absum.shape == (M, N)
    rel = Fraction(K, 2 ** 53)
    for m in range(M):
        for n in range(N):
            exact = ab_exact[m][n]
            assert exact > 0
            assert abs(Fraction(float(absum[m, n])) - exact) <= rel * exact


def test_abs_product_sums_edge_scales_and_signs():
    # one block per row, chosen by hand: the sum of magnitudes ignores the
    # signs of levels and activations, takes each half's own scale (0x7E =
    # 224, 0x01 = 2^-10, 0x00 = 0) and equals |y| when every term has one sign
    codes = np.zeros((3, 32), np.uint8)
    codes[0, :16] = 0            # -4 on half 0
    codes[0, 16:] = 3            # +4 on half 1
    codes[1] = np.arange(32) % 4
    codes[2] = 2                 # +1 everywhere
    eb = np.array([[0x7E, 0x01], [0x38, 0x00], [0x01, 0x7E]], np.uint8)
    packed = oracle.pack_matrix(codes, eb)
    q = np.concatenate([np.full(16, -3), np.full(16, 5)]).astype(np.int8)[None, :]
    d = np.array([[0.25]], np.float32)
    absum = oracle.abs_product_sums(packed, 3, 32, q, d)
    lv = np.array([-4, -1, 1, 4])
    exp0 = 16 * 4 * 224 * 3 * 0.25 + 16 * 4 * 2 ** -10 * 5 * 0.25
    exp1 = sum(abs(lv[i % 4]) * 0.5 * abs(int(q[0, i])) * 0.25 for i in range(16))
    exp2 = 16 * 2 ** -10 * 3 * 0.25 + 16 * 224 * 5 * 0.25
    assert absum[0].tolist() == [exp0, exp1, exp2]
    y = oracle.ref_gemv(packed, 3, 32, q, d)
    assert y[0, 0] == absum[0, 0]                 # (-4)(-3) and (+4)(+5): all positive
    assert abs(y[0, 2]) < absum[0, 2]             # mixed signs cancel in y only
