"""Pins of the oracle's int8 activation quantizer.

The report prints no worked activation block, so the quantizer is pinned by an
exact-rational brute force of its definition (d is the fp32 number nearest to
max|a|/127; q is the integer nearest to the fp32 quotient a/d, halves away from
zero, clamped to +-127) and by invariants.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _nearest_f32(x: Fraction) -> np.float32:
    """fp32 value nearest to the rational x, ties to the even significand."""
    c = np.float32(float(x))
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    best = None
    for v in cands:
        if not np.isfinite(v):
            continue
        err = abs(Fraction(float(v)) - x)
        even = int(np.array(v, np.float32).view(np.uint32)) & 1
        key = (err, even)
        if best is None or key < best[0]:
            best = (key, v)
    return np.float32(best[1])


def _round_half_away(x: Fraction) -> int:
    f = int(abs(x))                      # floor of |x|
    r = f + 1 if abs(x) - f >= Fraction(1, 2) else f
    return r if x >= 0 else -r


def _brute_block(a32):
    amax = max(abs(Fraction(float(v))) for v in a32)
    d = _nearest_f32(amax / 127)
    if d == 0:
        return [0] * 32, np.float32(0)
    q = []
    for v in a32:
        r = _nearest_f32(Fraction(float(v)) / Fraction(float(d)))
        q.append(max(-127, min(127, _round_half_away(Fraction(float(r))))))
    return q, d


@pytest.mark.parametrize("seed", range(6))
def test_matches_exact_definition(seed):
    rng = np.random.default_rng(200 + seed)
    scale = [1.0, 1e-3, 1e3, 1e-30, 7.0, 0.5][seed]
    a = (rng.standard_normal((3, 64)) * scale).astype(np.float32)
    q, d = oracle.quantize_acts(a)
    for m in range(3):
        for b in range(2):
            qb, db = _brute_block(a[m, 32 * b:32 * b + 32])
            assert d[m, b] == db
            assert list(q[m, 32 * b:32 * b + 32]) == qb


def test_halfway_quotients_round_away_from_zero():
    # amax = 127 gives d = 1 exactly, so a/d = a: halves are exact
    a = np.zeros((1, 32), np.float32)
    a[0, 0] = 127.0
    a[0, 1:7] = [0.5, -0.5, 1.5, -1.5, 2.5, -126.5]
    q, d = oracle.quantize_acts(a)
    assert d[0, 0] == 1.0
    assert list(q[0, :7]) == [127, 1, -1, 2, -2, 3, -127]
    qb, db = _brute_block(a[0])
    assert list(q[0]) == qb and db == d[0, 0]


def test_invariants():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((4, 256)).astype(np.float32)
    q, d = oracle.quantize_acts(a)
    A = a.reshape(4, 8, 32).astype(np.float64)
    Q = q.reshape(4, 8, 32).astype(np.float64)
    D = d.astype(np.float64)[..., None]
    assert np.all(np.abs(Q) <= 127)
    arg = np.abs(A).argmax(axis=2)
    assert np.all(np.abs(np.take_along_axis(Q, arg[..., None], 2)) == 127)
    # the error of a reconstructed activation is at most half a step (plus the
    # rounding of the fp32 quotient)
    assert np.all(np.abs(A - Q * D) <= D * (0.5 + 1e-6))


def test_zero_and_underflowing_blocks():
    a = np.zeros((1, 64), np.float32)
    a[0, 40] = np.float32(2.0 ** -149)          # amax/127 underflows to 0
    q, d = oracle.quantize_acts(a)
    assert np.all(d == 0) and np.all(q == 0)


def deep_subnormal_block():
    """32 activations n * 2^-149 with max n = 1327, so max / 127 = 10.449 *
    2^-149 rounds to the subnormal d = 10 * 2^-149 and the largest quotient
    is 132.7: past 127.5, where only the clamp keeps q at 127."""
    n = np.array([1327, 700, -1000, 3, -5, 1200, -1327, 0] * 4, np.float32)
    return n * np.float32(2.0 ** -149)


def test_subnormal_scale_quotients_are_clamped():
    q, d = oracle.quantize_acts(deep_subnormal_block()[None, :])
    assert d[0, 0] == np.float32(10 * 2.0 ** -149)
    # q = clamp(round(n / 10)), halves away from zero
    assert list(q[0, :8]) == [127, 70, -100, 0, -1, 120, -127, 0]


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize_acts(np.full((1, 32), np.inf, np.float32))
    with pytest.raises(TypeError):
        oracle.quantize_acts(np.zeros((1, 32)))
    with pytest.raises(ValueError):
        oracle.quantize_acts(np.zeros((1, 48), np.float32))
