"""Pins of the oracle's clipped quantizer and clip search (CPU only).

The pages give clipping only as an optional ratio in the quantizer's configuration: a min-max
clipping of the group range before the search ("009. AWQ Integration", 架构 and 关键设计 5).  The
reading pinned here: both ends of the group range (0 included) are multiplied by c in (0, 1]
before Delta and the zero are formed, and codes clamp to the 16 levels; c = 1 is the unclipped
quantizer.  A clip search scores the grid c_j = 1 - (1 - c_min) j / (n - 1) with the same loss.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import awq_oracle as O


def _bf16_round(a):
    a = np.asarray(a, dtype=np.float32)
    b = a.view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _brute_clip_codes(P, g, zero_point, c):
    """Nearest of the 16 levels by enumeration (ties -> even level), with the group range of
    the reading computed in Python floats: [c*min(min, 0), c*max(max, 0)] (or c*max|p|)."""
    K, N = P.shape
    c = float(np.float32(c))
    codes = np.zeros((K, N), dtype=np.int64)
    for n in range(N):
        for j in range(K // g):
            col = [float(P[j * g + i, n]) for i in range(g)]
            if zero_point:
                hi, lo = max(max(col), 0.0) * c, min(min(col), 0.0) * c
                d = float(np.float32((hi - lo) / 15.0)) or 1.0
                z = min(max(round(-lo / d), 0), 15)
                cands = [(q, q - z) for q in range(16)]
            else:
                d = float(np.float32(max(abs(v) for v in col) * c / 7.0)) or 1.0
                cands = [(lv + 8, lv) for lv in range(-7, 8)]
            for i, p in enumerate(col):
                best = None
                for q, lv in cands:
                    key = (abs(p / d - lv), lv % 2)
                    if best is None or key < best[0]:
                        best = (key, q)
                codes[j * g + i, n] = best[1]
    return codes


@pytest.mark.parametrize("zero_point", [True, False])
@pytest.mark.parametrize("c", [0.3, 0.65, 0.9, 1.0])
def test_clipped_quantizer_matches_level_enumeration(zero_point, c):
    rng = np.random.default_rng(31)
    P = _bf16_round(rng.standard_normal((16, 7)))
    P[3, 0], P[12, 1] = 9.0, -11.0            # outliers that the clipped range cuts off
    P[:8, 2] = np.abs(P[:8, 2])               # one-signed group
    codes, delta, zero = O.quantize_groups(P, 8, zero_point, clip=c)
    assert np.array_equal(codes, _brute_clip_codes(P, 8, zero_point, c))
    assert codes.min() >= 0 and codes.max() <= 15
    if c < 1.0:   # the outliers sit beyond the clipped range: end levels
        hi_code = 15 if zero_point else 15
        assert codes[3, 0] == hi_code
        assert codes[12, 1] == (0 if zero_point else 1)


def test_clip_one_is_the_unclipped_quantizer():
    rng = np.random.default_rng(32)
    P = rng.standard_normal((256, 24)) * 0.05
    for zp in (True, False):
        a = O.quantize_groups(P, 128, zp)
        b = O.quantize_groups(P, 128, zp, clip=1.0)
        for u, v in zip(a, b):
            assert np.array_equal(u, v)


def test_clipped_loss_exact_rational_8x8():
    rng = np.random.default_rng(33)
    X = _bf16_round(rng.standard_normal((8, 8)))
    W = _bf16_round(rng.standard_normal((8, 8)) * 0.5)
    W[2, 3] = 6.0
    s = np.float32([1.0, 0.5, 2.0, 1.0, 4.0, 0.25, 1.0, 2.0])
    for g in (4, 8):
        for zp in (True, False):
            for c in (0.5, 0.8):
                P = s.astype(np.float64)[:, None] * W
                codes, delta, zero = O.quantize_groups(P, g, zp, clip=c)
                Lf = O.loss(X, W, s, g, zp, clip=c)
                E = [[Fraction(int(codes[k, n]) - int(zero[k // g, n])) * Fraction(float(delta[k // g, n]))
                      / Fraction(float(s[k])) - Fraction(float(W[k, n])) for n in range(8)] for k in range(8)]
                Lq = Fraction(0)
                for t in range(8):
                    for n in range(8):
                        y = sum(Fraction(float(X[t, k])) * E[k][n] for k in range(8))
                        Lq += y * y
                assert abs(Lf - float(Lq)) <= 1e-12 * float(Lq)


def test_clipping_wins_when_the_outlier_channels_are_silent():
    # one group of 8 channels: outliers +-100 on channels 0 and 1, small values elsewhere.
    col = np.array([100.0, -100.0, 1.0, -1.0, 0.5, -0.5, 0.25, 0.0])
    W = col[:, None]
    s = np.ones(8, dtype=np.float32)
    X = np.eye(8)
    X[0, 0] = X[1, 1] = 0.0                    # the outlier channels carry no activation
    L1 = O.loss(X, W, s, 8, True, clip=1.0)
    # unclipped: Delta = 200/15, every small value rounds to the zero level: L = sum of squares
    assert L1 == pytest.approx(1 + 1 + 0.25 + 0.25 + 0.0625, rel=1e-12)
    Lc = O.loss(X, W, s, 8, True, clip=0.01)  # range [-1, 1]: 15 fine steps over the small values
    assert Lc < 0.02 * L1
    codes, _, _ = O.quantize_groups(s[:, None] * W, 8, True, clip=0.01)
    assert codes[0, 0] == 15 and codes[1, 0] == 0   # clamped to the end levels
    grid = O.clip_grid(0.01, 12)
    L = O.clip_losses(X, W, s, grid, 8, True)
    b = O.select(L)
    assert b > 0 and L[b] <= L[0]
    # the same outliers on active channels: clipping them costs far more than it saves
    X2 = np.eye(8)
    assert O.loss(X2, W, s, 8, True, clip=0.01) > 100 * O.loss(X2, W, s, 8, True, clip=1.0)


def test_clip_grid_closed_form():
    g = O.clip_grid(0.5, 11)
    assert g.dtype == np.float32 and g[0] == 1.0 and g[-1] == np.float32(0.5)
    assert np.array_equal(g, np.float32([1 - 0.05 * j for j in range(11)]))
    assert np.all(np.diff(g) < 0)
    assert np.all(O.clip_grid(1.0, 4) == 1.0)


def test_clip_search_never_loses_to_the_unclipped_quantizer():
    rng = np.random.default_rng(34)
    X = _bf16_round(rng.standard_normal((64, 256)))
    W = rng.standard_normal((256, 16)) / 16
    W.reshape(-1)[rng.choice(W.size, 8, replace=False)] *= 10     # weight outliers
    W = _bf16_round(W)
    s = np.ones(256, dtype=np.float32)
    grid = O.clip_grid(0.5, 11)
    for zp in (True, False):
        L = O.clip_losses(X, W, s, grid, 128, zp)
        assert L[O.select(L)] <= L[0]
        assert L[0] == O.loss(X, W, s, 128, zp)
