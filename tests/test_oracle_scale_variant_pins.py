"""Pins of the oracle's statistic and scale-family variants (CPU only).

* max |x| per input channel, the alternative the first page names next to the mean
  ("AWQ (Activation-aware Weight Quantization)", 重要通道识别的统计依据);
* the closed form s_i = (E|X_i|)^alpha / mean_j |W_ij| ("AWQ 激活感知量化", section 3);
* the normalization of the scale vector by its maximum (the same page's Python 演示).
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


def test_act_max_brute_force_and_accumulation():
    rng = np.random.default_rng(41)
    X = _bf16_round(rng.standard_normal((37, 11)) * rng.lognormal(0, 2, 11))
    X[:, 3] = 0.0
    X[5, 4] = -1000.0                          # the largest magnitude may be negative
    m = O.act_max(X)
    for k in range(11):
        best = 0.0
        for t in range(37):
            best = max(best, abs(float(X[t, k])))
        assert m[k] == np.float32(best)
    assert m[3] == 0.0 and m[4] == 1000.0
    assert np.array_equal(O.act_max(X[20:], O.act_max(X[:20])), m)    # accumulation by max


def test_weight_mean_abs_exact_rational():
    rng = np.random.default_rng(42)
    W = _bf16_round(rng.standard_normal((6, 13)) * 0.03)
    wm = O.weight_mean_abs(W)
    for k in range(6):
        q = sum(Fraction(abs(float(v))) for v in W[k]) / 13
        assert wm[k] == np.float32(float(q))


def test_scale_table_variant_closed_forms():
    m = np.float32([0.0, 1e-9, 0.25, 1.0, 4.0, 100.0])
    wm = np.float32([0.5, 0.02, 0.0, 0.125, 2.0, 0.01])
    S = O.scale_table_ex(m, 21, w_mean=wm)
    for k in range(6):
        mk, wk = max(float(m[k]), 1e-8), max(float(wm[k]), 1e-8)
        assert S[0, k] == np.float32(1.0 / wk)                 # alpha = 0: 1 / mean|W|
        assert S[20, k] == np.float32(mk / wk)                 # alpha = 1: m / mean|W|
    assert np.array_equal(O.scale_table_ex(m, 21), O.scale_table(m, 21))   # no denominator, no norm
    # the page's reading of the ratio: larger activation or smaller weight -> larger scale
    a = O.scale_table_ex(np.float32([1.0, 2.0]), 21, w_mean=np.float32([1.0, 1.0]))
    b = O.scale_table_ex(np.float32([1.0, 1.0]), 21, w_mean=np.float32([1.0, 0.5]))
    assert np.all(a[1:, 1] > a[1:, 0]) and np.all(b[:, 1] > b[:, 0])


@pytest.mark.parametrize("w_mean", [False, True])
def test_normalized_rows(w_mean):
    rng = np.random.default_rng(43)
    m = rng.lognormal(0, 1.5, 64).astype(np.float32)
    wm = rng.lognormal(-3, 0.3, 64).astype(np.float32) if w_mean else None
    S = O.scale_table_ex(m, 21, w_mean=wm)
    Sn = O.scale_table_ex(m, 21, w_mean=wm, normalize=True)
    assert np.all(Sn.max(axis=1) == 1.0)                        # the row maximum maps to exactly 1
    r = Sn.astype(np.float64) / S.astype(np.float64)
    assert np.all(np.abs(r / r[:, :1] - 1.0) <= 2.5e-7)          # one factor per row (two roundings)


def test_normalization_leaves_the_losses():
    # a global factor on s moves Delta with it and leaves codes and E (up to Delta's rounding)
    rng = np.random.default_rng(44)
    X = _bf16_round(rng.standard_normal((64, 256)))
    X[:, 7] *= 40.0
    W = _bf16_round(rng.standard_normal((256, 24)) * 0.02)
    stat = O.act_stats(X)[1]
    wm = O.weight_mean_abs(W)
    for zp in (True, False):
        L = O.losses(X, W, O.scale_table_ex(stat, 11, w_mean=wm), 128, zp)
        Ln = O.losses(X, W, O.scale_table_ex(stat, 11, w_mean=wm, normalize=True), 128, zp)
        assert np.all(np.abs(Ln - L) <= 1e-5 * L)
