"""Pins of the oracle's power-of-two greedy search (CPU only).

"009. AWQ Integration", 关键设计 1-3: per group of input channels, a coordinate greedy over
power-of-two scale candidates around 1 (20 by default, 3 passes), each scored with the
activation-weighted reconstruction error of the whole group under the packing quantizer; its
Consequences claim about 2.5x lower activation-weighted error than plain rounding on inputs with
salient channels and no loss on uniform ones.
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


def _exact_group_error(W_g, m_g, s_g, zp):
    """sum_n sum_i (m_i (What_in - w_in))^2 in rationals, with Delta, zero and codes found by
    enumerating the 16 levels (nearest level, ties to the even level)."""
    g, N = W_g.shape
    tot = Fraction(0)
    for n in range(N):
        p = [Fraction(float(s_g[i])) * Fraction(float(W_g[i, n])) for i in range(g)]
        if zp:
            hi, lo = max(max(p), 0), min(min(p), 0)
            d = Fraction(float(np.float32(float(hi - lo) / 15.0))) or Fraction(1)
            z = min(max(_rne(-lo / d), 0), 15)
            levels = [q - z for q in range(16)]
        else:
            d = Fraction(float(np.float32(float(max(abs(v) for v in p)) / 7.0))) or Fraction(1)
            levels = list(range(-7, 8))
        for i in range(g):
            lv = min(levels, key=lambda L: (abs(p[i] / d - L), L % 2))
            e = Fraction(float(m_g[i])) * (lv * d / Fraction(float(s_g[i])) - Fraction(float(W_g[i, n])))
            tot += e * e
    return tot


def _rne(q: Fraction) -> int:
    f = q.numerator // q.denominator
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def test_candidates():
    c = O.pow2_candidates(20)
    assert c[0] == 2.0 ** -10 and c[-1] == 2.0 ** 9 and c[10] == 1.0 and len(c) == 20
    assert np.all(c[1:] == 2 * c[:-1])
    assert list(O.pow2_candidates(4)) == [0.25, 0.5, 1.0, 2.0]


def test_worked_example_by_hand():
    # symmetric, one group of 2 channels, one column, candidates 1/4, 1/2, 1, 2, one pass.
    # w = (7/8, 5/16), only channel 1 carries activation (m = (0, 1)).
    # s = (1, 1): Delta = 7/8 / 7 = 1/8, 5/16 / (1/8) = 2.5 rounds to the even level 2,
    #   What_1 = 1/4, error (1/16)^2 = 1/256.
    # channel 0: s_0 = 1/2 gives Delta = 7/16 / 7 = 1/16 and w_1 = 5 Delta exactly (error 0);
    #   s_0 = 1/4 makes w_1 the maximum, Delta = fl32(5/112) is inexact and the error is a tiny
    #   positive number; s_0 = 2 gives Delta = 1/4, level 1, error 1/256.  Best: s_0 = 1/2.
    # channel 1 (now exact at s_1 = 1): nothing is strictly better, it stays.
    W = np.array([[0.875], [0.3125]])
    m = np.array([0.0, 1.0])
    tr = []
    r = O.greedy_search(W, m, 2, False, n_cand=4, passes=1, trace=tr)
    assert list(r["idx"]) == [1, 2] and list(r["s"]) == [0.5, 1.0]
    assert r["err_rtn"][0] == 1.0 / 256 and r["err"][0] == 0.0
    e0 = tr[0][3]
    assert e0[2] == 1.0 / 256 and e0[3] == 1.0 / 256 and e0[1] == 0.0 and 0.0 < e0[0] < 1e-15
    e1 = tr[1][3]
    assert e1[2] == 0.0 and e1[0] == e1[1] == 1.0 / 256 and e1[3] > 0.0


@pytest.mark.parametrize("zp", [True, False])
def test_group_error_exact_rational(zp):
    rng = np.random.default_rng(71)
    W = _bf16_round(rng.standard_normal((8, 5)) * 0.1)
    m = np.float32(rng.lognormal(0, 1, 8))
    s = O.pow2_candidates(20)[rng.integers(6, 14, 8)]
    Wg = W.copy()
    Wg[2, 1] = 0.0
    e = O.group_error(Wg, m, s, zp)
    q = _exact_group_error(Wg, m, s, zp)
    assert abs(e - float(q)) <= 1e-13 * float(q)


@pytest.mark.parametrize("zp", [True, False])
def test_every_decision_is_the_exact_best(zp):
    # tiny layer: each decision's candidate errors recomputed in rationals from the state the
    # decision saw; the chosen index is the current one unless a candidate is strictly better,
    # and then the first (ascending) of the strictly best ones
    rng = np.random.default_rng(72)
    K, N, g, n = 8, 3, 4, 5
    W = _bf16_round(rng.standard_normal((K, N)) * 0.05)
    m = np.float32(rng.lognormal(0, 1.5, K))
    tr = []
    r = O.greedy_search(W, m, g, zp, n_cand=n, passes=2, trace=tr)
    cand = O.pow2_candidates(n)
    idx = np.full(K, n // 2)
    for (j, p, k, errs, best) in tr:
        rows = slice(j * g, (j + 1) * g)
        ex = []
        for c in range(n):
            sg = cand[idx[rows]]
            sg[k - j * g] = cand[c]
            ex.append(_exact_group_error(W[rows], m[rows], sg, zp))
        for c in range(n):
            assert abs(errs[c] - float(ex[c])) <= 1e-12 * max(float(ex[c]), 1e-300)
        cur = idx[k]
        lo = min(ex)
        want = cur if ex[cur] == lo else min(c for c in range(n) if ex[c] == lo)
        assert best == want
        idx[k] = best
    assert np.array_equal(idx, r["idx"])


@pytest.mark.parametrize("zp", [True, False])
def test_never_worse_than_rounding_and_monotone(zp):
    rng = np.random.default_rng(73)
    W = _bf16_round(rng.standard_normal((256, 16)) * 0.02)
    m = np.float32(rng.lognormal(0, 1, 256))
    tr = []
    r = O.greedy_search(W, m, 128, zp, trace=tr)
    assert np.all(r["err"] <= r["err_rtn"])
    for j in range(2):
        chosen = [t[3][t[4]] for t in tr if t[0] == j]
        assert all(b <= a for a, b in zip(chosen, chosen[1:]))
        assert chosen[-1] == r["err"][j]


def test_power_of_two_rescaling_is_exact():
    rng = np.random.default_rng(74)
    W = _bf16_round(rng.standard_normal((128, 12)) * 0.02)
    m = np.float32(rng.lognormal(0, 1, 128))
    m[[5, 77]] *= 50
    for zp in (True, False):
        a = O.greedy_search(W, m, 64, zp, passes=2)
        b = O.greedy_search(8.0 * W, m, 64, zp, passes=2)       # every p, Delta, error x 8
        c = O.greedy_search(W, 0.25 * m, 64, zp, passes=2)      # every weighted error x 1/4
        assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["idx"], c["idx"])
        assert np.array_equal(b["err"], 64.0 * a["err"]) and np.array_equal(c["err"], a["err"] / 16.0)


def test_converged_state_is_coordinatewise_optimal():
    # enough passes that the last one changes nothing: no single channel's candidate is better
    rng = np.random.default_rng(75)
    W = _bf16_round(rng.standard_normal((8, 4)) * 0.05)
    m = np.float32(rng.lognormal(0, 1, 8))
    tr = []
    r = O.greedy_search(W, m, 8, True, n_cand=6, passes=6, trace=tr)
    last = [t for t in tr if t[1] == 5]
    prev = [t for t in tr if t[1] == 4]
    assert [t[4] for t in last] == [t[4] for t in prev]          # the last pass moved nothing
    cand = O.pow2_candidates(6)
    base = _exact_group_error(W, m, cand[r["idx"]], True)
    for k in range(8):
        for c in range(6):
            sg = cand[r["idx"]].copy()
            sg[k] = cand[c]
            assert _exact_group_error(W, m, sg, True) >= base


def test_salient_channels_and_uniform_inputs():
    # the design record's behaviour: far lower activation-weighted error than rounding when a
    # few channels carry large activations, and no loss when activations are uniform
    rng = np.random.default_rng(76)
    K, N = 256, 32
    W = _bf16_round(rng.standard_normal((K, N)) * 0.02)
    m = np.ones(K, dtype=np.float32)
    sal = rng.choice(K, 3, replace=False)
    m[sal] = 50.0
    r = O.greedy_search(W, m, 128, True)
    ratio = r["err_rtn"].sum() / r["err"].sum()
    assert ratio >= 2.0
    assert np.all(r["s"][sal] > 1.0)                              # salient weights are enlarged
    u = O.greedy_search(W, np.ones(K, dtype=np.float32), 128, True)
    assert np.all(u["err"] <= u["err_rtn"])
