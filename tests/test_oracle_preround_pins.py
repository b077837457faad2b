"""Pins of ``pre_round_values`` and ``near_tie``: the values the quantizer rounds, which choose
the elements that the GPU pack comparison may exempt as near-ties.

The quantizer of "AWQ 激活感知量化" section 4 rounds p/Delta to the nearest level (worked values
1.3 -> 1 and 1.8 -> 2); the asymmetric form ("大模型 AWQ 量化实战" section 2, ``zero_point``) also
rounds the zero -min/Delta.  The hand-computed groups below use steps that are powers of two,
so every pre-round value is exact and known in advance; they cover the asymmetric, symmetric and
clipped forms ("009. AWQ Integration", 关键设计 5), including a clipped group whose zero differs
from what the unclipped minimum would give with the clipped step.  A second test ties the
near-tie set to the rounding itself: moving an element by a relative 1e-9 changes its code only
where ``near_tie`` says it may.
"""
import numpy as np

from oracle import awq_oracle as O


def _col(*vals):
    return np.array(vals, dtype=np.float64)[:, None]


def test_asymmetric_group_by_hand():
    # range [-0.75, 3.0] -> Delta = 3.75/15 = 0.25 (exact); zero = 0.75/0.25 = 3
    P = _col(-0.75, 0.3, 1.5, 3.0, 0.125, -0.375, 0.0, 2.0)
    codes, delta, zero = O.quantize_groups(P, 8, True)
    assert delta[0, 0] == np.float32(0.25) and zero[0, 0] == 3
    t, tz = O.pre_round_values(P, delta, 8, True)
    assert np.array_equal(t[:, 0], [-3.0, 1.2, 6.0, 12.0, 0.5, -1.5, 0.0, 8.0])
    assert tz.shape == (1, 1) and tz[0, 0] == 3.0
    # the codes are rint(t) + zero with ties to even: 0.5 -> 0, -1.5 -> -2
    assert list(codes[:, 0]) == [0, 4, 9, 15, 3, 1, 3, 11]


def test_asymmetric_one_signed_group_by_hand():
    # all positive: the range is widened to include 0, so min = 0 and the zero is 0
    P = _col(0.5, 1.0, 1.875, 0.25)
    codes, delta, zero = O.quantize_groups(P, 4, True)
    assert delta[0, 0] == np.float32(0.125) and zero[0, 0] == 0
    t, tz = O.pre_round_values(P, delta, 4, True)
    assert np.array_equal(t[:, 0], [4.0, 8.0, 15.0, 2.0]) and tz[0, 0] == 0.0
    # all negative: max = 0, min = -1.875, the zero is 15
    P = -P
    codes, delta, zero = O.quantize_groups(P, 4, True)
    t, tz = O.pre_round_values(P, delta, 4, True)
    assert delta[0, 0] == np.float32(0.125) and zero[0, 0] == 15 and tz[0, 0] == 15.0
    assert np.array_equal(t[:, 0], [-4.0, -8.0, -15.0, -2.0])


def test_symmetric_group_by_hand():
    # max |p| = 1.75 -> Delta = 1.75/7 = 0.25; there is no zero to round (tz is 0)
    P = _col(1.75, -0.375, 0.125, 0.0, -1.75, 0.6, 1.0, -0.1)
    codes, delta, zero = O.quantize_groups(P, 8, False)
    assert delta[0, 0] == np.float32(0.25) and zero[0, 0] == 8
    t, tz = O.pre_round_values(P, delta, 8, False)
    assert np.array_equal(t[:, 0], [7.0, -1.5, 0.5, 0.0, -7.0, 2.4, 4.0, -0.4])
    assert np.array_equal(tz, np.zeros((1, 1)))


def test_clipped_group_by_hand():
    # asymmetric, clip 0.5: range [-0.375, 1.75] -> Delta = 2.125/15 is not exact, so take a
    # range whose clipped width is a power-of-two multiple of 15:
    # [-1.0, 2.75] -> clipped [-0.5, 1.375], width 1.875 -> Delta = 0.125, zero = 0.5/0.125 = 4.
    # Without the clip factor on the minimum, -min/Delta would be 8: the clipped zero differs.
    P = _col(-1.0, 2.75, 0.25, 1.0)
    codes, delta, zero = O.quantize_groups(P, 4, True, clip=0.5)
    assert delta[0, 0] == np.float32(0.125) and zero[0, 0] == 4
    t, tz = O.pre_round_values(P, delta, 4, True, clip=0.5)
    assert tz[0, 0] == 4.0
    assert np.array_equal(t[:, 0], [-8.0, 22.0, 2.0, 8.0])
    # the elements beyond the clipped range clamp to the end levels
    assert list(codes[:, 0]) == [0, 15, 6, 12]
    # the same group unclipped: Delta = 3.75/15 = 0.25, zero = 4 from -min/Delta = 4.0
    codes_u, delta_u, zero_u = O.quantize_groups(P, 4, True)
    t_u, tz_u = O.pre_round_values(P, delta_u, 4, True)
    assert delta_u[0, 0] == np.float32(0.25) and tz_u[0, 0] == 4.0
    assert np.array_equal(t_u[:, 0], [-4.0, 11.0, 1.0, 4.0])
    # symmetric clip 0.5: max |p| = 3.5 -> clipped 1.75 -> Delta 0.25
    Ps = _col(3.5, -0.625, 1.0, 0.0)
    _, ds, _ = O.quantize_groups(Ps, 4, False, clip=0.5)
    ts, tzs = O.pre_round_values(Ps, ds, 4, False, clip=0.5)
    assert ds[0, 0] == np.float32(0.25) and np.array_equal(ts[:, 0], [14.0, -2.5, 4.0, 0.0])


def test_multi_group_layout():
    # two groups of 4 rows and two columns: each (group, column) gets its own step and zero
    P = np.array([[-0.75, 1.75], [3.0, -0.375], [0.3, 0.125], [1.5, 0.0],
                  [0.5, -1.0], [1.0, 2.75], [1.875, 0.25], [0.25, 1.0]])
    _, delta, zero = O.quantize_groups(P, 4, True)
    t, tz = O.pre_round_values(P, delta, 4, True)
    assert t.shape == (8, 2) and tz.shape == (2, 2)
    assert np.array_equal(delta, np.array([[0.25, 0.14166666], [0.125, 0.25]], dtype=np.float32))
    assert tz[0, 0] == 3.0 and tz[1, 0] == 0.0 and tz[1, 1] == 4.0
    assert tz[0, 1] == 0.375 / float(np.float32(2.125 / 15))
    assert np.array_equal(t[4:, 0], [4.0, 8.0, 15.0, 2.0])
    assert t[0, 1] == 1.75 / float(np.float32(2.125 / 15))


def test_near_tie_flags():
    t = np.array([0.5, -1.5, 2.5 + 1e-6, 7.4999, 1.2, 0.0, 100.5 + 5e-4, 100.5 + 2e-3])
    assert list(O.near_tie(t)) == [True, True, True, False, False, False, True, False]


def _codes_after_nudge(P, g, zp, clip, rel):
    """Quantize P with every element that is not its group's range end moved by a relative
    ``rel``; the ends are left alone so Delta and the zero stay what they were."""
    K, N = P.shape
    G = P.reshape(K // g, g, N)
    ends = (G == G.max(axis=1, keepdims=True)) | (G == G.min(axis=1, keepdims=True))
    Q = np.where(ends, G, G * (1.0 + rel)).reshape(K, N)
    return O.quantize_groups(Q, g, zp, clip)


def test_near_ties_are_the_only_elements_a_nudge_can_flip():
    rng = np.random.default_rng(5)
    for zp in (True, False):
        for clip in (1.0, 0.75):
            g, K, N = 16, 64, 48
            # steps are powers of two and many elements sit exactly on a .5 boundary
            P = rng.standard_normal((K, N))
            Gv = P.reshape(K // g, g, N)
            Gv[:, 0, :] = 7.0 if not zp else 3.0
            Gv[:, 1, :] = -0.75 if zp else -1.0
            codes, delta, zero = O.quantize_groups(P, g, zp, clip)
            d = np.repeat(delta.astype(np.float64), g, axis=0)
            half = (np.floor(P / d) + 0.5) * d
            pick = rng.random((K, N)) < 0.3
            Gp = np.where(pick, half, P).reshape(K // g, g, N)
            Gp[:, :2, :] = P.reshape(K // g, g, N)[:, :2, :]
            P = Gp.reshape(K, N)
            codes, delta, zero = O.quantize_groups(P, g, zp, clip)
            t, tz = O.pre_round_values(P, delta, g, zp, clip)
            ties = O.near_tie(t)
            assert ties.sum() > 50
            for rel in (1e-9, -1e-9):
                c2, d2, z2 = _codes_after_nudge(P, g, zp, clip, rel)
                assert np.array_equal(d2, delta) and np.array_equal(z2, zero)
                flipped = c2 != codes
                assert flipped.any()
                assert not np.any(flipped & ~ties)
