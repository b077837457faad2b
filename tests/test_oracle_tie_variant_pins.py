"""Pins of oracle.loss_tie_variants: the search loss under every admissible rounding of near-tie
elements ("AWQ 激活感知量化", section 4: round to the nearest level; at a .5 tie both neighbours
are equally near).  Hand-computed cases with exact ties, a tied element at the end of the code
range, a clipped range, and inputs without ties.
"""
import numpy as np

from oracle import awq_oracle as O


def test_symmetric_two_ties_hand_values():
    # one group of 8, s = 1, max |p| = 7 so Delta = 1; p/Delta = 2.5 and 0.5 are ties, rounded
    # to 2 and 0 (half to even): errors -0.5, -0.5.  One token reads exactly those two channels:
    # X E = -1 (L = 1); flipping one tie gives 0, flipping both gives +1 (L = 1)
    W = np.zeros((8, 1))
    W[:, 0] = [7.0, 2.5, 0.5, 0, 0, 0, 0, 0]
    X = np.zeros((1, 8))
    X[0, 1] = X[0, 2] = 1.0
    s = np.ones(8)
    V = O.loss_tie_variants(X, W, s, 8, False)
    assert V.tolist() == [1.0, 0.0, 0.0, 1.0]
    assert V[0] == O.loss(X, W, s, 8, False)


def test_asymmetric_tie_at_the_end_of_the_code_range():
    # range [-3.5, 11.5]: Delta = 1, zero = rne(3.5) = 4; p = 11.5 rounds to level 12, code 16,
    # clamped to 15 (level 11, error -0.5); p = -3.5 rounds to level -4 (error -0.5).  The other
    # rounding of the top element is level 12, one step beyond the code range (error +0.5)
    W = np.zeros((8, 1))
    W[:, 0] = [11.5, -3.5, 0, 0, 0, 0, 0, 0]
    X = np.zeros((1, 8))
    X[0, 0] = X[0, 1] = 1.0
    s = np.ones(8)
    codes, delta, zero = O.quantize_groups(W, 8, True)
    assert delta[0, 0] == 1.0 and zero[0, 0] == 4 and codes[0, 0] == 15 and codes[1, 0] == 0
    V = O.loss_tie_variants(X, W, s, 8, True)
    assert V.tolist() == [1.0, 0.0, 0.0, 1.0]
    assert V[0] == O.loss(X, W, s, 8, True)


def test_clipped_range_clamps_both_roundings():
    # clip 0.5: range [-1.75, 5.75], Delta = 0.5, zero = 4; p = 10.25 gives p/Delta = 20.5, a tie
    # beyond the clipped range, whose neighbours 20 and 21 both clamp to level 11: one loss
    W = np.zeros((8, 1))
    W[:, 0] = [11.5, -3.5, 10.25, 0, 0, 0, 0, 0]
    X = np.ones((2, 8))
    X[1] = np.arange(8)
    s = np.ones(8)
    V = O.loss_tie_variants(X, W, s, 8, True, clip=0.5)
    assert len(V) == 2 and V[0] == V[1] == O.loss(X, W, s, 8, True, clip=0.5)


def test_no_ties_means_one_variant_equal_to_the_loss():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((16, 64))
    W = rng.standard_normal((64, 12)) * 0.1
    s = np.exp(0.3 * rng.standard_normal(64))
    for zp in (True, False):
        V = O.loss_tie_variants(X, W, s, 32, zp, rel=1e-12)
        assert V.tolist() == [O.loss(X, W, s, 32, zp)]


def test_scaled_tie_flips_the_sign_of_the_unscaled_error():
    # s = 2 on the tied channel: p = 2 w; with max |p| = 7 (Delta = 1) and p = 1.5 (w = 0.75) the
    # tie rounds to 2 (error (2 - 1.5)/2 = +0.25 in W units) or 1 (-0.25): X E = +-0.25 * x
    W = np.zeros((8, 1))
    W[:, 0] = [7.0, 0.75, 0, 0, 0, 0, 0, 0]
    s = np.ones(8)
    s[1] = 2.0
    X = np.zeros((1, 8))
    X[0, 1] = 4.0
    V = O.loss_tie_variants(X, W, s, 8, False)
    assert sorted(V.tolist()) == [1.0, 1.0]   # (+-0.25 * 4)^2
    X[0, 0] = 1.0                              # add the max channel (error 0): still +-1
    assert sorted(O.loss_tie_variants(X, W, s, 8, False).tolist()) == [1.0, 1.0]
    X[0, 1] = 0.0
    X[0, 2] = 1.0
    assert O.loss_tie_variants(X, W, s, 8, False).tolist() == [0.0, 0.0]
