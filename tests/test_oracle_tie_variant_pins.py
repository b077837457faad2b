"""Pins of oracle.loss_tie_variants: the search loss under every admissible rounding of near-tie
elements ("AWQ 激活感知量化", section 4: round to the nearest level; at a .5 tie both neighbours
are equally near).  Hand-computed cases with exact ties, a tied element at the end of the code
range, a clipped range, ties in two columns, and inputs without ties; and, on a small layer with
ties in several columns, the per-column enumeration against a brute-force recomputation of the
whole loss for every choice.
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


def test_ties_in_two_columns_combine_column_losses():
    # column 0: ties at rows 1 and 2 as in the first case (column loss 1, 0, 0, 1); column 1
    # (Delta = 1): p = 1.5 at row 3, a tie between 1 and 2 (error -+0.5, column loss 0.25 either
    # way).  The token reads rows 1, 2 and 3.  First tied column innermost.
    W = np.zeros((8, 2))
    W[:, 0] = [7.0, 2.5, 0.5, 0, 0, 0, 0, 0]
    W[:, 1] = [7.0, 0, 0, 1.5, 0, 0, 0, 0]
    X = np.zeros((1, 8))
    X[0, 1] = X[0, 2] = X[0, 3] = 1.0
    V = O.loss_tie_variants(X, W, np.ones(8), 8, False)
    assert V.tolist() == [1.25, 0.25, 0.25, 1.25, 1.25, 0.25, 0.25, 1.25]
    assert V[0] == O.loss(X, W, np.ones(8), 8, False)


def test_per_column_enumeration_matches_brute_force():
    # integer weights with Delta = 1 (max |p| = 7 in every group) and ten half-integers, exact
    # ties, spread over the columns; every choice recomputed as the whole layer's loss
    rng = np.random.default_rng(11)
    K, N, g = 16, 4, 8
    W = rng.integers(-6, 7, size=(K, N)).astype(np.float64)
    W[0::g, :] = 7.0
    rows = [1, 2, 3, 5, 9, 10, 12, 6, 14, 11]
    cols = [0, 0, 1, 1, 2, 2, 3, 3, 0, 1]
    for k, c in zip(rows, cols):
        W[k, c] += 0.5
    X = rng.standard_normal((5, K))
    s = np.ones(K)
    V = O.loss_tie_variants(X, W, s, g, False)
    codes, delta, zero = O.quantize_groups(W, g, False)
    t, _ = O.pre_round_values(W, delta, g, False)
    tie = np.argwhere(O.near_tie(t))
    assert len(tie) == 10 and len(set(tie[:, 1].tolist())) == 4
    d = np.repeat(delta.astype(np.float64), g, axis=0)
    level = codes.astype(np.float64) - np.repeat(zero.astype(np.float64), g, axis=0)
    brute = []
    for mask in range(2 ** len(tie)):
        lv = level.copy()
        for b, (k, c) in enumerate(tie):
            if (mask >> b) & 1:
                lv[k, c] = 2.0 * np.floor(t[k, c]) + 1.0 - lv[k, c]   # the other neighbour
        Y = X @ (lv * d - W)
        brute.append(float(np.sum(Y * Y)))
    assert len(V) == len(brute)
    assert np.allclose(np.sort(V), np.sort(brute), rtol=1e-12, atol=0.0)
    assert V[0] == O.loss(X, W, s, g, False)


def test_scaled_tie_with_a_cross_term():
    # as above (s = 2 on row 1, p = 1.5 a tie: error +0.25 or -0.25 in W units) plus row 2 with
    # p = w = 0.25 (level 0, error -0.25); the token reads row 1 four times and row 2 once:
    # X E = 4 (+-0.25) - 0.25, so L = 0.5625 for the quantizer's rounding and 1.5625 for the other
    W = np.zeros((8, 1))
    W[:, 0] = [7.0, 0.75, 0.25, 0, 0, 0, 0, 0]
    s = np.ones(8)
    s[1] = 2.0
    X = np.zeros((1, 8))
    X[0, 1] = 4.0
    X[0, 2] = 1.0
    assert O.loss_tie_variants(X, W, s, 8, False).tolist() == [0.5625, 1.5625]
