"""Pins of the oracle's joint search over projections that share one input X (CPU only).

Projections that read the same activations (q, k and v; gate and up) share one scale vector
once 1/s is applied to X a single time ("009. AWQ Integration", 关键设计 4, and the fused
``attn.qkv`` layer of its usage).  Their joint loss is the squared error over all outputs.
"""
from fractions import Fraction

import numpy as np

from oracle import awq_oracle as O


def _bf16_round(a):
    a = np.asarray(a, dtype=np.float32)
    b = a.view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _case(seed, T=48, K=256, Ns=(24, 8, 40)):
    rng = np.random.default_rng(seed)
    X = _bf16_round(rng.standard_normal((T, K)))
    X[:, rng.choice(K, 3, replace=False)] *= 30.0
    Ws = [_bf16_round(rng.standard_normal((K, n)) / np.sqrt(K)) for n in Ns]
    return X, Ws


def test_joint_is_the_loss_of_the_fused_layer():
    # the quantizer works per output column and ||.||^2 sums over columns, so the joint loss
    # equals the loss of the one layer whose columns are all projections' columns
    X, Ws = _case(51)
    S = O.scale_table(O.act_stats(X)[1], 9)
    for zp in (True, False):
        joint, each = O.losses_multi(X, Ws, S, 128, zp)
        fused = O.losses(X, np.hstack(Ws), S, 128, zp)
        assert each.shape == (3, 9)
        assert np.all(np.abs(joint - fused) <= 1e-12 * fused)
        for j, W in enumerate(Ws):
            assert np.array_equal(each[j], O.losses(X, W, S, 128, zp))


def test_joint_exact_rational_two_projections():
    rng = np.random.default_rng(52)
    X = _bf16_round(rng.standard_normal((5, 8)))
    W1 = _bf16_round(rng.standard_normal((8, 3)))
    W2 = _bf16_round(rng.standard_normal((8, 2)) * 4)
    S = np.float32([[1, 2, 0.5, 1, 4, 1, 0.25, 1], [1, 1, 1, 1, 1, 1, 1, 1]])
    joint, each = O.losses_multi(X, [W1, W2], S, 4, True)
    for i in range(2):
        total = Fraction(0)
        for W in (W1, W2):
            P = S[i].astype(np.float64)[:, None] * W
            codes, delta, zero = O.quantize_groups(P, 4, True)
            for t in range(5):
                for n in range(W.shape[1]):
                    y = sum(Fraction(float(X[t, k])) *
                            ((int(codes[k, n]) - int(zero[k // 4, n])) * Fraction(float(delta[k // 4, n]))
                             / Fraction(float(S[i, k])) - Fraction(float(W[k, n]))) for k in range(8))
                    total += y * y
        assert abs(joint[i] - float(total)) <= 1e-12 * float(total)


def test_power_of_two_copy_scales_the_loss_exactly():
    # W2 = 4 W1: Delta and every product scale by 4 exactly, the codes do not change
    X, (W1,) = _case(53, Ns=(24,))
    S = O.scale_table(O.act_stats(X)[1], 11)
    for zp in (True, False):
        joint, each = O.losses_multi(X, [W1, 4.0 * W1], S, 64, zp)
        assert np.array_equal(each[1], 16.0 * each[0])
        # every projection has its first minimum at the same alpha: so does the sum
        assert O.select(joint) == O.select(each[0]) == O.select(each[1])


def test_zero_projection_adds_nothing():
    # a projection of zeros quantizes exactly (the padding columns of a column tile)
    X, Ws = _case(54, Ns=(16, 16))
    S = O.scale_table(O.act_stats(X)[1], 5)
    for zp in (True, False):
        joint, each = O.losses_multi(X, Ws + [np.zeros((256, 8))], S, 128, zp)
        assert np.all(each[2] == 0.0)
        j2, _ = O.losses_multi(X, Ws, S, 128, zp)
        assert np.array_equal(joint, j2)

