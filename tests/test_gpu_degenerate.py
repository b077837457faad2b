"""GPU parity on the degenerate inputs the method defines, against the fp64 oracle.

* The smallest layers: one token, one quantization group (K = group size), eight output columns,
  a two-point alpha grid; a few tokens with one group of 64.
* Dead activation channels (all x of a channel zero: the statistic is floored at 1e-8 before the
  power, "AWQ (Activation-aware Weight Quantization)", 缩放因子优化的完整流程 step 3), a column
  whose weights are all zero and a zero group inside a column (the step of an all-zero group is 1,
  its codes the zero point).
* An all-zero weight matrix: every error tile is zero, every loss is exactly zero and the first
  alpha is kept ("量化推理算法 GPTQ / AWQ", 4.3: a loss replaces the best only when strictly
  smaller).

Each case runs stats -> search -> pack through the C ABI and is checked by the parity rules
(tests/gpu_util.check_layer), then the W4A16 product at M = 1 and M = T against the oracle's.
"""
import numpy as np
import pytest
import torch

from oracle import awq_oracle as O
from weight_only_int4_act_amd import inputs as I
from tests.gpu_util import check_layer, gpu_gemm, log, rel_fro

pytestmark = pytest.mark.gpu


def _products(L_X, gpu, g, label):
    T = L_X.shape[0]
    for M in sorted({1, T}):
        Xm = L_X[:M].contiguous()
        Y = gpu_gemm(Xm, gpu["q"])
        Yr = O.w4a16_ref(I.bf16_to_f64(Xm), gpu["s_best"], gpu["codes"], gpu["scales"], gpu["zeros"], g)
        assert np.all(np.isfinite(Y)), (label, M)
        if np.linalg.norm(Yr) == 0:
            # exact zeros in the reference: the product forms sum x' (128 + q) and subtracts
            # (128 + z) sum x' in float32, so only that cancellation's rounding may remain
            xs = np.abs(I.bf16_to_f64(Xm) / gpu["s_best"][None, :]).sum(axis=1, keepdims=True)
            assert np.all(np.abs(Y) <= 1e-4 * 128 * xs), (label, M, float(np.abs(Y).max()))
        else:
            err = rel_fro(Y, Yr)
            log(f"[degenerate] {label} M={M}: rel err {err:.2e}")
            assert err <= 2e-2, (label, M, err)


@pytest.mark.parametrize("T,K,N,g,zp,ng", [(1, 32, 8, 32, True, 2), (1, 32, 8, 32, False, 21),
                                           (3, 64, 8, 64, True, 21), (16, 128, 8, 128, False, 21)])
def test_smallest_layers(T, K, N, g, zp, ng):
    L = I.small(T, K, N, seed=50 + T + K, group_size=g, zero_point=zp)
    label = f"T={T} K={K} N={N} g={g} zp={zp} n_grid={ng}"
    gpu = check_layer(L.X, L.W, g, zp, ng, label)
    _products(L.X, gpu, g, label)


@pytest.mark.parametrize("zp", [True, False])
def test_dead_channels_and_zero_weight_groups(zp):
    L = I.small(200, 256, 32, seed=60, zero_point=zp)
    x = I.bf16_to_f64(L.X).copy()
    x[:, 5] = 0.0                 # one dead channel
    x[:, 100:110] = 0.0           # a run of dead channels
    w = I.bf16_to_f64(L.W).copy()
    w[:, 7] = 0.0                 # a column of zeros
    w[0:128, 3] = 0.0             # a zero group inside a column
    X = I.to_bf16(x.astype(np.float32))
    W = I.to_bf16(w.astype(np.float32))
    label = f"dead channels, zero groups, zp={zp}"
    gpu = check_layer(X, W, 128, zp, 21, label)
    assert np.all(gpu["mean_abs"][[5] + list(range(100, 110))] == 0.0)
    assert gpu["scales"][0, 3] == 1.0 and gpu["scales"][1, 7] == 1.0   # an all-zero group's step
    _products(X, gpu, 128, label)


def test_all_zero_weights_keep_the_first_alpha():
    L = I.small(64, 128, 16, seed=70)
    W = torch.zeros_like(L.W)
    gpu = check_layer(L.X, W, 128, True, 21, "all-zero W")
    assert np.all(gpu["losses"] == 0.0)
    assert gpu["best"] == 0
    _products(L.X, gpu, 128, "all-zero W")
