"""Parity of the clipped quantizer and the clip-ratio search (HIP path through the C ABI) with
the fp64 oracle.

Clipping is the optional min-max clip_ratio of the quantizer configuration ("009. AWQ
Integration", 架构 and 关键设计 5); the clip search scores the ratios c_j = 1 - (1 - c_min) j/(n-1)
at fixed scales with the loss of "AWQ (Activation-aware Weight Quantization)", 缩放因子优化的完整流程
step 4c.  Bars as for the alpha search: every L(c_j) within 1e-2 relative of the oracle, the
chosen ratio's oracle loss within 1e-2 of the oracle minimum, the returned ratio equal to the
grid's float32 value; pack at a clip ratio bit-exact except elements whose pre-round value lies
within 1e-5 relative of a .5 boundary.
"""
import numpy as np
import pytest
import torch

from oracle import awq_oracle as O
from weight_only_int4_act_amd import inputs as I
from tests.gpu_util import awq, log

pytestmark = pytest.mark.gpu

L_TOL = 1e-2

CASES = {
    # name: (T, K, N, group_size, zero_point, seed), weights with 0.5% outliers x10
    "zp128": (300, 384, 40, 128, True, 21),
    "sym64": (1030, 256, 48, 64, False, 22),
    "zp32": (100, 192, 24, 32, True, 23),
    "sym128_rows640": (1250, 512, 72, 128, False, 24),
}


def _gpu_clip_search(X, W, s, g, zp, n, clip_min):
    A = awq()
    dev = torch.device("cuda:0")
    Xd, Wd, sd = X.to(dev), W.to(dev), torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32)).to(dev)
    T, K = X.shape
    N = W.shape[1]
    cfg = A.qconfig(g, zp, n)
    ws = A.workspace(A.awq_search_workspace_size(T, K, N, cfg), dev)
    losses = torch.empty(n, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    cbest = torch.empty(1, dtype=torch.float32, device=dev)
    A.awq_clip_search(Xd, Wd, sd, cfg, clip_min, ws, losses, best, cbest)
    torch.cuda.synchronize()
    return losses.cpu().numpy(), int(best.item()), float(cbest.item())


def _gpu_pack(W, s, g, zp, clip):
    A = awq()
    dev = torch.device("cuda:0")
    K, N = W.shape
    cfg = A.qconfig(g, zp, 21, clip_ratio=clip)
    codes = torch.empty((K // 8, N), dtype=torch.int32, device=dev)
    scales = torch.empty((K // g, N), dtype=torch.float32, device=dev)
    zeros = torch.empty((K // g, N), dtype=torch.uint8, device=dev)
    A.awq_pack(W.to(dev), torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32)).to(dev), cfg, codes,
               scales, zeros)
    torch.cuda.synchronize()
    return codes.cpu().numpy().view(np.uint32), scales.cpu().numpy(), zeros.cpu().numpy()


def _check_clip_search(name, X, W, s, g, zp, n, clip_min):
    X64, W64 = I.bf16_to_f64(X), I.bf16_to_f64(W)
    Lg, b, cb = _gpu_clip_search(X, W, s, g, zp, n, clip_min)
    grid = O.clip_grid(clip_min, n)
    Lo = O.clip_losses(X64, W64, s, grid, g, zp)
    rel = np.abs(Lg - Lo) / Lo
    log(f"[clip] {name}: max rel loss err {rel.max():.2e}; c* gpu {grid[b]} oracle {grid[O.select(Lo)]}; "
        f"L(1)/L(c*) = {Lo[0] / Lo[b]:.4f}")
    assert np.all(rel <= L_TOL)
    assert Lo[b] <= (1 + L_TOL) * Lo.min()
    assert np.float32(cb) == grid[b]
    return grid[b]


def _check_pack(name, W, s, g, zp, clip):
    W64 = I.bf16_to_f64(W)
    codes, scales, zeros = _gpu_pack(W, s, g, zp, clip)
    w, d, z = O.pack(W64, s, g, zp, clip=clip)
    P = np.asarray(s, dtype=np.float64)[:, None] * W64
    t, tz = O.pre_round_values(P, d, g, zp, clip=clip)
    ties = O.near_tie(t) | np.repeat(O.near_tie(tz), g, axis=0)
    bad = O.unpack_nibbles(w) != O.unpack_nibbles(codes)
    log(f"[clip] {name}: pack at c={clip}: mismatches {int(bad.sum())}, near-ties {int(ties.sum())}")
    assert not np.any(bad & ~ties)
    assert np.array_equal(scales, d) and np.array_equal(zeros, z)


@pytest.mark.parametrize("name", list(CASES))
def test_clip_search_and_clipped_pack(name):
    T, K, N, g, zp, seed = CASES[name]
    L = I.small(T, K, N, seed=seed, group_size=g, zero_point=zp, w_outlier_frac=0.005)
    s = I.scale_vector(K, seed=seed, sigma=0.5)
    cstar = _check_clip_search(name, L.X, L.W, s, g, zp, 11, 0.5)
    for c in sorted({float(cstar), 0.8}):
        _check_pack(name, L.W, s, g, zp, c)


def test_clip_grid_edges():
    # clip_min = 1: every ratio is 1, all losses equal the unclipped loss, the first wins
    L = I.small(64, 128, 16, seed=25, w_outlier_frac=0.01)
    s = np.ones(128, dtype=np.float32)
    Lg, b, cb = _gpu_clip_search(L.X, L.W, s, 128, True, 4, 1.0)
    assert b == 0 and cb == 1.0 and np.all(Lg == Lg[0])
    Lo = O.loss(I.bf16_to_f64(L.X), I.bf16_to_f64(L.W), s, 128, True)
    assert abs(Lg[0] - Lo) <= L_TOL * Lo
    # two points: the unclipped quantizer and c_min
    _check_clip_search("two_points", L.X, L.W, s, 128, True, 2, 0.3)


def test_alpha_search_with_a_clip_ratio():
    from tests.gpu_util import gpu_layer
    A = awq()
    L = I.small(700, 256, 40, seed=26, w_outlier_frac=0.005)
    X64, W64 = I.bf16_to_f64(L.X), I.bf16_to_f64(L.W)
    dev = torch.device("cuda:0")
    cfg = A.qconfig(128, True, 21, clip_ratio=0.85)
    r = A.run_layer(L.X.to(dev), L.W.to(dev), cfg)
    torch.cuda.synchronize()
    Lg = r["losses"].cpu().numpy()
    b = int(r["best"].item())
    S = O.scale_table(O.act_stats(X64)[1], 21)
    Lo = O.losses(X64, W64, S, 128, True, clip=0.85)
    rel = np.abs(Lg - Lo) / Lo
    log(f"[clip] alpha search at c=0.85: max rel loss err {rel.max():.2e}, alpha* gpu {b} oracle {O.select(Lo)}")
    assert np.all(rel <= L_TOL) and Lo[b] <= (1 + L_TOL) * Lo.min()
    q = r["q"]   # run_layer packs with the same configuration
    w, d, z = O.pack(W64, S[b], 128, True, clip=0.85)
    assert np.array_equal(q.scales.cpu().numpy(), d) and np.array_equal(q.zeros.cpu().numpy(), z)


def test_clip_search_full_size_benchmarked_layer():
    # the 4096x4096 layer with 8192 tokens, at the s* of the GPU alpha search, 11 ratios
    from tests.gpu_util import gpu_layer
    L = I.make_config("c2", seed=0).layers[0]
    gpu = gpu_layer(L.X, L.W, 128, True, 21)
    _check_clip_search("c2", L.X, L.W, gpu["s_best"], 128, True, 11, 0.5)


def test_clip_search_full_k_and_n_with_weight_outliers():
    # c4's full 5120 x 13824 weights (0.1% outliers x10, symmetric g=64) at 512 tokens
    L = I.make_config("c4", seed=0).layers[0]
    X = L.X[:512].contiguous()
    s = np.ones(L.W.shape[0], dtype=np.float32)
    cstar = _check_clip_search("c4", X, L.W, s, 64, False, 11, 0.5)
    _check_pack("c4", L.W, s, 64, False, float(cstar))
