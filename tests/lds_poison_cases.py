"""Parity cases run against the LDS-poison debug build of libawq (child process of
tests/test_gpu_lds_poison.py; AWQ_LIBRARY names the library).

In that build every pipelined LDS buffer (the search's E tiles and staging ring, the W4A16 products'
staged x' and cross-wavefront sums) is filled with NaN between its last reader and its next writer,
and every other floating-point LDS array (statistic, packing, greedy and reduction kernels) at
kernel start,
so a read that a missing wait or barrier lets run early yields NaN instead of stale but plausible
data.  Each case is checked as the main parity tests check it: search losses within 1e-2 of the
fp64 oracle ("AWQ (Activation-aware Weight Quantization)", 缩放因子优化的完整流程 steps 3-6), the
chosen scale row, packed steps and zeros bit-exact and codes bit-exact outside near-ties, and the
W4A16 product within 2e-2 (Frobenius) of the oracle's (推理时的等效实现); the clip-ratio and joint
multi-projection searches likewise, and the power-of-two greedy's choices bit for bit ("009. AWQ
Integration", 关键设计 1-3).  Prints one line per case; exits non-zero on the first failure.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from oracle import awq_oracle as O  # noqa: E402
from weight_only_int4_act_amd import inputs as I  # noqa: E402
from tests.gpu_util import awq, gpu_gemm, log, rel_fro  # noqa: E402
from tests.gpu_util import check_layer as check_layer_vs_oracle  # noqa: E402


def check_layer(L, g, zp, ng, label):
    gpu = check_layer_vs_oracle(L.X, L.W, g, zp, ng, label)
    log(f"[poison] search {label}: ok")
    return gpu


def check_gemm(L, gpu, g, Ms, label):
    for M in Ms:
        Xm = L.X[:M].contiguous()
        Y = gpu_gemm(Xm, gpu["q"])
        assert np.all(np.isfinite(Y)), (label, M)
        Yr = O.w4a16_ref(I.bf16_to_f64(Xm), gpu["s_best"], gpu["codes"], gpu["scales"], gpu["zeros"], g)
        err = rel_fro(Y, Yr)
        assert err <= 2e-2, (label, M, err)
        log(f"[poison] gemm {label} M={M}: rel err {err:.2e}: ok")


def check_packed_gemm(M, K, N, g, zp, seed):
    """A W4A16 product on weights packed by the library at random scales (no search)."""
    A = awq()
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(seed)
    W = torch.from_numpy((rng.standard_normal((K, N)) / np.sqrt(K)).astype(np.float32)).to(torch.bfloat16)
    s = torch.from_numpy(np.exp(0.5 * rng.standard_normal(K)).astype(np.float32))
    X = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    cfg = A.qconfig(g, zp, 21)
    codes = torch.empty((K // 8, N), dtype=torch.int32, device=dev)
    scales = torch.empty((K // g, N), dtype=torch.float32, device=dev)
    zeros = torch.empty((K // g, N), dtype=torch.uint8, device=dev)
    A.awq_pack(W.to(dev), s.to(dev), cfg, codes, scales, zeros)
    q = A.Quantized(codes, scales, zeros, s.to(dev), g)
    Y = gpu_gemm(X, q)
    assert np.all(np.isfinite(Y)), (M, K, N)
    Yr = O.w4a16_ref(I.bf16_to_f64(X), s.numpy(), codes.cpu().numpy().view(np.uint32), scales.cpu().numpy(),
                     zeros.cpu().numpy(), g)
    err = rel_fro(Y, Yr)
    assert err <= 2e-2, (M, K, N, g, err)
    log(f"[poison] gemm M={M} K={K} N={N} g={g}: rel err {err:.2e}: ok")


def check_clip(L, g, zp, n, clip_min, label):
    """Clip-ratio search at the alpha search's chosen s (CLIP instance of the search kernel)."""
    A = awq()
    dev = torch.device("cuda:0")
    X64, W64 = I.bf16_to_f64(L.X), I.bf16_to_f64(L.W)
    s = O.scale_table(O.act_stats(X64)[1], 21)[8]
    T, K = L.X.shape
    N = L.W.shape[1]
    cfg = A.qconfig(g, zp, n)
    ws = A.workspace(A.awq_search_workspace_size(T, K, N, cfg), dev)
    losses = torch.empty(n, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    cbest = torch.empty(1, dtype=torch.float32, device=dev)
    A.awq_clip_search(L.X.to(dev), L.W.to(dev), torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32)).to(dev),
                      cfg, clip_min, ws, losses, best, cbest)
    torch.cuda.synchronize()
    Lg = losses.cpu().numpy()
    Lo = O.clip_losses(X64, W64, s, O.clip_grid(clip_min, n), g, zp)
    assert np.all(np.isfinite(Lg)), label
    rel = np.abs(Lg - Lo) / Lo
    assert np.all(rel <= 1e-2), (label, rel.max())
    log(f"[poison] clip search {label}: max rel loss err {rel.max():.2e}: ok")


def check_multi(T, K, Ns, g, zp, seed, label):
    """Joint search of projections that share X, each packed at the shared s."""
    A = awq()
    dev = torch.device("cuda:0")
    base = I.small(T, K, sum(Ns), seed=seed, group_size=g, zero_point=zp)
    Ws, c = [], 0
    for n in Ns:
        Ws.append(base.W[:, c:c + n].contiguous())
        c += n
    r = A.run_multi(base.X.to(dev), [W.to(dev) for W in Ws], A.qconfig(g, zp, 21))
    torch.cuda.synchronize()
    X64 = I.bf16_to_f64(base.X)
    S = O.scale_table(O.act_stats(X64)[1], 21)
    Lo, Eo = O.losses_multi(X64, [I.bf16_to_f64(W) for W in Ws], S, g, zp)
    Lg, Eg, b = r["losses"].cpu().numpy(), r["each"].cpu().numpy(), int(r["best"].item())
    assert np.all(np.isfinite(Lg)) and np.all(np.isfinite(Eg)), label
    rel, rel_e = np.abs(Lg - Lo) / Lo, np.abs(Eg - Eo) / Eo
    assert np.all(rel <= 1e-2) and np.all(rel_e <= 1e-2), (label, rel.max(), rel_e.max())
    assert Lo[b] <= 1.01 * Lo.min(), label
    for W, q in zip(Ws, r["q"]):
        w, d, z = O.pack(I.bf16_to_f64(W), S[b], g, zp)
        assert np.array_equal(q.scales.cpu().numpy(), d) and np.array_equal(q.zeros.cpu().numpy(), z), label
    log(f"[poison] multi search {label}: max rel err joint {rel.max():.2e}, each {rel_e.max():.2e}: ok")


def check_greedy(T, K, N, g, zp, n_cand, passes, seed, label):
    """Power-of-two greedy: the choices are exact, so they must equal the oracle's bit for bit."""
    A = awq()
    dev = torch.device("cuda:0")
    L = I.small(T, K, N, seed=seed, w_outlier_frac=0.003)
    X64, W64 = I.bf16_to_f64(L.X), I.bf16_to_f64(L.W)
    m = O.act_stats(X64)[1]
    r = A.run_greedy(L.X.to(dev), L.W.to(dev), A.qconfig(g, zp, 21), n_cand, passes)
    torch.cuda.synchronize()
    o = O.greedy_search(W64, m, g, zp, n_cand=n_cand, passes=passes)
    s_gpu = r["s_best"].cpu().numpy()
    assert np.all(np.isfinite(s_gpu)), label
    assert np.array_equal(s_gpu, o["s"]), (label, int(np.sum(s_gpu != o["s"])))
    err = r["err"].cpu().numpy()
    assert np.all(np.abs(err - o["err"]) <= 1e-12 * np.maximum(o["err"], 1e-300)), label
    log(f"[poison] greedy {label}: scales bit-identical to the oracle's: ok")


def main():
    A = awq()
    lib = os.path.basename(A.LIB_PATH)
    log(f"[poison] library {lib}")
    assert lib == "libawq_ldspoison.so", lib
    cases = [
        (I.small(700, 384, 48, seed=3), 128, True, 21, "T=700 K=384 N=48 g=128 asym"),
        (I.small(333, 256, 40, seed=4, group_size=64, zero_point=False), 64, False, 21, "T=333 g=64 sym"),
        (I.small(257, 128, 24, seed=5, group_size=32), 32, True, 21, "T=257 g=32 asym"),
        (I.small(600, 256, 32, seed=6), 128, True, 33, "n_grid=33"),
    ]
    for L, g, zp, ng, label in cases:
        gpu = check_layer(L, g, zp, ng, label)
        T = L.X.shape[0]
        check_gemm(L, gpu, g, [1, 7, 16, 37, min(T, 256)], label)
    # split-K products: M = 1 on 256- and 64-column workgroups, M = 16, 40 and 200 with K split
    check_packed_gemm(1, 8192, 1032, 128, True, seed=11)
    check_packed_gemm(1, 16384, 264, 128, True, seed=12)
    check_packed_gemm(16, 8192, 520, 128, True, seed=13)
    check_packed_gemm(40, 8192, 1032, 64, False, seed=14)
    check_packed_gemm(200, 8192, 520, 128, True, seed=16)   # four 64-row tiles, K split
    check_clip(I.small(500, 256, 40, seed=15), 128, True, 11, 0.5, "g=128 asym 11 ratios")
    check_clip(I.small(300, 128, 24, seed=16, group_size=64, zero_point=False), 64, False, 7, 0.7, "g=64 sym 7 ratios")
    check_multi(420, 256, [64, 16, 24], 128, True, 17, "3 projections g=128")
    check_greedy(64, 256, 40, 128, True, 20, 3, 18, "g=128 asym")
    check_greedy(48, 128, 24, 32, True, 20, 3, 19, "g=32 asym")
    log("[poison] all cases ok")


if __name__ == "__main__":
    main()
