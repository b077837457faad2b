"""Parity of the joint search over projections that share one input X (HIP path through the C
ABI) with the fp64 oracle.

Projections that read the same activations share one scale vector once 1/s is applied to X a
single time ("009. AWQ Integration", 关键设计 4, and the fused attn.qkv layer of its usage); the
joint loss sums the loss of "AWQ (Activation-aware Weight Quantization)", 缩放因子优化的完整流程
step 4c over the projections.  Bars as for the single search: every joint and per-projection loss
within 1e-2 relative of the oracle, the chosen alpha's oracle loss within 1e-2 of the oracle
minimum, s_best equal to the GPU scale table's row; and, where every projection has a multiple of
16 columns, the joint losses bit-identical to awq_search on the column-concatenated matrix (the
same tiles in the same order).  Packed side by side at the shared s, the projections are the
packing of the concatenated matrix (bit-exact) and one W4A16 call serves them all (relative
Frobenius error <= 2e-2 against the fp64 product, the single-layer bar).
"""
import numpy as np
import pytest
import torch

from oracle import awq_oracle as O
from weight_only_int4_act_amd import inputs as I
from tests.gpu_util import awq, log

pytestmark = pytest.mark.gpu

L_TOL = 1e-2
DEV = torch.device("cuda:0")

CASES = {
    # name: (T, K, column counts, group_size, zero_point, clip, seed); ragged counts pad with zeros
    "zp128_ragged": (300, 384, (24, 8, 40), 128, True, 1.0, 61),
    "sym64_two": (1030, 256, (48, 17), 64, False, 1.0, 62),
    "zp32_clip": (100, 192, (16, 40), 32, True, 0.85, 63),
    "zp128_rows640_one": (1250, 256, (72,), 128, True, 1.0, 64),
}


def _inputs(T, K, Ns, seed):
    base = I.small(T, K, sum(Ns), seed=seed, w_outlier_frac=0.003)
    Ws, c = [], 0
    for n in Ns:
        Ws.append(base.W[:, c:c + n].contiguous())
        c += n
    return base.X, Ws


@pytest.mark.parametrize("name", list(CASES))
def test_multi_search_matches_oracle(name):
    A = awq()
    T, K, Ns, g, zp, clip, seed = CASES[name]
    X, Ws = _inputs(T, K, Ns, seed)
    cfg = A.qconfig(g, zp, 21, clip_ratio=clip)
    r = A.run_multi(X.to(DEV), [W.to(DEV) for W in Ws], cfg)
    torch.cuda.synchronize()
    Lg, Eg, b = r["losses"].cpu().numpy(), r["each"].cpu().numpy(), int(r["best"].item())
    X64 = I.bf16_to_f64(X)
    S = O.scale_table(O.act_stats(X64)[1], 21)
    Lo, Eo = O.losses_multi(X64, [I.bf16_to_f64(W) for W in Ws], S, g, zp, clip=clip)
    rel, rel_e = np.abs(Lg - Lo) / Lo, np.abs(Eg - Eo) / Eo
    log(f"[multi] {name}: max rel err joint {rel.max():.2e}, each {rel_e.max():.2e}; "
        f"alpha* gpu {b} oracle {O.select(Lo)}")
    assert np.all(rel <= L_TOL) and np.all(rel_e <= L_TOL)
    assert Lo[b] <= (1 + L_TOL) * Lo.min()
    # the per-projection sums are reduced on their own: the same float32 partials in another order
    assert np.all(np.abs(Eg.sum(axis=0) - Lg) <= 1e-9 * Lg)
    # s_best is the table row of the chosen alpha, computed on the GPU
    st = torch.empty((21, K), dtype=torch.float32, device=DEV)
    A.awq_scale_table(r["mean_abs"], 21, st)
    assert np.array_equal(r["s_best"].cpu().numpy(), st[b].cpu().numpy())
    # every projection is packed at the shared s*, as the oracle packs it
    for W, q in zip(Ws, r["q"]):
        w, d, z = O.pack(I.bf16_to_f64(W), S[b], g, zp, clip=clip)
        assert np.array_equal(q.scales.cpu().numpy(), d) and np.array_equal(q.zeros.cpu().numpy(), z)


def _search(A, X, W, cfg, mean_abs):
    T, K = X.shape
    ws = A.workspace(A.awq_search_workspace_size(T, K, W.shape[1], cfg), DEV)
    losses = torch.empty(cfg.n_grid, dtype=torch.float64, device=DEV)
    best = torch.empty(1, dtype=torch.int32, device=DEV)
    s_best = torch.empty(K, dtype=torch.float32, device=DEV)
    A.awq_search(X, W, mean_abs, cfg, ws, losses, best, s_best)
    return losses, best, s_best


def _multi(A, X, Ws, cfg, mean_abs):
    T, K = X.shape
    ws = A.workspace(A.awq_search_multi_workspace_size(T, K, [W.shape[1] for W in Ws], cfg), DEV)
    losses = torch.empty(cfg.n_grid, dtype=torch.float64, device=DEV)
    each = torch.empty((len(Ws), cfg.n_grid), dtype=torch.float64, device=DEV)
    best = torch.empty(1, dtype=torch.int32, device=DEV)
    s_best = torch.empty(K, dtype=torch.float32, device=DEV)
    A.awq_search_multi(X, Ws, mean_abs, cfg, ws, losses, each, best, s_best)
    return losses, each, best, s_best


def _mean_abs(A, X):
    T, K = X.shape
    sum_abs = torch.empty(K, dtype=torch.float64, device=DEV)
    m = torch.empty(K, dtype=torch.float32, device=DEV)
    A.awq_act_stats(X, sum_abs, False, T, m, A.workspace(A.awq_act_stats_workspace_size(T, K), DEV))
    return m


def _same_as_fused_and_single(A, X, Ws, cfg):
    m = _mean_abs(A, X)
    L, E, b, s = _multi(A, X, Ws, cfg, m)
    Lf, bf, sf = _search(A, X, torch.cat(Ws, dim=1).contiguous(), cfg, m)
    torch.cuda.synchronize()
    assert torch.equal(L, Lf) and torch.equal(b, bf) and torch.equal(s, sf)
    for j, W in enumerate(Ws):
        Lj, _, _ = _search(A, X, W, cfg, m)
        torch.cuda.synchronize()
        assert torch.allclose(E[j], Lj, rtol=1e-12, atol=0.0)
    return L, E, b


def test_multi_equals_the_fused_layer_bitwise():
    A = awq()
    X, Ws = _inputs(700, 256, (32, 16, 48), 65)
    for zp, g in ((True, 128), (False, 64)):
        _same_as_fused_and_single(A, X.to(DEV), [W.to(DEV) for W in Ws], A.qconfig(g, zp, 21))


def test_losses_each_may_be_null_and_one_projection_is_the_single_search():
    A = awq()
    X, Ws = _inputs(200, 128, (40,), 66)
    Xd, Wd = X.to(DEV), Ws[0].to(DEV)
    cfg = A.qconfig(128, True, 21)
    m = _mean_abs(A, Xd)
    T, K = X.shape
    ws = A.workspace(A.awq_search_multi_workspace_size(T, K, [40], cfg), DEV)
    losses = torch.empty(21, dtype=torch.float64, device=DEV)
    best = torch.empty(1, dtype=torch.int32, device=DEV)
    s_best = torch.empty(K, dtype=torch.float32, device=DEV)
    A.awq_search_multi(Xd, [Wd], m, cfg, ws, losses, None, best, s_best)
    Ls, bs, ss = _search(A, Xd, Wd, cfg, m)
    torch.cuda.synchronize()
    assert torch.equal(losses, Ls) and torch.equal(best, bs) and torch.equal(s_best, ss)


def test_multi_full_size_attention_projections():
    # q, k and v of the 8-layer block's attention: one X [4096, 8192], W [8192, 8192 | 1024 | 1024]
    A = awq()
    names = ("q", "k", "v")
    ls = I.make_config("c5", seed=0, layers=names).layers
    assert [L.name for L in ls] == [f"c5.{n}" for n in names]
    X = ls[0].X.to(DEV)
    Ws = [L.W.to(DEV) for L in ls]
    log(f"[multi] c5 qkv: X {tuple(X.shape)}, W {[tuple(W.shape) for W in Ws]}")
    L, E, b = _same_as_fused_and_single(A, X, Ws, A.qconfig(128, True, 21))
    log(f"[multi] c5 qkv: alpha* {int(b.item())}, L(alpha*) {float(L[b].item()):.6e}")


def test_projections_sharing_s_run_as_one_product():
    # packing is per column, so the jointly searched projections packed side by side are the
    # packing of the concatenated matrix; one W4A16 call over it gives every projection's output
    A = awq()
    X, Ws = _inputs(300, 256, (48, 16, 64), 67)
    r = A.run_multi(X.to(DEV), [W.to(DEV) for W in Ws], A.qconfig(128, True, 21))
    qs = r["q"]
    cat = A.Quantized(torch.cat([q.codes for q in qs], 1).contiguous(), torch.cat([q.scales for q in qs], 1).contiguous(),
                      torch.cat([q.zeros for q in qs], 1).contiguous(), qs[0].s, 128)
    Wc = torch.cat(Ws, 1).contiguous()
    cw = torch.empty((256 // 8, 128), dtype=torch.int32, device=DEV)
    cs = torch.empty((2, 128), dtype=torch.float32, device=DEV)
    cz = torch.empty((2, 128), dtype=torch.uint8, device=DEV)
    A.awq_pack(Wc.to(DEV), r["s_best"], A.qconfig(128, True, 21), cw, cs, cz)
    torch.cuda.synchronize()
    assert torch.equal(cw, cat.codes) and torch.equal(cs, cat.scales) and torch.equal(cz, cat.zeros)
    for M in (1, 16):
        xm = X[:M].to(DEV).contiguous()
        Y = A.gemm(xm, cat)
        torch.cuda.synchronize()
        Yo = O.w4a16_ref(I.bf16_to_f64(X[:M]), r["s_best"].cpu().numpy(), cat.codes.cpu().numpy().view(np.uint32),
                         cat.scales.cpu().numpy(), cat.zeros.cpu().numpy(), 128)
        Yg = I.bf16_to_f64(Y.cpu())
        rel = np.linalg.norm(Yg - Yo) / np.linalg.norm(Yo)
        log(f"[multi] fused product M={M}: rel err {rel:.2e}")
        assert rel <= 2e-2   # the W4A16 bar of the single-layer parity tests
