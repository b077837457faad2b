"""Parity of the power-of-two greedy search (HIP path through the C ABI) with the fp64 oracle.

"009. AWQ Integration", 关键设计 1-3: per group of input channels, a coordinate greedy over
power-of-two scale candidates around 1, each scored with the activation-weighted reconstruction
error of the whole group under the packing quantizer.  Both sides compute every element's error
exactly; only the float64 sums differ in order, so the chosen scales must agree bit for bit, and
the group errors within 1e-12 relative.  At full size the oracle checks sampled groups: their
errors at s = 1 and at the result, and that the last decision of each is a minimum over the
candidates.
"""
import numpy as np
import pytest
import torch

from oracle import awq_oracle as O
from weight_only_int4_act_amd import inputs as I
from tests.gpu_util import awq, log

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

CASES = {
    # name: (T, K, N, group_size, zero_point, n_cand, passes, seed)
    "zp128": (64, 256, 40, 128, True, 20, 3, 81),
    "sym64_two_slices": (32, 128, 300, 64, False, 20, 3, 82),
    "zp32": (48, 128, 24, 32, True, 20, 3, 83),
    "sym128_ncand8": (40, 256, 72, 128, False, 8, 2, 84),
    "zp64_one_col": (16, 128, 1, 64, True, 20, 3, 85),
}


def _gpu(X, W, g, zp, n_cand, passes):
    A = awq()
    r = A.run_greedy(X.to(DEV), W.to(DEV), A.qconfig(g, zp, 21), n_cand, passes)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in r.items()}


@pytest.mark.parametrize("name", list(CASES))
def test_greedy_matches_oracle(name):
    T, K, N, g, zp, n_cand, passes, seed = CASES[name]
    L = I.small(T, K, N, seed=seed, w_outlier_frac=0.003)
    X64, W64 = I.bf16_to_f64(L.X), I.bf16_to_f64(L.W)
    m = O.act_stats(X64)[1]
    r = _gpu(L.X, L.W, g, zp, n_cand, passes)
    assert np.array_equal(r["mean_abs"], m)
    o = O.greedy_search(W64, m, g, zp, n_cand=n_cand, passes=passes)
    diff = int(np.sum(r["s_best"] != o["s"]))
    log(f"[greedy] {name}: {diff} of {K} scales differ; err_rtn/err oracle "
        f"{o['err_rtn'].sum() / max(o['err'].sum(), 1e-300):.3f}, "
        f"scales >1: {int(np.sum(o['s'] > 1))}, <1: {int(np.sum(o['s'] < 1))}")
    assert diff == 0
    assert np.all(np.abs(r["err_rtn"] - o["err_rtn"]) <= 1e-12 * np.maximum(o["err_rtn"], 1e-300))
    assert np.all(np.abs(r["err"] - o["err"]) <= 1e-12 * np.maximum(o["err"], 1e-300))
    # packed at the result exactly as the oracle packs
    w, d, z = O.pack(W64, o["s"], g, zp)
    q = r["q"]
    assert np.array_equal(q.codes.cpu().numpy().view(np.uint32), w)
    assert np.array_equal(q.scales.cpu().numpy(), d) and np.array_equal(q.zeros.cpu().numpy(), z)


def test_worked_example_in_a_group_of_32():
    # the hand example of the oracle pins (w = 7/8, 5/16; m = 0, 1; candidates 1/4 .. 2; one pass)
    # padded to a group of 32 with zero weights of zero activation, which no scale changes
    A = awq()
    W = torch.zeros((32, 8), dtype=torch.bfloat16)
    W[0, 0], W[1, 0] = 0.875, 0.3125
    m = torch.zeros(32, dtype=torch.float32)
    m[1] = 1.0
    cfg = A.qconfig(32, False, 21)
    ws = A.workspace(A.awq_greedy_workspace_size(32, 8, cfg, 4), DEV)
    s = torch.empty(32, dtype=torch.float32, device=DEV)
    er = torch.empty(1, dtype=torch.float64, device=DEV)
    e = torch.empty(1, dtype=torch.float64, device=DEV)
    A.awq_greedy_search(W.to(DEV), m.to(DEV), cfg, 4, 1, ws, s, er, e)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    assert s[0] == 0.5 and np.all(s[1:] == 1.0)
    assert er.item() == 1.0 / 256 and e.item() == 0.0


def test_greedy_full_size_layer():
    # the 4096x4096 layer, 8192 tokens, g = 128 asymmetric, 20 candidates, 3 passes
    A = awq()
    L = I.make_config("c2", seed=0).layers[0]
    X64 = None
    r = _gpu(L.X, L.W, 128, True, 20, 3)
    m = r["mean_abs"].astype(np.float64)
    W64 = I.bf16_to_f64(L.W)
    s = r["s_best"].astype(np.float64)
    assert np.all(r["err"] <= r["err_rtn"])
    ratio = r["err_rtn"].sum() / r["err"].sum()
    log(f"[greedy] c2: err_rtn/err = {ratio:.3f}; scales > 1: {int(np.sum(s > 1))}, < 1: {int(np.sum(s < 1))}")
    cand = O.pow2_candidates(20)
    for j in (0, 13, 31):
        rows = slice(j * 128, (j + 1) * 128)
        e_rtn = O.group_error(W64[rows], m[rows], np.ones(128), True)
        e_fin = O.group_error(W64[rows], m[rows], s[rows], True)
        assert abs(r["err_rtn"][j] - e_rtn) <= 1e-12 * e_rtn
        assert abs(r["err"][j] - e_fin) <= 1e-12 * e_fin
        # the group's last decision (its channel 127 in the third pass) is a minimum
        for c in range(20):
            sg = s[rows].copy()
            sg[127] = cand[c]
            assert O.group_error(W64[rows], m[rows], sg, True) >= e_fin * (1 - 1e-12)
