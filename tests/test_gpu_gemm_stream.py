"""The W4A16 product at decode-like sizes (split-K partials summed inside the product by the last
workgroup of each output tile to arrive) against the fp64 oracle.

One workspace serves a whole sequence of calls with changing activations and shapes, as a
serving loop would use it: a partial left over from an earlier call, or an arrival counter not
returned to zero, would show up as a wrong output of a later call.  Each output is compared in
relative Frobenius error (<= 2e-2) with ``oracle.w4a16_ref`` on the same packed weights ("AWQ
(Activation-aware Weight Quantization)", 推理时的等效实现: Y = (X / s*) Dequant(W_q)), and reruns
on the same inputs must be bit-identical (the partials are added in K-block order whatever
order the workgroups arrive in).
"""
import numpy as np
import pytest
import torch

from oracle import awq_oracle as O
from weight_only_int4_act_amd import inputs as I
from tests.gpu_util import awq, log, rel_fro

pytestmark = pytest.mark.gpu

# (M, K, N, group_size, zero_point): wide and narrow layers, ragged column blocks (N % 256 != 0,
# N % 16 == 8), K not a multiple of the slices per workgroup, every group size, both quantizers
SHAPES = [
    (1, 8192, 8192, 128, True),
    (16, 8192, 1024, 128, True),
    (5, 2048, 4104, 64, False),
    (1, 1024, 4128, 32, True),
    (16, 28672, 1032, 128, True),
    (2, 8832, 520, 128, True),
    (1, 384, 40, 128, True),
    (16, 128, 8, 128, False),
    (9, 4096, 12296, 128, True),
    # M = 1 with several slices per wavefront (64-column workgroups), ragged N, each group size
    (1, 16384, 1032, 128, True),
    (1, 12288, 520, 64, False),
    (1, 10240, 264, 32, True),
    # more than 32 rows with 33 groups split into 8 K blocks of 5: the last K block is empty (its
    # workgroups prefetch a neighbour's group, never use it, and add zeros); likewise at g = 64
    (64, 4224, 256, 128, True),
    (48, 2112, 264, 64, False),
    # 17..32 rows on 130 column tiles (K not split), 9 groups: wavefront 0 takes three (the odd
    # one after the two-group steps), the others two
    (24, 1152, 8320, 128, True),
    # more than 64 rows: several 64-row tiles, ragged in rows (M % 64 != 0) and in columns
    # (N % 256 == 8, 136 or 40), K split into blocks of an odd number of groups, each group size
    (96, 4224, 264, 128, False),
    (200, 2112, 136, 64, True),
    (130, 1280, 8232, 32, True),
]

_packed = {}


def _pack(K, N, g, zp):
    key = (K, N, g, zp)
    if key not in _packed:
        A = awq()
        dev = torch.device("cuda:0")
        W = I.small(2, K, N, seed=K * 7 + N, group_size=g, zero_point=zp).W.to(dev)
        s = torch.from_numpy(I.scale_vector(K, seed=K + 1)).to(dev)
        codes = torch.empty((K // 8, N), dtype=torch.int32, device=dev)
        scales = torch.empty((K // g, N), dtype=torch.float32, device=dev)
        zeros = torch.empty((K // g, N), dtype=torch.uint8, device=dev)
        A.awq_pack(W, s, A.qconfig(g, zp, 21), codes, scales, zeros)
        torch.cuda.synchronize()
        host = (s.cpu().numpy(), codes.cpu().numpy().view(np.uint32), scales.cpu().numpy(), zeros.cpu().numpy())
        _packed[key] = (A.Quantized(codes, scales, zeros, s, g), host)
    return _packed[key]


def _x(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 30.0
    return I.to_bf16(x)


def _run(X, q, ws):
    A = awq()
    M = X.shape[0]
    Y = torch.full((M, q.codes.shape[1]), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    A.awq_w4a16_gemm(X.to("cuda:0"), q.s, q.codes, q.scales, q.zeros, q.group_size, Y, ws)
    return Y


def test_shared_workspace_sequence_matches_oracle():
    A = awq()
    need = max(A.awq_w4a16_gemm_workspace_size(M, K, N, g) for M, K, N, g, _ in SHAPES)
    ws = A.workspace(need, torch.device("cuda:0"))
    for rnd in range(3):
        for i, (M, K, N, g, zp) in enumerate(SHAPES):
            q, (s, w, d, z) = _pack(K, N, g, zp)
            log(f"[stream] round {rnd} M={M} K={K} N={N} g={g} zp={zp}")
            X = _x(M, K, seed=1000 * rnd + i)
            Y = _run(X, q, ws)
            torch.cuda.synchronize()
            Yg = I.bf16_to_f64(Y.cpu())
            Yr = O.w4a16_ref(I.bf16_to_f64(X), s, w, d, z, g)
            err = rel_fro(Yg, Yr)
            assert np.all(np.isfinite(Yg)), (M, K, N)
            assert err <= 2e-2, (rnd, M, K, N, g, err)


def test_reruns_bit_identical_and_independent_of_workspace():
    A = awq()
    for M, K, N, g, zp in SHAPES[:5]:
        q, _ = _pack(K, N, g, zp)
        need = A.awq_w4a16_gemm_workspace_size(M, K, N, g)
        ws1 = A.workspace(need, torch.device("cuda:0"))
        ws2 = A.workspace(need + 4096, torch.device("cuda:0"))
        X = _x(M, K, seed=77 + M)
        ys = [_run(X, q, ws) for ws in (ws1, ws1, ws2, ws1)]
        torch.cuda.synchronize()
        for y in ys[1:]:
            assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16)), (M, K, N)


def test_rows_of_a_batch_match_single_row_products():
    # rows of an M = 16 product against the same rows computed as M = 1 products: both follow
    # the oracle, and they agree with each other to bf16 output rounding and float32 order
    A = awq()
    M, K, N, g, zp = 16, 4096, 2048, 128, True
    q, (s, w, d, z) = _pack(K, N, g, zp)
    ws = A.workspace(A.awq_w4a16_gemm_workspace_size(M, K, N, g), torch.device("cuda:0"))
    X = _x(M, K, seed=5)
    Y16 = I.bf16_to_f64(_run(X, q, ws).cpu())
    Yr = O.w4a16_ref(I.bf16_to_f64(X), s, w, d, z, g)
    for m in (0, 7, 15):
        y1 = I.bf16_to_f64(_run(X[m:m + 1].contiguous(), q, ws).cpu())[0]
        assert rel_fro(y1, Yr[m]) <= 2e-2 and rel_fro(Y16[m], Yr[m]) <= 2e-2
        assert rel_fro(y1, Y16[m]) <= 1e-2
