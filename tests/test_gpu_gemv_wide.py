"""The M = 1 W4A16 product on wide layers, which take 256-column workgroups (each lane reads every
code row of its own four columns and the matrix-core products carry x' in one A row per k-slot
group): every group size, both quantizers, column counts that are not a multiple of 256, slices of a
whole group, half and a quarter of one, and K split 8 or 16 ways ("AWQ (Activation-aware Weight
Quantization)", 推理时的等效实现: Y = (X / s*) Dequant(W_q); "大模型 AWQ 量化实战", section 3: 4-bit
weights unpacked on chip and multiplied with 16-bit activations).

Each output is compared with ``oracle.w4a16_ref`` (relative Frobenius error <= 2e-2) on the first
256 columns, 256 columns in the middle and the last 264 (the ragged tail), on the same packed
weights; a rerun on the same workspace must be bit-identical.
"""
import numpy as np
import pytest
import torch

from oracle import awq_oracle as O
from weight_only_int4_act_amd import inputs as I
from tests.gpu_util import awq, log, rel_fro

pytestmark = pytest.mark.gpu

# (K, N, group_size, zero_point): rows of K per wavefront slice and K split in the comment
SHAPES = [
    (4096, 40968, 128, True),    # half-group slices, 16 K blocks
    (2048, 24584, 32, False),    # whole-group slices of 32 rows, symmetric
    (4096, 24840, 64, True),     # whole-group slices of 64 rows
    (4096, 49160, 128, False),   # whole-group slices of 128 rows, 8 K blocks, symmetric
    (2048, 49160, 64, True),     # 8 K blocks of 64-row slices
]


def _cols(N):
    return np.r_[0:256, N // 2 - 128:N // 2 + 128, N - 264:N]


@pytest.mark.parametrize("K,N,g,zp", SHAPES)
def test_wide_m1_product_matches_oracle(K, N, g, zp):
    A = awq()
    dev = torch.device("cuda:0")
    log(f"[gemv-wide] K={K} N={N} g={g} zp={zp}")
    W = I.small(2, K, N, seed=K + 3 * N, group_size=g, zero_point=zp).W.to(dev)
    s = torch.from_numpy(I.scale_vector(K, seed=K + 9)).to(dev)
    codes = torch.empty((K // 8, N), dtype=torch.int32, device=dev)
    scales = torch.empty((K // g, N), dtype=torch.float32, device=dev)
    zeros = torch.empty((K // g, N), dtype=torch.uint8, device=dev)
    A.awq_pack(W, s, A.qconfig(g, zp, 21), codes, scales, zeros)
    del W
    rng = np.random.default_rng(K ^ N)
    x = rng.standard_normal((1, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 40.0
    X = I.to_bf16(x)
    ws = A.workspace(A.awq_w4a16_gemm_workspace_size(1, K, N, g), dev)
    ys = []
    for _ in range(2):
        Y = torch.full((1, N), float("nan"), dtype=torch.bfloat16, device=dev)
        A.awq_w4a16_gemm(X.to(dev), s, codes, scales, zeros, g, Y, ws)
        ys.append(Y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))
    assert not torch.any(ws[:65536]), "counter region not zero after the call"
    cols = _cols(N)
    w = codes.cpu().numpy().view(np.uint32)[:, cols]
    d = scales.cpu().numpy()[:, cols]
    z = zeros.cpu().numpy()[:, cols]
    Yr = O.w4a16_ref(I.bf16_to_f64(X), s.cpu().numpy(), w, d, z, g)
    Yg = I.bf16_to_f64(ys[0].cpu())[:, cols]
    assert np.all(np.isfinite(Yg))
    err = rel_fro(Yg, Yr)
    assert err <= 2e-2, (K, N, g, zp, err)
