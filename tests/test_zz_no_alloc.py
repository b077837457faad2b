"""awq_w4a16_gemm_noalloc: the W4A16 product for callers that cannot allocate (graph capture,
serving loops), with its scratch in one fixed per-GPU buffer of the library instead of a caller
workspace.

Called through the C ABI (ctypes, device pointers of torch tensors) and compared with
awq_w4a16_gemm on the same inputs: the same kernels and plan run, so the outputs must agree bit
for bit; both are also held to the product's bar against the fp64 oracle ("AWQ (Activation-aware
Weight Quantization)", 推理时的等效实现: Y = (X / s*) Dequant(W_q), relative Frobenius error
<= 2e-2).  Consecutive calls share the buffer, each later one smaller than the one before, so a
value left over from an earlier call (a partial, an arrival counter not back at zero) would show.
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import awq_oracle as O
from weight_only_int4_act_amd import inputs as I
from tests.gpu_util import awq, log, rel_fro


def _pack(K, N, g, zp, seed):
    A = awq()
    dev = torch.device("cuda:0")
    W = I.small(2, K, N, seed=seed, group_size=g, zero_point=zp).W.to(dev)
    s = torch.from_numpy(I.scale_vector(K, seed=seed + 1)).to(dev)
    codes = torch.empty((K // 8, N), dtype=torch.int32, device=dev)
    scales = torch.empty((K // g, N), dtype=torch.float32, device=dev)
    zeros = torch.empty((K // g, N), dtype=torch.uint8, device=dev)
    A.awq_pack(W, s, A.qconfig(g, zp, 21), codes, scales, zeros)
    return s, codes, scales, zeros


def _noalloc_c(lib, X, s, codes, scales, zeros, g, Y):
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    M, K = X.shape
    return lib.awq_w4a16_gemm_noalloc(P(X), M, P(s), P(codes), P(scales), P(zeros), K, codes.shape[1], g, P(Y),
                                      stream)


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    A = awq()
    lib = A.library()
    dev = torch.device("cuda:0")
    # (M, K, N, group size, zero point): each call smaller than the one before
    calls = [(1, 8192, 8192, 128, True), (16, 4096, 4104, 128, True), (1, 1024, 520, 64, False)]
    for i, (M, K, N, g, zp) in enumerate(calls):
        log(f"[noalloc] call {i}: M={M} K={K} N={N} g={g} zp={zp}")
        s, codes, scales, zeros = _pack(K, N, g, zp, seed=100 + i)
        rng = np.random.default_rng(7 + i)
        X = I.to_bf16(rng.standard_normal((M, K)).astype(np.float32)).to(dev)
        Y_ref = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
        ws = A.workspace(A.awq_w4a16_gemm_workspace_size(M, K, N, g), dev)
        A.awq_w4a16_gemm(X, s, codes, scales, zeros, g, Y_ref, ws)
        Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
        st = _noalloc_c(lib, X, s, codes, scales, zeros, g, Y)
        assert st == A.AWQ_OK, A.awq_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16)), f"call {i} differs from awq_w4a16_gemm"
        Yr = O.w4a16_ref(I.bf16_to_f64(X.cpu()), s.cpu().numpy(), codes.cpu().numpy().view(np.uint32),
                         scales.cpu().numpy(), zeros.cpu().numpy(), g)
        err = rel_fro(I.bf16_to_f64(Y.cpu()), Yr)
        log(f"[noalloc] call {i}: rel Frobenius err {err:.2e}")
        assert err <= 2e-2


def test_noalloc_rejects_calls_beyond_its_scratch_before_launch():
    # needs no GPU: the size check comes before anything touches the device
    A = awq()
    lib = A.library()
    cap = A.awq_w4a16_gemm_static_scratch_bytes()
    assert cap >= 16 << 20
    p = ctypes.c_void_p(256)
    M, K, N = 1, 8192, 4194304 - 256
    assert A.awq_w4a16_gemm_workspace_size(M, K, N, 128) > cap
    assert lib.awq_w4a16_gemm_noalloc(p, M, p, p, p, p, K, N, 128, p, None) == A.AWQ_ERR_SCRATCH
    assert "scratch" in A.awq_status_string(A.AWQ_ERR_SCRATCH)
    # ordinary argument errors are reported as for awq_w4a16_gemm
    assert lib.awq_w4a16_gemm_noalloc(p, 1, p, p, p, p, 128, 12, 128, p, None) == A.AWQ_ERR_INVALID_ARG
    assert lib.awq_w4a16_gemm_noalloc(p, 1, p, p, p, p, 128, 16, 96, p, None) == A.AWQ_ERR_UNSUPPORTED
