"""Host-side checks of libawq that need no GPU: the shared library loads, exports every
function include/awq.h declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")
LIB = os.path.join(ROOT, "weight_only_int4_act_amd", "libawq.so")


def _declared():
    txt = open(HEADER, encoding="utf-8").read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"\b(awq_\w+)\s*\(", txt)
    return sorted(set(names))


@pytest.fixture(scope="module")
def awq():
    if not os.path.exists(LIB):
        pytest.fail("libawq.so is not built (python -m weight_only_int4_act_amd.build)")
    from weight_only_int4_act_amd import awq as mod
    return mod


def test_header_declares_the_boundary():
    names = _declared()
    for fn in ("awq_act_stats", "awq_search", "awq_pack", "awq_w4a16_gemm", "awq_scale_table",
               "awq_search_workspace_size", "awq_status_string"):
        assert fn in names


def test_library_exports_every_declared_symbol(awq):
    lib = awq.library()
    for name in _declared():
        assert hasattr(lib, name), f"{name} is declared in awq.h but not exported"
    assert set(_declared()) == set(awq.EXPORTED)


def test_lds_poison_build_exports_the_same_symbols(awq):
    # the debug build used by the race test (tests/test_gpu_lds_poison.py) is the same ABI
    import ctypes
    path = os.path.join(os.path.dirname(awq.LIB_PATH), "libawq_ldspoison.so")
    assert os.path.exists(path), path
    lib = ctypes.CDLL(path)
    for name in _declared():
        assert hasattr(lib, name), f"{name} is declared in awq.h but not exported by the debug build"
    assert os.path.basename(awq.LIB_PATH) == "libawq.so"   # the product path loads the product build


def test_status_strings(awq):
    assert awq.awq_status_string(0) == "ok"
    for st in (-1, -2, -3, -4):
        assert awq.awq_status_string(st) not in ("ok", "unknown status")
    assert awq.awq_status_string(7) == "unknown status"
    assert "gfx950" in awq.awq_version()


def test_workspace_sizes(awq):
    cfg = awq.qconfig(128, True, 21)
    assert awq.awq_search_workspace_size(8192, 4096, 4096, cfg) > 0
    assert awq.awq_search_workspace_size(8192, 4100, 4096, cfg) == 0          # K % g != 0
    assert awq.awq_search_workspace_size(8192, 4096, 4096, awq.qconfig(48, True, 21)) == 0
    assert awq.awq_act_stats_workspace_size(8192, 4096) >= 8 * 4096
    assert awq.awq_act_stats_workspace_size(0, 4096) == 0


def test_host_validation_rejects_before_launch(awq):
    lib = awq.library()
    p = ctypes.c_void_p(256)          # never dereferenced: every call below fails validation first
    nul = ctypes.c_void_p(0)
    cfg = awq.qconfig(128, True, 21)
    ws = ctypes.c_size_t(1 << 40)
    # search: null pointers, bad shapes, unsupported configurations, misalignment
    assert lib.awq_search(nul, 8, p, 128, 16, p, ctypes.byref(cfg), p, ws, p, p, p, nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_search(p, 0, p, 128, 16, p, ctypes.byref(cfg), p, ws, p, p, p, nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_search(p, 8, p, 100, 16, p, ctypes.byref(cfg), p, ws, p, p, p, nul) == awq.AWQ_ERR_INVALID_ARG
    for bad in (awq.qconfig(128, True, 21, w_bit=3), awq.qconfig(96, True, 21), awq.qconfig(128, True, 1),
                awq.qconfig(128, True, 65)):
        assert lib.awq_search(p, 8, p, 128, 16, p, ctypes.byref(bad), p, ws, p, p, p, nul) == awq.AWQ_ERR_UNSUPPORTED
    assert lib.awq_search(ctypes.c_void_p(258), 8, p, 128, 16, p, ctypes.byref(cfg), p, ws, p, p, p,
                          nul) == awq.AWQ_ERR_INVALID_ARG
    need = awq.awq_search_workspace_size(8, 128, 16, cfg)
    assert lib.awq_search(p, 8, p, 128, 16, p, ctypes.byref(cfg), p, need - 1, p, p, p,
                          nul) == awq.AWQ_ERR_WORKSPACE
    # clipping: ratio outside [0, 1] (NaN included) in the configuration, clip_min outside (0, 1]
    for c in (1.5, -0.1, float("nan")):
        bad = awq.qconfig(128, True, 21, clip_ratio=c)
        assert lib.awq_search(p, 8, p, 128, 16, p, ctypes.byref(bad), p, ws, p, p, p, nul) == awq.AWQ_ERR_UNSUPPORTED
        assert lib.awq_pack(p, 128, 16, p, ctypes.byref(bad), p, p, p, nul) == awq.AWQ_ERR_UNSUPPORTED
    for cm in (0.0, -0.5, 1.01, float("nan")):
        assert lib.awq_clip_search(p, 8, p, 128, 16, p, ctypes.byref(cfg), ctypes.c_float(cm), p, ws, p, p, p,
                                   nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_clip_search(p, 8, p, 128, 16, nul, ctypes.byref(cfg), ctypes.c_float(0.5), p, ws, p, p, p,
                               nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_clip_search(p, 8, p, 128, 16, p, ctypes.byref(cfg), ctypes.c_float(0.5), p, need - 1, p, p, p,
                               nul) == awq.AWQ_ERR_WORKSPACE
    # statistic and scale variants, search over a given table
    assert lib.awq_act_max(nul, 8, 16, p, 0, p, ws, nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_act_max(p, 8, 16, p, 3, p, ws, nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_act_max(p, 4096, 4096, p, 0, p, 8, nul) == awq.AWQ_ERR_WORKSPACE
    assert lib.awq_weight_mean_abs(p, 0, 16, p, nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_scale_table_ex(p, nul, 16, 1, 0, p, nul) == awq.AWQ_ERR_UNSUPPORTED
    assert lib.awq_scale_table_ex(p, nul, 16, 21, 2, p, nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_scale_table_ex(nul, p, 16, 21, 0, p, nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_search_table(p, 8, p, 128, 16, nul, ctypes.byref(cfg), p, ws, p, p, p,
                                nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_search_table(p, 8, p, 128, 16, p, ctypes.byref(cfg), p, need - 1, p, p, p,
                                nul) == awq.AWQ_ERR_WORKSPACE
    # projections sharing X: count, null or misaligned matrices, column counts, workspace
    Ns = (ctypes.c_int64 * 3)(24, 8, 40)
    Ws = (ctypes.c_void_p * 3)(256, 512, 768)
    need_m = lib.awq_search_multi_workspace_size(8, 128, 3, Ns, ctypes.byref(cfg))
    assert need_m == lib.awq_search_workspace_size(8, 128, 32 + 16 + 48, ctypes.byref(cfg))
    assert lib.awq_search_multi_workspace_size(8, 128, 0, Ns, ctypes.byref(cfg)) == 0
    assert lib.awq_search_multi_workspace_size(8, 128, awq.AWQ_MAX_PROJECTIONS + 1, Ns, ctypes.byref(cfg)) == 0
    for n_w in (0, awq.AWQ_MAX_PROJECTIONS + 1):
        assert lib.awq_search_multi(p, 8, n_w, Ws, Ns, 128, p, ctypes.byref(cfg), p, ws, p, nul, p, p,
                                    nul) == awq.AWQ_ERR_INVALID_ARG
    bad_w = (ctypes.c_void_p * 3)(256, 0, 768)
    odd_w = (ctypes.c_void_p * 3)(256, 513, 768)
    bad_n = (ctypes.c_int64 * 3)(24, 0, 40)
    for W_, N_ in ((bad_w, Ns), (odd_w, Ns), (Ws, bad_n), (None, Ns), (Ws, None)):
        assert lib.awq_search_multi(p, 8, 3, W_, N_, 128, p, ctypes.byref(cfg), p, ws, p, nul, p, p,
                                    nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_search_multi(p, 8, 3, Ws, Ns, 128, p, ctypes.byref(cfg), p, ws, p, ctypes.c_void_p(260), p, p,
                                nul) == awq.AWQ_ERR_INVALID_ARG          # losses_each misaligned
    assert lib.awq_search_multi(p, 8, 3, Ws, Ns, 128, p, ctypes.byref(cfg), p, need_m - 1, p, nul, p, p,
                                nul) == awq.AWQ_ERR_WORKSPACE
    # power-of-two greedy: candidate count, passes, clip ratio, sizes, workspace
    need_g = lib.awq_greedy_workspace_size(256, 40, ctypes.byref(cfg), 20)
    assert need_g > 0 and lib.awq_greedy_workspace_size(256, 40, ctypes.byref(cfg), 1) == 0
    assert lib.awq_greedy_workspace_size(256, 40, ctypes.byref(cfg), awq.AWQ_MAX_POW2_CANDIDATES + 1) == 0
    for n_cand, passes in ((1, 3), (awq.AWQ_MAX_POW2_CANDIDATES + 1, 3), (20, 0), (20, 65)):
        assert lib.awq_greedy_search(p, 256, 40, p, ctypes.byref(cfg), n_cand, passes, p, ws, p, nul, nul,
                                     nul) == awq.AWQ_ERR_INVALID_ARG
    clipped = awq.qconfig(128, True, 21, clip_ratio=0.9)
    assert lib.awq_greedy_search(p, 256, 40, p, ctypes.byref(clipped), 20, 3, p, ws, p, nul, nul,
                                 nul) == awq.AWQ_ERR_UNSUPPORTED
    assert lib.awq_greedy_search(nul, 256, 40, p, ctypes.byref(cfg), 20, 3, p, ws, p, nul, nul,
                                 nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_greedy_search(p, 200, 40, p, ctypes.byref(cfg), 20, 3, p, ws, p, nul, nul,
                                 nul) == awq.AWQ_ERR_INVALID_ARG                      # K % g
    assert lib.awq_greedy_search(p, 256, 40, p, ctypes.byref(cfg), 20, 3, p, ws, p, ctypes.c_void_p(260), nul,
                                 nul) == awq.AWQ_ERR_INVALID_ARG                      # misaligned err_rtn
    assert lib.awq_greedy_search(p, 256, 40, p, ctypes.byref(cfg), 20, 3, p, need_g - 1, p, nul, nul,
                                 nul) == awq.AWQ_ERR_WORKSPACE
    # stats
    assert lib.awq_act_stats(p, 8, 16, nul, 0, 8, p, p, ws, nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_act_stats(p, 8, 16, p, 0, 7, p, p, ws, nul) == awq.AWQ_ERR_INVALID_ARG   # total < T
    assert lib.awq_act_stats(p, 8, 16, p, 2, 8, p, p, ws, nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_act_stats(p, 4096, 4096, p, 0, 4096, p, p, 8, nul) == awq.AWQ_ERR_WORKSPACE
    # scale table
    assert lib.awq_scale_table(p, 16, 1, p, nul) == awq.AWQ_ERR_UNSUPPORTED
    assert lib.awq_scale_table(nul, 16, 21, p, nul) == awq.AWQ_ERR_INVALID_ARG
    # pack
    assert lib.awq_pack(p, 100, 16, p, ctypes.byref(cfg), p, p, p, nul) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_pack(p, 128, 16, p, ctypes.byref(awq.awq_qconfig(4, 128, 2, 21)), p, p, p, nul) == awq.AWQ_ERR_INVALID_ARG
    # gemm
    assert lib.awq_w4a16_gemm(p, 1, p, p, p, p, 128, 12, 128, p, p, ws, nul) == awq.AWQ_ERR_INVALID_ARG  # N % 8
    assert lib.awq_w4a16_gemm(p, 1, p, p, p, p, 128, 16, 256, p, p, ws, nul) == awq.AWQ_ERR_UNSUPPORTED
    assert lib.awq_w4a16_gemm(p, 0, p, p, p, p, 128, 16, 128, p, p, ws, nul) == awq.AWQ_ERR_INVALID_ARG


def test_binding_refuses_host_tensors(awq):
    import torch
    X = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        awq.awq_act_stats(X, torch.zeros(128, dtype=torch.float64), False, 4, None, torch.zeros(8, dtype=torch.uint8))


def test_gemm_rejects_misaligned_workspace(awq):
    lib = awq.library()
    p = ctypes.c_void_p(256)
    need = awq.awq_w4a16_gemm_workspace_size(1, 8192, 8192, 128)
    assert need > 0
    assert lib.awq_w4a16_gemm(p, 1, p, p, p, p, 8192, 8192, 128, p, ctypes.c_void_p(256 + 16), need,
                              None) == awq.AWQ_ERR_INVALID_ARG
    assert lib.awq_w4a16_gemm(p, 1, p, p, p, p, 8192, 8192, 128, p, p, need - 1, None) == awq.AWQ_ERR_WORKSPACE


def test_gemm_workspace_sizes(awq):
    # M <= 16: partials and counters only when K is split; M > 16 adds x/s in operand order
    for M in (1, 7, 16):
        assert awq.awq_w4a16_gemm_workspace_size(M, 8192, 8192, 128) >= 4 * M * 8192 * 2
    assert awq.awq_w4a16_gemm_workspace_size(256, 8192, 8192, 128) >= 256 * 8192 * 2
    assert awq.awq_w4a16_gemm_workspace_size(1, 8192, 8192, 96) == 0


def _host(nbytes, fill=0xA5):
    buf = (ctypes.c_uint8 * nbytes)()
    ctypes.memset(buf, fill, nbytes)
    return buf


def test_rejected_calls_write_nothing(awq):
    """Every rejected call returns before anything is enqueued: buffers passed as outputs (host
    memory here, never dereferenced by the library on these paths) keep their contents."""
    lib = awq.library()
    outs = [_host(4096) for _ in range(6)]
    before = [bytes(b) for b in outs]
    P = [ctypes.cast(b, ctypes.c_void_p) for b in outs]
    src = ctypes.c_void_p(256)
    cfg = awq.qconfig(128, True, 21)
    bad_cfg = awq.qconfig(96, True, 21)
    big = ctypes.c_size_t(1 << 40)
    calls = [
        lib.awq_act_stats(src, 8, 16, P[0], 2, 8, P[1], P[2], big, None),
        lib.awq_act_max(src, 8, 16, P[0], 5, P[1], big, None),
        lib.awq_scale_table(P[0], 16, 1, P[1], None),
        lib.awq_scale_table_ex(P[0], None, 16, 21, 3, P[1], None),
        lib.awq_weight_mean_abs(src, 0, 16, P[0], None),
        lib.awq_search(src, 8, src, 128, 16, src, ctypes.byref(bad_cfg), P[0], big, P[1], P[2], P[3], None),
        lib.awq_search_table(src, 8, src, 100, 16, src, ctypes.byref(cfg), P[0], big, P[1], P[2], P[3], None),
        lib.awq_clip_search(src, 8, src, 128, 16, src, ctypes.byref(cfg), ctypes.c_float(0.0), P[0], big, P[1],
                            P[2], P[3], None),
        lib.awq_pack(src, 128, 16, src, ctypes.byref(bad_cfg), P[0], P[1], P[2], None),
        lib.awq_w4a16_gemm(src, 1, src, src, src, src, 128, 12, 128, P[0], P[1], big, None),
        lib.awq_w4a16_gemm(src, 1, src, src, src, src, 8192, 8192, 128, P[0], P[1], 16, None),
        lib.awq_greedy_search(src, 256, 40, src, ctypes.byref(cfg), 20, 0, P[0], big, P[1], P[2], P[3], None),
    ]
    assert all(st < 0 for st in calls), calls
    assert [bytes(b) for b in outs] == before


def test_binding_checks_shapes_and_dtypes_before_launch(awq):
    """The binding refuses mis-shaped or wrongly typed companions of a call (which the C ABI
    cannot see) before anything reaches the device; CPU tensors show that no launch happens."""
    import torch
    K, N, g, M = 256, 64, 128, 4
    bf, f32 = torch.bfloat16, torch.float32
    X = torch.zeros(M, K, dtype=bf)
    s = torch.ones(K, dtype=f32)
    codes = torch.zeros(K // 8, N, dtype=torch.int32)
    scales = torch.ones(K // g, N, dtype=f32)
    zeros = torch.zeros(K // g, N, dtype=torch.uint8)
    Y = torch.zeros(M, N, dtype=bf)
    ws = torch.zeros(8, dtype=torch.uint8)

    def gemm(**kw):
        a = dict(X=X, s=s, codes=codes, scales=scales, zeros=zeros, group_size=g, Y=Y, ws=ws)
        a.update(kw)
        with pytest.raises(ValueError) as e:
            awq.awq_w4a16_gemm(**a)
        return str(e.value)

    assert "X must be" in gemm(X=X.float())
    assert "s must have shape" in gemm(s=torch.ones(K + 8, dtype=f32))
    assert "codes must" in gemm(codes=torch.zeros(K // 8, N, dtype=torch.int64))
    assert "scales must have shape" in gemm(scales=torch.ones(K // 64, N, dtype=f32))
    assert "zeros must be" in gemm(zeros=zeros.int())
    assert "Y must have shape" in gemm(Y=torch.zeros(M, N + 8, dtype=bf))
    assert "multiple of the group size" in gemm(group_size=96)
    assert "device tensors" in gemm()      # every shape right: only the device check is left

    cfg = awq.qconfig(g, True, 21)
    W = torch.zeros(K, N, dtype=bf)
    m = torch.ones(K, dtype=f32)
    losses = torch.zeros(21, dtype=torch.float64)
    best = torch.zeros(1, dtype=torch.int32)
    sb = torch.zeros(K, dtype=f32)
    for bad in (dict(losses=torch.zeros(20, dtype=torch.float64)), dict(best=torch.zeros(1, dtype=torch.int64)),
                dict(s_best=torch.zeros(K - 8, dtype=f32)), dict(W=torch.zeros(K + 8, N, dtype=bf)),
                dict(mean_abs=m.double())):
        a = dict(X=X, W=W, mean_abs=m, cfg=cfg, ws=ws, losses=losses, best=best, s_best=sb)
        a.update(bad)
        with pytest.raises(ValueError, match="must|is \\["):
            awq.awq_search(**a)
    with pytest.raises(ValueError, match="zeros must"):
        awq.awq_pack(W, s, cfg, codes, scales, zeros.float())
    with pytest.raises(ValueError, match="s_table must"):
        awq.awq_scale_table(m, 21, torch.zeros(20, K, dtype=f32))
    with pytest.raises(ValueError, match="sum_abs must"):
        awq.awq_act_stats(X, torch.zeros(K, dtype=f32), False, M, None, ws)
    with pytest.raises(ValueError, match="losses_each must"):
        awq.awq_search_multi(X, [W, W], m, cfg, ws, losses, torch.zeros(3, 21, dtype=torch.float64), best, sb)
    with pytest.raises(ValueError, match="err must"):
        awq.awq_greedy_search(W, m, cfg, 20, 3, ws, sb, None, torch.zeros(K // g + 1, dtype=torch.float64))
    with pytest.raises(ValueError, match="output must"):
        awq.awq_clip_search(X, W, s, cfg, 0.5, ws, losses, best, torch.zeros(2, dtype=f32))


def test_gemm_rejects_sizes_beyond_buffer_addressing(awq):
    # M > 32 stages x/s and its sums for buffer addressing: x/s at or above 4 GiB is rejected
    lib = awq.library()
    p = ctypes.c_void_p(256)
    M, K, N = 262144, 8192, 64          # M K 2 bytes = 4 GiB
    assert awq.awq_w4a16_gemm_workspace_size(M, K, N, 128) == 0
    assert lib.awq_w4a16_gemm(p, M, p, p, p, p, K, N, 128, p, p, ctypes.c_size_t(1 << 40),
                              None) == awq.AWQ_ERR_INVALID_ARG
    assert awq.awq_w4a16_gemm_workspace_size(M - 64, K, N, 128) > 0   # just below the limit
