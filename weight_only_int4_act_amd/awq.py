"""Thin Python binding of libawq (include/awq.h).

Argument marshalling only: every function passes device pointers of torch tensors, sizes and
the current HIP stream to the C entry point of the same name, and raises ``AwqError`` on a
non-zero status.  torch is used for device memory and streams; every step of the path runs
in the library's HIP kernels.  If ``libawq.so`` has not been built the import of this module
fails loudly -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# AWQ_LIBRARY names another build of the same ABI to load instead (the LDS-poison debug build,
# libawq_ldspoison.so, for the race test); the product path loads libawq.so
LIB_PATH = os.environ.get("AWQ_LIBRARY") or os.path.join(_PKG, "libawq.so")

AWQ_OK = 0
AWQ_ERR_INVALID_ARG = -1
AWQ_ERR_UNSUPPORTED = -2
AWQ_ERR_WORKSPACE = -3
AWQ_ERR_HIP = -4
AWQ_ERR_SCRATCH = -5
AWQ_MAX_POW2_CANDIDATES = 32   # most power-of-two candidates of awq_greedy_search
AWQ_MAX_PROJECTIONS = 16   # most matrices one awq_search_multi call takes


class AwqError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str, hip: int = 0):
        super().__init__(f"{fn} failed with status {status}: {msg}" + (f" (hipError {hip})" if hip else ""))
        self.status = status
        self.hip_error = hip


class awq_qconfig(ctypes.Structure):
    _fields_ = [("w_bit", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("zero_point", ctypes.c_int32), ("n_grid", ctypes.c_int32), ("clip_ratio", ctypes.c_float)]


def qconfig(group_size: int = 128, zero_point: bool = True, n_grid: int = 21, w_bit: int = 4,
            clip_ratio: float = 1.0) -> awq_qconfig:
    return awq_qconfig(int(w_bit), int(group_size), 1 if zero_point else 0, int(n_grid), float(clip_ratio))


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_CFG = ctypes.POINTER(awq_qconfig)

_SIGNATURES = {
    "awq_act_stats_workspace_size": (_SZ, [_I64, _I64]),
    "awq_act_stats": (ctypes.c_int, [_P, _I64, _I64, _P, ctypes.c_int, _I64, _P, _P, _SZ, _P]),
    "awq_scale_table": (ctypes.c_int, [_P, _I64, _I32, _P, _P]),
    "awq_search_workspace_size": (_SZ, [_I64, _I64, _I64, _CFG]),
    "awq_search": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _P, _CFG, _P, _SZ, _P, _P, _P, _P]),
    "awq_pack": (ctypes.c_int, [_P, _I64, _I64, _P, _CFG, _P, _P, _P, _P]),
    "awq_clip_search": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _P, _CFG, ctypes.c_float, _P, _SZ, _P, _P, _P, _P]),
    "awq_search_table": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _P, _CFG, _P, _SZ, _P, _P, _P, _P]),
    "awq_search_multi_workspace_size": (_SZ, [_I64, _I64, _I32, _P, _CFG]),
    "awq_search_multi": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _I64, _P, _CFG, _P, _SZ, _P, _P, _P, _P, _P]),
    "awq_greedy_workspace_size": (_SZ, [_I64, _I64, _CFG, _I32]),
    "awq_greedy_search": (ctypes.c_int, [_P, _I64, _I64, _P, _CFG, _I32, _I32, _P, _SZ, _P, _P, _P, _P]),
    "awq_act_max": (ctypes.c_int, [_P, _I64, _I64, _P, ctypes.c_int, _P, _SZ, _P]),
    "awq_weight_mean_abs": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "awq_scale_table_ex": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _P, _P]),
    "awq_w4a16_gemm_workspace_size": (_SZ, [_I64, _I64, _I64, _I32]),
    "awq_w4a16_gemm": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _I64, _I32, _P, _P, _SZ, _P]),
    "awq_w4a16_gemm_static_scratch_bytes": (_SZ, []),
    "awq_w4a16_gemm_noalloc": (ctypes.c_int, [_P, _I64, _P, _P, _P, _P, _I64, _I64, _I32, _P, _P]),
    "awq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "awq_last_hip_error": (ctypes.c_int, []),
    "awq_version": (ctypes.c_char_p, []),
}
EXPORTED = tuple(_SIGNATURES)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m weight_only_int4_act_amd.build` "
                          "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


_CODE_DTYPES = tuple(d for d in (torch.int32, getattr(torch, "uint32", None)) if d is not None)


def _expect(fn: str, name: str, t: Optional[torch.Tensor], dtypes, shape, optional: bool = False) -> None:
    """Refuse a tensor whose dtype or shape differs from what the C entry point will assume: the
    C ABI receives only pointers and the sizes taken from the other arguments, so a mis-shaped
    buffer would otherwise be read or written out of bounds on the device."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{fn}: {name} is required")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{fn}: {name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{fn}: {name} must have shape {tuple(int(v) for v in shape)}, got {tuple(t.shape)}")


def _matrix(fn: str, name: str, t: torch.Tensor, dtype=torch.bfloat16):
    if t.dim() != 2:
        raise ValueError(f"{fn}: {name} must be a matrix, got shape {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{fn}: {name} must be {dtype}, got {t.dtype}")
    return t.shape


def _group_rows(fn: str, K: int, g: int) -> int:
    if g <= 0 or K % g or K % 8:
        raise ValueError(f"{fn}: K = {K} must be a multiple of the group size {g} and of 8")
    return K // g


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libawq takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libawq takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, status: int) -> None:
    if status != AWQ_OK:
        msg = _lib.awq_status_string(status).decode()
        raise AwqError(fn, status, msg, _lib.awq_last_hip_error() if status == AWQ_ERR_HIP else 0)


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-filled device scratch of at least ``nbytes`` bytes (256-byte aligned by torch).  Zero
    filling is what awq_w4a16_gemm's arrival counters need before their first use."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points
def awq_act_stats_workspace_size(T: int, K: int) -> int:
    return int(_lib.awq_act_stats_workspace_size(T, K))


def awq_act_stats(X: torch.Tensor, sum_abs: torch.Tensor, accumulate: bool, total_tokens: int,
                  mean_abs: Optional[torch.Tensor], ws: torch.Tensor, stream=None) -> None:
    T, K = _matrix("awq_act_stats", "X", X)
    _expect("awq_act_stats", "sum_abs", sum_abs, torch.float64, (K,))
    _expect("awq_act_stats", "mean_abs", mean_abs, torch.float32, (K,), optional=True)
    _check("awq_act_stats", _lib.awq_act_stats(_ptr(X), T, K, _ptr(sum_abs), 1 if accumulate else 0,
                                               int(total_tokens), _ptr(mean_abs), _ptr(ws), _nbytes(ws),
                                               _stream(stream)))


def awq_scale_table(mean_abs: torch.Tensor, n_grid: int, s_table: torch.Tensor, stream=None) -> None:
    _expect("awq_scale_table", "mean_abs", mean_abs, torch.float32, (mean_abs.numel(),))
    _expect("awq_scale_table", "s_table", s_table, torch.float32, (n_grid, mean_abs.numel()))
    _check("awq_scale_table", _lib.awq_scale_table(_ptr(mean_abs), mean_abs.numel(), int(n_grid),
                                                   _ptr(s_table), _stream(stream)))


def awq_search_workspace_size(T: int, K: int, N: int, cfg: awq_qconfig) -> int:
    return int(_lib.awq_search_workspace_size(T, K, N, ctypes.byref(cfg)))


def _search_outputs(fn: str, X, W, vec, vec_shape, cfg, losses, best, out, out_shape):
    T, K = _matrix(fn, "X", X)
    K2, N = _matrix(fn, "W", W)
    if K2 != K:
        raise ValueError(f"{fn}: X is [T, {K}] but W is [{K2}, N]")
    _expect(fn, "scales", vec, torch.float32, vec_shape)
    _expect(fn, "losses", losses, torch.float64, (cfg.n_grid,))
    _expect(fn, "best", best, torch.int32, (1,))
    _expect(fn, "output", out, torch.float32, out_shape)
    return T, K, N


def awq_search(X: torch.Tensor, W: torch.Tensor, mean_abs: torch.Tensor, cfg: awq_qconfig, ws: torch.Tensor,
               losses: torch.Tensor, best: torch.Tensor, s_best: torch.Tensor, stream=None) -> None:
    T, K, N = _search_outputs("awq_search", X, W, mean_abs, (X.shape[-1],), cfg, losses, best, s_best,
                              (X.shape[-1],))
    _check("awq_search", _lib.awq_search(_ptr(X), T, _ptr(W), K, N, _ptr(mean_abs), ctypes.byref(cfg), _ptr(ws),
                                         _nbytes(ws), _ptr(losses), _ptr(best), _ptr(s_best), _stream(stream)))


def awq_pack(W: torch.Tensor, s: torch.Tensor, cfg: awq_qconfig, codes: torch.Tensor, scales: torch.Tensor,
             zeros: torch.Tensor, stream=None) -> None:
    K, N = _matrix("awq_pack", "W", W)
    ng = _group_rows("awq_pack", K, cfg.group_size)
    _expect("awq_pack", "s", s, torch.float32, (K,))
    _expect("awq_pack", "codes", codes, _CODE_DTYPES, (K // 8, N))
    _expect("awq_pack", "scales", scales, torch.float32, (ng, N))
    _expect("awq_pack", "zeros", zeros, torch.uint8, (ng, N))
    _check("awq_pack", _lib.awq_pack(_ptr(W), K, N, _ptr(s), ctypes.byref(cfg), _ptr(codes), _ptr(scales),
                                     _ptr(zeros), _stream(stream)))


def awq_act_max(X: torch.Tensor, max_abs: torch.Tensor, accumulate: bool, ws: torch.Tensor, stream=None) -> None:
    T, K = _matrix("awq_act_max", "X", X)
    _expect("awq_act_max", "max_abs", max_abs, torch.float32, (K,))
    _check("awq_act_max", _lib.awq_act_max(_ptr(X), T, K, _ptr(max_abs), 1 if accumulate else 0, _ptr(ws),
                                           _nbytes(ws), _stream(stream)))


def awq_weight_mean_abs(W: torch.Tensor, w_mean: torch.Tensor, stream=None) -> None:
    K, N = _matrix("awq_weight_mean_abs", "W", W)
    _expect("awq_weight_mean_abs", "w_mean", w_mean, torch.float32, (K,))
    _check("awq_weight_mean_abs", _lib.awq_weight_mean_abs(_ptr(W), K, N, _ptr(w_mean), _stream(stream)))


def awq_scale_table_ex(stat: torch.Tensor, w_mean: Optional[torch.Tensor], n_grid: int, normalize: bool,
                       s_table: torch.Tensor, stream=None) -> None:
    K = stat.numel()
    _expect("awq_scale_table_ex", "stat", stat, torch.float32, (K,))
    _expect("awq_scale_table_ex", "w_mean", w_mean, torch.float32, (K,), optional=True)
    _expect("awq_scale_table_ex", "s_table", s_table, torch.float32, (n_grid, K))
    _check("awq_scale_table_ex", _lib.awq_scale_table_ex(_ptr(stat), _ptr(w_mean) if w_mean is not None else None,
                                                         stat.numel(), int(n_grid), 1 if normalize else 0,
                                                         _ptr(s_table), _stream(stream)))


def awq_search_table(X: torch.Tensor, W: torch.Tensor, s_table: torch.Tensor, cfg: awq_qconfig, ws: torch.Tensor,
                     losses: torch.Tensor, best: torch.Tensor, s_best: torch.Tensor, stream=None) -> None:
    T, K, N = _search_outputs("awq_search_table", X, W, s_table, (cfg.n_grid, X.shape[-1]), cfg, losses, best,
                              s_best, (X.shape[-1],))
    _check("awq_search_table", _lib.awq_search_table(_ptr(X), T, _ptr(W), K, N, _ptr(s_table), ctypes.byref(cfg),
                                                     _ptr(ws), _nbytes(ws), _ptr(losses), _ptr(best), _ptr(s_best),
                                                     _stream(stream)))


def awq_clip_search(X: torch.Tensor, W: torch.Tensor, s: torch.Tensor, cfg: awq_qconfig, clip_min: float,
                    ws: torch.Tensor, losses: torch.Tensor, best: torch.Tensor, clip_best: torch.Tensor,
                    stream=None) -> None:
    T, K, N = _search_outputs("awq_clip_search", X, W, s, (X.shape[-1],), cfg, losses, best, clip_best, (1,))
    _check("awq_clip_search", _lib.awq_clip_search(_ptr(X), T, _ptr(W), K, N, _ptr(s), ctypes.byref(cfg),
                                                   float(clip_min), _ptr(ws), _nbytes(ws), _ptr(losses),
                                                   _ptr(best), _ptr(clip_best), _stream(stream)))


def awq_w4a16_gemm_workspace_size(M: int, K: int, N: int, group_size: int) -> int:
    return int(_lib.awq_w4a16_gemm_workspace_size(M, K, N, group_size))


def awq_w4a16_gemm(X: torch.Tensor, s: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                   zeros: torch.Tensor, group_size: int, Y: torch.Tensor, ws: Optional[torch.Tensor],
                   stream=None) -> None:
    fn = "awq_w4a16_gemm"
    M, K = _matrix(fn, "X", X)
    _, N = _matrix(fn, "codes", codes, codes.dtype if codes.dtype in _CODE_DTYPES else torch.int32)
    ng = _group_rows(fn, K, int(group_size))
    _expect(fn, "s", s, torch.float32, (K,))
    _expect(fn, "codes", codes, _CODE_DTYPES, (K // 8, N))
    _expect(fn, "scales", scales, torch.float32, (ng, N))
    _expect(fn, "zeros", zeros, torch.uint8, (ng, N))
    _expect(fn, "Y", Y, torch.bfloat16, (M, N))
    _check("awq_w4a16_gemm", _lib.awq_w4a16_gemm(_ptr(X), M, _ptr(s), _ptr(codes), _ptr(scales), _ptr(zeros),
                                                 K, N, int(group_size), _ptr(Y), _ptr(ws), _nbytes(ws),
                                                 _stream(stream)))


def awq_w4a16_gemm_static_scratch_bytes() -> int:
    return int(_lib.awq_w4a16_gemm_static_scratch_bytes())


def awq_w4a16_gemm_noalloc(X: torch.Tensor, s: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                           zeros: torch.Tensor, group_size: int, Y: torch.Tensor, stream=None) -> None:
    fn = "awq_w4a16_gemm_noalloc"
    M, K = _matrix(fn, "X", X)
    _, N = _matrix(fn, "codes", codes, codes.dtype if codes.dtype in _CODE_DTYPES else torch.int32)
    ng = _group_rows(fn, K, int(group_size))
    _expect(fn, "s", s, torch.float32, (K,))
    _expect(fn, "codes", codes, _CODE_DTYPES, (K // 8, N))
    _expect(fn, "scales", scales, torch.float32, (ng, N))
    _expect(fn, "zeros", zeros, torch.uint8, (ng, N))
    _expect(fn, "Y", Y, torch.bfloat16, (M, N))
    _check(fn, _lib.awq_w4a16_gemm_noalloc(_ptr(X), M, _ptr(s), _ptr(codes), _ptr(scales), _ptr(zeros), K, N,
                                           int(group_size), _ptr(Y), _stream(stream)))


def awq_status_string(status: int) -> str:
    return _lib.awq_status_string(status).decode()


def awq_version() -> str:
    return _lib.awq_version().decode()


# ------------------------------------------------------------------ allocation helpers (plumbing only)
class Quantized:
    """Device buffers of one packed layer: codes uint32 [K/8, N] (stored as int32), scales float32
    [K/g, N], zeros uint8 [K/g, N], the input scales s* [K] and the group size."""

    def __init__(self, codes, scales, zeros, s, group_size):
        self.codes, self.scales, self.zeros, self.s, self.group_size = codes, scales, zeros, s, group_size


def run_layer(X: torch.Tensor, W: torch.Tensor, cfg: awq_qconfig, stream=None) -> dict:
    """Allocate outputs and run stats -> search -> pack for one layer on the current device."""
    dev = X.device
    T, K = X.shape
    N = W.shape[1]
    sum_abs = torch.empty(K, dtype=torch.float64, device=dev)
    mean_abs = torch.empty(K, dtype=torch.float32, device=dev)
    ws_stats = workspace(awq_act_stats_workspace_size(T, K), dev)
    awq_act_stats(X, sum_abs, False, T, mean_abs, ws_stats, stream)
    ws = workspace(awq_search_workspace_size(T, K, N, cfg), dev)
    losses = torch.empty(cfg.n_grid, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    s_best = torch.empty(K, dtype=torch.float32, device=dev)
    awq_search(X, W, mean_abs, cfg, ws, losses, best, s_best, stream)
    g = cfg.group_size
    codes = torch.empty((K // 8, N), dtype=torch.int32, device=dev)
    scales = torch.empty((K // g, N), dtype=torch.float32, device=dev)
    zeros = torch.empty((K // g, N), dtype=torch.uint8, device=dev)
    awq_pack(W, s_best, cfg, codes, scales, zeros, stream)
    return {"sum_abs": sum_abs, "mean_abs": mean_abs, "losses": losses, "best": best,
            "q": Quantized(codes, scales, zeros, s_best, g)}


def gemm(X: torch.Tensor, q: Quantized, stream=None) -> torch.Tensor:
    M, K = X.shape
    N = q.codes.shape[1]
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    ws = workspace(awq_w4a16_gemm_workspace_size(M, K, N, q.group_size), X.device)
    awq_w4a16_gemm(X, q.s, q.codes, q.scales, q.zeros, q.group_size, Y, ws, stream)
    return Y


def _host_arrays(Ns, Ws=()):
    n = len(Ns)
    N = (ctypes.c_int64 * n)(*[int(v) for v in Ns])
    P = (ctypes.c_void_p * n)(*[W.data_ptr() for W in Ws]) if Ws else None
    return N, P


def awq_search_multi_workspace_size(T: int, K: int, Ns, cfg: awq_qconfig) -> int:
    N, _ = _host_arrays(Ns)
    return int(_lib.awq_search_multi_workspace_size(T, K, len(Ns), N, ctypes.byref(cfg)))


def awq_search_multi(X: torch.Tensor, Ws, mean_abs: torch.Tensor, cfg: awq_qconfig, ws: torch.Tensor,
                     losses: torch.Tensor, losses_each: Optional[torch.Tensor], best: torch.Tensor,
                     s_best: torch.Tensor, stream=None) -> None:
    fn = "awq_search_multi"
    T, K = _matrix(fn, "X", X)
    for W in Ws:
        if _matrix(fn, "W", W)[0] != K:
            raise ValueError(f"{fn}: X is [T, {K}] but a projection is {tuple(W.shape)}")
    _expect(fn, "mean_abs", mean_abs, torch.float32, (K,))
    _expect(fn, "losses", losses, torch.float64, (cfg.n_grid,))
    _expect(fn, "losses_each", losses_each, torch.float64, (len(Ws), cfg.n_grid), optional=True)
    _expect(fn, "best", best, torch.int32, (1,))
    _expect(fn, "s_best", s_best, torch.float32, (K,))
    for W in Ws:
        _ptr(W)
    N, P = _host_arrays([W.shape[1] for W in Ws], Ws)
    _check("awq_search_multi", _lib.awq_search_multi(_ptr(X), T, len(Ws), P, N, K, _ptr(mean_abs),
                                                     ctypes.byref(cfg), _ptr(ws), _nbytes(ws), _ptr(losses),
                                                     _ptr(losses_each), _ptr(best), _ptr(s_best),
                                                     _stream(stream)))


def run_multi(X: torch.Tensor, Ws, cfg: awq_qconfig, stream=None) -> dict:
    """Statistic of the shared X, one joint search over the projections Ws, and each projection
    packed at the shared s*: the layers that read X are quantized with one scale vector."""
    dev = X.device
    T, K = X.shape
    sum_abs = torch.empty(K, dtype=torch.float64, device=dev)
    mean_abs = torch.empty(K, dtype=torch.float32, device=dev)
    awq_act_stats(X, sum_abs, False, T, mean_abs, workspace(awq_act_stats_workspace_size(T, K), dev), stream)
    ws = workspace(awq_search_multi_workspace_size(T, K, [W.shape[1] for W in Ws], cfg), dev)
    losses = torch.empty(cfg.n_grid, dtype=torch.float64, device=dev)
    each = torch.empty((len(Ws), cfg.n_grid), dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    s_best = torch.empty(K, dtype=torch.float32, device=dev)
    awq_search_multi(X, Ws, mean_abs, cfg, ws, losses, each, best, s_best, stream)
    g = cfg.group_size
    qs = []
    for W in Ws:
        N = W.shape[1]
        codes = torch.empty((K // 8, N), dtype=torch.int32, device=dev)
        scales = torch.empty((K // g, N), dtype=torch.float32, device=dev)
        zeros = torch.empty((K // g, N), dtype=torch.uint8, device=dev)
        awq_pack(W, s_best, cfg, codes, scales, zeros, stream)
        qs.append(Quantized(codes, scales, zeros, s_best, g))
    return {"mean_abs": mean_abs, "losses": losses, "each": each, "best": best, "s_best": s_best, "q": qs}


def awq_greedy_workspace_size(K: int, N: int, cfg: awq_qconfig, n_cand: int = 20) -> int:
    return int(_lib.awq_greedy_workspace_size(K, N, ctypes.byref(cfg), int(n_cand)))


def awq_greedy_search(W: torch.Tensor, mean_abs: torch.Tensor, cfg: awq_qconfig, n_cand: int, passes: int,
                      ws: torch.Tensor, s_best: torch.Tensor, err_rtn: Optional[torch.Tensor] = None,
                      err: Optional[torch.Tensor] = None, stream=None) -> None:
    fn = "awq_greedy_search"
    K, N = _matrix(fn, "W", W)
    ng = _group_rows(fn, K, cfg.group_size)
    _expect(fn, "mean_abs", mean_abs, torch.float32, (K,))
    _expect(fn, "s_best", s_best, torch.float32, (K,))
    _expect(fn, "err_rtn", err_rtn, torch.float64, (ng,), optional=True)
    _expect(fn, "err", err, torch.float64, (ng,), optional=True)
    _check("awq_greedy_search", _lib.awq_greedy_search(_ptr(W), K, N, _ptr(mean_abs), ctypes.byref(cfg), int(n_cand),
                                                       int(passes), _ptr(ws), _nbytes(ws), _ptr(s_best),
                                                       _ptr(err_rtn), _ptr(err), _stream(stream)))


def run_greedy(X: torch.Tensor, W: torch.Tensor, cfg: awq_qconfig, n_cand: int = 20, passes: int = 3,
               stream=None) -> dict:
    """Statistic of X, the power-of-two greedy over W's scales, and W packed at the result."""
    dev = X.device
    T, K = X.shape
    N = W.shape[1]
    sum_abs = torch.empty(K, dtype=torch.float64, device=dev)
    mean_abs = torch.empty(K, dtype=torch.float32, device=dev)
    awq_act_stats(X, sum_abs, False, T, mean_abs, workspace(awq_act_stats_workspace_size(T, K), dev), stream)
    ws = workspace(awq_greedy_workspace_size(K, N, cfg, n_cand), dev)
    s_best = torch.empty(K, dtype=torch.float32, device=dev)
    err_rtn = torch.empty(K // cfg.group_size, dtype=torch.float64, device=dev)
    err = torch.empty_like(err_rtn)
    awq_greedy_search(W, mean_abs, cfg, n_cand, passes, ws, s_best, err_rtn, err, stream)
    g = cfg.group_size
    codes = torch.empty((K // 8, N), dtype=torch.int32, device=dev)
    scales = torch.empty((K // g, N), dtype=torch.float32, device=dev)
    zeros = torch.empty((K // g, N), dtype=torch.uint8, device=dev)
    awq_pack(W, s_best, cfg, codes, scales, zeros, stream)
    return {"mean_abs": mean_abs, "s_best": s_best, "err_rtn": err_rtn, "err": err,
            "q": Quantized(codes, scales, zeros, s_best, g)}
