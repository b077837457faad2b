"""Seeded synthetic inputs for the AWQ hot path.

This module holds random draws and bf16 casting only -- none of the method's
arithmetic -- so that the fp64 oracle and the HIP path can both be fed from it
without sharing any computation.

The workloads mimic what the pages describe: calibration activations where
about 1% of input channels carry much larger magnitudes than the rest
("大模型 AWQ 量化实战", section 1: most activations ~0.1, 1% salient channels
~50) and Llama-shaped linear layers.  No dataset or trained weight is used; the
pages' pileval calibration set and WikiText2/MMLU/GSM8K evaluations are stood in
for by these distributions.

Recipe (numpy ``default_rng`` / PCG64; draws are float32, in the order listed;
values are cast to bf16 with round-to-nearest-even through torch on the CPU):

``c1``  K=512, N=512, T=256. W = 0.02*N(0,1) [K,N]; X = N(0,1) [T,K];
        idx = choice(K, 5, no replace); X[:, idx] *= 50.  asym, g=128.
``c2``  K=N=4096, T=8192. W = N(0,1)/sqrt(K); mag = lognormal(0,1,K);
        o = choice(K, 41, no replace); mag[o] *= U(20,100) (41 draws);
        X = N(0,1)[T,K] * mag.  asym, g=128.
``c3``  K=11008, N=4096, T=8192. W = N(0,1)/sqrt(K);
        X = silu(N1) * N2 [T,K]; o = choice(K, 110, no replace); X[:, o] *= 30.
        asym, g=128.
``c4``  K=5120, N=13824, T=16384. W = N(0,1)/sqrt(K);
        pos = choice(K*N, 70779, no replace); W.flat[pos] *= 10;
        mag = lognormal(0, 1.5, K); X = N(0,1)[T,K] * mag.  sym, g=64.
``c5``  Seven linears of a 70B-shaped block at T=4096 calibration tokens; each
        distinct input j uses ``default_rng([seed, j])``: X_attn [T,8192]
        (shared by q,k,v), X_o [T,8192], X_mlp [T,8192] (shared by gate,up),
        X_down [T,28672]; each N(0,1) with 1% of channels *50.
        W_l = N(0,1)/sqrt(K_l) with ``default_rng([seed, 100 + l])``.  asym, g=128.
``small(T,K,N,...)``  Parity-test shapes: c1-like draws at any size, used for
        ragged tails (T, N not multiples of the tile sizes).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = ["Layer", "Config", "make_config", "small", "to_bf16", "bf16_to_f64",
           "CONFIG_NAMES", "C5_LAYERS"]

CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5")

# (name, K, N, input index) of the seven linears of the c5 block.
C5_LAYERS = (
    ("q", 8192, 8192, 0), ("k", 8192, 1024, 0), ("v", 8192, 1024, 0),
    ("o", 8192, 8192, 1), ("gate", 8192, 28672, 2), ("up", 8192, 28672, 2),
    ("down", 28672, 8192, 3),
)
_C5_INPUT_K = (8192, 8192, 8192, 28672)


def to_bf16(a: np.ndarray):
    """float32 numpy array -> torch.bfloat16 CPU tensor (round to nearest even)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_to_f64(t) -> np.ndarray:
    """torch bf16 tensor (any device) -> float64 numpy array (exact upcast)."""
    return t.detach().to("cpu").float().numpy().astype(np.float64)


@dataclass
class Layer:
    name: str
    X: object            # torch.bfloat16 [T, K] (CPU)
    W: object            # torch.bfloat16 [K, N] (CPU)
    group_size: int
    zero_point: bool     # True: asymmetric min-max with zero point; False: symmetric absmax


@dataclass
class Config:
    name: str
    layers: List[Layer] = field(default_factory=list)


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def _silu(a):
    return a / (1.0 + np.exp(-a))


def small(T: int, K: int, N: int, seed: int = 0, group_size: int = 128,
          zero_point: bool = True, n_salient: Optional[int] = None,
          salient_gain: float = 50.0, w_std: float = 0.02, w_outlier_frac: float = 0.0,
          w_outlier_gain: float = 10.0) -> Layer:
    """c1-like draws at an arbitrary shape (for parity tests with ragged tails).  With
    w_outlier_frac > 0, that fraction of the weights (drawn last) is multiplied by
    w_outlier_gain, as in c4."""
    rng = np.random.default_rng(seed)
    W = _normal(rng, (K, N)) * np.float32(w_std)
    X = _normal(rng, (T, K))
    ns = max(1, K // 100) if n_salient is None else n_salient
    if ns > 0:
        idx = rng.choice(K, ns, replace=False)
        X[:, idx] *= np.float32(salient_gain)
    if w_outlier_frac > 0:
        pos = rng.choice(K * N, max(1, int(round(w_outlier_frac * K * N))), replace=False)
        W.reshape(-1)[pos] *= np.float32(w_outlier_gain)
    return Layer(f"small_{T}x{K}x{N}", to_bf16(X), to_bf16(W), group_size, zero_point)


def scale_vector(K: int, seed: int = 0, sigma: float = 1.0) -> np.ndarray:
    """A positive float32 per-input-channel scale vector (lognormal draws), standing in for the
    s* of a search when a product is tested on its own."""
    rng = np.random.default_rng(seed)
    return rng.lognormal(0.0, sigma, K).astype(np.float32)


def _c1(seed):
    rng = np.random.default_rng(seed)
    W = _normal(rng, (512, 512)) * np.float32(0.02)
    X = _normal(rng, (256, 512))
    idx = rng.choice(512, 5, replace=False)
    X[:, idx] *= np.float32(50.0)
    return [Layer("c1", to_bf16(X), to_bf16(W), 128, True)]


def _c2(seed):
    K, N, T = 4096, 4096, 8192
    rng = np.random.default_rng(seed)
    W = _normal(rng, (K, N)) / np.float32(np.sqrt(K))
    mag = rng.lognormal(0.0, 1.0, K).astype(np.float32)
    o = rng.choice(K, 41, replace=False)
    mag[o] *= rng.uniform(20.0, 100.0, 41).astype(np.float32)
    X = _normal(rng, (T, K))
    X *= mag[None, :]
    return [Layer("c2", to_bf16(X), to_bf16(W), 128, True)]


def _c3(seed):
    K, N, T = 11008, 4096, 8192
    rng = np.random.default_rng(seed)
    W = _normal(rng, (K, N)) / np.float32(np.sqrt(K))
    X = _silu(_normal(rng, (T, K)))
    X *= _normal(rng, (T, K))
    o = rng.choice(K, 110, replace=False)
    X[:, o] *= np.float32(30.0)
    return [Layer("c3", to_bf16(X), to_bf16(W), 128, True)]


def _c4(seed):
    K, N, T = 5120, 13824, 16384
    rng = np.random.default_rng(seed)
    W = _normal(rng, (K, N)) / np.float32(np.sqrt(K))
    pos = rng.choice(K * N, 70779, replace=False)
    W.reshape(-1)[pos] *= np.float32(10.0)
    mag = rng.lognormal(0.0, 1.5, K).astype(np.float32)
    X = _normal(rng, (T, K))
    X *= mag[None, :]
    return [Layer("c4", to_bf16(X), to_bf16(W), 64, False)]


def c5_input(seed: int, j: int, T: int = 4096):
    """The j-th distinct calibration input of the c5 block (bf16 [T, K_j])."""
    K = _C5_INPUT_K[j]
    rng = np.random.default_rng([seed, j])
    X = _normal(rng, (T, K))
    idx = rng.choice(K, K // 100, replace=False)
    X[:, idx] *= np.float32(50.0)
    return to_bf16(X)


def c5_weight(seed: int, l: int):
    """Weight of the l-th c5 linear (bf16 [K, N])."""
    name, K, N, _ = C5_LAYERS[l]
    rng = np.random.default_rng([seed, 100 + l])
    W = _normal(rng, (K, N)) / np.float32(np.sqrt(K))
    return to_bf16(W)


def _c5(seed, layers=None):
    out = []
    xs: Dict[int, object] = {}
    for l, (name, K, N, j) in enumerate(C5_LAYERS):
        if layers is not None and name not in layers:
            continue
        if j not in xs:
            xs[j] = c5_input(seed, j)
        out.append(Layer(f"c5.{name}", xs[j], c5_weight(seed, l), 128, True))
    return out


def make_config(name: str, seed: int = 0, layers: Optional[Tuple[str, ...]] = None) -> Config:
    """Build config ``name`` (c1..c5) with the recipe in the module docstring."""
    if name == "c1":
        ls = _c1(seed)
    elif name == "c2":
        ls = _c2(seed)
    elif name == "c3":
        ls = _c3(seed)
    elif name == "c4":
        ls = _c4(seed)
    elif name == "c5":
        ls = _c5(seed, layers)
    else:
        raise ValueError(f"unknown config {name!r}")
    return Config(name, ls)
