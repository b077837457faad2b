"""Plain fp64 CPU oracle for the AWQ hot path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never uses it, and it shares no code, tables or constants with the HIP
path; it imports nothing from the product package.

Everything here is float64 numpy, written to be checked against the pages by eye:
no blocking, no fusion, no reordering beyond what each definition states.  A
library matmul (BLAS dgemm) is used as a step where the definition is a matrix
product.

Sources (page title -- section):

* [P1] "AWQ (Activation-aware Weight Quantization)" (compassingai.com concept
  page) -- sections 量化数学基础 (per-group quantizer), AWQ 的缩放如何改变量化误差
  (error analysis), 重要通道识别的统计依据 (per-channel statistic),
  缩放因子优化的完整流程 (steps 1-6 of the search), 推理时的等效实现 (offline
  quantization and the online W4A16 product).
* [P2] "大模型 AWQ 量化实战：激活感知权重量化（Activation-aware Weight
  Quantization）部署" (CSDN) -- section 2, the ``quant_config`` with
  ``zero_point``, ``q_group_size`` and ``w_bit``.
* [P3] "AWQ 激活感知量化" (aiqz.cc) -- section 1 (importance E|X_i|), section 4
  (symmetric quantizer, worked values), section 5 (relative error epsilon),
  section 6 (memory model M = N*b/8, R = 16/b).
* [P4] "009. AWQ Integration" (blog.yoooo.fun) -- 关键设计 3: the search scores
  exactly the quantizer that packing uses; Consequences: 4-bit packing, two
  weights per byte.
* [P5] "量化推理算法 GPTQ / AWQ" (slowleelab) -- 4.3 AWQ search loop (keep the
  best loss with a strict "<", so the first minimum wins).
* [P4] 架构 and 关键设计 5: the config carries an optional clip_ratio, a min-max
  clipping of the group range applied before the search (default: none).

Readings where the pages are silent or disagree (each is listed with its reason
in the design notes of the repository):

* statistic is mean |x| over all calibration tokens; stored as float32;
* scale family s_k(alpha) = max(m_k, 1e-8)**alpha, unnormalised, alpha_i = i/20,
  evaluated in float64 and rounded once to float32;
* asymmetric quantizer: the group range is widened to include 0,
  Delta = fl32((max - min)/15) (Delta := 1 if it is 0), zero = clamp(rne(-min/Delta), 0, 15),
  code = clamp(rne(p/Delta) + zero, 0, 15);
* symmetric quantizer: Delta = fl32(max|p|/7) (1 if 0), level = clamp(rne(p/Delta), -7, 7),
  stored code = level + 8, zero = 8 (so one dequant formula (code - zero)*Delta serves both);
* rounding is round-half-to-even;
* loss is the plain sum of squares ||X (What - W)||^2, argmin takes the smallest alpha
  among equal losses;
* clipping with ratio c in (0, 1] multiplies both ends of the group range (0 included)
  by c before Delta and zero are formed; codes beyond the clipped range clamp to its end
  levels; c = 1 is the unclipped quantizer.  A clip search scores c_j = 1 - (1 - c_min)
  j/(n-1), j = 0..n-1, at fixed scales s with the same loss and takes the first minimum.

* power-of-two greedy ([P4] 关键设计 1-3): candidates c_j = 2**(j - n//2), j = 0..n-1
  (n = 20: 2**-10 .. 2**9, 1 among them), s starts at 1; for each group independently, each
  pass visits its channels in ascending order and sets s_k to the candidate with the smallest
  group error, keeping the current value unless another is strictly smaller (scanning the
  candidates in ascending order); the group error is sum_n sum_{i in group} (m_i (What_in -
  W_in))^2 with What from the packing quantizer and m_i = mean |x_i|.

No function here is "parity unpinned": each is pinned by tests under
``tests/test_oracle_*.py`` against worked values, closed forms, invariants and
brute force.
"""
from __future__ import annotations

import numpy as np

SCALE_FLOOR = 1e-8   # floor on the statistic before taking powers (degenerate zero channels)
INT4_LEVELS = 16     # [P3] section 4: INT4 has 16 levels


# ----------------------------------------------------------------------------- a1
def act_stats(X: np.ndarray, sum_abs: np.ndarray | None = None,
              total_tokens: int | None = None):
    """Per-input-channel statistic m_k = (1/T) sum_t |x_tk|.

    [P1] 重要通道识别的统计依据 (activation_scale[j] = mean |X_calib[:, j]|) and
    [P3] section 1 (I_i = E[|X_i|], an average over the calibration samples).

    ``X`` is float64 [T, K] (exact upcast of the bf16 input).  ``sum_abs`` (float64
    [K]) lets the statistic be accumulated over several calibration batches; then
    ``total_tokens`` is the token count over all batches.  Returns
    (sum_abs float64 [K], mean_abs float32 [K]); the float32 mean is the stored
    statistic that everything downstream consumes.
    """
    X = np.asarray(X, dtype=np.float64)
    s = np.abs(X).sum(axis=0)
    if sum_abs is not None:
        s = np.asarray(sum_abs, dtype=np.float64) + s
    n = X.shape[0] if total_tokens is None else int(total_tokens)
    return s, (s / n).astype(np.float32)


def act_max(X: np.ndarray, max_abs: np.ndarray | None = None) -> np.ndarray:
    """Per-input-channel statistic max_t |x_tk|, the alternative that [P1] 重要通道识别的统计依据
    names next to the mean ("或 max").  ``max_abs`` (float32 [K]) accumulates it over
    calibration batches.  float32 [K]; exact (the max of bf16 magnitudes)."""
    m = np.abs(np.asarray(X, dtype=np.float64)).max(axis=0)
    if max_abs is not None:
        m = np.maximum(m, np.asarray(max_abs, dtype=np.float64))
    return m.astype(np.float32)


def weight_mean_abs(W: np.ndarray) -> np.ndarray:
    """mean_j |W_kj| over the output columns of input channel k: the denominator of the closed
    form of [P3] section 3.  Summed in float64, divided by N, rounded once to float32 [K]."""
    W = np.asarray(W, dtype=np.float64)
    return (np.abs(W).sum(axis=1) / W.shape[1]).astype(np.float32)


# ----------------------------------------------------------------------------- a2
def alpha_grid(n_grid: int = 21) -> np.ndarray:
    """alpha_i = i/(n_grid-1): [P1] 缩放因子优化的完整流程 step 3, {0, 0.05, ..., 1.0}."""
    return np.arange(n_grid, dtype=np.float64) / float(n_grid - 1)


def scale_table_ex(stat: np.ndarray, n_grid: int = 21, w_mean: np.ndarray | None = None,
                   normalize: bool = False) -> np.ndarray:
    """Variants of the scale family, each row rounded once to float32 from float64:
    t[i, k] = max(stat_k, 1e-8) ** alpha_i, divided by max(w_mean_k, 1e-8) when ``w_mean`` is
    given ([P3] section 3: s_i* = (E|X_i|)^alpha / mean_j |W_ij|), and divided by the row's
    maximum when ``normalize`` ([P3] section Python 演示: the demo divides s by its maximum); stat is mean |x| or
    max |x| ([P1] 重要通道识别的统计依据)."""
    m = np.maximum(np.asarray(stat, dtype=np.float32).astype(np.float64), SCALE_FLOOR)
    a = alpha_grid(n_grid)
    t = m[None, :] ** a[:, None]
    if w_mean is not None:
        t = t / np.maximum(np.asarray(w_mean, dtype=np.float32).astype(np.float64), SCALE_FLOOR)[None, :]
    if normalize:
        t = t / t.max(axis=1, keepdims=True)
    return t.astype(np.float32)


def scale_table(mean_abs: np.ndarray, n_grid: int = 21) -> np.ndarray:
    """s[i, k] = fl32(max(m_k, 1e-8) ** alpha_i) -- [P1] step 3, s_j(alpha) = activation_scale[j]**alpha."""
    m = np.maximum(np.asarray(mean_abs, dtype=np.float32).astype(np.float64), SCALE_FLOOR)
    a = alpha_grid(n_grid)
    return np.power(m[None, :], a[:, None]).astype(np.float32)


# ----------------------------------------------------------------------------- quantizer
def quantize_groups(P: np.ndarray, group_size: int, zero_point: bool, clip: float = 1.0):
    """Group-wise INT4 quantization of P (float64 [K, N]) along K, per output column.

    [P1] 量化数学基础 (per-group step, round, clamp), [P3] section 4 (symmetric
    absmax: Delta = max|w_s| / (2**(b-1) - 1) = max|w_s|/7), [P2] section 2
    (``zero_point`` selects the min-max form with a zero point), [P4] 关键设计 5
    (optional min-max clipping: ``clip`` scales both ends of the range, float64).

    Returns (codes int64 [K, N] in 0..15, delta float32 [K/g, N], zero int64 [K/g, N]).
    The dequantized value of an element is (code - zero) * delta.
    """
    P = np.asarray(P, dtype=np.float64)
    K, N = P.shape
    g = int(group_size)
    c = float(np.float32(clip))
    G = P.reshape(K // g, g, N)
    if zero_point:
        mx = np.maximum(G.max(axis=1), 0.0) * c
        mn = np.minimum(G.min(axis=1), 0.0) * c
        delta = ((mx - mn) / 15.0).astype(np.float32)
        delta[delta == 0] = 1.0
        d = delta.astype(np.float64)
        zero = np.clip(np.rint(-mn / d), 0, 15)
        codes = np.clip(np.rint(G / d[:, None, :]) + zero[:, None, :], 0, 15)
    else:
        amax = np.abs(G).max(axis=1) * c
        delta = (amax / 7.0).astype(np.float32)
        delta[delta == 0] = 1.0
        d = delta.astype(np.float64)
        zero = np.full(amax.shape, 8.0)
        codes = np.clip(np.rint(G / d[:, None, :]), -7, 7) + 8
    return codes.reshape(K, N).astype(np.int64), delta, zero.astype(np.int64)


def pre_round_values(P: np.ndarray, delta: np.ndarray, group_size: int, zero_point: bool,
                     clip: float = 1.0):
    """The values that the quantizer rounds: p/Delta per element and, for the
    asymmetric form, -min/Delta per group.  Used only to count near-ties."""
    P = np.asarray(P, dtype=np.float64)
    K, N = P.shape
    g = int(group_size)
    d = np.repeat(delta.astype(np.float64), g, axis=0)
    t = P / d
    if zero_point:
        G = P.reshape(K // g, g, N)
        mn = np.minimum(G.min(axis=1), 0.0) * float(np.float32(clip))
        tz = -mn / delta.astype(np.float64)
    else:
        tz = np.zeros(delta.shape)
    return t, tz


def near_tie(t: np.ndarray, rel: float = 1e-5) -> np.ndarray:
    """True where t lies within rel*max(1,|t|) of a .5 rounding boundary."""
    f = np.abs(t - np.floor(t) - 0.5)
    return f <= rel * np.maximum(1.0, np.abs(t))


def loss_tie_variants(X: np.ndarray, W: np.ndarray, s: np.ndarray, group_size: int, zero_point: bool,
                      clip: float = 1.0, rel: float = 1e-5, max_ties: int = 22) -> np.ndarray:
    """L = ||X (S^-1 Q'(S W) - W)||^2 for every admissible rounding Q' of the near-tie elements.

    An element whose pre-round value p/Delta lies within ``rel`` of a .5 boundary (``near_tie``)
    may take either neighbouring level, floor(p/Delta) or floor(p/Delta) + 1: both are correct
    roundings up to the precision in which p/Delta is evaluated ([P3] section 4 rounds to the
    nearest level; at a tie either neighbour is equally near).  Every other element keeps the
    quantizer's level, and the step and zero of each group are the quantizer's.  A tie level is
    taken as is, beyond the code range by one step at a tied range end, unless the range is
    clipped (c < 1), where levels clamp to the clipped range as in ``quantize_groups``.

    The loss is a sum over output columns, ||X E||^2 = sum_n ||X e_n||^2, and an element's level
    enters only its own column e_n, so the choices are enumerated column by column: each column
    with ties contributes the change of its own loss under each of its 2**m roundings, and every
    combination's loss is the base loss plus one change per column.

    Returns the 2**n losses of the n near-tie elements' choices (n <= max_ties).  The first has
    every tie rounded as ``quantize_groups`` rounds it and equals ``loss(...)``; within one column
    the choices count in binary over that column's ties (the first tie the lowest bit), and the
    columns' counts nest with the first tied column innermost.  Used only by the parity tests, to
    accept a search loss that took a tie the other way.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    s64 = np.asarray(s, dtype=np.float64)
    g = int(group_size)
    P = s64[:, None] * W
    codes, delta, zero = quantize_groups(P, g, zero_point, clip)
    d = np.repeat(delta.astype(np.float64), g, axis=0)
    z = np.repeat(zero.astype(np.float64), g, axis=0)
    level = codes.astype(np.float64) - z            # the quantizer's level of every element
    t, _ = pre_round_values(P, delta, g, zero_point, clip)
    tie = np.argwhere(near_tie(t, rel))
    n = len(tie)
    if n > max_ties:
        raise ValueError(f"{n} near-tie elements: more than max_ties={max_ties}")
    lo_hi = None
    if float(np.float32(clip)) < 1.0:
        lo_hi = (-z, 15.0 - z) if zero_point else (np.full_like(z, -7.0), np.full_like(z, 7.0))
    E0 = level * d / s64[:, None] - W
    Y0 = X @ E0
    total = np.array([float(np.sum(Y0 * Y0))])
    cols = []
    for k, c in tie:
        if c not in cols:
            cols.append(int(c))
    for c in cols:
        rows = [int(k) for k, cc in tie if cc == c]
        y0 = X @ E0[:, c]                       # the column's base, by the variants' own route
        base_c = float(np.dot(y0, y0))
        change = []
        for mask in range(2 ** len(rows)):
            e = E0[:, c].copy()
            for b, k in enumerate(rows):
                if (mask >> b) & 1:
                    lf = np.floor(t[k, c])
                    v = lf + 1.0 if level[k, c] == lf else lf
                    if lo_hi is not None:
                        v = min(max(v, lo_hi[0][k, c]), lo_hi[1][k, c])
                    e[k] = v * d[k, c] / s64[k] - W[k, c]
            y = X @ e
            change.append(float(np.dot(y, y)) - base_c)
        total = (np.asarray(change)[:, None] + total[None, :]).reshape(-1)
    return total


def dequantize(codes: np.ndarray, delta: np.ndarray, zero: np.ndarray, group_size: int) -> np.ndarray:
    """(code - zero) * Delta, broadcast per group along K -- float64 [K, N]."""
    g = int(group_size)
    d = np.repeat(np.asarray(delta, dtype=np.float64), g, axis=0)
    z = np.repeat(np.asarray(zero, dtype=np.float64), g, axis=0)
    return (np.asarray(codes, dtype=np.float64) - z) * d


def fake_quant(W: np.ndarray, s: np.ndarray, group_size: int, zero_point: bool,
               quantizer=None, clip: float = 1.0) -> np.ndarray:
    """What = S^-1 Q(S W): [P1] step 4a-4b and [P5] 4.3 (What = quant(W diag(s)) diag(s)^-1).

    ``W`` float64 [K, N] (input channel k is row k), ``s`` float32/64 [K].
    ``quantizer`` (default: the group INT4 quantizer followed by dequantization)
    maps the scaled weights to their dequantized values; tests substitute the
    identity to check that scaling alone is exact.
    """
    W = np.asarray(W, dtype=np.float64)
    s64 = np.asarray(s, dtype=np.float64)
    P = s64[:, None] * W
    if quantizer is None:
        codes, delta, zero = quantize_groups(P, group_size, zero_point, clip)
        Ph = dequantize(codes, delta, zero, group_size)
    else:
        Ph = quantizer(P)
    return Ph / s64[:, None]


# ----------------------------------------------------------------------------- a3/a4
def loss(X: np.ndarray, W: np.ndarray, s: np.ndarray, group_size: int, zero_point: bool,
         quantizer=None, clip: float = 1.0) -> float:
    """L = ||X (S^-1 Q(S W) - W)||^2: [P1] step 4c, with the error analysis of
    AWQ 的缩放如何改变量化误差 (Delta Y = X S^-1 eps_SW)."""
    E = fake_quant(W, s, group_size, zero_point, quantizer, clip) - np.asarray(W, dtype=np.float64)
    Y = np.asarray(X, dtype=np.float64) @ E
    return float(np.sum(Y * Y))


def losses(X: np.ndarray, W: np.ndarray, S: np.ndarray, group_size: int, zero_point: bool,
           quantizer=None, clip: float = 1.0) -> np.ndarray:
    """L(alpha_i) for every row s_i of the scale table S [n_grid, K]."""
    return np.array([loss(X, W, S[i], group_size, zero_point, quantizer, clip) for i in range(S.shape[0])])


def losses_multi(X: np.ndarray, Ws, S: np.ndarray, group_size: int, zero_point: bool,
                 clip: float = 1.0):
    """Joint search of several projections that read the same X and so must share one scale
    vector (the 1/s division happens once, on X, before every projection; [P4] 关键设计 4 and
    the fused ``attn.qkv`` layer of its usage).  The joint loss is the squared error over all
    their outputs, L(alpha_i) = sum_j ||X (S_i^-1 Q(S_i W_j) - W_j)||^2 ([P1] step 4c per
    projection).  Returns (joint [n_grid], each [n_w, n_grid])."""
    each = np.array([losses(X, W, S, group_size, zero_point, clip=clip) for W in Ws])
    return each.sum(axis=0), each


def clip_grid(clip_min: float, n: int) -> np.ndarray:
    """Clip ratios c_j = fl32(1 - (1 - c_min) * j / (n - 1)), j = 0..n-1, in float64 before
    the rounding; c_0 = 1 (no clipping) comes first, so ties keep the unclipped quantizer."""
    cm = float(np.float32(clip_min))
    return np.array([np.float32(1.0 - (1.0 - cm) * j / (n - 1)) for j in range(n)], dtype=np.float32)


def clip_losses(X: np.ndarray, W: np.ndarray, s: np.ndarray, ratios: np.ndarray, group_size: int,
                zero_point: bool) -> np.ndarray:
    """L(c_j) = ||X (S^-1 Q_c_j(S W) - W)||^2 at fixed scales s, for every clip ratio: the
    loss of [P1] step 4c with the clipped quantizer of [P4] 关键设计 5."""
    return np.array([loss(X, W, s, group_size, zero_point, clip=float(c)) for c in ratios])


def select(L: np.ndarray) -> int:
    """alpha* = argmin L, first minimum on ties: [P1] step 5, [P5] 4.3 (strict "<")."""
    best = 0
    for i in range(1, len(L)):
        if L[i] < L[best]:
            best = i
    return best


def search(X: np.ndarray, W: np.ndarray, mean_abs: np.ndarray, group_size: int,
           zero_point: bool, n_grid: int = 21):
    """The whole per-layer search ([P1] steps 3-6).  Returns a dict with the scale
    table, every loss, the chosen index and s* = s[best]."""
    S = scale_table(mean_abs, n_grid)
    L = losses(X, W, S, group_size, zero_point)
    b = select(L)
    return {"S": S, "losses": L, "best": b, "s_best": S[b].copy()}


def pow2_candidates(n: int = 20) -> np.ndarray:
    """The candidate scales of the greedy search, 2**(j - n//2) for j = 0..n-1: powers of two
    around 1 ([P4] 关键设计 1; the default count there is 20)."""
    return np.array([2.0 ** (j - n // 2) for j in range(n)])


def group_error(W_g: np.ndarray, m_g: np.ndarray, s_g: np.ndarray, zero_point: bool,
                clip: float = 1.0) -> float:
    """Activation-weighted reconstruction error of one quantization group ([P4] 关键设计 1):
    W_g [g, N] are the group's rows of W, m_g [g] the mean |x| of its channels and s_g [g]
    their scales; the group is quantized as packing quantizes it ([P4] 关键设计 3) and
    sum_n sum_i (m_i (What_in - W_in))^2 is returned."""
    W_g = np.asarray(W_g, dtype=np.float64)
    s_g = np.asarray(s_g, dtype=np.float64)
    g = W_g.shape[0]
    codes, delta, zero = quantize_groups(s_g[:, None] * W_g, g, zero_point, clip)
    What = dequantize(codes, delta, zero, g) / s_g[:, None]
    E = np.asarray(m_g, dtype=np.float64)[:, None] * (What - W_g)
    return float(np.sum(E * E))


def greedy_search(W: np.ndarray, mean_abs: np.ndarray, group_size: int, zero_point: bool,
                  n_cand: int = 20, passes: int = 3, trace: list | None = None):
    """Per-group coordinate greedy over power-of-two scales ([P4] 关键设计 1-2; its cost
    O(passes * K * n * N * g), Consequences).  Groups of input channels are independent because
    each group's quantization sees only its own channels' scales.  Every channel starts at
    s = 1; a pass visits the group's channels in ascending order and, for channel k, scores
    every candidate with the group error (the other channels at their current scales), then
    moves s_k to the best candidate only if its error is strictly below the current one (first
    such candidate in ascending order on ties).  Three passes let a channel whose enlarged
    weight became the group maximum be revisited.

    Returns a dict: ``idx`` int [K] (s_k = pow2_candidates(n)[idx_k]), ``s`` float32 [K],
    ``err_rtn`` and ``err`` float64 [K/g] (group errors at s = 1 and at the result).  With
    ``trace`` a list, (group, pass, k, errors of every candidate, chosen index) is appended
    per decision."""
    W = np.asarray(W, dtype=np.float64)
    m = np.asarray(mean_abs, dtype=np.float64)
    K, N = W.shape
    g = int(group_size)
    cand = pow2_candidates(n_cand)
    one = n_cand // 2
    idx = np.full(K, one, dtype=np.int64)
    err_rtn = np.zeros(K // g)
    err = np.zeros(K // g)
    for j in range(K // g):
        rows = slice(j * g, (j + 1) * g)
        Wg, mg = W[rows], m[rows]
        err_rtn[j] = group_error(Wg, mg, np.ones(g), zero_point)
        for p in range(passes):
            for i in range(g):
                k = j * g + i
                e = np.zeros(n_cand)
                for c in range(n_cand):
                    sg = cand[idx[rows]]
                    sg[i] = cand[c]
                    e[c] = group_error(Wg, mg, sg, zero_point)
                best = idx[k]
                for c in range(n_cand):
                    if e[c] < e[best]:
                        best = c
                idx[k] = best
                if trace is not None:
                    trace.append((j, p, k, e, best))
        err[j] = group_error(Wg, mg, cand[idx[rows]], zero_point)
    return {"idx": idx, "s": cand[idx].astype(np.float32), "err_rtn": err_rtn, "err": err}


def relative_error(L: float, X: np.ndarray, W: np.ndarray) -> float:
    """epsilon = ||X (W - What)||^2 / ||X W||^2: [P3] section 5."""
    Y = np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64)
    return float(L / np.sum(Y * Y))


# ----------------------------------------------------------------------------- a5
def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte ([P4] Consequences): word (i, n) of the uint32
    [K/8, N] result holds codes[8i + j, n] in bits 4j..4j+3."""
    codes = np.asarray(codes)
    K, N = codes.shape
    c = codes.reshape(K // 8, 8, N).astype(np.uint32)
    out = np.zeros((K // 8, N), dtype=np.uint32)
    for j in range(8):
        out |= (c[:, j, :] & np.uint32(0xF)) << np.uint32(4 * j)
    return out


def unpack_nibbles(words: np.ndarray) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint32)
    Kw, N = words.shape
    out = np.empty((Kw, 8, N), dtype=np.int64)
    for j in range(8):
        out[:, j, :] = (words >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(Kw * 8, N)


def pack(W: np.ndarray, s: np.ndarray, group_size: int, zero_point: bool, clip: float = 1.0):
    """Offline quantization W_q = Quantize(diag(s*) W) ([P1] 推理时的等效实现),
    stored as (codes uint32 [K/8, N], scales float32 [K/g, N], zeros uint8 [K/g, N])."""
    P = np.asarray(s, dtype=np.float64)[:, None] * np.asarray(W, dtype=np.float64)
    codes, delta, zero = quantize_groups(P, group_size, zero_point, clip)
    return pack_nibbles(codes), delta.astype(np.float32), zero.astype(np.uint8)


# ----------------------------------------------------------------------------- a6
def w4a16_ref(X: np.ndarray, s: np.ndarray, words: np.ndarray, scales: np.ndarray,
              zeros: np.ndarray, group_size: int) -> np.ndarray:
    """Y = (X diag(1/s*)) Dequant(W_q) ([P1] 推理时的等效实现, online step) in float64."""
    Wd = dequantize(unpack_nibbles(words), scales, zeros, group_size)
    Xs = np.asarray(X, dtype=np.float64) / np.asarray(s, dtype=np.float64)[None, :]
    return Xs @ Wd


# ----------------------------------------------------------------------------- sizes
def packed_bytes(n_params: float, bits: int) -> float:
    """M = N*b/8 bytes ([P3] section 6)."""
    return n_params * bits / 8.0


def compression_ratio(bits: int) -> float:
    """R = 16/b relative to 16-bit weights ([P3] section 6)."""
    return 16.0 / bits


def storage_bytes(K: int, N: int, group_size: int) -> dict:
    """Bytes of the stored layer: nibble codes plus float32 scales and uint8 zeros."""
    return {"codes": K * N // 2, "scales": 4 * (K // group_size) * N, "zeros": (K // group_size) * N}
