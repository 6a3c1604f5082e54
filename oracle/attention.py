"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. The product path never imports this package; only
the tests, the smoke check and the benchmark's CPU-baseline leg do. It shares
no code with the HIP kernels or their C-ABI library.

What it computes, one head at a time, in float64, with nothing fused, blocked
or reordered beyond what the definition states:

  S = scale * Q K^T [+ bias]        'FlashAttention' (josueisai.com), section on
                                    the matrix that should never be stored: the
                                    three-step definition S = QK^T, row softmax,
                                    O = PV. The scale factor is an argument
                                    (the pages omit it; every workload passes
                                    1/sqrt(d) rounded to float32). An
                                    optional additive bias [Nq, Nk] (any
                                    broadcastable shape; -inf removes a key)
                                    is added to the scaled scores: the masks
                                    and biases that the page's section on what
                                    you gain and what not warns may push
                                    libraries off their fast path.
  masks: S_ij = -inf outside a band key j is visible to query i when
                                    diag_i - left <= j <= diag_i + right,
                                    diag_i = i + Nk - Nq (query rows aligned
                                    with the last Nq keys, as when new queries
                                    attend over a cache of earlier keys). A
                                    bound of None is absent. causal is
                                    right = 0 (for Nq = Nk: key j > query i is
                                    masked); a window of `left` earlier keys is
                                    the local attention that the josueisai.com
                                    page, section on what you gain and what
                                    not, names as the way to cut the compute
                                    of very long sequences.
  P = rowsoftmax(S)                 same page, section on the softmax trick:
                                    subtract the row maximum, divide by the sum
                                    of exponentials.
  O = P V
  LSE_i = m_i + ln l_i              natural-log log-sum-exp of the scaled scores
                                    (the 'log-sum-exp' rescaling named on the
                                    kerneldigest.dev glossary entry; the pages
                                    keep the row max and row sum, section on
                                    recomputing instead of remembering).

Backward (the pages only say the gradient needs P; these are the chain rule
applied to the definition above, so the oracle is the exact gradient of its own
forward):  dV = P^T dO;  dP = dO V^T;  D_i = sum_j P_ij dP_ij;
           dS = P * (dP - D 1^T);  dQ = scale dS K;  dK = scale dS^T Q.

A fully masked row (with Nq > Nk under the causal mask, or a band that
leaves a row no key) is defined as O = 0, LSE = -inf, zero gradients: the
empty sum of exponentials is 0 and the row takes no part in any product.

Rows may be processed in chunks to bound memory, but every query row always
sees its whole key row at once: there is no online rescaling anywhere here.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_ROW_CHUNK = 1024


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _band(causal: bool, window):
    """(left, right) bounds of the visible band; None is unbounded."""
    left, right = (None, None) if window is None else window
    if causal:
        if right is not None and right != 0:
            raise ValueError("causal sets right = 0; window gives another right bound")
        right = 0
    for w in (left, right):
        if w is not None and w < 0:
            raise ValueError("window bounds are >= 0 or None")
    return left, right


def _scores(q_rows: np.ndarray, row_idx: np.ndarray, k: np.ndarray,
            scale: float, nq: int, left, right, bias_rows=None) -> np.ndarray:
    s = float(scale) * (q_rows @ k.T)
    if bias_rows is not None:
        s = s + bias_rows
    if left is None and right is None:
        return s
    diag = row_idx + (k.shape[0] - nq)      # key aligned with each query row
    j = np.arange(k.shape[0])[None, :]
    masked = np.zeros(s.shape, dtype=bool)
    if right is not None:
        masked |= j > diag[:, None] + right
    if left is not None:
        masked |= j < diag[:, None] - left
    return np.where(masked, -np.inf, s)


def _softmax_rows(s: np.ndarray):
    """Full-row softmax with the row max subtracted. Returns P, m, l."""
    m = s.max(axis=1)
    dead = ~np.isfinite(m)                     # fully masked rows
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(s - m_safe[:, None])            # exp(-inf) = 0 on masked entries
    l = e.sum(axis=1)
    p = e / np.where(dead, 1.0, l)[:, None]
    p[dead] = 0.0
    return p, m, l, dead


def _bias_2d(bias, nq, nk):
    return None if bias is None else np.broadcast_to(_as_f64(bias), (nq, nk))


def forward_head(q, k, v, scale: float, causal: bool = False, rows=None, window=None, bias=None):
    """One head. q [Nq, d], k [Nk, d], v [Nk, dv] -> O [R, dv], LSE [R].

    ``rows`` selects query rows (default: all); masks use the absolute query
    index. ``window`` = (left, right) bounds the visible keys around each
    row's aligned key (None = unbounded); ``causal`` sets right = 0.
    ``bias`` (broadcastable to [Nq, Nk]) is added to the scaled scores.
    """
    left, right = _band(causal, window)
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    bias = _bias_2d(bias, q.shape[0], k.shape[0])
    if rows is None:
        rows = np.arange(q.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.zeros(rows.size, dtype=np.float64)
    for c0 in range(0, rows.size, _ROW_CHUNK):
        idx = rows[c0:c0 + _ROW_CHUNK]
        s = _scores(q[idx], idx, k, scale, q.shape[0], left, right, None if bias is None else bias[idx])
        p, m, l, dead = _softmax_rows(s)
        o[c0:c0 + idx.size] = p @ v
        with np.errstate(divide="ignore"):
            lse[c0:c0 + idx.size] = np.where(dead, -np.inf, m + np.log(l))
    return o, lse


def backward_head(q, k, v, do, scale: float, causal: bool = False, window=None, bias=None):
    """One head: gradients of sum(O * dO) w.r.t. Q, K, V (LSE and the bias are
    not differentiated)."""
    left, right = _band(causal, window)
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    bias = _bias_2d(bias, q.shape[0], k.shape[0])
    nq = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for c0 in range(0, nq, _ROW_CHUNK):
        idx = np.arange(c0, min(nq, c0 + _ROW_CHUNK))
        s = _scores(q[idx], idx, k, scale, nq, left, right, None if bias is None else bias[idx])
        p, _, _, _ = _softmax_rows(s)
        g = do[idx]
        dv += p.T @ g
        dp = g @ v.T
        d_row = (p * dp).sum(axis=1)
        ds = p * (dp - d_row[:, None])
        dq[idx] = float(scale) * (ds @ k)
        dk += float(scale) * (ds.T @ q[idx])
    return dq, dk, dv


def _heads(x):
    x = _as_f64(x)
    return x.reshape(-1, x.shape[-2], x.shape[-1]), x.shape[:-2]


def _pool(workers):
    if workers is None:
        workers = len(os.sched_getaffinity(0))
    return max(1, int(workers))


def _limit_blas(n_workers):
    """One BLAS thread per worker when heads run in parallel."""
    if n_workers <= 1:
        return None
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1, user_api="blas")
    except Exception:  # pragma: no cover - threadpoolctl is optional
        return None


def _bias_heads(bias, lead, nq, nk):
    """Per-head [Nq, Nk] bias views (None when there is no bias)."""
    if bias is None:
        return None
    b = np.broadcast_to(_as_f64(bias), tuple(lead) + (nq, nk))
    return b.reshape(-1, nq, nk)


def forward(q, k, v, scale: float, causal: bool = False, workers=None, window=None, bias=None):
    """[..., N, d] batched forward; heads are independent and run in threads.
    ``bias`` broadcasts to [..., Nq, Nk]."""
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    bh = _bias_heads(bias, lead, qh.shape[1], kh.shape[1])
    n = _pool(workers)
    lim = _limit_blas(n)
    try:
        with ThreadPoolExecutor(n) as ex:
            res = list(ex.map(lambda i: forward_head(qh[i], kh[i], vh[i], scale, causal, window=window,
                                                           bias=None if bh is None else bh[i]),
                              range(qh.shape[0])))
    finally:
        if lim is not None:
            lim.unregister() if hasattr(lim, "unregister") else lim.__exit__(None, None, None)
    o = np.stack([r[0] for r in res]).reshape(*lead, qh.shape[1], vh.shape[2])
    lse = np.stack([r[1] for r in res]).reshape(*lead, qh.shape[1])
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool = False, workers=None, window=None, bias=None):
    """[..., N, d] batched backward; returns dQ, dK, dV."""
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    bh = _bias_heads(bias, lead, qh.shape[1], kh.shape[1])
    gh, _ = _heads(do)
    n = _pool(workers)
    lim = _limit_blas(n)
    try:
        with ThreadPoolExecutor(n) as ex:
            res = list(ex.map(lambda i: backward_head(qh[i], kh[i], vh[i], gh[i], scale, causal, window=window,
                                                            bias=None if bh is None else bh[i]),
                              range(qh.shape[0])))
    finally:
        if lim is not None:
            lim.unregister() if hasattr(lim, "unregister") else lim.__exit__(None, None, None)
    shp = lambda a, ref: np.stack(a).reshape(*lead, ref.shape[1], ref.shape[2])
    return (shp([r[0] for r in res], qh), shp([r[1] for r in res], kh),
            shp([r[2] for r in res], vh))
