"""Plain fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. The product path never imports this package; only
the tests, the smoke check and the benchmark's CPU-baseline leg do. It shares
no code with the HIP kernels or their C-ABI library.

What it computes, one head at a time, in float64, with nothing fused, blocked
or reordered beyond what the definition states:

  S = scale * Q K^T                 'FlashAttention' (josueisai.com), section on
                                    the matrix that should never be stored: the
                                    three-step definition S = QK^T, row softmax,
                                    O = PV. The scale factor is an argument
                                    (the pages omit it; every workload passes
                                    1/sqrt(d) rounded to float32).
  causal: S_ij = -inf for j > i     key j after query i is masked (top-left).
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

A fully masked row (never produced by the top-left causal mask with equal
query and key lengths) is defined as O = 0, LSE = -inf, zero gradients.

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


def _scores(q_rows: np.ndarray, row_idx: np.ndarray, k: np.ndarray,
            scale: float, causal: bool) -> np.ndarray:
    s = float(scale) * (q_rows @ k.T)
    if causal:
        masked = np.arange(k.shape[0])[None, :] > row_idx[:, None]
        s = np.where(masked, -np.inf, s)
    return s


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


def forward_head(q, k, v, scale: float, causal: bool = False, rows=None):
    """One head. q [Nq, d], k [Nk, d], v [Nk, dv] -> O [R, dv], LSE [R].

    ``rows`` selects query rows (default: all); the causal mask uses the
    absolute query index.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if rows is None:
        rows = np.arange(q.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.zeros(rows.size, dtype=np.float64)
    for c0 in range(0, rows.size, _ROW_CHUNK):
        idx = rows[c0:c0 + _ROW_CHUNK]
        s = _scores(q[idx], idx, k, scale, causal)
        p, m, l, dead = _softmax_rows(s)
        o[c0:c0 + idx.size] = p @ v
        with np.errstate(divide="ignore"):
            lse[c0:c0 + idx.size] = np.where(dead, -np.inf, m + np.log(l))
    return o, lse


def backward_head(q, k, v, do, scale: float, causal: bool = False):
    """One head: gradients of sum(O * dO) w.r.t. Q, K, V (LSE not differentiated)."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    nq = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for c0 in range(0, nq, _ROW_CHUNK):
        idx = np.arange(c0, min(nq, c0 + _ROW_CHUNK))
        s = _scores(q[idx], idx, k, scale, causal)
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


def forward(q, k, v, scale: float, causal: bool = False, workers=None):
    """[..., N, d] batched forward; heads are independent and run in threads."""
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    n = _pool(workers)
    lim = _limit_blas(n)
    try:
        with ThreadPoolExecutor(n) as ex:
            res = list(ex.map(lambda i: forward_head(qh[i], kh[i], vh[i], scale, causal),
                              range(qh.shape[0])))
    finally:
        if lim is not None:
            lim.unregister() if hasattr(lim, "unregister") else lim.__exit__(None, None, None)
    o = np.stack([r[0] for r in res]).reshape(*lead, qh.shape[1], vh.shape[2])
    lse = np.stack([r[1] for r in res]).reshape(*lead, qh.shape[1])
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool = False, workers=None):
    """[..., N, d] batched backward; returns dQ, dK, dV."""
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    gh, _ = _heads(do)
    n = _pool(workers)
    lim = _limit_blas(n)
    try:
        with ThreadPoolExecutor(n) as ex:
            res = list(ex.map(lambda i: backward_head(qh[i], kh[i], vh[i], gh[i], scale, causal),
                              range(qh.shape[0])))
    finally:
        if lim is not None:
            lim.unregister() if hasattr(lim, "unregister") else lim.__exit__(None, None, None)
    shp = lambda a, ref: np.stack(a).reshape(*lead, ref.shape[1], ref.shape[2])
    return (shp([r[0] for r in res], qh), shp([r[1] for r in res], kh),
            shp([r[2] for r in res], vh))
