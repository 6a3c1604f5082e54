"""Blockwise online-softmax replay, fp64, for pinning the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/attention.py).

This follows the procedure described on 'FlashAttention' (josueisai.com),
section on the softmax trick and its numpy sketch of one query row: keep a
running row maximum m and a running sum l of exponentials; for every K/V block
compute that block's scores, raise m if the block holds a larger score, rescale
the partial output and the partial sum by exp(m_old - m_new), add the block's
exponentials and their product with V; after the last block divide by l.
The sketch has no attention scale; here the block scores are multiplied by
``scale`` before the softmax, as in the oracle. The log-sum-exp m + ln l is
returned too, since the method saves those two row statistics.

It is written for many query rows at once and takes an arbitrary partition of
the keys into blocks, so tests can check that every partition reproduces the
full-row softmax of attention.forward_head.
"""
from __future__ import annotations

import numpy as np


def partition_keys(n_keys: int, block: int):
    """Contiguous blocks of ``block`` keys (the last one may be shorter)."""
    return [(s, min(n_keys, s + block)) for s in range(0, n_keys, block)]


def online_softmax_attention(q, k, v, scale: float, blocks, causal=False,
                             row_idx=None):
    """Replay the running-max / running-sum recurrence over key ``blocks``.

    q [R, d], k [Nk, d], v [Nk, dv]; ``blocks`` is a list of (start, stop)
    key ranges covering 0..Nk exactly once, visited in the given order.
    Returns O [R, dv], LSE [R].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = q.shape[0]
    if row_idx is None:
        row_idx = np.arange(rows)
    running_max = np.full(rows, -np.inf)
    running_sum = np.zeros(rows)
    acc = np.zeros((rows, v.shape[1]))
    for start, stop in blocks:
        s = float(scale) * (q @ k[start:stop].T)
        if causal:
            s = np.where(np.arange(start, stop)[None, :] > np.asarray(row_idx)[:, None],
                         -np.inf, s)
        new_max = np.maximum(running_max, s.max(axis=1, initial=-np.inf))
        # rows that have seen no unmasked key yet keep a zero state
        alive = np.isfinite(new_max)
        ref = np.where(alive, new_max, 0.0)
        e = np.exp(s - ref[:, None])
        with np.errstate(invalid="ignore"):
            shrink = np.where(alive, np.exp(running_max - ref), 1.0)
        running_sum = running_sum * shrink + e.sum(axis=1)
        acc = acc * shrink[:, None] + e @ v[start:stop]
        running_max = new_max
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(running_sum[:, None] > 0, acc / running_sum[:, None], 0.0)
        lse = np.where(running_sum > 0, running_max + np.log(running_sum), -np.inf)
    return out, lse
