"""Blockwise replay of the online softmax, fp64, for pinning the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/attention.py).

The method's central claim ('FlashAttention' on josueisai.com, section on the
softmax trick; the log-sum-exp rescaling named on the kerneldigest.dev
glossary entry) is that attention over all keys can be assembled from
attention over blocks of keys, carrying only a couple of numbers per query
row, so the blocks can be visited one at a time and exactly the full-row
softmax comes out. This module restates that claim from its algebra.

For one query row and a set J of keys, with scaled scores s_j, let
    LSE_J = ln sum_{j in J} exp(s_j)
    O_J   = sum_{j in J} exp(s_j - LSE_J) v_j
(the log-sum-exp over J, and the softmax-weighted mean of V over J). For two
disjoint key sets A and B,
    LSE_{A+B} = ln(exp(LSE_A) + exp(LSE_B))
    O_{A+B}   = exp(LSE_A - LSE_{A+B}) O_A + exp(LSE_B - LSE_{A+B}) O_B.
This merge is associative and commutative, and the empty set (LSE = -inf,
O = 0) is its identity. Each block's pair is computed on its own, from that
block's scores alone; the pairs are then merged either left to right in the
given block order (the method's one-block-at-a-time order: the running pair is
all the state it carries, and each merge rescales the running output) or as a
balanced tree. Every partition and every order must reproduce the full-row
softmax of attention.forward_head: O = O_{all keys}, LSE = LSE_{all keys}.
"""
from __future__ import annotations

import numpy as np


def partition_keys(n_keys: int, block: int):
    """Contiguous blocks of ``block`` keys (the last one may be shorter)."""
    return [(s, min(n_keys, s + block)) for s in range(0, n_keys, block)]


def block_pair(q, k_blk, v_blk, scale: float, visible):
    """(O_J, LSE_J) of every query row over one key block J.

    ``visible`` [R, |J|] marks the (row, key) pairs the mask keeps. A row that
    sees no key of the block gets the empty pair (O = 0, LSE = -inf)."""
    s = np.where(visible, float(scale) * (q @ k_blk.T), -np.inf)
    top = s.max(axis=1, initial=-np.inf)          # shift for a stable exponent
    seen = np.isfinite(top)
    shift = np.where(seen, top, 0.0)
    w = np.exp(s - shift[:, None])                # exp(-inf) = 0 on hidden pairs
    total = np.where(seen, w.sum(axis=1), 1.0)
    lse = np.where(seen, shift + np.log(total), -np.inf)
    o = np.where(seen[:, None], (w @ v_blk) / total[:, None], 0.0)
    return o, lse


def merge(a, b):
    """The pair of the union of two disjoint key sets, from their pairs."""
    (oa, la), (ob, lb) = a, b
    with np.errstate(invalid="ignore"):
        lse = np.logaddexp(la, lb)                # -inf only when both are empty
    live = np.isfinite(lse)
    ref = np.where(live, lse, 0.0)
    wa = np.where(live, np.exp(la - ref), 0.0)
    wb = np.where(live, np.exp(lb - ref), 0.0)
    return wa[:, None] * oa + wb[:, None] * ob, lse


def online_softmax_attention(q, k, v, scale: float, blocks, causal=False, row_idx=None, order="sequential"):
    """Attention assembled from per-block pairs over key ``blocks``.

    q [R, d], k [Nk, d], v [Nk, dv]; ``blocks`` is a list of (start, stop)
    key ranges covering 0..Nk exactly once. ``order`` = "sequential" merges
    them left to right in the given order, "tree" pairwise in rounds.
    ``causal`` hides key j from row i when j > row_idx[i] (default: i).
    Returns O [R, dv], LSE [R].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.arange(q.shape[0]) if row_idx is None else np.asarray(row_idx)
    pairs = []
    for start, stop in blocks:
        keys = np.arange(start, stop)
        visible = np.ones((q.shape[0], keys.size), dtype=bool)
        if causal:
            visible = keys[None, :] <= rows[:, None]
        pairs.append(block_pair(q, k[start:stop], v[start:stop], scale, visible))
    empty = (np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf))
    if order == "sequential":
        state = empty
        for p in pairs:
            state = merge(state, p)
        return state
    if order == "tree":
        level = pairs or [empty]
        while len(level) > 1:
            nxt = [merge(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
            if len(level) % 2:
                nxt.append(level[-1])
            level = nxt
        return level[0]
    raise ValueError(f"unknown order {order!r}")
