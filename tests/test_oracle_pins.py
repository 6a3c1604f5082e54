"""Pins for the fp64 CPU oracle: nothing here compares the oracle with itself.

Each test ties the oracle to something outside it: hand-derived closed forms,
invariants the mathematics fixes, the blockwise replay of the pages' online
softmax procedure, PyTorch's float64 CPU attention and autograd, and central
finite differences.
"""
import ast
import json
import math
import operator
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oa
from oracle import replay as orp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")

# ---------------------------------------------------------------- helpers ---

_BIN = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv}


def _eval(expr: str) -> float:
    """Evaluate a closed form made of numbers, inf, + - * /, unary -, log()."""
    def ev(n):
        if isinstance(n, ast.Expression):
            return ev(n.body)
        if isinstance(n, ast.Constant) and isinstance(n.value, (int, float)):
            return float(n.value)
        if isinstance(n, ast.BinOp) and type(n.op) in _BIN:
            return _BIN[type(n.op)](ev(n.left), ev(n.right))
        if isinstance(n, ast.UnaryOp) and isinstance(n.op, ast.USub):
            return -ev(n.operand)
        if (isinstance(n, ast.Call) and isinstance(n.func, ast.Name)
                and n.func.id == "log" and len(n.args) == 1):
            return math.log(ev(n.args[0]))
        if isinstance(n, ast.Name) and n.id == "inf":
            return math.inf
        raise ValueError(f"unsupported expression: {expr!r}")
    return ev(ast.parse(expr, mode="eval"))


def _arr(x):
    return np.vectorize(_eval, otypes=[np.float64])(np.array(x, dtype=object))


def _load_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _bias(case):
    return None if "bias" not in case else _arr(case["bias"])


def _window(case):
    w = case.get("window")
    return None if w is None else tuple(w)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------ hand-worked cases ---

@pytest.mark.parametrize("case", _load_cases(), ids=lambda c: c["name"])
def test_hand_worked_forward(case):
    q, k, v = _arr(case["q"]), _arr(case["k"]), _arr(case["v"])
    o, lse = oracle.forward_head(q, k, v, _eval(case["scale"]), case["causal"], window=_window(case),
                                 bias=_bias(case))
    np.testing.assert_allclose(o, _arr(case["o"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, _arr(case["lse"]), rtol=0, atol=1e-13)


@pytest.mark.parametrize("case", _load_cases(), ids=lambda c: c["name"])
def test_hand_worked_backward(case):
    q, k, v, do = (_arr(case[n]) for n in ("q", "k", "v", "do"))
    dq, dk, dv = oracle.backward_head(q, k, v, do, _eval(case["scale"]), case["causal"],
                                      window=_window(case), bias=_bias(case))
    np.testing.assert_allclose(dq, _arr(case["dq"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, _arr(case["dk"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, _arr(case["dv"]), rtol=0, atol=1e-13)


# ------------------------------------------------------------- invariants ---

@pytest.mark.parametrize("causal", [False, True])
def test_probabilities_implied_by_lse_sum_to_one(causal):
    n, d, scale = 37, 8, 0.3
    q, k = _rand((n, d), 1), _rand((n, d), 2)
    _, lse = oracle.forward_head(q, k, _rand((n, 3), 3), scale, causal)
    s = scale * q @ k.T
    if causal:
        s = np.where(np.triu(np.ones((n, n), bool), 1), -np.inf, s)
    np.testing.assert_allclose(np.exp(s - lse[:, None]).sum(axis=1), 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_that_constant(causal):
    n, d = 50, 16
    c = _rand((1, 5), 4)
    o, _ = oracle.forward_head(_rand((n, d), 5), _rand((n, d), 6), np.repeat(c, n, 0), 0.25, causal)
    np.testing.assert_allclose(o, np.repeat(c, n, 0), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(causal):
    n, d, scale = 40, 8, 0.7
    q = _rand((n, d), 7)
    krow = _rand((1, d), 8)
    v = _rand((n, 6), 9)
    o, lse = oracle.forward_head(q, np.repeat(krow, n, 0), v, scale, causal)
    cnt = np.arange(1, n + 1) if causal else np.full(n, n)
    mean = np.cumsum(v, 0) / cnt[:, None] if causal else np.repeat(v.mean(0, keepdims=True), n, 0)
    np.testing.assert_allclose(o, mean, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, scale * (q @ krow[0]) + np.log(cnt), rtol=0, atol=1e-12)


def test_single_key_returns_v_and_score():
    q, k, v = _rand((1, 5), 10), _rand((1, 5), 11), _rand((1, 4), 12)
    o, lse = oracle.forward_head(q, k, v, 0.9)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.9 * q @ k[0], rtol=0, atol=1e-15)


def test_causal_first_row_is_first_value_row():
    n, d = 20, 4
    q, k, v = _rand((n, d), 13), _rand((n, d), 14), _rand((n, d), 15)
    o, lse = oracle.forward_head(q, k, v, 0.5, causal=True)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], 0.5 * q[0] @ k[0], rtol=0, atol=1e-15)


def test_joint_key_value_permutation_invariance():
    n, d = 33, 8
    q, k, v = _rand((n, d), 16), _rand((n, d), 17), _rand((n, 5), 18)
    perm = np.random.default_rng(19).permutation(n)
    o1, l1 = oracle.forward_head(q, k, v, 0.4)
    o2, l2 = oracle.forward_head(q, k[perm], v[perm], 0.4)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_moves_lse_only(causal):
    n, d, scale = 30, 6, 0.45
    q, k, v = _rand((n, d), 20), _rand((n, d), 21), _rand((n, 4), 22)
    u = _rand((d,), 23)
    o1, l1 = oracle.forward_head(q, k, v, scale, causal)
    o2, l2 = oracle.forward_head(q, k + u, v, scale, causal)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, scale * q @ u, rtol=0, atol=1e-12)


def test_causal_row_equals_attention_over_prefix():
    n, d = 25, 8
    q, k, v = _rand((n, d), 24), _rand((n, d), 25), _rand((n, 3), 26)
    o, lse = oracle.forward_head(q, k, v, 0.6, causal=True)
    for i in (0, 1, 7, 24):
        oi, li = oracle.forward_head(q[i:i + 1], k[:i + 1], v[:i + 1], 0.6)
        np.testing.assert_allclose(o[i], oi[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[i], li[0], rtol=0, atol=1e-13)


def test_row_subset_matches_full():
    n, d = 40, 8
    q, k, v = _rand((n, d), 27), _rand((n, d), 28), _rand((n, 8), 29)
    rows = np.array([0, 5, 39, 17])
    for causal in (False, True):
        o, lse = oracle.forward_head(q, k, v, 0.3, causal)
        os_, ls_ = oracle.forward_head(q, k, v, 0.3, causal, rows=rows)
        np.testing.assert_array_equal(os_, o[rows])
        np.testing.assert_array_equal(ls_, lse[rows])


def test_large_scores_do_not_overflow():
    # scores near 1e3 would overflow exp() without the row max subtracted
    q = np.array([[1000.0], [-1000.0], [1000.0]])
    k = np.array([[1.0], [0.999], [-1.0]])
    v = np.array([[1.0], [2.0], [3.0]])
    o, lse = oracle.forward_head(q, k, v, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    # row 0: s = [1000, 999, -1000]; the last key carries weight exp(-2000) = 0
    p1 = 1.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(o[0, 0], p1 * 1 + (1 - p1) * 2, rtol=1e-14)
    np.testing.assert_allclose(lse[0], 1000 + math.log(1 + math.exp(-1.0)), rtol=1e-14)
    # row 1: s = [-1000, -999, 1000]: the last key takes all the weight
    np.testing.assert_allclose(o[1, 0], 3.0, rtol=1e-14)
    np.testing.assert_allclose(lse[1], 1000.0, rtol=1e-14)


def test_fully_masked_row_reading():
    # Five queries over three keys under the causal mask: queries 0 and 1 are
    # aligned before the first key and see nothing; a band that excludes a
    # row's keys does the same.
    q, k, v = _rand((5, 4), 30), _rand((3, 4), 31), _rand((3, 2), 32)
    o, lse = oracle.forward_head(q, k, v, 1.0, causal=True)
    assert np.all(o[:2] == 0) and np.all(lse[:2] == -np.inf)
    assert np.all(np.isfinite(lse[2:]))
    do = _rand((5, 2), 33)
    dq, _, _ = oracle.backward_head(q, k, v, do, 1.0, causal=True)
    assert np.all(dq[:2] == 0)


# ------------------------------------- unequal lengths and banded masks ---

def test_decode_rows_are_the_last_rows_of_square_causal():
    # Nq queries over Nk keys with the causal mask are the last Nq rows of
    # square causal attention whose last Nq queries are these (new tokens
    # attending over a cache of earlier keys).
    nk, nq, d = 40, 7, 8
    q_full = _rand((nk, d), 60)
    k, v = _rand((nk, d), 61), _rand((nk, 5), 62)
    do = _rand((nq, 5), 63)
    o_sq, lse_sq = oracle.forward_head(q_full, k, v, 0.3, causal=True)
    o, lse = oracle.forward_head(q_full[-nq:], k, v, 0.3, causal=True)
    np.testing.assert_allclose(o, o_sq[-nq:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_sq[-nq:], rtol=0, atol=1e-13)
    # gradients: the square problem with dO zero on the first rows
    do_full = np.zeros((nk, 5))
    do_full[-nq:] = do
    dq_sq, dk_sq, dv_sq = oracle.backward_head(q_full, k, v, do_full, 0.3, causal=True)
    dq, dk, dv = oracle.backward_head(q_full[-nq:], k, v, do, 0.3, causal=True)
    np.testing.assert_allclose(dq, dq_sq[-nq:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, dk_sq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, dv_sq, rtol=0, atol=1e-12)


def test_more_queries_than_keys_pads_dead_rows_in_front():
    nq, nk, d = 11, 6, 4
    q, k, v = _rand((nq, d), 64), _rand((nk, d), 65), _rand((nk, 3), 66)
    o, lse = oracle.forward_head(q, k, v, 0.7, causal=True)
    o_sq, lse_sq = oracle.forward_head(q[nq - nk:], k, v, 0.7, causal=True)
    assert np.all(o[:nq - nk] == 0) and np.all(lse[:nq - nk] == -np.inf)
    np.testing.assert_allclose(o[nq - nk:], o_sq, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[nq - nk:], lse_sq, rtol=0, atol=1e-13)


@pytest.mark.parametrize("nq,nk", [(5, 9), (9, 5), (8, 8)])
def test_unmasked_unequal_lengths_match_torch_sdpa(nq, nk):
    torch = pytest.importorskip("torch")
    q, k, v = _rand((nq, 6), 67), _rand((nk, 6), 68), _rand((nk, 3), 69)
    o, lse = oracle.forward_head(q, k, v, 0.4)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    o_ref = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], scale=0.4)[0]
    np.testing.assert_allclose(o, o_ref.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(0.4 * tq @ tk.T, dim=1).numpy(), rtol=0, atol=1e-13)


def test_window_of_zero_returns_the_aligned_value_row():
    # left = right = 0: each query sees exactly its aligned key, so O_i is
    # that key's value row and LSE_i its scaled score
    nq, nk, d = 6, 10, 5
    q, k, v = _rand((nq, d), 70), _rand((nk, d), 71), _rand((nk, 4), 72)
    o, lse = oracle.forward_head(q, k, v, 0.5, window=(0, 0))
    j = np.arange(nq) + nk - nq
    np.testing.assert_allclose(o, v[j], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * np.einsum("id,id->i", q, k[j]), rtol=0, atol=1e-14)


def test_window_wider_than_the_keys_is_the_plain_mask():
    nq, nk, d = 7, 12, 4
    q, k, v = _rand((nq, d), 73), _rand((nk, d), 74), _rand((nk, 3), 75)
    for causal in (False, True):
        o_ref, lse_ref = oracle.forward_head(q, k, v, 0.6, causal=causal)
        o, lse = oracle.forward_head(q, k, v, 0.6, window=(nk + nq, 0 if causal else nk + nq))
        np.testing.assert_array_equal(o, o_ref)
        np.testing.assert_array_equal(lse, lse_ref)


@pytest.mark.parametrize("window", [(3, 0), (0, 2), (2, 5), (None, 1), (4, None)])
@pytest.mark.parametrize("nq,nk", [(9, 9), (5, 12), (12, 5)])
def test_banded_rows_equal_torch_sdpa_over_their_key_range(window, nq, nk):
    # Each row of banded attention is plain attention (PyTorch's float64 CPU
    # SDPA) of that query over the contiguous range of keys the band keeps.
    torch = pytest.importorskip("torch")
    q, k, v = _rand((nq, 4), 76), _rand((nk, 4), 77), _rand((nk, 3), 78)
    o, lse = oracle.forward_head(q, k, v, 0.8, window=window)
    left, right = window
    for i in range(nq):
        a = i + nk - nq
        lo = 0 if left is None else max(0, a - left)
        hi = nk - 1 if right is None else min(nk - 1, a + right)
        if hi < lo:
            assert np.all(o[i] == 0) and lse[i] == -np.inf
            continue
        tq = torch.from_numpy(q[i:i + 1])
        tk, tv = torch.from_numpy(k[lo:hi + 1]), torch.from_numpy(v[lo:hi + 1])
        o_ref = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], scale=0.8)[0]
        np.testing.assert_allclose(o[i], o_ref[0].numpy(), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[i], torch.logsumexp(0.8 * tq @ tk.T, dim=1).item(), rtol=0, atol=1e-13)


@pytest.mark.parametrize("window,nq,nk", [((2, 0), 6, 6), ((1, 1), 4, 7), ((None, 0), 7, 4)])
def test_banded_backward_matches_central_finite_differences(window, nq, nk):
    d, dv_ = 3, 2
    q, k, v = _rand((nq, d), 79), _rand((nk, d), 80), _rand((nk, dv_), 81)
    do = _rand((nq, dv_), 82)
    scale = 0.9
    dq, dk, dv = oracle.backward_head(q, k, v, do, scale, window=window)

    def loss(q_, k_, v_):
        o, _ = oracle.forward_head(q_, k_, v_, scale, window=window)
        return float((o * do).sum())

    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if a is x else a for a in (q, k, v)]
            args_m = [xm if a is x else a for a in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("window,nq,nk", [((3, 0), 16, 16), ((None, 0), 20, 9), ((2, 4), 9, 20)])
def test_banded_gradient_invariants(window, nq, nk):
    # rows of dS sum to 0, hence sum_j dK_j = 0; sum_j dV_j = sum of dO over
    # the rows that see at least one key
    q, k, v = _rand((nq, 5), 83), _rand((nk, 5), 84), _rand((nk, 3), 85)
    do = _rand((nq, 3), 86)
    _, lse = oracle.forward_head(q, k, v, 0.5, window=window)
    dq, dk, dv = oracle.backward_head(q, k, v, do, 0.5, window=window)
    live = np.isfinite(lse)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do[live].sum(axis=0), atol=1e-12)
    assert np.all(dq[~live] == 0)


def test_band_arguments_are_checked():
    q = _rand((3, 2), 87)
    with pytest.raises(ValueError):
        oracle.forward_head(q, q, q, 1.0, causal=True, window=(2, 1))
    with pytest.raises(ValueError):
        oracle.forward_head(q, q, q, 1.0, window=(-1, 0))


# ------------------------------------------------------------ additive bias ---

def test_row_constant_bias_moves_lse_only():
    q, k, v = _rand((9, 4), 90), _rand((13, 4), 91), _rand((13, 3), 92)
    c = _rand((9, 1), 93)
    o0, l0 = oracle.forward_head(q, k, v, 0.7, window=(3, 2))
    o1, l1 = oracle.forward_head(q, k, v, 0.7, window=(3, 2), bias=c)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l0 + c[:, 0], rtol=0, atol=1e-13)


def test_log_multiplicity_bias_equals_repeated_keys():
    # a bias of ln(m_j) on key j weighs it like m_j copies of that key
    q, k, v = _rand((6, 5), 94), _rand((4, 5), 95), _rand((4, 2), 96)
    m = np.array([1, 3, 2, 5])
    o, lse = oracle.forward_head(q, k, v, 0.6, bias=np.log(m)[None, :])
    o_rep, lse_rep = oracle.forward_head(q, np.repeat(k, m, axis=0), np.repeat(v, m, axis=0), 0.6)
    np.testing.assert_allclose(o, o_rep, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_rep, rtol=0, atol=1e-13)


def test_minus_inf_bias_removes_keys():
    q, k, v = _rand((5, 4), 97), _rand((8, 4), 98), _rand((8, 3), 99)
    keep = np.array([1, 0, 1, 1, 0, 0, 1, 1], bool)
    bias = np.where(keep, 0.0, -np.inf)[None, :]
    o, lse = oracle.forward_head(q, k, v, 0.9, bias=bias)
    o_ref, lse_ref = oracle.forward_head(q, k[keep], v[keep], 0.9)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)
    do = _rand((5, 3), 100)
    dq, dk, dv = oracle.backward_head(q, k, v, do, 0.9, bias=bias)
    rq, rk, rv = oracle.backward_head(q, k[keep], v[keep], do, 0.9)
    np.testing.assert_allclose(dq, rq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk[keep], rk, rtol=0, atol=1e-12)
    assert np.all(dk[~keep] == 0) and np.all(dv[~keep] == 0)


def test_bias_matches_torch_sdpa_float_mask_and_autograd():
    torch = pytest.importorskip("torch")
    q, k, v = _rand((7, 4), 101), _rand((11, 4), 102), _rand((11, 3), 103)
    bias, do = _rand((7, 11), 104), _rand((7, 3), 105)
    o, lse = oracle.forward_head(q, k, v, 0.5, bias=bias)
    dq, dk, dv = oracle.backward_head(q, k, v, do, 0.5, bias=bias)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    tb = torch.from_numpy(bias)
    to = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=tb[None],
                                                          scale=0.5)[0]
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(0.5 * tq @ tk.T + tb, dim=1).detach().numpy(),
                               rtol=0, atol=1e-13)
    (to * torch.from_numpy(do)).sum().backward()
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def test_bias_broadcasts_over_heads_in_the_batched_oracle():
    q, k, v = _rand((2, 3, 5, 4), 106), _rand((2, 3, 6, 4), 107), _rand((2, 3, 6, 2), 108)
    bias = _rand((1, 3, 1, 6), 109)           # per head, per key: a key-padding style bias
    o, lse = oracle.forward(q, k, v, 0.4, bias=bias, workers=1)
    for b in range(2):
        for h in range(3):
            ro, rl = oracle.forward_head(q[b, h], k[b, h], v[b, h], 0.4, bias=bias[0, h])
            np.testing.assert_allclose(o[b, h], ro, rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse[b, h], rl, rtol=0, atol=1e-14)


# -------------------------------------------- blockwise replay (the pages) ---

@pytest.mark.parametrize("block", [1, 3, 7, 16, 64, 100])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("order", ["sequential", "tree"])
def test_online_softmax_replay_equals_full_softmax(block, causal, order):
    n, d = 100, 16
    q, k, v = _rand((n, d), 33), _rand((n, d), 34), _rand((n, 12), 35)
    o_full, l_full = oracle.forward_head(q, k, v, 0.25, causal)
    o_rep, l_rep = orp.online_softmax_attention(q, k, v, 0.25, orp.partition_keys(n, block),
                                                causal=causal, order=order)
    np.testing.assert_allclose(o_rep, o_full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l_rep, l_full, rtol=1e-12, atol=1e-13)


def test_block_pair_merge_is_associative_commutative_with_empty_identity():
    """The algebra the replay rests on, checked directly on three key blocks:
    (A+B)+C = A+(B+C) = C+(A+B), the empty pair changes nothing, and a row
    hidden from a block contributes its empty pair."""
    rng = np.random.default_rng(7)
    q, k, v = rng.standard_normal((6, 4)), rng.standard_normal((9, 4)), rng.standard_normal((9, 3))
    vis = np.ones((6, 3), dtype=bool)
    a, b, c = (orp.block_pair(q, k[i:i + 3], v[i:i + 3], 0.7, vis) for i in (0, 3, 6))
    left = orp.merge(orp.merge(a, b), c)
    right = orp.merge(a, orp.merge(b, c))
    swapped = orp.merge(c, orp.merge(b, a))
    full = orp.block_pair(q, k, v, 0.7, np.ones((6, 9), dtype=bool))
    for x in (left, right, swapped):
        np.testing.assert_allclose(x[0], full[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(x[1], full[1], rtol=1e-13, atol=1e-14)
    empty = (np.zeros((6, 3)), np.full(6, -np.inf))
    e = orp.merge(empty, a)
    np.testing.assert_array_equal(e[0], a[0])
    np.testing.assert_array_equal(e[1], a[1])
    hidden = orp.block_pair(q, k[:3], v[:3], 0.7, np.zeros((6, 3), dtype=bool))
    np.testing.assert_array_equal(hidden[0], 0.0)
    assert np.all(np.isneginf(hidden[1]))
    both = orp.merge(hidden, hidden)
    assert np.all(np.isneginf(both[1])) and np.all(both[0] == 0.0)


@pytest.mark.parametrize("seed", range(5))
def test_replay_random_partitions_and_rising_max(seed):
    rng = np.random.default_rng(100 + seed)
    n, d = 77, 8
    q = rng.standard_normal((n, d)) * 4          # peaky rows
    k = rng.standard_normal((n, d)) * (1 + np.arange(n) / n)[:, None]  # rising max
    v = rng.standard_normal((n, 5))
    cuts = np.sort(rng.choice(np.arange(1, n), size=rng.integers(1, 20), replace=False))
    bounds = np.concatenate([[0], cuts, [n]])
    blocks = list(zip(bounds[:-1], bounds[1:]))
    if seed % 2:
        blocks = blocks[::-1]                     # order does not matter (exact maths)
    o_full, l_full = oracle.forward_head(q, k, v, 0.5)
    for order in ("sequential", "tree"):
        o_rep, l_rep = orp.online_softmax_attention(q, k, v, 0.5, blocks, order=order)
        np.testing.assert_allclose(o_rep, o_full, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(l_rep, l_full, rtol=1e-12, atol=1e-12)


# --------------------------------------- independent library special case ---

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_torch_sdpa_float64(causal):
    b, h, n, d = 2, 3, 45, 16
    q, k, v = (_rand((b, h, n, d), s) for s in (40, 41, 42))
    scale = 0.19
    o, lse = oracle.forward(q, k, v, scale, causal, workers=2)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale,
                                                           is_causal=causal)
    s = scale * tq @ tk.transpose(-1, -2)
    if causal:
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd_float64(causal):
    b, h, n, d = 1, 2, 29, 8
    q, k, v, do = (_rand((b, h, n, d), s) for s in (50, 51, 52, 53))
    scale = 0.37
    dq, dk, dv = oracle.backward(q, k, v, do, scale, causal, workers=2)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale,
                                                           is_causal=causal)
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------- finite differences ---

@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_finite_differences(causal):
    n, d, scale, eps = 6, 3, 0.8, 1e-6
    q, k, v, do = _rand((n, d), 60), _rand((n, d), 61), _rand((n, d), 62), _rand((n, d), 63)
    dq, dk, dv = oracle.backward_head(q, k, v, do, scale, causal)

    def loss(qq, kk, vv):
        return float((oracle.forward_head(qq, kk, vv, scale, causal)[0] * do).sum())

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * eps)
        err = np.abs(num - g).max() / max(1e-12, np.abs(g).max())
        assert err < 1e-6, (name, err)


# ---------------------------------------------------- gradient invariants ---

@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    n, d = 31, 8
    q, k, v, do = _rand((n, d), 70), _rand((n, d), 71), _rand((n, d), 72), _rand((n, d), 73)
    dq, dk, dv = oracle.backward_head(q, k, v, do, 0.3, causal)
    # shifting every key by the same vector leaves O unchanged
    np.testing.assert_allclose(dk.sum(0), 0.0, rtol=0, atol=1e-12)
    # each probability row sums to one
    np.testing.assert_allclose(dv.sum(0), do.sum(0), rtol=0, atol=1e-12)
    # constant V: O does not depend on Q or K
    dq0, dk0, _ = oracle.backward_head(q, k, np.repeat(v[:1], n, 0), do, 0.3, causal)
    np.testing.assert_allclose(dq0, 0.0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk0, 0.0, rtol=0, atol=1e-13)


def test_batched_equals_per_head():
    b, h, n, d = 2, 2, 19, 4
    q, k, v, do = (_rand((b, h, n, d), s) for s in (80, 81, 82, 83))
    o, lse = oracle.forward(q, k, v, 0.5, True, workers=3)
    dq, dk, dv = oracle.backward(q, k, v, do, 0.5, True, workers=3)
    for bi in range(b):
        for hi in range(h):
            oh, lh = oracle.forward_head(q[bi, hi], k[bi, hi], v[bi, hi], 0.5, True)
            gq, gk, gv = oracle.backward_head(q[bi, hi], k[bi, hi], v[bi, hi], do[bi, hi], 0.5, True)
            np.testing.assert_array_equal(o[bi, hi], oh)
            np.testing.assert_array_equal(lse[bi, hi], lh)
            np.testing.assert_array_equal(dq[bi, hi], gq)
            np.testing.assert_array_equal(dk[bi, hi], gk)
            np.testing.assert_array_equal(dv[bi, hi], gv)


def test_row_chunking_does_not_change_results(monkeypatch):
    n, d = 50, 8
    q, k, v, do = _rand((n, d), 90), _rand((n, d), 91), _rand((n, d), 92), _rand((n, d), 93)
    o1, l1 = oracle.forward_head(q, k, v, 0.5, True)
    g1 = oracle.backward_head(q, k, v, do, 0.5, True)
    monkeypatch.setattr(oa, "_ROW_CHUNK", 7)
    o2, l2 = oracle.forward_head(q, k, v, 0.5, True)
    g2 = oracle.backward_head(q, k, v, do, 0.5, True)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-14)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_score_matrix_size_at_8k_tokens():
    # The pages count about 64 million score entries at 8,000 tokens per head;
    # the long-context workload (8192 tokens) has exactly 2**26 of them.
    assert 8192 * 8192 == 2 ** 26
    assert abs(8000 * 8000 - 64e6) < 1
