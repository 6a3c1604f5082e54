"""Plant plausible mistakes in the oracle and check the pins catch each one.

Each mutation edits one expression of the oracle's source (a dropped term, a
wrong sign or index, a transposed operand, a dropped scale), rebuilds that
function and runs the hand-worked cases plus two invariants against it. A
mutation that no pin notices would mean the pins are too weak.
"""
import inspect
import textwrap

import numpy as np
import pytest

from oracle import attention as oa

import test_oracle_pins as pins

MUTATIONS = [
    ("_scores", "float(scale) * (q_rows @ k.T)", "(q_rows @ k.T)"),
    ("_scores", "float(scale) * (q_rows @ k.T)", "float(scale) * (q_rows @ k.T) + 0.01"),
    ("_scores", "j > diag[:, None] + right", "j >= diag[:, None] + right"),
    ("_scores", "j < diag[:, None] - left", "j <= diag[:, None] - left"),
    ("_scores", "j < diag[:, None] - left", "j < diag[:, None] + left"),
    ("_scores", "row_idx + (k.shape[0] - nq)", "row_idx"),
    ("_scores", "row_idx + (k.shape[0] - nq)", "row_idx + (nq - k.shape[0])"),
    ("_band", "        right = 0\n", "        right = None\n"),
    ("_scores", "s = s + bias_rows", "s = s - bias_rows"),
    ("_scores", "s = s + bias_rows", "s = s + float(scale) * bias_rows"),
    ("_softmax_rows", "m = s.max(axis=1)", "m = s.min(axis=1)"),
    ("_softmax_rows", "p = e / np.where(dead, 1.0, l)[:, None]", "p = e / np.where(dead, 1.0, l.max())"),
    ("forward_head", "m + np.log(l)", "np.log(l)"),
    ("forward_head", "p @ v", "p @ v[::-1]"),
    ("backward_head", "dv += p.T @ g", "dv += p.T @ g[::-1]"),
    ("backward_head", "dp - d_row[:, None]", "dp + d_row[:, None]"),
    ("backward_head", "d_row = (p * dp).sum(axis=1)", "d_row = dp.sum(axis=1)"),
    ("backward_head", "dq[idx] = float(scale) * (ds @ k)", "dq[idx] = (ds @ k)"),
    ("backward_head", "dk += float(scale) * (ds.T @ q[idx])", "dk += (ds.T @ q[idx])"),
    ("backward_head", "dp = g @ v.T", "dp = g @ v[::-1].T"),
]


def _mutated(fn_name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(oa, fn_name)))
    assert src.count(old) == 1, (fn_name, old)
    ns = dict(vars(oa))
    exec(compile(src.replace(old, new), f"<mutant {fn_name}>", "exec"), ns)
    return ns[fn_name], ns


def _pins_pass():
    checks = []
    for case in pins._load_cases():
        checks.append(lambda c=case: pins.test_hand_worked_forward(c))
        checks.append(lambda c=case: pins.test_hand_worked_backward(c))
    for causal in (False, True):
        checks.append(lambda c=causal: pins.test_identical_keys_give_mean_of_v(c))
        checks.append(lambda c=causal: pins.test_gradient_invariants(c))
    checks.append(pins.test_large_scores_do_not_overflow)
    for check in checks:
        try:
            with np.errstate(all="ignore"):
                check()
        except Exception:
            return False
    return True


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("fn_name,old,new", MUTATIONS,
                         ids=[f"{m[0]}:{m[2]}" for m in MUTATIONS])
def test_each_planted_mistake_is_caught(monkeypatch, fn_name, old, new):
    mutant, ns = _mutated(fn_name, old, new)
    monkeypatch.setattr(oa, fn_name, mutant)
    # helpers called by other oracle functions are looked up in oa's globals
    for name in ("_scores", "_softmax_rows", "_band"):
        if name == fn_name:
            ns[name] = mutant
    # the public entry points in oracle/__init__ are the same objects as oa's
    import oracle
    if hasattr(oracle, fn_name):
        monkeypatch.setattr(oracle, fn_name, mutant)
    assert not _pins_pass(), f"mutation survived: {fn_name}: {old!r} -> {new!r}"
