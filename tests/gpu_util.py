"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
compare with the fp64 oracle element by element."""
import json
import os

import numpy as np

from exact_attention_122_amd import fa, inputs

# When FA_PARITY_LOG names a file, every comparison appends one JSON line to
# it (test, output, measured max-abs and relative Frobenius errors, bound), so
# a run records the errors it measured and not only that they passed.
_LOG = os.environ.get("FA_PARITY_LOG")


def _log(name, err, fro, atol, rel, n):
    if not _LOG:
        return
    rec = {"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], "output": name,
           "max_abs": err, "rel_fro": fro, "atol": atol, "rel_bound": rel, "elements": int(n)}
    with open(_LOG, "a") as f:
        f.write(json.dumps(rec) + "\n")

# Tolerances (max abs error vs the fp64 oracle). bf16 inputs, fp32 accumulation:
# O and dQ/dK/dV 2e-2, LSE 1e-3; float32 end to end: 1e-5 on O and LSE.
TOL = {
    "bf16": dict(o=2e-2, lse=1e-3, grad=2e-2),
    "fp32": dict(o=1e-5, lse=1e-5, grad=None),
    # fp16 keeps 11 significant bits to bf16's 8: the same rounding steps (P,
    # dS and the outputs) err 8x less, so the bf16 bounds shrink 4x for O and
    # 2x for the gradients, keeping a 2-4x margin; LSE is fp32 in both.
    "fp16": dict(o=5e-3, lse=1e-3, grad=1e-2),
}
# Relative Frobenius bound on top of max-abs. The max-abs bound alone is loose
# for outputs whose entries are ~1/sqrt(N); bf16 rounding of P and of the
# outputs keeps the relative error near 2^-8, so 2e-2 leaves ample room while
# still catching a dropped tile or a wrong row.
REL_FRO = 2e-2


def to_dev(t: "inputs.Tensor"):
    return t.to_torch("cuda")


def f64(x):
    return x.detach().float().cpu().numpy().astype(np.float64)


def compare(name, got, ref, atol, rel=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    # rows with no visible key: the oracle's LSE is -inf and so must ours be
    dead = np.isneginf(ref)
    if dead.any():
        assert np.all(np.isneginf(got[dead])), f"{name}: expected -inf where no key is visible"
        got, ref = got[~dead], ref[~dead]
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    diff = got - ref
    err = float(np.abs(diff).max()) if got.size else 0.0
    den = float(np.linalg.norm(ref)) if got.size else 0.0
    fro = float(np.linalg.norm(diff) / den) if den > 0 else None
    del diff
    _log(name, err, fro, atol, rel, got.size)
    assert err <= atol, f"{name}: max abs err {err:.3e} > {atol:.1e}"
    if rel is not None and fro is not None:
        assert fro <= rel, f"{name}: relative Frobenius err {fro:.3e} > {rel:.1e}"
    return err


def gpu_fwd(g, causal, scale):
    q, k, v = (to_dev(g[n]) for n in ("q", "k", "v"))
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    import torch
    torch.cuda.synchronize()
    return q, k, v, o, lse
