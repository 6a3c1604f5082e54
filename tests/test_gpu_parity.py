"""GPU parity at small sizes: the HIP path (through the C ABI) against the fp64
oracle, element by element, over shapes that span several tiles and ragged
tails, both head dimensions, causal and not, and the degenerate cases."""
import numpy as np
import pytest

import oracle
from exact_attention_122_amd import fa, inputs

from gpu_util import REL_FRO, TOL, compare, f64, gpu_fwd, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SHAPES_N = [1, 17, 64, 128, 200, 256, 320]


def _oracle_fwd(g, scale, causal):
    return oracle.forward(g["q"].to_f64(), g["k"].to_f64(), g["v"].to_f64(), scale, causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", SHAPES_N)
def test_fwd_bf16_small(n, d, causal):
    g = inputs.generate(1, 2, n, d, "bf16", seed=1000 + n + d)
    scale = inputs.default_scale(d)
    _, _, _, o, lse = gpu_fwd(g, causal, scale)
    ro, rl = _oracle_fwd(g, scale, causal)
    compare("O", f64(o), ro, TOL["bf16"]["o"], REL_FRO)
    compare("LSE", f64(lse), rl, TOL["bf16"]["lse"])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 31, 64, 100, 256])
def test_fwd_fp32_small(n, d, causal):
    g = inputs.generate(1, 2, n, d, "fp32", seed=2000 + n + d)
    scale = inputs.default_scale(d)
    _, _, _, o, lse = gpu_fwd(g, causal, scale)
    ro, rl = _oracle_fwd(g, scale, causal)
    compare("O", f64(o), ro, TOL["fp32"]["o"])
    compare("LSE", f64(lse), rl, TOL["fp32"]["lse"])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 17, 64, 200, 320])
def test_bwd_bf16_small_end_to_end(n, d, causal):
    g = inputs.generate(1, 2, n, d, "bf16", seed=3000 + n + d, with_grad_output=True)
    scale = inputs.default_scale(d)
    q, k, v, o, lse = gpu_fwd(g, causal, scale)
    do = to_dev(g["do"])
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward(g["q"].to_f64(), g["k"].to_f64(), g["v"].to_f64(), g["do"].to_f64(),
                                 scale, causal)
    tol = TOL["bf16"]["grad"]
    compare("dQ", f64(dq), rq, tol, REL_FRO)
    compare("dK", f64(dk), rk, tol, REL_FRO)
    compare("dV", f64(dv), rv, tol, REL_FRO)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_fed_with_oracle_forward(causal):
    """fa_bwd alone: O (rounded to bf16) and LSE come from the oracle."""
    n, d = 192, 128
    g = inputs.generate(2, 2, n, d, "bf16", seed=3500, with_grad_output=True)
    scale = inputs.default_scale(d)
    ro, rl = _oracle_fwd(g, scale, causal)
    o = torch.from_numpy(ro.astype(np.float32)).to(torch.bfloat16).cuda()
    lse = torch.from_numpy(rl.astype(np.float32)).cuda()
    q, k, v, do = (to_dev(g[x]) for x in ("q", "k", "v", "do"))
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward(g["q"].to_f64(), g["k"].to_f64(), g["v"].to_f64(), g["do"].to_f64(),
                                 scale, causal)
    for name, a, b in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        compare(name, f64(a), b, TOL["bf16"]["grad"], REL_FRO)


@pytest.mark.parametrize("scale", [-0.0883883, 0.0, 1.0, 0.5])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_bwd_unusual_scales(scale, causal):
    """Negative scale (sign flip of Q), zero scale (uniform attention) and large
    scales (scores with std ~ 11: the running max moves a lot)."""
    n, d = 160, 128
    g = inputs.generate(1, 2, n, d, "bf16", seed=4000, with_grad_output=True)
    scale = float(np.float32(scale))
    q, k, v, o, lse = gpu_fwd(g, causal, scale)
    ro, rl = _oracle_fwd(g, scale, causal)
    compare("O", f64(o), ro, TOL["bf16"]["o"], REL_FRO)
    # LSE is summed in fp32 from fp32 probabilities: the 1e-3 bound holds at
    # every scale (measured below 1e-5 at scale 1)
    compare("LSE", f64(lse), rl, TOL["bf16"]["lse"])
    do = to_dev(g["do"])
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward(g["q"].to_f64(), g["k"].to_f64(), g["v"].to_f64(), g["do"].to_f64(),
                                 scale, causal)
    # bf16 rounding error grows with the magnitude of what is rounded: the
    # bound is 2e-2 per unit of the largest reference entry (at least 1)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        compare(name, f64(got), ref, TOL["bf16"]["grad"] * max(1.0, float(np.abs(ref).max())), REL_FRO)


@pytest.mark.parametrize("kind", ["peaky", "rising_max"])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_adversarial_rescale(kind, causal):
    """Inputs that force the online-softmax rescale: near one-hot rows (Q x 8)
    and keys whose scale grows along the sequence, so the max keeps rising."""
    n, d = 512, 128
    rng = np.random.Generator(np.random.PCG64(4500))
    q = rng.standard_normal((1, 2, n, d), dtype=np.float32)
    k = rng.standard_normal((1, 2, n, d), dtype=np.float32)
    v = rng.standard_normal((1, 2, n, d), dtype=np.float32)
    if kind == "peaky":
        q *= 8
    else:
        k *= (1 + 3 * np.arange(n, dtype=np.float32) / n)[None, None, :, None]
    g = {name: inputs.Tensor(inputs.f32_to_bf16_bits(x), "bf16") for name, x in zip("qkv", (q, k, v))}
    scale = inputs.default_scale(d)
    _, _, _, o, lse = gpu_fwd(g, causal, scale)
    ro, rl = _oracle_fwd(g, scale, causal)
    compare("O", f64(o), ro, TOL["bf16"]["o"], REL_FRO)
    compare("LSE", f64(lse), rl, TOL["bf16"]["lse"])


@pytest.mark.parametrize("kind", ["overflow", "jump", "rise", "crowd"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_fwd_reference_point_fallback(kind, causal, d):
    """Tiles far above a row's reference point. The kernel takes the
    exponentials against the current reference first and checks their lane
    sum; past 2^16 it forms the scores again and moves the reference. Cases: a
    key hundreds of log2 units above the earlier ones (the first exponentials
    overflow to inf) and a jump of about 40 units, both through the fallback; a
    rise of about 12 units and a crowd of 64 keys about 5 units up, both kept
    against the old reference (p up to 2^12 and large sums)."""
    n = 333
    rng = np.random.Generator(np.random.PCG64(4600 + d))
    scale = inputs.default_scale(d)
    q = 1.0 + 0.1 * rng.standard_normal((1, 2, n, d), dtype=np.float32)
    k = 0.1 * rng.standard_normal((1, 2, n, d), dtype=np.float32)
    v = rng.standard_normal((1, 2, n, d), dtype=np.float32)
    if kind == "overflow":
        k[:, :, 150, :] = 20.0
    elif kind == "jump":
        k[:, :, 150, :] = 30.0 / (d * scale)
    elif kind == "rise":
        k[:, :, 150, :] = 8.5 / (d * scale)
    else:
        k[:, :, 200:264, :] = 3.5 / (d * scale)
    g = {name: inputs.Tensor(inputs.f32_to_bf16_bits(x), "bf16") for name, x in zip("qkv", (q, k, v))}
    _, _, _, o, lse = gpu_fwd(g, causal, scale)
    ro, rl = _oracle_fwd(g, scale, causal)
    compare("O", f64(o), ro, TOL["bf16"]["o"], REL_FRO)
    compare("LSE", f64(lse), rl, TOL["bf16"]["lse"])


def test_constant_v_and_identical_keys_on_gpu():
    n, d = 256, 64
    rng = np.random.Generator(np.random.PCG64(4600))
    q = rng.standard_normal((1, 1, n, d), dtype=np.float32)
    krow = rng.standard_normal((1, 1, 1, d), dtype=np.float32)
    k = np.repeat(krow, n, axis=2)
    v = np.repeat(rng.standard_normal((1, 1, 1, d), dtype=np.float32), n, axis=2)
    g = {name: inputs.Tensor(inputs.f32_to_bf16_bits(x), "bf16") for name, x in zip("qkv", (q, k, v))}
    for causal in (False, True):
        _, _, _, o, lse = gpu_fwd(g, causal, 0.125)
        # constant V: every output row is that row (exact up to bf16 rounding)
        np.testing.assert_allclose(f64(o), np.repeat(g["v"].to_f64()[:, :, :1], n, 2), rtol=0, atol=1e-2)
        cnt = np.arange(1, n + 1) if causal else np.full(n, n)
        qf, kf = g["q"].to_f64()[0, 0], g["k"].to_f64()[0, 0, 0]
        np.testing.assert_allclose(f64(lse)[0, 0], 0.125 * qf @ kf + np.log(cnt), rtol=0, atol=1e-3)


def test_fwd_is_bitwise_deterministic():
    g = inputs.generate(2, 3, 300, 128, "bf16", seed=4700)
    _, _, _, o1, l1 = gpu_fwd(g, True, 0.088388)
    _, _, _, o2, l2 = gpu_fwd(g, True, 0.088388)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("d,causal", [(128, False), (128, True), (64, False), (256, False)])
def test_fwd_repeated_launches_bitwise(d, causal):
    """Ten back-to-back launches on a grid that fills every CU, each equal bit for
    bit to the first: a tile read before its global -> LDS copy has landed, or
    a copy that overwrites a tile still being read, would show up as launches
    that differ."""
    B, H, N = 1, 32, 2048 if d == 256 else 4096
    g = inputs.generate(B, H, N, d, "bf16", seed=5100 + d + causal)
    q, k, v = (to_dev(g[x]) for x in ("q", "k", "v"))
    scale = inputs.default_scale(d)
    outs = []
    for _ in range(10):
        outs.append(fa.fa_fwd(q, k, v, causal=causal, scale=scale))
    torch.cuda.synchronize()
    o0, l0 = outs[0]
    for o, lse in outs[1:]:
        assert torch.equal(o, o0) and torch.equal(lse, l0)
    # and the first launch is right: sampled rows against the oracle
    rows = np.array([0, 1, 255, 256, 1000, N - 1])
    ro, rl = oracle.forward(g["q"].to_f64()[:, :2], g["k"].to_f64()[:, :2], g["v"].to_f64()[:, :2], scale, causal)
    compare("O", f64(o0[:, :2])[:, :, rows], ro[:, :, rows], TOL["bf16"]["o"])
    compare("LSE", f64(l0[:, :2])[:, :, rows], rl[:, :, rows], TOL["bf16"]["lse"])


def test_bwd_is_bitwise_deterministic():
    g = inputs.generate(1, 2, 256, 64, "bf16", seed=4800, with_grad_output=True)
    q, k, v, o, lse = gpu_fwd(g, False, 0.125)
    do = to_dev(g["do"])
    a = fa.fa_bwd(q, k, v, o, do, lse, scale=0.125)
    b = fa.fa_bwd(q, k, v, o, do, lse, scale=0.125)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_non_default_stream():
    g = inputs.generate(1, 4, 384, 128, "bf16", seed=4900)
    q, k, v, o_ref, l_ref = gpu_fwd(g, False, 0.088388)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, lse = fa.fa_fwd(q, k, v, scale=0.088388)
    s.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_library_allocates_nothing():
    """Extra memory is linear in N: outputs only, no N x N buffer anywhere."""
    g = inputs.generate(1, 8, 4096, 128, "bf16", seed=5000, with_grad_output=True)
    q, k, v, do = (to_dev(g[x]) for x in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(1, 8, 4096, 128), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    fa.fa_fwd(q, k, v, out=o, lse=lse)
    fa.fa_bwd(q, k, v, o, do, lse, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == base


def test_empty_problem_on_gpu():
    q = torch.empty(0, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = fa.fa_fwd(q, q, q)
    assert o.shape == q.shape and lse.shape == (0, 2, 16)
    q = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = fa.fa_fwd(q, q, q)
    dq, dk, dv = fa.fa_bwd(q, q, q, o, q, lse)
    torch.cuda.synchronize()
    assert dq.shape == q.shape


def test_unsupported_requests_raise():
    q = torch.zeros(1, 1, 64, 80, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        fa.fa_fwd(q, q, q)
    q = torch.zeros(1, 1, 64, 64, dtype=torch.float64, device="cuda")
    with pytest.raises(RuntimeError, match="not built"):
        fa.fa_fwd(q, q, q)
    q = torch.zeros(1, 1, 64, 64, dtype=torch.float32, device="cuda")
    o, lse = fa.fa_fwd(q, q, q)
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        fa.fa_bwd(q, q, q, o, q, lse)
