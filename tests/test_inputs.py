"""The seeded input generator: determinism, recipe, bf16 rounding."""
import numpy as np
import pytest

from exact_attention_122_amd import inputs


def test_same_seed_same_bytes():
    a = inputs.generate(1, 2, 33, 16, "bf16", 7, with_grad_output=True)
    b = inputs.generate(1, 2, 33, 16, "bf16", 7, with_grad_output=True)
    for name in ("q", "k", "v", "do"):
        assert a[name].sha256 == b[name].sha256
        np.testing.assert_array_equal(a[name].storage, b[name].storage)
    c = inputs.generate(1, 2, 33, 16, "bf16", 8)
    assert c["q"].sha256 != a["q"].sha256


def test_draw_order_and_distribution():
    g = inputs.generate(1, 1, 64, 32, "fp32", 1221, with_grad_output=True)
    rng = np.random.Generator(np.random.PCG64(1221))
    for name in ("q", "k", "v", "do"):
        ref = rng.standard_normal(size=(1, 1, 64, 32), dtype=np.float32)
        np.testing.assert_array_equal(g[name].storage, ref)
    big = inputs.generate(1, 1, 4096, 64, "fp32", 3)["q"].storage
    assert abs(big.mean()) < 0.01 and abs(big.std() - 1) < 0.01


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.00390625, 3.4e38, 1e-40,
                                  0.0, -0.0, np.inf, -np.inf], np.float32)])
    bits = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = inputs.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_to_torch_roundtrip():
    torch = pytest.importorskip("torch")
    g = inputs.generate(1, 1, 8, 4, "bf16", 5)
    t = g["q"].to_torch()
    assert t.dtype == torch.bfloat16 and tuple(t.shape) == (1, 1, 8, 4)
    np.testing.assert_array_equal(t.float().numpy(), g["q"].to_f32())


def test_workload_table():
    w = inputs.WORKLOADS["fwd_n8192_d128"]
    assert (w["B"], w["H"], w["N"], w["d"], w["dtype"], w["causal"]) == (1, 32, 8192, 128, "bf16", False)
    assert inputs.WORKLOADS["causal_fwd_n16384_d128"]["causal"]
    assert inputs.WORKLOADS["train_n4096_d128"]["backward"]
    assert inputs.default_scale(64) == 0.125
    assert inputs.default_scale(128) == float(np.float32(1 / np.sqrt(128)))


def test_fp16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    g = inputs.generate(1, 2, 40, 16, "fp16", 9)
    x = np.random.Generator(np.random.PCG64(9)).standard_normal(size=(1, 2, 40, 16), dtype=np.float32)
    ref = torch.from_numpy(x).to(torch.float16).numpy()
    np.testing.assert_array_equal(g["q"].storage, ref)
    t = g["q"].to_torch()
    assert t.dtype == torch.float16
    np.testing.assert_array_equal(t.float().numpy(), g["q"].to_f32())


def test_unequal_key_length_keeps_the_draw_order():
    g = inputs.generate(1, 1, 5, 8, "fp32", 11, with_grad_output=True, nk=7)
    rng = np.random.Generator(np.random.PCG64(11))
    for name, rows in (("q", 5), ("k", 7), ("v", 7), ("do", 5)):
        np.testing.assert_array_equal(g[name].storage, rng.standard_normal(size=(1, 1, rows, 8), dtype=np.float32))
