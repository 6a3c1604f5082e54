"""Seeded synthetic inputs for attention workloads.

This module only draws random numbers and converts their storage type. It
holds none of the attention arithmetic, so both the fp64 CPU oracle (through
the tests and the benchmark) and the HIP path can consume the same bytes.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per workload):
  draw order Q, K, V, then dO (only when a backward pass is needed);
  each tensor is ``standard_normal(size=(B, H, N, d), dtype=float32)``;
  for bf16 workloads the fp32 draw is rounded to bfloat16 with
  round-to-nearest-even on the bit pattern (the same rule as
  ``torch.Tensor.to(torch.bfloat16)``); fp16 workloads round it to IEEE half
  (numpy's float32 -> float16 cast, also round-to-nearest-even).
Layout: contiguous [B, H, N, d], d innermost (K and V may have their own
row count Nk). bf16 tensors are carried as their uint16 bit patterns.

The workloads mirror the pages' long-context self-attention (score matrices
of tens of millions of entries per head, 'FlashAttention' on josueisai.com,
section on the matrix that should never be stored).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

# Named workloads. Seeds are fixed so every run sees identical bytes.
WORKLOADS = {
    "tiny_fp32": dict(B=1, H=1, N=256, d=64, dtype="fp32", causal=False,
                      backward=False, seed=1221),
    "fwd_n2048_d64": dict(B=4, H=16, N=2048, d=64, dtype="bf16", causal=False,
                          backward=False, seed=1222),
    "fwd_n8192_d128": dict(B=1, H=32, N=8192, d=128, dtype="bf16",
                           causal=False, backward=False, seed=1223),
    "causal_fwd_n16384_d128": dict(B=2, H=32, N=16384, d=128, dtype="bf16",
                                   causal=True, backward=False, seed=1224),
    "train_n4096_d128": dict(B=2, H=16, N=4096, d=128, dtype="bf16",
                             causal=False, backward=True, seed=1225),
    # General shapes and masks (beyond equal-length, top-left causal
    # self-attention), each at a long-context size:
    #   a local window of 1024 earlier keys over 16k tokens;
    "window_n16384_d128_w1024": dict(B=2, H=32, N=16384, d=128, dtype="bf16",
                                     causal=False, window=(1024, 0),
                                     backward=True, seed=1226),
    #   512 new queries per head over a 16k-key cache, causal (aligned with
    #   the last keys);
    "prefill_q512_k16384_d128": dict(B=8, H=32, N=512, nk=16384, d=128,
                                     dtype="bf16", causal=True,
                                     backward=True, seed=1227),
    #   the 8k self-attention shape in fp16, and in [B, N, H, d] memory.
    "fp16_n8192_d128": dict(B=1, H=32, N=8192, d=128, dtype="fp16",
                            causal=False, backward=True, seed=1228),
    "bnhd_n8192_d128": dict(B=1, H=32, N=8192, d=128, dtype="bf16",
                            causal=False, backward=True, layout="bnhd",
                            seed=1229),
    #   other head dimensions at the 8k length (H * d = 4096 where it divides)
    "d32_n8192": dict(B=1, H=128, N=8192, d=32, dtype="bf16", causal=False,
                      backward=True, seed=1230),
    "d96_n8192": dict(B=1, H=32, N=8192, d=96, dtype="bf16", causal=False,
                      backward=True, seed=1231),
    "d256_n8192": dict(B=1, H=16, N=8192, d=256, dtype="bf16", causal=False,
                       backward=True, seed=1232),
    #   an additive fp32 bias per head, shared over the batch (the shape of a
    #   learned relative-position bias), drawn N(0,1) after Q, K, V, dO
    "bias_n4096_d128": dict(B=2, H=16, N=4096, d=128, dtype="bf16", causal=False,
                            backward=True, bias=(1, 16, 4096, 4096), seed=1233),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = (b + 0x7FFF + lsb) >> 16
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tensor:
    """A host tensor as the GPU will see it: raw storage plus its dtype."""
    storage: np.ndarray          # uint16 bits (bf16), float16 or float32 values
    dtype: str                   # "bf16" | "fp16" | "fp32"
    sha256: str = field(default="")

    def __post_init__(self):
        if not self.sha256:
            self.sha256 = hashlib.sha256(self.storage.tobytes()).hexdigest()

    @property
    def shape(self):
        return self.storage.shape

    def to_f32(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.storage)
        return self.storage.astype(np.float32, copy=False)

    def to_f64(self) -> np.ndarray:
        """Exact values widened to float64."""
        return self.to_f32().astype(np.float64)

    def to_torch(self, device="cpu"):
        import torch
        if self.dtype == "bf16":
            t = torch.from_numpy(self.storage.view(np.int16).copy()).view(torch.bfloat16)
        else:
            t = torch.from_numpy(self.storage.copy())
        return t.to(device)

    @staticmethod
    def from_f32(x: np.ndarray, dtype: str) -> "Tensor":
        """Round float32 values to the storage type (round-to-nearest-even)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        if dtype == "bf16":
            return Tensor(f32_to_bf16_bits(x), "bf16")
        if dtype == "fp16":
            return Tensor(x.astype(np.float16), "fp16")
        if dtype == "fp32":
            return Tensor(x, "fp32")
        raise ValueError(f"unknown dtype {dtype!r}")


def _draw(rng: np.random.Generator, shape, dtype: str) -> Tensor:
    return Tensor.from_f32(rng.standard_normal(size=shape, dtype=np.float32), dtype)


def generate(B: int, H: int, N: int, d: int, dtype: str, seed: int,
             with_grad_output: bool = False, nk: int | None = None) -> dict:
    """Draw Q [B, H, N, d], K and V [B, H, nk, d] (nk = N by default) and dO
    [B, H, N, d] from one seeded PCG64, in that order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nk = N if nk is None else nk
    out = {"q": _draw(rng, (B, H, N, d), dtype), "k": _draw(rng, (B, H, nk, d), dtype),
           "v": _draw(rng, (B, H, nk, d), dtype)}
    if with_grad_output:
        out["do"] = _draw(rng, (B, H, N, d), dtype)
    return out


def generate_workload(name: str) -> dict:
    w = WORKLOADS[name]
    return generate(w["B"], w["H"], w["N"], w["d"], w["dtype"], w["seed"],
                    with_grad_output=w["backward"], nk=w.get("nk"))


def generate_bias(shape, seed: int) -> np.ndarray:
    """A float32 N(0,1) bias of `shape` from its own PCG64(seed)."""
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(size=shape, dtype=np.float32)


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32, the value handed to both sides."""
    return float(np.float32(1.0 / np.sqrt(np.float64(d))))
