"""fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. Shares no code with
the HIP kernels or their C-ABI library.

Every function is pinned by the CPU test suite (closed forms, hand-worked
cases, invariants, the blockwise replay of the pages' procedure, PyTorch's
float64 CPU attention and autograd, finite differences).
"""
from .attention import forward, backward, forward_head, backward_head  # noqa: F401
from .replay import online_softmax_attention, partition_keys  # noqa: F401
