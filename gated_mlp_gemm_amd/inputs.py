"""Seeded synthetic inputs for the SwiGLU GEMM workloads.

This module only draws random numbers; it holds none of the method's
arithmetic.  Both the HIP path's tests/bench and the CPU oracle's tests take
their inputs from here, and from nowhere else.

Recipe (the same for every workload): a CPU ``torch.Generator`` seeded with
the workload's seed draws, in this order, A [M,K], W1 [K,N] and W2 [K,N] as
float32 standard normals; A is rounded to bf16, W1 and W2 are first divided
by sqrt(K) in float32 and then rounded to bf16 (torch's cast rounds to
nearest, ties to even).  So A ~ N(0,1) and W ~ N(0,1/K), which makes Gate and
Up ~ N(0,1) per element.  These stand in for the Qwen-2.5 MLP activations and
weights that the pages evaluate on (paper abstract: Qwen-2.5 0.5B-72B); the
K x N shapes below are Qwen-2.5-class MLP shapes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    seed: int
    note: str

    @property
    def flops(self) -> int:
        """4 M N K: two M x N x K contractions, 2 flops per multiply-add."""
        return 4 * self.M * self.N * self.K


# The five synthetic workloads (shapes and seeds of the benchmark configs).
WORKLOADS = (
    Workload("qwen0.5b_m128", 128, 896, 4864, 0, "0.5B-class gated MLP, small batch"),
    Workload("m2048_k1536_n8960", 2048, 1536, 8960, 1, "M at the S/I crossover"),
    Workload("m512_k3584_n18944", 512, 3584, 18944, 2, "small batch, interleaved variant"),
    Workload("m8192_k5120_n13824", 8192, 5120, 13824, 3, "large batch, sequential variant"),
    Workload("m4096_k8192_n29568", 4096, 8192, 29568, 4, "72B-class MLP, compute-bound limit"),
)


def make_inputs(M: int, K: int, N: int, seed: int,
                a_scale: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """A [M,K], W1 [K,N], W2 [K,N] as CPU bf16 tensors (recipe above).

    ``a_scale`` multiplies A before rounding (edge-case inputs with large
    |Gate|); the default reproduces the benchmark recipe exactly.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    A = torch.randn(M, K, dtype=torch.float32, generator=g)
    if a_scale != 1.0:
        A = A * a_scale
    A = A.to(torch.bfloat16)
    root_k = math.sqrt(K) if K > 0 else 1.0
    W1 = (torch.randn(K, N, dtype=torch.float32, generator=g) / root_k).to(torch.bfloat16)
    W2 = (torch.randn(K, N, dtype=torch.float32, generator=g) / root_k).to(torch.bfloat16)
    return A, W1, W2


def make_mlp_inputs(M: int, K: int, N: int, seed: int):
    """A, W1, W2 exactly as make_inputs(M, K, N, seed), then the down
    projection's weight W3 [N, K] drawn next from the same generator:
    float32 standard normals divided by sqrt(N) (its fan-in), rounded to
    bf16.  So W3 ~ N(0, 1/N) and every output of the block has the variance
    of one SwiGLU output (about 0.35)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    A = torch.randn(M, K, dtype=torch.float32, generator=g).to(torch.bfloat16)
    root_k = math.sqrt(K) if K > 0 else 1.0
    W1 = (torch.randn(K, N, dtype=torch.float32, generator=g) / root_k).to(torch.bfloat16)
    W2 = (torch.randn(K, N, dtype=torch.float32, generator=g) / root_k).to(torch.bfloat16)
    root_n = math.sqrt(N) if N > 0 else 1.0
    W3 = (torch.randn(N, K, dtype=torch.float32, generator=g) / root_n).to(torch.bfloat16)
    return A, W1, W2, W3


def device_inputs(M: int, K: int, N: int, seed: int, device):
    """The recipe of make_inputs drawn by a seeded generator on `device`
    (A [M,K], W1 [K,N], W2 [K,N], bf16, in that order): for operands of
    several GiB, which the CPU generator would take minutes to draw.  The
    numbers differ from make_inputs' for the same seed (another generator);
    the oracle gets the drawn values copied to the host."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    A = torch.randn(M, K, dtype=torch.float32, device=device, generator=g).to(torch.bfloat16)
    root_k = math.sqrt(K) if K > 0 else 1.0
    W1 = (torch.randn(K, N, dtype=torch.float32, device=device, generator=g) / root_k).to(
        torch.bfloat16)
    W2 = (torch.randn(K, N, dtype=torch.float32, device=device, generator=g) / root_k).to(
        torch.bfloat16)
    return A, W1, W2


def workload_inputs(w: Workload):
    return make_inputs(w.M, w.K, w.N, w.seed)


def random_bf16(shape, seed: int, scale: float = 1.0) -> torch.Tensor:
    """Standard normals times ``scale``, rounded to bf16 (CPU)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return (torch.randn(*shape, dtype=torch.float32, generator=g) * scale).to(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (CPU) -> numpy uint16 array of its bit patterns (no copy of values)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> CPU bf16 tensor."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
