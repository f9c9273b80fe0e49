"""Seeded synthetic operands in Llama-3-8B linear-layer shapes.

This module draws random bf16 tensors and nothing else: it holds none of the
quantizer's or the GEMM's arithmetic, so the GPU path and the CPU oracle can
both take their inputs from it.  Every tensor comes from its own torch CPU
``Generator`` (seed = 1000 * config_seed + tensor_index), is sampled in fp32
and rounded once to bf16 (round-to-nearest-even, torch's ``.to``).

Distributions (the workload the pages measure is Llama-3 8B pretraining;
these stand in for its activations, weights and gradients):
  activation  N(0, 1) with i.i.d. Bernoulli(0.001) entries multiplied by 50
  weight      N(0, 0.02^2)
  swiglu      |z1| * z2 with z1, z2 ~ N(0, 1)   (SiLU-product-like)
  grad        1e-3 * t(3): z / sqrt(chi2_3 / 3) with z, chi2_3 from normals
"""
from __future__ import annotations

import numpy as np
import torch

OUTLIER_P = 0.001
OUTLIER_MUL = 50.0
WEIGHT_STD = 0.02
GRAD_SCALE = 1e-3


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def activation(rows: int, cols: int, seed: int) -> torch.Tensor:
    g = _gen(seed)
    z = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    mask = torch.rand(rows, cols, generator=g, dtype=torch.float32) < OUTLIER_P
    z = torch.where(mask, z * OUTLIER_MUL, z)
    return z.to(torch.bfloat16)


def weight(rows: int, cols: int, seed: int) -> torch.Tensor:
    g = _gen(seed)
    return (torch.randn(rows, cols, generator=g, dtype=torch.float32) * WEIGHT_STD).to(torch.bfloat16)


def swiglu_like(rows: int, cols: int, seed: int) -> torch.Tensor:
    g = _gen(seed)
    z1 = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    z2 = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    return (z1.abs() * z2).to(torch.bfloat16)


def grad_student_t3(rows: int, cols: int, seed: int) -> torch.Tensor:
    g = _gen(seed)
    z = torch.randn(rows, cols, generator=g, dtype=torch.float32)
    chi2 = torch.zeros(rows, cols, dtype=torch.float32)
    for _ in range(3):
        chi2 += torch.randn(rows, cols, generator=g, dtype=torch.float32) ** 2
    t = z / torch.sqrt(chi2 / 3.0)
    return (t * GRAD_SCALE).to(torch.bfloat16)


def sign_mask(seed: int) -> int:
    """A fixed 32-bit sign pattern for the Hadamard-32 (bit i set -> d_i = -1)."""
    g = _gen(seed)
    return int(torch.randint(0, 2**32, (1,), generator=g, dtype=torch.int64).item())


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 array of the same bits (no arithmetic)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bf16_bits(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 tensor with the same bits."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)


# The five workloads: (name, tensors).  Each tensor is (role, maker, rows, cols,
# index); the seed of tensor i of config c is 1000 * 0 + i (config seed 0).
SR_SEED = 7
HADAMARD_MASK_SEED = 7

CONFIGS = {
    "tiny": dict(desc="MXFP4 quantize + GEMM 256x256x256, RNE",
                 A=("activation", 256, 256, 0), B=("weight", 256, 256, 1)),
    "qkv": dict(desc="Llama-3-8B QKV forward, MXFP4 RNE, GEMM 8192x6144x4096",
                X=("activation", 8192, 4096, 0), W=("weight", 6144, 4096, 1)),
    "mlp_gate_up": dict(desc="Llama-3-8B MLP gate/up, MXFP4 RNE, GEMM 8192x28672x4096",
                        X=("activation", 8192, 4096, 0), W=("weight", 28672, 4096, 1)),
    "mlp_down": dict(desc="Llama-3-8B MLP down, MXFP4 RNE, GEMM 8192x4096x14336",
                     H=("swiglu_like", 8192, 14336, 2), W=("weight", 4096, 14336, 3)),
    "backward": dict(desc="Llama-3-8B o_proj backward, MXFP4, SR on dY, Hadamard-32 on wgrad",
                     dY=("grad_student_t3", 8192, 4096, 0), W=("weight", 4096, 4096, 1),
                     X=("activation", 8192, 4096, 2)),
    "nvfp4": dict(desc="NVFP4 global and per-128x128-tile domains, GEMM 8192x14336x4096",
                  X=("activation", 8192, 4096, 0), W=("weight", 14336, 4096, 1)),
}

_MAKERS = {"activation": activation, "weight": weight, "swiglu_like": swiglu_like,
           "grad_student_t3": grad_student_t3}


def make(kind: str, rows: int, cols: int, index: int, config_seed: int = 0) -> torch.Tensor:
    return _MAKERS[kind](rows, cols, 1000 * config_seed + index)


def config_tensor(config: str, role: str, rows: int | None = None) -> torch.Tensor:
    """Tensor ``role`` of ``config``; ``rows`` optionally truncates the row count
    (the leading rows of the full tensor are NOT reproduced -- a smaller
    generator call is made -- so use it only for shape-reduced test cases)."""
    kind, r, c, idx = CONFIGS[config][role]
    return make(kind, r if rows is None else rows, c, idx)
