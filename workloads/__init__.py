"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws random numbers and names shapes.  It holds none of the
method's arithmetic (no quantisation, no packing, no GEMM), so both sides of a
parity test can take their inputs from here without sharing any computation.

Workloads follow the TinyLoop loop block described on the "β-Informed
Deployment Features" page (CTX-TIER section: the loop block's projections) and
the "Model" page (config() example: dim 2048, ffn_dim 8192, default_loops 8).
Weights stand in for a GPTQ artifact: W ~ N(0, 0.02) FP32, activations
X ~ N(0, 1) rounded to FP16.  Draw order for a block: Wqkv, Wout, Wup, Wdown,
then X; a gated (SwiGLU) block draws the pages' five weights in their order,
Wqkv, Wout, Wgate, Wup, Wdown, then X.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

D_MODEL = 2048
D_FFN = 8192
GROUP = 128
W_STD = 0.02


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def weight(K: int, N: int, g: torch.Generator, std: float = W_STD) -> torch.Tensor:
    """FP32 weight [K][N] (the math object of Y = X @ W), N(0, std)."""
    return torch.randn(K, N, generator=g, dtype=torch.float32) * std


def activations(M: int, K: int, g: torch.Generator) -> torch.Tensor:
    """FP16 activations [M][K], N(0, 1) rounded to FP16."""
    return torch.randn(M, K, generator=g, dtype=torch.float32).to(torch.float16)


def block_shapes(D: int = D_MODEL, F: int = D_FFN, gated: bool = False) -> dict[str, tuple[int, int]]:
    """(K, N) of the loop-block projections, in draw order."""
    if gated:
        return {"qkv": (D, 3 * D), "out": (D, D), "gate": (D, F), "up": (D, F), "down": (F, D)}
    return {"qkv": (D, 3 * D), "out": (D, D), "up": (D, F), "down": (F, D)}


@dataclass
class BlockInputs:
    D: int
    F: int
    W: dict  # name -> FP32 [K][N]
    X: torch.Tensor  # FP16 [M][D]


def block(M: int, seed: int = 0, D: int = D_MODEL, F: int = D_FFN,
          gated: bool = False) -> BlockInputs:
    g = generator(seed)
    W = {name: weight(K, N, g) for name, (K, N) in block_shapes(D, F, gated).items()}
    X = activations(M, D, g)
    return BlockInputs(D=D, F=F, W=W, X=X)


def single_gemm(M: int, K: int, N: int, seed: int = 0):
    """One weight then one activation batch, drawn from the same seed."""
    g = generator(seed)
    W = weight(K, N, g)
    X = activations(M, K, g)
    return W, X


# The five measured workloads (names used by the bench and the tests).
CONFIGS = {
    "c1_int4_gemm_m1": dict(kind="gemm", bits=4, M=1, K=2048, N=2048),
    "c2_int4_block_m1_l8": dict(kind="loop", bits=4, M=1, L=8),
    "c3_int4_block_m512_l8": dict(kind="loop", bits=4, M=512, L=8),
    "c4a_int2_block_m1_l16": dict(kind="loop", bits=2, M=1, L=16),
    "c4b_int2_block_m128_l8": dict(kind="loop", bits=2, M=128, L=8),
    "c5a_int4_block_m16_l32": dict(kind="loop", bits=4, M=16, L=32),
    "c5b_int4_down_m2048": dict(kind="gemm", bits=4, M=2048, K=8192, N=2048),
}
