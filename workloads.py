"""Seeded synthetic inputs for INT8 mixed-precision linear layers.

Shared by the tests, the smoke check and the benchmark; holds none of the
method's arithmetic (no quantization, no matmul), only the shapes and value
distributions of the workloads and a seeded way to draw them.

The source pages train Llama-family models on public text datasets; none is
used here.  Synthetic tensors with the layer shapes of those runs stand in:

* activations X ~ N(0, 1) with 0.5 % of the input-feature columns scaled by
  20 (outlier channels; round(0.005 * K) columns picked by a seeded
  permutation, scaled in fp32 before the cast to bf16),
* weights W ~ N(0, 0.02) (standard deviation 0.02),
* output gradients dY ~ N(0, 1e-3) (standard deviation 1e-3),

all drawn in fp32 from one ``torch.Generator`` seeded per workload, in the
fixed order (outlier columns, X, W, dY), then rounded to bf16 (nearest-even).

Workloads:

* ``single_linear``: X [256, 512], W [512, 512] (one small layer),
* ``square(n)``: M = N = K = n for n in 1024, 2048, 4096, operands ~N(0, 1),
* ``llama_1b_layers``: the seven linears of a Llama-style 1B decoder block at
  16 x 2048 = 32768 tokens ("Quantized model training", section "INT8 mixed
  precision training": Llama2-1B, batch 16, sequence 2048),
* ``llama3_8b_layers``: the linears of a Llama-3-8B block plus the LM head
  [4096 -> 128256] at 8192 tokens (the 8B shapes of the torchtune
  integration thread "Integrate INT8 mixed-precision from torchao 0.7").
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

# Layer shapes as (name, in_features K, out_features N).
LLAMA_1B_LAYERS = [
    ("q_proj", 2048, 2048),
    ("k_proj", 2048, 256),
    ("v_proj", 2048, 256),
    ("o_proj", 2048, 2048),
    ("gate_proj", 2048, 5632),
    ("up_proj", 2048, 5632),
    ("down_proj", 5632, 2048),
]
LLAMA_1B_TOKENS = 16 * 2048

LLAMA3_8B_LAYERS = [
    ("q_proj", 4096, 4096),
    ("k_proj", 4096, 1024),
    ("v_proj", 4096, 1024),
    ("o_proj", 4096, 4096),
    ("gate_proj", 4096, 14336),
    ("up_proj", 4096, 14336),
    ("down_proj", 14336, 4096),
    ("lm_head", 4096, 128256),
]
LLAMA3_8B_TOKENS = 8192

SQUARE_SIZES = (1024, 2048, 4096)


@dataclass(frozen=True)
class LinearShape:
    name: str
    M: int  # tokens
    N: int  # out_features
    K: int  # in_features


def single_linear() -> LinearShape:
    """Small single linear: X [256, 512], W [512, 512]."""
    return LinearShape("single_linear", 256, 512, 512)


def square(n: int) -> LinearShape:
    return LinearShape(f"square_{n}", n, n, n)


def llama_1b_layers():
    return [LinearShape(f"llama1b_{nm}", LLAMA_1B_TOKENS, n, k) for nm, k, n in LLAMA_1B_LAYERS]


def llama3_8b_layers():
    return [LinearShape(f"llama3_8b_{nm}", LLAMA3_8B_TOKENS, n, k)
            for nm, k, n in LLAMA3_8B_LAYERS]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, std: float, g: torch.Generator, device) -> torch.Tensor:
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def linear_inputs(shape: LinearShape, seed: int = 0, device="cpu", outliers: bool = True,
                  x_std: float = 1.0, w_std: float = 0.02, dy_std: float = 1e-3,
                  want=("X", "W", "dY")):
    """bf16 X [M,K], W [N,K], dY [M,N] for one linear layer (see module docstring).

    Tensors not named in ``want`` are still drawn (so the others do not
    depend on ``want``) but not kept.
    """
    g = _gen(seed, device)
    M, N, K = shape.M, shape.N, shape.K
    n_out = int(round(0.005 * K)) if outliers else 0
    cols = torch.randperm(K, generator=g, device=device)[:n_out]
    out = {}
    x = _randn((M, K), x_std, g, device)
    if n_out:
        x[:, cols] *= 20.0
    out["X"] = x.to(torch.bfloat16) if "X" in want else None
    del x
    w = _randn((N, K), w_std, g, device)
    out["W"] = w.to(torch.bfloat16) if "W" in want else None
    del w
    dy = _randn((M, N), dy_std, g, device)
    out["dY"] = dy.to(torch.bfloat16) if "dY" in want else None
    del dy
    return out


def gaussian_bf16(rows: int, cols: int, seed: int = 0, std: float = 1.0,
                  device="cpu") -> torch.Tensor:
    """bf16 [rows, cols] ~ N(0, std), one seeded generator."""
    g = _gen(seed, device)
    return _randn((rows, cols), std, g, device).to(torch.bfloat16)


def square_operands(n: int, layout: str, seed: int = 0, device="cpu"):
    """bf16 operands of the square GEMM sweep in their storage layouts.

    NT: A [M,K], B [N,K].  NN: A [M,K], B [K,N].  TN: A [K,M], B [K,N].
    All ~N(0,1).  (n is M = N = K.)
    """
    g = _gen(seed, device)
    a = _randn((n, n), 1.0, g, device).to(torch.bfloat16)
    b = _randn((n, n), 1.0, g, device).to(torch.bfloat16)
    return a, b


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bf16 CPU tensor (the oracle's input format)."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")
