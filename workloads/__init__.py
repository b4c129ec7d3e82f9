"""Seeded synthetic inputs and workload shapes.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It holds no part of the method's arithmetic: it only draws seeded
random tensors (weights, activations, adapter factors, upstream gradients) and
names the shapes of the workloads. Everything it returns is plain data that is
handed, byte for byte, to both sides.

Distributions follow the workloads the pages measure: linear weights drawn from
N(0, 0.02) (standard deviation 0.02), bf16 activations from N(0, 1), LoRA A from
N(0, 1/r) and B from N(0, 0.01); the second argument of N(.,.) is read as a
standard deviation throughout.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Sequence, Tuple

import numpy as np
import torch

# Seeds: weight matrix i uses 1000 + i; activations 1; A 2; B 3; dY 4; outlier mask 5;
# optimizer state (gradient, first and second moment) 6.
SEED_X, SEED_A, SEED_B, SEED_DY, SEED_OUTLIER, SEED_OPT = 1, 2, 3, 4, 5, 6


def weight_seed(i: int) -> int:
    return 1000 + int(i)


def _gen(seed: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_f32(shape: Sequence[int], std: float, seed: int, device: str = "cpu") -> torch.Tensor:
    """fp32 tensor ~ N(0, std) drawn from a seeded torch generator on `device`."""
    return torch.randn(tuple(int(s) for s in shape), generator=_gen(seed, device),
                       dtype=torch.float32, device=device) * float(std)


def normal_bf16(shape: Sequence[int], std: float, seed: int, device: str = "cpu") -> torch.Tensor:
    """bf16 tensor: a seeded fp32 N(0, std) sample converted by torch to bfloat16."""
    return normal_f32(shape, std, seed, device).to(torch.bfloat16)


def weight_with_outliers(shape: Sequence[int], seed: int, std: float = 0.02,
                         outlier_frac: float = 0.01, outlier_scale: float = 10.0,
                         device: str = "cpu") -> torch.Tensor:
    """fp32 weights ~ N(0, std) with a seeded uniform mask of `outlier_frac`
    elements multiplied by `outlier_scale` (the quantize/dequantize workload)."""
    w = normal_f32(shape, std, seed, device)
    u = torch.rand(tuple(int(s) for s in shape), generator=_gen(SEED_OUTLIER * 1_000_003 + seed, device),
                   dtype=torch.float32, device=device)
    return torch.where(u < outlier_frac, w * outlier_scale, w)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a bf16 tensor as uint16 (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_from_bits(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


@dataclasses.dataclass(frozen=True)
class Linear:
    """One frozen NF4 linear layer: weight [n_out, k_in] (PyTorch nn.Linear layout)."""
    name: str
    n_out: int
    k_in: int
    lora_rank: int = 0  # 0: no adapter on this projection


def llama8b_layer(rank: int = 16) -> List[Linear]:
    """Llama-8B-shaped decoder layer: hidden 4096, kv 1024, intermediate 14336."""
    h, kv, ff = 4096, 1024, 14336
    return [Linear("q_proj", h, h, rank), Linear("k_proj", kv, h, rank), Linear("v_proj", kv, h, rank),
            Linear("o_proj", h, h, rank), Linear("gate_proj", ff, h, rank), Linear("up_proj", ff, h, rank),
            Linear("down_proj", h, ff, rank)]


def smollm2_stack(rank: int = 8, layers: int = 30) -> List[Linear]:
    """SmolLM2-135M-shaped stack: hidden 576, kv 192, intermediate 1536; LoRA on q and v only."""
    h, kv, ff = 576, 192, 1536
    out: List[Linear] = []
    for i in range(layers):
        out += [Linear(f"l{i}.q_proj", h, h, rank), Linear(f"l{i}.k_proj", kv, h, 0),
                Linear(f"l{i}.v_proj", kv, h, rank), Linear(f"l{i}.o_proj", h, h, 0),
                Linear(f"l{i}.gate_proj", ff, h, 0), Linear(f"l{i}.up_proj", ff, h, 0),
                Linear(f"l{i}.down_proj", h, ff, 0)]
    return out


def smollm2_all_matrices() -> List[Tuple[int, int]]:
    """Every NF4 matrix of SmolLM2-135M: 30 x 7 decoder linears + the tied 49152 x 576 embedding."""
    return [(l.n_out, l.k_in) for l in smollm2_stack()] + [(49152, 576)]


def quant_throughput_matrices() -> List[Tuple[int, int]]:
    """7,499,415,552 synthetic parameters as 96 x (4096 x 14336) + 111 x (4096 x 4096)."""
    return [(4096, 14336)] * 96 + [(4096, 4096)] * 111


# Workload table (sizes only). "tokens" is the GEMM M dimension.
WORKLOADS: Dict[str, dict] = {
    "single_576": dict(layers=[Linear("proj", 576, 576, 16)], tokens=512, alpha=32.0, rslora=False),
    "smollm2_stack": dict(layers=smollm2_stack(), tokens=512, alpha=16.0, rslora=False),
    "llama8b_layer": dict(layers=llama8b_layer(), tokens=4096, alpha=32.0, rslora=False),
    "down_proj_bwd": dict(layers=[Linear("down_proj", 4096, 14336, 64)], tokens=8192, alpha=16.0,
                          rslora=True, dy_std=0.01),
}


def lora_inputs(layer: Linear, tokens: int, seed_offset: int = 0, device: str = "cpu",
                dy_std: float = 1.0) -> dict:
    """Seeded activations, adapter factors and upstream gradient for one linear."""
    r = layer.lora_rank
    out = dict(
        x=normal_bf16((tokens, layer.k_in), 1.0, SEED_X + 10 * seed_offset, device),
        dy=normal_bf16((tokens, layer.n_out), dy_std, SEED_DY + 10 * seed_offset, device),
    )
    if r > 0:
        out["A"] = normal_f32((r, layer.k_in), 1.0 / r, SEED_A + 10 * seed_offset, device)
        out["B"] = normal_f32((layer.n_out, r), 0.01, SEED_B + 10 * seed_offset, device)
    return out


def adamw_state(shape: Sequence[int], seed_offset: int = 0, std: float = 1e-3, device: str = "cpu") -> dict:
    """Seeded fp32 optimizer inputs of one tensor: a gradient g ~ N(0, std), a
    first moment m ~ N(0, std) and a second moment v = (N(0, std))^2 >= 0, as
    left by earlier updates."""
    base = SEED_OPT + 10 * seed_offset
    g = normal_f32(shape, std, base * 3 + 0, device)
    m = normal_f32(shape, std, base * 3 + 1, device)
    v = normal_f32(shape, std, base * 3 + 2, device) ** 2
    return dict(g=g, m=m, v=v)
