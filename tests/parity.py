"""Comparison helpers for the GPU parity tests.

Tolerances (GEMM outputs against the fp64 oracle):
  bf16 path (bf16 operands, fp32 accumulation, bf16 output):
      relative Frobenius error <= 5e-3 and max |err| <= 2e-2 * max |ref|;
  fp32 path (fp32 operands and output, fp32 accumulation, fp32 adapter terms):
      relative Frobenius error <= 1e-5.
Packed codes, scales, nested maxima, offsets and dequantized weights: bit-exact.
"""
import numpy as np
import torch

BF16_FROB, BF16_MAXABS, F32_FROB = 5e-3, 2e-2, 1e-5


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return (t.contiguous().view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return t.numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def rel_frob(got: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, np.float64)
    d = np.asarray(got, np.float64) - ref
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(d) / den) if den > 0 else float(np.linalg.norm(d))


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert got.size > 0, f"{what}: nothing compared"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    fro = rel_frob(got, ref)
    mx = float(np.max(np.abs(got - ref)))
    scale = float(np.max(np.abs(ref)))
    if dtype == "bf16":
        assert fro <= BF16_FROB, f"{what}: rel frob {fro:.3e} > {BF16_FROB}"
        assert mx <= BF16_MAXABS * scale, f"{what}: max abs {mx:.3e} > {BF16_MAXABS} * {scale:.3e}"
    else:
        assert fro <= F32_FROB, f"{what}: rel frob {fro:.3e} > {F32_FROB}"
    return dict(rel_frob=fro, max_abs=mx, ref_max=scale)
