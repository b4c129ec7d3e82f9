"""Comparison helpers for the GPU parity tests.

Tolerances (GEMM outputs against the fp64 oracle):
  bf16 path (bf16 operands, fp32 accumulation, bf16 output):
      relative Frobenius error <= 5e-3 and max |err| <= 2e-2 * max |ref|;
  fp32 path (fp32 operands and output, fp32 accumulation, fp32 adapter terms):
      relative Frobenius error <= 1e-5.
Packed codes, scales, nested maxima, offsets and dequantized weights: bit-exact.

AdamW step (fp32 per-entry arithmetic against the fp64 oracle, same fp32
inputs): an entrywise bound from first-order propagation of the fp32 rounding
of every operation (see adamw_bounds). LoRA-FA preconditioner (fp64 Gram and
inversion, fp32 output): the fp32 rounding of P plus (K + r) r kappa eps64 ||P||.
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


U32 = 2.0 ** -24  # unit roundoff of fp32
U64 = 2.0 ** -53


def adamw_bounds(p0, g, m0, v0, e_g, hp, step: int, safety: float = 2.0, e_state=(0.0, 0.0, 0.0)):
    """Entrywise bounds on |gpu - oracle| for p, m, v after one AdamW update
    computed with separately rounded fp32 operations.

    p0, m0, v0: the oracle's inputs; g: the exact (fp64) gradient the update
    uses; e_g: a bound on the error of the gradient the GPU forms (0 when it is
    an input used as is); e_state: bounds on how far the GPU's own p, m, v
    inputs already are from p0, m0, v0 (nonzero when both sides run a chain of
    updates each on its own state). Every fp32 operation and every host
    constant (1 - b, 1 - lr wd, lr / (1 - b1^t), 1 / sqrt(1 - b2^t)) contributes
    one rounding of its result; errors are propagated to first order."""
    f = lambda a: np.abs(np.asarray(a, np.float64))
    m0s = np.asarray(m0, np.float64)
    p0, g, m0, v0, e_g = f(p0), np.asarray(g, np.float64), f(m0), np.asarray(v0, np.float64), f(e_g)
    e_p0, e_m0, e_v0 = (f(e) for e in e_state)
    b1, b2 = float(np.float32(hp["beta1"])), float(np.float32(hp["beta2"]))
    lr, wd, eps = float(np.float32(hp["lr"])), float(np.float32(hp["weight_decay"])), float(np.float32(hp["eps"]))
    ag = np.abs(g)
    m1 = b1 * m0s + (1 - b1) * g
    v1 = b2 * v0 + (1 - b2) * g * g
    e_m = (1 - b1) * e_g + b1 * e_m0 + 4 * U32 * (b1 * m0 + (1 - b1) * ag)
    e_v = (1 - b2) * 2 * ag * e_g + b2 * e_v0 + 5 * U32 * (b2 * v0 + (1 - b2) * g * g)
    bc1, bc2 = 1 - b1 ** step, 1 - b2 ** step
    rb = 1 / np.sqrt(bc2)
    sv = np.sqrt(v1)
    with np.errstate(divide="ignore", invalid="ignore"):
        e_sqrt = np.minimum(np.where(sv > 0, e_v / (2 * sv), np.inf), np.sqrt(e_v)) + U32 * sv
    den = sv * rb + eps
    e_den = rb * e_sqrt + 4 * U32 * den
    q = np.abs(m1) / den
    e_q = e_m / den + np.abs(m1) * e_den / den ** 2 + U32 * q
    stepsz = lr / bc1
    p1 = np.abs(p0 * (1 - lr * wd)) + stepsz * q
    e_p = (1 - lr * wd) * e_p0 + 2 * U32 * p0 + stepsz * e_q + 2 * U32 * stepsz * q + U32 * p1
    return safety * e_p, safety * e_m, safety * e_v


def assert_within(got, ref, bound, what: str) -> float:
    """|got - ref| <= bound entrywise; returns the largest ratio |err| / bound."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = np.argmax(np.where(bad, err - bound, -np.inf))
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} entries outside the bound; worst at flat "
                             f"{i}: got {got.ravel()[i]!r} ref {ref.ravel()[i]!r} bound {np.ravel(bound)[i]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, 0.0)
    return float(ratio.max()) if ratio.size else 0.0
