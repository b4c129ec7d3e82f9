"""CPU oracle for NF4 double-quantized storage and the NF4 + LoRA linear layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the benchmark's ``cpu_baseline`` leg, never by the GPU product path.

The storage and linear-layer arithmetic lives in ``nf4_oracle.c`` (plain C,
fp64 accumulation, no FMA contraction); this module builds it with gcc, loads
it with ctypes and converts numpy arrays in and out. See the C file's header
for the passages each function follows and for the readings taken where the
pages are silent.

The optimizer step after the LoRA gradients (the LoRA-FA preconditioner and
AdamW) is written here in numpy fp64, in the order of its definition; see the
section "LoRA-FA preconditioning and AdamW" below.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nf4_oracle.c")
_LIB = os.path.join(_HERE, "libnf4_oracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile the oracle library with gcc (always, when force is true)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            lib.orc_norm_ppf.restype = ctypes.c_double
            lib.orc_norm_ppf.argtypes = [ctypes.c_double]
            lib.orc_nf4_table.argtypes = [P, P]
            lib.orc_dyn8_table.argtypes = [P, P]
            lib.orc_thresholds.argtypes = [P, ctypes.c_int, P]
            lib.orc_encode_array.argtypes = [P, ctypes.c_int, P, I64, P]
            lib.orc_layout.argtypes = [I64, ctypes.c_int, P]
            lib.orc_quantize.restype = ctypes.c_int
            lib.orc_quantize.argtypes = [P, I64, ctypes.c_int, P, P, P, P, P]
            lib.orc_dequantize.argtypes = [P, I64, ctypes.c_int, P, P, P, ctypes.c_float, P, P]
            lib.orc_linear_fwd.argtypes = [P, I64, I64, P, I64, P, P, ctypes.c_int, ctypes.c_float, P, P]
            lib.orc_linear_bwd_input.argtypes = [P, I64, I64, P, I64, P, P, ctypes.c_int, ctypes.c_float, P, P]
            lib.orc_lora_grad.argtypes = [P, P, I64, I64, I64, P, P, ctypes.c_int, ctypes.c_float, P, P]
            lib.orc_set_threads.argtypes = [ctypes.c_int]
            lib.orc_get_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


# --------------------------------------------------------------------------- tables

def norm_ppf(p: float) -> float:
    return float(_load().orc_norm_ppf(float(p)))


def nf4_table(f64: bool = False) -> np.ndarray:
    t64 = np.zeros(16, np.float64)
    t32 = np.zeros(16, np.float32)
    _load().orc_nf4_table(_ptr(t64), _ptr(t32))
    return t64 if f64 else t32


def dyn8_table(f64: bool = False) -> np.ndarray:
    t64 = np.zeros(256, np.float64)
    t32 = np.zeros(256, np.float32)
    _load().orc_dyn8_table(_ptr(t64), _ptr(t32))
    return t64 if f64 else t32


def thresholds(table: np.ndarray) -> np.ndarray:
    table = _c(table, np.float32)
    thr = np.zeros(table.size - 1, np.float32)
    _load().orc_thresholds(_ptr(table), int(table.size), _ptr(thr))
    return thr


def encode(thr: np.ndarray, x: np.ndarray) -> np.ndarray:
    thr = _c(thr, np.float32)
    x = _c(x, np.float32).ravel()
    out = np.zeros(x.size, np.uint8)
    _load().orc_encode_array(_ptr(thr), int(thr.size), _ptr(x), int(x.size), _ptr(out))
    return out


# --------------------------------------------------------------------------- storage

def layout(n: int, double_quant: bool) -> Dict[str, int]:
    out = np.zeros(8, np.int64)
    _load().orc_layout(int(n), int(bool(double_quant)), _ptr(out))
    keys = ["codes", "scales", "nested", "offset", "device_bytes", "total_bytes", "nb", "nn"]
    return {k: int(v) for k, v in zip(keys, out)}


def quantize(w: np.ndarray, double_quant: bool = True) -> Dict[str, np.ndarray]:
    """Quantize a flat (or flattened row-major) fp32 weight array.

    Returns codes u8[ceil(n/2)], absmax f32[nb] and, with double quantization,
    qabs u8[nb], nested f32[nn] and offset f32[1]. Raises ValueError on
    non-finite weights."""
    w = _c(w, np.float32).ravel()
    n = w.size
    lay = layout(n, double_quant)
    codes = np.zeros(lay["codes"], np.uint8)
    absmax = np.zeros(lay["nb"], np.float32)
    qabs = np.zeros(lay["nb"] if double_quant else 0, np.uint8)
    nested = np.zeros(lay["nn"] if double_quant else 0, np.float32)
    offset = np.zeros(1 if double_quant else 0, np.float32)
    rc = _load().orc_quantize(_ptr(w), n, int(bool(double_quant)), _ptr(codes), _ptr(absmax),
                              _ptr(qabs) if double_quant else None, _ptr(nested) if double_quant else None,
                              _ptr(offset) if double_quant else None)
    if rc != 0:
        raise ValueError("non-finite weight")
    out = dict(n=n, double_quant=bool(double_quant), codes=codes, absmax=absmax)
    if double_quant:
        out.update(qabs=qabs, nested=nested, offset=offset)
    return out


def dequantize(q: Dict[str, np.ndarray], out: str = "f32") -> np.ndarray:
    """Reconstruct the weights of a packed tensor from `quantize` (or one with the
    same keys). out='f32' gives fp32 values, out='bf16' gives uint16 bf16 bits."""
    n = int(q["n"])
    dq = bool(q["double_quant"])
    codes = _c(q["codes"], np.uint8)
    absmax = _c(q["absmax"], np.float32) if not dq else None
    qabs = _c(q["qabs"], np.uint8) if dq else None
    nested = _c(q["nested"], np.float32) if dq else None
    offset = float(np.float32(q["offset"][0])) if dq else 0.0
    f = np.zeros(n, np.float32) if out == "f32" else None
    h = np.zeros(n, np.uint16) if out == "bf16" else None
    _load().orc_dequantize(_ptr(codes), n, int(dq), _ptr(absmax), _ptr(qabs), _ptr(nested),
                           ctypes.c_float(offset), _ptr(f), _ptr(h))
    return f if out == "f32" else h


def embedding_rows(q: Dict[str, np.ndarray], D: int, ids, out: str = "f32") -> np.ndarray:
    """Decoded rows ids[0..T) of a packed [V, D] embedding table.

    Aner docs "Native model adaptation and NF4", section "Packed NF4 and the
    portable QLoRA profile" (embeddings decode only the selected rows) and
    section "Fused GPU NF4 decodes inside the matrix kernel" (the selected-row
    kernel decodes codes and nested scales on the device): row i of the result
    is row ids[i] of the decoded table, so this is the full decode followed by
    a row selection. out='f32' gives fp32 values, out='bf16' uint16 bf16 bits.
    Raises IndexError for an id outside [0, V)."""
    D = int(D)
    n = int(q["n"])
    if D < 1 or n % D:
        raise ValueError("table size is not a multiple of the row width")
    V = n // D
    ids = np.asarray(ids, dtype=np.int64).ravel()
    if ids.size and (ids.min() < 0 or ids.max() >= V):
        raise IndexError("embedding id out of range")
    table = dequantize(q, out).reshape(V, D)
    return table[ids]


# --------------------------------------------------------------------------- bf16 helpers

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact: the bits become the top half)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- linear

def linear_fwd(x: np.ndarray, W: np.ndarray, A: Optional[np.ndarray] = None, B: Optional[np.ndarray] = None,
               s: float = 0.0):
    """y = x W^T + s (x A^T) B^T in fp64. x [M,K] and W [N,K] hold fp32 values
    (bf16 operands are passed as their exact fp32 values). Returns (y, T)."""
    x = _c(x, np.float32)
    W = _c(W, np.float32)
    M, K = x.shape
    N = W.shape[0]
    assert W.shape[1] == K
    r = 0 if A is None else int(A.shape[0])
    A = _c(A, np.float32) if r else None
    B = _c(B, np.float32) if r else None
    y = np.zeros((M, N), np.float64)
    T = np.zeros((M, r), np.float64)
    _load().orc_linear_fwd(_ptr(x), M, K, _ptr(W), N, _ptr(A), _ptr(B), r, ctypes.c_float(np.float32(s)),
                           _ptr(y), _ptr(T) if r else None)
    return y, T


def linear_bwd_input(dy: np.ndarray, W: np.ndarray, A: Optional[np.ndarray] = None,
                     B: Optional[np.ndarray] = None, s: float = 0.0):
    """dX = dY W + s (dY B) A in fp64. Returns (dX, U)."""
    dy = _c(dy, np.float32)
    W = _c(W, np.float32)
    M, N = dy.shape
    K = W.shape[1]
    assert W.shape[0] == N
    r = 0 if A is None else int(A.shape[0])
    A = _c(A, np.float32) if r else None
    B = _c(B, np.float32) if r else None
    dx = np.zeros((M, K), np.float64)
    U = np.zeros((M, r), np.float64)
    _load().orc_linear_bwd_input(_ptr(dy), M, N, _ptr(W), K, _ptr(A), _ptr(B), r,
                                 ctypes.c_float(np.float32(s)), _ptr(dx), _ptr(U) if r else None)
    return dx, U


def lora_down(x: np.ndarray, A: np.ndarray) -> np.ndarray:
    """T = x A^T in fp64: the rank-r projection the forward keeps for dB."""
    return np.asarray(x, np.float64) @ np.asarray(A, np.float64).T


def lora_up_grad(dy: np.ndarray, B: np.ndarray) -> np.ndarray:
    """U = dY B in fp64: the rank-r projection the backward keeps for dA."""
    return np.asarray(dy, np.float64) @ np.asarray(B, np.float64)


def lora_grad(x: np.ndarray, dy: np.ndarray, T: np.ndarray, U: Optional[np.ndarray], s: float,
              fa: bool = False):
    """dA = s U^T x (None when fa, LoRA-FA) and dB = s dY^T T, in fp64."""
    x = _c(x, np.float32)
    dy = _c(dy, np.float32)
    M, K = x.shape
    N = dy.shape[1]
    T = _c(T, np.float64)
    r = T.shape[1]
    Uc = None if fa else _c(U, np.float64)
    dA = None if fa else np.zeros((r, K), np.float64)
    dB = np.zeros((N, r), np.float64)
    _load().orc_lora_grad(_ptr(x), _ptr(dy), M, K, N, _ptr(T), _ptr(Uc), r, ctypes.c_float(np.float32(s)),
                          _ptr(dA), _ptr(dB))
    return dA, dB


def lora_scale(alpha: float, r: int, rslora: bool = False) -> np.float32:
    """Resolved adapter scale s = alpha / r (LoRA) or alpha / sqrt(r) (rsLoRA),
    formed in fp64 and rounded once to fp32."""
    return np.float32(alpha / (np.sqrt(r) if rslora else r))


# --------------------------------------------------------------------------- LoRA-FA preconditioning and AdamW
#
# Aner docs "Native model adaptation and NF4", section "LoRA FA includes
# gradient preconditioning": A is frozen (no gradient, no moments) and the
# gradient of B is replaced, before the Adam moments see it, by
#     s^-2 g_B pinv(A A^T + 1e-8 I),   s = alpha / rank,
# where the r x r matrix pinv(...) is computed once and stored with the adapter
# (the qualification record "native_training_accelerated" lists 277,440 frozen
# adapter bytes for 60 rank-2 targets of width 576: A plus a 2 x 2 fp32 matrix
# per target).
#
# The optimizer is AdamW with FP32 masters and moments (same page, sections
# "Explicit accelerated training profiles", "Mixed precision keeps stable state
# in FP32" and "Paged AdamW uses real CUDA managed memory"; the paged variant
# runs the same AdamW equations). The pages do not print those equations; they
# are taken from the published AdamW definition (Loshchilov and Hutter,
# decoupled weight decay) in the form the LibTorch optimizer uses (READING):
# the decay multiplies the parameter by (1 - lr * wd), the moments are
# bias-corrected by 1 - beta^t, and eps is added to the root of the corrected
# second moment.
#
# Everything below is fp64. Inputs given as fp32 arrays are widened exactly;
# scalar hyperparameters are taken at their fp32 values, since that is the
# precision in which a caller hands them over.

LORAFA_DAMPING = 1e-8


def _f32val(x) -> float:
    return float(np.float32(x))


def lorafa_preconditioner(A: np.ndarray) -> np.ndarray:
    """P = pinv(A A^T + 1e-8 I) in fp64 for a frozen A [r, K] (fp32 values).

    A A^T + 1e-8 I is symmetric positive definite, so its Moore-Penrose inverse
    is its inverse; the pseudo-inverse is taken with no singular-value cutoff
    (READING: the damping term already makes the matrix nonsingular, and a
    relative cutoff would silently drop the damped directions)."""
    A64 = np.asarray(A, np.float32).astype(np.float64)
    r = A64.shape[0]
    G = A64 @ A64.T + LORAFA_DAMPING * np.eye(r)
    return np.linalg.pinv(G, rcond=0.0)


def lorafa_precondition(dB: np.ndarray, P: np.ndarray, s: float) -> np.ndarray:
    """s^-2 dB P in fp64: dB [N, r] is the gradient of B, P [r, r] the stored
    preconditioner, s the resolved adapter scale (its fp32 value)."""
    s64 = _f32val(s)
    return (np.asarray(dB, np.float64) @ np.asarray(P, np.float64)) / (s64 * s64)


def adamw_step(p: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray, *, lr: float, beta1: float,
               beta2: float, eps: float, weight_decay: float, step: int, grad_scale: float = 1.0):
    """One AdamW update of parameters p with gradient g and moments m, v (all
    widened to fp64). `step` is the 1-based index t of this update. The
    gradient is first multiplied by grad_scale (a clipping or unscaling
    factor). Returns the new (p, m, v) in fp64."""
    t = int(step)
    if t < 1:
        raise ValueError("step must be >= 1")
    lr, b1, b2 = _f32val(lr), _f32val(beta1), _f32val(beta2)
    eps, wd, gs = _f32val(eps), _f32val(weight_decay), _f32val(grad_scale)
    g = np.asarray(g, np.float64) * gs
    p = np.asarray(p, np.float64) * (1.0 - lr * wd)       # decoupled weight decay
    m = b1 * np.asarray(m, np.float64) + (1.0 - b1) * g    # first moment
    v = b2 * np.asarray(v, np.float64) + (1.0 - b2) * g * g  # second moment
    m_hat = m / (1.0 - b1 ** t)
    v_hat = v / (1.0 - b2 ** t)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v


def lora_adamw_step(B, dB, mB, vB, *, A=None, dA=None, mA=None, vA=None, P=None, s=None, lr, beta1, beta2, eps,
                    weight_decay, step, grad_scale=1.0) -> dict:
    """The optimizer step of one adapter. LoRA: A and B each take an AdamW
    update with their own gradients. LoRA-FA (A is None): only B is updated,
    and with P given its gradient is first replaced by s^-2 (grad_scale dB) P.
    Returns {"B", "mB", "vB"} (and {"A", "mA", "vA"} for LoRA) in fp64."""
    hp = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay, step=step)
    out = {}
    if A is not None:
        if P is not None:
            raise ValueError("the LoRA-FA preconditioner applies only with A frozen")
        out["A"], out["mA"], out["vA"] = adamw_step(A, dA, mA, vA, grad_scale=grad_scale, **hp)
    gB = np.asarray(dB, np.float64)
    gs = grad_scale
    if P is not None:
        gB = lorafa_precondition(gB * _f32val(grad_scale), P, s)
        gs = 1.0
    out["B"], out["mB"], out["vB"] = adamw_step(B, gB, mB, vB, grad_scale=gs, **hp)
    return out
