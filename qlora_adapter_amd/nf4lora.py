"""Thin ctypes binding of libnf4lora.so (include/nf4lora.h).

Argument marshalling only: every step runs in the library's HIP kernels. PyTorch
supplies device memory and the current HIP stream. There is no fallback: if the
library is missing or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import functools
import dataclasses
import math
import os
import threading
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnf4lora.so")

NF4_F32, NF4_BF16 = 0, 1
_DT = {torch.float32: NF4_F32, torch.bfloat16: NF4_BF16}

EXPORTS = ["nf4_layout", "nf4_code_tables", "nf4_quantize", "nf4_quantize_noalloc", "nf4_quantize_noalloc_max_elements",
           "nf4_quantize_many", "nf4_quantize_many_workspace_bytes", "nf4_dequantize", "nf4_dequantize_many",
           "nf4_embedding_rows", "nf4_linear_fwd", "nf4_linear_fwd_group", "nf4_linear_fwd_group_workspace_bytes",
           "nf4_linear_bwd_input_sum", "nf4_linear_bwd_input_sum_workspace_bytes",
           "nf4_linear_bwd_input", "nf4_linear_workspace_bytes", "lora_grad", "lora_grad_workspace_bytes", "lorafa_preconditioner",
           "lorafa_preconditioner_workspace_bytes", "lora_adamw_step", "lora_adamw_step_many", "lora_adamw_step_paged",
           "nf4_add_rmsnorm", "nf4_rmsnorm_bwd", "nf4_rope", "nf4_attention_fwd", "nf4_attention_bwd", "nf4_swiglu",
           "nf4_swiglu_bwd", "nf4_cross_entropy", "nf4_add", "nf4_status_string", "nf4lora_abi_version"]

MAX_ADAPTERS_PER_CALL = 16
MAX_TENSORS_PER_CALL = 16
MAX_PROJECTIONS_PER_GROUP = 4


class NF4Error(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {code})")
        self.code = code


class _Sizes(ctypes.Structure):
    _fields_ = [("codes_bytes", ctypes.c_int64), ("scales_bytes", ctypes.c_int64),
                ("nested_bytes", ctypes.c_int64), ("offset_bytes", ctypes.c_int64),
                ("nb", ctypes.c_int64), ("nn", ctypes.c_int64),
                ("quantize_workspace_bytes", ctypes.c_int64)]


class _Tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("nested", ctypes.c_void_p),
                ("offset", ctypes.c_void_p), ("n", ctypes.c_int64), ("double_quant", ctypes.c_int32)]


class _Adamw(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int64)]


class _LoraState(ctypes.Structure):
    _fields_ = [("r", ctypes.c_int32), ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("A", ctypes.c_void_p), ("dA", ctypes.c_void_p), ("mA", ctypes.c_void_p), ("vA", ctypes.c_void_p),
                ("B", ctypes.c_void_p), ("dB", ctypes.c_void_p), ("mB", ctypes.c_void_p), ("vB", ctypes.c_void_p),
                ("precond", ctypes.c_void_p), ("s", ctypes.c_float)]


_lib = None
_lock = threading.Lock()


def load() -> ctypes.CDLL:
    """Load libnf4lora.so (built in-tree by qlora_adapter_amd.build)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m qlora_adapter_amd.build` "
                                   "(the NF4 path has no CPU fallback)")
            lib = ctypes.CDLL(LIB_PATH)
            P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
            lib.nf4_layout.argtypes = [I64, ctypes.c_int, ctypes.POINTER(_Sizes)]
            lib.nf4_code_tables.argtypes = [P, P]
            lib.nf4_quantize.argtypes = [P, I64, ctypes.c_int, ctypes.POINTER(_Tensor), P, ctypes.c_size_t, P, P]
            lib.nf4_quantize_noalloc.argtypes = [P, I64, ctypes.c_int, ctypes.POINTER(_Tensor), P, P]
            lib.nf4_quantize_noalloc_max_elements.restype = I64
            lib.nf4_quantize_noalloc_max_elements.argtypes = []
            lib.nf4_quantize_many.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(_Tensor), I32, P,
                                              ctypes.c_size_t, P, P]
            lib.nf4_quantize_many_workspace_bytes.restype = I64
            lib.nf4_quantize_many_workspace_bytes.argtypes = [ctypes.POINTER(_Tensor), I32]
            lib.nf4_dequantize.argtypes = [ctypes.POINTER(_Tensor), ctypes.c_int, P, P]
            lib.nf4_dequantize_many.argtypes = [ctypes.POINTER(_Tensor), ctypes.POINTER(ctypes.c_void_p), I32,
                                                ctypes.c_int, P]
            lib.nf4_embedding_rows.argtypes = [ctypes.POINTER(_Tensor), I64, I64, P, I64, ctypes.c_int, P, P, P]
            lib.nf4_linear_fwd.argtypes = [P, ctypes.c_int, I64, I64, ctypes.POINTER(_Tensor), I64, P, P, I32, F, P,
                                           P, P, ctypes.c_size_t, P]
            lib.nf4_linear_fwd_group.argtypes = [P, ctypes.c_int, I64, I64, I32, ctypes.POINTER(ctypes.POINTER(_Tensor)),
                                                 ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_void_p),
                                                 ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(I32),
                                                 ctypes.POINTER(F), ctypes.POINTER(ctypes.c_void_p),
                                                 ctypes.POINTER(ctypes.c_void_p), P, ctypes.c_size_t, P]
            lib.nf4_linear_fwd_group_workspace_bytes.restype = I64
            lib.nf4_linear_fwd_group_workspace_bytes.argtypes = [I64, I64, I32, ctypes.POINTER(I64), ctypes.POINTER(I32)]
            lib.nf4_linear_bwd_input_sum.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, I64, I64, I32,
                                                     ctypes.POINTER(ctypes.POINTER(_Tensor)), ctypes.POINTER(I64),
                                                     ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.POINTER(I32), ctypes.POINTER(F), P,
                                                     ctypes.POINTER(ctypes.c_void_p), P, ctypes.c_size_t, P]
            lib.nf4_linear_bwd_input_sum_workspace_bytes.restype = I64
            lib.nf4_linear_bwd_input_sum_workspace_bytes.argtypes = [I64, I64, I32, ctypes.POINTER(I64),
                                                                     ctypes.POINTER(I32), ctypes.c_int]
            lib.nf4_linear_bwd_input.argtypes = [P, ctypes.c_int, I64, I64, ctypes.POINTER(_Tensor), I64, P, P, I32,
                                                 F, P, P, P, ctypes.c_size_t, P]
            lib.nf4_linear_workspace_bytes.restype = I64
            lib.nf4_linear_workspace_bytes.argtypes = [I64, I64, I64, I32, ctypes.c_int]
            lib.lora_grad.argtypes = [P, P, ctypes.c_int, I64, I64, I64, P, P, P, P, I32, F, P, P, P,
                                      ctypes.c_size_t, P]
            lib.lora_grad_workspace_bytes.restype = I64
            lib.lora_grad_workspace_bytes.argtypes = [I64, I64, I64, I32, ctypes.c_int, ctypes.c_int]
            lib.lorafa_preconditioner_workspace_bytes.restype = I64
            lib.lorafa_preconditioner_workspace_bytes.argtypes = [I32, I64]
            lib.lorafa_preconditioner.argtypes = [P, I32, I64, P, P, ctypes.c_size_t, P]
            lib.lora_adamw_step.argtypes = [ctypes.POINTER(_Adamw), I32, I64, I64, P, P, P, P, P, P, P, P, P, F, P, P]
            lib.lora_adamw_step_many.argtypes = [ctypes.POINTER(_Adamw), ctypes.POINTER(_LoraState), I32, P, P]
            lib.lora_adamw_step_paged.argtypes = [ctypes.POINTER(_Adamw), ctypes.POINTER(_LoraState), I32, P, P,
                                                  ctypes.c_size_t, ctypes.c_size_t, P]
            C = ctypes.c_int
            lib.nf4_add_rmsnorm.argtypes = [P, P, C, I64, I64, P, F, P, P, P, P]
            lib.nf4_rmsnorm_bwd.argtypes = [P, P, P, C, I64, I64, P, P, P, P]
            lib.nf4_rope.argtypes = [P, C, I64, I32, I32, I64, ctypes.c_double, C, P]
            lib.nf4_attention_fwd.argtypes = [P, P, P, C, I64, I32, I32, I32, I64, P, P, P]
            lib.nf4_attention_bwd.argtypes = [P, P, P, P, P, P, C, I64, I32, I32, I32, I64, P, P, P, P, P]
            lib.nf4_swiglu.argtypes = [P, P, C, I64, I64, I64, P, P]
            lib.nf4_swiglu_bwd.argtypes = [P, P, P, C, I64, I64, I64, P, P, P]
            lib.nf4_cross_entropy.argtypes = [P, C, I64, I64, P, P, P, P, P, P]
            lib.nf4_add.argtypes = [P, P, P, C, I64, P, P]
            lib.nf4_status_string.restype = ctypes.c_char_p
            lib.nf4_status_string.argtypes = [ctypes.c_int]
            for fn in EXPORTS:
                getattr(lib, fn).restype = getattr(lib, fn).restype or ctypes.c_int
            lib.lora_grad_workspace_bytes.restype = I64
            lib.lorafa_preconditioner_workspace_bytes.restype = I64
            lib.nf4_quantize_noalloc_max_elements.restype = I64
            lib.nf4_quantize_many_workspace_bytes.restype = I64
            lib.nf4_status_string.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise NF4Error(fn, rc, load().nf4_status_string(rc).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _addr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _arrays(*specs) -> None:
    """Check (tensor, name, dtype, shape) specs: every dtype and exact shape
    first, then device and contiguity, so that a wrong size is reported as such
    before anything reaches the library (which sees only pointers and could not
    tell). A None tensor or a None dtype/shape is skipped."""
    for t, name, dtype, shape in specs:
        if t is None:
            continue
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    for t, name, _, _ in specs:
        if t is not None:
            _dev(t, name)


# --------------------------------------------------------------------------- layout and tables

@functools.lru_cache(maxsize=1024)
def _layout(n: int, dq: int) -> Tuple[Tuple[str, int], ...]:
    s = _Sizes()
    _check("nf4_layout", load().nf4_layout(n, dq, ctypes.byref(s)))
    return tuple((f, int(getattr(s, f))) for f, _ in _Sizes._fields_)


def layout(n: int, double_quant: bool = True) -> dict:
    return dict(_layout(int(n), int(bool(double_quant))))


def code_tables() -> Tuple[np.ndarray, np.ndarray]:
    a = np.zeros(16, np.float32)
    b = np.zeros(256, np.float32)
    _check("nf4_code_tables", load().nf4_code_tables(a.ctypes.data_as(ctypes.c_void_p),
                                                     b.ctypes.data_as(ctypes.c_void_p)))
    return a, b


def lora_scale(alpha: float, r: int, rslora: bool = False) -> float:
    """s = alpha / r (LoRA) or alpha / sqrt(r) (rsLoRA), rounded once to fp32."""
    return float(np.float32(alpha / (math.sqrt(r) if rslora else r)))


# --------------------------------------------------------------------------- packed tensor

@dataclasses.dataclass
class NF4Tensor:
    """A packed NF4 matrix on the device: codes, scales (fp32 absmax or u8 qabs),
    nested fp32 maxima and the fp32 offset (double quantization)."""
    codes: torch.Tensor
    scales: torch.Tensor
    nested: Optional[torch.Tensor]
    offset: Optional[torch.Tensor]
    shape: Tuple[int, ...]
    double_quant: bool

    @property
    def n(self) -> int:
        return int(np.prod(self.shape))

    @property
    def device(self) -> torch.device:
        return self.codes.device

    def nbytes(self, with_offset: bool = True) -> int:
        b = self.codes.numel() + self.scales.numel() * self.scales.element_size()
        if self.double_quant:
            b += self.nested.numel() * 4 + (4 if with_offset else 0)
        return b

    def c_struct(self) -> _Tensor:
        return _Tensor(self.codes.data_ptr(), self.scales.data_ptr(),
                       self.nested.data_ptr() if self.double_quant else None,
                       self.offset.data_ptr() if self.double_quant else None,
                       self.n, int(self.double_quant))

    @staticmethod
    def empty(shape, double_quant: bool = True, device="cuda") -> "NF4Tensor":
        n = int(np.prod(shape))
        lay = layout(n, double_quant)
        codes = torch.empty(lay["codes_bytes"], dtype=torch.uint8, device=device)
        if double_quant:
            scales = torch.empty(lay["nb"], dtype=torch.uint8, device=device)
            nested = torch.empty(lay["nn"], dtype=torch.float32, device=device)
            offset = torch.empty(1, dtype=torch.float32, device=device)
        else:
            scales = torch.empty(lay["nb"], dtype=torch.float32, device=device)
            nested = offset = None
        return NF4Tensor(codes, scales, nested, offset, tuple(int(s) for s in shape), double_quant)


# --------------------------------------------------------------------------- operations

def quantize(w: torch.Tensor, double_quant: bool = True, out: Optional[NF4Tensor] = None,
             workspace: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None) -> NF4Tensor:
    """Pack an fp32 device tensor (flattened row-major) into NF4."""
    _dev(w, "w", torch.float32)
    n = w.numel()
    lay = layout(n, double_quant)
    if out is None:
        out = NF4Tensor.empty(tuple(w.shape), double_quant, w.device)
    need = lay["quantize_workspace_bytes"]
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=w.device)
    st = out.c_struct()
    _check("nf4_quantize", load().nf4_quantize(_ptr(w), n, int(bool(double_quant)), ctypes.byref(st),
                                               _ptr(workspace), need, _ptr(status), _stream(w.device)))
    return out


def quantize_many_workspace_bytes(outs) -> int:
    """Device workspace nf4_quantize_many needs for these packed outputs."""
    outs = list(outs)
    arr = (_Tensor * len(outs))(*[o.c_struct() for o in outs])
    v = int(load().nf4_quantize_many_workspace_bytes(arr, len(outs)))
    if v < 0:
        _check("nf4_quantize_many_workspace_bytes", v)
    return v


def quantize_many(ws, double_quant=True, outs=None, workspace: Optional[torch.Tensor] = None,
                  status: Optional[torch.Tensor] = None):
    """Pack up to 16 fp32 device tensors in one nf4_quantize_many call (three
    launches for all of them); double_quant is one flag or one per tensor.
    Returns the packed tensors; each equals a separate quantize() bit for bit."""
    ws = list(ws)
    if not 1 <= len(ws) <= MAX_TENSORS_PER_CALL:
        raise ValueError(f"quantize_many takes 1 to {MAX_TENSORS_PER_CALL} tensors, got {len(ws)}")
    dqs = list(double_quant) if isinstance(double_quant, (list, tuple)) else [double_quant] * len(ws)
    if len(dqs) != len(ws):
        raise ValueError("one double_quant flag per tensor")
    for i, w in enumerate(ws):
        _dev(w, f"ws[{i}]", torch.float32)
    if outs is None:
        outs = [NF4Tensor.empty(tuple(w.shape), bool(dq), w.device) for w, dq in zip(ws, dqs)]
    outs = list(outs)
    if len(outs) != len(ws):
        raise ValueError("one output per input")
    for i, (w, o) in enumerate(zip(ws, outs)):
        if o.n != w.numel() or o.double_quant != bool(dqs[i]):
            raise ValueError(f"outs[{i}] does not match ws[{i}] (size or double_quant)")
    arr = (_Tensor * len(outs))(*[o.c_struct() for o in outs])
    need = int(load().nf4_quantize_many_workspace_bytes(arr, len(outs)))
    if need < 0:
        _check("nf4_quantize_many_workspace_bytes", need)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=ws[0].device)
    ptrs = (ctypes.c_void_p * len(ws))(*[w.data_ptr() for w in ws])
    _check("nf4_quantize_many", load().nf4_quantize_many(ptrs, arr, len(ws), _ptr(workspace),
                                                         workspace.numel() * workspace.element_size(), _ptr(status),
                                                         _stream(ws[0].device)))
    return outs


def quantize_noalloc(w: torch.Tensor, out: NF4Tensor, status: Optional[torch.Tensor] = None) -> NF4Tensor:
    """nf4_quantize into a caller-allocated `out` with no workspace (the library's
    fixed device scratch): allocates nothing. Calls that overlap on one device
    race on that scratch."""
    _dev(w, "w", torch.float32)
    n = w.numel()
    if out.n != n:
        raise ValueError(f"out holds {out.n} elements, w has {n}")
    st = out.c_struct()
    _check("nf4_quantize_noalloc", load().nf4_quantize_noalloc(_ptr(w), n, int(out.double_quant), ctypes.byref(st),
                                                               _ptr(status), _stream(w.device)))
    return out


def quantize_noalloc_max_elements() -> int:
    return int(load().nf4_quantize_noalloc_max_elements())


def dequantize(t: NF4Tensor, dtype=torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.empty(t.shape, dtype=dtype, device=t.device)
    _dev(out, "out", dtype)
    st = t.c_struct()
    _check("nf4_dequantize", load().nf4_dequantize(ctypes.byref(st), _DT[dtype], _ptr(out), _stream(t.device)))
    return out



def dequantize_many(tensors, dtype=torch.bfloat16, outs=None):
    """nf4_dequantize of up to 16 packed tensors in one launch; returns the outputs."""
    tensors = list(tensors)
    if outs is None:
        outs = [torch.empty(t.shape, dtype=dtype, device=t.device) for t in tensors]
    for o in outs:
        _dev(o, "out", dtype)
    arr = (_Tensor * len(tensors))(*[t.c_struct() for t in tensors])
    ptrs = (ctypes.c_void_p * len(outs))(*[o.data_ptr() for o in outs])
    _check("nf4_dequantize_many", load().nf4_dequantize_many(arr, ptrs, len(tensors), _DT[dtype],
                                                             _stream(tensors[0].device)))
    return outs


def embedding_rows(E: NF4Tensor, ids: torch.Tensor, dtype=torch.bfloat16, out: Optional[torch.Tensor] = None,
                   status: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decoded rows ids of a packed [V, D] table: out[t] = dequantize(E)[ids[t]].
    An id outside [0, V) gives a zero row and NF4_EINVAL (-1) in `status`."""
    if len(E.shape) != 2:
        raise ValueError("the embedding table must be 2-D [V, D]")
    V, D = E.shape
    _dev(ids, "ids", torch.int64)
    T = ids.numel()
    if out is None:
        out = torch.empty((T, D), dtype=dtype, device=E.device)
    _dev(out, "out", dtype)
    st = E.c_struct()
    _check("nf4_embedding_rows", load().nf4_embedding_rows(ctypes.byref(st), V, D, _ptr(ids), T, _DT[dtype],
                                                           _ptr(out), _ptr(status), _stream(E.device)))
    return out


WS_BACKWARD, WS_NO_SIDE_OUT = 1, 2


def linear_workspace_bytes(M: int, K: int, N: int, r: int = 0, backward: bool = False, side_out: bool = True) -> int:
    """Device workspace the linear call needs for these sizes and adapter rank
    r: the bf16 split partial sums (0 for most shapes), the partial sums of a
    split side product (bf16, r > 32) and, with side_out=False (no t_out /
    u_out), room for the M x r fp32 side product itself."""
    flags = (WS_BACKWARD if backward else 0) | (0 if side_out else WS_NO_SIDE_OUT)
    v = int(load().nf4_linear_workspace_bytes(int(M), int(K), int(N), int(r), flags))
    if v < 0:
        _check("nf4_linear_workspace_bytes", v)
    return v


def _linear_ws(workspace, M, K, N, backward, dtype, device, r, side_out):
    if dtype == torch.bfloat16:
        need = linear_workspace_bytes(M, K, N, r, backward, side_out)
    else:  # fp32: neither reduction is split; only the side product itself
        need = 0 if (side_out or not r) else (M * r * 4 + 255) // 256 * 256
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    _dev(workspace, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


def _lora_rank(A, B, what):
    if (A is None) != (B is None):
        raise ValueError(f"{what}: A and B are given together or not at all")
    return 0 if A is None else int(A.shape[0])


def linear_fwd(x: torch.Tensor, W: NF4Tensor, A: Optional[torch.Tensor] = None, B: Optional[torch.Tensor] = None,
               s: float = 0.0, y: Optional[torch.Tensor] = None, t_out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None,
               want_t: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """y = x W^T + s (x A^T) B^T; returns (y, T) with T = x A^T (fp32), or None
    without an adapter or with want_t=False (T then stays in the workspace).
    `workspace` (device bytes, linear_workspace_bytes) is allocated here when
    needed and not given."""
    if x.dim() != 2 or len(W.shape) != 2:
        raise ValueError("x must be [M, K] and W [N, K]")
    M, K = x.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError(f"W is {tuple(W.shape)} but x has {K} columns")
    r = _lora_rank(A, B, "linear_fwd")
    _arrays((x, "x", None, None), (A, "A", torch.float32, (r, K) if r else None),
            (B, "B", torch.float32, (N, r) if r else None), (y, "y", x.dtype, (M, N)),
            (t_out, "t_out", torch.float32, (M, r)))
    if x.dtype not in _DT:
        raise ValueError(f"x must be bfloat16 or float32, got {x.dtype}")
    if y is None:
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if r and t_out is None and want_t:
        t_out = torch.empty((M, r), dtype=torch.float32, device=x.device)
    st = W.c_struct()
    ws, wsb = _linear_ws(workspace, M, K, N, False, x.dtype, x.device, r, t_out is not None)
    _check("nf4_linear_fwd", load().nf4_linear_fwd(_ptr(x), _DT[x.dtype], M, K, ctypes.byref(st), N, _ptr(A),
                                                   _ptr(B), r, float(s), _ptr(y), _ptr(t_out), _ptr(ws), wsb,
                                                   _stream(x.device)))
    return y, t_out


def linear_fwd_group_workspace_bytes(M: int, K: int, N: Sequence[int], r: Sequence[int]) -> int:
    """Workspace bytes of linear_fwd_group with these widths and ranks when no
    projection passes t_out (an upper bound for every such call)."""
    n = len(N)
    if n != len(r):
        raise ValueError("N and r have different lengths")
    v = int(load().nf4_linear_fwd_group_workspace_bytes(int(M), int(K), n, (ctypes.c_int64 * n)(*map(int, N)),
                                                        (ctypes.c_int32 * n)(*map(int, r))))
    if v < 0:
        _check("nf4_linear_fwd_group_workspace_bytes", v)
    return v


def linear_fwd_group(x: torch.Tensor, Ws: Sequence[NF4Tensor], As: Sequence[Optional[torch.Tensor]],
                     Bs: Sequence[Optional[torch.Tensor]], s: Sequence[float],
                     ys: Optional[Sequence[torch.Tensor]] = None,
                     t_outs: Optional[Sequence[Optional[torch.Tensor]]] = None,
                     workspace: Optional[torch.Tensor] = None) -> Tuple[List[torch.Tensor], List[Optional[torch.Tensor]]]:
    """linear_fwd for up to MAX_PROJECTIONS_PER_GROUP projections of the same
    x (e.g. q, k and v): y[i] = x W[i]^T + s[i] (x A[i]^T) B[i]^T in one call
    whose matrix products share one launch set when the shapes allow. Returns
    (ys, Ts); T[i] is allocated here for adapted projections when t_outs is
    not given."""
    n = len(Ws)
    if not 1 <= n <= MAX_PROJECTIONS_PER_GROUP or not (len(As) == len(Bs) == len(s) == n):
        raise ValueError(f"linear_fwd_group takes 1..{MAX_PROJECTIONS_PER_GROUP} projections with one A, B, s each")
    if x.dim() != 2 or x.dtype not in _DT:
        raise ValueError("x must be a bfloat16 or float32 [M, K] tensor")
    M, K = x.shape
    ys = list(ys) if ys is not None else [None] * n
    t_outs = list(t_outs) if t_outs is not None else [None] * n
    if len(ys) != n or len(t_outs) != n:
        raise ValueError("ys and t_outs need one entry per projection")
    Ns, rs = [], []
    for i, W in enumerate(Ws):
        if len(W.shape) != 2 or W.shape[1] != K:
            raise ValueError(f"W[{i}] is {tuple(W.shape)} but x has {K} columns")
        N = W.shape[0]
        r = _lora_rank(As[i], Bs[i], "linear_fwd_group")
        _arrays((As[i], f"A[{i}]", torch.float32, (r, K) if r else None),
                (Bs[i], f"B[{i}]", torch.float32, (N, r) if r else None), (ys[i], f"y[{i}]", x.dtype, (M, N)),
                (t_outs[i], f"t_out[{i}]", torch.float32, (M, r)))
        if ys[i] is None:
            ys[i] = torch.empty((M, N), dtype=x.dtype, device=x.device)
        if r and t_outs[i] is None:
            t_outs[i] = torch.empty((M, r), dtype=torch.float32, device=x.device)
        Ns.append(N)
        rs.append(r)
    _arrays((x, "x", None, None))
    if workspace is None:
        need = linear_fwd_group_workspace_bytes(M, K, Ns, rs)
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
    if workspace is not None:
        _dev(workspace, "workspace")
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sts = [W.c_struct() for W in Ws]
    VP = ctypes.c_void_p * n
    _check("nf4_linear_fwd_group",
           load().nf4_linear_fwd_group(_ptr(x), _DT[x.dtype], M, K, n,
                                       (ctypes.POINTER(_Tensor) * n)(*[ctypes.pointer(t) for t in sts]),
                                       (ctypes.c_int64 * n)(*Ns), VP(*[_addr(a) for a in As]), VP(*[_addr(b) for b in Bs]),
                                       (ctypes.c_int32 * n)(*rs), (ctypes.c_float * n)(*map(float, s)),
                                       VP(*[_addr(y) for y in ys]), VP(*[_addr(t) for t in t_outs]), _ptr(workspace), wsb,
                                       _stream(x.device)))
    return ys, t_outs


def linear_bwd_input_sum_workspace_bytes(M: int, K: int, N: Sequence[int], r: Sequence[int],
                                         dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace bytes of linear_bwd_input_sum with these widths and ranks and
    no u_outs (an upper bound for every such call)."""
    n = len(N)
    if n != len(r) or dtype not in _DT:
        raise ValueError("N and r need equal lengths and dtype bfloat16 or float32")
    v = int(load().nf4_linear_bwd_input_sum_workspace_bytes(int(M), int(K), n, (ctypes.c_int64 * n)(*map(int, N)),
                                                            (ctypes.c_int32 * n)(*map(int, r)), _DT[dtype]))
    if v < 0:
        _check("nf4_linear_bwd_input_sum_workspace_bytes", v)
    return v


def linear_bwd_input_sum(dys: Sequence[torch.Tensor], Ws: Sequence[NF4Tensor], As: Sequence[Optional[torch.Tensor]],
                         Bs: Sequence[Optional[torch.Tensor]], s: Sequence[float], dx: Optional[torch.Tensor] = None,
                         u_outs: Optional[Sequence[Optional[torch.Tensor]]] = None,
                         workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, List[Optional[torch.Tensor]]]:
    """Input gradient of one activation read by up to MAX_PROJECTIONS_PER_GROUP
    projections (e.g. q, k and v): dX = sum_i (dY[i] W[i] + s[i] (dY[i] B[i])
    A[i]). Returns (dX, Us); U[i] = dY[i] B[i] is allocated here for adapted
    projections when u_outs is not given."""
    n = len(Ws)
    if not 1 <= n <= MAX_PROJECTIONS_PER_GROUP or not (len(dys) == len(As) == len(Bs) == len(s) == n):
        raise ValueError(f"linear_bwd_input_sum takes 1..{MAX_PROJECTIONS_PER_GROUP} projections with one dY, A, B, "
                         "s each")
    dt = dys[0].dtype
    if dt not in _DT or any(d.dim() != 2 or d.dtype != dt for d in dys):
        raise ValueError("every dY must be a [M, N] tensor of one dtype, bfloat16 or float32")
    M = dys[0].shape[0]
    K = Ws[0].shape[1]
    u_outs = list(u_outs) if u_outs is not None else [None] * n
    if len(u_outs) != n:
        raise ValueError("u_outs needs one entry per projection")
    Ns, rs = [], []
    for i, W in enumerate(Ws):
        N = W.shape[0]
        if len(W.shape) != 2 or W.shape[1] != K or tuple(dys[i].shape) != (M, N):
            raise ValueError(f"W[{i}] is {tuple(W.shape)} and dY[{i}] {tuple(dys[i].shape)}; want [N, {K}] and [{M}, N]")
        r = _lora_rank(As[i], Bs[i], "linear_bwd_input_sum")
        _arrays((dys[i], f"dY[{i}]", None, None), (As[i], f"A[{i}]", torch.float32, (r, K) if r else None),
                (Bs[i], f"B[{i}]", torch.float32, (N, r) if r else None),
                (u_outs[i], f"u_out[{i}]", torch.float32, (M, r)))
        if r and u_outs[i] is None:
            u_outs[i] = torch.empty((M, r), dtype=torch.float32, device=dys[0].device)
        Ns.append(N)
        rs.append(r)
    _arrays((dx, "dx", dt, (M, K)))
    if dx is None:
        dx = torch.empty((M, K), dtype=dt, device=dys[0].device)
    if workspace is None:
        need = linear_bwd_input_sum_workspace_bytes(M, K, Ns, rs, dt)
        workspace = torch.empty(need, dtype=torch.uint8, device=dx.device) if need else None
    if workspace is not None:
        _dev(workspace, "workspace")
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sts = [W.c_struct() for W in Ws]
    VP = ctypes.c_void_p * n
    _check("nf4_linear_bwd_input_sum",
           load().nf4_linear_bwd_input_sum(VP(*[_addr(d) for d in dys]), _DT[dt], M, K, n,
                                           (ctypes.POINTER(_Tensor) * n)(*[ctypes.pointer(t) for t in sts]),
                                           (ctypes.c_int64 * n)(*Ns), VP(*[_addr(a) for a in As]),
                                           VP(*[_addr(b) for b in Bs]), (ctypes.c_int32 * n)(*rs),
                                           (ctypes.c_float * n)(*map(float, s)), _ptr(dx),
                                           VP(*[_addr(u) for u in u_outs]), _ptr(workspace), wsb, _stream(dx.device)))
    return dx, u_outs


def linear_bwd_input(dy: torch.Tensor, W: NF4Tensor, A: Optional[torch.Tensor] = None,
                     B: Optional[torch.Tensor] = None, s: float = 0.0, dx: Optional[torch.Tensor] = None,
                     u_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     want_u: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """dX = dY W + s (dY B) A; returns (dX, U) with U = dY B (fp32), or None
    without an adapter or with want_u=False. `workspace`: as for linear_fwd."""
    if dy.dim() != 2 or len(W.shape) != 2:
        raise ValueError("dy must be [M, N] and W [N, K]")
    M, N = dy.shape
    K = W.shape[1]
    if W.shape[0] != N:
        raise ValueError(f"W is {tuple(W.shape)} but dy has {N} columns")
    r = _lora_rank(A, B, "linear_bwd_input")
    _arrays((dy, "dy", None, None), (A, "A", torch.float32, (r, K) if r else None),
            (B, "B", torch.float32, (N, r) if r else None), (dx, "dx", dy.dtype, (M, K)),
            (u_out, "u_out", torch.float32, (M, r)))
    if dy.dtype not in _DT:
        raise ValueError(f"dy must be bfloat16 or float32, got {dy.dtype}")
    if dx is None:
        dx = torch.empty((M, K), dtype=dy.dtype, device=dy.device)
    if r and u_out is None and want_u:
        u_out = torch.empty((M, r), dtype=torch.float32, device=dy.device)
    st = W.c_struct()
    ws, wsb = _linear_ws(workspace, M, K, N, True, dy.dtype, dy.device, r, u_out is not None)
    _check("nf4_linear_bwd_input",
           load().nf4_linear_bwd_input(_ptr(dy), _DT[dy.dtype], M, N, ctypes.byref(st), K, _ptr(A), _ptr(B), r,
                                       float(s), _ptr(dx), _ptr(u_out), _ptr(ws), wsb, _stream(dy.device)))
    return dx, u_out


RECOMPUTE_T, RECOMPUTE_U = 1, 2


def lora_grad_workspace_bytes(M: int, K: int, N: int, r: int, fa: bool = False, recompute: int = 0) -> int:
    v = int(load().lora_grad_workspace_bytes(M, K, N, r, int(fa), int(recompute)))
    if v < 0:
        _check("lora_grad_workspace_bytes", v)
    return v


def lora_grad(x: Optional[torch.Tensor], dy: torch.Tensor, T: Optional[torch.Tensor], U: Optional[torch.Tensor],
              s: float, fa: bool = False, dA: Optional[torch.Tensor] = None, dB: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, A: Optional[torch.Tensor] = None,
              B: Optional[torch.Tensor] = None, K: Optional[int] = None) -> Tuple[Optional[torch.Tensor], torch.Tensor]:
    """dA = s U^T x ([r,K], None for LoRA-FA) and dB = s dY^T T ([N,r]).
    T (or U) may be None: it is then recomputed from x and A (or dY and B)."""
    if dy.dim() != 2:
        raise ValueError("dy must be [M, N]")
    M, N = dy.shape
    r = next((int(t.shape[1]) for t in (T, U) if t is not None), None)
    if r is None:
        r = int(A.shape[0]) if A is not None else (int(B.shape[1]) if B is not None else 0)
    if r < 1:
        raise ValueError("lora_grad: the rank comes from T, U, A or B; none was given")
    if K is None:
        K = int(x.shape[1]) if x is not None else (int(A.shape[1]) if A is not None else 1)
    need_t, need_u = T is None, (not fa) and U is None
    if (not fa or need_t) and x is None:
        raise ValueError("lora_grad: x is required for dA or to recompute T")
    if need_t and A is None:
        raise ValueError("lora_grad: A is required when T is None")
    if need_u and B is None:
        raise ValueError("lora_grad: B is required when U is None and dA is wanted")
    _arrays((dy, "dy", None, None), (x, "x", dy.dtype, (M, K)), (T, "T", torch.float32, (M, r)),
            (None if fa else U, "U", torch.float32, (M, r)), (A, "A", torch.float32, (r, K)),
            (B, "B", torch.float32, (N, r)), (None if fa else dA, "dA", torch.float32, (r, K)),
            (dB, "dB", torch.float32, (N, r)))
    if not fa and dA is None:
        dA = torch.empty((r, K), dtype=torch.float32, device=dy.device)
    if dB is None:
        dB = torch.empty((N, r), dtype=torch.float32, device=dy.device)
    recompute = (RECOMPUTE_T if need_t else 0) | (RECOMPUTE_U if need_u else 0)
    need = lora_grad_workspace_bytes(M, K, N, r, fa, recompute)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dy.device)
    _dev(workspace, "workspace")
    wsb = workspace.numel() * workspace.element_size()
    _check("lora_grad", load().lora_grad(_ptr(x), _ptr(dy), _DT[dy.dtype], M, K, N, _ptr(A if need_t else None),
                                         _ptr(B if need_u else None), _ptr(T), _ptr(None if fa else U), r, float(s),
                                         _ptr(None if fa else dA), _ptr(dB), _ptr(workspace), wsb,
                                         _stream(dy.device)))
    return (None if fa else dA), dB


# --------------------------------------------------------------------------- optimizer step

def lorafa_preconditioner_workspace_bytes(r: int, K: int) -> int:
    v = int(load().lorafa_preconditioner_workspace_bytes(int(r), int(K)))
    if v < 0:
        _check("lorafa_preconditioner_workspace_bytes", v)
    return v


def lorafa_preconditioner(A: torch.Tensor, out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """P = pinv(A A^T + 1e-8 I) ([r, r] fp32) for a frozen LoRA-FA factor A [r, K]."""
    _dev(A, "A", torch.float32)
    r, K = A.shape
    if out is None:
        out = torch.empty((r, r), dtype=torch.float32, device=A.device)
    _dev(out, "out", torch.float32)
    need = lorafa_preconditioner_workspace_bytes(r, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=A.device)
    _check("lorafa_preconditioner", load().lorafa_preconditioner(_ptr(A), r, K, _ptr(out), _ptr(workspace), need,
                                                                 _stream(A.device)))
    return out


def _host_pinned(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.is_cuda or not t.is_pinned() or not t.is_contiguous() or t.dtype != torch.float32:
        raise ValueError(f"{name} must be a contiguous pinned fp32 host tensor")
    return t


def _grad_scale(g: Optional[torch.Tensor]) -> None:
    if g is not None:
        if g.numel() != 1:
            raise ValueError(f"grad_scale must hold one element, got {g.numel()}")
        _dev(g, "grad_scale", torch.float32)


def _adapter_specs(B, dB, mB, vB, A, dA, mA, vA, precond, paged: bool) -> None:
    """Shape and dtype of every adapter tensor (moments and gradients the shape
    of their factor, P [r, r]); then device, or pinned host for paged moments."""
    if B is None or B.dim() != 2:
        raise ValueError("B must be a 2-D [N, r] tensor")
    N, r = B.shape
    if A is not None and (A.dim() != 2 or A.shape[0] != r):
        raise ValueError(f"A must be [{r}, K], got {tuple(A.shape)}")
    if A is None and any(t is not None for t in (dA, mA, vA)):
        raise ValueError("dA, mA and vA need A")
    if A is not None:
        for name, t in (("dA", dA), ("mA", mA), ("vA", vA)):
            if t is None:
                raise ValueError(f"{name} is required when A is trained")
    shpA = None if A is None else tuple(A.shape)
    specs = [(B, "B", torch.float32, (N, r)), (dB, "dB", torch.float32, (N, r)),
             (A, "A", torch.float32, shpA), (dA, "dA", torch.float32, shpA),
             (precond, "precond", torch.float32, (r, r))]
    moments = [(mB, "mB", (N, r)), (vB, "vB", (N, r)), (mA, "mA", shpA), (vA, "vA", shpA)]
    for t, name, shp in moments:
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shp):
            raise ValueError(f"{name} must be float32 of shape {shp}, got {t.dtype} {tuple(t.shape)}")
    _arrays(*specs)
    for t, name, _ in moments:
        if t is None:
            continue
        if paged:
            _host_pinned(t, name)
        else:
            _dev(t, name)


def _state(ad: dict, paged: bool = False) -> _LoraState:
    g = lambda k: ad.get(k)
    _adapter_specs(g("B"), g("dB"), g("mB"), g("vB"), g("A"), g("dA"), g("mA"), g("vA"), g("precond"), paged)
    N, r = ad["B"].shape
    K = ad["A"].shape[1] if ad.get("A") is not None else 1
    p = lambda k: None if ad.get(k) is None else ad[k].data_ptr()
    return _LoraState(r, K, N, p("A"), p("dA"), p("mA"), p("vA"), p("B"), p("dB"), p("mB"), p("vB"), p("precond"),
                      float(ad.get("s", 0.0)))


def lora_adamw_step_many(adapters, *, step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                         eps: float = 1e-8, weight_decay: float = 0.01,
                         grad_scale: Optional[torch.Tensor] = None) -> None:
    """lora_adamw_step for up to 16 adapters in one launch. Each adapter is a
    dict with B, dB, mB, vB and, for LoRA, A, dA, mA, vA; for LoRA-FA optionally
    precond and s."""
    adapters = list(adapters)
    if not adapters:
        return
    _grad_scale(grad_scale)
    arr = (_LoraState * len(adapters))(*[_state(a) for a in adapters])
    opt = _Adamw(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), int(step))
    _check("lora_adamw_step_many", load().lora_adamw_step_many(ctypes.byref(opt), arr, len(adapters),
                                                               _ptr(grad_scale), _stream(adapters[0]["B"].device)))


def lora_adamw_step_paged(adapters, *, step: int, lr: float, staging: Optional[torch.Tensor] = None,
                          page_bytes: int = 2 << 20, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                          weight_decay: float = 0.01, grad_scale: Optional[torch.Tensor] = None) -> None:
    """lora_adamw_step_many with every moment tensor in pinned host memory,
    which the update kernel reads and writes in place (one launch for all
    adapters; `staging` is accepted and unused). Synchronize the stream before
    reading the moments."""
    adapters = list(adapters)
    if not adapters:
        return
    _grad_scale(grad_scale)
    arr = (_LoraState * len(adapters))(*[_state(a, paged=True) for a in adapters])
    opt = _Adamw(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), int(step))
    _check("lora_adamw_step_paged",
           load().lora_adamw_step_paged(ctypes.byref(opt), arr, len(adapters), _ptr(grad_scale), _ptr(staging),
                                        0 if staging is None else staging.numel() * staging.element_size(),
                                        int(page_bytes),
                                        _stream(adapters[0]["B"].device)))


def lora_adamw_step(B: torch.Tensor, dB: torch.Tensor, mB: torch.Tensor, vB: torch.Tensor, *, step: int,
                    lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                    weight_decay: float = 0.01, A: Optional[torch.Tensor] = None, dA: Optional[torch.Tensor] = None,
                    mA: Optional[torch.Tensor] = None, vA: Optional[torch.Tensor] = None,
                    precond: Optional[torch.Tensor] = None, s: float = 0.0,
                    grad_scale: Optional[torch.Tensor] = None) -> None:
    """One in-place AdamW update of an adapter: A and B (LoRA) or B alone
    (LoRA-FA: A, dA, mA, vA None), with B's gradient replaced by s^-2 dB P when
    `precond` P is given. `grad_scale` is an optional one-element fp32 device
    tensor that multiplies every gradient first."""
    if grad_scale is not None and grad_scale.numel() != 1:
        raise ValueError(f"grad_scale must hold one element, got {grad_scale.numel()}")
    _adapter_specs(B, dB, mB, vB, A, dA, mA, vA, precond, paged=False)
    N, r = B.shape
    K = 1 if A is None else A.shape[1]
    _grad_scale(grad_scale)
    opt = _Adamw(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), int(step))
    _check("lora_adamw_step", load().lora_adamw_step(ctypes.byref(opt), r, K, N, _ptr(A), _ptr(dA), _ptr(mA),
                                                     _ptr(vA), _ptr(B), _ptr(dB), _ptr(mB), _ptr(vB),
                                                     _ptr(precond), float(s), _ptr(grad_scale),
                                                     _stream(B.device)))


# --------------------------------------------------------------------------- decoder-layer operations

def add_rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float, res: Optional[torch.Tensor] = None,
                sum_out: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                rstd: Optional[torch.Tensor] = None):
    """(sum, y, rstd): sum = x + res (None without res), y = RMSNorm(sum or x) * gamma."""
    _dev(x, "x")
    _dev(gamma, "gamma", torch.float32)
    rows, width = x.shape
    if res is not None:
        _dev(res, "res", x.dtype)
        if sum_out is None:
            sum_out = torch.empty_like(x)
    if y is None:
        y = torch.empty_like(x)
    if rstd is None:
        rstd = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check("nf4_add_rmsnorm", load().nf4_add_rmsnorm(_ptr(x), _ptr(res), _DT[x.dtype], rows, width, _ptr(gamma),
                                                     float(eps), _ptr(sum_out), _ptr(y), _ptr(rstd),
                                                     _stream(x.device)))
    return sum_out, y, rstd


def rmsnorm_bwd(dy: torch.Tensor, x: torch.Tensor, rstd: torch.Tensor, gamma: torch.Tensor,
                dres: Optional[torch.Tensor] = None, dx: Optional[torch.Tensor] = None) -> torch.Tensor:
    _dev(dy, "dy")
    rows, width = dy.shape
    if dx is None:
        dx = torch.empty_like(dy)
    _check("nf4_rmsnorm_bwd", load().nf4_rmsnorm_bwd(_ptr(dy), _ptr(x), _ptr(rstd), _DT[dy.dtype], rows, width,
                                                     _ptr(gamma), _ptr(dres), _ptr(dx), _stream(dy.device)))
    return dx


def _rows(t: torch.Tensor, name: str, width: int) -> int:
    """Row stride (elements) of a 2-D activation whose rows hold `width`
    contiguous entries: a dense array or a column block of a wider one."""
    if t.dim() != 2 or t.shape[1] != width or (t.shape[0] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be [rows, {width}] with contiguous rows")
    return int(t.stride(0)) if t.shape[0] > 1 else width


def _same_dtype(dtype, *named) -> None:
    for name, t in named:
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _on_device(*named) -> None:
    for name, t in named:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def rope_(x: torch.Tensor, heads: int, d: int, theta: float, inverse: bool = False) -> torch.Tensor:
    """Rotary embedding of x [S, heads*d] in place (x may be a column block of a
    wider array: its row stride is passed on)."""
    ld = _rows(x, "x", int(heads) * int(d))
    _on_device(("x", x))
    _check("nf4_rope", load().nf4_rope(_ptr(x), _DT[x.dtype], x.shape[0], int(heads), int(d), ld, float(theta),
                                       int(bool(inverse)), _stream(x.device)))
    return x


def _qkv_stride(q, k, v, hq: int, hkv: int, d: int, names=("q", "k", "v")) -> int:
    """Common row stride of q, k, v (0 when all three are dense); shapes, row
    counts and dtypes are checked here, the device by the caller."""
    lq, lk, lv = _rows(q, names[0], hq * d), _rows(k, names[1], hkv * d), _rows(v, names[2], hkv * d)
    if not (q.shape[0] == k.shape[0] == v.shape[0]):
        raise ValueError(f"{', '.join(names)} must have the same number of rows")
    _same_dtype(q.dtype, (names[1], k), (names[2], v))
    if lq == hq * d and lk == hkv * d and lv == hkv * d:
        return 0
    if not (lq == lk == lv):
        raise ValueError(f"{', '.join(names)} must be dense or share one row stride")
    return lq


def attention_fwd(q, k, v, hq: int, hkv: int, d: int, o=None, lse=None):
    """Causal GQA attention; q, k, v may be column blocks of one wider array."""
    ld = _qkv_stride(q, k, v, hq, hkv, d)
    S = q.shape[0]
    if o is None:
        o = torch.empty((S, hq * d), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((hq, S), dtype=torch.float32, device=q.device)
    _arrays((o, "o", q.dtype, (S, hq * d)), (lse, "lse", torch.float32, (hq, S)))
    _on_device(("q", q), ("k", k), ("v", v))
    _check("nf4_attention_fwd", load().nf4_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _DT[q.dtype], S, hq, hkv, d, ld,
                                                         _ptr(o), _ptr(lse), _stream(q.device)))
    return o, lse


def attention_bwd(dout, q, k, v, o, lse, hq: int, hkv: int, d: int, dq=None, dk=None, dv=None, delta=None):
    """Input gradients of attention_fwd. q, k, v and dq, dk, dv may be column
    blocks of wider arrays, all with one row stride."""
    S = q.shape[0]
    ld = _qkv_stride(q, k, v, hq, hkv, d)
    if ld and (dq is None or dk is None or dv is None):
        raise ValueError("with strided q, k, v pass dq, dk, dv of the same row stride")
    dq = torch.empty((S, hq * d), dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty((S, hkv * d), dtype=q.dtype, device=q.device) if dk is None else dk
    dv = torch.empty((S, hkv * d), dtype=q.dtype, device=q.device) if dv is None else dv
    if _qkv_stride(dq, dk, dv, hq, hkv, d, ("dq", "dk", "dv")) != ld or dq.shape[0] != S:
        raise ValueError("dq, dk, dv must have the rows, dtype and row stride of q, k, v")
    _same_dtype(q.dtype, ("dq", dq))
    if delta is None:
        delta = torch.empty((hq, S), dtype=torch.float32, device=q.device)
    _arrays((dout, "dout", q.dtype, (S, hq * d)), (o, "o", q.dtype, (S, hq * d)),
            (lse, "lse", torch.float32, (hq, S)), (delta, "delta", torch.float32, (hq, S)))
    _on_device(("q", q), ("k", k), ("v", v), ("dq", dq), ("dk", dk), ("dv", dv))
    _check("nf4_attention_bwd", load().nf4_attention_bwd(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                         _DT[q.dtype], S, hq, hkv, d, ld, _ptr(delta), _ptr(dq),
                                                         _ptr(dk), _ptr(dv), _stream(q.device)))
    return dq, dk, dv


def _gu_stride(g, u, names=("g", "u")) -> Tuple[int, int, int]:
    """(rows, width, row stride) of a SwiGLU pair, which share one shape,
    dtype and stride (the device is checked by the caller)."""
    if g.dim() != 2 or u.shape != g.shape:
        raise ValueError(f"{names[0]} and {names[1]} must be [rows, width] of one shape")
    rows, width = g.shape
    lg, lu = _rows(g, names[0], width), _rows(u, names[1], width)
    if lg != lu:
        raise ValueError(f"{names[0]} and {names[1]} must share one row stride")
    _same_dtype(g.dtype, (names[1], u))
    return rows, width, lg


def swiglu(g, u, a=None):
    """a = silu(g) * u for [rows, width] g, u (which may be column blocks of one
    wider array); a is dense."""
    rows, width, ld = _gu_stride(g, u)
    a = torch.empty((rows, width), dtype=g.dtype, device=g.device) if a is None else a
    _arrays((a, "a", g.dtype, (rows, width)))
    _on_device(("g", g), ("u", u))
    _check("nf4_swiglu", load().nf4_swiglu(_ptr(g), _ptr(u), _DT[g.dtype], rows, width, ld, _ptr(a),
                                           _stream(g.device)))
    return a


def swiglu_bwd(da, g, u, dg=None, du=None):
    """Input gradients of swiglu; dg, du take the row stride of g, u (given
    together, as column blocks with that stride, or allocated dense when g, u
    are dense)."""
    rows, width, ld = _gu_stride(g, u)
    if dg is None and du is None:
        if ld != width:
            raise ValueError("dg and du must be given when g and u are strided")
        dg, du = torch.empty_like(g), torch.empty_like(u)
    if dg is None or du is None or dg.shape != g.shape or _gu_stride(dg, du, ("dg", "du"))[2] != ld:
        raise ValueError("dg, du must have the shape and row stride of g, u")
    _same_dtype(g.dtype, ("dg", dg))
    _arrays((da, "da", g.dtype, (rows, width)))
    _on_device(("g", g), ("u", u), ("dg", dg), ("du", du))
    _check("nf4_swiglu_bwd", load().nf4_swiglu_bwd(_ptr(da), _ptr(g), _ptr(u), _DT[g.dtype], rows, width, ld,
                                                   _ptr(dg), _ptr(du), _stream(g.device)))
    return dg, du


def cross_entropy(z, target, dz=None, want_grad: bool = True, tok_loss=None, loss=None, status=None):
    """(loss [1], tok_loss [T], dz or None) for logits z [T, V] and int64 targets [T]."""
    _dev(z, "z")
    _dev(target, "target", torch.int64)
    T, V = z.shape
    tok_loss = torch.empty(T, dtype=torch.float32, device=z.device) if tok_loss is None else tok_loss
    loss = torch.empty(1, dtype=torch.float32, device=z.device) if loss is None else loss
    if want_grad and dz is None:
        dz = torch.empty_like(z)
    _check("nf4_cross_entropy", load().nf4_cross_entropy(_ptr(z), _DT[z.dtype], T, V, _ptr(target), _ptr(tok_loss),
                                                         _ptr(loss), _ptr(dz if want_grad else None), _ptr(status),
                                                         _stream(z.device)))
    return loss, tok_loss, (dz if want_grad else None)


def add(a, b, c=None, out=None):
    """out = a + b (+ c), one fp32 sum rounded once."""
    out = torch.empty_like(a) if out is None else out
    _check("nf4_add", load().nf4_add(_ptr(a), _ptr(b), _ptr(c), _DT[a.dtype], a.numel(), _ptr(out),
                                     _stream(a.device)))
    return out
