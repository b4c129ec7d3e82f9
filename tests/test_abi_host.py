"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/nf4lora.h declares, answers the host-only queries, and
rejects bad arguments before touching a device."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nf4lora.h")


@pytest.fixture(scope="module")
def lib():
    from qlora_adapter_amd import nf4lora
    return nf4lora.load(), nf4lora


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", txt, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"nf4_quantize", "nf4_dequantize", "nf4_linear_fwd", "nf4_linear_bwd_input", "lora_grad"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", lib[1].LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\S+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(lib[0], n)


def test_abi_version(lib):
    assert lib[0].nf4lora_abi_version() == 8


def test_layout_matches_oracle(lib, orc):
    for n in [1, 2, 63, 64, 65, 331776, 4096 * 14336, 3 * 16384 + 17]:
        for dq in (False, True):
            a = lib[1].layout(n, dq)
            o = orc.layout(n, dq)
            assert a["codes_bytes"] == o["codes"] and a["scales_bytes"] == o["scales"]
            assert a["nested_bytes"] == o["nested"] and a["offset_bytes"] == o["offset"]
            assert a["nb"] == o["nb"] and a["nn"] == o["nn"]


def test_code_tables_match_oracle_bitwise(lib, orc):
    c4, d8 = lib[1].code_tables()
    np.testing.assert_array_equal(c4.view(np.uint32), orc.nf4_table().view(np.uint32))
    np.testing.assert_array_equal(d8.view(np.uint32), orc.dyn8_table().view(np.uint32))


def test_generated_tables_are_current():
    """nf4_tables.inc is what gen_tables.py produces."""
    import io
    import importlib.util
    spec = importlib.util.spec_from_file_location("gen_tables", os.path.join(ROOT, "qlora_adapter_amd", "csrc",
                                                                             "gen_tables.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    buf = io.StringIO()
    mod.main(buf)
    assert buf.getvalue() == open(os.path.join(ROOT, "qlora_adapter_amd", "csrc", "nf4_tables.inc")).read()


def test_status_strings(lib):
    for code in range(-6, 1):
        assert len(lib[0].nf4_status_string(code)) > 0


def test_argument_errors_before_device(lib):
    L, m = lib
    EINVAL, EALIGN, EUNSUP, EWS = -1, -2, -3, -6
    s = m._Sizes()
    assert L.nf4_layout(0, 1, ctypes.byref(s)) == EINVAL
    assert L.nf4_layout(10, 2, ctypes.byref(s)) == EINVAL
    assert L.nf4_layout(10, 1, None) == EINVAL
    # null weights, zero size, bad flag
    t = m._Tensor(16, 16, 16, 16, 64, 1)
    assert L.nf4_quantize(None, 64, 1, ctypes.byref(t), None, 0, None, None) == EINVAL
    assert L.nf4_quantize(16, 0, 1, ctypes.byref(t), None, 0, None, None) == EINVAL
    assert L.nf4_quantize(16, 64, 3, ctypes.byref(t), None, 0, None, None) == EINVAL
    # tensor size mismatch and double-quant flag mismatch
    t2 = m._Tensor(16, 16, 16, 16, 65, 1)
    assert L.nf4_quantize(16, 64, 1, ctypes.byref(t2), None, 0, None, None) == EINVAL
    assert L.nf4_quantize(16, 64, 0, ctypes.byref(t), None, 0, None, None) == EINVAL
    # misaligned codes pointer
    t3 = m._Tensor(17, 16, 16, 16, 64, 1)
    assert L.nf4_quantize(16, 64, 1, ctypes.byref(t3), None, 0, None, None) == EALIGN
    # missing workspace for double quantization
    assert L.nf4_quantize(16, 64, 1, ctypes.byref(t), None, 0, None, None) == EWS
    # unsupported dtype
    assert L.nf4_dequantize(ctypes.byref(t), 7, 16, None) == EUNSUP
    # linear: bad rank, missing adapter buffers, size mismatch
    w = m._Tensor(16, 16, 16, 16, 64 * 32, 1)
    assert L.nf4_linear_fwd(16, 1, 8, 64, ctypes.byref(w), 32, None, None, 4, 1.0, 16, None, None, 0, None) == EINVAL
    assert L.nf4_linear_fwd(16, 1, 8, 64, ctypes.byref(w), 32, 16, 16, 257, 1.0, 16, 16, None, 0, None) == EINVAL
    assert L.nf4_linear_fwd(16, 1, 8, 64, ctypes.byref(w), 33, None, None, 0, 0.0, 16, None, None, 0, None) == EINVAL
    assert L.nf4_linear_fwd(16, 1, 8, 64, ctypes.byref(w), 32, 16, 16, 4, float("nan"), 16, 16, None, 0,
                            None) == EINVAL
    assert L.nf4_linear_fwd(24, 1, 8, 64, ctypes.byref(w), 32, None, None, 0, 0.0, 16, None, None, 0, None) == EALIGN
    assert L.nf4_linear_fwd(16, 1, 8, 64, ctypes.byref(w), 32, None, None, 0, 0.0, 16, None, 24, 64, None) == EALIGN
    assert L.nf4_linear_bwd_input(16, 5, 8, 32, ctypes.byref(w), 64, None, None, 0, 0.0, 16, None, None, 0,
                                  None) == EUNSUP
    # split-reduction workspace: 512 tokens through a 4096 x 14336 projection need one in bf16
    assert L.nf4_linear_workspace_bytes(0, 64, 64, 0, 0) == EINVAL
    assert L.nf4_linear_workspace_bytes(8, 64, 64, 0, 4) == EINVAL    # unknown flag
    assert L.nf4_linear_workspace_bytes(8, 64, 64, 257, 0) == EINVAL
    assert L.nf4_linear_workspace_bytes(4096, 4096, 4096, 0, 0) == 0   # large problems: no split
    need = L.nf4_linear_workspace_bytes(512, 14336, 4096, 0, 0)
    assert need > 0 and need % (512 * 4096 * 4) == 0
    assert L.nf4_linear_workspace_bytes(512, 4096, 14336, 0, 1) > 0
    wd = m._Tensor(16, 16, 16, 16, 4096 * 14336, 1)
    assert L.nf4_linear_fwd(16, 1, 512, 14336, ctypes.byref(wd), 4096, None, None, 0, 0.0, 16, None, None, 0,
                            None) == EWS
    assert L.nf4_linear_fwd(16, 1, 512, 14336, ctypes.byref(wd), 4096, None, None, 0, 0.0, 16, None, 256, need - 16,
                            None) == EWS
    # lora_grad(x, dy, dt, M, K, N, A, B, t, u, r, s, dA, dB, ws, ws_bytes, stream): rank bounds, workspace
    assert L.lora_grad(16, 16, 1, 8, 64, 32, None, None, 16, 16, 0, 1.0, 16, 16, 256, 1 << 20, None) == EINVAL
    assert L.lora_grad(16, 16, 1, 8, 64, 32, None, None, 16, 16, 4, 1.0, 16, 16, None, 0, None) == EWS
    assert L.lora_grad_workspace_bytes(8, 64, 32, 0, 0, 0) == EINVAL
    assert L.lora_grad_workspace_bytes(8, 64, 32, 4, 0, 4) == EINVAL
    assert L.lora_grad_workspace_bytes(4096, 4096, 4096, 16, 0, 0) > L.lora_grad_workspace_bytes(4096, 4096, 4096,
                                                                                                  16, 1, 0)


def test_grouped_forward_arguments_before_device(lib):
    L, m = lib
    EINVAL, EALIGN, EWS = -1, -2, -6
    I64s, I32s, Fs, VPs = ctypes.c_int64 * 4, ctypes.c_int32 * 4, ctypes.c_float * 4, ctypes.c_void_p * 4
    # workspace query: the sum of each projection's own query with no side output, each rounded up to 256
    N, r = I64s(4096, 1024, 1024, 0), I32s(16, 16, 0, 0)
    want = sum((L.nf4_linear_workspace_bytes(4096, 4096, n, k, 2) + 255) // 256 * 256
               for n, k in ((4096, 16), (1024, 16), (1024, 0)))
    assert want > 0 and L.nf4_linear_fwd_group_workspace_bytes(4096, 4096, 3, N, r) == want
    assert L.nf4_linear_fwd_group_workspace_bytes(4096, 4096, 0, N, r) == EINVAL
    assert L.nf4_linear_fwd_group_workspace_bytes(4096, 4096, 5, N, r) == EINVAL
    assert L.nf4_linear_fwd_group_workspace_bytes(4096, 4096, 2, None, r) == EINVAL
    assert L.nf4_linear_fwd_group_workspace_bytes(4096, 4096, 2, N, I32s(16, 257)) == EINVAL
    assert L.nf4_linear_fwd_group_workspace_bytes(4096, 4096, 4, N, r) == EINVAL  # a zero width
    # the call: counts, NULL arrays, a part's size mismatch, alignment, and the workspace of a part without t_out
    wa, wb = m._Tensor(16, 16, 16, 16, 64 * 32, 1), m._Tensor(16, 16, 16, 16, 64 * 16, 1)
    Ws = (ctypes.POINTER(m._Tensor) * 4)(ctypes.pointer(wa), ctypes.pointer(wb))
    Ng, rg, sg = I64s(32, 16), I32s(4, 4), Fs(1.0, 1.0)
    ab, ys, ts = VPs(16, 16), VPs(16, 16), VPs(16, 16)
    G = L.nf4_linear_fwd_group
    assert G(16, 1, 8, 64, 0, Ws, Ng, ab, ab, rg, sg, ys, ts, None, 0, None) == EINVAL
    assert G(16, 1, 8, 64, 5, Ws, Ng, ab, ab, rg, sg, ys, ts, None, 0, None) == EINVAL
    assert G(16, 1, 8, 64, 2, None, Ng, ab, ab, rg, sg, ys, ts, None, 0, None) == EINVAL
    assert G(None, 1, 8, 64, 2, Ws, Ng, ab, ab, rg, sg, ys, ts, None, 0, None) == EINVAL
    assert G(16, 1, 8, 64, 2, Ws, I64s(32, 17), ab, ab, rg, sg, ys, ts, None, 0, None) == EINVAL
    assert G(16, 1, 8, 64, 2, Ws, Ng, None, None, rg, sg, ys, ts, None, 0, None) == EINVAL  # r > 0 needs A, B
    assert G(16, 1, 8, 64, 2, Ws, Ng, ab, ab, rg, Fs(1.0, float("inf")), ys, ts, None, 0, None) == EINVAL
    assert G(16, 1, 8, 64, 2, Ws, Ng, ab, ab, rg, sg, VPs(16, 24), ts, None, 0, None) == EALIGN
    assert G(16, 1, 8, 64, 2, Ws, Ng, ab, ab, rg, sg, ys, ts, 128, 1 << 20, None) == EALIGN
    assert G(16, 1, 8, 64, 2, Ws, Ng, ab, ab, rg, sg, ys, VPs(16, None), None, 0, None) == EWS


def test_summed_input_gradient_arguments_before_device(lib):
    L, m = lib
    EINVAL, EALIGN, EUNSUP, EWS = -1, -2, -3, -6
    I64s, I32s, Fs, VPs = ctypes.c_int64 * 4, ctypes.c_int32 * 4, ctypes.c_float * 4, ctypes.c_void_p * 4
    Q = L.nf4_linear_bwd_input_sum_workspace_bytes
    # the per-projection workspaces with no side output plus count - 1 outputs of M x K, each rounded up to 256
    want = sum((L.nf4_linear_workspace_bytes(4096, 4096, n, 16, 3) + 255) // 256 * 256 for n in (4096, 1024, 1024))
    assert Q(4096, 4096, 3, I64s(4096, 1024, 1024), I32s(16, 16, 16), 1) == want + 2 * 4096 * 4096 * 2
    assert Q(4096, 4096, 1, I64s(4096), I32s(0), 0) == L.nf4_linear_workspace_bytes(4096, 4096, 4096, 0, 1)
    assert Q(4096, 4096, 0, I64s(1), I32s(1), 1) == EINVAL
    assert Q(4096, 4096, 5, I64s(1), I32s(1), 1) == EINVAL
    assert Q(4096, 4096, 2, I64s(64, 64), I32s(16, 300), 1) == EINVAL
    assert Q(4096, 4096, 2, I64s(64, 64), I32s(16, 16), 9) == EUNSUP
    wa, wb = m._Tensor(16, 16, 16, 16, 64 * 32, 1), m._Tensor(16, 16, 16, 16, 64 * 16, 1)
    Ws = (ctypes.POINTER(m._Tensor) * 4)(ctypes.pointer(wa), ctypes.pointer(wb))
    Ng, rg, sg, ab, us = I64s(32, 16), I32s(4, 4), Fs(1.0, 1.0), VPs(16, 16), VPs(16, 16)
    G = L.nf4_linear_bwd_input_sum
    assert G(VPs(16, 16), 7, 8, 64, 2, Ws, Ng, ab, ab, rg, sg, 16, us, None, 0, None) == EUNSUP
    assert G(VPs(16, 16), 1, 8, 64, 0, Ws, Ng, ab, ab, rg, sg, 16, us, None, 0, None) == EINVAL
    assert G(None, 1, 8, 64, 2, Ws, Ng, ab, ab, rg, sg, 16, us, None, 0, None) == EINVAL
    assert G(VPs(16, None), 1, 8, 64, 2, Ws, Ng, ab, ab, rg, sg, 16, us, None, 0, None) == EINVAL
    assert G(VPs(16, 16), 1, 8, 64, 2, Ws, I64s(32, 15), ab, ab, rg, sg, 16, us, None, 0, None) == EINVAL
    assert G(VPs(16, 16), 1, 8, 64, 2, Ws, Ng, None, None, rg, sg, 16, us, None, 0, None) == EINVAL
    assert G(VPs(16, 16), 1, 8, 64, 2, Ws, Ng, ab, ab, rg, sg, None, us, None, 0, None) == EINVAL
    assert G(VPs(16, 24), 1, 8, 64, 2, Ws, Ng, ab, ab, rg, sg, 16, us, None, 0, None) == EALIGN
    assert G(VPs(16, 16), 1, 8, 64, 2, Ws, Ng, ab, ab, rg, sg, 24, us, None, 0, None) == EALIGN
    # too few tiles for one launch: the parts' sum needs room for the other part's output
    assert G(VPs(16, 16), 1, 8, 64, 2, Ws, Ng, ab, ab, rg, sg, 16, us, None, 0, None) == EWS


def test_optional_side_products_and_recompute(lib):
    """t_out / u_out may be NULL (the side product then lives in the workspace),
    and lora_grad recomputes T from x and A, or U from dY and B, when they are
    NULL; the required buffers and workspace are checked before any launch."""
    L, m = lib
    EINVAL, EWS = -1, -6
    M, K, N, r = 64, 576, 192, 8
    side = ((M * r * 4 + 255) // 256) * 256
    # without t_out / u_out the side product adds M r fp32 (256-byte rounded) to
    # the linear workspace (NF4_WS_NO_SIDE_OUT = 2; NF4_WS_BACKWARD = 1)
    for bwd in (0, 1):
        assert L.nf4_linear_workspace_bytes(M, K, N, r, bwd | 2) == L.nf4_linear_workspace_bytes(M, K, N, r, bwd) + side
        assert L.nf4_linear_workspace_bytes(M, K, N, r, bwd) == L.nf4_linear_workspace_bytes(M, K, N, 0, bwd)
    w = m._Tensor(16, 16, 16, 16, K * N, 1)
    # no t_out and no workspace: the side product has nowhere to go
    assert L.nf4_linear_fwd(16, 1, M, K, ctypes.byref(w), N, 16, 16, r, 1.0, 16, None, None, 0, None) == EWS
    assert L.nf4_linear_fwd(16, 1, M, K, ctypes.byref(w), N, 16, 16, r, 1.0, 16, None, 256, side - 4, None) == EWS
    assert L.nf4_linear_bwd_input(16, 1, M, N, ctypes.byref(w), K, 16, 16, r, 1.0, 16, None, None, 0, None) == EWS
    base = L.lora_grad_workspace_bytes(M, K, N, r, 0, 0)
    assert L.lora_grad_workspace_bytes(M, K, N, r, 0, 1) == base + side
    assert L.lora_grad_workspace_bytes(M, K, N, r, 0, 3) == base + 2 * side
    fa = L.lora_grad_workspace_bytes(M, K, N, r, 1, 0)
    assert L.lora_grad_workspace_bytes(M, K, N, r, 1, 3) == fa + side   # LoRA-FA never needs U
    # T NULL needs A and x; U NULL (with dA) needs B
    assert L.lora_grad(16, 16, 1, M, K, N, None, 16, None, 16, r, 1.0, 16, 16, 256, 1 << 24, None) == EINVAL
    assert L.lora_grad(None, 16, 1, M, K, N, 16, 16, None, None, r, 1.0, None, 16, 256, 1 << 24, None) == EINVAL
    assert L.lora_grad(16, 16, 1, M, K, N, 16, None, 16, None, r, 1.0, 16, 16, 256, 1 << 24, None) == EINVAL
    # LoRA-FA with T given needs neither x nor U nor the factors
    assert L.lora_grad(None, 16, 1, M, K, N, None, None, 16, None, r, 1.0, None, 16, None, 0, None) == EWS
    # recomputing needs the larger workspace
    assert L.lora_grad(16, 16, 1, M, K, N, 16, 16, None, None, r, 1.0, 16, 16, 256, base + side, None) == EWS


def test_wide_rank_side_product_workspace(lib):
    """The side product's reduction (over K forward, N backward) is split for
    ranks beyond 32, for reductions of 8192 or more, and when fewer than 4096
    token rows meet a reduction of at least 2048 (16-row workgroups would leave
    most of the chip idle): parts of at least 128 indices, about 512 workgroups of 128
    rows x 64 ranks in all. Reductions of 8192 or more (a multiple of 8) at
    ranks up to 16 (a multiple of 4) may instead take the streamed kernel:
    parts of at least 256 indices, about 512 workgroups of 128 rows. The
    workspace holds one M x r fp32 partial product per part of the larger
    plan, and lora_grad's recomputation takes the larger of its two."""
    L, _ = lib
    def wide_parts(M, I, r):
        if not (r > 32 or I >= 8192 or (-(-M // 16) < 256 and I >= 2048)):
            return 1
        tiles = -(-M // 128) * -(-r // 64)
        steps = -(-I // 32)
        ks = min(-(-512 // tiles), max(steps // 4, 1))
        kc = -(-steps // ks) * 32
        return -(-I // kc)
    def tile_parts(M, I, r):
        if not (I % 8 == 0 and r % 4 == 0 and r <= 16 and I >= 8192):
            return 1
        steps = -(-I // 64)
        ks = min(-(-512 // -(-M // 128)), max(steps // 4, 1))
        kc = -(-steps // ks) * 64
        return -(-I // kc)
    parts = lambda M, I, r: max(wide_parts(M, I, r), tile_parts(M, I, r))
    rnd = lambda b: (b + 255) // 256 * 256
    cases = ((8192, 14336, 4096, 64), (4096, 4096, 4096, 100), (512, 4096, 14336, 256), (64, 576, 192, 33),
             (512, 4096, 1024, 16), (512, 14336, 4096, 8), (4080, 4096, 4096, 32), (512, 576, 1536, 8),
             (4096, 4096, 4096, 16), (4096, 14336, 4096, 16), (4096, 4096, 14336, 16))
    for M, K, N, r in cases:
        for bwd in (0, 1):
            I = N if bwd else K
            ks = parts(M, I, r)
            extra = rnd(ks * M * r * 4) if ks > 1 else 0
            assert L.nf4_linear_workspace_bytes(M, K, N, r, bwd) == L.nf4_linear_workspace_bytes(M, K, N, 0, bwd) + extra
        side = rnd(M * r * 4)
        pt = rnd(parts(M, K, r) * M * r * 4) if parts(M, K, r) > 1 else 0
        pu = rnd(parts(M, N, r) * M * r * 4) if parts(M, N, r) > 1 else 0
        base = L.lora_grad_workspace_bytes(M, K, N, r, 0, 0)
        assert L.lora_grad_workspace_bytes(M, K, N, r, 0, 3) == base + 2 * side + max(pt, pu)
        assert L.lora_grad_workspace_bytes(M, K, N, r, 0, 1) == base + side + pt
    # the split engages where the model says it does
    assert parts(512, 4096, 16) > 1 and parts(512, 1024, 16) == 1 and parts(4096, 4096, 16) == 1
    assert parts(4096, 14336, 16) > 1 and parts(4096, 8191, 16) == 1
    assert tile_parts(4096, 14336, 16) == 16 and tile_parts(512, 14336, 8) == 56 and wide_parts(512, 14336, 8) == 112
    # 32 and below at 4096 or more tokens over a reduction under 8192: no split
    assert L.nf4_linear_workspace_bytes(8192, 14336, 4096, 32, 1) == L.nf4_linear_workspace_bytes(8192, 14336, 4096, 0, 1)


def test_strided_decoder_ops_reject_bad_arrays(lib):
    """Rotary, attention and SwiGLU accept column blocks of a wider array (one
    shared row stride) and check every shape, row count, dtype and stride on
    the host before the device check: a malformed call is a ValueError naming
    the array, a well-formed one (host tensors here) stops at the device."""
    import torch
    _, m = lib
    S, hq, hkv, d = 6, 4, 2, 16
    qkv = torch.zeros(S, (hq + 2 * hkv) * d, dtype=torch.bfloat16)
    q, k, v = qkv[:, :hq * d], qkv[:, hq * d:(hq + hkv) * d], qkv[:, (hq + hkv) * d:]
    o, lse = torch.zeros(S, hq * d, dtype=torch.bfloat16), torch.zeros(hq, S)

    def raises(fn, *a, match, **kw):
        with pytest.raises(ValueError, match=match):
            fn(*a, **kw)

    raises(m.rope_, q, hq + 1, d, 1e4, match=r"x must be \[rows, 80\]")
    raises(m.rope_, qkv[:, :hq * d], hq, d, 1e4, match="device")  # well-formed strided block
    raises(m.attention_fwd, q, k, v[:5], hq, hkv, d, match="same number of rows")
    raises(m.attention_fwd, q, k, v.contiguous(), hq, hkv, d, match="share one row stride")
    raises(m.attention_fwd, q, k.float(), v, hq, hkv, d, match="k must be torch.bfloat16")
    raises(m.attention_fwd, q, k, v, hq, hkv, d, o=torch.zeros(S, hq * d + 1, dtype=torch.bfloat16),
           match="o must have shape")
    raises(m.attention_fwd, q, k, v, hq, hkv, d, lse=torch.zeros(hq, S + 1), match="lse must have shape")
    raises(m.attention_fwd, q, k, v, hq, hkv, d, o=o, lse=lse, match="device")
    g = torch.zeros(S, 3 * hq * d, dtype=torch.bfloat16)
    dq, dk, dv = g[:, :hq * d], g[:, hq * d:(hq + hkv) * d], g[:, (hq + hkv) * d:(hq + 2 * hkv) * d]
    raises(m.attention_bwd, o, q, k, v, o, lse, hq, hkv, d, match="pass dq, dk, dv")
    raises(m.attention_bwd, o, q, k, v, o, lse, hq, hkv, d, dq=dq, dk=dk, dv=dv, match="row stride")
    raises(m.attention_bwd, o[:, 1:], q, k, v, o, lse, hq, hkv, d, dq=q, dk=k, dv=v, match="dout must have shape")
    raises(m.attention_bwd, o, q, k, v, o, lse, hq, hkv, d, dq=q, dk=k, dv=v, delta=torch.zeros(hq + 1, S),
           match="delta must have shape")
    raises(m.attention_bwd, o, q, k, v, o, lse, hq, hkv, d, dq=q, dk=k, dv=v, match="device")
    gu = torch.zeros(S, 2 * 40, dtype=torch.bfloat16)
    gg, uu = gu[:, :40], gu[:, 40:]
    raises(m.swiglu, gg, uu[:, :32], match="one shape")
    raises(m.swiglu, gg, gu.float()[:, 40:], match="u must be torch.bfloat16")
    raises(m.swiglu, gg, uu, a=torch.zeros(S, 41, dtype=torch.bfloat16), match="a must have shape")
    raises(m.swiglu, gg, uu, match="device")
    da = torch.zeros(S, 40, dtype=torch.bfloat16)
    raises(m.swiglu_bwd, da, gg, uu, match="must be given when g and u are strided")
    raises(m.swiglu_bwd, da, gg, uu, dg=gg[:, :32], du=uu[:, :32], match="shape and row stride")
    raises(m.swiglu_bwd, da[:, 1:], gg, uu, dg=gg, du=uu, match="da must have shape")
    raises(m.swiglu_bwd, da, gg, uu, dg=gg, du=uu, match="device")


def test_small_kernel_offsets_stay_32_bit(lib):
    """The small-tile kernels keep per-lane activation offsets (tile row times
    reduction length) and code offsets in 32 bits, so a reduction of 2^22 or
    more, or 4 GiB of codes, leaves the fast path: such shapes then need no
    split-reduction workspace (the general kernel has none), while the longest
    accepted reduction still splits."""
    L, _ = lib
    assert L.nf4_linear_workspace_bytes(512, (1 << 22) - 64, 128, 0, 0) > 0
    assert L.nf4_linear_workspace_bytes(512, 1 << 22, 128, 0, 0) == 0
    assert L.nf4_linear_workspace_bytes(512, 128, (1 << 22) - 64, 0, 1) > 0
    assert L.nf4_linear_workspace_bytes(512, 128, 1 << 22, 0, 1) == 0
    # the codes are read through 32-bit buffer offsets: 4 GiB of codes or more
    # (N x K / 2 >= 2^32) also leaves the fast path
    assert L.nf4_linear_workspace_bytes(512, 1 << 21, 4032, 0, 0) > 0
    assert L.nf4_linear_workspace_bytes(512, 1 << 21, 4096, 0, 0) == 0


def test_binding_rejects_bad_shapes_and_dtypes(lib):
    """The ctypes binding checks dtype and exact shape of every fp32 factor,
    side product, gradient, output and moment before calling the library (which
    sees only pointers): a wrong shape or dtype is a ValueError, never an
    out-of-bounds access. Tensors here are host tensors, so a well-formed call
    stops at the device check."""
    import torch
    _, m = lib
    M, K, N, r = 8, 64, 32, 4
    W = m.NF4Tensor(torch.zeros(K * N // 2, dtype=torch.uint8), torch.zeros(K * N // 64, dtype=torch.uint8),
                    torch.zeros(1), torch.zeros(1), (N, K), True)
    x = torch.zeros(M, K, dtype=torch.bfloat16)
    dy = torch.zeros(M, N, dtype=torch.bfloat16)
    A, B = torch.zeros(r, K), torch.zeros(N, r)
    T, U = torch.zeros(M, r), torch.zeros(M, r)

    def raises(fn, *a, match, **k):
        with pytest.raises(ValueError, match=match):
            fn(*a, **k)

    raises(m.linear_fwd, x, W, torch.zeros(r, K + 1), B, 1.0, match="A must have shape")
    raises(m.linear_fwd, x, W, A, torch.zeros(N, r + 1), 1.0, match="B must have shape")
    raises(m.linear_fwd, x, W, A.double(), B, 1.0, match="A must be torch.float32")
    raises(m.linear_fwd, x, W, A, B, 1.0, y=torch.zeros(M, N + 1, dtype=torch.bfloat16), match="y must have shape")
    raises(m.linear_fwd, x, W, A, B, 1.0, y=torch.zeros(M, N), match="y must be torch.bfloat16")
    raises(m.linear_fwd, x, W, A, B, 1.0, t_out=torch.zeros(M, r + 1), match="t_out must have shape")
    raises(m.linear_fwd, x, W, A, None, 1.0, match="A and B")
    raises(m.linear_fwd, x, W, A, B, 1.0, match="x must be a device tensor")
    raises(m.linear_bwd_input, dy, W, torch.zeros(r, K - 1), B, 1.0, match="A must have shape")
    raises(m.linear_bwd_input, dy, W, A, B.bfloat16(), 1.0, match="B must be torch.float32")
    raises(m.linear_bwd_input, dy, W, A, B, 1.0, dx=torch.zeros(M + 1, K, dtype=torch.bfloat16),
           match="dx must have shape")
    raises(m.linear_bwd_input, dy, W, A, B, 1.0, u_out=torch.zeros(M, r, dtype=torch.bfloat16),
           match="u_out must be torch.float32")
    raises(m.linear_bwd_input, dy, W, A, B, 1.0, match="dy must be a device tensor")
    raises(m.lora_grad, x, dy, torch.zeros(M + 1, r), U, 1.0, match="T must have shape")
    raises(m.lora_grad, x, dy, T, torch.zeros(M, r + 1), 1.0, match="U must have shape")
    raises(m.lora_grad, x, dy, T, U, 1.0, dA=torch.zeros(r, K + 1), match="dA must have shape")
    raises(m.lora_grad, x, dy, T, U, 1.0, dB=torch.zeros(N, r, dtype=torch.bfloat16), match="dB must be")
    raises(m.lora_grad, x, dy, None, U, 1.0, match="A is required")
    raises(m.lora_grad, x, dy, T, None, 1.0, match="B is required")
    raises(m.lora_grad, None, dy, T, U, 1.0, match="x is required")
    raises(m.lora_grad, x, dy, None, U, 1.0, A=torch.zeros(r + 1, K), match="A must have shape")
    raises(m.lora_grad, x, dy, T, U, 1.0, match="dy must be a device tensor")
    # optimizer: every gradient and moment has its factor's shape, P is [r, r]
    g = lambda *s: torch.zeros(*s)
    raises(m.lora_adamw_step, g(N, r), g(N, r + 1), g(N, r), g(N, r), step=1, lr=1e-3, match="dB must have shape")
    raises(m.lora_adamw_step, g(N, r), g(N, r), g(N - 1, r), g(N, r), step=1, lr=1e-3, match="mB must be float32")
    raises(m.lora_adamw_step, g(N, r), g(N, r), g(N, r), g(N, r), step=1, lr=1e-3, A=g(r, K), dA=g(r, K),
           mA=g(r, K), vA=g(r, K + 1), match="vA must be float32")
    raises(m.lora_adamw_step, g(N, r), g(N, r), g(N, r), g(N, r), step=1, lr=1e-3, A=g(r + 1, K), dA=g(r, K),
           mA=g(r, K), vA=g(r, K), match="A must be")
    raises(m.lora_adamw_step, g(N, r), g(N, r), g(N, r), g(N, r), step=1, lr=1e-3, precond=g(r, r + 1), s=1.0,
           match="precond must have shape")
    raises(m.lora_adamw_step, g(N, r), g(N, r), g(N, r), g(N, r), step=1, lr=1e-3, grad_scale=g(2),
           match="grad_scale must hold one element")
    raises(m.lora_adamw_step_many, [dict(B=g(N, r), dB=g(N, r), mB=g(N, r), vB=g(N, r + 2))], step=1, lr=1e-3,
           match="vB must be float32")
    raises(m.lora_adamw_step, g(N, r), g(N, r), g(N, r), g(N, r), step=1, lr=1e-3, match="B must be a device tensor")


def test_optimizer_argument_errors_before_device(lib):
    """The LoRA-FA preconditioner and the AdamW step reject bad arguments on the
    host (fake, 16-byte aligned addresses are never dereferenced)."""
    L, m = lib
    EINVAL, EALIGN, EWS = -1, -2, -6
    assert L.lorafa_preconditioner_workspace_bytes(0, 64) == EINVAL
    assert L.lorafa_preconditioner_workspace_bytes(257, 64) == EINVAL
    assert L.lorafa_preconditioner_workspace_bytes(16, 0) == EINVAL
    ws = L.lorafa_preconditioner_workspace_bytes(16, 4096)
    assert ws >= 16 * 16 * 8
    assert L.lorafa_preconditioner(None, 16, 4096, 256, 256, ws, None) == EINVAL
    assert L.lorafa_preconditioner(256, 16, 4096, None, 256, ws, None) == EINVAL
    assert L.lorafa_preconditioner(258, 16, 4096, 256, 256, ws, None) == EALIGN
    assert L.lorafa_preconditioner(256, 16, 4096, 256, None, 0, None) == EWS
    assert L.lorafa_preconditioner(256, 16, 4096, 256, 256, ws - 8, None) == EWS
    assert L.lorafa_preconditioner(256, 16, 4096, 256, 272, ws, None) == EALIGN

    def step(opt, r=16, K=64, N=32, A=(256, 256, 256, 256), Bp=(256, 256, 256, 256), P=None, s=2.0, gs=None):
        return L.lora_adamw_step(ctypes.byref(opt) if opt is not None else None, r, K, N, *A, *Bp, P, s, gs, None)

    good = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1)
    opt = m._Adamw(**good)
    assert step(None) == EINVAL
    assert step(opt, r=0) == EINVAL and step(opt, r=257) == EINVAL
    assert step(opt, K=0) == EINVAL and step(opt, N=0) == EINVAL
    for key, bad in [("lr", -1.0), ("lr", float("inf")), ("beta1", 1.0), ("beta2", -0.1), ("eps", 0.0),
                     ("eps", float("nan")), ("weight_decay", -0.5), ("step", 0)]:
        assert step(m._Adamw(**{**good, key: bad})) == EINVAL, key
    # A-side pointers all or none; B side required
    assert step(opt, A=(256, None, 256, 256)) == EINVAL
    assert step(opt, Bp=(256, 256, None, 256)) == EINVAL
    # the preconditioner needs LoRA-FA and a finite non-zero scale
    assert step(opt, P=256) == EINVAL
    assert step(opt, A=(None,) * 4, P=256, s=0.0) == EINVAL
    assert step(opt, A=(None,) * 4, P=256, s=float("inf")) == EINVAL
    # 16-byte alignment of every array
    assert step(opt, Bp=(256, 260, 256, 256)) == EALIGN
    assert step(opt, A=(None,) * 4, P=264) == EALIGN
    assert step(opt, gs=258) == EALIGN


def test_embedding_argument_errors_before_device(lib):
    L, m = lib
    EINVAL, EALIGN, EUNSUP = -1, -2, -3
    E = m._Tensor(16, 16, 16, 16, 100 * 64, 1)
    assert L.nf4_embedding_rows(ctypes.byref(E), 100, 64, 256, 10, 9, 256, None, None) == EUNSUP
    assert L.nf4_embedding_rows(ctypes.byref(E), 0, 64, 256, 10, 1, 256, None, None) == EINVAL
    assert L.nf4_embedding_rows(ctypes.byref(E), 100, 63, 256, 10, 1, 256, None, None) == EINVAL  # n != V*D
    assert L.nf4_embedding_rows(ctypes.byref(E), 100, 64, None, 10, 1, 256, None, None) == EINVAL
    assert L.nf4_embedding_rows(ctypes.byref(E), 100, 64, 256, 10, 1, None, None, None) == EINVAL
    assert L.nf4_embedding_rows(ctypes.byref(E), 100, 64, 256, -1, 1, 256, None, None) == EINVAL
    assert L.nf4_embedding_rows(ctypes.byref(E), 100, 64, 260, 10, 1, 256, None, None) == EALIGN
    assert L.nf4_embedding_rows(ctypes.byref(E), 100, 64, 256, 10, 1, 264, None, None) == EALIGN
    assert L.nf4_embedding_rows(ctypes.byref(E), 100, 64, 256, 10, 1, 256, 258, None) == EALIGN
    assert L.nf4_embedding_rows(None, 100, 64, 256, 10, 1, 256, None, None) == EINVAL


def test_many_adapter_step_argument_errors(lib):
    L, m = lib
    EINVAL, EALIGN = -1, -2
    opt = m._Adamw(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    good = dict(r=16, K=64, N=32, A=256, dA=256, mA=256, vA=256, B=256, dB=256, mB=256, vB=256, precond=None,
                s=2.0)
    arr = lambda *ds: (m._LoraState * len(ds))(*[m._LoraState(**d) for d in ds])
    assert L.lora_adamw_step_many(ctypes.byref(opt), None, 1, None, None) == EINVAL
    assert L.lora_adamw_step_many(ctypes.byref(opt), arr(good), 0, None, None) == EINVAL
    assert L.lora_adamw_step_many(ctypes.byref(opt), arr(*[good] * 17), 17, None, None) == EINVAL
    assert L.lora_adamw_step_many(None, arr(good), 1, None, None) == EINVAL
    assert L.lora_adamw_step_many(ctypes.byref(opt), arr(good, {**good, "r": 0}), 2, None, None) == EINVAL
    assert L.lora_adamw_step_many(ctypes.byref(opt), arr(good, {**good, "precond": 256}), 2, None, None) == EINVAL
    assert L.lora_adamw_step_many(ctypes.byref(opt), arr(good, {**good, "vB": 264}), 2, None, None) == EALIGN
    assert L.lora_adamw_step_many(ctypes.byref(opt), arr(good), 1, 258, None) == EALIGN


def test_dequantize_many_argument_errors(lib):
    L, m = lib
    EINVAL, EALIGN, EUNSUP = -1, -2, -3
    arr = lambda *ts: (m._Tensor * len(ts))(*ts)
    outs = lambda *ps: (ctypes.c_void_p * len(ps))(*ps)
    good = m._Tensor(16, 16, 16, 16, 100, 1)
    assert L.nf4_dequantize_many(arr(good), outs(256), 1, 9, None) == EUNSUP
    assert L.nf4_dequantize_many(None, outs(256), 1, 1, None) == EINVAL
    assert L.nf4_dequantize_many(arr(good), None, 1, 1, None) == EINVAL
    assert L.nf4_dequantize_many(arr(good), outs(256), 0, 1, None) == EINVAL
    assert L.nf4_dequantize_many(arr(*[good] * 17), outs(*[256] * 17), 17, 1, None) == EINVAL
    assert L.nf4_dequantize_many(arr(good, good), outs(256, None), 2, 1, None) == EINVAL
    assert L.nf4_dequantize_many(arr(good, m._Tensor(16, 16, 16, 16, 0, 1)), outs(256, 256), 2, 1, None) == EINVAL
    assert L.nf4_dequantize_many(arr(good, m._Tensor(17, 16, 16, 16, 64, 1)), outs(256, 256), 2, 1, None) == EALIGN
    assert L.nf4_dequantize_many(arr(good), outs(264), 1, 1, None) == EALIGN


def test_quantize_many_argument_errors(lib):
    """nf4_quantize_many sizes its workspace per tensor (maxima with double
    quantization, one fp64 partial per 16384 weights, each rounded to 256
    bytes, plus 256 for the flags) and rejects bad arguments before any
    device work."""
    L, m = lib
    EINVAL, EALIGN, EWS = -1, -2, -6
    arr = lambda *ts: (m._Tensor * len(ts))(*ts)
    ptrs = lambda *ps: (ctypes.c_void_p * len(ps))(*ps)
    good = m._Tensor(16, 16, 16, 16, 100, 1)          # nb 2, one group
    single = m._Tensor(16, 16, None, None, 5000, 0)   # no maxima in the workspace
    big = m._Tensor(16, 16, 16, 16, 16384 * 3 + 1, 1)  # nb 769 (3076 B -> 3328), 4 groups
    assert L.nf4_quantize_many_workspace_bytes(arr(good), 1) == 256 + 256 + 256
    assert L.nf4_quantize_many_workspace_bytes(arr(good, single, big), 3) == (512 + 256 + 3328 + 256) + 256
    assert L.nf4_quantize_many_workspace_bytes(None, 1) == EINVAL
    assert L.nf4_quantize_many_workspace_bytes(arr(good), 0) == EINVAL
    assert L.nf4_quantize_many_workspace_bytes(arr(*[good] * 17), 17) == EINVAL
    assert L.nf4_quantize_many_workspace_bytes(arr(m._Tensor(16, 16, 16, 16, 0, 1)), 1) == EINVAL
    need = L.nf4_quantize_many_workspace_bytes(arr(good, single), 2)
    W = ptrs(16, 32)
    assert L.nf4_quantize_many(None, arr(good, single), 2, 256, need, None, None) == EINVAL
    assert L.nf4_quantize_many(W, None, 2, 256, need, None, None) == EINVAL
    assert L.nf4_quantize_many(W, arr(good, single), 0, 256, need, None, None) == EINVAL
    assert L.nf4_quantize_many(ptrs(*[16] * 17), arr(*[good] * 17), 17, 256, 1 << 20, None, None) == EINVAL
    assert L.nf4_quantize_many(ptrs(16, None), arr(good, single), 2, 256, need, None, None) == EINVAL
    assert L.nf4_quantize_many(W, arr(good, m._Tensor(16, 16, 16, 16, 0, 1)), 2, 256, need, None, None) == EINVAL
    assert L.nf4_quantize_many(W, arr(good, m._Tensor(16, 16, None, None, 64, 1)), 2, 256, need, None, None) == EINVAL
    assert L.nf4_quantize_many(ptrs(16, 40), arr(good, single), 2, 256, need, None, None) == EALIGN
    assert L.nf4_quantize_many(W, arr(good, single), 2, 256, need, 2, None) == EALIGN      # status
    assert L.nf4_quantize_many(W, arr(good, single), 2, None, need, None, None) == EWS
    assert L.nf4_quantize_many(W, arr(good, single), 2, 256, need - 1, None, None) == EWS
    assert L.nf4_quantize_many(W, arr(good, single), 2, 264, need, None, None) == EALIGN
    with pytest.raises(ValueError):
        m.quantize_many([])


def test_paged_step_argument_errors(lib):
    L, m = lib
    EINVAL = -1
    opt = m._Adamw(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    st = (m._LoraState * 1)(m._LoraState(r=16, K=64, N=32, A=256, dA=256, mA=256, vA=256, B=256, dB=256, mB=256,
                                         vB=256, precond=None, s=2.0))
    assert L.lora_adamw_step_paged(ctypes.byref(opt), st, 1, None, 256, 8192, 4095, None) == EINVAL
    assert L.lora_adamw_step_paged(ctypes.byref(opt), st, 1, None, 256, 8192, 2048, None) == EINVAL
    assert L.lora_adamw_step_paged(ctypes.byref(opt), st, 1, None, 256, 1 << 28, 128 << 20, None) == EINVAL
    assert L.lora_adamw_step_paged(ctypes.byref(opt), st, 0, None, 256, 8192, 4096, None) == EINVAL
    # staging is not used (the kernel reads the moments in place), so any staging argument gets as far as
    # the device check (no device: NF4_EDEVICE) or, with a device, the pinned-memory check of the moments
    # (these are not host pointers: NF4_EINVAL)
    import torch
    expect = EINVAL if torch.cuda.is_available() else -4
    for staging, nbytes in ((None, 0), (264, 8192), (256, 4096)):
        assert L.lora_adamw_step_paged(ctypes.byref(opt), st, 1, None, staging, nbytes, 4096, None) == expect


def test_decoder_op_argument_errors(lib):
    L, _ = lib
    EINVAL, EALIGN, EUNSUP = -1, -2, -3
    c = ctypes.c_float
    # fused residual add + RMSNorm and its backward
    assert L.nf4_add_rmsnorm(256, None, 9, 4, 64, 256, c(1e-5), None, 256, 256, None) == EUNSUP
    assert L.nf4_add_rmsnorm(256, 256, 1, 4, 64, 256, c(1e-5), None, 256, 256, None) == EINVAL  # res without sum
    assert L.nf4_add_rmsnorm(256, None, 1, 4, 64, 256, c(-1.0), None, 256, 256, None) == EINVAL
    assert L.nf4_add_rmsnorm(256, None, 1, 0, 64, 256, c(1e-5), None, 256, 256, None) == EINVAL
    assert L.nf4_add_rmsnorm(258, None, 1, 4, 64, 256, c(1e-5), None, 256, 256, None) == EALIGN
    assert L.nf4_rmsnorm_bwd(256, 256, 256, 1, 4, 64, None, None, 256, None) == EINVAL
    assert L.nf4_rmsnorm_bwd(256, 256, 256, 1, 4, 64, 256, 264, 256, None) == EALIGN
    # rotary embedding
    assert L.nf4_rope(256, 1, 8, 2, 3, 0, ctypes.c_double(1e4), 0, None) == EINVAL  # odd head dim
    assert L.nf4_rope(256, 1, 8, 2, 64, 0, ctypes.c_double(1.0), 0, None) == EINVAL
    assert L.nf4_rope(256, 1, 8, 2, 64, 0, ctypes.c_double(1e4), 2, None) == EINVAL
    assert L.nf4_rope(260, 1, 8, 2, 64, 0, ctypes.c_double(1e4), 0, None) == EALIGN
    # row strides: at least the row width, whole 16-byte units
    assert L.nf4_rope(256, 1, 8, 2, 64, 120, ctypes.c_double(1e4), 0, None) == EINVAL  # below 2 * 64
    assert L.nf4_rope(256, 1, 8, 2, 64, 132, ctypes.c_double(1e4), 0, None) == EALIGN  # 264 bytes
    assert L.nf4_rope(256, 0, 8, 2, 64, 130, ctypes.c_double(1e4), 0, None) == EALIGN  # fp32: 520 bytes
    assert L.nf4_rope(256, 0, 8, 2, 64, 126, ctypes.c_double(1e4), 0, None) == EINVAL
    # attention: head dim a multiple of 16 up to 128, whole groups of query heads
    assert L.nf4_attention_fwd(256, 256, 256, 1, 8, 4, 2, 72, 0, 256, 256, None) == EINVAL
    assert L.nf4_attention_fwd(256, 256, 256, 1, 8, 4, 2, 144, 0, 256, 256, None) == EINVAL
    assert L.nf4_attention_fwd(256, 256, 256, 1, 8, 4, 3, 64, 0, 256, 256, None) == EINVAL
    assert L.nf4_attention_fwd(256, 256, 256, 1, 8, 4, 2, 64, 0, 256, None, None) == EINVAL
    assert L.nf4_attention_fwd(256, 264, 256, 1, 8, 4, 2, 64, 0, 256, 256, None) == EALIGN
    # a shared q/k/v row stride must hold the 4 query heads' 256 entries
    assert L.nf4_attention_fwd(256, 256, 256, 1, 8, 4, 2, 64, 200, 256, 256, None) == EINVAL
    assert L.nf4_attention_fwd(256, 256, 256, 1, 8, 4, 2, 64, 260, 256, 256, None) == EALIGN
    assert L.nf4_attention_bwd(256, 256, 256, 256, 256, 256, 1, 8, 4, 2, 64, 0, None, 256, 256, 256, None) == EINVAL
    assert L.nf4_attention_bwd(256, 256, 256, 256, 256, 256, 1, 8, 4, 2, 64, 136, 256, 256, 256, 256,
                               None) == EINVAL
    # elementwise
    assert L.nf4_add(256, 256, None, 9, 10, 256, None) == EUNSUP
    assert L.nf4_add(256, None, None, 1, 10, 256, None) == EINVAL
    assert L.nf4_add(256, 256, None, 1, 0, 256, None) == EINVAL
    assert L.nf4_add(256, 256, 258, 1, 10, 256, None) == EALIGN
    assert L.nf4_swiglu(256, 256, 1, 0, 8, 0, 256, None) == EINVAL
    assert L.nf4_swiglu(256, 256, 1, 4, 0, 0, 256, None) == EINVAL
    assert L.nf4_swiglu(256, 256, 1, 4, 16, 12, 256, None) == EINVAL  # stride below the width
    assert L.nf4_swiglu(256, 256, 1, 4, 16, 20, 256, None) == EALIGN  # 40-byte rows
    assert L.nf4_swiglu_bwd(256, 256, 256, 1, 2, 5, 0, 256, 264, None) == EALIGN
    # cross-entropy
    assert L.nf4_cross_entropy(256, 1, 4, 0, 256, 256, 256, None, None, None) == EINVAL
    assert L.nf4_cross_entropy(256, 1, 4, 10, None, 256, 256, None, None, None) == EINVAL
    assert L.nf4_cross_entropy(256, 1, 4, 10, 256, 256, 256, None, 258, None) == EALIGN


def test_quantize_noalloc_arguments_before_device(lib):
    """nf4_quantize_noalloc validates as nf4_quantize does, and a matrix whose
    double-quantization scratch exceeds the fixed device array is refused with
    NF4_EWORKSPACE before anything touches a device."""
    L, m = lib
    EINVAL, EALIGN, EWS = -1, -2, -6
    nmax = L.nf4_quantize_noalloc_max_elements()
    assert m.layout(nmax)["quantize_workspace_bytes"] <= 16 << 20 < m.layout(nmax + 1)["quantize_workspace_bytes"]
    t = m._Tensor(16, 16, 16, 16, nmax + 1, 1)
    assert L.nf4_quantize_noalloc(16, nmax + 1, 1, ctypes.byref(t), None, None) == EWS
    t = m._Tensor(16, 16, 16, 16, 64, 1)
    assert L.nf4_quantize_noalloc(None, 64, 1, ctypes.byref(t), None, None) == EINVAL
    assert L.nf4_quantize_noalloc(16, 64, 0, ctypes.byref(t), None, None) == EINVAL   # flag disagrees with out
    assert L.nf4_quantize_noalloc(24, 64, 1, ctypes.byref(t), None, None) == EALIGN
    assert L.nf4_quantize_noalloc(16, 65, 1, ctypes.byref(t), None, None) == EINVAL   # n disagrees with out
