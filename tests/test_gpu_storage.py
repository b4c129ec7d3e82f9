"""GPU parity of nf4_quantize / nf4_dequantize against the CPU oracle: packed
codes, scales, nested maxima, offset and decoded weights must match bit for bit
(Aner docs "Packed NF4 and the portable QLoRA profile"; Soup gate results "P3
is solved": repeated quantization is byte-identical)."""
import numpy as np
import pytest
import torch

import workloads
from tests.parity import bits

pytestmark = pytest.mark.gpu

SIZES = [1, 2, 7, 8, 9, 63, 64, 65, 127, 1001, 16383, 16384, 16385, 3 * 16384 + 17, 192 * 576, 576 * 576,
         1536 * 576, 64 * 1000 + 33, 4 * 16384 * 3 + 5]


def _gpu_quant(gpu, w: np.ndarray, dq: bool):
    wt = torch.from_numpy(w).cuda()
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    q = gpu.quantize(wt, dq, status=status)
    torch.cuda.synchronize()
    return q, int(status.item())


def _compare_packed(q, ref, dq):
    np.testing.assert_array_equal(q.codes.cpu().numpy(), ref["codes"])
    if dq:
        np.testing.assert_array_equal(q.scales.cpu().numpy(), ref["qabs"])
        np.testing.assert_array_equal(bits(q.nested), ref["nested"].view(np.uint32))
        np.testing.assert_array_equal(bits(q.offset), ref["offset"].view(np.uint32))
    else:
        np.testing.assert_array_equal(bits(q.scales), ref["absmax"].view(np.uint32))


@pytest.mark.parametrize("dq", [True, False])
@pytest.mark.parametrize("n", SIZES)
def test_quantize_dequantize_bitexact(gpu, orc, n, dq):
    print(f"[storage] n={n} dq={dq}", flush=True)
    w = workloads.weight_with_outliers((n,), seed=n).numpy()
    q, status = _gpu_quant(gpu, w, dq)
    assert status == 0
    ref = orc.quantize(w, dq)
    _compare_packed(q, ref, dq)
    f32 = gpu.dequantize(q, torch.float32)
    b16 = gpu.dequantize(q, torch.bfloat16)
    np.testing.assert_array_equal(bits(f32), orc.dequantize(ref, "f32").view(np.uint32))
    np.testing.assert_array_equal(bits(b16), orc.dequantize(ref, "bf16"))


def test_special_blocks(gpu, orc):
    """Zero blocks, constant-magnitude blocks, fp32 denormals and values on the
    codebook grid, in one matrix."""
    c4 = orc.nf4_table()
    parts = [np.zeros(64 * 3, np.float32),
             np.full(64 * 5, -0.25, np.float32),
             (np.arange(64 * 4) % 7 - 3).astype(np.float32) * np.float32(1e-42),   # denormals
             np.float32(4.0) * c4[np.arange(64 * 2) % 16],
             workloads.normal_f32((64 * 300 + 11,), 0.02, 77).numpy()]
    w = np.concatenate(parts).astype(np.float32)
    for dq in (True, False):
        q, status = _gpu_quant(gpu, w, dq)
        assert status == 0
        ref = orc.quantize(w, dq)
        _compare_packed(q, ref, dq)
        np.testing.assert_array_equal(bits(gpu.dequantize(q, torch.float32)), orc.dequantize(ref).view(np.uint32))


def test_extreme_block_maxima(gpu, orc):
    """Blocks whose maximum lies above 2^126 (so 1/m is subnormal), at 2^126
    exactly, between it and the largest float, in [2^-126, 2^-120) (where
    128 / m overflows), at 2^-120, subnormal, and at 1 and 2^-1, with subnormal
    weights beside normal maxima: every weight's code is that of the correctly
    rounded w / m (each block holds +-m itself, so the quotients reach +-1)."""
    rng = np.random.default_rng(17)

    def block(m):
        b = (rng.uniform(-1.0, 1.0, 64) * m).astype(np.float32)
        b[rng.integers(64)] = np.float32(m) * np.float32(rng.choice([-1.0, 1.0]))
        return b

    maxima = [3.0e38, 1.5e38, 2.0 ** 126, 1.5 * 2.0 ** 126, 1.0e38, 3.4e38, 2.0 ** -126, 3 * 2.0 ** -126,
              1.5 * 2.0 ** -121, 2.0 ** -120, 1.25 * 2.0 ** -120, 1.0e-40, 5.0e-45, 1.0, 0.5, 2.0 ** 100]
    parts = [block(m) for m in maxima]
    parts.append(workloads.normal_f32((64 * 700 + 9,), 0.02, 5).numpy())
    w = np.concatenate(parts).astype(np.float32)
    assert np.all(np.isfinite(w))
    for dq in (True, False):
        print(f"[storage] extreme maxima dq={dq}", flush=True)
        q, status = _gpu_quant(gpu, w, dq)
        assert status == 0
        ref = orc.quantize(w, dq)
        _compare_packed(q, ref, dq)
        np.testing.assert_array_equal(bits(gpu.dequantize(q, torch.float32)), orc.dequantize(ref).view(np.uint32))


def test_repeat_identical_and_nonfinite(gpu):
    w = workloads.weight_with_outliers((64 * 5000 + 3,), seed=8).cuda()
    a = gpu.quantize(w, True)
    b = gpu.quantize(w.clone(), True)
    torch.cuda.synchronize()
    for x, y in [(a.codes, b.codes), (a.scales, b.scales), (a.nested, b.nested), (a.offset, b.offset)]:
        assert torch.equal(x, y)
    for bad in (float("nan"), float("inf")):
        v = w.clone()
        v[1234] = bad
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        gpu.quantize(v, True, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == -5  # NF4_ENONFINITE
        gpu.quantize(w, True, status=st)  # a finite call clears it again
        torch.cuda.synchronize()
        assert int(st.item()) == 0


def test_dequantize_from_oracle_packed(gpu, orc):
    """Decode buffers written by the oracle (not by the GPU quantizer)."""
    n = 4096 * 37 + 5
    w = workloads.weight_with_outliers((n,), seed=3).numpy()
    ref = orc.quantize(w, True)
    t = gpu.NF4Tensor(torch.from_numpy(ref["codes"]).cuda(), torch.from_numpy(ref["qabs"]).cuda(),
                      torch.from_numpy(ref["nested"]).cuda(), torch.from_numpy(ref["offset"]).cuda(), (n,), True)
    np.testing.assert_array_equal(bits(gpu.dequantize(t, torch.bfloat16)), orc.dequantize(ref, "bf16"))


@pytest.mark.parametrize("shape", [(4096, 14336), (4096, 4096)])
def test_full_size_matrix(gpu, orc, shape):
    """One matrix of each shape of the 7.5e9-parameter quantize/dequantize
    workload (N(0, 0.02) with 1% outliers at 10x), full comparison."""
    print(f"[storage] full {shape}", flush=True)
    w = workloads.weight_with_outliers(shape, seed=workloads.weight_seed(0), device="cuda")
    q = gpu.quantize(w, True)
    d = gpu.dequantize(q, torch.bfloat16)
    torch.cuda.synchronize()
    ref = orc.quantize(w.cpu().numpy(), True)
    _compare_packed(q, ref, True)
    np.testing.assert_array_equal(bits(d).ravel(), orc.dequantize(ref, "bf16"))


@pytest.mark.parametrize("n", [1024 * 16384, 1024 * 16384 + 1, 4096 * 16384, 4096 * 16384 + 7, (1 << 27) + 12345])
def test_mean_over_many_groups(gpu, orc, n):
    """The mean's pairwise tree over the quantizer's partial sums (one per
    4096 weights): 4096 partials (the mean formed in every nested-block
    workgroup, one full round), 4097 (the separate 1024-thread mean kernel, one
    zero-padded round of 16384), 16384 (one full round), 16385 and 32772 (two
    and four rounds joined by the binary counter)."""
    print(f"[storage] mean tree n={n}", flush=True)
    w = workloads.weight_with_outliers((n,), seed=n % 1000, device="cuda")
    q = gpu.quantize(w, True)
    torch.cuda.synchronize()
    ref = orc.quantize(w.cpu().numpy(), True)
    _compare_packed(q, ref, True)


def test_dequantize_many_equals_single_calls(gpu, orc):
    """One launch over mixed tensors (double and single quantization, sizes with
    tails, one tiny) equals per-tensor nf4_dequantize bit for bit, and the
    oracle for two of them."""
    sizes = [(64 * 5000 + 3, True), (1, True), (4096 * 37 + 5, False), (16384 * 3, True), (127, False),
             (1536 * 576, True)]
    ws = [workloads.weight_with_outliers((n,), seed=i + 11).numpy() for i, (n, _) in enumerate(sizes)]
    qs = [gpu.quantize(torch.from_numpy(w).cuda(), dq) for w, (_, dq) in zip(ws, sizes)]
    for dtype in (torch.bfloat16, torch.float32):
        many = gpu.dequantize_many(qs, dtype)
        single = [gpu.dequantize(q, dtype) for q in qs]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(many, single)):
            assert torch.equal(a.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                               b.view(torch.int16 if dtype == torch.bfloat16 else torch.int32)), (i, dtype)
    for i in (0, 2):
        ref = orc.quantize(ws[i], sizes[i][1])
        np.testing.assert_array_equal(bits(many[i]), orc.dequantize(ref, "f32").view(np.uint32))


def _same_packed(a, b):
    assert torch.equal(a.codes, b.codes)
    assert torch.equal(a.scales.view(torch.uint8), b.scales.view(torch.uint8))
    if a.double_quant:
        assert torch.equal(a.nested.view(torch.int32), b.nested.view(torch.int32))
        assert torch.equal(a.offset.view(torch.int32), b.offset.view(torch.int32))


def test_quantize_many_equals_single_calls(gpu, orc):
    """One nf4_quantize_many call over mixed tensors (double and single
    quantization, sizes with tails, tiny ones, one past 4096 groups whose mean
    a single call forms in its own kernel) equals per-tensor nf4_quantize bit
    for bit, and the oracle for three of them; the status word reports a
    non-finite weight in any tensor and is cleared by the next finite call."""
    sizes = [(64 * 5000 + 3, True), (1, True), (4096 * 37 + 5, False), (16384 * 3, True), (127, False),
             (1536 * 576, True), (4097 * 16384 + 5, True), (64, False)]
    ws = [workloads.weight_with_outliers((n,), seed=i + 21, device="cuda") for i, (n, _) in enumerate(sizes)]
    dqs = [dq for _, dq in sizes]
    st = torch.full((1,), 77, dtype=torch.int32, device="cuda")
    many = gpu.quantize_many(ws, dqs, status=st)
    single = [gpu.quantize(w, dq) for w, dq in zip(ws, dqs)]
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i, (a, b) in enumerate(zip(many, single)):
        print(f"[storage] many item {i} n={sizes[i][0]}", flush=True)
        _same_packed(a, b)
    for i in (0, 2, 5):
        _compare_packed(many[i], orc.quantize(ws[i].cpu().numpy(), dqs[i]), dqs[i])
    for bad_item in (2, 6):  # single, then double quantization
        v = [w.clone() for w in ws]
        v[bad_item][sizes[bad_item][0] // 2] = float("nan")
        gpu.quantize_many(v, dqs, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == -5  # NF4_ENONFINITE
        gpu.quantize_many(ws, dqs, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
    # single quantization only: no nested blocks, one workgroup writes the status
    outs = gpu.quantize_many([ws[2], ws[4]], False, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    _same_packed(outs[0], single[2])
    _same_packed(outs[1], single[4])


def test_quantizer_decision_boundaries(gpu, orc):
    """Inputs on the decision boundaries, where a reciprocal multiply and the
    correctly rounded division pick different codes: NF4 codes of elements
    within a few ulps of the midpoints between adjacent codes (single and
    double quantization), and dynamic8 codes of centred block maxima within a
    few ulps of the dynamic8 midpoints (exact mean and nested maxima by
    construction). The GPU packs them bit for bit like the oracle, whose codes
    the CPU tests pin to an exact nearest search with true division."""
    from tests import boundary_sets
    w, dis = boundary_sets.nf4_division_boundary(orc.nf4_table())
    assert dis > 20
    for dq in (False, True):
        print(f"[storage] NF4 division boundaries n={w.size} dq={dq}", flush=True)
        q, status = _gpu_quant(gpu, w, dq)
        assert status == 0
        _compare_packed(q, orc.quantize(w, dq), dq)
    w, mu0, nested, dis = boundary_sets.dyn8_midpoint_maxima(orc.dyn8_table())
    assert dis > 20
    print(f"[storage] dynamic8 midpoint maxima n={w.size}", flush=True)
    q, status = _gpu_quant(gpu, w, True)
    assert status == 0
    ref = orc.quantize(w, True)
    assert ref["offset"][0] == mu0
    np.testing.assert_array_equal(ref["nested"], nested)
    _compare_packed(q, ref, True)
    np.testing.assert_array_equal(bits(gpu.dequantize(q, torch.float32)), orc.dequantize(ref, "f32").view(np.uint32))


def test_double_quant_decode_golden(gpu):
    """The hand-built double-quantized matrix of tests/golden/dq_decode_golden.json,
    whose block scales a fused multiply-add would round differently: both
    nf4_dequantize outputs, and the weights the fused forward GEMM decodes
    (x = I, so y = W_hat^T exactly), equal the stored bits."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "dq_decode_golden.json")))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    u32 = lambda v: np.asarray(v, np.uint32).view(np.float32)
    W = gpu.NF4Tensor(dev(np.frombuffer(bytes.fromhex(g["codes_hex"]), np.uint8).copy()),
                      dev(np.array(g["qabs"], np.uint8)), dev(u32([g["nested_f32_bits"]])),
                      dev(u32([g["offset_f32_bits"]])), (5, 64), True)
    f32 = gpu.dequantize(W, torch.float32)
    b16 = gpu.dequantize(W, torch.bfloat16)
    y, _ = gpu.linear_fwd(torch.eye(64, dtype=torch.bfloat16, device="cuda"), W)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(f32).ravel(), np.array(g["expected_f32_bits"], np.uint32))
    np.testing.assert_array_equal(bits(b16).ravel(), np.array(g["expected_bf16_bits"], np.uint16))
    np.testing.assert_array_equal(bits(y.T.contiguous()).ravel(), np.array(g["expected_bf16_bits"], np.uint16))
