"""nf4_quantize_noalloc (the quantize entry point for callers that cannot
allocate: it keeps its double-quantization scratch in a fixed device array)
against nf4_quantize with a caller workspace, through the C ABI: packed codes,
block scales, nested maxima and offset bit for bit, on two calls in a row (the
second smaller, so the shared scratch holds stale entries of the first), with
double and single quantization and a non-finite weight."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from tests.parity import bits

pytestmark = pytest.mark.gpu


def _noalloc(gpu, w: torch.Tensor, dq: bool, status=None):
    out = gpu.NF4Tensor.empty(tuple(w.shape), dq, w.device)
    st = out.c_struct()
    rc = gpu.load().nf4_quantize_noalloc(ctypes.c_void_p(w.data_ptr()), w.numel(), int(dq), ctypes.byref(st),
                                         None if status is None else ctypes.c_void_p(status.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, gpu.load().nf4_status_string(rc)
    return out


def _same(a, b, dq):
    assert torch.equal(a.codes, b.codes)
    assert np.array_equal(bits(a.scales), bits(b.scales))
    if dq:
        assert np.array_equal(bits(a.nested), bits(b.nested))
        assert np.array_equal(bits(a.offset), bits(b.offset))


@pytest.mark.parametrize("dq", [True, False])
def test_noalloc_quantize_matches_workspace_call(gpu, dq):
    sizes = [(4096, 14336), (576, 576)]          # the second call is smaller
    for i, shape in enumerate(sizes):
        print(f"[noalloc] call {i} shape={shape} dq={dq}", flush=True)
        w = workloads.weight_with_outliers(shape, seed=70 + i, device="cuda")
        got = _noalloc(gpu, w, dq)
        ref = gpu.quantize(w, dq)
        torch.cuda.synchronize()
        _same(got, ref, dq)


def test_noalloc_quantize_largest_and_nonfinite(gpu):
    n = gpu.quantize_noalloc_max_elements()
    assert gpu.layout(n)["quantize_workspace_bytes"] <= 16 << 20 < gpu.layout(n + 1)["quantize_workspace_bytes"]
    print(f"[noalloc] largest n={n}", flush=True)
    w = workloads.normal_f32((n,), 0.02, 81, "cuda")
    got = _noalloc(gpu, w, True)
    ref = gpu.quantize(w, True)
    torch.cuda.synchronize()
    _same(got, ref, True)
    del w, got, ref
    # a NaN weight is reported through the status word, as nf4_quantize does
    w = workloads.normal_f32((1000, 64), 0.02, 82, "cuda")
    w[123, 5] = float("nan")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    _noalloc(gpu, w, True, status)
    torch.cuda.synchronize()
    assert int(status.item()) == -5
    # one more small call afterwards is again exact
    w = workloads.weight_with_outliers((192, 576), seed=83, device="cuda")
    got = _noalloc(gpu, w, True)
    ref = gpu.quantize(w, True)
    torch.cuda.synchronize()
    _same(got, ref, True)
