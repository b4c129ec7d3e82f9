"""Pins of the packed layout against the integers the pages print
(tests/golden/layout_pins.json names the page and key of each)."""
import json
import os

import pytest

from workloads import smollm2_all_matrices, quant_throughput_matrices

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layout_pins.json")))


@pytest.mark.parametrize("case", GOLDEN["component_benchmarks"]["cases"], ids=lambda c: f"{c['rows']}x{c['columns']}")
def test_device_copy_bytes(orc, case):
    n = case["rows"] * case["columns"]
    lay = orc.layout(n, True)
    assert lay["device_bytes"] == case["packed_gpu_bytes"]
    assert 4 * n == case["dense_float32_bytes"]


def test_smollm2_totals(orc):
    g = GOLDEN["smollm2_135m"]
    mats = smollm2_all_matrices()
    assert len(mats) == 211  # 30 x 7 decoder linears + tied embedding
    host = sum(orc.layout(n * k, True)["total_bytes"] for n, k in mats)
    dev = sum(orc.layout(n * k, True)["device_bytes"] for n, k in mats)
    assert host == g["packed_base_bytes"]
    assert dev == g["gpu_packed_base_bytes"]
    assert host - dev == 4 * len(mats)  # one 4-byte fp32 mean per matrix
    # norm vectors stay fp32 and make up the rest of the parameters
    matrix_params = sum(n * k for n, k in mats)
    norm_params = g["floating_base_bytes"] // 4
    assert matrix_params + norm_params == g["parameters"]
    assert 4 * g["parameters"] == g["decoded_float32_bytes"]
    assert host + g["floating_base_bytes"] == g["weight_bytes_host_tiled"]
    assert host + dev + g["floating_base_bytes"] == g["weight_bytes_fused"]


def test_adapter_shapes(orc):
    """A is [r, in], B is [out, r]: parameter counts of rank-2 LoRA on q and v."""
    g = GOLDEN["adapters"]
    r, h, kv, layers = g["rank"], 576, 192, 30
    a_params = layers * (r * h + r * h)            # A of q and v (both take hidden inputs)
    b_params = layers * (h * r + kv * r)           # B of q (out 576) and v (out 192)
    assert a_params + b_params == g["lora_trainable_parameters"]
    assert 4 * (a_params + b_params) == g["lora_adapter_bytes"]
    # LoRA-FA trains B only; A and a persisted r x r preconditioner per target are frozen
    assert b_params == g["lora_fa_trainable_parameters"]
    assert 4 * a_params + 4 * (2 * layers) * r * r == g["lora_fa_frozen_adapter_bytes"]


def test_per_weight_formula(orc):
    for n, k in [(4096, 14336), (4096, 4096), (1024, 4096), (14336, 4096)]:
        N = n * k
        assert N % 16384 == 0
        assert orc.layout(N, True)["total_bytes"] == N // 2 + N // 64 + N // 4096 + 4
        assert abs(orc.layout(N, True)["total_bytes"] / N - GOLDEN["per_weight_formula"]["bytes_per_param_approx"]) < 1e-3


def test_quant_workload_size(orc):
    mats = quant_throughput_matrices()
    assert sum(n * k for n, k in mats) == 7_499_415_552


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 16383, 16384, 16385, 3 * 16384 + 17])
def test_tail_layout(orc, n):
    lay = orc.layout(n, True)
    nb = -(-n // 64)
    assert lay["codes"] == -(-n // 2)
    assert lay["scales"] == nb and lay["nb"] == nb
    assert lay["nested"] == 4 * -(-nb // 256)
    assert orc.layout(n, False)["scales"] == 4 * nb and orc.layout(n, False)["nested"] == 0
