"""Pins of the oracle's quantize / double-quantize / dequantize.

Format: Aner docs, "Native model adaptation and NF4", section "Packed NF4 and
the portable QLoRA profile"; determinism: Soup gate results, "P3 is solved".
The checks use facts that do not depend on the oracle's own code: a
hand-derived worked example, nearest-code search by argmin (no thresholds),
exact special cases, the round-trip error bound implied by nearest rounding,
and torch's own bf16 conversion.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from tests import boundary_sets

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "nf4_worked_example.json")))


def unpack(codes: np.ndarray, n: int) -> np.ndarray:
    hi = codes >> 4
    lo = codes & 0x0F
    return np.stack([hi, lo], axis=1).ravel()[:n]


def blocks(a: np.ndarray, size: int):
    return [a[i:i + size] for i in range(0, a.size, size)]


def weights(n, seed=7, outliers=True):
    if outliers:
        return workloads.weight_with_outliers((n,), seed=seed).numpy()
    return workloads.normal_f32((n,), 0.02, seed).numpy()


# ----------------------------------------------------------------------------- worked example

def test_worked_example(orc):
    c4 = orc.nf4_table()
    w = np.concatenate([np.float32(2.0) * c4[np.arange(64) % 16], np.zeros(64, np.float32),
                        np.array([-0.5], np.float32)]).astype(np.float32)
    assert w.size == GOLD["n"]
    for dq in (False, True):
        q = orc.quantize(w, double_quant=dq)
        assert q["codes"].tobytes().hex() == GOLD["expected_codes_hex"]
        np.testing.assert_array_equal(q["absmax"], np.array(GOLD["expected_absmax"], np.float32))
    q = orc.quantize(w, double_quant=False)
    r = orc.dequantize(q)
    np.testing.assert_array_equal(r[:64], w[:64])
    np.testing.assert_array_equal(r[64:128], np.zeros(64, np.float32))
    assert r[128] == np.float32(-0.5)


# ----------------------------------------------------------------------------- codes

@pytest.mark.parametrize("n", [1, 63, 64, 65, 1001, 16385, 70001])
def test_codes_are_nearest(orc, n):
    w = weights(n, seed=n)
    q = orc.quantize(w, double_quant=True)
    c4 = orc.nf4_table().astype(np.float64)
    codes = unpack(q["codes"], n)
    if n % 2:
        assert q["codes"][-1] & 0x0F == 0, "odd tail pads the low nibble with 0"
    absmax = np.array([np.abs(b).max() for b in blocks(w, 64)], np.float32)
    np.testing.assert_array_equal(q["absmax"], absmax)
    a = np.repeat(absmax, 64)[:n]
    x = (w / a).astype(np.float32)            # IEEE fp32 division
    want = np.argmin(np.abs(x[:, None].astype(np.float64) - c4[None, :]), axis=1)  # first min = lower index
    np.testing.assert_array_equal(codes, want)


def test_repeat_is_byte_identical(orc):
    w = weights(300_001, seed=3)
    q1 = orc.quantize(w, True)
    q2 = orc.quantize(w.copy(), True)
    for k in ("codes", "qabs", "nested", "offset"):
        assert q1[k].tobytes() == q2[k].tobytes()


def test_nonfinite_rejected(orc):
    w = weights(1000)
    for bad in (np.nan, np.inf, -np.inf):
        v = w.copy()
        v[500] = bad
        with pytest.raises(ValueError):
            orc.quantize(v, True)


# ----------------------------------------------------------------------------- double quantization

def test_double_quant_fields(orc):
    n = 64 * 1000 + 33
    w = weights(n, seed=11)
    q = orc.quantize(w, True)
    absmax = q["absmax"]
    nb = absmax.size
    # mean of the block maxima: the fp64 sum is exact for these values (checked
    # against the correctly rounded fsum), so the stored mean is fixed.
    S = math.fsum(float(v) for v in absmax)
    assert np.float32(S / nb) == q["offset"][0]
    mu = q["offset"][0]
    c = (absmax - mu).astype(np.float32)
    m = np.array([np.abs(b).max() for b in blocks(c, 256)], np.float32)
    np.testing.assert_array_equal(q["nested"], m)
    d8 = orc.dyn8_table().astype(np.float64)
    y = (c / np.repeat(m, 256)[:nb]).astype(np.float32)
    want = np.argmin(np.abs(y[:, None].astype(np.float64) - d8[None, :]), axis=1)
    np.testing.assert_array_equal(q["qabs"], want)


def test_mean_small_example(orc):
    # four blocks with maxima 1, 2, 3, 4 -> mean 2.5; centred 1.5 is the nested max
    w = np.concatenate([np.full(64, v, np.float32) for v in (1.0, -2.0, 3.0, -4.0)])
    q = orc.quantize(w, True)
    assert q["offset"][0] == np.float32(2.5)
    assert q["nested"][0] == np.float32(1.5)
    d8 = orc.dyn8_table()
    # centred values -1.5, -0.5, 0.5, 1.5 over 1.5: -1, -1/3, 1/3, 1
    assert d8[q["qabs"][3]] == 1.0 and q["qabs"][0] == 0  # -1 -> nearest is the smallest entry
    codes = unpack(q["codes"], w.size)
    assert set(codes[:64]) == {15} and set(codes[64:128]) == {0}


def test_constant_magnitude_reconstructs_exactly(orc):
    rng = np.random.default_rng(5)
    w = (np.where(rng.random(64 * 700) < 0.5, -1, 1) * 0.25).astype(np.float32)
    q = orc.quantize(w, True)
    assert q["offset"][0] == np.float32(0.25)
    assert np.all(q["nested"] == 0) and np.all(q["qabs"] == 127)
    np.testing.assert_array_equal(orc.dequantize(q), w)


def test_zero_matrix(orc):
    w = np.zeros(64 * 300 + 5, np.float32)
    for dq in (False, True):
        q = orc.quantize(w, dq)
        assert np.all(unpack(q["codes"], w.size) == 7)
        r = orc.dequantize(q)
        assert np.all(r == 0)
    q = orc.quantize(w, True)
    assert q["offset"][0] == 0 and np.all(q["qabs"] == 127) and np.all(q["nested"] == 0)


def test_block_max_reconstructs_exactly_single(orc):
    w = weights(64 * 512, seed=21)
    q = orc.quantize(w, False)
    r = orc.dequantize(q)
    for b, (wb, rb) in enumerate(zip(blocks(w, 64), blocks(r, 64))):
        i = int(np.argmax(np.abs(wb)))
        assert rb[i] == wb[i], b  # the max element sits on code 0 or 15 (= -1 or +1)


# ----------------------------------------------------------------------------- round trip

def _half_gaps(table):
    t = table.astype(np.float64)
    g = np.diff(t)
    left = np.concatenate([[0.0], g]) / 2
    right = np.concatenate([g, [0.0]]) / 2
    return np.maximum(left, right)


@pytest.mark.parametrize("dq", [False, True])
def test_round_trip_bound(orc, dq):
    """|w - w_hat| <= a * halfgap(code) + |C4[code]| * |a - a'| + rounding, where the
    nearest-code choice bounds the first term and the dynamic8 grid the second."""
    n = 64 * 4096 + 17
    w = weights(n, seed=99)
    q = orc.quantize(w, dq)
    r = orc.dequantize(q).astype(np.float64)
    c4 = orc.nf4_table().astype(np.float64)
    codes = unpack(q["codes"], n)
    a = np.repeat(q["absmax"].astype(np.float64), 64)[:n]
    eps = 2.0 ** -23
    bound = a * (_half_gaps(c4)[codes] + eps) + np.abs(r) * eps
    if dq:
        d8 = orc.dyn8_table()
        nb = q["absmax"].size
        m = np.repeat(q["nested"].astype(np.float64), 256)[:nb]
        ascale = m * (_half_gaps(d8).max() + 4 * eps) + q["absmax"] * 4 * eps
        bound += np.abs(c4[codes]) * np.repeat(ascale, 64)[:n]
    err = np.abs(w.astype(np.float64) - r)
    assert np.all(err <= bound)
    assert err.max() > 0.25 * bound.max()  # the bound is not vacuous


def test_bf16_output_matches_torch_rounding(orc):
    w = weights(64 * 2000 + 3, seed=4)
    q = orc.quantize(w, True)
    f = orc.dequantize(q, "f32")
    h = orc.dequantize(q, "bf16")
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(h, ref)


def test_normalisation_is_true_division(orc):
    """Inputs placed within a few ulps of the decision boundaries, where
    w * (1/a) and the correctly rounded w / a fall on different sides; the codes
    must follow w / a (reading: IEEE division, round to nearest)."""
    c4 = orc.nf4_table().astype(np.float64)
    w, disagreements = boundary_sets.nf4_division_boundary(orc.nf4_table())
    assert disagreements > 20
    q = orc.quantize(w, False)
    codes = unpack(q["codes"], w.size)
    a = np.repeat(q["absmax"], 64)
    x = (w / a).astype(np.float32)
    want = np.argmin(np.abs(x[:, None].astype(np.float64) - c4[None, :]), axis=1)
    np.testing.assert_array_equal(codes, want)


def test_nested_codes_at_dynamic8_midpoints(orc):
    """Block maxima whose centred values sit within a few ulps of the midpoints
    between dynamic8 codes (the mean and nested maximum are exact by
    construction): the mean is the construction's, the nested maxima are
    exact, and every nested code is the argmin (ties to the lower index) of
    |D8[k] - fl32(c / m)| with true division, which differs from the
    reciprocal-multiply code on some of them."""
    d8 = orc.dyn8_table().astype(np.float64)
    w, mu0, nested, disagreements = boundary_sets.dyn8_midpoint_maxima(orc.dyn8_table())
    assert disagreements > 20
    q = orc.quantize(w, True)
    assert q["offset"][0] == mu0
    np.testing.assert_array_equal(q["nested"], nested)
    c = (q["absmax"] - mu0).astype(np.float32)       # exact: the maxima are mu0 +- d
    m = np.repeat(nested, 256)[:c.size]
    x = (c / m).astype(np.float32).astype(np.float64)
    want = np.argmin(np.abs(x[:, None] - d8[None, :]), axis=1)
    np.testing.assert_array_equal(q["qabs"], want)


# --------------------------------------------------------------------------- selected-row embedding decode

def _exact_table(V: int, D: int, seed: int, double_quant: bool) -> np.ndarray:
    """A [V, D] fp32 table that NF4 stores exactly: every value is C4[k] * a with
    one shared a, and every 64-block holds a +-a entry, so each block absmax is
    a; then every centred absmax is 0 and double quantization is exact too."""
    rng = np.random.default_rng(seed)
    a = np.float32(0.03125)
    import oracle
    c4 = oracle.nf4_table()
    codes = rng.integers(0, 16, size=V * D)
    flat = (c4[codes] * a).astype(np.float32)
    flat[::64] = np.where(rng.random(flat[::64].size) < 0.5, -a, a)
    return flat.reshape(V, D)


@pytest.mark.parametrize("V,D,dq", [(300, 576, True), (257, 77, True), (40, 64, False), (5, 3, True)])
def test_embedding_rows_return_the_selected_rows(orc, V, D, dq):
    """On a table NF4 represents exactly, the decoded rows are the table's rows:
    ids in any order, repeated, first and last row."""
    W = _exact_table(V, D, V + D, dq)
    q = orc.quantize(W, dq)
    ids = np.array([V - 1, 0, 7 % V, 7 % V, V // 2, 1 % V, V - 1], np.int64)
    got = orc.embedding_rows(q, D, ids)
    np.testing.assert_array_equal(got, W[ids])
    bits = orc.embedding_rows(q, D, ids, out="bf16")
    assert bits.dtype == np.uint16 and bits.shape == (ids.size, D)
    want_bits = torch.from_numpy(W[ids]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, want_bits)  # torch's round-to-nearest-even of the exact rows


def test_embedding_rows_reject_out_of_range(orc):
    W = _exact_table(10, 64, 1, True)
    q = orc.quantize(W, True)
    with pytest.raises(IndexError):
        orc.embedding_rows(q, 64, [0, 10])
    with pytest.raises(IndexError):
        orc.embedding_rows(q, 64, [-1])
    assert orc.embedding_rows(q, 64, np.zeros(0, np.int64)).shape == (0, 64)


# --------------------------------------------------------------------------- double-quant decode rounding

DQG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "dq_decode_golden.json")))


def _f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def test_double_quant_decode_golden(orc):
    """The hand-built double-quantized matrix of tests/golden/dq_decode_golden.json
    (decode rule: separately rounded fp32 steps, no fused multiply-add). The
    block-0 derivation is checked in integers, every stored value against exact
    rational arithmetic on the tables (not the oracle's decoder), and the oracle's
    dequantize against the stored bits; a fused multiply-add for the block scale
    would change the first three blocks."""
    from fractions import Fraction as F
    from tests.golden import make_dq_decode_golden as gen
    # block 0 by hand: D8[7] = -229/256, m = 13421773 * 2^-29, mu = 2^-5
    assert F(float(orc.dyn8_table()[7])) == F(-229, 256)
    assert F(float(_f32(DQG["nested_f32_bits"]))) == F(13421773, 2 ** 29)
    assert -229 * 13421773 == -3073586017 and round(3073586017 / 2 ** 8 - 0.5) == 12006195
    assert F(float(_f32(DQG["block_scale_f32_bits"][0]))) == F(16777216 - 12006195, 2 ** 29) == F(4771021, 2 ** 29)
    assert F(float(_f32(DQG["block_scale_if_fused_f32_bits"][0]))) == F(9542041, 2 ** 30)
    # every stored value from exact arithmetic on the two tables
    m, blocks = gen.derive(orc.nf4_table(), orc.dyn8_table())
    assert [gen.f32_bits(b["a_sep"]) for b in blocks] == DQG["block_scale_f32_bits"]
    assert [gen.f32_bits(b["w"][i % 16]) for b in blocks for i in range(64)] == DQG["expected_f32_bits"]
    assert [gen.bf16_bits(b["w"][i % 16]) for b in blocks for i in range(64)] == DQG["expected_bf16_bits"]
    sep, fused = DQG["block_scale_f32_bits"], DQG["block_scale_if_fused_f32_bits"]
    assert all(sep[b] != fused[b] for b in range(3)) and sep[3:] == fused[3:]
    # the oracle decodes the packed fields to the stored bits
    q = dict(codes=np.frombuffer(bytes.fromhex(DQG["codes_hex"]), np.uint8), qabs=np.array(DQG["qabs"], np.uint8),
             nested=_f32([DQG["nested_f32_bits"]]), offset=_f32([DQG["offset_f32_bits"]]), n=DQG["n"],
             double_quant=True)
    np.testing.assert_array_equal(orc.dequantize(q, "f32").view(np.uint32), np.array(DQG["expected_f32_bits"],
                                                                                      np.uint32))
    np.testing.assert_array_equal(orc.dequantize(q, "bf16"), np.array(DQG["expected_bf16_bits"], np.uint16))


# --------------------------------------------------------------------------- property test over odd sizes

from hypothesis import given, settings, strategies as st


@settings(max_examples=40, deadline=None)
@given(half=st.integers(min_value=0, max_value=49_999), seed=st.integers(min_value=0, max_value=2**31 - 1),
       dq=st.booleans())
def test_odd_sizes_property(orc, half, seed, dq):
    """For any odd n in [1, 1e5] (format: Aner docs "Packed NF4 and the portable
    QLoRA profile"): the layout sizes, a zero low nibble in the last byte,
    codes equal to the exact nearest search, repeat quantization byte-identical,
    and every decoded weight within the nearest-code round-trip bound."""
    n = 2 * half + 1
    w = workloads.weight_with_outliers((n,), seed=seed % 100_000).numpy()
    q = orc.quantize(w, dq)
    nb = (n + 63) // 64
    assert q["codes"].size == (n + 1) // 2 and q["absmax"].size == nb
    if dq:
        assert q["qabs"].size == nb and q["nested"].size == (nb + 255) // 256 and q["offset"].size == 1
    assert q["codes"][-1] & 0x0F == 0
    q2 = orc.quantize(w, dq)
    assert all(np.array_equal(q[k], q2[k]) for k in q if isinstance(q[k], np.ndarray))
    c4 = orc.nf4_table().astype(np.float64)
    codes = unpack(q["codes"], n)
    a = np.repeat(q["absmax"], 64)[:n]
    x = np.where(a > 0, (w / np.where(a > 0, a, 1)).astype(np.float32), 0).astype(np.float64)
    want = np.where(a > 0, np.argmin(np.abs(x[:, None] - c4[None, :]), axis=1), 7)
    np.testing.assert_array_equal(codes, want)
    r = orc.dequantize(q).astype(np.float64)
    eps = 2.0 ** -23
    bound = a.astype(np.float64) * (_half_gaps(c4)[codes] + eps) + np.abs(r) * eps
    if dq:
        d8 = orc.dyn8_table()
        m = np.repeat(q["nested"].astype(np.float64), 256)[:nb]
        bound += np.abs(c4[codes]) * np.repeat(m * (_half_gaps(d8).max() + 4 * eps) + q["absmax"] * 4 * eps, 64)[:n]
    assert np.all(np.abs(w.astype(np.float64) - r) <= bound)
