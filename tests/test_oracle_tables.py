"""Pins of the oracle's code tables, thresholds and encoder.

The pages name the tables (16-value NF4, signed dynamic8 with 256 entries, the
same for every weight: Aner docs "Packed NF4 and the portable QLoRA profile";
Soup gate results "P3 is solved") but print no values. The pins below come from
outside the oracle: an independent library inverse normal CDF (scipy, and
Python's statistics module), exact rational arithmetic over the dynamic8 bit
layout, and exhaustive comparison of the threshold encoder with a nearest-code
search that uses no thresholds.
"""
import ctypes
import os
import statistics
import subprocess
from fractions import Fraction

import numpy as np
import pytest
from scipy.stats import norm

HERE = os.path.dirname(os.path.abspath(__file__))


def _f32_bits(x):
    return int(np.float32(x).view(np.uint32))


def _nearest_f32_of_fraction(q: Fraction) -> np.float32:
    """fp32 nearest to an exact rational (ties to even), decided exactly."""
    f = np.float32(float(q))  # candidate (may be off by double rounding)
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - q)
        key = (d, int(np.float32(cand).view(np.uint32)) & 1)  # tie -> even mantissa
        if best is None or key < best[0]:
            best = (key, np.float32(cand))
    return best[1]


# ----------------------------------------------------------------------------- NF4

def test_nf4_structure(orc):
    t = orc.nf4_table()
    assert t.dtype == np.float32 and t.size == 16
    assert np.all(np.diff(t) > 0), "strictly increasing"
    assert t[0] == -1.0 and t[7] == 0.0 and t[15] == 1.0
    assert (t < 0).sum() == 7 and (t > 0).sum() == 8


def test_nf4_ppf_matches_libraries(orc):
    # the oracle's own inverse normal CDF against two independent implementations
    for p in np.linspace(0.5, 0.99, 50):
        a = orc.norm_ppf(p)
        assert abs(a - norm.ppf(p)) <= 4e-15 * max(1.0, abs(a))
        assert abs(a - statistics.NormalDist().inv_cdf(p)) <= 1e-13


def test_nf4_values_match_scipy_construction(orc):
    # Same construction evaluated with scipy's quantile function, rounded to fp32.
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    top = norm.ppf(delta)
    pos = [norm.ppf(delta + (0.5 - delta) * k / 8) / top for k in range(8)]
    neg = [-norm.ppf(delta + (0.5 - delta) * k / 7) / top for k in range(7)]
    ref = np.array(sorted(pos + [0.0] + neg), dtype=np.float32)
    np.testing.assert_array_equal(orc.nf4_table().view(np.uint32), ref.view(np.uint32))


def test_nf4_is_normal_quantile_grid(orc):
    # Each positive code is the normalised N(0,1) quantile at an equally spaced
    # probability between 1/2 and delta: Phi(c * Phi^-1(delta)) is linear in the index.
    t64 = orc.nf4_table(f64=True)
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    top = norm.ppf(delta)
    pos = norm.cdf(t64[8:] * top)          # 8 positive codes, ascending
    neg = norm.cdf(-t64[:7] * top)         # 7 negative codes, as positive quantiles
    np.testing.assert_allclose(np.diff(pos), np.full(7, (delta - 0.5) / 8), rtol=1e-9)
    np.testing.assert_allclose(np.diff(neg[::-1]), np.full(6, (delta - 0.5) / 7), rtol=1e-9)


# ----------------------------------------------------------------------------- dynamic8

def _dyn8_from_bit_layout():
    """Decode every 8-bit code of the signed dynamic tree from its bit layout:
    bit 7 = sign; in the remaining 7 bits the count of leading zeros E is the
    decimal exponent, the first 1 is an indicator, and the bits after it are a
    linear fraction f of width w = 6 - E naming the bucket midpoint
    0.1 + 0.9 (f + 1/2) / 2^w of [0.1, 1]; value = sign * 10^-E * that. The
    all-zero 7-bit pattern is the special pair {0, +1}."""
    vals = set()
    for code in range(256):
        sign = -1 if code & 0x80 else 1
        rest = code & 0x7F
        if rest == 0:
            vals.add(Fraction(0) if sign > 0 else Fraction(1))
            continue
        E = 7 - rest.bit_length()           # leading zeros within 7 bits
        w = 6 - E                           # fraction bits after the indicator
        f = rest & ((1 << w) - 1)
        mid = Fraction(1, 10) + Fraction(9, 10) * (Fraction(f) + Fraction(1, 2)) / (1 << w)
        vals.add(sign * mid / (10 ** E))
    return sorted(vals)


def test_dyn8_exact_against_bit_layout(orc):
    exact = _dyn8_from_bit_layout()
    assert len(exact) == 256
    ref = np.array([_nearest_f32_of_fraction(q) for q in exact], dtype=np.float32)
    np.testing.assert_array_equal(orc.dyn8_table().view(np.uint32), ref.view(np.uint32))


def test_dyn8_structure(orc):
    d = orc.dyn8_table()
    assert d.size == 256 and np.all(np.diff(d) > 0)
    assert d[127] == 0.0 and d[255] == 1.0
    assert d[0] == np.float32(-0.99296875)
    assert d[128] == np.float32(5.5e-7)
    assert (d < 0).sum() == 127 and (d > 0).sum() == 128


# ----------------------------------------------------------------------------- thresholds

@pytest.mark.parametrize("which", ["nf4", "dyn8"])
def test_thresholds_round_down_exact_midpoints(orc, which):
    t = orc.nf4_table() if which == "nf4" else orc.dyn8_table()
    thr = orc.thresholds(t)
    for k in range(t.size - 1):
        mid = (Fraction(float(t[k])) + Fraction(float(t[k + 1]))) / 2
        lo = Fraction(float(thr[k]))
        hi = Fraction(float(np.nextafter(thr[k], np.float32(np.inf))))
        assert lo <= mid < hi, (k, float(thr[k]))


# ----------------------------------------------------------------------------- encoder

@pytest.fixture(scope="module")
def brute(tmp_path_factory):
    src = os.path.join(HERE, "helpers", "encoder_bruteforce.c")
    so = str(tmp_path_factory.mktemp("bf") / "bf.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", src, "-o", so, "-lm"], check=True)
    lib = ctypes.CDLL(so)
    P = ctypes.c_void_p
    lib.brute_check.restype = ctypes.c_int64
    lib.brute_check.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32,
                                ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_uint32)]
    return lib


def _run_brute(orc, brute, table, mode, stride, window):
    lib = orc._load()
    thr = orc.thresholds(table)
    P = ctypes.c_void_p
    visited = ctypes.c_int64()
    first_bad = ctypes.c_uint32()
    bad = brute.brute_check(ctypes.cast(lib.orc_encode_array, P), thr.ctypes.data_as(P),
                            table.ctypes.data_as(P), table.size, mode, stride, window,
                            ctypes.byref(visited), ctypes.byref(first_bad))
    return bad, visited.value, first_bad.value


def test_nf4_encoder_exhaustive(orc, brute):
    """Every fp32 in [-1, 1] (2,130,706,434 inputs): the threshold encoder equals
    the brute-force argmin over the 16 codes with ties to the lower index."""
    bad, visited, first = _run_brute(orc, brute, orc.nf4_table(), mode=0, stride=1, window=0)
    assert visited == 2 * (0x3F800000 + 1)
    assert bad == 0, hex(first)


def test_dyn8_encoder_sweep(orc, brute):
    """dynamic8 encoder against a bracketing search on the code values: every
    29th fp32 in [-1, 1] plus every input within 4096 ulps of each midpoint."""
    bad, visited, first = _run_brute(orc, brute, orc.dyn8_table(), mode=1, stride=29, window=4096)
    assert visited > 7.0e7
    assert bad == 0, hex(first)


def test_encoder_ties_go_low(orc):
    t = orc.nf4_table()
    thr = orc.thresholds(t)
    # an exact midpoint that is representable in fp32: between C4[6] and 0
    mid = np.float32(t[6] / 2)
    assert Fraction(float(mid)) == (Fraction(float(t[6])) + 0) / 2
    assert orc.encode(thr, np.array([mid]))[0] == 6
    assert orc.encode(thr, np.array([np.nextafter(mid, np.float32(1))]))[0] == 7
    # every code value encodes to itself
    np.testing.assert_array_equal(orc.encode(thr, t), np.arange(16))
    d = orc.dyn8_table()
    np.testing.assert_array_equal(orc.encode(orc.thresholds(d), d), np.arange(256))
