"""Writes dq_decode_golden.json: a packed double-quantized matrix built by hand
and its decoded weights, computed here with exact rational arithmetic and one
explicit round-to-nearest-even per operation, from the oracle's code tables.

Decode rule (Aner native training accelerated qualification, key
jit.kernel_identity, "fmad-off" and "decode-separate-rn"): the block scale is
a' = fl32(fl32(D8[q] * m) + mu), the weight fl32(C4[c] * a'), bf16 by
round-to-nearest-even of that. The values of m, mu and q are chosen so that a
single rounding of D8[q] * m + mu (a fused multiply-add) gives different bits
for the first three blocks.

Usage: python tests/golden/make_dq_decode_golden.py   (from the repository root)
"""
import json
import os
import sys
from fractions import Fraction as F

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

QS = [7, 17, 32, 127, 255]   # dynamic8 codes of the five blocks
M_BITS = 0x3CCCCCCD          # fp32 nearest to 1/40 = 13421773 * 2^-29
MU = F(1, 32)


def rn(x: F, mant: int = 24, emin: int = -126) -> F:
    """Round a rational to the nearest binary float with `mant` significand bits
    (ties to even), exponent clamped at emin (gradual underflow)."""
    if x == 0:
        return F(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = F(2) ** (e - mant + 1)
    n = a / ulp
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > F(1, 2) or (rem == F(1, 2) and lo % 2 == 1):
        lo += 1
    return s * lo * ulp


def f32_bits(x: F) -> int:
    v = np.float32(float(x))
    assert F(float(v)) == x, "not an fp32 value"
    return int(v.view(np.uint32))


def bf16_bits(x32: F) -> int:
    return f32_bits(rn(x32, 8)) >> 16


def derive(c4, d8):
    m = F(float(np.uint32(M_BITS).view(np.float32)))
    blocks = []
    for q in QS:
        d = F(float(d8[q]))
        a_sep = rn(rn(d * m) + MU)
        a_fused = rn(d * m + MU)
        w = [rn(F(float(c4[c])) * a_sep) for c in range(16)]
        blocks.append(dict(q=q, a_sep=a_sep, a_fused=a_fused, w=w))
    return m, blocks


def main():
    import oracle
    c4, d8 = oracle.nf4_table(), oracle.dyn8_table()
    m, blocks = derive(c4, d8)
    codes = bytes((2 * i << 4 | (2 * i + 1)) & 0xFF for i in range(8)) * 4   # 0x01 0x23 ... 0xef per 16 elements
    out = {
        "_about": ("A hand-built double-quantized matrix of 5 blocks x 64 weights (n = 320, one nested block): "
                   "block b has dynamic8 code qabs[b], the nested maximum is m = fl32(1/40) and the offset mu = "
                   "1/32; element i of every block has NF4 code i % 16. Expected decode: a'_b = fl32(fl32(D8[q_b] m) "
                   "+ mu), w = fl32(C4[c] a'_b), bf16 = RNE(w). Blocks 0-2 are chosen so that a fused multiply-add "
                   "for a'_b (one rounding) gives different bits."),
        "_source": ("Aner native training accelerated qualification (31 Oct 2026), key jit.kernel_identity "
                    "('fmad-off', 'decode-separate-rn'); Aner docs 'Native model adaptation and NF4', section "
                    "'Packed NF4 and the portable QLoRA profile' (format). Written by "
                    "tests/golden/make_dq_decode_golden.py (exact rational arithmetic on the oracle's tables)."),
        "_derivation_block0": ("D8[7] = -229/256 and m = 13421773 * 2^-29, so D8[7] m = -3073586017 * 2^-37 "
                               "(32 significant bits); rounded to 24 bits: -12006195 * 2^-29 (the dropped part "
                               "0.378 * 2^-29 is below half an ulp). Adding mu = 16777216 * 2^-29 gives "
                               "4771021 * 2^-29 exactly, so a' = 4771021 * 2^-29 = 0.0088867191... A single "
                               "rounding of D8[7] m + mu = 1221381279 * 2^-37 gives 9542041 * 2^-30 instead, "
                               "one ulp lower."),
        "n": 320,
        "codes_hex": codes.hex() * 5,
        "qabs": QS,
        "nested_f32_bits": M_BITS,
        "offset_f32_bits": f32_bits(MU),
        "block_scale_f32_bits": [f32_bits(b["a_sep"]) for b in blocks],
        "block_scale_if_fused_f32_bits": [f32_bits(b["a_fused"]) for b in blocks],
        "expected_f32_bits": [f32_bits(b["w"][i % 16]) for b in blocks for i in range(64)],
        "expected_bf16_bits": [bf16_bits(b["w"][i % 16]) for b in blocks for i in range(64)],
    }
    with open(os.path.join(HERE, "dq_decode_golden.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
