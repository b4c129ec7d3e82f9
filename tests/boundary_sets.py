"""Weight sets placed on the quantizer's decision boundaries (test inputs only).

Both sets are fp32 host arrays built from the two code tables; the CPU tests
check that the oracle codes them by exact nearest search with true division,
and the GPU tests that nf4_quantize packs them bit for bit like the oracle.
The format they probe: Aner docs "Native model adaptation and NF4", section
"Packed NF4 and the portable QLoRA profile" (nearest NF4 code of w / absmax;
block maxima centred by their mean and coded with dynamic8 in blocks of 256).
"""
import numpy as np


def nf4_division_boundary(c4: np.ndarray, seed: int = 123, scales: int = 400):
    """Blocks whose elements sit within a few ulps of the midpoints between
    adjacent NF4 codes, kept only where w * fl32(1/a) and the correctly rounded
    w / a pick different nearest codes. Returns (weights, disagreements)."""
    c4 = np.asarray(c4, np.float64)
    mids = (c4[:-1] + c4[1:]) / 2
    rng = np.random.default_rng(seed)
    blocks_out, disagreements = [], 0
    for a in rng.uniform(0.01, 0.1, scales).astype(np.float32):
        cand = []
        for mid in mids:
            w0 = np.float32(mid * float(a))
            for d in range(-6, 7):
                w = np.float32(w0)
                for _ in range(abs(d)):
                    w = np.nextafter(w, np.float32(np.inf if d > 0 else -np.inf))
                if abs(w) < a:
                    cand.append(w)
        cand = np.array(cand, np.float32)
        x_div = (cand / a).astype(np.float32)
        x_rcp = (cand * np.float32(np.float32(1) / a)).astype(np.float32)
        code_div = np.argmin(np.abs(x_div[:, None].astype(np.float64) - c4[None, :]), axis=1)
        code_rcp = np.argmin(np.abs(x_rcp[:, None].astype(np.float64) - c4[None, :]), axis=1)
        pick = cand[code_div != code_rcp][:63]
        disagreements += pick.size
        if pick.size:
            blk = np.zeros(64, np.float32)
            blk[0] = a
            blk[1:1 + pick.size] = pick
            blocks_out.append(blk)
    return np.concatenate(blocks_out), disagreements


def dyn8_midpoint_maxima(d8: np.ndarray, seed: int = 5, groups: int = 24):
    """Blocks whose maxima, once centred, divide by their nested maximum to
    within a few ulps of the midpoints between adjacent dynamic8 codes.

    The maxima come in pairs mu0 +- d around mu0 = 2^-4, with every d a
    multiple of 2^-27 and |d| <= m < 2^-6, so each maximum is an fp32 number,
    any fixed-order sum of them is exact in fp64 and the matrix mean is mu0
    exactly; the centred maxima are then exactly +-d. Each of `groups` values
    of m (multiples of 2^-27, not powers of two, so d / m is rounded) gets its
    own nested blocks, every one of which holds the pair mu0 +- m, so its
    nested maximum is exactly m. Each block holds its maximum first and seeded
    values of smaller magnitude after it. Returns (weights, mu0, nested maxima
    per nested block, rcp_disagreements), the last counting centred maxima
    whose dynamic8 code under d * fl32(1/m) differs from the one under the
    correctly rounded d / m.
    """
    d8 = np.asarray(d8, np.float64)
    q = 2.0 ** -27
    mu0 = 2.0 ** -4
    mids = (d8[:-1] + d8[1:]) / 2
    rng = np.random.default_rng(seed)
    maxima, nested, disagreements = [], [], 0
    for m_target in rng.uniform(0.008, 0.0155, groups):
        m = round(m_target / q) * q
        cands = []
        for t in mids:
            d0 = round(t * m / q)
            if abs(d0) < 64:  # too close to zero for the 2^-27 grid to resolve the midpoint
                continue
            for dd in range(-2, 3):
                d = (d0 + dd) * q
                if 0 < abs(d) < m:
                    cands.append(d)
        cands = np.array(sorted(set(cands)), np.float64)
        d32 = cands.astype(np.float32)
        m32 = np.float32(m)
        x_div = (d32 / m32).astype(np.float32).astype(np.float64)
        x_rcp = (d32 * (np.float32(1) / m32)).astype(np.float32).astype(np.float64)
        c_div = np.argmin(np.abs(x_div[:, None] - d8[None, :]), axis=1)
        c_rcp = np.argmin(np.abs(x_rcp[:, None] - d8[None, :]), axis=1)
        disagreements += int(np.count_nonzero(c_div != c_rcp))
        # nested blocks of 256 maxima: the pair mu0 +- m, then 127 pairs mu0 +- d
        # (the last nested block of a group is filled up with more mu0 +- m pairs)
        per = 127
        for j in range(0, cands.size, per):
            grp = list(cands[j:j + per])
            grp += [m] * (per - len(grp))
            maxima += [mu0 + m, mu0 - m]
            for d in grp:
                maxima += [mu0 + d, mu0 - d]
            nested.append(m)
    maxima = np.array(maxima, np.float64)
    assert np.all(maxima.astype(np.float32).astype(np.float64) == maxima)  # every maximum is an fp32 number
    w = rng.uniform(-0.9, 0.9, (maxima.size, 64)).astype(np.float32) * maxima[:, None].astype(np.float32)
    sign = np.where(rng.random(maxima.size) < 0.5, -1.0, 1.0).astype(np.float32)
    w[:, 0] = sign * maxima.astype(np.float32)
    return w.ravel(), np.float32(mu0), np.array(nested, np.float32), disagreements
