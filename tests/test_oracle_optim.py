"""Pins of the oracle's optimizer step: the LoRA-FA preconditioner
pinv(A A^T + 1e-8 I), the preconditioned gradient s^-2 g_B P and AdamW.

Aner docs "Native model adaptation and NF4", section "LoRA FA includes gradient
preconditioning" defines the preconditioner; AdamW follows its published
definition (decoupled weight decay, bias-corrected moments). Each pin below
checks the oracle against something other than itself: closed forms, exact
rational arithmetic, the Moore-Penrose conditions and PyTorch's own AdamW."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

EPS64 = np.finfo(np.float64).eps
DAMP = 1e-8


def hadamard(n: int) -> np.ndarray:
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


# --------------------------------------------------------------------------- preconditioner

def test_orthogonal_rows_give_scaled_identity(orc):
    """Rows of a Hadamard matrix are orthogonal: A A^T = c^2 K I exactly, so
    P = I / (c^2 K + 1e-8)."""
    for r, K, c in [(16, 64, 0.125), (4, 256, 0.5), (1, 8, 1.0), (64, 64, 2.0 ** -3)]:
        A = (c * hadamard(K)[:r]).astype(np.float32)
        P = orc.lorafa_preconditioner(A)
        want = np.eye(r) / (c * c * K + DAMP)
        np.testing.assert_allclose(P, want, rtol=8 * EPS64, atol=8 * EPS64 * want.max())


def test_rank_one(orc):
    rng = np.random.default_rng(11)
    a = rng.standard_normal((1, 300)).astype(np.float32)
    n2 = math.fsum(float(x) * float(x) for x in a[0])  # fp32 squares are exact in fp64
    P = orc.lorafa_preconditioner(a)
    assert P.shape == (1, 1)
    assert abs(P[0, 0] - 1.0 / (n2 + DAMP)) <= 4 * EPS64 / n2


def test_zero_adapter_is_pure_damping(orc):
    P = orc.lorafa_preconditioner(np.zeros((5, 33), np.float32))
    np.testing.assert_allclose(P, np.eye(5) * 1e8, rtol=4 * EPS64)


def test_duplicate_rows_keep_the_damped_direction(orc):
    """Two equal rows: A A^T = a [[1,1],[1,1]] is singular and only the damping
    makes it invertible; the inverse is [[a+e, -a], [-a, a+e]] / (e (2a + e)).
    A singular-value cutoff would lose the 1/e direction and fail here."""
    rng = np.random.default_rng(5)
    row = rng.standard_normal(40).astype(np.float32)
    a = math.fsum(float(x) * float(x) for x in row)
    P = orc.lorafa_preconditioner(np.stack([row, row]))
    e = DAMP
    want = np.array([[a + e, -a], [-a, a + e]]) / (e * (2 * a + e))
    kappa = (2 * a + e) / e
    assert np.abs(P - want).max() <= 16 * kappa * EPS64 * np.abs(want).max()
    assert np.abs(P).max() > 1e7


def test_disjoint_supports_give_diagonal(orc):
    """Rows supported on disjoint columns: A A^T is diagonal with the squared
    row norms, so P is diagonal with 1 / (norm_i^2 + 1e-8) in row order."""
    rng = np.random.default_rng(3)
    r, w = 6, 7
    A = np.zeros((r, r * w), np.float32)
    for i in range(r):
        A[i, i * w:(i + 1) * w] = rng.standard_normal(w) * (i + 1)
    P = orc.lorafa_preconditioner(A)
    n2 = [math.fsum(float(x) ** 2 for x in A[i]) for i in range(r)]
    np.testing.assert_allclose(np.diag(P), [1.0 / (n + DAMP) for n in n2], rtol=8 * EPS64)
    assert np.abs(P - np.diag(np.diag(P))).max() <= 8 * EPS64 * np.abs(P).max()


def _exact_inverse(A: np.ndarray):
    """Brute force: (A A^T + 1e-8 I)^-1 by Gauss-Jordan in exact rationals.
    The damping is the double nearest to 1e-8, taken exactly."""
    r, K = A.shape
    F = [[Fraction(float(x)) for x in row] for row in A]
    d = Fraction(DAMP)
    G = [[sum(F[i][k] * F[j][k] for k in range(K)) + (d if i == j else 0) for j in range(r)] for i in range(r)]
    aug = [G[i] + [Fraction(int(i == j)) for j in range(r)] for i in range(r)]
    for c in range(r):
        piv = next(i for i in range(c, r) if aug[i][c] != 0)
        aug[c], aug[piv] = aug[piv], aug[c]
        pv = aug[c][c]
        aug[c] = [x / pv for x in aug[c]]
        for i in range(r):
            if i != c and aug[i][c] != 0:
                f = aug[i][c]
                aug[i] = [x - f * y for x, y in zip(aug[i], aug[c])]
    return np.array([[float(x) for x in row[r:]] for row in aug])


@pytest.mark.parametrize("r,K,seed", [(2, 5, 1), (3, 7, 2), (4, 4, 3), (5, 3, 4)])
def test_matches_exact_rational_inverse(orc, r, K, seed):
    """Small dyadic-valued A (rank-deficient when K < r) against the exact
    rational inverse."""
    rng = np.random.default_rng(seed)
    A = (rng.integers(-8, 9, size=(r, K)) / 4.0).astype(np.float32)
    want = _exact_inverse(A)
    P = orc.lorafa_preconditioner(A)
    ev = np.linalg.eigvalsh(A.astype(np.float64) @ A.T.astype(np.float64) + DAMP * np.eye(r))
    kappa = ev.max() / ev.min()
    assert np.abs(P - want).max() <= 32 * r * kappa * EPS64 * np.abs(want).max()


@pytest.mark.parametrize("r,K,rank", [(16, 4096, 16), (8, 300, 4), (64, 1024, 64)])
def test_moore_penrose_conditions(orc, r, K, rank):
    """G P G = G, P G P = P and G P, P G symmetric: the four conditions that
    define the pseudo-inverse, for full-rank and rank-deficient A."""
    rng = np.random.default_rng(r + rank)
    A = (rng.standard_normal((r, rank)) @ rng.standard_normal((rank, K)) / math.sqrt(K * r)).astype(np.float32)
    A64 = A.astype(np.float64)
    G = A64 @ A64.T + DAMP * np.eye(r)
    P = orc.lorafa_preconditioner(A)
    ev = np.linalg.eigvalsh(G)
    kappa = ev.max() / ev.min()
    tol = 64 * r * kappa * EPS64
    assert np.abs(G @ P @ G - G).max() <= tol * np.abs(G).max()
    assert np.abs(P @ G @ P - P).max() <= tol * np.abs(P).max()
    assert np.abs(G @ P - (G @ P).T).max() <= tol
    assert np.abs(P @ G - (P @ G).T).max() <= tol


# --------------------------------------------------------------------------- preconditioned gradient

def test_preconditioned_gradient_orthogonal_rows(orc):
    """With A A^T = c^2 K I the preconditioned gradient is g / (s^2 (c^2 K + 1e-8)):
    the scale enters squared and inverted."""
    r, K, c, s = 8, 32, 0.25, 2.0
    A = (c * hadamard(K)[:r]).astype(np.float32)
    g = np.random.default_rng(0).standard_normal((50, r)).astype(np.float32)
    got = orc.lorafa_precondition(g, orc.lorafa_preconditioner(A), s)
    want = g.astype(np.float64) / (s * s * (c * c * K + DAMP))
    np.testing.assert_allclose(got, want, rtol=16 * EPS64)


def test_preconditioner_acts_on_columns(orc):
    """Diagonal A A^T with distinct row norms: column i of g_B is divided by
    s^2 (norm_i^2 + 1e-8), so P multiplies g_B from the right."""
    r, w, s = 4, 5, 0.5
    A = np.zeros((r, r * w), np.float32)
    for i in range(r):
        A[i, i * w:(i + 1) * w] = float(i + 1)
    g = np.random.default_rng(1).standard_normal((9, r)).astype(np.float32)
    got = orc.lorafa_precondition(g, orc.lorafa_preconditioner(A), s)
    n2 = np.array([w * (i + 1) ** 2 for i in range(r)], np.float64)
    want = g.astype(np.float64) / (s * s * (n2 + DAMP))[None, :]
    np.testing.assert_allclose(got, want, rtol=16 * EPS64)


# --------------------------------------------------------------------------- AdamW

HP = dict(lr=2.0 ** -10, beta1=0.875, beta2=0.99609375, eps=2.0 ** -20, weight_decay=0.0625)  # fp32-exact


def test_adamw_matches_torch_optimizer(orc):
    """Five updates with changing gradients against torch.optim.AdamW in fp64."""
    for hp in (HP, dict(lr=float(np.float32(2e-4)), beta1=float(np.float32(0.9)), beta2=float(np.float32(0.999)),
                        eps=float(np.float32(1e-8)), weight_decay=float(np.float32(0.01)))):
        rng = np.random.default_rng(7)
        p0 = rng.standard_normal(257).astype(np.float32)
        grads = [rng.standard_normal(257).astype(np.float32) * 10.0 ** -k for k in range(5)]
        tp = torch.nn.Parameter(torch.from_numpy(p0.astype(np.float64)))
        opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                                weight_decay=hp["weight_decay"], foreach=False)
        p, m, v = p0.astype(np.float64), np.zeros(257), np.zeros(257)
        for t, g in enumerate(grads, start=1):
            tp.grad = torch.from_numpy(g.astype(np.float64))
            opt.step()
            p, m, v = orc.adamw_step(p, g, m, v, step=t, **hp)
            st = opt.state[tp]
            np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-14, atol=1e-16)
            np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-14, atol=0)
            np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-14, atol=0)


def test_adamw_constant_gradient_closed_form(orc):
    """With a constant gradient g the bias-corrected moments are exactly g and
    g^2 at every step, so p_t = q^t p_0 - lr u (1 - q^t) / (1 - q) with
    q = 1 - lr wd and u = g / (|g| + eps)."""
    lr, wd, eps = HP["lr"], HP["weight_decay"], HP["eps"]
    g = np.array([3.0, -0.5, 1e-6, -2.0 ** -20], np.float32)
    p = p0 = np.array([1.0, 2.0, -1.0, 0.0])
    m = v = np.zeros(4)
    g64 = g.astype(np.float64)
    u = g64 / (np.abs(g64) + eps)
    for t in range(1, 21):
        p, m, v = orc.adamw_step(p, g, m, v, step=t, **HP)
        one_minus_qt = -math.expm1(t * math.log1p(-lr * wd))  # 1 - q^t without cancellation
        want = (1.0 - one_minus_qt) * p0 - lr * u * one_minus_qt / (lr * wd)
        np.testing.assert_allclose(p, want, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(m / (1 - HP["beta1"] ** t), g, rtol=1e-12)
        np.testing.assert_allclose(v / (1 - HP["beta2"] ** t), g64 ** 2, rtol=1e-12)


def test_adamw_eps_outside_root(orc):
    """First step from zero moments with g = eps: m_hat = eps, sqrt(v_hat) = eps,
    so the step is lr * eps / (eps + eps) = lr / 2."""
    eps = 2.0 ** -20
    p, m, v = orc.adamw_step(np.zeros(3), np.full(3, eps, np.float32), np.zeros(3), np.zeros(3), lr=0.5,
                             beta1=0.9, beta2=0.999, eps=eps, weight_decay=0.0, step=1)
    np.testing.assert_allclose(p, -0.25, rtol=1e-12)


def test_adamw_zero_gradient_is_pure_decay(orc):
    """Decoupled decay: a zero gradient with zero moments only scales p by
    (1 - lr wd); it does not enter the moments."""
    p0 = np.array([1.5, -3.0, 0.25])
    p, m, v = orc.adamw_step(p0, np.zeros(3, np.float32), np.zeros(3), np.zeros(3), step=1, **HP)
    np.testing.assert_allclose(p, p0 * (1 - HP["lr"] * HP["weight_decay"]), rtol=1e-15)
    assert not m.any() and not v.any()


def test_adamw_grad_scale_is_a_gradient_multiplier(orc):
    rng = np.random.default_rng(2)
    p, g, m = rng.standard_normal((3, 40))
    v = rng.standard_normal(40) ** 2
    a = orc.adamw_step(p, (g * 0.375).astype(np.float32), m, v, step=3, **HP)
    b = orc.adamw_step(p, g.astype(np.float32), m, v, step=3, grad_scale=0.375, **HP)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-7)  # g rounded to fp32 in the first call


def test_lorafa_step_against_torch(orc):
    """LoRA-FA: only B moves, with the preconditioned gradient; checked against
    torch.optim.AdamW fed s^-2 (gs g_B) inv(A A^T + 1e-8 I) computed by torch's
    solver (a different routine from the oracle's pseudo-inverse)."""
    rng = np.random.default_rng(9)
    r, K, N, s, gs = 4, 96, 33, 2.0, 0.5
    A = (rng.standard_normal((r, K)) / r).astype(np.float32)
    B = (rng.standard_normal((N, r)) * 0.01).astype(np.float32)
    dBs = [rng.standard_normal((N, r)).astype(np.float32) for _ in range(3)]
    A64 = torch.from_numpy(A.astype(np.float64))
    G = A64 @ A64.T + DAMP * torch.eye(r, dtype=torch.float64)
    Pt = torch.linalg.solve(G, torch.eye(r, dtype=torch.float64))
    tp = torch.nn.Parameter(torch.from_numpy(B.astype(np.float64)))
    opt = torch.optim.AdamW([tp], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"], foreach=False)
    P = orc.lorafa_preconditioner(A)
    Bo, mB, vB = B.astype(np.float64), np.zeros((N, r)), np.zeros((N, r))
    for t, dB in enumerate(dBs, start=1):
        tp.grad = (gs * torch.from_numpy(dB.astype(np.float64))) @ Pt / (s * s)
        opt.step()
        out = orc.lora_adamw_step(Bo, dB, mB, vB, P=P, s=s, step=t, grad_scale=gs, **HP)
        Bo, mB, vB = out["B"], out["mB"], out["vB"]
        assert "A" not in out
        np.testing.assert_allclose(Bo, tp.detach().numpy(), rtol=1e-12, atol=1e-15)


def test_lora_step_updates_both_factors(orc):
    rng = np.random.default_rng(4)
    A, dA, mA = rng.standard_normal((3, 2, 10))
    B, dB, mB = rng.standard_normal((3, 10, 2))
    vA, vB = rng.standard_normal((2, 10)) ** 2, rng.standard_normal((10, 2)) ** 2
    out = orc.lora_adamw_step(B, dB, mB, vB, A=A, dA=dA, mA=mA, vA=vA, step=2, **HP)
    ra = orc.adamw_step(A, dA, mA, vA, step=2, **HP)
    rb = orc.adamw_step(B, dB, mB, vB, step=2, **HP)
    for k, ref in zip(["A", "mA", "vA", "B", "mB", "vB"], list(ra) + list(rb)):
        np.testing.assert_array_equal(out[k], ref)
    with pytest.raises(ValueError):
        orc.lora_adamw_step(B, dB, mB, vB, A=A, dA=dA, mA=mA, vA=vA, P=np.eye(2), s=1.0, step=1, **HP)
