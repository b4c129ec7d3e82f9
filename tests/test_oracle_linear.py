"""Pins of the oracle's linear layer, input gradient and LoRA gradients.

The layer is y = x W^T + s (x A^T) B^T (Aner docs, "Adapter API" and "LoRA FA
includes gradient preconditioning": s = alpha / rank; rsLoRA uses alpha /
sqrt(rank)); the input gradient runs through the frozen base (section "Packed
NF4 and the portable QLoRA profile"). Checks: brute force with exactly rounded
sums on tiny shapes, numpy fp64 matmul, torch fp64 autograd of <dY, y>, the
adjoint identity, and the degenerate cases B = 0 and A = 0 (Soup gate results,
"What the gate caught": with B = 0 the adapter path is inert and dL/dA is zero).
"""
import math

import numpy as np
import pytest
import torch


def _rand(shape, std, seed):
    return (np.random.default_rng(seed).standard_normal(shape) * std).astype(np.float32)


def _problem(M, K, N, r, seed=0):
    x = _rand((M, K), 1.0, seed)
    W = _rand((N, K), 0.02, seed + 1)
    A = _rand((r, K), 1.0 / r, seed + 2) if r else None
    B = _rand((N, r), 0.01, seed + 3) if r else None
    dy = _rand((M, N), 1.0, seed + 4)
    return x, W, A, B, dy


def test_bruteforce_tiny(orc):
    M, K, N, r, s = 3, 5, 4, 2, np.float32(1.5)
    x, W, A, B, dy = _problem(M, K, N, r, seed=1)
    y, T = orc.linear_fwd(x, W, A, B, s)
    dx, U = orc.linear_bwd_input(dy, W, A, B, s)
    for m in range(M):
        for rho in range(r):
            t = math.fsum(float(x[m, k]) * float(A[rho, k]) for k in range(K))
            assert abs(T[m, rho] - t) <= 1e-14 * (1 + abs(t))
        for n in range(N):
            base = math.fsum(float(x[m, k]) * float(W[n, k]) for k in range(K))
            lora = math.fsum(T[m, rho] * float(B[n, rho]) for rho in range(r))
            want = base + float(s) * lora
            assert abs(y[m, n] - want) <= 1e-14 * (1 + abs(want))
        for k in range(K):
            base = math.fsum(float(dy[m, n]) * float(W[n, k]) for n in range(N))
            u = [math.fsum(float(dy[m, n]) * float(B[n, rho]) for n in range(N)) for rho in range(r)]
            want = base + float(s) * math.fsum(u[rho] * float(A[rho, k]) for rho in range(r))
            assert abs(dx[m, k] - want) <= 1e-14 * (1 + abs(want))


@pytest.mark.parametrize("M,K,N,r", [(17, 70, 33, 4), (64, 128, 96, 16), (5, 64, 7, 1)])
def test_against_numpy(orc, M, K, N, r):
    s = np.float32(2.0)
    x, W, A, B, dy = _problem(M, K, N, r, seed=M)
    xd, Wd, Ad, Bd, dyd = (v.astype(np.float64) for v in (x, W, A, B, dy))
    y, T = orc.linear_fwd(x, W, A, B, s)
    np.testing.assert_allclose(T, xd @ Ad.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, xd @ Wd.T + 2.0 * (xd @ Ad.T) @ Bd.T, rtol=1e-12, atol=1e-12)
    dx, U = orc.linear_bwd_input(dy, W, A, B, s)
    np.testing.assert_allclose(U, dyd @ Bd, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx, dyd @ Wd + 2.0 * (dyd @ Bd) @ Ad, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("rslora", [False, True])
def test_gradients_match_torch_autograd(orc, rslora):
    M, K, N, r = 24, 80, 40, 8
    alpha = 16.0
    s = orc.lora_scale(alpha, r, rslora)
    assert s == (np.float32(16 / math.sqrt(8)) if rslora else np.float32(2.0))
    x, W, A, B, dy = _problem(M, K, N, r, seed=5)
    y, T = orc.linear_fwd(x, W, A, B, s)
    dx, U = orc.linear_bwd_input(dy, W, A, B, s)
    dA, dB = orc.lora_grad(x, dy, T, U, s)
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tA = torch.tensor(A, dtype=torch.float64, requires_grad=True)
    tB = torch.tensor(B, dtype=torch.float64, requires_grad=True)
    tW = torch.tensor(W, dtype=torch.float64)
    ty = tx @ tW.T + float(s) * (tx @ tA.T) @ tB.T
    (ty * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dA, tA.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dB, tB.grad.numpy(), rtol=1e-11, atol=1e-12)
    # LoRA-FA: A frozen, only dB, and it is the same dB
    dA_fa, dB_fa = orc.lora_grad(x, dy, T, None, s, fa=True)
    assert dA_fa is None
    np.testing.assert_array_equal(dB_fa, dB)
    # the rank-r side products on their own are the same T and U
    np.testing.assert_allclose(orc.lora_down(x, A), T, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(orc.lora_up_grad(dy, B), U, rtol=1e-12, atol=1e-13)


def test_adjoint_identity(orc):
    M, K, N, r = 16, 96, 48, 4
    x, W, A, B, dy = _problem(M, K, N, r, seed=9)
    y, _ = orc.linear_fwd(x, W, A, B, 0.75)
    dx, _ = orc.linear_bwd_input(dy, W, A, B, 0.75)
    lhs = math.fsum((y * dy.astype(np.float64)).ravel())
    rhs = math.fsum((dx * x.astype(np.float64)).ravel())
    assert abs(lhs - rhs) <= 1e-11 * (abs(lhs) + 1)


def test_zero_B_is_inert(orc):
    M, K, N, r = 12, 64, 20, 4
    x, W, A, B, dy = _problem(M, K, N, r, seed=13)
    B0 = np.zeros_like(B)
    y_lora, T = orc.linear_fwd(x, W, A, B0, 2.0)
    y_base, _ = orc.linear_fwd(x, W)
    np.testing.assert_array_equal(y_lora, y_base)
    dx, U = orc.linear_bwd_input(dy, W, A, B0, 2.0)
    dA, dB = orc.lora_grad(x, dy, T, U, 2.0)
    assert np.all(dA == 0)
    assert np.any(dB != 0)


def test_zero_A_gives_zero_dB(orc):
    M, K, N, r = 12, 64, 20, 4
    x, W, A, B, dy = _problem(M, K, N, r, seed=17)
    A0 = np.zeros_like(A)
    y, T = orc.linear_fwd(x, W, A0, B, 2.0)
    assert np.all(T == 0)
    dx, U = orc.linear_bwd_input(dy, W, A0, B, 2.0)
    dA, dB = orc.lora_grad(x, dy, T, U, 2.0)
    assert np.all(dB == 0) and np.any(dA != 0)
