"""Pins of the decoder-layer oracle (oracle/llama.py): closed forms, invariants
and PyTorch's own fp64 implementations of the same standard definitions
(RMSNorm, rotary embedding, causal grouped-query attention, SwiGLU,
cross-entropy), with input gradients against torch autograd in fp64."""
import math

import numpy as np
import pytest
import torch

from oracle import llama as L

EPS64 = np.finfo(np.float64).eps


def _t(a):
    return torch.tensor(np.asarray(a, np.float64), requires_grad=True)


# --------------------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_forms():
    gamma = np.linspace(0.5, 2.0, 8)
    y, rstd = L.rmsnorm(np.full((1, 8), -3.0), gamma, 0.0)
    np.testing.assert_allclose(y[0], -gamma, rtol=4 * EPS64)       # constant row -> -gamma
    x = np.random.default_rng(0).standard_normal((5, 64))
    y1, _ = L.rmsnorm(x, np.ones(64), 0.0)
    y2, _ = L.rmsnorm(7.5 * x, np.ones(64), 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)                  # scale invariance without eps
    np.testing.assert_allclose(np.mean(y1 * y1, axis=1), 1.0, rtol=1e-13)  # unit RMS


def test_rmsnorm_against_torch():
    rng = np.random.default_rng(1)
    x, gamma, dy = rng.standard_normal((6, 96)), rng.standard_normal(96), rng.standard_normal((6, 96))
    eps = float(np.float32(1e-5))
    xt = _t(x)
    yt = torch.nn.functional.rms_norm(xt, (96,), torch.tensor(gamma), eps=eps)
    yt.backward(torch.tensor(dy))
    y, _ = L.rmsnorm(x, gamma, 1e-5)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L.rmsnorm_bwd(dy, x, gamma, 1e-5), xt.grad.numpy(), rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------- rotary embedding

def test_rope_position_zero_and_norms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, 2 * 64))
    y = L.rope(x, 2, 64, 500000.0)
    np.testing.assert_allclose(y[0], x[0], rtol=0, atol=0)        # position 0: no rotation
    h = 32
    for hd in range(2):
        a, b = x[:, hd * 64:hd * 64 + h], x[:, hd * 64 + h:(hd + 1) * 64]
        c, e = y[:, hd * 64:hd * 64 + h], y[:, hd * 64 + h:(hd + 1) * 64]
        np.testing.assert_allclose(c * c + e * e, a * a + b * b, rtol=1e-12)  # each pair keeps its length
    np.testing.assert_allclose(L.rope(y, 2, 64, 500000.0, inverse=True), x, rtol=1e-12, atol=1e-12)


def test_rope_two_dims_is_a_rotation_by_position():
    """d = 2: the single pair rotates by pos * theta^0 = pos radians."""
    S = 7
    x = np.tile([[1.0, 0.0]], (S, 1))
    y = L.rope(x, 1, 2, 10000.0)
    pos = np.arange(S)
    np.testing.assert_allclose(y, np.stack([np.cos(pos), np.sin(pos)], axis=1), rtol=1e-13, atol=1e-15)


def test_rope_scores_depend_on_relative_position():
    """q_m . k_n after rotation depends only on m - n."""
    rng = np.random.default_rng(3)
    d = 16
    q1, k1 = rng.standard_normal(d), rng.standard_normal(d)
    Q = np.tile(q1, (12, 1))
    K = np.tile(k1, (12, 1))
    rq, rk = L.rope(Q, 1, d, 10000.0), L.rope(K, 1, d, 10000.0)
    for m, n in [(5, 2), (9, 6), (11, 8)]:
        assert abs(rq[m] @ rk[n] - rq[3] @ rk[0]) < 1e-12


# --------------------------------------------------------------------------- attention

def test_attention_special_cases():
    rng = np.random.default_rng(4)
    S, d = 9, 8
    v = rng.standard_normal((S, d))
    k = rng.standard_normal((S, d))
    o, _ = L.attention(np.zeros((S, d)), k, v, 1, 1, d)            # equal scores: prefix means
    np.testing.assert_allclose(o, np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None], rtol=1e-13)
    o1, lse = L.attention(rng.standard_normal((1, d)), k[:1], v[:1], 1, 1, d)   # one position: o = v
    np.testing.assert_allclose(o1, v[:1], rtol=1e-15)


@pytest.mark.parametrize("S,hq,hkv,d", [(17, 4, 2, 16), (33, 8, 2, 32)])
def test_attention_against_torch(S, hq, hkv, d):
    rng = np.random.default_rng(S)
    q, k, v = rng.standard_normal((S, hq * d)), rng.standard_normal((S, hkv * d)), rng.standard_normal((S, hkv * d))
    do = rng.standard_normal((S, hq * d))
    qt, kt, vt = _t(q), _t(k), _t(v)
    grp = hq // hkv
    Q = qt.view(S, hq, d).transpose(0, 1)
    Kr = kt.view(S, hkv, d).transpose(0, 1).repeat_interleave(grp, dim=0)
    Vr = vt.view(S, hkv, d).transpose(0, 1).repeat_interleave(grp, dim=0)
    ot = torch.nn.functional.scaled_dot_product_attention(Q, Kr, Vr, is_causal=True)
    ot = ot.transpose(0, 1).reshape(S, hq * d)
    ot.backward(torch.tensor(do))
    o, lse = L.attention(q, k, v, hq, hkv, d)
    np.testing.assert_allclose(o, ot.detach().numpy(), rtol=1e-10, atol=1e-12)
    dq, dk, dv = L.attention_bwd(do, q, k, v, hq, hkv, d)
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=1e-9, atol=1e-11)
    # lse: log of the softmax denominator of each (head, row)
    s0 = (q[:, :d] @ k[:, :d].T) / math.sqrt(d)
    row = 5
    assert abs(lse[0, row] - math.log(np.sum(np.exp(s0[row, :row + 1])))) < 1e-12


# --------------------------------------------------------------------------- SwiGLU and cross-entropy

def test_swiglu_values_and_gradient():
    np.testing.assert_allclose(L.silu([0.0, 40.0, -40.0]), [0.0, 40.0, -40.0 / (1 + math.exp(40.0))], rtol=1e-14)
    rng = np.random.default_rng(5)
    g, u, da = rng.standard_normal((4, 50)) * 3, rng.standard_normal((4, 50)), rng.standard_normal((4, 50))
    gt, ut = _t(g), _t(u)
    at = torch.nn.functional.silu(gt) * ut
    at.backward(torch.tensor(da))
    np.testing.assert_allclose(L.swiglu(g, u), at.detach().numpy(), rtol=1e-13)
    dg, du = L.swiglu_bwd(da, g, u)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(du, ut.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_cross_entropy():
    V, T = 1000, 6
    loss, grad = L.cross_entropy(np.zeros((T, V)), np.arange(T))
    assert abs(loss - math.log(V)) < 1e-12                          # uniform logits
    np.testing.assert_allclose(grad.sum(axis=1), 0.0, atol=1e-15)
    rng = np.random.default_rng(6)
    z, t = rng.standard_normal((T, V)) * 4, rng.integers(0, V, T)
    zt = _t(z)
    lt = torch.nn.functional.cross_entropy(zt, torch.tensor(t))
    lt.backward()
    loss, grad = L.cross_entropy(z, t)
    assert abs(loss - lt.item()) < 1e-12
    np.testing.assert_allclose(grad, zt.grad.numpy(), rtol=1e-11, atol=1e-15)


# --------------------------------------------------------------------------- the assembled layer

def _torch_rope(x, heads, d, theta):
    """Half-split rotation, built from torch.polar (a complex phase per pair)."""
    S = x.shape[0]
    pos = torch.arange(S, dtype=torch.float64)[:, None]
    inv = torch.tensor(theta, dtype=torch.float64) ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    rot = torch.polar(torch.ones(S, d // 2, dtype=torch.float64), pos * inv[None, :])
    xh = x.view(S, heads, 2, d // 2)
    z = torch.complex(xh[:, :, 0], xh[:, :, 1]) * rot[:, None, :]
    return torch.stack((z.real, z.imag), dim=2).reshape(S, heads * d)


@pytest.mark.parametrize("targets", [("q_proj", "v_proj"),
                                     ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")])
def test_decoder_layer_against_torch_autograd(orc, targets):
    """The oracle's layer (fp64 between the linears, fp32 linear inputs) against
    the same pre-norm Llama layer written with torch library routines
    (rms_norm, scaled_dot_product_attention, silu) and differentiated by
    autograd: output, input gradient and every adapter's dA, dB. Catches a
    missing residual, a wrong operand in an adapter gradient or a head
    mapping error."""
    S, D, H, Hkv, d, F_, r = 11, 32, 4, 2, 8, 48, 3
    rng = np.random.default_rng(21)
    f32 = lambda *sh, std=1.0: (rng.standard_normal(sh) * std).astype(np.float32)
    names = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")
    shapes = dict(q_proj=(H * d, D), k_proj=(Hkv * d, D), v_proj=(Hkv * d, D), o_proj=(D, H * d),
                  gate_proj=(F_, D), up_proj=(F_, D), down_proj=(D, F_))
    p = {"W_" + n: f32(*shapes[n], std=0.3) for n in names}
    for n in targets:
        p["A_" + n], p["B_" + n] = f32(r, shapes[n][1], std=0.3), f32(shapes[n][0], r, std=0.3)
    p["gamma1"], p["gamma2"] = 1 + f32(D, std=0.2), 1 + f32(D, std=0.2)
    s, eps, theta = 0.75, 1e-5, 10000.0
    cfg = dict(heads=H, kv_heads=Hkv, head_dim=d, eps=eps, theta=theta, s=s, targets=targets)
    xin, res, dx3 = f32(S, D), f32(S, D), f32(S, D)
    ref = L.decoder_layer(p, xin, res, dx3, cfg, bf16=False)

    T = {k: torch.tensor(v, dtype=torch.float64, requires_grad=k.startswith(("A_", "B_"))) for k, v in p.items()}
    tx = torch.tensor(xin, dtype=torch.float64, requires_grad=True)
    fn = torch.nn.functional

    def lin(n, a):
        y = a @ T["W_" + n].T
        return y + s * (a @ T["A_" + n].T) @ T["B_" + n].T if n in targets else y

    x = tx + torch.tensor(res, dtype=torch.float64)
    h1 = fn.rms_norm(x, (D,), T["gamma1"], eps=eps)
    q = _torch_rope(lin("q_proj", h1), H, d, theta).view(S, H, d).transpose(0, 1)
    k = _torch_rope(lin("k_proj", h1), Hkv, d, theta).view(S, Hkv, d).transpose(0, 1)
    v = lin("v_proj", h1).view(S, Hkv, d).transpose(0, 1)
    k, v = k.repeat_interleave(H // Hkv, 0), v.repeat_interleave(H // Hkv, 0)
    a = fn.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True)[0]
    x2 = x + lin("o_proj", a.transpose(0, 1).reshape(S, H * d))
    h2 = fn.rms_norm(x2, (D,), T["gamma2"], eps=eps)
    out = x2 + lin("down_proj", fn.silu(lin("gate_proj", h2)) * lin("up_proj", h2))
    out.backward(torch.tensor(dx3, dtype=torch.float64))
    # fp32 inputs of every linear on the oracle side bound the agreement
    tol = dict(rtol=2e-5, atol=2e-5)
    np.testing.assert_allclose(ref["out"], out.detach().numpy(), **tol)
    np.testing.assert_allclose(ref["x2"], x2.detach().numpy(), **tol)
    np.testing.assert_allclose(ref["dx"], tx.grad.numpy(), **tol)
    for n in targets:
        dA, dB = ref["grads"][n]
        gA, gB = T["A_" + n].grad.numpy(), T["B_" + n].grad.numpy()
        np.testing.assert_allclose(dA, gA, rtol=2e-5, atol=2e-5 * np.abs(gA).max())
        np.testing.assert_allclose(dB, gB, rtol=2e-5, atol=2e-5 * np.abs(gB).max())
