"""CPU oracle (numpy fp64) for the operations around the NF4 linears in a
Llama-shaped decoder layer: RMSNorm, rotary position embedding, causal
grouped-query attention, the SwiGLU gate and the token cross-entropy, each with
its input gradient, and the decoder layer assembled from them.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the benchmark's ``cpu_baseline`` leg, never by the GPU product path.

Context: Soup, "NF4 Layer Streaming - Gate results", section on throughput
accounting: the measured loop is a full training step of a Llama-3.1-8B-shaped
model whose decoder layers are checkpointed (the forward runs twice, C = 6)
with a frozen NF4 base and LoRA adapters. The pages do not print the layer's
equations; these are the standard Llama definitions, written from the
mathematics (READING, each one stated in its docstring):

- RMSNorm: y = x / sqrt(mean(x^2) + eps) * gamma, gamma frozen.
- Rotary embedding in the half-split form: for i < d/2, with
  angle = pos * theta^(-2 i / d), the pair (x_i, x_{i+d/2}) is rotated by that
  angle.
- Attention: softmax((q k^T) / sqrt(d) + causal mask) v per head; query head h
  reads key/value head h // (Hq / Hkv).
- SwiGLU: a = silu(g) * u with silu(z) = z / (1 + exp(-z)).
- Cross-entropy: mean over tokens of logsumexp(logits) - logits[target].

Layouts (row-major, tokens first): q [S, Hq*d], k and v [S, Hkv*d] with head h
in columns h*d .. h*d + d - 1.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- RMSNorm

def rmsnorm(x, gamma, eps: float):
    """y = x / sqrt(mean(x^2, last axis) + eps) * gamma. Returns (y, rstd) with
    rstd = 1 / sqrt(mean(x^2) + eps) per row."""
    x = _f64(x)
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + float(np.float32(eps)))
    return x * rstd * _f64(gamma), rstd[..., 0]


def rmsnorm_bwd(dy, x, gamma, eps: float):
    """Input gradient of rmsnorm (gamma frozen): with n = x * rstd and
    g = dy * gamma, dx = rstd * (g - n * mean(g * n))."""
    x, dy = _f64(x), _f64(dy)
    _, rstd = rmsnorm(x, gamma, eps)
    rstd = rstd[..., None]
    n = x * rstd
    g = dy * _f64(gamma)
    return rstd * (g - n * np.mean(g * n, axis=-1, keepdims=True))


# --------------------------------------------------------------------------- rotary embedding

def rope_angles(S: int, d: int, theta: float) -> np.ndarray:
    """angle[pos, i] = pos * theta^(-2 i / d), i < d / 2, in fp64."""
    i = np.arange(d // 2, dtype=np.float64)
    inv = float(theta) ** (-2.0 * i / d)
    return np.arange(S, dtype=np.float64)[:, None] * inv[None, :]


def rope(x, heads: int, d: int, theta: float, inverse: bool = False):
    """Rotate every head of x [S, heads*d]: (x_i, x_{i+d/2}) -> (x_i cos - x_{i+d/2} sin,
    x_{i+d/2} cos + x_i sin). inverse=True rotates by the negative angle, which
    is the input gradient of the forward rotation (the map is orthogonal)."""
    x = _f64(x)
    S = x.shape[0]
    ang = rope_angles(S, d, theta)
    c, s = np.cos(ang), np.sin(ang)
    if inverse:
        s = -s
    out = np.empty_like(x)
    h = d // 2
    for hd in range(heads):
        a = x[:, hd * d:hd * d + h]
        b = x[:, hd * d + h:(hd + 1) * d]
        out[:, hd * d:hd * d + h] = a * c - b * s
        out[:, hd * d + h:(hd + 1) * d] = b * c + a * s
    return out


# --------------------------------------------------------------------------- attention

def attention(q, k, v, hq: int, hkv: int, d: int):
    """Causal grouped-query attention. Returns (o [S, hq*d], lse [hq, S]) with
    lse the natural log of the softmax denominator of each query row (scores
    scaled by 1/sqrt(d))."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    S = q.shape[0]
    grp = hq // hkv
    o = np.zeros((S, hq * d))
    lse = np.zeros((hq, S))
    mask = np.tril(np.ones((S, S), dtype=bool))
    for h in range(hq):
        kh = h // grp
        qh, kk, vv = q[:, h * d:(h + 1) * d], k[:, kh * d:(kh + 1) * d], v[:, kh * d:(kh + 1) * d]
        s = (qh @ kk.T) / np.sqrt(d)
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        o[:, h * d:(h + 1) * d] = (e / z) @ vv
        lse[h] = (m + np.log(z))[:, 0]
    return o, lse


def attention_bwd(do, q, k, v, hq: int, hkv: int, d: int):
    """Input gradients (dq, dk, dv) of attention: with P the softmax matrix of a
    head, dv = P^T do, dP = do v^T, dS = P * (dP - rowsum(do * o)),
    dq = dS k / sqrt(d), dk = dS^T q / sqrt(d); key/value gradients add over the
    query heads of their group."""
    do, q, k, v = _f64(do), _f64(q), _f64(k), _f64(v)
    S = q.shape[0]
    grp = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    mask = np.tril(np.ones((S, S), dtype=bool))
    for h in range(hq):
        kh = h // grp
        sl, kl = slice(h * d, (h + 1) * d), slice(kh * d, (kh + 1) * d)
        s = np.where(mask, (q[:, sl] @ k[:, kl].T) / np.sqrt(d), -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ v[:, kl]
        dv[:, kl] += p.T @ do[:, sl]
        dp = do[:, sl] @ v[:, kl].T
        ds = p * (dp - np.sum(do[:, sl] * o, axis=1, keepdims=True))
        dq[:, sl] = ds @ k[:, kl] / np.sqrt(d)
        dk[:, kl] += ds.T @ q[:, sl] / np.sqrt(d)
    return dq, dk, dv


# --------------------------------------------------------------------------- SwiGLU

def silu(z):
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def swiglu(g, u):
    """a = silu(g) * u."""
    return silu(g) * _f64(u)


def swiglu_bwd(da, g, u):
    """(dg, du) with silu'(z) = s (1 + z (1 - s)), s = 1 / (1 + exp(-z))."""
    da, g, u = _f64(da), _f64(g), _f64(u)
    sg = 1.0 / (1.0 + np.exp(-g))
    return da * u * sg * (1.0 + g * (1.0 - sg)), da * g * sg


# --------------------------------------------------------------------------- cross-entropy

def cross_entropy(logits, target):
    """Mean token loss and its gradient (softmax - onehot) / T for logits [T, V]."""
    z = _f64(logits)
    T = z.shape[0]
    m = z.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
    t = np.asarray(target, dtype=np.int64)
    loss = float(np.mean(lse - z[np.arange(T), t]))
    grad = np.exp(z - lse[:, None])
    grad[np.arange(T), t] -= 1.0
    return loss, grad / T


# --------------------------------------------------------------------------- one decoder layer

def _bf16(a) -> np.ndarray:
    """Round to bf16 (nearest even) and back to fp64: the activation storage of
    the layer, applied where the GPU stores an activation."""
    import torch
    return torch.from_numpy(np.asarray(a, np.float64)).to(torch.bfloat16).double().numpy()


def decoder_layer(p: dict, xin, res, dx3, cfg: dict, bf16: bool = True) -> dict:
    """Forward and input/adapter gradients of one pre-norm Llama layer:
        x = xin + res; h1 = rmsnorm(x); q, k, v = linears(h1) (+ LoRA on the
        adapted ones); q, k rotated; a = attention(q, k, v); x2 = x + o(a);
        h2 = rmsnorm(x2); out = x2 + down(swiglu(gate(h2), up(h2))),
    then, for the upstream gradient dx3 of out: dx (gradient of x) and dA, dB
    of every adapted projection. Returns out, x2, dn (so out = x2 + dn), dx
    and grads[name] = (dA, dB). p holds the decoded weights W_<name> [N, K]
    (fp32 values, already rounded as the GPU multiplies them), gamma1, gamma2,
    and A_<name>, B_<name> for adapted names; cfg holds heads, kv_heads,
    head_dim, eps, theta, s and targets. With bf16=True every stored
    activation is rounded to bf16 where the GPU path stores one. Uses the
    NF4-linear oracle for the projections."""
    import oracle as O
    rb = _bf16 if bf16 else (lambda a: _f64(a))
    H, Hkv, d, eps, th, s = cfg["heads"], cfg["kv_heads"], cfg["head_dim"], cfg["eps"], cfg["theta"], cfg["s"]
    tg = cfg["targets"]

    def lin(name, inp):
        if name in tg:
            y, T = O.linear_fwd(inp, p["W_" + name], p["A_" + name], p["B_" + name], s)
            return rb(y), T
        y, _ = O.linear_fwd(inp, p["W_" + name])
        return rb(y), None

    def lin_bwd(name, dy):
        if name in tg:
            dxx, U = O.linear_bwd_input(dy, p["W_" + name], p["A_" + name], p["B_" + name], s)
            return rb(dxx), U
        dxx, _ = O.linear_bwd_input(dy, p["W_" + name])
        return rb(dxx), None

    x = rb(_f64(xin) + _f64(res)) if res is not None else _f64(xin)
    h1 = rb(rmsnorm(x, p["gamma1"], eps)[0])
    q, Tq = lin("q_proj", h1)
    k, Tk = lin("k_proj", h1)
    v, Tv = lin("v_proj", h1)
    q, k = rb(rope(q, H, d, th)), rb(rope(k, Hkv, d, th))
    a = rb(attention(q, k, v, H, Hkv, d)[0])
    o, To = lin("o_proj", a)
    x2 = rb(x + o)
    h2 = rb(rmsnorm(x2, p["gamma2"], eps)[0])
    g, Tg = lin("gate_proj", h2)
    u, Tu = lin("up_proj", h2)
    sw = rb(swiglu(g, u))
    dn, Td = lin("down_proj", sw)
    out = rb(x2 + dn)
    T = {"q_proj": Tq, "k_proj": Tk, "v_proj": Tv, "o_proj": To, "gate_proj": Tg, "up_proj": Tu, "down_proj": Td}

    dx3 = _f64(dx3)
    dsw, Ud = lin_bwd("down_proj", dx3)
    dg, du = swiglu_bwd(dsw, g, u)
    dg, du = rb(dg), rb(du)
    dh2a, Ug = lin_bwd("gate_proj", dg)
    dh2b, Uu = lin_bwd("up_proj", du)
    dh2 = rb(dh2a + dh2b)
    dx2 = rb(rmsnorm_bwd(dh2, x2, p["gamma2"], eps) + dx3)
    da, Uo = lin_bwd("o_proj", dx2)
    dq, dk, dv = attention_bwd(da, q, k, v, H, Hkv, d)
    dq, dk, dv = rb(dq), rb(dk), rb(dv)
    dq, dk = rb(rope(dq, H, d, th, inverse=True)), rb(rope(dk, Hkv, d, th, inverse=True))
    dh1q, Uq = lin_bwd("q_proj", dq)
    dh1k, Uk = lin_bwd("k_proj", dk)
    dh1v, Uv = lin_bwd("v_proj", dv)
    dh1 = rb(dh1q + dh1k + dh1v)
    dx = rb(rmsnorm_bwd(dh1, x, p["gamma1"], eps) + dx2)
    U = {"q_proj": Uq, "k_proj": Uk, "v_proj": Uv, "o_proj": Uo, "gate_proj": Ug, "up_proj": Uu, "down_proj": Ud}
    ins = {"q_proj": (h1, dq), "k_proj": (h1, dk), "v_proj": (h1, dv), "o_proj": (a, dx2), "gate_proj": (h2, dg),
           "up_proj": (h2, du), "down_proj": (sw, dx3)}
    grads = {}
    for name in tg:
        xi, dyi = ins[name]
        grads[name] = O.lora_grad(xi, dyi, T[name], U[name], s)
    return {"out": out, "dx": dx, "grads": grads, "x2": x2, "dn": dn}
