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
