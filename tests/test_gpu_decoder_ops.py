"""GPU parity of the decoder-layer operations (RMSNorm, rotary embedding,
causal grouped-query attention, SwiGLU, cross-entropy, with input gradients)
against the fp64 oracle in oracle/llama.py on the same seeded inputs. bf16
outputs: tests/parity.py's bf16 bar; fp32 outputs: relative Frobenius 1e-5
(fp32 arithmetic throughout)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import llama as OL
from tests.parity import assert_close, bits, to_np

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def rnd(shape, std, seed, dt):
    return workloads.normal_f32(shape, std, seed, "cuda").to(DT[dt])


@pytest.mark.parametrize("rows,width", [(512, 4096), (3, 100), (1, 16), (5, 8192), (7, 2056)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_add_rmsnorm_and_backward(gpu, rows, width, dt):
    x, res = rnd((rows, width), 1.0, 1, dt), rnd((rows, width), 0.5, 2, dt)
    gamma = workloads.normal_f32((width,), 1.0, 3, "cuda")
    eps = 1e-5
    s, y, rstd = gpu.add_rmsnorm(x, gamma, eps, res=res)
    _, y0, rstd0 = gpu.add_rmsnorm(x, gamma, eps)
    dy = rnd((rows, width), 1.0, 4, dt)
    dres = rnd((rows, width), 1.0, 5, dt)
    dx = gpu.rmsnorm_bwd(dy, s, rstd, gamma, dres=dres)
    torch.cuda.synchronize()
    # the stored sum is the activation-type rounding of the fp32 sum x + res
    s_ref = to_np(x).astype(np.float32) + to_np(res).astype(np.float32)
    if dt == "bf16":
        s_ref = OL._bf16(s_ref)
    np.testing.assert_array_equal(to_np(s), s_ref)
    g = gamma.cpu().numpy()
    y_ref, r_ref = OL.rmsnorm(s_ref, g, eps)
    assert_close(to_np(y), y_ref, dt, "y")
    assert_close(rstd.cpu().numpy(), r_ref, "f32", "rstd")
    y0_ref, _ = OL.rmsnorm(to_np(x), g, eps)
    assert_close(to_np(y0), y0_ref, dt, "y without residual")
    dx_ref = OL.rmsnorm_bwd(to_np(dy), s_ref, g, eps) + to_np(dres)
    assert_close(to_np(dx), dx_ref, dt, "dx")


@pytest.mark.parametrize("S,heads,d", [(512, 32, 128), (37, 3, 64), (5, 1, 2)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_rope(gpu, S, heads, d, dt):
    x = rnd((S, heads * d), 1.0, 7, dt)
    y = gpu.rope_(x.clone(), heads, d, 500000.0)
    z = gpu.rope_(y.clone(), heads, d, 500000.0, inverse=True)
    torch.cuda.synchronize()
    assert_close(to_np(y), OL.rope(to_np(x), heads, d, 500000.0), dt, "rope")
    assert_close(to_np(z), OL.rope(to_np(y), heads, d, 500000.0, inverse=True), dt, "inverse rope")


@pytest.mark.parametrize("S,hq,hkv,d", [(512, 32, 8, 128), (100, 8, 2, 64), (17, 4, 4, 16), (1, 2, 1, 32),
                                        (130, 4, 1, 128)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_attention_forward_backward(gpu, S, hq, hkv, d, dt):
    print(f"[attention] S={S} hq={hq} hkv={hkv} d={d} {dt}", flush=True)
    q, k, v = rnd((S, hq * d), 1.0, 11, dt), rnd((S, hkv * d), 1.0, 12, dt), rnd((S, hkv * d), 1.0, 13, dt)
    do = rnd((S, hq * d), 1.0, 14, dt)
    o, lse = gpu.attention_fwd(q, k, v, hq, hkv, d)
    dq, dk, dv = gpu.attention_bwd(do, q, k, v, o, lse, hq, hkv, d)
    dq2, dk2, dv2 = gpu.attention_bwd(do, q, k, v, o, lse, hq, hkv, d)
    torch.cuda.synchronize()
    qn, kn, vn, don = to_np(q), to_np(k), to_np(v), to_np(do)
    o_ref, lse_ref = OL.attention(qn, kn, vn, hq, hkv, d)
    assert_close(to_np(o), o_ref, dt, "o")
    np.testing.assert_allclose(lse.cpu().numpy(), lse_ref, rtol=0, atol=1e-4)
    dq_ref, dk_ref, dv_ref = OL.attention_bwd(don, qn, kn, vn, hq, hkv, d)
    if S == 1:
        # one key: dS = P (dP - rowsum(dO * O)) = 0 exactly, so dQ and dK are 0 up to the
        # cancellation of two equal sums of d products
        bound = 64 * np.finfo(np.float32).eps * np.abs(don).max() * np.abs(vn).max() * d * np.abs(kn).max()
        assert np.abs(to_np(dq)).max() <= bound and np.abs(to_np(dk)).max() <= bound
    else:
        assert_close(to_np(dq), dq_ref, dt, "dq")
        assert_close(to_np(dk), dk_ref, dt, "dk")
    assert_close(to_np(dv), dv_ref, dt, "dv")
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a, b), "attention backward not run-to-run identical"


@pytest.mark.parametrize("n", [(512, 14336), (3, 100)])  # 16-byte vectors; 100 bf16 per row: one entry per lane
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_swiglu(gpu, dt, n):
    g, u, da = rnd(n, 2.0, 21, dt), rnd(n, 1.0, 22, dt), rnd(n, 1.0, 23, dt)
    a = gpu.swiglu(g, u)
    dg, du = gpu.swiglu_bwd(da, g, u)
    torch.cuda.synchronize()
    gn, un, dan = to_np(g), to_np(u), to_np(da)
    assert_close(to_np(a), OL.swiglu(gn, un), dt, "a")
    dg_ref, du_ref = OL.swiglu_bwd(dan, gn, un)
    assert_close(to_np(dg), dg_ref, dt, "dg")
    assert_close(to_np(du), du_ref, dt, "du")


@pytest.mark.parametrize("S,hq,hkv,d", [(512, 32, 8, 128), (100, 8, 2, 64), (37, 4, 2, 16)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_strided_qkv_matches_dense(gpu, S, hq, hkv, d, dt):
    """q, k, v as column blocks of one [S, (hq + 2 hkv) d] projection output
    (rows one stride apart): rope on the q and k blocks together, attention
    forward and backward with dq, dk, dv written into the same blocks of a
    second such array; every result equals the dense calls' bit for bit (the
    stride only moves the addresses)."""
    print(f"[strided] S={S} hq={hq} hkv={hkv} d={d} {dt}", flush=True)
    w = (hq + 2 * hkv) * d
    qkv = rnd((S, w), 1.0, 31, dt)
    do = rnd((S, hq * d), 1.0, 32, dt)
    q, k, v = qkv[:, :hq * d], qkv[:, hq * d:(hq + hkv) * d], qkv[:, (hq + hkv) * d:]
    dense = [t.contiguous() for t in (q, k, v)]
    gpu.rope_(qkv[:, :(hq + hkv) * d], hq + hkv, d, 500000.0)  # q and k heads in one call
    gpu.rope_(dense[0], hq, d, 500000.0)
    gpu.rope_(dense[1], hkv, d, 500000.0)
    o, lse = gpu.attention_fwd(q, k, v, hq, hkv, d)
    o_d, lse_d = gpu.attention_fwd(*dense, hq, hkv, d)
    g = torch.full((S, w), 7.0, dtype=DT[dt], device="cuda")
    gq, gk, gv = g[:, :hq * d], g[:, hq * d:(hq + hkv) * d], g[:, (hq + hkv) * d:]
    gpu.attention_bwd(do, q, k, v, o, lse, hq, hkv, d, dq=gq, dk=gk, dv=gv)
    dq_d, dk_d, dv_d = gpu.attention_bwd(do, *dense, o_d, lse_d, hq, hkv, d)
    torch.cuda.synchronize()
    for a, b, what in ((q, dense[0], "rope q"), (k, dense[1], "rope k"), (o, o_d, "o"), (lse, lse_d, "lse"),
                       (gq, dq_d, "dq"), (gk, dk_d, "dk"), (gv, dv_d, "dv")):
        assert torch.equal(a.contiguous(), b), what


@pytest.mark.parametrize("rows,width", [(512, 14336), (37, 100)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_strided_swiglu_matches_dense(gpu, rows, width, dt):
    """g and u as the two column blocks of one [rows, 2 width] array (the
    fused gate/up projection output), dg and du written into the blocks of
    another: equal to the dense calls bit for bit, and a dense."""
    if (width * (2 if dt == "bf16" else 4)) % 16:
        width += 8 - width % 8  # keep the second block 16-byte aligned
    gu = rnd((rows, 2 * width), 2.0, 41, dt)
    da = rnd((rows, width), 1.0, 42, dt)
    g, u = gu[:, :width], gu[:, width:]
    a = gpu.swiglu(g, u)
    a_d = gpu.swiglu(g.contiguous(), u.contiguous())
    dgu = torch.full((rows, 2 * width), 3.0, dtype=DT[dt], device="cuda")
    gpu.swiglu_bwd(da, g, u, dg=dgu[:, :width], du=dgu[:, width:])
    dg_d, du_d = gpu.swiglu_bwd(da, g.contiguous(), u.contiguous())
    torch.cuda.synchronize()
    assert a.is_contiguous() and torch.equal(a, a_d)
    assert torch.equal(dgu[:, :width].contiguous(), dg_d) and torch.equal(dgu[:, width:].contiguous(), du_d)


@pytest.mark.parametrize("T,V,dt", [(512, 128256, "bf16"), (7, 1000, "f32"), (1, 3, "bf16"), (9, 1000, "bf16")])
def test_cross_entropy(gpu, T, V, dt):
    z = rnd((T, V), 2.0, 31, dt)
    t = torch.from_numpy(np.random.default_rng(T).integers(0, V, size=T, dtype=np.int64)).cuda()
    st = torch.full((1,), 9, dtype=torch.int32, device="cuda")
    loss, tok, dz = gpu.cross_entropy(z, t, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    l_ref, g_ref = OL.cross_entropy(to_np(z), t.cpu().numpy())
    assert abs(float(loss.item()) - l_ref) <= 1e-5 * abs(l_ref) + 1e-6
    assert_close(to_np(dz), g_ref, dt, "dz")


@pytest.mark.parametrize("dt,V", [("f32", 50), ("bf16", 48)])
def test_cross_entropy_bad_target(gpu, dt, V):
    z = rnd((4, V), 1.0, 32, dt)
    t = torch.tensor([0, V, -1, V - 1], dtype=torch.int64, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    loss, tok, _ = gpu.cross_entropy(z, t, status=st, want_grad=False)
    torch.cuda.synchronize()
    assert int(st.item()) == -1
    tk = tok.cpu().numpy()
    assert tk[1] == 0.0 and tk[2] == 0.0 and tk[0] > 0 and tk[3] > 0
