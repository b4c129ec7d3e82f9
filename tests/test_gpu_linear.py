"""GPU parity of the fused NF4 + LoRA linear layer against the fp64 CPU oracle.

y = x W^T + s (x A^T) B^T, dX = dY W + s (dY B) A, dA = s U^T x, dB = s dY^T T
(Aner docs "Adapter API", "LoRA FA includes gradient preconditioning", "Mixed
precision keeps stable state in FP32"). The GPU quantizes W itself; the oracle
quantizes the same fp32 W on the CPU and multiplies its own decoded weights
(bf16-rounded on the bf16 path), so the two sides share only the inputs.
Tolerances: tests/parity.py. B is random in every case so the adapter path is
exercised (Soup gate results, "What the gate caught").
"""
import numpy as np
import pytest
import torch

import workloads
from tests.parity import assert_close, bits, to_np

pytestmark = pytest.mark.gpu


def make_case(M, K, N, r, dtype, seed=0, dy_std=1.0, device="cuda"):
    lay = workloads.Linear("t", N, K, r)
    inp = workloads.lora_inputs(lay, M, seed_offset=seed, device=device, dy_std=dy_std)
    W = workloads.normal_f32((N, K), 0.02, workloads.weight_seed(seed), device)
    if dtype == torch.float32:
        inp["x"] = inp["x"].float()
        inp["dy"] = inp["dy"].float()
    inp["W"] = W
    return inp


def oracle_weight(orc, W: torch.Tensor, dtype, dq=True):
    q = orc.quantize(W.cpu().numpy(), dq)
    if dtype == torch.bfloat16:
        return orc.bf16_bits_to_f32(orc.dequantize(q, "bf16")).reshape(W.shape)
    return orc.dequantize(q, "f32").reshape(W.shape)


def run_all(gpu, c, s, dq=True, fa=False):
    Wq = gpu.quantize(c["W"], dq)
    A, B = c.get("A"), c.get("B")
    y, T = gpu.linear_fwd(c["x"], Wq, A, B, s)
    dx, U = gpu.linear_bwd_input(c["dy"], Wq, A, B, s)
    grads = gpu.lora_grad(c["x"], c["dy"], T, U, s, fa=fa) if A is not None else (None, None)
    torch.cuda.synchronize()
    return Wq, y, T, dx, U, grads


CASES = [
    # (M, K, N, r): the 576x576 layer, tails in every dimension, rank 1 and odd ranks
    (512, 576, 576, 16),
    (37, 100, 70, 3),
    (1, 64, 1, 1),
    (130, 192, 576, 8),
    (64, 1536, 576, 8),
    (200, 576, 1536, 16),
    (33, 129, 65, 5),
    # 512 tokens through 2048-wide reductions: the side products take the split
    # skinny GEMM at rank 16 in both directions
    (512, 2048, 2048, 16),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("M,K,N,r", CASES)
def test_linear_parity(gpu, orc, M, K, N, r, dt):
    print(f"[linear] M={M} K={K} N={N} r={r} {dt}", flush=True)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    c = make_case(M, K, N, r, dtype, seed=M + K)
    s = gpu.lora_scale(32.0, r)
    Wq, y, T, dx, U, (dA, dB) = run_all(gpu, c, s)
    Wref = oracle_weight(orc, c["W"], dtype)
    x, dy = to_np(c["x"]), to_np(c["dy"])
    A, B = c["A"].cpu().numpy(), c["B"].cpu().numpy()
    y_ref, T_ref = orc.linear_fwd(x, Wref, A, B, s)
    dx_ref, U_ref = orc.linear_bwd_input(dy, Wref, A, B, s)
    assert_close(to_np(y), y_ref, dt, "y")
    assert_close(to_np(dx), dx_ref, dt, "dx")
    # adapter side products and gradients are fp32 arithmetic on both paths
    assert_close(T.cpu().numpy(), T_ref, "f32", "T")
    assert_close(U.cpu().numpy(), U_ref, "f32", "U")
    dA_ref, dB_ref = orc.lora_grad(x, dy, T_ref, U_ref, s)
    assert_close(dA.cpu().numpy(), dA_ref, "f32", "dA")
    assert_close(dB.cpu().numpy(), dB_ref, "f32", "dB")
    assert np.any(dA.cpu().numpy() != 0) and np.any(dB.cpu().numpy() != 0)


def test_single_quant_and_rslora(gpu, orc):
    M, K, N, r = 96, 256, 192, 8
    c = make_case(M, K, N, r, torch.bfloat16, seed=5)
    s = gpu.lora_scale(16.0, r, rslora=True)
    _, y, T, dx, U, _ = run_all(gpu, c, s, dq=False)
    Wref = oracle_weight(orc, c["W"], torch.bfloat16, dq=False)
    y_ref, _ = orc.linear_fwd(to_np(c["x"]), Wref, c["A"].cpu().numpy(), c["B"].cpu().numpy(), s)
    dx_ref, _ = orc.linear_bwd_input(to_np(c["dy"]), Wref, c["A"].cpu().numpy(), c["B"].cpu().numpy(), s)
    assert_close(to_np(y), y_ref, "bf16", "y")
    assert_close(to_np(dx), dx_ref, "bf16", "dx")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_zero_B_equals_base_bitwise(gpu, dt):
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    c = make_case(256, 576, 576, 16, dtype, seed=2)
    Wq = gpu.quantize(c["W"], True)
    B0 = torch.zeros_like(c["B"])
    y_lora, T = gpu.linear_fwd(c["x"], Wq, c["A"], B0, 2.0)
    y_base, _ = gpu.linear_fwd(c["x"], Wq)
    dx_lora, U = gpu.linear_bwd_input(c["dy"], Wq, c["A"], B0, 2.0)
    dx_base, _ = gpu.linear_bwd_input(c["dy"], Wq)
    torch.cuda.synchronize()
    assert torch.equal(y_lora, y_base) and torch.equal(dx_lora, dx_base)
    dA, dB = gpu.lora_grad(c["x"], c["dy"], T, U, 2.0)
    assert torch.count_nonzero(dA) == 0 and torch.count_nonzero(dB) > 0


def test_repeat_bitwise_and_lora_fa(gpu):
    c = make_case(300, 576, 192, 8, torch.bfloat16, seed=3)
    r1 = run_all(gpu, c, 2.0)
    r2 = run_all(gpu, c, 2.0)
    for a, b in zip(r1[1:5], r2[1:5]):
        assert torch.equal(a, b)
    assert torch.equal(r1[5][0], r2[5][0]) and torch.equal(r1[5][1], r2[5][1])
    _, dB_fa = gpu.lora_grad(None, c["dy"], r1[2], None, 2.0, fa=True)
    torch.cuda.synchronize()
    assert torch.equal(dB_fa, r1[5][1])


def test_fused_matches_dequantize_then_matmul(gpu):
    """The fused kernel against torch's own GEMM on nf4_dequantize's bf16 output
    (fp32 copies, so torch uses an fp32 GEMM)."""
    c = make_case(256, 1024, 512, 0, torch.bfloat16, seed=9)
    Wq = gpu.quantize(c["W"], True)
    y, _ = gpu.linear_fwd(c["x"], Wq)
    Wd = gpu.dequantize(Wq, torch.bfloat16).float()
    ref = c["x"].float() @ Wd.T
    torch.cuda.synchronize()
    assert_close(to_np(y), ref.double().cpu().numpy(), "bf16", "y vs torch")


@pytest.mark.parametrize("K,N,dq", [(576, 192, True), (4096, 1024, True), (640, 4100, False), (1536, 576, True)])
def test_fused_decode_bitexact(gpu, K, N, dq):
    """With x = I (M = K), y[m][n] = W_hat[n][m] exactly (one nonzero product per
    output, exact in fp32), so the weights decoded inside the GEMM must equal
    nf4_dequantize's bf16 output bit for bit."""
    W = workloads.weight_with_outliers((N, K), seed=K + N, device="cuda")
    Wq = gpu.quantize(W, dq)
    eye = torch.eye(K, dtype=torch.bfloat16, device="cuda")
    y, _ = gpu.linear_fwd(eye, Wq)
    d = gpu.dequantize(Wq, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y, d.T.contiguous())


FULL = [("q_proj", 4096, 4096), ("k_proj", 1024, 4096), ("gate_proj", 14336, 4096), ("down_proj", 4096, 14336)]


@pytest.mark.parametrize("name,N,K", FULL)
def test_llama8b_shapes_sampled(gpu, orc, name, N, K):
    """Llama-8B-shaped projections at 4096 tokens, r = 16, in the launch
    configuration the benchmark times: y and dX on 24 sampled token rows, T and
    U on the same rows, dA and dB in full (from the oracle's own T and U)."""
    print(f"[linear] full {name} {N}x{K}", flush=True)
    M, r = 4096, 16
    c = make_case(M, K, N, r, torch.bfloat16, seed=11)
    s = gpu.lora_scale(32.0, r)
    Wq, y, T, dx, U, (dA, dB) = run_all(gpu, c, s)
    Wref = oracle_weight(orc, c["W"], torch.bfloat16)
    rows = np.sort(np.random.default_rng(N + K).choice(M, 24, replace=False))
    x = to_np(c["x"])
    dy = to_np(c["dy"])
    A, B = c["A"].cpu().numpy(), c["B"].cpu().numpy()
    y_ref, T_ref = orc.linear_fwd(x[rows], Wref, A, B, s)
    dx_ref, U_ref = orc.linear_bwd_input(dy[rows], Wref, A, B, s)
    assert_close(to_np(y)[rows], y_ref, "bf16", "y rows")
    assert_close(to_np(dx)[rows], dx_ref, "bf16", "dx rows")
    assert_close(T.cpu().numpy()[rows], T_ref, "f32", "T rows")
    assert_close(U.cpu().numpy()[rows], U_ref, "f32", "U rows")
    dA_ref, dB_ref = orc.lora_grad(x, dy, orc.lora_down(x, A), orc.lora_up_grad(dy, B), s)
    assert_close(dA.cpu().numpy(), dA_ref, "f32", "dA")
    assert_close(dB.cpu().numpy(), dB_ref, "f32", "dB")


RAGGED_LARGE = [
    # (M, K, N): enough 256 x 256 tiles for the shared-decode kernel, with a
    # part-filled last token tile and (first case) a part-filled column tile;
    # the second leaves a last round of 16 tiles, run as half-height tiles; the
    # third (128 tiles) is the largest problem left to the small-tile kernels
    (2000, 1024, 4160),
    (4000, 4096, 4352),
    (2047, 2048, 4096),
    # odd and single reduction-step counts on the shared-decode kernel: the
    # forward of a 576-wide input (9 steps of 64) and of a 64-wide input (one
    # step), the input gradient of a 576-wide output (9 steps) and of a 64-wide
    # output (one step), each with 256 whole tiles
    (4096, 576, 4096),
    (4096, 64, 4096),
    (4096, 4096, 576),
    (4096, 4096, 64),
    # 8196 output columns (not a multiple of 8): the forward's 8-byte output
    # stores instead of the staged 16-byte ones
    (1024, 1024, 8196),
]


@pytest.mark.parametrize("M,K,N", RAGGED_LARGE)
def test_large_ragged_sampled(gpu, orc, M, K, N):
    """Large problems at ragged sizes: y and dX on 24 sampled token
    rows (always including the last few rows of the part-filled token tile)
    against the oracle, r = 8."""
    print(f"[linear] large ragged M={M} K={K} N={N}", flush=True)
    r = 8
    c = make_case(M, K, N, r, torch.bfloat16, seed=M + N)
    s = gpu.lora_scale(16.0, r)
    Wq = gpu.quantize(c["W"], True)
    y, _ = gpu.linear_fwd(c["x"], Wq, c["A"], c["B"], s)
    dx, _ = gpu.linear_bwd_input(c["dy"], Wq, c["A"], c["B"], s)
    torch.cuda.synchronize()
    Wref = oracle_weight(orc, c["W"], torch.bfloat16)
    rng = np.random.default_rng(M + K)
    rows = np.unique(np.concatenate([rng.choice(M - 4, 20, replace=False), np.arange(M - 4, M)]))
    A, B = c["A"].cpu().numpy(), c["B"].cpu().numpy()
    y_ref, _ = orc.linear_fwd(to_np(c["x"])[rows], Wref, A, B, s)
    dx_ref, _ = orc.linear_bwd_input(to_np(c["dy"])[rows], Wref, A, B, s)
    assert_close(to_np(y)[rows], y_ref, "bf16", "y rows")
    assert_close(to_np(dx)[rows], dx_ref, "bf16", "dx rows")


@pytest.mark.parametrize("K,N,dq", [(576, 192, True), (4096, 1024, True), (640, 4096, False), (576, 1536, True)])
def test_fused_decode_bitexact_bwd(gpu, K, N, dq):
    """With dY = I (M = N), dX[m][k] = W_hat[m][k] exactly: the weights the input
    gradient decodes (transposed, in LDS) equal nf4_dequantize's bf16 output."""
    W = workloads.weight_with_outliers((N, K), seed=K * 3 + N, device="cuda")
    Wq = gpu.quantize(W, dq)
    eye = torch.eye(N, dtype=torch.bfloat16, device="cuda")
    dx, _ = gpu.linear_bwd_input(eye, Wq)
    d = gpu.dequantize(Wq, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(dx, d)


def test_backward_heavy_down_proj(gpu, orc):
    """The backward-heavy configuration: down_proj W [4096, 14336], 8192 tokens,
    dY ~ N(0, 0.01), rank-64 rsLoRA with alpha 16, in the launch configuration
    the benchmark times. dX and U on 24 sampled token rows; dA and dB in full,
    then the LoRA-FA variant (dB only; at 8192 tokens it cuts its token reduction
    differently from the full call, so it is held to the oracle and to run-to-run
    identity)."""
    print("[linear] backward-heavy down_proj 8192 tokens r=64", flush=True)
    wl = workloads.WORKLOADS["down_proj_bwd"]
    L = wl["layers"][0]
    M, r = wl["tokens"], L.lora_rank
    s = gpu.lora_scale(wl["alpha"], r, rslora=wl["rslora"])
    c = make_case(M, L.k_in, L.n_out, r, torch.bfloat16, seed=21, dy_std=wl["dy_std"])
    Wq, y, T, dx, U, (dA, dB) = run_all(gpu, c, s)
    _, dB_fa = gpu.lora_grad(c["x"], c["dy"], T, None, s, fa=True)
    _, dB_fa2 = gpu.lora_grad(c["x"], c["dy"], T, None, s, fa=True)
    torch.cuda.synchronize()
    assert torch.equal(dB_fa.view(torch.int32), dB_fa2.view(torch.int32))  # fixed-order sums
    Wref = oracle_weight(orc, c["W"], torch.bfloat16)
    rows = np.sort(np.random.default_rng(5).choice(M, 24, replace=False))
    dy = to_np(c["dy"])
    A, B = c["A"].cpu().numpy(), c["B"].cpu().numpy()
    dx_ref, U_ref = orc.linear_bwd_input(dy[rows], Wref, A, B, s)
    assert_close(to_np(dx)[rows], dx_ref, "bf16", "dx rows")
    assert_close(U.cpu().numpy()[rows], U_ref, "f32", "U rows")
    x = to_np(c["x"])
    dA_ref, dB_ref = orc.lora_grad(x, dy, orc.lora_down(x, A), orc.lora_up_grad(dy, B), s)
    assert_close(dA.cpu().numpy(), dA_ref, "f32", "dA")
    assert_close(dB.cpu().numpy(), dB_ref, "f32", "dB")
    assert_close(dB_fa.cpu().numpy(), dB_ref, "f32", "LoRA-FA dB")


SPLIT = [
    # (M, K, N, r, backward): reductions over few output tiles, which the bf16
    # path splits in parts whose fp32 partial sums are added in order
    (512, 14336, 4096, 16, False),   # down_proj forward at 512 tokens
    (512, 4096, 14336, 16, True),    # gate/up input gradient at 512 tokens
    (300, 8320, 1000, 5, False),     # ragged tokens, 130 steps in unequal parts, partial column tile
    (300, 1024, 8320, 5, True),
    (128, 4096, 1024, 16, False),    # too few tiles for the large kernel: small tiles in parts
    (128, 1024, 4096, 16, True),
    (100, 4096, 1024, 3, False),
]


@pytest.mark.parametrize("M,K,N,r,bwd", SPLIT)
def test_split_reduction(gpu, orc, M, K, N, r, bwd):
    """The split path on 32 sampled token rows against the oracle, the run-to-run
    identity of the fixed-order sum, and B = 0 giving the base result bit for
    bit (part 0 of the split adds the LoRA term to its partial sum before the
    parts are summed)."""
    print(f"[linear] split M={M} K={K} N={N} r={r} bwd={bwd}", flush=True)
    assert gpu.linear_workspace_bytes(M, K, N, backward=bwd) > 0
    c = make_case(M, K, N, r, torch.bfloat16, seed=M + N)
    s = gpu.lora_scale(32.0, r)
    Wq = gpu.quantize(c["W"], True)
    fn = gpu.linear_bwd_input if bwd else gpu.linear_fwd
    a = c["dy"] if bwd else c["x"]
    out, side = fn(a, Wq, c["A"], c["B"], s)
    out2, _ = fn(a, Wq, c["A"], c["B"], s)
    base, _ = fn(a, Wq)
    zero, _ = fn(a, Wq, c["A"], torch.zeros_like(c["B"]), s)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(zero, base)
    Wref = oracle_weight(orc, c["W"], torch.bfloat16)
    rows = np.sort(np.random.default_rng(M + K).choice(M, 32, replace=False))
    A, B = c["A"].cpu().numpy(), c["B"].cpu().numpy()
    if bwd:
        ref, U_ref = orc.linear_bwd_input(to_np(a)[rows], Wref, A, B, s)
    else:
        ref, U_ref = orc.linear_fwd(to_np(a)[rows], Wref, A, B, s)
    assert_close(to_np(out)[rows], ref, "bf16", "split output rows")
    assert_close(side.cpu().numpy()[rows], U_ref, "f32", "side product rows")


@pytest.mark.parametrize("M,K,N,r", [(512, 576, 576, 16), (4096, 4096, 1024, 16), (300, 1024, 8320, 5)])
def test_side_products_optional_and_recomputed(gpu, orc, M, K, N, r):
    """t_out / u_out may be omitted (the side product then lives in the
    workspace): y and dX are bit-identical to the calls that return T and U.
    lora_grad recomputes T from x and A, and U from dY and B, when they are not
    given: bit-identical to the calls that pass them (the same kernels form
    them), and dA, dB against the oracle; LoRA-FA recomputing T gives the dB
    of LoRA-FA given T."""
    print(f"[linear] optional side products M={M} K={K} N={N} r={r}", flush=True)
    c = make_case(M, K, N, r, torch.bfloat16, seed=M + 7)
    s = gpu.lora_scale(32.0, r)
    Wq = gpu.quantize(c["W"], True)
    y, T = gpu.linear_fwd(c["x"], Wq, c["A"], c["B"], s)
    y2, T2 = gpu.linear_fwd(c["x"], Wq, c["A"], c["B"], s, want_t=False)
    dx, U = gpu.linear_bwd_input(c["dy"], Wq, c["A"], c["B"], s)
    dx2, U2 = gpu.linear_bwd_input(c["dy"], Wq, c["A"], c["B"], s, want_u=False)
    dA, dB = gpu.lora_grad(c["x"], c["dy"], T, U, s)
    dA_t, dB_t = gpu.lora_grad(c["x"], c["dy"], None, U, s, A=c["A"])
    dA_u, dB_u = gpu.lora_grad(c["x"], c["dy"], T, None, s, B=c["B"])
    dA_tu, dB_tu = gpu.lora_grad(c["x"], c["dy"], None, None, s, A=c["A"], B=c["B"])
    _, dB_fa = gpu.lora_grad(c["x"], c["dy"], None, None, s, fa=True, A=c["A"])
    _, dB_fa_t = gpu.lora_grad(c["x"], c["dy"], T, None, s, fa=True)
    torch.cuda.synchronize()
    assert T2 is None and U2 is None
    assert torch.equal(y, y2) and torch.equal(dx, dx2)
    for a in (dA_t, dA_u, dA_tu):
        assert torch.equal(a.view(torch.int32), dA.view(torch.int32))
    for b in (dB_t, dB_u, dB_tu):
        assert torch.equal(b.view(torch.int32), dB.view(torch.int32))
    # LoRA-FA recomputing T equals LoRA-FA given T (its own token chunking,
    # which matches the full call's up to a few hundred tokens)
    assert torch.equal(dB_fa.view(torch.int32), dB_fa_t.view(torch.int32))
    x, dy = to_np(c["x"]), to_np(c["dy"])
    A, B = c["A"].cpu().numpy(), c["B"].cpu().numpy()
    dA_ref, dB_ref = orc.lora_grad(x, dy, orc.lora_down(x, A), orc.lora_up_grad(dy, B), s)
    assert_close(dA_tu.cpu().numpy(), dA_ref, "f32", "dA (T, U recomputed)")
    assert_close(dB_tu.cpu().numpy(), dB_ref, "f32", "dB (T, U recomputed)")
    assert_close(dB_fa.cpu().numpy(), dB_ref, "f32", "LoRA-FA dB (T recomputed)")


@pytest.mark.parametrize("M,I,r", [(1000, 8200, 16), (1000, 8200, 4), (130, 16384, 12), (4096, 14336, 16),
                                   (513, 8192, 8)])
def test_side_product_streamed_split(gpu, orc, M, I, r):
    """Reductions of 8192 or more at ranks up to 16 take the streamed split
    side product (128-row workgroups, 64-wide steps, partial sums added in
    split order): T = x A^T and U = dY B, whole, against the oracle, with ragged
    rows, a last step shorter than 64 and ranks below 16; run to run bitwise."""
    print(f"[linear] streamed side product M={M} I={I} r={r}", flush=True)
    cf = make_case(M, I, 64, r, torch.bfloat16, seed=M + I)
    cb = make_case(M, 64, I, r, torch.bfloat16, seed=M + I + 1)
    s = gpu.lora_scale(32.0, r)
    Wf = gpu.quantize(cf["W"], True)
    Wb = gpu.quantize(cb["W"], True)
    _, T = gpu.linear_fwd(cf["x"], Wf, cf["A"], cf["B"], s)
    _, T2 = gpu.linear_fwd(cf["x"], Wf, cf["A"], cf["B"], s)
    _, U = gpu.linear_bwd_input(cb["dy"], Wb, cb["A"], cb["B"], s)
    _, U2 = gpu.linear_bwd_input(cb["dy"], Wb, cb["A"], cb["B"], s)
    torch.cuda.synchronize()
    assert torch.equal(T.view(torch.int32), T2.view(torch.int32)) and torch.equal(U.view(torch.int32), U2.view(torch.int32))
    assert_close(T.cpu().numpy(), orc.lora_down(to_np(cf["x"]), cf["A"].cpu().numpy()), "f32", "T")
    assert_close(U.cpu().numpy(), orc.lora_up_grad(to_np(cb["dy"]), cb["B"].cpu().numpy()), "f32", "U")


@pytest.mark.parametrize("M,K,N,r", [(300, 1024, 576, 64), (129, 576, 1536, 100), (200, 640, 512, 256),
                                     (64, 256, 320, 33), (40, 448, 192, 128)])
def test_large_ranks(gpu, orc, M, K, N, r):
    """Ranks past 32 on the bf16 path (the side products in workgroups of 64
    ranks with a split reduction, the LoRA-gradient reduction in blocks of 32,
    64 or 128 ranks per launch): y, dX against the oracle at the bf16 bar, T, U,
    dA, dB at the fp32 bar, LoRA-FA's dB equal to the full call's (at these
    token counts both cut the token reduction into the same 32-token chunks),
    and the workspace-held and recomputed side products equal to the returned
    ones."""
    print(f"[linear] large rank M={M} K={K} N={N} r={r}", flush=True)
    c = make_case(M, K, N, r, torch.bfloat16, seed=M + r)
    s = gpu.lora_scale(16.0, r, rslora=True)
    Wq, y, T, dx, U, (dA, dB) = run_all(gpu, c, s)
    _, dB_fa = gpu.lora_grad(c["x"], c["dy"], T, None, s, fa=True)
    torch.cuda.synchronize()
    assert torch.equal(dB.view(torch.int32), dB_fa.view(torch.int32))
    Wref = oracle_weight(orc, c["W"], torch.bfloat16)
    x, dy = to_np(c["x"]), to_np(c["dy"])
    A, B = c["A"].cpu().numpy(), c["B"].cpu().numpy()
    y_ref, T_ref = orc.linear_fwd(x, Wref, A, B, s)
    dx_ref, U_ref = orc.linear_bwd_input(dy, Wref, A, B, s)
    assert_close(to_np(y), y_ref, "bf16", "y")
    assert_close(to_np(dx), dx_ref, "bf16", "dx")
    assert_close(T.cpu().numpy(), T_ref, "f32", "T")
    assert_close(U.cpu().numpy(), U_ref, "f32", "U")
    dA_ref, dB_ref = orc.lora_grad(x, dy, T_ref, U_ref, s)
    assert_close(dA.cpu().numpy(), dA_ref, "f32", "dA")
    assert_close(dB.cpu().numpy(), dB_ref, "f32", "dB")
    # side products left in the workspace, and T, U recomputed inside lora_grad:
    # the same kernels and split, so the same bits
    y2, _ = gpu.linear_fwd(c["x"], Wq, c["A"], c["B"], s, want_t=False)
    dx2, _ = gpu.linear_bwd_input(c["dy"], Wq, c["A"], c["B"], s, want_u=False)
    dA2, dB2 = gpu.lora_grad(c["x"], c["dy"], None, None, s, A=c["A"], B=c["B"])
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))
    assert torch.equal(dx2.view(torch.int16), dx.view(torch.int16))
    assert torch.equal(dA2.view(torch.int32), dA.view(torch.int32))
    assert torch.equal(dB2.view(torch.int32), dB.view(torch.int32))


GROUPS = [
    # (M, K, widths, ranks, double quant): projections of one activation in one call
    (4096, 4096, (4096, 1024, 1024), (16, 16, 16), True),     # q, k, v at 4096 tokens: 384 tiles, half-tile last round
    (4096, 4096, (14336, 14336), (16, 16), True),              # gate, up at 4096 tokens: 1792 tiles, 7 whole rounds
    (2000, 1024, (4160, 520, 1028), (8, 0, 4), False),         # ragged widths, a part with no adapter, single quant
    (4000, 1024, (2304, 1100, 1028, 264), (16, 8, 4, 12), True),  # four parts, 336 tiles: a last round of 80
    (512, 576, (576, 192, 192), (8, 8, 8), True),              # 10 tiles: each projection runs as its own call
]


@pytest.mark.parametrize("M,K,Ns,rs,dq", GROUPS)
def test_linear_fwd_group(gpu, orc, M, K, Ns, rs, dq):
    """Grouped forward over projections of one x: every y[i] and T[i] against
    the oracle on sampled token rows (including the last rows), T[i] bitwise
    equal to the projection's own call, y[i] too where that call also takes the
    256 x 256 kernel (at least 129 tiles), and run-to-run identical."""
    print(f"[linear] group M={M} K={K} N={Ns} r={rs}", flush=True)
    n = len(Ns)
    cs = [make_case(M, K, N, max(r, 1), torch.bfloat16, seed=7 + i) for i, (N, r) in enumerate(zip(Ns, rs))]
    x = cs[0]["x"]
    Ws = [gpu.quantize(c["W"], dq) for c in cs]
    As = [c["A"] if r else None for c, r in zip(cs, rs)]
    Bs = [c["B"] if r else None for c, r in zip(cs, rs)]
    ss = [gpu.lora_scale(2.0 * r, r) if r else 0.0 for r in rs]
    ys, Ts = gpu.linear_fwd_group(x, Ws, As, Bs, ss)
    ys2, Ts2 = gpu.linear_fwd_group(x, Ws, As, Bs, ss)
    alone = [gpu.linear_fwd(x, Ws[i], As[i], Bs[i], ss[i]) for i in range(n)]
    torch.cuda.synchronize()
    rng = np.random.default_rng(M + K + n)
    rows = np.unique(np.concatenate([rng.choice(M - 4, 12, replace=False), np.arange(M - 4, M)]))
    xs = to_np(x)[rows]
    for i, (N, r) in enumerate(zip(Ns, rs)):
        assert torch.equal(ys[i], ys2[i]), f"y[{i}] differs between runs"
        if r:
            assert torch.equal(Ts[i], Ts2[i]) and torch.equal(Ts[i], alone[i][1]), f"T[{i}]"
        if ((M + 255) // 256) * ((N + 255) // 256) >= 129:
            assert torch.equal(ys[i], alone[i][0]), f"y[{i}] differs from its own call"
        Wref = oracle_weight(orc, cs[i]["W"], torch.bfloat16, dq)
        A = As[i].cpu().numpy() if r else None
        B = Bs[i].cpu().numpy() if r else None
        y_ref, T_ref = orc.linear_fwd(xs, Wref, A, B, ss[i])
        assert_close(to_np(ys[i])[rows], y_ref, "bf16", f"y[{i}] rows")
        if r:
            assert_close(Ts[i].cpu().numpy()[rows], T_ref, "f32", f"T[{i}] rows")


@pytest.mark.parametrize("case", ["f32", "mixed_quant"])
def test_linear_fwd_group_fallbacks(gpu, orc, case):
    """Groups the one-launch path does not take run each projection as its own
    call: fp32 activations (the general kernel), and bf16 projections of which
    one is single and one double quantized (enough tiles otherwise). Each y[i]
    and T[i] equals its own call bit for bit."""
    print(f"[linear] group fallback {case}", flush=True)
    M, K, Ns, r = (300, 640, (576, 192), 8) if case == "f32" else (2048, 1024, (4096, 4096), 16)
    dt = torch.float32 if case == "f32" else torch.bfloat16
    cs = [make_case(M, K, N, r, dt, seed=3 + i) for i, N in enumerate(Ns)]
    x = cs[0]["x"]
    Ws = [gpu.quantize(c["W"], case == "f32" or i == 0) for i, c in enumerate(cs)]
    As, Bs = [c["A"] for c in cs], [c["B"] for c in cs]
    s = [gpu.lora_scale(16.0, r)] * len(Ns)
    ys, Ts = gpu.linear_fwd_group(x, Ws, As, Bs, s)
    for i in range(len(Ns)):
        y1, T1 = gpu.linear_fwd(x, Ws[i], As[i], Bs[i], s[i])
        torch.cuda.synchronize()
        assert torch.equal(ys[i], y1) and torch.equal(Ts[i], T1), f"part {i}"
    if case == "f32":
        Wref = oracle_weight(orc, cs[0]["W"], dt, True)
        y_ref, _ = orc.linear_fwd(to_np(x), Wref, As[0].cpu().numpy(), Bs[0].cpu().numpy(), s[0])
        assert_close(to_np(ys[0]), y_ref, "f32", "y[0]")


SUMS = [
    # (M, K, widths, ranks, double quant): the input gradient of one activation read by several projections
    (4096, 4096, (4096, 1024, 1024), (16, 16, 16), True),         # q, k, v at 4096 tokens: 64 + 16 + 16 steps
    (4096, 4096, (14336, 14336), (16, 16), True),                 # gate, up at 4096 tokens: 448 steps
    (4000, 2304, (576, 128, 1088), (8, 0, 4), False),             # odd step counts, a part with no adapter, ragged M
    (512, 576, (576, 192, 192), (8, 8, 8), True),                 # 6 tiles: separate calls added in order
    (4000, 4352, (1024, 512), (16, 8), True),                     # 272 tiles: a last round of 16, half tiles
]


@pytest.mark.parametrize("M,K,Ns,rs,dq", SUMS)
def test_linear_bwd_input_sum(gpu, orc, M, K, Ns, rs, dq):
    """Summed input gradient against the oracle's sum of the projections'
    input gradients on sampled token rows (including the last rows), each U[i]
    bitwise equal to its projection's own call, the whole run-to-run identical."""
    print(f"[linear] bwd sum M={M} K={K} N={Ns} r={rs}", flush=True)
    n = len(Ns)
    cs = [make_case(M, K, N, max(r, 1), torch.bfloat16, seed=21 + i) for i, (N, r) in enumerate(zip(Ns, rs))]
    dys = [c["dy"] for c in cs]
    Ws = [gpu.quantize(c["W"], dq) for c in cs]
    As = [c["A"] if r else None for c, r in zip(cs, rs)]
    Bs = [c["B"] if r else None for c, r in zip(cs, rs)]
    ss = [gpu.lora_scale(2.0 * r, r) if r else 0.0 for r in rs]
    dx, Us = gpu.linear_bwd_input_sum(dys, Ws, As, Bs, ss)
    dx2, _ = gpu.linear_bwd_input_sum(dys, Ws, As, Bs, ss)
    alone = [gpu.linear_bwd_input(dys[i], Ws[i], As[i], Bs[i], ss[i]) for i in range(n)]
    torch.cuda.synchronize()
    assert torch.equal(dx, dx2), "dx differs between runs"
    for i, r in enumerate(rs):
        if r:
            assert torch.equal(Us[i], alone[i][1]), f"U[{i}]"
    rng = np.random.default_rng(M + K + 7 * n)
    rows = np.unique(np.concatenate([rng.choice(M - 4, 12, replace=False), np.arange(M - 4, M)]))
    ref = 0.0
    for i, r in enumerate(rs):
        Wref = oracle_weight(orc, cs[i]["W"], torch.bfloat16, dq)
        A = As[i].cpu().numpy() if r else None
        B = Bs[i].cpu().numpy() if r else None
        d, _ = orc.linear_bwd_input(to_np(dys[i])[rows], Wref, A, B, ss[i])
        ref = ref + d
    assert_close(to_np(dx)[rows], ref, "bf16", "dx rows")


def test_linear_bwd_input_sum_f32(gpu, orc):
    """fp32 summed input gradient (separate general-kernel calls added in
    order) against the oracle's sum, in full."""
    print("[linear] bwd sum f32", flush=True)
    M, K, Ns, r = 300, 640, (576, 192, 64), 8
    cs = [make_case(M, K, N, r, torch.float32, seed=31 + i) for i, N in enumerate(Ns)]
    Ws = [gpu.quantize(c["W"], True) for c in cs]
    s = gpu.lora_scale(16.0, r)
    dx, Us = gpu.linear_bwd_input_sum([c["dy"] for c in cs], Ws, [c["A"] for c in cs], [c["B"] for c in cs],
                                      [s] * len(Ns))
    torch.cuda.synchronize()
    ref = 0.0
    for i, c in enumerate(cs):
        Wref = oracle_weight(orc, c["W"], torch.float32, True)
        d, U_ref = orc.linear_bwd_input(to_np(c["dy"]), Wref, c["A"].cpu().numpy(), c["B"].cpu().numpy(), s)
        assert_close(Us[i].cpu().numpy(), U_ref, "f32", f"U[{i}]")
        ref = ref + d
    assert_close(to_np(dx), ref, "f32", "dx")
