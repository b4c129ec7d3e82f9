"""GPU parity of the adapter's optimizer step: lorafa_preconditioner and
lora_adamw_step through the C ABI against the fp64 oracle on the same seeded
fp32 inputs. Bounds: see tests/parity.py (derived from the fp32 rounding of
each operation; the preconditioner from its conditioning)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import U32, U64, adamw_bounds, assert_within

pytestmark = pytest.mark.gpu

HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)  # the pages' adapter learning rate


def _np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def _check_precond(P_gpu: np.ndarray, A: np.ndarray, what: str) -> float:
    P = oracle.lorafa_preconditioner(A)
    r, K = A.shape
    A64 = A.astype(np.float64)
    ev = np.linalg.eigvalsh(A64 @ A64.T + 1e-8 * np.eye(r))
    kappa = ev.max() / ev.min()
    bound = 1.01 * U32 * 2 * np.abs(P) + 4.0 * (K + r) * r * kappa * U64 * np.abs(P).max()
    return assert_within(P_gpu, P, bound, what)


@pytest.mark.parametrize("r,K", [(1, 576), (2, 576), (5, 333), (16, 4096), (16, 14336), (64, 14336), (100, 1000),
                                 (128, 4096), (200, 4096), (256, 1024)])
def test_preconditioner_matches_oracle(gpu, r, K):
    print(f"[precond] r={r} K={K}", flush=True)
    A = workloads.normal_f32((r, K), 1.0 / r, workloads.SEED_A + r, "cuda")
    P = gpu.lorafa_preconditioner(A)
    P2 = gpu.lorafa_preconditioner(A)
    torch.cuda.synchronize()
    _check_precond(_np(P), _np(A), f"P r={r} K={K}")
    assert torch.equal(P, P2), "preconditioner not run-to-run identical"


def test_preconditioner_degenerate_adapters(gpu):
    """A = 0 (pure damping, P = 1e8 I) and duplicated rows (singular Gram
    matrix made invertible only by the damping)."""
    Z = torch.zeros((4, 300), dtype=torch.float32, device="cuda")
    Pz = _np(gpu.lorafa_preconditioner(Z))
    np.testing.assert_array_equal(Pz, np.eye(4, dtype=np.float32) * np.float32(1e8))
    row = workloads.normal_f32((1, 640), 0.05, 91, "cuda")
    A = torch.cat([row, row, workloads.normal_f32((6, 640), 0.05, 92, "cuda")])
    _check_precond(_np(gpu.lorafa_preconditioner(A)), _np(A), "P duplicate rows")


def _state(shape, seed, zero_moments: bool):
    st = workloads.adamw_state(shape, seed, device="cuda")
    if zero_moments:
        st["m"].zero_()
        st["v"].zero_()
    st["p"] = workloads.normal_f32(shape, 0.02, 500 + seed, "cuda")
    return st


def _lora_case(gpu, r, K, N, step, gs_value, fa, precond, seed=0):
    zero = step == 1
    sA = None if fa else _state((r, K), seed, zero)
    sB = _state((N, r), seed + 1, zero)
    host = {k: {n: _np(t) for n, t in st.items()} for k, st in (("A", sA), ("B", sB)) if st is not None}
    s = 2.0
    P = Pn = None
    if precond:
        # The oracle's preconditioner, rounded to fp32, is the input of both
        # sides (the device's own preconditioner is checked on its own above).
        Af = workloads.normal_f32((r, K), 1.0 / r, workloads.SEED_A, "cpu")
        Pn = oracle.lorafa_preconditioner(_np(Af)).astype(np.float32)
        P = torch.from_numpy(Pn).to("cuda")
    gs = None if gs_value is None else torch.full((1,), gs_value, dtype=torch.float32, device="cuda")
    kw = {}
    if sA is not None:
        kw = dict(A=sA["p"], dA=sA["g"], mA=sA["m"], vA=sA["v"])
    gpu.lora_adamw_step(sB["p"], sB["g"], sB["m"], sB["v"], step=step, precond=P, s=s, grad_scale=gs, **HP, **kw)
    torch.cuda.synchronize()
    gsv = 1.0 if gs_value is None else gs_value
    hB = host["B"]
    ref = oracle.lora_adamw_step(hB["p"], hB["g"], hB["m"], hB["v"], P=Pn, s=s, step=step, grad_scale=gsv,
                                 **({} if fa else dict(A=host["A"]["p"], dA=host["A"]["g"], mA=host["A"]["m"],
                                                       vA=host["A"]["v"])), **HP)
    worst = 0.0
    if not fa:
        hA = host["A"]
        g = hA["g"].astype(np.float64) * gsv
        b = adamw_bounds(hA["p"], g, hA["m"], hA["v"], U32 * np.abs(g), HP, step)
        for name, key, bd in zip(("A", "mA", "vA"), ("p", "m", "v"), b):
            worst = max(worst, assert_within(_np(sA[key]), ref[name], bd, f"{name} r={r} K={K} t={step}"))
    if P is not None:
        g = oracle.lorafa_precondition(hB["g"].astype(np.float64) * gsv, Pn, s)
        e_g = (r + 3) * U32 * (np.abs(hB["g"].astype(np.float64)) * gsv) @ np.abs(Pn.astype(np.float64)) / (s * s)
    else:
        g = hB["g"].astype(np.float64) * gsv
        e_g = U32 * np.abs(g)
    b = adamw_bounds(hB["p"], g, hB["m"], hB["v"], e_g, HP, step)
    for name, key, bd in zip(("B", "mB", "vB"), ("p", "m", "v"), b):
        worst = max(worst, assert_within(_np(sB[key]), ref[name], bd, f"{name} r={r} N={N} t={step}"))
    return worst


@pytest.mark.parametrize("r,K,N", [(16, 4096, 4096), (16, 4096, 14336), (5, 333, 77), (1, 3, 5), (64, 14336, 4096)])
@pytest.mark.parametrize("step,gs", [(1, None), (7, 0.5), (100000, None)])
def test_lora_adamw_matches_oracle(gpu, r, K, N, step, gs):
    print(f"[adamw lora] r={r} K={K} N={N} step={step} gs={gs}", flush=True)
    _lora_case(gpu, r, K, N, step, gs, fa=False, precond=False)


@pytest.mark.parametrize("r,K,N", [(16, 4096, 4096), (2, 576, 576), (6, 100, 37), (64, 14336, 4096),
                                   (256, 1024, 300), (3, 64, 1)])
@pytest.mark.parametrize("step,gs", [(1, None), (9, 0.25)])
def test_lorafa_preconditioned_step_matches_oracle(gpu, r, K, N, step, gs):
    print(f"[adamw lorafa] r={r} K={K} N={N} step={step} gs={gs}", flush=True)
    _lora_case(gpu, r, K, N, step, gs, fa=True, precond=True)


def test_lorafa_without_preconditioner_updates_b_only(gpu):
    _lora_case(gpu, 8, 256, 129, 3, None, fa=True, precond=False)


def test_chained_steps_follow_the_oracle(gpu):
    """Three updates in a row: the device chains its fp32 state, the oracle
    chains its own fp64 state from the same seeded start, and each step's
    bound carries the previous step's bound forward."""
    r, K, N = 16, 1024, 768
    sA, sB = _state((r, K), 40, True), _state((N, r), 41, True)
    ref = {n: _np(x).astype(np.float64) for n, x in (("A", sA["p"]), ("mA", sA["m"]), ("vA", sA["v"]),
                                                      ("B", sB["p"]), ("mB", sB["m"]), ("vB", sB["v"]))}
    carried = {"A": (0.0, 0.0, 0.0), "B": (0.0, 0.0, 0.0)}
    for t in range(1, 4):
        dA = workloads.normal_f32((r, K), 1e-3, 700 + t, "cuda")
        dB = workloads.normal_f32((N, r), 1e-3, 800 + t, "cuda")
        gpu.lora_adamw_step(sB["p"], dB, sB["m"], sB["v"], step=t, A=sA["p"], dA=dA, mA=sA["m"], vA=sA["v"], **HP)
        torch.cuda.synchronize()
        new = oracle.lora_adamw_step(ref["B"], _np(dB), ref["mB"], ref["vB"], A=ref["A"], dA=_np(dA),
                                     mA=ref["mA"], vA=ref["vA"], step=t, **HP)
        for side, g, st in (("A", _np(dA), sA), ("B", _np(dB), sB)):
            g64 = g.astype(np.float64)
            b = adamw_bounds(ref[side], g64, ref["m" + side], ref["v" + side], U32 * np.abs(g64), HP, t,
                             e_state=carried[side])
            for key, name, bd in zip(("p", "m", "v"), (side, "m" + side, "v" + side), b):
                assert_within(_np(st[key]), new[name], bd, f"{name} t={t}")
            carried[side] = b
        ref = new


def test_llama8b_layer_adapters_one_update(gpu):
    """All seven rank-16 adapters of the Llama-8B-shaped layer, one
    lora_adamw_step call each."""
    for i, L in enumerate(workloads.WORKLOADS["llama8b_layer"]["layers"]):
        print(f"[adamw llama8b] {L.name}", flush=True)
        _lora_case(gpu, L.lora_rank, L.k_in, L.n_out, 5, None, fa=False, precond=False, seed=20 + 2 * i)


def _adapter(r, K, N, fa, precond, seed):
    d = {}
    st = _state((N, r), seed, False)
    d.update(B=st["p"], dB=st["g"], mB=st["m"], vB=st["v"])
    if not fa:
        sa = _state((r, K), seed + 1, False)
        d.update(A=sa["p"], dA=sa["g"], mA=sa["m"], vA=sa["v"])
    if precond:
        d.update(precond=gpu_precond(r, K, seed), s=2.0)
    return d


def gpu_precond(r, K, seed):
    from qlora_adapter_amd import nf4lora
    return nf4lora.lorafa_preconditioner(workloads.normal_f32((r, K), 1.0 / r, 900 + seed, "cuda"))


def test_many_adapters_in_one_launch_equal_separate_calls(gpu):
    """lora_adamw_step_many over a mixed set (LoRA, LoRA-FA with and without
    the preconditioner, r % 4 != 0, ragged sizes) is bit-identical to one
    lora_adamw_step call per adapter."""
    specs = [(16, 4096, 4096, False, False), (5, 333, 77, False, False), (16, 1024, 512, True, True),
             (6, 100, 37, True, True), (8, 256, 129, True, False), (64, 14336, 4096, False, False),
             (1, 3, 5, False, False)]
    many = [_adapter(*sp, seed=10 * i) for i, sp in enumerate(specs)]
    single = [{k: v.clone() for k, v in ad.items() if isinstance(v, torch.Tensor)} | {"s": ad.get("s", 0.0)}
              for ad in many]
    gs = torch.full((1,), 0.75, dtype=torch.float32, device="cuda")
    gpu.lora_adamw_step_many(many, step=4, grad_scale=gs, **HP)
    for ad in single:
        kw = {k: ad[k] for k in ("A", "dA", "mA", "vA") if k in ad}
        gpu.lora_adamw_step(ad["B"], ad["dB"], ad["mB"], ad["vB"], step=4, precond=ad.get("precond"), s=ad["s"],
                            grad_scale=gs, **kw, **HP)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(many, single)):
        for k in ("A", "mA", "vA", "B", "mB", "vB"):
            if k in a:
                assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), (i, k)


def test_llama8b_layer_adapters_one_launch(gpu):
    """The seven rank-16 adapters of the Llama-8B-shaped layer in one launch
    (the benchmark's call), each checked against the oracle."""
    layers = workloads.WORKLOADS["llama8b_layer"]["layers"]
    ads, host = [], []
    for i, L in enumerate(layers):
        ad = _adapter(L.lora_rank, L.k_in, L.n_out, False, False, seed=300 + 10 * i)
        ads.append(ad)
        host.append({k: _np(v) for k, v in ad.items()})
    gpu.lora_adamw_step_many(ads, step=3, **HP)
    torch.cuda.synchronize()
    for L, ad, h in zip(layers, ads, host):
        print(f"[adamw many] {L.name}", flush=True)
        ref = oracle.lora_adamw_step(h["B"], h["dB"], h["mB"], h["vB"], A=h["A"], dA=h["dA"], mA=h["mA"],
                                     vA=h["vA"], step=3, **HP)
        for side in ("A", "B"):
            g = h["d" + side].astype(np.float64)
            b = adamw_bounds(h[side], g, h["m" + side], h["v" + side], U32 * np.abs(g), HP, 3)
            for key, name, bd in zip((side, "m" + side, "v" + side), (side, "m" + side, "v" + side), b):
                assert_within(_np(ad[key]), ref[name], bd, f"{L.name} {name}")


def _to_pinned(t: torch.Tensor) -> torch.Tensor:
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


@pytest.mark.parametrize("page_bytes", [4096, 2 << 20])
def test_paged_moments_equal_device_moments(gpu, page_bytes):
    """lora_adamw_step_paged with the moments in pinned host memory (read and
    written in place by the update kernel) gives the same parameters and
    moments as lora_adamw_step_many, bit for bit: LoRA, LoRA-FA with the preconditioner (r % 4 == 0 and r = 6), and
    tensors spanning many 4 KiB pages."""
    specs = [(16, 4096, 4096, False, False), (5, 333, 77, False, False), (16, 1024, 512, True, True),
             (6, 100, 37, True, True), (64, 14336, 4096, False, False)]
    dev_ads = [_adapter(*sp, seed=40 + 10 * i) for i, sp in enumerate(specs)]
    paged = []
    for ad in dev_ads:
        q = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in ad.items()}
        for k in ("mA", "vA", "mB", "vB"):
            if k in q:
                q[k] = _to_pinned(q[k])
        paged.append(q)
    staging = torch.empty(2 * page_bytes, dtype=torch.uint8, device="cuda")
    gs = torch.full((1,), 0.5, dtype=torch.float32, device="cuda")
    for step in (1, 2):
        gpu.lora_adamw_step_many(dev_ads, step=step, grad_scale=gs, **HP)
        gpu.lora_adamw_step_paged(paged, step=step, grad_scale=gs, staging=staging, page_bytes=page_bytes, **HP)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(dev_ads, paged)):
            for k in ("A", "mA", "vA", "B", "mB", "vB"):
                if k in a:
                    assert torch.equal(a[k].cpu().view(torch.int32), b[k].cpu().view(torch.int32)), (i, k, step)


@pytest.mark.parametrize("page_bytes", [4096, 2 << 20])
def test_paged_chain_follows_oracle(gpu, page_bytes):
    """Two chained lora_adamw_step_paged updates (moments in pinned host
    memory, page by page) against the fp64 oracle chaining its own state from
    the same start: a LoRA adapter (A and B) and a LoRA-FA adapter with the
    preconditioner (B only), with a gradient scale; each step's bound carries
    the previous step's forward (e_state)."""
    print(f"[adamw paged chain] page_bytes={page_bytes}", flush=True)
    r, K, N = 16, 1024, 768
    rf, Kf, Nf, sf = 6, 100, 37, 2.0
    sA, sB = _state((r, K), 60, True), _state((N, r), 61, True)
    sF = _state((Nf, rf), 62, True)
    Af = workloads.normal_f32((rf, Kf), 1.0 / rf, workloads.SEED_A + 7, "cpu")
    Pn = oracle.lorafa_preconditioner(_np(Af)).astype(np.float32)
    P = torch.from_numpy(Pn).to("cuda")
    ref = {n: _np(x).astype(np.float64) for n, x in (("A", sA["p"]), ("mA", sA["m"]), ("vA", sA["v"]),
                                                      ("B", sB["p"]), ("mB", sB["m"]), ("vB", sB["v"]),
                                                      ("F", sF["p"]), ("mF", sF["m"]), ("vF", sF["v"]))}
    host = {k: _to_pinned(st["m" if k[0] == "m" else "v"]) for k, st in (("mA", sA), ("vA", sA), ("mB", sB),
                                                                          ("vB", sB), ("mF", sF), ("vF", sF))}
    staging = torch.empty(2 * page_bytes, dtype=torch.uint8, device="cuda")
    gsv = 0.5
    gs = torch.full((1,), gsv, dtype=torch.float32, device="cuda")
    carried = {k: (0.0, 0.0, 0.0) for k in ("A", "B", "F")}
    for t in (1, 2):
        dA = workloads.normal_f32((r, K), 1e-3, 710 + t, "cuda")
        dB = workloads.normal_f32((N, r), 1e-3, 810 + t, "cuda")
        dF = workloads.normal_f32((Nf, rf), 1e-3, 910 + t, "cuda")
        ads = [dict(A=sA["p"], dA=dA, mA=host["mA"], vA=host["vA"], B=sB["p"], dB=dB, mB=host["mB"], vB=host["vB"]),
               dict(B=sF["p"], dB=dF, mB=host["mF"], vB=host["vF"], precond=P, s=sf)]
        gpu.lora_adamw_step_paged(ads, step=t, grad_scale=gs, staging=staging, page_bytes=page_bytes, **HP)
        torch.cuda.synchronize()
        new = oracle.lora_adamw_step(ref["B"], _np(dB), ref["mB"], ref["vB"], A=ref["A"], dA=_np(dA), mA=ref["mA"],
                                     vA=ref["vA"], step=t, grad_scale=gsv, **HP)
        newf = oracle.lora_adamw_step(ref["F"], _np(dF), ref["mF"], ref["vF"], P=Pn, s=sf, step=t, grad_scale=gsv,
                                      **HP)
        got = {"A": _np(sA["p"]), "mA": host["mA"].numpy(), "vA": host["vA"].numpy(), "B": _np(sB["p"]),
               "mB": host["mB"].numpy(), "vB": host["vB"].numpy(), "F": _np(sF["p"]), "mF": host["mF"].numpy(),
               "vF": host["vF"].numpy()}
        grads = {"A": _np(dA).astype(np.float64) * gsv, "B": _np(dB).astype(np.float64) * gsv}
        for side in ("A", "B"):
            g = grads[side]
            b = adamw_bounds(ref[side], g, ref["m" + side], ref["v" + side], U32 * np.abs(g), HP, t,
                             e_state=carried[side])
            for name, bd in zip((side, "m" + side, "v" + side), b):
                assert_within(got[name], new[name], bd, f"paged {name} t={t}")
            carried[side] = b
        gF = _np(dF).astype(np.float64) * gsv
        g = oracle.lorafa_precondition(gF, Pn, sf)
        e_g = (rf + 3) * U32 * np.abs(gF) @ np.abs(Pn.astype(np.float64)) / (sf * sf)
        b = adamw_bounds(ref["F"], g, ref["mF"], ref["vF"], e_g, HP, t, e_state=carried["F"])
        for name, key, bd in zip(("F", "mF", "vF"), ("B", "mB", "vB"), b):
            assert_within(got[name], newf[key], bd, f"paged LoRA-FA {name} t={t}")
        carried["F"] = b
        ref = dict(new, F=newf["B"], mF=newf["mB"], vF=newf["vB"])


def test_paged_moments_reject_pageable_memory(gpu):
    ad = _adapter(8, 64, 32, False, False, seed=3)
    ad["mB"] = ad["mB"].cpu()  # pageable host memory
    ad["vB"] = _to_pinned(ad["vB"])
    ad["mA"], ad["vA"] = _to_pinned(ad["mA"]), _to_pinned(ad["vA"])
    staging = torch.empty(8192, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        gpu.lora_adamw_step_paged([ad], step=1, staging=staging, page_bytes=4096, **HP)
