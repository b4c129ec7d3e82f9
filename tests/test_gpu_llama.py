"""GPU parity of the assembled decoder step (qlora_adapter_amd/llama.py: one
layer's forward and backward, and the whole checkpointed training step)
against the oracle's layer (oracle/llama.py decoder_layer) composed on the
CPU on the same seeded inputs.

Soup, "NF4 Layer Streaming - Gate results": full training step of a
Llama-shaped model with an NF4 base and LoRA on q_proj and v_proj, layers
checkpointed. The GPU quantizes every weight itself; the oracle quantizes the
same fp32 weights and multiplies its own decoded values (bf16-rounded on the
bf16 path). On the bf16 path the oracle rounds every stored activation to bf16
where the GPU stores one; since a tiny difference before a rounding can become
a whole ulp after it, a bf16 composition is held to the bf16 oracle's own
accuracy (check_bf16_chain). The fp32 path (fp32 activations) is held to
relative Frobenius 1e-4 over the chain of about twenty fp32 operations.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import llama as OL
from tests.parity import assert_close, rel_frob, to_np

pytestmark = pytest.mark.gpu

F32_CHAIN = 1e-4
ALL = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")


def small_cfg(llama, targets, layers=1, vocab=1000):
    return llama.LlamaConfig(hidden=256, heads=4, kv_heads=2, head_dim=64, ffn=512, vocab=vocab, layers=layers,
                             lora_rank=8, lora_alpha=16.0, lora_targets=tuple(targets))


def make_layer(llama, cfg, seed):
    """Seeded fp32 weights (std 0.05), norm weights 1 + N(0, 0.2), A ~ N(0, 1/r),
    B ~ N(0, 0.05) so the adapter path is active; returns the GPU layer and the
    fp32 host copies."""
    W = {n: workloads.normal_f32(cfg.shape(n), 0.05, workloads.weight_seed(100 * seed + j), "cuda")
         for j, n in enumerate(ALL)}
    g1 = 1 + workloads.normal_f32((cfg.hidden,), 0.2, 7000 + seed, "cuda")
    g2 = 1 + workloads.normal_f32((cfg.hidden,), 0.2, 7001 + seed, "cuda")
    r = cfg.lora_rank
    ad = {n: (workloads.normal_f32((r, cfg.shape(n)[1]), 1.0 / r, 8000 + 10 * seed + j, "cuda"),
              workloads.normal_f32((cfg.shape(n)[0], r), 0.05, 9000 + 10 * seed + j, "cuda"))
          for j, n in enumerate(cfg.lora_targets)}
    host = dict(W={n: w.cpu().numpy() for n, w in W.items()}, g1=g1.cpu().numpy(), g2=g2.cpu().numpy(),
                A={n: a.cpu().numpy() for n, (a, _) in ad.items()}, B={n: b.cpu().numpy() for n, (_, b) in ad.items()})
    return llama.Layer(cfg, W, g1, g2, ad), host


def decoded(orc, w, bf16):
    q = orc.quantize(w, True)
    if bf16:
        return orc.bf16_bits_to_f32(orc.dequantize(q, "bf16")).reshape(w.shape)
    return orc.dequantize(q, "f32").reshape(w.shape)


def oracle_params(orc, host, targets, bf16):
    """The oracle layer's parameters: every projection's decoded weight, taken
    from the matrix it is stored in (the model packs q/k/v and gate/up as one
    NF4 matrix each, so the oracle quantizes the same stacks and slices them)."""
    from qlora_adapter_amd import llama
    p = {}
    for mem in llama.STACKS.values():
        w = np.concatenate([host["W"][n] for n in mem])
        dw = decoded(orc, w, bf16)
        off = 0
        for n in mem:
            rows = host["W"][n].shape[0]
            p["W_" + n] = dw[off:off + rows]
            off += rows
    p["gamma1"], p["gamma2"] = host["g1"], host["g2"]
    for n in targets:
        p["A_" + n], p["B_" + n] = host["A"][n], host["B"][n]
    return p


def oracle_cfg(cfg, s):
    return dict(heads=cfg.heads, kv_heads=cfg.kv_heads, head_dim=cfg.head_dim, eps=cfg.eps, theta=cfg.theta,
                s=float(s), targets=tuple(cfg.lora_targets))


def close(got, ref, dt, what):
    if dt == "bf16":
        return assert_close(got, ref, "bf16", what)
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), what
    fro = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert fro <= F32_CHAIN, f"{what}: rel frob {fro:.3e} > {F32_CHAIN}"
    return fro


@pytest.mark.parametrize("dt,targets,S", [("bf16", ("q_proj", "v_proj"), 96), ("f32", ("q_proj", "v_proj"), 96),
                                          ("bf16", ALL, 130), ("f32", ALL, 37)])
def test_layer_forward_backward(gpu, orc, dt, targets, S):
    """One layer: output x2 + dn, the mid residual x2, the input gradient and
    every adapter's dA, dB, for a ragged token count (several attention key
    blocks and a partial one)."""
    print(f"[llama] layer {dt} targets={len(targets)} S={S}", flush=True)
    from qlora_adapter_amd import llama
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    cfg = small_cfg(llama, targets)
    L, host = make_layer(llama, cfg, seed=S)
    m = llama.LlamaNF4(cfg, S, dtype=dtype, layers=[L], with_head=False)
    xin = workloads.normal_f32((S, cfg.hidden), 1.0, 11, "cuda").to(dtype)
    res = workloads.normal_f32((S, cfg.hidden), 0.5, 12, "cuda").to(dtype)
    dout = workloads.normal_f32((S, cfg.hidden), 1.0, 13, "cuda").to(dtype)
    x_sum = torch.empty_like(xin)
    x2, dn = m.layer_forward(L, xin, res, x_out=x_sum)
    out = gpu.add(x2, dn)
    x2 = x2.clone()
    dx = m.layer_backward(L, dout, torch.empty_like(xin))
    torch.cuda.synchronize()
    p = oracle_params(orc, host, targets, dt == "bf16")
    args = (p, to_np(xin), to_np(res), to_np(dout), oracle_cfg(cfg, m.s))
    got = {"x2": to_np(x2), "out": to_np(out), "dx": to_np(dx)}
    for n in targets:
        got[f"{n} dA"], got[f"{n} dB"] = L.lora[n]["dA"].cpu().numpy(), L.lora[n]["dB"].cpu().numpy()
    if dt == "f32":
        ref = flat(OL.decoder_layer(*args, bf16=False), targets)
        for what, g in got.items():
            close(g, ref[what], dt, what)
    else:
        check_bf16_chain(got, flat(OL.decoder_layer(*args, bf16=True), targets),
                         flat(OL.decoder_layer(*args, bf16=False), targets))


def flat(r, targets):
    out = {"x2": r["x2"], "out": r["out"], "dx": r["dx"]}
    for n in targets:
        out[f"{n} dA"], out[f"{n} dB"] = r["grads"][n]
    return out


def check_bf16_chain(got, ref16, ref64):
    """A composition of bf16-stored steps against the oracle: a difference far
    below one ulp before a rounding becomes a whole ulp after it, and the
    matrix-core attention also rounds its probabilities to bf16, so the GPU
    result is held to the bf16 oracle's own accuracy: its distance to the same
    chain without activation rounding at most 1.5x the oracle's, plus 1e-3."""
    for what, g in got.items():
        assert np.all(np.isfinite(g)), what
        e_gpu, e_orc = rel_frob(g, ref64[what]), rel_frob(ref16[what], ref64[what])
        print(f"{what}: gpu {e_gpu:.2e} oracle-bf16 {e_orc:.2e}", flush=True)
        assert e_gpu <= 1.5 * e_orc + 1e-3, (what, e_gpu, e_orc)


def test_recompute_is_bitwise(gpu):
    """Running a layer's forward again from its saved input reproduces every
    activation bit for bit (the checkpointed backward relies on it)."""
    from qlora_adapter_amd import llama
    cfg = small_cfg(llama, ("q_proj", "v_proj"))
    L, _ = make_layer(llama, cfg, seed=3)
    S = 77
    m = llama.LlamaNF4(cfg, S, layers=[L], with_head=False)
    x = workloads.normal_f32((S, cfg.hidden), 1.0, 14, "cuda").to(torch.bfloat16)
    m.layer_forward(L, x)
    first = {k: v.clone() for k, v in m.b.items()}
    m.layer_forward(L, x)
    torch.cuda.synchronize()
    for k in ("h1", "qkv", "a", "lse", "o", "x2", "h2", "gu", "sw", "dn"):
        assert torch.equal(first[k], m.b[k]), k


def oracle_step(orc, ps, emb, Wlm_d, gfn, tgt, ocfg, eps, bf16):
    """The oracle's step: forward through the layers keeping each layer's
    input, final add + RMSNorm, lm_head, mean cross-entropy, then the lm_head
    and final-norm backward and each layer's backward in reverse. With bf16
    every stored activation is rounded as the GPU stores it."""
    rb = OL._bf16 if bf16 else (lambda a: np.asarray(a, np.float64))
    zero = np.zeros_like(emb, dtype=np.float64)
    xs, x, res = [], emb.astype(np.float64), None
    for p in ps:
        xs.append((x, res))
        r = OL.decoder_layer(p, x, res, zero, ocfg, bf16=bf16)
        x, res = r["x2"], r["dn"]
    h_in = r["out"]  # the final norm's fused add of the last layer's x2 and dn
    hf = rb(OL.rmsnorm(h_in, gfn, eps)[0])
    logits = rb(orc.linear_fwd(hf, Wlm_d)[0])
    loss, dlogits = OL.cross_entropy(logits, tgt)
    dhf = rb(orc.linear_bwd_input(rb(dlogits), Wlm_d)[0])
    g = rb(OL.rmsnorm_bwd(dhf, h_in, gfn, eps))
    grads = [None] * len(ps)
    for i in reversed(range(len(ps))):
        r = OL.decoder_layer(ps[i], *xs[i], g, ocfg, bf16=bf16)
        grads[i] = r["grads"]
        g = r["dx"]
    return loss, grads


def test_training_step(gpu, orc):
    """Two layers with embedding, final norm, lm_head and mean cross-entropy:
    the loss and every adapter gradient of the checkpointed GPU step against
    the oracle's forward pass followed by its layer-by-layer backward; then
    the AdamW update moves every adapter."""
    print("[llama] two-layer training step", flush=True)
    from qlora_adapter_amd import llama
    cfg = small_cfg(llama, ("q_proj", "v_proj"), layers=2, vocab=1000)
    S = 96
    layers, hosts = zip(*[make_layer(llama, cfg, seed=40 + i) for i in range(2)])
    E = workloads.normal_f32((cfg.vocab, cfg.hidden), 0.5, 15, "cuda")
    Wlm = workloads.normal_f32((cfg.vocab, cfg.hidden), 0.05, 16, "cuda")
    gf = 1 + workloads.normal_f32((cfg.hidden,), 0.2, 17, "cuda")
    m = llama.LlamaNF4(cfg, S, layers=list(layers), head_weights=(E, Wlm, gf))
    ids = torch.randint(0, cfg.vocab, (S,), generator=torch.Generator().manual_seed(18)).cuda()
    tgt = torch.randint(0, cfg.vocab, (S,), generator=torch.Generator().manual_seed(19)).cuda()
    B0 = [ad["B"].clone() for ad in m.adapters()]
    loss = m.forward_backward(ids, tgt)
    torch.cuda.synchronize()
    # per projection: its views inside the layer's stacked adapter
    grads = [[(L.lora[n]["dA"].cpu().numpy(), L.lora[n]["dB"].cpu().numpy()) for n in cfg.lora_targets]
             for L in layers]

    ocfg = oracle_cfg(cfg, m.s)
    ps = [oracle_params(orc, h, cfg.lora_targets, True) for h in hosts]
    emb = orc.bf16_bits_to_f32(orc.embedding_rows(orc.quantize(E.cpu().numpy(), True), cfg.hidden,
                                                  ids.cpu().numpy(), "bf16"))
    Wlm_d = decoded(orc, Wlm.cpu().numpy(), True)
    l16, g16 = oracle_step(orc, ps, emb, Wlm_d, gf.cpu().numpy(), tgt.cpu().numpy(), ocfg, cfg.eps, True)
    l64, g64 = oracle_step(orc, ps, emb, Wlm_d, gf.cpu().numpy(), tgt.cpu().numpy(), ocfg, cfg.eps, False)
    # the loss is an fp32 mean of per-token terms of bf16 logits on both sides
    assert abs(float(loss.item()) - l16) <= 1e-3 * abs(l16), (float(loss.item()), l16)
    # through two layers of bf16 storage the adapter gradients carry about 1%
    # rounding noise on both sides (check_bf16_chain)
    got, r16, r64 = {}, {}, {}
    for i in range(len(ps)):
        for t, n in enumerate(cfg.lora_targets):
            for j, name in ((0, "dA"), (1, "dB")):
                key = f"layer {i} {n} {name}"
                got[key], r16[key], r64[key] = grads[i][t][j], g16[i][n][j], g64[i][n][j]
    check_bf16_chain(got, r16, r64)
    m.optimizer_step(lr=1e-3)
    torch.cuda.synchronize()
    for b0, ad in zip(B0, m.adapters()):
        assert not torch.equal(b0, ad["B"])


def test_layer_full_width(gpu, orc):
    """One layer at the Llama-3.1-8B width (hidden 4096, 32 query and 8 key/value
    heads of 128, FFN 14336, LoRA r = 16 on q_proj and v_proj) for 64 tokens,
    bf16: the output, input gradient and adapter gradients (check_bf16_chain)."""
    print("[llama] full-width layer, 64 tokens", flush=True)
    from qlora_adapter_amd import llama
    cfg = llama.LlamaConfig(layers=1)
    S = 64
    L, host = make_layer(llama, cfg, seed=5)
    m = llama.LlamaNF4(cfg, S, layers=[L], with_head=False)
    xin = workloads.normal_f32((S, cfg.hidden), 1.0, 21, "cuda").to(torch.bfloat16)
    res = workloads.normal_f32((S, cfg.hidden), 0.5, 22, "cuda").to(torch.bfloat16)
    dout = workloads.normal_f32((S, cfg.hidden), 1.0, 23, "cuda").to(torch.bfloat16)
    x2, dn = m.layer_forward(L, xin, res, x_out=torch.empty_like(xin))
    out = gpu.add(x2, dn)
    dx = m.layer_backward(L, dout, torch.empty_like(xin))
    torch.cuda.synchronize()
    p = oracle_params(orc, host, cfg.lora_targets, True)
    args = (p, to_np(xin), to_np(res), to_np(dout), oracle_cfg(cfg, m.s))
    got = {"out": to_np(out), "dx": to_np(dx)}
    for n in cfg.lora_targets:
        got[f"{n} dA"], got[f"{n} dB"] = L.lora[n]["dA"].cpu().numpy(), L.lora[n]["dB"].cpu().numpy()
    check_bf16_chain(got, flat(OL.decoder_layer(*args, bf16=True), cfg.lora_targets),
                     flat(OL.decoder_layer(*args, bf16=False), cfg.lora_targets))


def test_llama8b_step_invariants(gpu):
    """The 32-layer Llama-3.1-8B-shaped step at 512 tokens, as the benchmark
    runs it: finite loss; with B = 0 at the start every dA is exactly zero
    (dY B = 0) and every dB is finite and nonzero; the first AdamW update
    (no weight decay) leaves every A bit for bit and moves every B entry by at
    most lr; repeating the step on the same batch lowers the loss."""
    print("[llama] 8B-shaped step invariants", flush=True)
    from qlora_adapter_amd import llama
    cfg = llama.LlamaConfig()
    S, lr = 512, 1e-3
    m = llama.LlamaNF4(cfg, S)
    g = torch.Generator().manual_seed(31)
    ids = torch.randint(0, cfg.vocab, (S + 1,), generator=g).cuda()
    x, y = ids[:-1].clone(), ids[1:].clone()
    A0 = [ad["A"].clone() for ad in m.adapters()]
    loss0 = float(m.forward_backward(x, y).item())
    assert np.isfinite(loss0)
    for ad in m.adapters():
        assert torch.count_nonzero(ad["dA"]) == 0
        assert torch.isfinite(ad["dB"]).all() and torch.count_nonzero(ad["dB"]) > 0
    m.optimizer_step(lr=lr)
    torch.cuda.synchronize()
    for a0, ad in zip(A0, m.adapters()):
        assert torch.equal(a0, ad["A"])
        assert float(ad["B"].abs().max()) <= lr * (1 + 1e-5)
    losses = [loss0]
    for _ in range(3):
        losses.append(float(m.train_step(x, y, lr=lr).item()))
    print("losses", losses, flush=True)
    assert all(np.isfinite(losses)) and losses[-1] < losses[0], losses
