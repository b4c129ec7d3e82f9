"""Benchmark of the NF4 double-quant + LoRA hot path on one MI355X.

One step = the whole path over one batch of the Llama-8B-shaped decoder layer
(hidden 4096, kv 1024, intermediate 14336; q/k/v/o/gate/up/down, 4096 tokens,
LoRA r = 16, alpha = 32 on all 7 projections), per projection:
  nf4_quantize (absmax + NF4 codes + double quantization of the fp32 weight)
  nf4_linear_fwd (fused dequant-GEMM + LoRA side path)
  nf4_linear_bwd_input (fused dequant-GEMM through the frozen base + LoRA)
  lora_grad (dA, dB)
  lora_adamw_step_many (fused AdamW update of A and B of all seven adapters in
  one launch, fp32 masters and moments)
  nf4_dequantize_many (packed -> bf16, all seven matrices in one launch)
with every input already resident in device memory. Prints one JSON line.
Outside the timed step it also runs the standalone quantize/dequantize
throughput workload (7.5e9 parameters, cold passes; its dequant rate is the
reported dequant roofline), times the LoRA-FA variant of the optimizer
step (lorafa_preconditioner once per adapter, then the preconditioned update of
B) on the rank-64 down_proj shape, times the selected-row decode of packed
embedding tables (nf4_embedding_rows) and the AdamW update with paged host
moments (lora_adamw_step_paged), and reports the other configurations of
the workload table (the 576x576 layer, the SmolLM2 stack, the backward-heavy
rank-64 down_proj).

value = algorithmic FLOPs of the step (4MNK + 6Mr(N+K) per projection) /
step time: whole-step throughput including the quantize and dequantize work.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
ADAMW = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)  # adapter learning rate of the pages
ADAMW_BYTES = 28  # per parameter: p, g, m, v read (16 B) and p, m, v written (12 B), fp32


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=800, help="token rows of the oracle sample")
    p.add_argument("--no-ceilings", action="store_true", help="skip the same-session copy / library GEMM ceilings")
    p.add_argument("--no-throughput", action="store_true",
                   help="skip the 7.5e9-parameter quantize/dequantize throughput pass")
    p.add_argument("--no-decoder-step", action="store_true",
                   help="skip the 32-layer Llama-8B-shaped training step (tokens/s)")
    p.add_argument("--decoder-step-only", action="store_true",
                   help="only the Llama-8B-shaped training step (--steps timed after --warmup), for profiling")
    p.add_argument("--throughput-only", action="store_true",
                   help="only the 7.5e9-parameter quantize/dequantize pass (one timed pass; for counter runs)")
    p.add_argument("--gemm-sustained-only", action="store_true",
                   help="only the back-to-back fused calls of gate_proj and down_proj (for profiling)")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run device-to-device copies of a known size (counter calibration for rocprofv3)")
    return p.parse_args()


COPY_PROBE_BYTES = 1 << 30  # 1 GiB read + 1 GiB written per copy


def copy_probe():
    """Plain device copies of a known size: under rocprofv3 --pmc FETCH_SIZE /
    WRITE_SIZE they give the factor between counter KiB and true bytes."""
    import torch
    a = torch.empty(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "copies": 3}), flush=True)


def ceilings():
    """Same-session ceilings (context, never the metric): a 2 GiB device copy
    and torch's bf16 GEMM (hipBLASLt) at the gate_proj shape 4096x4096x14336."""
    import torch
    a = torch.empty(1 << 29, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * a.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    x = torch.randn(4096, 4096, dtype=torch.bfloat16, device="cuda")
    w = torch.randn(14336, 4096, dtype=torch.bfloat16, device="cuda").t().contiguous()
    for _ in range(3):
        x @ w
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        x @ w
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 10 * 2 * 4096 * 4096 * 14336 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    return {"device_copy_GBps": round(copy_gbps, 1), "torch_bf16_gemm_TFLOPs_4096x4096x14336": round(gemm_tf, 1),
            "note": "measured in this run; context only (torch's GEMM multiplies dense bf16 weights)"}


def _counter_summary(name: str, sources):
    """key = value lines of a rocprofv3 counter summary under profiles/, or None
    when the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    h = hashlib.sha256()
    for s in sources:
        h.update(open(os.path.join(ROOT, "qlora_adapter_amd", "csrc", s), "rb").read())
    return kv if kv.get("kernel_source_sha256") == h.hexdigest() else None


def counter_traffic(kernel: str):
    """HBM-side bytes per forward / input-gradient call (all its dispatches,
    averaged over the layer's 4 calls of that kind: q, k, v and gate, up
    grouped or summed, o and down alone) from the rocprofv3
    FETCH_SIZE / WRITE_SIZE summary under profiles/, scaled by the copy-probe
    calibration; None when the kernel sources changed since the counters."""
    kv = _counter_summary("fused_gemm_counters_llama8b_layer.txt", ("nf4_gemm_fast.hip", "nf4_linear.hip"))
    key = "fwd" if kernel == "nf4_linear_fwd" else "bwd"
    try:
        return float(kv[f"{key}_hbm_bytes_per_launch"]) if kv else None
    except KeyError:
        return None


def dequant_counter_traffic():
    """Calibrated HBM-side bytes of one decode pass of the 7.5e9-parameter
    workload (207 launches), or None when nf4_storage.hip changed since."""
    kv = _counter_summary("dequant_quantize_counters_7p5e9.txt", ("nf4_storage.hip",))
    try:
        return float(kv["dequant_pass_hbm_bytes"]) if kv else None
    except KeyError:
        return None


def fwd_groups(names):
    """Index groups of the projections that read the same activation: q, k, v
    and gate, up (each other projection alone), in layer order."""
    shared = ({"q_proj", "k_proj", "v_proj"}, {"gate_proj", "up_proj"})
    out, seen = [], set()
    for i, n in enumerate(names):
        if i in seen:
            continue
        g = [i]
        for S in shared:
            if n in S:
                g = [j for j, m in enumerate(names) if m in S]
        seen.update(g)
        out.append(g)
    return out


def layer_flops(M, N, K, r):
    base = 4 * M * N * K
    lora = 6 * M * r * (N + K)
    return base, lora


def packed_bytes(n, nl):
    lay = nl.layout(n, True)
    return lay["codes_bytes"] + lay["scales_bytes"] + lay["nested_bytes"] + lay["offset_bytes"]


def cpu_baseline(layers, M, r, s, rows):
    """The oracle on the host cores over a bounded sample of the same step:
    quantize + dequantize of all 7 weights, forward, input gradient and LoRA
    gradients for the first `rows` token rows of every projection, and the
    AdamW update of every adapter."""
    import numpy as np
    import oracle
    import workloads
    oracle.build(force=False)
    threads = oracle.get_threads()
    t_total, flops = 0.0, 0
    for i, L in enumerate(layers):
        W = workloads.normal_f32((L.n_out, L.k_in), 0.02, workloads.weight_seed(i)).numpy()
        inp = workloads.lora_inputs(L, rows, seed_offset=i)
        x = inp["x"].float().numpy()
        dy = inp["dy"].float().numpy()
        A, B = inp["A"].numpy(), inp["B"].numpy()
        t0 = time.perf_counter()
        q = oracle.quantize(W, True)
        Wd = oracle.bf16_bits_to_f32(oracle.dequantize(q, "bf16")).reshape(W.shape)
        y, T = oracle.linear_fwd(x, Wd, A, B, s)
        dx, U = oracle.linear_bwd_input(dy, Wd, A, B, s)
        dA, dB = oracle.lora_grad(x, dy, T, U, s)
        oracle.lora_adamw_step(B, dB, np.zeros_like(B), np.zeros_like(B), A=A, dA=dA, mA=np.zeros_like(A),
                               vA=np.zeros_like(A), step=1, **ADAMW)
        t_total += time.perf_counter() - t0
        b, l = layer_flops(rows, L.n_out, L.k_in, r)
        flops += b + l
    return dict(value=flops / t_total / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"all 7 weights quantized + dequantized, fwd/bwd-input/LoRA grads on {rows} of {M} "
                       f"token rows per projection, AdamW on all 7 adapters; {flops / 1e9:.1f} GFLOP in {t_total:.1f} s (fp64 accumulation)",
                seconds=round(t_total, 2))


def gpu_time_ms(fn, dev, reps: int = 20, block: int = 4) -> float:
    """Mean device time of fn() over `reps` back-to-back calls. `block` bf16
    GEMMs of ~1 ms each are queued first, so the calls are all enqueued before
    the GPU reaches the start event and host-side call overhead (argument
    checks, ~50-100 us per call, longer than many of the calls measured) does
    not leave gaps in the measured region. HIP events on the launch stream."""
    import torch
    for _ in range(3):
        fn()
    a = torch.ones((8192, 8192), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(block):
        torch.matmul(a, a)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def gemm_sustained(nl, dev, reps: int = 100, warm: int = 100):
    """The fused NF4 + LoRA calls of the two widest projections (gate_proj
    4096 -> 14336 and down_proj 14336 -> 4096, 4096 tokens, r = 16, the layer
    step's inputs), each direction called `warm` times and then `reps` times
    back to back: the rate the GPU sustains on a stream of such calls once its
    clock has settled (in the layer step the same calls alternate with the
    memory-bound quantize and dequantize passes). Event-timed per direction."""
    import torch
    import workloads
    wl = workloads.WORKLOADS["llama8b_layer"]
    M, r = wl["tokens"], wl["layers"][0].lora_rank
    s = nl.lora_scale(wl["alpha"], r)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for i, name in ((4, "gate_proj"), (6, "down_proj")):
        L = wl["layers"][i]
        inp = workloads.lora_inputs(L, M, seed_offset=i, device="cuda")
        W = nl.quantize(workloads.normal_f32((L.n_out, L.k_in), 0.02, workloads.weight_seed(i), "cuda"), True)
        y = torch.empty((M, L.n_out), dtype=torch.bfloat16, device=dev)
        dx = torch.empty((M, L.k_in), dtype=torch.bfloat16, device=dev)
        T = torch.empty((M, r), dtype=torch.float32, device=dev)
        U = torch.empty((M, r), dtype=torch.float32, device=dev)
        ws = torch.empty(max(nl.linear_workspace_bytes(M, L.k_in, L.n_out, r, backward=b) for b in (False, True)) or 1,
                         dtype=torch.uint8, device=dev)
        calls = {"fwd": lambda: nl.linear_fwd(inp["x"], W, inp["A"], inp["B"], s, y=y, t_out=T, workspace=ws),
                 "bwd_input": lambda: nl.linear_bwd_input(inp["dy"], W, inp["A"], inp["B"], s, dx=dx, u_out=U,
                                                          workspace=ws)}
        flops = 2 * M * L.n_out * L.k_in + 2 * M * r * (L.n_out + L.k_in)
        for kind, fn in calls.items():
            for _ in range(warm):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            out[f"{name}_{kind}"] = {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                                     "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del W, inp
    out["calls"] = f"{warm} warm-up + {reps} timed back-to-back calls per entry"
    return out


def lorafa_measure(nl, dev, reps: int = 20):
    """LoRA-FA optimizer step on the rank-64 down_proj adapter (A [64, 14336]
    frozen, B [4096, 64]): the one-off preconditioner and the preconditioned
    AdamW update of B, each timed with gpu_time_ms."""
    import torch
    import workloads
    wl = workloads.WORKLOADS["down_proj_bwd"]
    L = wl["layers"][0]
    r, K, N = L.lora_rank, L.k_in, L.n_out
    s = nl.lora_scale(wl["alpha"], r, wl["rslora"])
    inp = workloads.lora_inputs(L, 1, device="cuda")
    A, B = inp["A"], inp["B"]
    st = workloads.adamw_state((N, r), 0, device="cuda")
    Pm = torch.empty((r, r), dtype=torch.float32, device=dev)
    ws = torch.empty(nl.lorafa_preconditioner_workspace_bytes(r, K), dtype=torch.uint8, device=dev)
    pre_ms = gpu_time_ms(lambda: nl.lorafa_preconditioner(A, out=Pm, workspace=ws), dev, reps)
    k = [0]

    def upd():
        k[0] += 1
        nl.lora_adamw_step(B, st["g"], st["m"], st["v"], step=k[0], precond=Pm, s=s, **ADAMW)
    upd_ms = gpu_time_ms(upd, dev, reps)
    upd_bytes = ADAMW_BYTES * N * r + 4 * r * r
    return {"shape": f"A [{r}, {K}] frozen, B [{N}, {r}], s = {s}", "preconditioner_us": round(pre_ms * 1e3, 1),
            "preconditioned_update_us": round(upd_ms * 1e3, 2),
            "preconditioned_update_gbps": round(upd_bytes / (upd_ms * 1e-3) / 1e9, 1)}


def paged_adamw_measure(nl, dev, reps: int = 10):
    """The AdamW update of the seven Llama-8B adapters (r = 16) with the moments
    in pinned host memory, read and written in place by the update kernel
    (lora_adamw_step_paged), against the same update with device-resident
    moments. Per update 16 bytes of moments per parameter cross PCIe (m and v,
    in and out)."""
    import torch
    import workloads
    ads_dev, ads_host = [], []
    for i, L in enumerate(workloads.llama8b_layer()):
        r = L.lora_rank
        d = dict(A=workloads.normal_f32((r, L.k_in), 1.0 / r, 2 + 10 * i, "cuda"),
                 B=workloads.normal_f32((L.n_out, r), 0.01, 3 + 10 * i, "cuda"))
        d["dA"] = workloads.normal_f32((r, L.k_in), 1e-3, 70 + i, "cuda")
        d["dB"] = workloads.normal_f32((L.n_out, r), 1e-3, 80 + i, "cuda")
        for k, shape in (("mA", (r, L.k_in)), ("vA", (r, L.k_in)), ("mB", (L.n_out, r)), ("vB", (L.n_out, r))):
            d[k] = torch.zeros(shape, dtype=torch.float32, device=dev)
        h = dict(d)
        for k in ("mA", "vA", "mB", "vB"):
            h[k] = torch.zeros(d[k].shape, dtype=torch.float32, pin_memory=True)
        ads_dev.append(d)
        ads_host.append(h)
    page = 2 << 20
    k = [0]

    def paged():
        k[0] += 1
        nl.lora_adamw_step_paged(ads_host, step=k[0], page_bytes=page, **ADAMW)

    def resident():
        k[0] += 1
        nl.lora_adamw_step_many(ads_dev, step=k[0], **ADAMW)
    t_p = gpu_time_ms(paged, dev, reps)
    t_d = gpu_time_ms(resident, dev, reps)
    params = sum(a["A"].numel() + a["B"].numel() for a in ads_dev)
    return {"params": params, "page_bytes": page, "paged_ms": round(t_p, 3), "resident_ms": round(t_d, 4),
            "pcie_gbps": round(16 * params / (t_p * 1e-3) / 1e9, 1)}


def embedding_measure(nl, dev, reps: int = 20):
    """Selected-row decode of packed embedding tables (outside the timed step):
    the SmolLM2 tied 49152 x 576 table for 512 tokens and a Llama-8B-sized
    128256 x 4096 vocabulary for 4096 tokens, bf16 rows, HIP events on the
    launch stream (gpu_time_ms). Algorithmic bytes per row: codes D/2, qabs
    D/64, the nested maxima the row touches, and 2D of output."""
    import numpy as np
    import torch
    import workloads
    res = {}
    for name, V, D, T in (("smollm2_tied_49152x576", 49152, 576, 512), ("llama8b_vocab_128256x4096", 128256, 4096, 4096)):
        W = workloads.normal_f32((V, D), 0.02, 4242, "cuda")
        E = nl.quantize(W, True)
        del W
        ids = torch.from_numpy(np.random.default_rng(7).integers(0, V, size=T, dtype=np.int64)).to(dev)
        out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
        ms = gpu_time_ms(lambda: nl.embedding_rows(E, ids, out=out), dev, reps)
        row_bytes = D // 2 + D // 64 + 4 * (-(-D // 16384)) + 2 * D
        res[name] = {"tokens": T, "us": round(ms * 1e3, 2),
                     "gbps": round(T * row_bytes / (ms * 1e-3) / 1e9, 1)}
        del E
    return res


def decoder_step_measure(dev, steps: int = 3, warmup: int = 1, seq: int = 512):
    """The full checkpointed training step of a Llama-3.1-8B-shaped model on the
    NF4 base (32 layers, hidden 4096, GQA 32/8 heads of 128, FFN 14336, vocab
    128256; LoRA r = 16, alpha 32 on q_proj and v_proj; 512 tokens, batch 1):
    embedding rows, 32 layers, final norm, lm_head, cross-entropy, the
    lm_head backward, 32 recomputed layers with their backward, and the AdamW
    update of the 64 adapters. Synthetic seeded weights and token ids. Work is
    counted as the pages do: 6 flops per decoder projection parameter and 4 per
    lm_head parameter per token (43.98 GFLOP/token)."""
    import torch
    from qlora_adapter_amd import llama
    cfg = llama.LlamaConfig()
    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    t0 = time.perf_counter()
    m = llama.LlamaNF4(cfg, seq, device=dev)
    torch.cuda.synchronize(dev)
    build_s = time.perf_counter() - t0
    g = torch.Generator().manual_seed(31)
    ids = torch.randint(0, cfg.vocab, (seq + 1,), generator=g).to(dev)
    x, y = ids[:-1].clone(), ids[1:].clone()
    # train_step returns the model's one loss buffer, so the first loss is copied
    # out before the next step overwrites it (outside the timed region)
    losses = []
    for i in range(warmup):
        loss = m.train_step(x, y)
        if i == 0:
            losses.append(loss.clone())
    torch.cuda.synchronize(dev)
    st = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        loss = m.train_step(x, y)
    e1.record(st)
    losses.append(loss)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    fpt = cfg.flops_per_token()
    peak_gb = torch.cuda.max_memory_allocated(dev) / 2 ** 30
    out = {"model": "Llama-3.1-8B shape, NF4 + double quantization, random init", "seq": seq, "batch": 1,
           "layers": cfg.layers, "lora": "r=16 alpha=32 on q_proj, v_proj", "steps": steps, "warmup": warmup,
           "ms_per_step": round(ms, 2), "tokens_per_s": round(seq / (ms * 1e-3), 1),
           "gflop_per_token": round(fpt / 1e9, 2), "effective_tflops": round(fpt * seq / (ms * 1e-3) / 1e12, 1),
           "loss_first_last": [round(float(losses[0].item()), 4), round(float(losses[-1].item()), 4)],
           "peak_allocated_gib": round(peak_gb, 2), "build_s": round(build_s, 2)}
    del m
    torch.cuda.empty_cache()
    return out


def quant_dequant_throughput(nl, dev, passes: int = 3, batch: int = 1):
    """The standalone quantize + dequantize workload: 7,499,415,552 fp32
    parameters (96 matrices of 4096 x 14336 and 111 of 4096 x 4096, N(0, 0.02)
    with 1% outliers at 10x), all resident. One pass quantizes (or decodes)
    every matrix once, back to back, so each pass walks 3.87 GB of packed
    weights: far more than the 256 MB last-level cache. Each matrix decodes
    into its own output. With batch > 1, nf4_dequantize_many decodes that many
    matrices per launch (slower on matrices this large: one launch per matrix
    measured 5.70 TB/s against 5.36-5.57 with 16 per launch). Quantize is timed
    both ways: one nf4_quantize call per matrix, and nf4_quantize_many over 16
    matrices per call (three launches per call, so the double-quantization
    tail is paid per call, not per matrix). HIP events around whole passes on
    the launch stream."""
    import torch
    import workloads
    mats = workloads.quant_throughput_matrices()
    W, Q, OUT = [], [], []
    for i, shape in enumerate(mats):
        w = workloads.weight_with_outliers(shape, seed=workloads.weight_seed(i), device="cuda")
        W.append(w)
        Q.append(nl.NF4Tensor.empty(shape, True, dev))
        OUT.append(torch.empty(shape, dtype=torch.bfloat16, device=dev))
    lay = {sh: nl.layout(sh[0] * sh[1], True) for sh in set(mats)}
    ws = torch.empty(max(l["quantize_workspace_bytes"] for l in lay.values()), dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    n_total = sum(a * b for a, b in mats)
    packed = sum(lay[sh]["codes_bytes"] + lay[sh]["scales_bytes"] + lay[sh]["nested_bytes"] + lay[sh]["offset_bytes"]
                 for sh in mats)
    stream = torch.cuda.current_stream(dev)

    def run(fn):
        fn()  # warm-up pass
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(passes):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / passes

    def quant_pass():
        for w, q in zip(W, Q):
            nl.quantize(w, True, out=q, workspace=ws, status=status)

    many = nl.MAX_TENSORS_PER_CALL
    ws_many = torch.empty(max(nl.quantize_many_workspace_bytes(Q[i:i + many]) for i in range(0, len(Q), many)),
                          dtype=torch.uint8, device=dev)

    def quant_many_pass():  # 16 matrices per nf4_quantize_many call
        for i in range(0, len(W), many):
            nl.quantize_many(W[i:i + many], True, outs=Q[i:i + many], workspace=ws_many, status=status)

    def deq_pass():  # `batch` matrices per launch
        for i in range(0, len(Q), batch):
            if batch == 1:
                nl.dequantize(Q[i], torch.bfloat16, out=OUT[i])
            else:
                nl.dequantize_many(Q[i:i + batch], torch.bfloat16, outs=OUT[i:i + batch])

    q_ms = run(quant_pass)
    assert int(status.item()) == 0
    qm_ms = run(quant_many_pass)
    assert int(status.item()) == 0
    d_ms = run(deq_pass)
    del W, Q, OUT
    torch.cuda.empty_cache()
    q_bytes, d_bytes = 4 * n_total + packed, packed + 2 * n_total
    return {"params": n_total, "matrices": len(mats), "packed_bytes": packed, "dequant_bf16_bytes": d_bytes,
            "dequant_bf16_ms": round(d_ms, 3), "dequant_bf16_gbps": round(d_bytes / (d_ms * 1e-3) / 1e9, 1),
            "quantize_ms": round(q_ms, 3), "quantize_gbps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
            "quantize_many_ms": round(qm_ms, 3), "quantize_many_gbps": round(q_bytes / (qm_ms * 1e-3) / 1e9, 1)}


def other_configs(nl, dev):
    """The other configurations of the workload table, each timed with
    gpu_time_ms (device time of back-to-back calls):
      single_576: one 576x576 layer, 512 tokens, r = 16: latency of the forward,
        the input gradient and the LoRA gradients;
      smollm2_stack: 30 SmolLM2-shaped layers (7 linears each, LoRA r = 8 on q
        and v), 512 tokens: one forward + input-gradient + LoRA-gradient pass
        over all 210 linears, as TFLOP/s and microseconds per layer (device time
        with the launches queued back to back, as a captured graph would run);
      down_proj_bwd: down_proj [4096, 14336], 8192 tokens, rank-64 rsLoRA: the
        input gradient (with U), the LoRA gradients and the LoRA-FA dB alone."""
    import torch
    import workloads

    def setup(layers, M, alpha, rslora, dy_std=1.0, seed0=0):
        out = []
        for i, L in enumerate(layers):
            inp = workloads.lora_inputs(L, M, seed_offset=seed0 + i, device="cuda", dy_std=dy_std)
            W = workloads.normal_f32((L.n_out, L.k_in), 0.02, workloads.weight_seed(seed0 + i), "cuda")
            r = L.lora_rank
            s = nl.lora_scale(alpha, r, rslora) if r else 0.0
            e = dict(L=L, x=inp["x"], dy=inp["dy"], Wq=nl.quantize(W, True), s=s, r=r,
                     A=inp.get("A"), B=inp.get("B"))
            e["y"], e["T"] = nl.linear_fwd(e["x"], e["Wq"], e["A"], e["B"], s)
            e["dx"], e["U"] = nl.linear_bwd_input(e["dy"], e["Wq"], e["A"], e["B"], s)
            if r:
                e["dA"], e["dB"] = nl.lora_grad(e["x"], e["dy"], e["T"], e["U"], s)
                e["ws"] = torch.empty(nl.lora_grad_workspace_bytes(M, L.k_in, L.n_out, r), dtype=torch.uint8,
                                      device=dev)
            out.append(e)
        return out

    fwd = lambda e: nl.linear_fwd(e["x"], e["Wq"], e["A"], e["B"], e["s"], y=e["y"], t_out=e["T"])
    bwd = lambda e: nl.linear_bwd_input(e["dy"], e["Wq"], e["A"], e["B"], e["s"], dx=e["dx"], u_out=e["U"])
    grad = lambda e: nl.lora_grad(e["x"], e["dy"], e["T"], e["U"], e["s"], dA=e["dA"], dB=e["dB"],
                                  workspace=e["ws"])
    res = {}

    wl = workloads.WORKLOADS["single_576"]
    (e,) = setup(wl["layers"], wl["tokens"], wl["alpha"], wl["rslora"])
    tf, tb, tg = gpu_time_ms(lambda: fwd(e), dev), gpu_time_ms(lambda: bwd(e), dev), gpu_time_ms(lambda: grad(e), dev)
    res["single_576"] = {"tokens": wl["tokens"], "rank": 16, "fwd_us": round(tf * 1e3, 2), "bwd_input_us": round(tb * 1e3, 2),
                         "lora_grad_us": round(tg * 1e3, 2), "total_us": round((tf + tb + tg) * 1e3, 2)}

    wl = workloads.WORKLOADS["smollm2_stack"]
    M = wl["tokens"]
    E = setup(wl["layers"], M, wl["alpha"], wl["rslora"])

    def stack_pass():
        for e in E:
            fwd(e)
        for e in reversed(E):
            bwd(e)
            if e["r"]:
                grad(e)
    # 480 calls per pass: queue ~70 ms of GEMMs first so that all five passes are enqueued before timing starts
    ms = gpu_time_ms(stack_pass, dev, reps=5, block=70)
    flops = sum(4 * M * e["L"].n_out * e["L"].k_in + (6 * M * e["r"] * (e["L"].n_out + e["L"].k_in) if e["r"] else 0)
                for e in E)
    res["smollm2_stack"] = {"tokens": M, "linears": len(E), "pass_ms": round(ms, 3),
                            "us_per_layer": round(ms * 1e3 / 30, 1), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                            "gflop": round(flops / 1e9, 1)}
    del E

    wl = workloads.WORKLOADS["down_proj_bwd"]
    M = wl["tokens"]
    (e,) = setup(wl["layers"], M, wl["alpha"], wl["rslora"], dy_std=wl.get("dy_std", 1.0))
    L, r = e["L"], e["r"]
    ws_fa = torch.empty(nl.lora_grad_workspace_bytes(M, L.k_in, L.n_out, r, fa=True), dtype=torch.uint8, device=dev)
    tb = gpu_time_ms(lambda: bwd(e), dev, reps=10)
    tg = gpu_time_ms(lambda: grad(e), dev, reps=10)
    tfa = gpu_time_ms(lambda: nl.lora_grad(e["x"], e["dy"], e["T"], None, e["s"], fa=True, dB=e["dB"], workspace=ws_fa),
                      dev, reps=10)
    bwd_flops = 2 * M * L.n_out * L.k_in + 2 * M * r * (L.n_out + L.k_in)
    res["down_proj_bwd"] = {"tokens": M, "rank": r, "scale": e["s"], "bwd_input_ms": round(tb, 3),
                            "bwd_input_tflops": round(bwd_flops / (tb * 1e-3) / 1e12, 1),
                            "lora_grad_ms": round(tg, 3), "lora_fa_dB_ms": round(tfa, 3),
                            "lora_grad_gbps": round(2 * M * (L.k_in + L.n_out) / (tg * 1e-3) / 1e9, 1)}
    del e
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.copy_probe:
        copy_probe()
        return
    if args.throughput_only:
        import torch
        from qlora_adapter_amd import nf4lora as nl
        nl.load()
        print(json.dumps(quant_dequant_throughput(nl, torch.device("cuda:0"), passes=1)), flush=True)
        return
    if args.gemm_sustained_only:
        import torch
        from qlora_adapter_amd import nf4lora as nl
        nl.load()
        print(json.dumps(gemm_sustained(nl, torch.device("cuda:0"))), flush=True)
        return
    if args.decoder_step_only:
        import torch
        from qlora_adapter_amd import nf4lora as nl
        nl.load()
        print(json.dumps(decoder_step_measure(torch.device("cuda:0"), steps=args.steps, warmup=args.warmup)),
              flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    from qlora_adapter_amd import nf4lora as nl

    assert torch.cuda.is_available(), "bench.py needs a ROCm device"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nl.load()
    wl = workloads.WORKLOADS["llama8b_layer"]
    layers, M = wl["layers"], wl["tokens"]
    r = layers[0].lora_rank
    s = nl.lora_scale(wl["alpha"], r)

    # ---- resident inputs and outputs (untimed) ----
    # q, k and v read one activation, and so do gate and up (as in the decoder
    # block); their forward passes run as one grouped call each, and their
    # input gradients as one summed call each (the gradient that activation
    # receives)
    groups = fwd_groups([L.name for L in layers])
    first = {i: g[0] for g in groups for i in g}
    P = []
    for i, L in enumerate(layers):
        inp = workloads.lora_inputs(L, M, seed_offset=i, device="cuda")
        if first[i] != i:
            inp["x"] = P[first[i]]["x"]
        W = workloads.normal_f32((L.n_out, L.k_in), 0.02, workloads.weight_seed(i), "cuda")
        P.append(dict(
            L=L, W=W, x=inp["x"], dy=inp["dy"], A=inp["A"], B=inp["B"],
            Wq=nl.NF4Tensor.empty(W.shape, True, dev),
            y=torch.empty((M, L.n_out), dtype=torch.bfloat16, device=dev),
            T=torch.empty((M, r), dtype=torch.float32, device=dev),
            dx=torch.empty((M, L.k_in), dtype=torch.bfloat16, device=dev),
            U=torch.empty((M, r), dtype=torch.float32, device=dev),
            dA=torch.empty((r, L.k_in), dtype=torch.float32, device=dev),
            dB=torch.empty((L.n_out, r), dtype=torch.float32, device=dev),
            gws=torch.empty(nl.lora_grad_workspace_bytes(M, L.k_in, L.n_out, r), dtype=torch.uint8, device=dev),
            lws=torch.empty(max(1, *(nl.linear_workspace_bytes(M, L.k_in, L.n_out, r, backward=b) for b in (False, True))),
                            dtype=torch.uint8, device=dev),
            mA=torch.zeros((r, L.k_in), dtype=torch.float32, device=dev),
            vA=torch.zeros((r, L.k_in), dtype=torch.float32, device=dev),
            mB=torch.zeros((L.n_out, r), dtype=torch.float32, device=dev),
            vB=torch.zeros((L.n_out, r), dtype=torch.float32, device=dev),
            Wd=torch.empty(W.shape, dtype=torch.bfloat16, device=dev),
        ))
    group_ws = {g[0]: torch.empty(max(1, nl.linear_fwd_group_workspace_bytes(
        M, layers[g[0]].k_in, [layers[i].n_out for i in g], [r] * len(g))), dtype=torch.uint8, device=dev)
        for g in groups if len(g) > 1}
    sum_ws = {g[0]: torch.empty(max(1, nl.linear_bwd_input_sum_workspace_bytes(
        M, layers[g[0]].k_in, [layers[i].n_out for i in g], [r] * len(g))), dtype=torch.uint8, device=dev)
        for g in groups if len(g) > 1}
    stream = torch.cuda.current_stream(dev)
    adapters = [dict(A=p["A"], dA=p["dA"], mA=p["mA"], vA=p["vA"], B=p["B"], dB=p["dB"], mB=p["mB"], vB=p["vB"])
                for p in P]
    wq_all, wd_all = [p["Wq"] for p in P], [p["Wd"] for p in P]
    w_all = [p["W"] for p in P]
    qm_ws = torch.empty(nl.quantize_many_workspace_bytes(wq_all), dtype=torch.uint8, device=dev)
    q_status = torch.zeros(1, dtype=torch.int32, device=dev)
    kinds = ["quantize", "fwd", "bwd", "grad", "adamw", "dequant"]
    opt_step = [0]

    def step(events=None):
        opt_step[0] += 1
        t = opt_step[0]
        def mark(kind, i, fn):
            if events is None:
                fn()
                return
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            events.append((kind, i, e0, e1))
        # one launch set packs all seven matrices
        mark("quantize", 0, lambda: nl.quantize_many(w_all, True, outs=wq_all, workspace=qm_ws, status=q_status))
        for g in groups:  # a grouped call's time is recorded at its first projection
            if len(g) == 1:
                p = P[g[0]]
                mark("fwd", g[0], lambda p=p: nl.linear_fwd(p["x"], p["Wq"], p["A"], p["B"], s, y=p["y"],
                                                            t_out=p["T"], workspace=p["lws"]))
            else:
                q = [P[i] for i in g]
                mark("fwd", g[0], lambda q=q, w=group_ws[g[0]]: nl.linear_fwd_group(
                    q[0]["x"], [p["Wq"] for p in q], [p["A"] for p in q], [p["B"] for p in q], [s] * len(q),
                    ys=[p["y"] for p in q], t_outs=[p["T"] for p in q], workspace=w))
        for g in groups:  # a group's summed input gradient lands in its first projection's dx
            if len(g) == 1:
                p = P[g[0]]
                mark("bwd", g[0], lambda p=p: nl.linear_bwd_input(p["dy"], p["Wq"], p["A"], p["B"], s, dx=p["dx"],
                                                                  u_out=p["U"], workspace=p["lws"]))
            else:
                q = [P[i] for i in g]
                mark("bwd", g[0], lambda q=q, w=sum_ws[g[0]]: nl.linear_bwd_input_sum(
                    [p["dy"] for p in q], [p["Wq"] for p in q], [p["A"] for p in q], [p["B"] for p in q],
                    [s] * len(q), dx=q[0]["dx"], u_outs=[p["U"] for p in q], workspace=w))
        for i, p in enumerate(P):
            mark("grad", i, lambda p=p: nl.lora_grad(p["x"], p["dy"], p["T"], p["U"], s, dA=p["dA"], dB=p["dB"],
                                                     workspace=p["gws"]))
        # one launch updates all seven adapters
        mark("adamw", 0, lambda: nl.lora_adamw_step_many(adapters, step=t, **ADAMW))
        # one launch decodes all seven matrices
        mark("dequant", 0, lambda: nl.dequantize_many(wq_all, torch.bfloat16, outs=wd_all))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(q_status.item()) == 0

    # ---- timed region: whole steps, no per-call events ----
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3

    # ---- per-call HIP events on the launch stream (separate pass, same work) ----
    events = []
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    per = {k: [0.0] * len(P) for k in kinds}
    for kind, i, e0, e1 in events:
        per[kind][i] += e0.elapsed_time(e1) / args.steps  # ms per call

    flops_base = flops_lora = 0
    fwd_flops = fwd_ms = bwd_flops = bwd_ms = 0.0
    dq_bytes = dq_ms = q_bytes = q_ms = ad_bytes = ad_ms = 0.0
    for i, p in enumerate(P):
        L = p["L"]
        b, l = layer_flops(M, L.n_out, L.k_in, r)
        flops_base += b
        flops_lora += l
        fwd_flops += 2 * M * L.n_out * L.k_in + 2 * M * r * (L.n_out + L.k_in)
        bwd_flops += 2 * M * L.n_out * L.k_in + 2 * M * r * (L.n_out + L.k_in)
        fwd_ms += per["fwd"][i]
        bwd_ms += per["bwd"][i]
        n = L.n_out * L.k_in
        pb = packed_bytes(n, nl)
        dq_bytes += pb + 2 * n
        dq_ms += per["dequant"][i]  # the whole decode is recorded at index 0
        q_bytes += 4 * n + pb
        q_ms += per["quantize"][i]  # the whole pack is recorded at index 0
        ad_bytes += ADAMW_BYTES * r * (L.k_in + L.n_out)
        ad_ms += per["adamw"][i]  # the whole update is recorded at index 0
    total_flops = flops_base + flops_lora
    fwd_tf = fwd_flops / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bwd_flops / (bwd_ms * 1e-3) / 1e12
    dominant = "nf4_linear_fwd" if fwd_ms >= bwd_ms else "nf4_linear_bwd_input"
    dom_tf = fwd_tf if fwd_ms >= bwd_ms else bwd_tf
    dq_gbps = dq_bytes / (dq_ms * 1e-3) / 1e9
    q_gbps = q_bytes / (q_ms * 1e-3) / 1e9
    ad_gbps = ad_bytes / (ad_ms * 1e-3) / 1e9
    qd = None if args.no_throughput else quant_dequant_throughput(nl, dev)
    sustained = gemm_sustained(nl, dev)
    fa = lorafa_measure(nl, dev)
    emb = embedding_measure(nl, dev)
    paged = paged_adamw_measure(nl, dev)
    others = other_configs(nl, dev)
    decoder = None if args.no_decoder_step else decoder_step_measure(dev)

    ceil = None if args.no_ceilings else ceilings()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layers, M, r, s, args.cpu_rows)

    out = {
        "metric": "fused NF4+LoRA linear TFLOP/s & dequant GB/s, % of MI355X roofline",
        "value": round(total_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) fp32 weights, N(0,1) bf16 activations and upstream gradients)",
        "config": {"workload": "llama8b_layer", "tokens": M, "hidden": 4096, "kv_dim": 1024,
                   "intermediate": 14336, "projections": 7, "lora_rank": r, "lora_alpha": wl["alpha"],
                   "double_quant": True, "block": 64, "nested_block": 256,
                   "step": "quantize + fused fwd + fused bwd-input + lora_grad + AdamW(A, B) + dequantize, "
                           "all 7 projections (q, k, v read one x, gate, up another; their forward passes "
                           "run as one grouped call each, their input gradients as one summed call each)"},
        "roofline": {"kernel": dominant, "bound": "mfma", "achieved": round(dom_tf, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": counter_traffic(dominant)},
        "roofline_dequant": (
            {"kernel": "nf4_dequantize (bf16 out, one launch per matrix)",
             "workload": "7.5e9-parameter quantize/dequantize throughput "
             "(96 x 4096x14336 + 111 x 4096x4096, cold passes)", "bound": "hbm",
             "achieved": qd["dequant_bf16_gbps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
             "frac": round(qd["dequant_bf16_gbps"] / PEAK_HBM_GBPS, 4), "traffic": dequant_counter_traffic(),
             "traffic_per": "pass of 207 launches (algorithmic bytes per pass: %d)" % qd["dequant_bf16_bytes"],
             "in_layer_step_gbps": round(dq_gbps, 1)} if qd else
            {"kernel": "nf4_dequantize_many (bf16 out)", "workload": "the layer step's seven matrices", "bound": "hbm",
             "achieved": round(dq_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
             "frac": round(dq_gbps / PEAK_HBM_GBPS, 4), "traffic": None}),
        "quant_dequant_throughput": qd,
        "kernels": {"fwd_tflops": round(fwd_tf, 1), "bwd_tflops": round(bwd_tf, 1),
                    "fwd_ms": round(fwd_ms, 3), "bwd_ms": round(bwd_ms, 3),
                    "grad_ms": round(sum(per["grad"]), 3), "quantize_ms": round(q_ms, 3),
                    "quantize_gbps": round(q_gbps, 1), "dequant_ms": round(dq_ms, 3),
                    "dequant_gbps": round(dq_gbps, 1), "adamw_ms": round(ad_ms, 4),
                    "adamw_gbps": round(ad_gbps, 1),
                    "fwd_calls": [[layers[i].name for i in g] for g in groups],
                    "bwd_calls": [[layers[i].name for i in g] for g in groups],
                    "per_projection_ms": {k: [round(v, 4) for v in per[k]] for k in kinds
                                          if k not in ("adamw", "dequant", "quantize")}},
        "roofline_adamw": {"kernel": "lora_adamw_step_many (A and B of all 7 adapters, one launch)",
                           "bound": "hbm", "achieved": round(ad_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                           "frac": round(ad_gbps / PEAK_HBM_GBPS, 4), "traffic": None,
                           "note": "28 B per parameter, 1.31 M parameters (36.7 MB) per launch"},
        "gemm_sustained": sustained,
        "lorafa": fa,
        "embedding_rows": emb,
        "paged_adamw": paged,
        "other_configs": others,
        "decoder_step": decoder,
        "ceilings": ceil,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
