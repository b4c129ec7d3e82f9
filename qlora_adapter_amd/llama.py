"""A Llama-shaped decoder training step on a frozen NF4 base with LoRA adapters,
built from the library's calls. This module only orders the calls and owns
the buffers: every arithmetic step is one of the C ABI's operations.

Soup, "NF4 Layer Streaming - Gate results": the pages time a full training
step of a Llama-3.1-8B-shaped model (512 tokens, batch 1, NF4 base, LoRA r = 16
on q_proj and v_proj) whose decoder layers are checkpointed, and count its work
as 6 flops per decoder parameter per token (forward, recomputed forward, input
gradient; 2 each) plus 4 per lm_head parameter (forward and input gradient).

Step: embedding rows -> per layer: x = xin + res, RMSNorm, q/k/v (LoRA on the
adapted ones), rotary q and k, causal GQA attention, o, x2 = x + o, RMSNorm,
gate and up, SwiGLU, down -> final add + RMSNorm -> lm_head -> mean token
cross-entropy. Backward: lm_head and final norm, then per layer in reverse:
recompute its forward from the saved x, run its backward. Last: one AdamW
update of every adapter. The only activation kept per layer is x (one [S, D]
tensor); everything else lives in buffers shared by all layers.

Projections that read the same input are stored as one packed NF4 matrix
(q, k, v stacked as [(hq + 2 hkv) d, D]; gate, up as [2 F, D]) and run as one
linear call each way: the forward writes q, k, v (or gate, up) as column
blocks of one output whose row stride the rotary, attention and SwiGLU calls
take, and the input gradient of the stacked matrix is the sum over its members
in one reduction. Adapters on members of a stack become one adapter of the
stack: A stacked along the rank, B block-diagonal (member j's B in its rows and
its rank block, zeros elsewhere); the zero blocks add exact zeros, and their
gradients are cleared after every lora_grad, so they stay zero under AdamW.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import torch

from . import nf4lora as nl

PROJ = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")
# Stacked matrices (one packed NF4 tensor each) and their members, in row order.
STACKS = {"qkv": ("q_proj", "k_proj", "v_proj"), "o_proj": ("o_proj",), "gate_up": ("gate_proj", "up_proj"),
          "down_proj": ("down_proj",)}


@dataclasses.dataclass(frozen=True)
class LlamaConfig:
    hidden: int = 4096
    heads: int = 32
    kv_heads: int = 8
    head_dim: int = 128
    ffn: int = 14336
    vocab: int = 128256
    layers: int = 32
    eps: float = 1e-5
    theta: float = 500000.0
    lora_rank: int = 16
    lora_alpha: float = 32.0
    lora_targets: Sequence[str] = ("q_proj", "v_proj")

    def shape(self, name: str):
        """[N, K] of a projection's weight (y = x W^T)."""
        D, F, d = self.hidden, self.ffn, self.head_dim
        return {"q_proj": (self.heads * d, D), "k_proj": (self.kv_heads * d, D), "v_proj": (self.kv_heads * d, D),
                "o_proj": (D, self.heads * d), "gate_proj": (F, D), "up_proj": (F, D), "down_proj": (D, F)}[name]

    def decoder_params(self) -> int:
        return self.layers * sum(n * k for n, k in (self.shape(p) for p in PROJ))

    def flops_per_token(self) -> float:
        """6 per decoder projection parameter, 4 per lm_head parameter."""
        return 6.0 * self.decoder_params() + 4.0 * self.vocab * self.hidden


def synthetic_normal(shape, std: float, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32) * std


class Layer:
    """One decoder layer: packed NF4 stacked projections (STACKS), fp32 norm
    weights, fp32 adapters with their gradients and AdamW moments.

    lora[stack] is the adapter of a stack (A [R, K], B [N, R] block-diagonal,
    R = r times its adapted members); lora[name] holds views of one member's
    A, B, dA and dB inside it (dB's view is that member's block)."""

    def __init__(self, cfg: LlamaConfig, weights: Dict[str, torch.Tensor], gamma1: torch.Tensor,
                 gamma2: torch.Tensor, adapters: Dict[str, tuple]):
        self.W: Dict[str, nl.NF4Tensor] = {
            st: nl.quantize(torch.cat([weights[n] for n in mem]) if len(mem) > 1 else weights[mem[0]], True)
            for st, mem in STACKS.items()}
        self.gamma1, self.gamma2 = gamma1, gamma2
        self.lora: Dict[str, dict] = {}
        self.stack_lora: Dict[str, dict] = {}
        for st, mem in STACKS.items():
            ad = [n for n in mem if n in adapters]
            if not ad:
                continue
            r = adapters[ad[0]][0].shape[0]
            rows = [cfg.shape(n)[0] for n in mem]
            K = cfg.shape(mem[0])[1]
            dev = adapters[ad[0]][0].device
            A = torch.cat([adapters[n][0] for n in ad]).contiguous()
            B = torch.zeros((sum(rows), r * len(ad)), dtype=torch.float32, device=dev)
            mask = torch.zeros_like(B)
            for j, n in enumerate(ad):
                off = sum(rows[:mem.index(n)])
                B[off:off + rows[mem.index(n)], r * j:r * (j + 1)] = adapters[n][1]
                mask[off:off + rows[mem.index(n)], r * j:r * (j + 1)] = 1.0
            full = dict(A=A, B=B, dA=torch.zeros_like(A), dB=torch.zeros_like(B), mA=torch.zeros_like(A),
                        vA=torch.zeros_like(A), mB=torch.zeros_like(B), vB=torch.zeros_like(B),
                        mask=None if len(mem) == 1 else mask, K=K)
            self.stack_lora[st] = full
            for j, n in enumerate(ad):
                off, nr = sum(rows[:mem.index(n)]), rows[mem.index(n)]
                blk = (slice(off, off + nr), slice(r * j, r * (j + 1)))
                self.lora[n] = dict(A=A[r * j:r * (j + 1)], B=B[blk], dA=full["dA"][r * j:r * (j + 1)],
                                    dB=full["dB"][blk])

    @staticmethod
    def synthetic(cfg: LlamaConfig, idx: int, device, w_std: float = 0.02) -> "Layer":
        """Seeded N(0, w_std) weights, unit norm weights, A ~ N(0, 1/r), B = 0."""
        dev = torch.device(device)
        W = {}
        for j, name in enumerate(PROJ):
            W[name] = synthetic_normal(cfg.shape(name), w_std, 100000 + 16 * idx + j, dev)
        one = torch.ones(cfg.hidden, dtype=torch.float32, device=dev)
        r = cfg.lora_rank
        ad = {}
        for j, name in enumerate(cfg.lora_targets):
            n, k = cfg.shape(name)
            ad[name] = (synthetic_normal((r, k), 1.0 / r, 300000 + 16 * idx + j, dev),
                        torch.zeros((n, r), dtype=torch.float32, device=dev))
        layer = Layer(cfg, W, one, one.clone(), ad)
        del W
        return layer


class LlamaNF4:
    """Decoder stack with the embedding and lm_head on NF4 storage and LoRA on
    cfg.lora_targets, at a fixed sequence length S and activation dtype."""

    def __init__(self, cfg: LlamaConfig, seq: int, device="cuda", dtype=torch.bfloat16,
                 layers: Optional[List[Layer]] = None, with_head: bool = True, head_weights=None):
        """layers: prebuilt Layer objects (default: Layer.synthetic); head_weights:
        optional fp32 (embedding [V, D], lm_head [V, D], final norm [D]) to
        quantize instead of the seeded synthetic ones."""
        self.cfg, self.S, self.dev, self.dt = cfg, int(seq), torch.device(device), dtype
        self.s = nl.lora_scale(cfg.lora_alpha, cfg.lora_rank)
        self.layers = layers if layers is not None else [Layer.synthetic(cfg, i, self.dev) for i in range(cfg.layers)]
        if len(self.layers) != cfg.layers:
            raise ValueError("cfg.layers does not match the number of layers given")
        self.with_head = with_head
        if with_head:
            V, D = cfg.vocab, cfg.hidden
            if head_weights is None:
                head_weights = (synthetic_normal((V, D), 0.02, 500000, self.dev),
                                synthetic_normal((V, D), 0.02, 500001, self.dev),
                                torch.ones(D, dtype=torch.float32, device=self.dev))
            self.embed = nl.quantize(head_weights[0], True)
            self.lm_head = nl.quantize(head_weights[1], True)
            self.gamma_f = head_weights[2]
            del head_weights
        self._alloc()
        self.step_count = 0

    def _stack_shape(self, st: str):
        """[N, K] of a stacked matrix."""
        mem = STACKS[st]
        return sum(self.cfg.shape(n)[0] for n in mem), self.cfg.shape(mem[0])[1]

    def _alloc(self):
        c, S = self.cfg, self.S
        e = lambda *sh: torch.empty(sh, dtype=self.dt, device=self.dev)
        f = lambda *sh: torch.empty(sh, dtype=torch.float32, device=self.dev)
        H, Hkv, d, D, F = c.heads, c.kv_heads, c.head_dim, c.hidden, c.ffn
        QKV = (H + 2 * Hkv) * d
        self.b = dict(x=e(S, D), h1=e(S, D), qkv=e(S, QKV), a=e(S, H * d), o=e(S, D), x2=e(S, D), h2=e(S, D),
                      gu=e(S, 2 * F), sw=e(S, F), dn=e(S, D), lse=f(H, S), r1=f(S), r2=f(S), delta=f(H, S),
                      dsw=e(S, F), dgu=e(S, 2 * F), dh2=e(S, D), dx2=e(S, D), da=e(S, H * d), dqkv=e(S, QKV),
                      dh1=e(S, D), gA=e(S, D), gB=e(S, D))
        # column blocks of the stacked outputs (and of their gradients)
        cols = lambda t, a, b: t[:, a:b]
        self.v_ = dict(q=cols(self.b["qkv"], 0, H * d), k=cols(self.b["qkv"], H * d, (H + Hkv) * d),
                       v=cols(self.b["qkv"], (H + Hkv) * d, QKV), qk=cols(self.b["qkv"], 0, (H + Hkv) * d),
                       dq=cols(self.b["dqkv"], 0, H * d), dk=cols(self.b["dqkv"], H * d, (H + Hkv) * d),
                       dv=cols(self.b["dqkv"], (H + Hkv) * d, QKV), dqk=cols(self.b["dqkv"], 0, (H + Hkv) * d),
                       g=cols(self.b["gu"], 0, F), u=cols(self.b["gu"], F, 2 * F),
                       dg=cols(self.b["dgu"], 0, F), du=cols(self.b["dgu"], F, 2 * F))
        ranks = {st: c.lora_rank * sum(n in c.lora_targets for n in mem) for st, mem in STACKS.items()}
        self.T = {st: f(S, R) for st, R in ranks.items() if R}
        self.U = {st: f(S, R) for st, R in ranks.items() if R}
        self.gws = {st: torch.empty(nl.lora_grad_workspace_bytes(S, self._stack_shape(st)[1], self._stack_shape(st)[0],
                                                                 R), dtype=torch.uint8, device=self.dev)
                    for st, R in ranks.items() if R}
        shapes = [(self._stack_shape(st)[1], self._stack_shape(st)[0], ranks[st]) for st in STACKS]
        if self.with_head:
            shapes.append((c.hidden, c.vocab, 0))
        need = max(nl.linear_workspace_bytes(S, k, n, r, backward=bwd) for k, n, r in shapes for bwd in (False, True))
        self.lws = torch.empty(need, dtype=torch.uint8, device=self.dev) if need else None
        self.cur_x = None
        if self.with_head:
            self.saved: List[torch.Tensor] = [e(S, D) for _ in range(c.layers)]
            self.hb = dict(xf=e(S, D), hf=e(S, D), rf=f(S), logits=e(S, c.vocab), dlogits=e(S, c.vocab),
                           dhf=e(S, D), loss=f(1), tok_loss=f(S))

    # ---------------------------------------------------------------- one layer
    def _lin(self, L: Layer, st: str, inp, out):
        ad = L.stack_lora.get(st)
        if ad is None:
            nl.linear_fwd(inp, L.W[st], y=out, workspace=self.lws)
        else:
            nl.linear_fwd(inp, L.W[st], ad["A"], ad["B"], self.s, y=out, t_out=self.T[st], workspace=self.lws)

    def _lin_bwd(self, L: Layer, st: str, dy, out):
        ad = L.stack_lora.get(st)
        if ad is None:
            nl.linear_bwd_input(dy, L.W[st], dx=out, workspace=self.lws)
        else:
            nl.linear_bwd_input(dy, L.W[st], ad["A"], ad["B"], self.s, dx=out, u_out=self.U[st],
                                workspace=self.lws)

    def layer_forward(self, L: Layer, xin, res=None, x_out=None):
        """Runs the layer on x = xin + res (written to x_out) or on x = xin when
        res is None. Returns (x2, dn): the layer output is x2 + dn, which the
        next layer's fused add + RMSNorm forms. Everything the backward needs
        stays in the shared buffers until the next call."""
        c, b, v = self.cfg, self.b, self.v_
        if res is None:
            x = xin
            nl.add_rmsnorm(x, L.gamma1, c.eps, y=b["h1"], rstd=b["r1"])
        else:
            x = b["x"] if x_out is None else x_out
            nl.add_rmsnorm(xin, L.gamma1, c.eps, res=res, sum_out=x, y=b["h1"], rstd=b["r1"])
        self.cur_x = x
        self._lin(L, "qkv", b["h1"], b["qkv"])
        nl.rope_(v["qk"], c.heads + c.kv_heads, c.head_dim, c.theta)  # the q and k heads in one call
        nl.attention_fwd(v["q"], v["k"], v["v"], c.heads, c.kv_heads, c.head_dim, o=b["a"], lse=b["lse"])
        self._lin(L, "o_proj", b["a"], b["o"])
        nl.add_rmsnorm(x, L.gamma2, c.eps, res=b["o"], sum_out=b["x2"], y=b["h2"], rstd=b["r2"])
        self._lin(L, "gate_up", b["h2"], b["gu"])
        nl.swiglu(v["g"], v["u"], a=b["sw"])
        self._lin(L, "down_proj", b["sw"], b["dn"])
        return b["x2"], b["dn"]

    def layer_backward(self, L: Layer, dout, dx_out):
        """Backward of the layer whose forward ran last: dout is the gradient
        of its output x2 + dn. Writes the gradient of its input x into dx_out
        (which must not alias dout) and every adapter's dA, dB."""
        c, b, v = self.cfg, self.b, self.v_
        self._lin_bwd(L, "down_proj", dout, b["dsw"])
        nl.swiglu_bwd(b["dsw"], v["g"], v["u"], dg=v["dg"], du=v["du"])
        self._lin_bwd(L, "gate_up", b["dgu"], b["dh2"])  # gate's and up's input gradients, summed
        nl.rmsnorm_bwd(b["dh2"], b["x2"], b["r2"], L.gamma2, dres=dout, dx=b["dx2"])
        self._lin_bwd(L, "o_proj", b["dx2"], b["da"])
        nl.attention_bwd(b["da"], v["q"], v["k"], v["v"], b["a"], b["lse"], c.heads, c.kv_heads, c.head_dim,
                         dq=v["dq"], dk=v["dk"], dv=v["dv"], delta=b["delta"])
        nl.rope_(v["dqk"], c.heads + c.kv_heads, c.head_dim, c.theta, inverse=True)
        self._lin_bwd(L, "qkv", b["dqkv"], b["dh1"])  # q's, k's and v's input gradients, summed
        nl.rmsnorm_bwd(b["dh1"], self.cur_x, b["r1"], L.gamma1, dres=b["dx2"], dx=dx_out)
        ins = {"qkv": (b["h1"], b["dqkv"]), "o_proj": (b["a"], b["dx2"]), "gate_up": (b["h2"], b["dgu"]),
               "down_proj": (b["sw"], dout)}
        for st, ad in L.stack_lora.items():
            xi, dyi = ins[st]
            nl.lora_grad(xi, dyi, self.T[st], self.U[st], self.s, dA=ad["dA"], dB=ad["dB"], workspace=self.gws[st])
            if ad["mask"] is not None:
                ad["dB"].mul_(ad["mask"])  # only the members' own blocks of B are parameters
        return dx_out

    # ---------------------------------------------------------------- the step
    def forward_backward(self, ids: torch.Tensor, targets: torch.Tensor) -> torch.Tensor:
        """Loss (device [1]) over token ids [S] (int64) with targets [S], and
        every adapter's gradient of it; the base weights stay frozen."""
        if not self.with_head:
            raise ValueError("the model was built without embedding and lm_head")
        c, hb = self.cfg, self.hb
        nl.embedding_rows(self.embed, ids, self.dt, out=self.saved[0])
        x2, dn = self.layer_forward(self.layers[0], self.saved[0])
        for i in range(1, c.layers):
            x2, dn = self.layer_forward(self.layers[i], x2, dn, x_out=self.saved[i])
        nl.add_rmsnorm(x2, self.gamma_f, c.eps, res=dn, sum_out=hb["xf"], y=hb["hf"], rstd=hb["rf"])
        nl.linear_fwd(hb["hf"], self.lm_head, y=hb["logits"], workspace=self.lws)
        nl.cross_entropy(hb["logits"], targets, dz=hb["dlogits"], tok_loss=hb["tok_loss"], loss=hb["loss"])
        nl.linear_bwd_input(hb["dlogits"], self.lm_head, dx=hb["dhf"], workspace=self.lws)
        grad = [self.b["gA"], self.b["gB"]]
        nl.rmsnorm_bwd(hb["dhf"], hb["xf"], hb["rf"], self.gamma_f, dx=grad[0])
        for i in reversed(range(c.layers)):
            L = self.layers[i]
            self.layer_forward(L, self.saved[i])  # recompute from the saved x
            self.layer_backward(L, grad[0], grad[1])
            grad.reverse()
        return hb["loss"]

    def adapters(self) -> List[dict]:
        return [dict((k, ad[k]) for k in ("A", "dA", "mA", "vA", "B", "dB", "mB", "vB"))
                for L in self.layers for ad in L.stack_lora.values()]

    def optimizer_step(self, lr: float = 2e-4, weight_decay: float = 0.0) -> None:
        self.step_count += 1
        ads = self.adapters()
        for j in range(0, len(ads), nl.MAX_ADAPTERS_PER_CALL):
            nl.lora_adamw_step_many(ads[j:j + nl.MAX_ADAPTERS_PER_CALL], step=self.step_count, lr=lr,
                                    weight_decay=weight_decay)

    def train_step(self, ids: torch.Tensor, targets: torch.Tensor, lr: float = 2e-4) -> torch.Tensor:
        loss = self.forward_backward(ids, targets)
        self.optimizer_step(lr)
        return loss
