"""OLMo-2-370M-style decoder stack whose linear layers all run through libtj2.

The stack the pages train (TetraJet-v2 technical summary, section 4: OLMo-2
models up to 370M parameters) is the setting of the quantized linear layer:
every linear layer -- the fused QKV projection, the attention output, the
SwiGLU gate, up and down projections and the LM head -- is an NVFP4 linear
(section 2.A) with static FP8 outlier channels (section 2.C) and fp32 master
weights updated by the fused master-weight pass (AdamW, then OsciReset,
section 2.B, with the reset switched on once the learning rate is low).

Everything outside the linear layers is glue and is plain PyTorch on the GPU:
token embedding, RMSNorm (pre-norm), rotary position embedding, causal bf16
attention (the fused flash / memory-efficient kernels only), SwiGLU, the
cross-entropy loss, and AdamW on the embedding and norm weights.  The pages
give no OLMo-2 details; the layout here (pre-norm blocks, RoPE theta 10000,
16 heads of 64, untied LM head) is the plainest one of that family.

With linear="bf16" the same stack runs its linear layers as bf16 products
(torch.mm, hipBLASLt) on bf16 copies of the masters, with AdamW on the
masters: the comparator of the pages' end-to-end speed figure on this part.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch
import torch.nn.functional as F
from torch.nn.attention import SDPBackend, sdpa_kernel

from . import (FP8, NVFP4, OSCI_ACCUM, OSCI_INIT, OSCI_WINDOW_END, MasterBatch, NextBwd, QTensor, bwd_operands,
               channel_sumsq, lib, linear_bwd, linear_fwd, master_update_step_multi, osci_reset_step,
               select_outliers)


@dataclass
class DecoderConfig:
    vocab: int = 50304
    d_model: int = 1024
    layers: int = 16
    heads: int = 16
    ffn: int = 4096
    seq: int = 2048
    batch: int = 8
    p_outliers: float = 0.10        # OutControl: top 10% input channels of each linear in FP8
    lr_start: float = 1e-4          # linear decay lr_start -> lr_end over total_steps
    lr_end: float = 1e-6
    total_steps: int = 200
    window: int = 50                # OsciReset risk window (optimizer steps)
    tau: float = 4.0                # reset where dist_Q > tau * dist_M over the window
    reset_lr: float = 2e-5          # resets are enabled once lr <= reset_lr ("when the learning rate is low")
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    rope_theta: float = 10000.0
    norm_eps: float = 1e-6
    init_std: float = 0.02
    seed: int = 0                   # parameters and Philox stream
    linear: str = "nvfp4"           # "nvfp4" (libtj2) or "bf16" (comparator)

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def lr(self, step: int) -> float:
        f = min(max(step, 0), self.total_steps) / self.total_steps
        return self.lr_start + (self.lr_end - self.lr_start) * f

    def linear_flops_per_step(self) -> float:
        d, f, V, M = self.d_model, self.ffn, self.vocab, self.tokens
        per_layer = 3 * d * d + d * d + 2 * f * d + d * f
        return 6.0 * M * (self.layers * per_layer + V * d)


class _LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, X, lin):
        Y, saved = lin.forward(X)
        ctx.lin, ctx.saved = lin, saved
        return Y

    @staticmethod
    def backward(ctx, dY):
        return ctx.lin.backward(dY.contiguous(), ctx.saved), None


class Linear:
    """One linear layer Y = X W^T of the stack (W [N, K]): the fp32 master with its AdamW moments and
    OsciReset state, the forward codes under the layer's outlier plan, and the next backward's
    re-grouped weights that the master pass forms."""

    def __init__(self, stack: "Decoder", idx: int, name: str, N: int, K: int, gen: torch.Generator):
        self.stack, self.idx, self.name, self.N, self.K = stack, idx, name, N, K
        dev = stack.device
        self.W = (torch.randn(N, K, generator=gen, device=dev) * stack.cfg.init_std).contiguous()
        self.grad = torch.zeros_like(self.W)
        self.m, self.v = torch.zeros_like(self.W), torch.zeros_like(self.W)
        self.plan = None
        self.sumsq = None
        self.capture = None  # dict: the call's inputs and outputs are recorded into it
        self.w_given = False
        self.Wf = None       # bf16 comparator: bf16 copies of W^T [K, N] (forward) and W [N, K] (backward)
        self.Wg = None

    # ---- set-up ---------------------------------------------------------------------------------
    def finalize(self):
        """After calibration: codes, OsciReset state (INIT) and next-backward buffers under the plan."""
        n = self.plan.n if self.plan is not None else 0
        K1 = self.K - n
        self.Q_prev, self.dQ, self.dM = (torch.empty_like(self.W) for _ in range(3))
        self.Wq = QTensor(NVFP4, self.N, K1)
        self.W8 = QTensor(FP8, self.N, n) if n else None
        W_prev = torch.empty_like(self.W)
        osci_reset_step(self.W, W_prev, self.Q_prev, self.dQ, self.dM, mode=OSCI_INIT, plan=self.plan,
                        Wq_out=self.Wq, W8_out=self.W8)
        del W_prev
        self.next = NextBwd(QTensor(NVFP4, K1, self.N), QTensor(FP8, n, self.N) if n else None,
                            seed=self.stack.cfg.seed, offset=0, rht=True)

    # ---- products -------------------------------------------------------------------------------
    def forward(self, X: torch.Tensor):
        st = self.stack
        if st.cfg.linear == "bf16":
            return torch.mm(X, self.Wf), X
        if st.calibrating:
            channel_sumsq(X, self.sumsq)
            return linear_fwd(X, self.W, self.N)
        Y, saved = linear_fwd(X, None, self.N, Wq=self.Wq, W8=self.W8, plan=self.plan)
        if self.capture is not None:
            self.capture.update(X=X.clone(), W=self.W.clone(), Y=Y.clone(), step=st.step,
                                saved={k: (q.clone() if q is not None else None) for k, q in saved.items()})
        return Y, saved

    def backward(self, dY: torch.Tensor, saved):
        st = self.stack
        if st.cfg.linear == "bf16":
            X = saved
            torch.mm(dY.t(), X, out=self.gradb)
            self.grad.copy_(self.gradb)
            return torch.mm(dY, self.Wg)
        offset = st.offset(self.idx, st.step)
        cap = self.capture
        ops = bwd_operands(dY.shape[0], self.N, self.K, self.plan) if cap is not None else dict(st.ops_for(self))
        if self.w_given:
            ops["Wt"] = self.next.Wt
            if self.plan is not None:
                ops["W8t"] = self.next.W8t
        dX, _, _ = linear_bwd(dY, saved, self.K, seed=st.cfg.seed, offset=offset, plan=self.plan,
                              dx_dtype=torch.bfloat16, operands=ops, w_given=self.w_given, workspace=st.bwd_ws,
                              dW=self.grad)
        if cap is not None:
            cap.update(dY=dY.clone(), dX=dX.clone(), dW=self.grad.clone(), offset=offset, w_given=self.w_given,
                       ops={k: q.clone() for k, q in ops.items()})
        return dX

    def __call__(self, X):
        return _LinearFn.apply(X, self)


class Decoder:
    """The decoder stack, its optimizer state and one training step."""

    def __init__(self, cfg: DecoderConfig, device="cuda"):
        self.cfg, self.device = cfg, device
        assert cfg.d_model % cfg.heads == 0 and cfg.linear in ("nvfp4", "bf16")
        g = torch.Generator(device=device)
        g.manual_seed(cfg.seed)
        d = cfg.d_model
        self.emb = (torch.randn(cfg.vocab, d, generator=g, device=device) * cfg.init_std).requires_grad_(True)
        self.final_norm = torch.ones(d, device=device, requires_grad=True)
        self.blocks = []
        self.linears = []

        def lin(name, N, K):
            L = Linear(self, len(self.linears), name, N, K, g)
            self.linears.append(L)
            return L

        for i in range(cfg.layers):
            self.blocks.append({
                "attn_norm": torch.ones(d, device=device, requires_grad=True),
                "qkv": lin(f"{i}.qkv", 3 * d, d), "o": lin(f"{i}.o", d, d),
                "mlp_norm": torch.ones(d, device=device, requires_grad=True),
                "gate": lin(f"{i}.gate", cfg.ffn, d), "up": lin(f"{i}.up", cfg.ffn, d),
                "down": lin(f"{i}.down", d, cfg.ffn)})
        self.head = lin("head", cfg.vocab, d)
        norms = [self.final_norm] + [b[k] for b in self.blocks for k in ("attn_norm", "mlp_norm")]
        self.glue_opt = torch.optim.AdamW([{"params": [self.emb], "weight_decay": cfg.weight_decay},
                                           {"params": norms, "weight_decay": 0.0}],
                                          lr=cfg.lr_start, betas=(cfg.beta1, cfg.beta2), eps=cfg.eps)
        hd = d // cfg.heads
        inv = 1.0 / (cfg.rope_theta ** (torch.arange(0, hd, 2, device=device, dtype=torch.float32) / hd))
        ang = torch.arange(cfg.seq, device=device, dtype=torch.float32)[:, None] * inv[None, :]
        self.cos, self.sin = ang.cos(), ang.sin()
        self.step = 0
        self.calibrating = False
        self.ready = False
        self._ops = {}
        self.bwd_ws = None
        self.reset_count = torch.zeros(1, dtype=torch.int64, device=device)

    # ---- glue -------------------------------------------------------------------------------------
    def _rmsnorm(self, x, w):
        xf = x.float()
        return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + self.cfg.norm_eps) * w).to(torch.bfloat16)

    def _rope(self, t):  # t [B, H, S, hd]
        t1, t2 = t.float().unflatten(-1, (-1, 2)).unbind(-1)
        c, s = self.cos[: t.shape[2]], self.sin[: t.shape[2]]
        return torch.stack((t1 * c - t2 * s, t1 * s + t2 * c), dim=-1).flatten(-2).to(torch.bfloat16)

    def forward(self, tokens: torch.Tensor) -> torch.Tensor:
        """Logits [B*S, vocab] (bf16) of tokens [B, S]."""
        cfg = self.cfg
        B, S = tokens.shape
        M, d, H = B * S, cfg.d_model, cfg.heads
        x = F.embedding(tokens.reshape(-1), self.emb).to(torch.bfloat16)
        for blk in self.blocks:
            qkv = blk["qkv"](self._rmsnorm(x, blk["attn_norm"]))
            q, k, v = qkv.view(B, S, 3, H, d // H).permute(2, 0, 3, 1, 4).unbind(0)
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
                o = F.scaled_dot_product_attention(self._rope(q), self._rope(k), v.contiguous(), is_causal=True)
            x = x + blk["o"](o.transpose(1, 2).reshape(M, d).contiguous())
            h = self._rmsnorm(x, blk["mlp_norm"])
            a = F.silu(blk["gate"](h)) * blk["up"](h)
            x = x + blk["down"](a.contiguous())
        return self.head(self._rmsnorm(x, self.final_norm))

    # ---- set-up -----------------------------------------------------------------------------------
    def offset(self, idx: int, step: int) -> int:
        """Philox offset slot (8 per call) of linear idx's backward at a step."""
        return 8 * (step * len(self.linears) + idx)

    def ops_for(self, lin: Linear) -> dict:
        key = (self.cfg.tokens, lin.N, lin.K, lin.plan.n if lin.plan is not None else 0)
        if key not in self._ops:
            self._ops[key] = bwd_operands(self.cfg.tokens, lin.N, lin.K, lin.plan)
        return self._ops[key]

    def calibrate(self, batches):
        """OutControl: the top p% input channels of every linear from a short calibration window
        (forward passes with plain NVFP4 products), then the codes and OsciReset state under the plans."""
        if self.cfg.linear == "nvfp4":
            for L in self.linears:
                L.sumsq = torch.zeros(L.K, dtype=torch.float64, device=self.device)
            self.calibrating = True
            with torch.no_grad():
                for tokens in batches:
                    self.forward(tokens)
            self.calibrating = False
            for L in self.linears:
                L.plan = select_outliers(L.sumsq, self.cfg.p_outliers, device=self.device)
                L.sumsq = None
                L.finalize()
            # split-K partial sums of the backward products (the operands have buffers of their own)
            M = self.cfg.tokens
            ws = max(max(int(lib().nvfp4_gemm_workspace_size(M, L.K, L.N, 0)),
                          int(lib().nvfp4_gemm_workspace_size(L.N, L.K, M, 0))) for L in self.linears)
            self.bwd_ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=self.device)
            self.master_batch = MasterBatch([(L.W, L.m, L.v, L.grad, L.Q_prev, L.dQ, L.dM, L.Wq, L.plan, L.W8, L.next)
                                             for L in self.linears])
        else:
            self.lin_opt = torch.optim.AdamW([L.W for L in self.linears], lr=self.cfg.lr_start,
                                             betas=(self.cfg.beta1, self.cfg.beta2), eps=self.cfg.eps,
                                             weight_decay=self.cfg.weight_decay)
            for L in self.linears:
                L.W.grad = L.grad
                L.gradb = torch.empty(L.N, L.K, dtype=torch.bfloat16, device=self.device)
                L.Wf = L.W.t().contiguous().to(torch.bfloat16)
                L.Wg = L.W.to(torch.bfloat16)
        self.ready = True

    # ---- training ---------------------------------------------------------------------------------
    def train_step(self, tokens: torch.Tensor, targets: torch.Tensor, before_update=None) -> torch.Tensor:
        """One optimizer step on one batch; returns the loss (a device scalar).  before_update(self),
        if given, runs after the backward pass and before the optimizer updates (for inspection)."""
        assert self.ready, "calibrate() first"
        cfg = self.cfg
        t = self.step
        lr = cfg.lr(t)
        logits = self.forward(tokens)
        loss = F.cross_entropy(logits.float(), targets.reshape(-1))
        loss.backward()
        if before_update is not None:
            before_update(self)
        for grp in self.glue_opt.param_groups:
            grp["lr"] = lr
        self.glue_opt.step()
        self.glue_opt.zero_grad(set_to_none=True)
        if cfg.linear == "nvfp4":
            bc1, bc2 = 1.0 - cfg.beta1 ** (t + 1), 1.0 - cfg.beta2 ** (t + 1)
            end = (t + 1) % cfg.window == 0
            self.master_batch.set_next_offsets([self.offset(L.idx, t + 1) for L in self.linears])
            master_update_step_multi(self.master_batch, lr=lr, bias_correction1=bc1, bias_correction2=bc2,
                                     beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps, weight_decay=cfg.weight_decay,
                                     mode=OSCI_WINDOW_END if end else OSCI_ACCUM, tau=cfg.tau,
                                     reset_enabled=lr <= cfg.reset_lr, reset_count=self.reset_count)
            for L in self.linears:
                L.w_given = True
        else:
            for grp in self.lin_opt.param_groups:
                grp["lr"] = lr
            self.lin_opt.step()
            for L in self.linears:
                L.Wf.copy_(L.W.t())
                L.Wg.copy_(L.W)
        self.step += 1
        return loss.detach()

    def linear_params(self) -> int:
        return sum(L.N * L.K for L in self.linears)


def random_tokens(cfg: DecoderConfig, seed: int, device="cuda"):
    """Synthetic batch: uniformly random token ids [batch, seq] and next-token targets."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randint(0, cfg.vocab, (cfg.batch, cfg.seq + 1), generator=g, device=device)
    return t[:, :-1].contiguous(), t[:, 1:].contiguous()
