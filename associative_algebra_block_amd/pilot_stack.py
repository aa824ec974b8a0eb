"""A decoder stack shaped like the pilot 110M model, for fixed-length
generation timing with a dense FFN and with the algebra FFN.

The agihunt.info review of "Change the Product, Keep the Parameters" describes
the pilot models (model paragraph): 12 layers, width 768, 32 heads, context
1536, the GPT-2 vocabulary, a SwiGLU FFN of width 1536 whose three projections
use the tensor square of Q2 (every other part dense), 110,631,168 parameters.
Its limitations paragraph asks for fixed-length full-model timing to isolate
the layer's effect on generation speed, and its closing discussion attributes
the small end-to-end gain to attention, the LM head, sampling and memory.

The parameter count fixes the rest of the block, read as GPT-2's: a tied
50257 x 768 token embedding, a learned 1536 x 768 position embedding, per
layer two LayerNorms (weight and bias), attention projections with biases
(QKV 768 -> 2304 and output 768 -> 768) and a SwiGLU FFN without biases, and a
final LayerNorm; pre-LN residual blocks; greedy sampling.  The weights are
seeded synthetic values (no trained model is used): embeddings N(0, 0.02^2),
projections N(0, 1/fan_in), biases N(0, 0.02^2), LayerNorms the identity.

Only the FFN is the library's: with ffn="algebra" it is aa_swiglu_ffn_fwd
under the Q2 x Q2 law (row type = position mod 4); with ffn="dense" it is
three torch.matmul products and silu * mul on the same weights.  Everything
else (embedding lookups, LayerNorms, the attention projections, attention over
a KV cache, the LM head, argmax) is plain torch, identical in both models.
Attention runs in float32 (scores and cache); the projections take bf16
operands, as the FFN does.

One decode step advances every sequence of the batch by one token at the
position held in a device tensor, so a step can be captured in a HIP graph
and replayed for any position: the algebra FFN takes the row types from a
device tensor (pos mod 4) through an explicitly typed plan.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import aa_plan_create, aa_swiglu_ffn_fwd, pack


@dataclass(frozen=True)
class PilotConfig:
    layers: int = 12
    d: int = 768
    heads: int = 32
    ffn: int = 1536
    ctx: int = 1536
    vocab: int = 50257
    q: int = 4                 # Q2 x Q2: four feature groups

    def parameter_count(self) -> int:
        d, F = self.d, self.ffn
        per_layer = (4 * d * d + 4 * d) + 3 * d * F + 2 * 2 * d
        return self.vocab * d + self.ctx * d + self.layers * per_layer + 2 * d


def _normal(shape, seed, std, dtype, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    return (torch.randn(tuple(shape), generator=g, device=dev, dtype=torch.float32) * std).to(dtype)


def make_weights(cfg: PilotConfig, seed: int, dev) -> dict:
    """Seeded synthetic parameters of the whole model (both FFN variants use
    the same ones).  Matrices are bf16, biases and norms float32."""
    d, F = cfg.d, cfg.ffn
    s = 100000 + 1000 * seed
    w = {"E": _normal((cfg.vocab, d), s + 1, 0.02, torch.bfloat16, dev),
         "P": _normal((cfg.ctx, d), s + 2, 0.02, torch.float32, dev),
         "lnf_w": torch.ones(d, device=dev), "lnf_b": torch.zeros(d, device=dev), "layers": []}
    w["E_T"] = w["E"].t().contiguous()   # the tied LM head, stored transposed for a plain product
    for l in range(cfg.layers):
        b = s + 100 * (l + 1)
        w["layers"].append({
            "ln1_w": torch.ones(d, device=dev), "ln1_b": torch.zeros(d, device=dev),
            "Wqkv": _normal((d, 3 * d), b + 1, d ** -0.5, torch.bfloat16, dev),
            "bqkv": _normal((3 * d,), b + 2, 0.02, torch.float32, dev),
            "Wo": _normal((d, d), b + 3, d ** -0.5, torch.bfloat16, dev),
            "bo": _normal((d,), b + 4, 0.02, torch.float32, dev),
            "ln2_w": torch.ones(d, device=dev), "ln2_b": torch.zeros(d, device=dev),
            "Wg": _normal((d, F), b + 5, d ** -0.5, torch.bfloat16, dev),
            "Wu": _normal((d, F), b + 6, d ** -0.5, torch.bfloat16, dev),
            "Wd": _normal((F, d), b + 7, F ** -0.5, torch.bfloat16, dev),
        })
    return w


class PilotGenerator:
    """Batched greedy generation through the stack, with a KV cache.

    prefill(tokens) runs a [B, P] prompt (P a multiple of 4) in one pass and
    leaves the next token of each sequence in `self.token`; decode_step()
    advances all B sequences by one position (device-side position, so the
    step can be captured in a HIP graph)."""

    def __init__(self, cfg: PilotConfig, weights: dict, ffn: str, batch: int, dev, argmax_in_step=True):
        if ffn not in ("algebra", "dense"):
            raise ValueError("ffn must be 'algebra' or 'dense'")
        self.cfg, self.w, self.ffn, self.B, self.dev = cfg, weights, ffn, batch, dev
        self.argmax_in_step = argmax_in_step
        # when a list: every FFN call appends (layer, FFN input, FFN output,
        # prompt length of a prefill or 0, the decode row types or None);
        # for checks, in eager use only
        self.trace = None
        H, hd, L = cfg.heads, cfg.d // cfg.heads, cfg.layers
        self.hd = hd
        # K cache stored transposed (head dim before position) so that q K^T is
        # a product with a contiguous right operand
        self.Kt = torch.zeros(L, batch * H, hd, cfg.ctx, device=dev)
        self.V = torch.zeros(L, batch * H, cfg.ctx, hd, device=dev)
        self.pos = torch.zeros(1, dtype=torch.int64, device=dev)
        self.token = torch.zeros(batch, dtype=torch.int64, device=dev)
        self.types = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.logits = torch.zeros(batch, cfg.vocab, dtype=torch.bfloat16, device=dev)
        self.hidden = torch.zeros(batch, cfg.d, device=dev)   # final LayerNorm output of the last step
        self.ar = torch.arange(cfg.ctx, device=dev)
        if ffn == "algebra":
            law, q, d, F = "Q2xQ2", cfg.q, cfg.d, cfg.ffn
            self.up_dec = aa_plan_create(law, q, d, F, "explicit", 0, "bf16", "bf16")
            self.down_dec = aa_plan_create(law, q, F, d, "explicit", 0, "bf16", "f32")
            self.packed = [(pack(self.up_dec, lw["Wg"]), pack(self.up_dec, lw["Wu"]), pack(self.down_dec, lw["Wd"]))
                           for lw in weights["layers"]]
            self.H_dec = torch.empty(batch, F, dtype=torch.bfloat16, device=dev)
            self.Y_dec = torch.empty(batch, d, dtype=torch.float32, device=dev)
            self._pre = {}

    # ------------------------------------------------------------ pieces ---

    def _ffn(self, l: int, f: torch.Tensor, prefill_len: int = 0) -> torch.Tensor:
        """FFN of layer l on bf16 rows f [M, d]; float32 [M, d]."""
        lw = self.w["layers"][l]
        if self.ffn == "dense":
            h = torch.nn.functional.silu(torch.matmul(f, lw["Wg"])) * torch.matmul(f, lw["Wu"])
            y = torch.matmul(h, lw["Wd"]).float()
        else:
            g, u, dn = self.packed[l]
            M = f.shape[0]
            if prefill_len:
                # rows are B sequences of prefill_len positions laid end to end
                up, down, H, y = self._prefill_plans(prefill_len, M)
                aa_swiglu_ffn_fwd(up, down, f, g, u, dn, H, y, None, 0)
            else:
                y = self.Y_dec
                aa_swiglu_ffn_fwd(self.up_dec, self.down_dec, f, g, u, dn, self.H_dec, y, None, 0, self.types)
        if self.trace is not None:
            self.trace.append((l, f.clone(), y.clone(), prefill_len, None if prefill_len else self.types.clone()))
        return y

    def _prefill_plans(self, P: int, M: int):
        key = (P, M)
        if key not in self._pre:
            law, q, d, F = "Q2xQ2", self.cfg.q, self.cfg.d, self.cfg.ffn
            up = aa_plan_create(law, q, d, F, "pos_mod", P, "bf16", "bf16")
            down = aa_plan_create(law, q, F, d, "pos_mod", P, "bf16", "f32")
            self._pre[key] = (up, down, torch.empty(M, F, dtype=torch.bfloat16, device=self.dev),
                              torch.empty(M, d, dtype=torch.float32, device=self.dev))
        return self._pre[key]

    def _ln(self, x, wt, b):
        return torch.nn.functional.layer_norm(x, (self.cfg.d,), wt, b, 1e-5)

    def _qkv(self, lw, a_bf16):
        return torch.matmul(a_bf16, lw["Wqkv"]).float() + lw["bqkv"]

    # ---------------------------------------------------------- prefill ---

    def prefill(self, tokens: torch.Tensor) -> torch.Tensor:
        """Run a [B, P] prompt; returns the float32 final hidden states
        [B, P, d] and leaves the next tokens in self.token, P in self.pos."""
        cfg, B = self.cfg, self.B
        P = tokens.shape[1]
        if tokens.shape[0] != B or P % cfg.q or P > cfg.ctx:
            raise ValueError("prompt must be [batch, P] with P a multiple of 4 and at most the context")
        Hh, hd, d = cfg.heads, self.hd, cfg.d
        M = B * P
        x = self.w["E"][tokens.reshape(-1)].float() + self.w["P"][:P].repeat(B, 1)   # [M, d]
        causal = torch.triu(torch.full((P, P), float("-inf"), device=self.dev), diagonal=1)
        for l, lw in enumerate(self.w["layers"]):
            a = self._ln(x, lw["ln1_w"], lw["ln1_b"]).to(torch.bfloat16)
            qkv = self._qkv(lw, a).view(B, P, 3, Hh, hd)
            q = qkv[:, :, 0].permute(0, 2, 1, 3).reshape(B * Hh, P, hd)
            k = qkv[:, :, 1].permute(0, 2, 1, 3).reshape(B * Hh, P, hd)
            v = qkv[:, :, 2].permute(0, 2, 1, 3).reshape(B * Hh, P, hd).contiguous()
            kt = k.transpose(1, 2).contiguous()
            self.Kt[l, :, :, :P] = kt
            self.V[l, :, :P] = v
            s = torch.bmm(q.contiguous(), kt) * (1.0 / math.sqrt(hd)) + causal
            o = torch.bmm(torch.softmax(s, dim=-1), v)                       # [B H, P, hd]
            o = o.view(B, Hh, P, hd).permute(0, 2, 1, 3).reshape(M, d)
            x = x + torch.matmul(o.to(torch.bfloat16), lw["Wo"]).float() + lw["bo"]
            f = self._ln(x, lw["ln2_w"], lw["ln2_b"]).to(torch.bfloat16)
            x = x + self._ffn(l, f, prefill_len=P)
        hf = self._ln(x, self.w["lnf_w"], self.w["lnf_b"])
        last = hf.view(B, P, d)[:, -1].to(torch.bfloat16)
        self.logits.copy_(torch.matmul(last, self.w["E_T"]))
        self.token.copy_(torch.argmax(self.logits, dim=-1))
        self.pos.fill_(P)
        return hf.view(B, P, d)

    # ----------------------------------------------------------- decode ---

    def decode_step(self) -> None:
        """Feed self.token at position self.pos for every sequence; write the
        logits, the next token (argmax) and advance the position.  Reads the
        position only from device memory."""
        cfg, B = self.cfg, self.B
        Hh, hd, d = cfg.heads, self.hd, cfg.d
        pos = self.pos
        self.types.copy_(torch.remainder(pos, cfg.q).to(torch.int32).expand(B))
        x = torch.index_select(self.w["E"], 0, self.token).float() + torch.index_select(self.w["P"], 0, pos)
        keep = self.ar.le(pos)                                         # positions 0 .. pos
        bias = torch.where(keep, 0.0, float("-inf"))                   # [ctx]
        for l, lw in enumerate(self.w["layers"]):
            a = self._ln(x, lw["ln1_w"], lw["ln1_b"]).to(torch.bfloat16)
            qkv = self._qkv(lw, a).view(B, 3, Hh, hd)
            q = qkv[:, 0].reshape(B * Hh, 1, hd)
            k = qkv[:, 1].reshape(B * Hh, hd, 1)
            v = qkv[:, 2].reshape(B * Hh, 1, hd)
            self.Kt[l].index_copy_(2, pos, k)
            self.V[l].index_copy_(1, pos, v)
            s = torch.bmm(q, self.Kt[l]) * (1.0 / math.sqrt(hd)) + bias       # [B H, 1, ctx]
            o = torch.bmm(torch.softmax(s, dim=-1), self.V[l]).view(B, d)
            x = x + torch.matmul(o.to(torch.bfloat16), lw["Wo"]).float() + lw["bo"]
            f = self._ln(x, lw["ln2_w"], lw["ln2_b"]).to(torch.bfloat16)
            x = x + self._ffn(l, f)
        hf = self._ln(x, self.w["lnf_w"], self.w["lnf_b"])
        self.hidden.copy_(hf)
        self.logits.copy_(torch.matmul(hf.to(torch.bfloat16), self.w["E_T"]))
        if self.argmax_in_step:
            self.pick()
        pos.add_(1)

    def pick(self) -> None:
        """Greedy sampling of the next tokens from the last logits."""
        self.token.copy_(torch.argmax(self.logits, dim=-1))
