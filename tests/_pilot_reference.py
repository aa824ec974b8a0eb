"""CPU reference of the pilot decoder stack (associative_algebra_block_amd.pilot_stack)
for the parity tests: the same architecture in float64 on the host, with
values rounded to bf16 wherever the GPU model stores bf16 (inputs of every
matrix product, the products' bf16 results, the SwiGLU hidden activation),
and the FFN computed by the fp64 oracle (the row-typed projection under the
model's law, or a plain matrix product for the dense FFN).

Teacher-forced: given the full token sequences (prompt plus the tokens the
GPU chose), it returns the final hidden state (after the last LayerNorm,
before rounding) and the logits at every position.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _h(t):
    return t.detach().double().cpu().numpy()


def _ln(x, w, b, eps=1e-5):
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * w + b


def host_weights(w):
    """float64 host copies of the model's parameters (exact values of the
    bf16 and float32 tensors the GPU holds)."""
    out = {k: _h(w[k]) for k in ("E", "P", "lnf_w", "lnf_b")}
    out["layers"] = [{k: _h(v) for k, v in lw.items()} for lw in w["layers"]]
    return out


def forward(cfg, hw, tokens, ffn: str, last_only=False):
    """tokens: int array [B, T].  Returns (hidden [B, T, d], logits [B, T, V])
    in float64; logits are the bf16-rounded products, like the GPU's."""
    B, T = tokens.shape
    d, Hh = cfg.d, cfg.heads
    hd = d // Hh
    x = hw["E"][tokens] + hw["P"][:T][None]                       # [B, T, d]
    types = oracle.types_pos_mod(T, cfg.q)                           # row type = position mod 4
    causal = np.triu(np.full((T, T), -np.inf), 1)
    for lw in hw["layers"]:
        a = _bf16(_ln(x, lw["ln1_w"], lw["ln1_b"]))
        qkv = _bf16(a @ lw["Wqkv"]) + lw["bqkv"]
        qkv = qkv.reshape(B, T, 3, Hh, hd)
        q, k, v = (qkv[:, :, i].transpose(0, 2, 1, 3) for i in range(3))   # [B, H, T, hd]
        s = q @ k.transpose(0, 1, 3, 2) / math.sqrt(hd) + causal
        s = np.exp(s - s.max(axis=-1, keepdims=True))
        p = s / s.sum(axis=-1, keepdims=True)
        o = (p @ v).transpose(0, 2, 1, 3).reshape(B, T, d)
        x = x + _bf16(_bf16(o) @ lw["Wo"]) + lw["bo"]
        f = _bf16(_ln(x, lw["ln2_w"], lw["ln2_b"]))
        y = np.empty_like(x)
        for b in range(B):
            if ffn == "algebra":
                G = oracle.project(f[b], lw["Wg"], "Q2xQ2", cfg.q, types)
                U = oracle.project(f[b], lw["Wu"], "Q2xQ2", cfg.q, types)
                Hb = _bf16(oracle.silu(G) * U)
                y[b] = oracle.project(Hb, lw["Wd"], "Q2xQ2", cfg.q, types)
            else:
                # torch's bf16 ops: both products and silu's result are rounded to bf16
                Hb = _bf16(_bf16(oracle.silu(_bf16(f[b] @ lw["Wg"]))) * _bf16(f[b] @ lw["Wu"]))
                y[b] = _bf16(Hb @ lw["Wd"])
        x = x + y
    hf = _ln(x, hw["lnf_w"], hw["lnf_b"])
    if last_only:
        hf = hf[:, -1:]
    logits = _bf16(_bf16(hf) @ hw["E"].T)
    return hf, logits
