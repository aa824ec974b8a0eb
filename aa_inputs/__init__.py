"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it draws Gaussian tensors from
seeded torch generators, rounds them to the storage dtype, and describes the
workload shapes.  Both the oracle side and the HIP side take their inputs from
here, and from nowhere else.

Recipe: X ~ N(0, 1); a weight with d_in input features ~ N(0, 1/d_in); values
drawn in float32 and rounded to bf16 with round-to-nearest-even (torch's
conversion) unless the workload is float32.  Seeds are 1000 * role + workload,
with the roles below.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

ROLE_X = 1
ROLE_W = 2      # the projection weight, or the SwiGLU gate weight
ROLE_WU = 3     # SwiGLU up weight
ROLE_WD = 4     # SwiGLU down weight
ROLE_W2 = 5     # second weight for associativity / composition checks
ROLE_TYPES = 6  # explicit row types


def seed_for(role: int, workload: int) -> int:
    return 1000 * role + workload


def gaussian(shape, seed: int, std: float = 1.0, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """N(0, std^2) drawn in float32 from a seeded generator, then cast to dtype."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def small_integers(shape, seed: int, lo: int = -3, hi: int = 3, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """Uniform integers in [lo, hi]; exactly representable in bf16."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randint(lo, hi + 1, tuple(shape), generator=g, device=device, dtype=torch.int32)
    return t.to(dtype)


def random_edges(q: int, density: float, seed: int) -> list:
    """Seeded edge set of a directed graph on q vertices: each ordered pair
    (i, k), i != k, is an edge with probability `density`."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    u = torch.rand((q, q), generator=g)
    return [(i, k) for i in range(q) for k in range(q) if i != k and float(u[i, k]) < density]


def random_types(M: int, q: int, seed: int, device="cpu") -> torch.Tensor:
    """Explicit per-row types, uniform over [0, q)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randint(0, q, (M,), generator=g, device=device, dtype=torch.int32)


@dataclass(frozen=True)
class Workload:
    """One workload from the pages' kernel measurements (shapes only)."""
    index: int
    name: str
    law: str            # "Qq" or "Q2xQ2"
    q: int
    M: int
    d_in: int
    d_out: int          # projection output width, or the FFN intermediate width
    kind: str           # "project", "ffn", "square"
    dtype: str          # "bf16" or "f32"
    type_map: str       # "pos_mod" or "block_rows"
    ffn: bool = False   # also run the SwiGLU forward at this shape
    decode_tokens: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def w_std(self, d_in: int | None = None) -> float:
        return 1.0 / math.sqrt(d_in if d_in is not None else self.d_in)


# Shapes of the pages' workloads (agihunt.info review: kernel speedup table,
# square-product sentence, SwiGLU sentence, and the pilot model paragraph).
WORKLOADS = {
    1: Workload(1, "q2_f32_small", "Qq", 2, 256, 64, 64, "project", "f32", "pos_mod",
                notes="Q_2, fp32, 32x32 blocks; also the full 64x64 product and associativity"),
    2: Workload(2, "pilot_ffn_q2xq2", "Q2xQ2", 4, 8 * 1536, 768, 1536, "ffn", "bf16", "pos_mod",
                ffn=True, notes="batch 8 x context 1536, width 768, SwiGLU width 1536",
                extra={"period": 1536}),
    3: Workload(3, "qwen3_8b_q32", "Qq", 32, 2048, 4096, 12288, "project", "bf16", "pos_mod",
                ffn=True, decode_tokens=32, notes="Qwen3-8B FFN shape, M=2048, q=32"),
    4: Workload(4, "qwen3_30b_a3b_expert_q16", "Qq", 16, 2048, 2048, 768, "ffn", "bf16", "pos_mod",
                ffn=True, notes="narrow expert FFN D=2048, F=768, q=16"),
    5: Workload(5, "square_n32768_b128", "Qq", 256, 32768, 32768, 32768, "square", "bf16", "block_rows",
                notes="fixed-block square product, b=128, q=256"),
    # a further row of the pages' projection table; widths from the model's
    # public configuration (hidden 2048, intermediate 6144)
    6: Workload(6, "qwen3_1p7b_q32", "Qq", 32, 2048, 2048, 6144, "project", "bf16", "pos_mod",
                notes="Qwen3-1.7B FFN shape, M=2048, q=32 (blocks 64 x 192)"),
    # the down projection of the Qwen3-8B SwiGLU FFN on its own
    7: Workload(7, "qwen3_8b_down_q32", "Qq", 32, 2048, 12288, 4096, "project", "bf16", "pos_mod",
                notes="Qwen3-8B FFN down projection, M=2048, q=32 (blocks 384 x 128)"),
    # the Qwen3-32B row of the pages' projection table; widths from the
    # model's public configuration (hidden 5120, intermediate 25600)
    8: Workload(8, "qwen3_32b_q256", "Qq", 256, 32768, 5120, 25600, "project", "bf16", "pos_mod",
                notes="Qwen3-32B FFN shape, M=32768, q=256 (blocks 20 x 100, packed layout 2)"),
}
