"""The SwiGLU gate/up kernel for leaves with many rows per type (32 x 32
fragments, both operands staged in LDS) through the C ABI, against the fp64
oracle: ragged row tiles, output groups that are not a multiple of the
128-output tile, odd numbers of K stages, both laws, both typings, bf16 and
fp32 hidden outputs.  Each case also runs the 16 x 16 tile kernel (AA_TILE=501)
on the same inputs.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

import aa_inputs as inp
import associative_algebra_block_amd as aa
import oracle
from tests._gpu_util import assert_parity, host, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available()
    aa.load()


CASES = [
    # law, q, M, b_in, b_out, typing, pos_offset
    ("Q2xQ2", 4, 4 * 700 + 3, 64, 144, "pos_mod", 1),     # 9 strips: second n-tile of 16 columns
    ("Q2xQ2", 4, 4 * 300, 192, 384, "block_rows", 0),     # the pilot's block shape, fewer rows
    ("Qq", 3, 3 * 300 + 1, 96, 160, "pos_mod", 2),        # three K stages per group: odd counts
    ("Qq", 5, 5 * 260, 32, 128, "block_rows", 0),         # one K stage per group
    ("Qq", 2, 2 * 1000 + 1, 128, 256, "pos_mod", 7),      # q = 2, two n-tiles
]


def _gate_up(law, q, M, b_in, b_out, kind, pos, h_dt, seed, monkeypatch, tile=None):
    if tile is None:
        monkeypatch.delenv("AA_TILE", raising=False)
    else:
        monkeypatch.setenv("AA_TILE", tile)
    D, F = q * b_in, q * b_out
    up = aa.aa_plan_create(law, q, D, F, kind, 0, "bf16", h_dt)
    down = aa.aa_plan_create(law, q, F, D, kind, 0, h_dt, "f32")   # H is down's input
    monkeypatch.delenv("AA_TILE", raising=False)
    X = inp.gaussian((M, D), seed + 1, 1.0, torch.bfloat16, DEV)
    Wg = inp.gaussian((D, F), seed + 2, D ** -0.5, torch.bfloat16, DEV)
    Wu = inp.gaussian((D, F), seed + 3, D ** -0.5, torch.bfloat16, DEV)
    Wd = inp.gaussian((F, D), seed + 4, F ** -0.5, torch.bfloat16, DEV).to(TD[h_dt])
    H = torch.full((M, F), float("nan"), dtype=TD[h_dt], device=DEV)
    Y = torch.empty(M, D, dtype=torch.float32, device=DEV)
    aa.aa_swiglu_ffn_fwd(up, down, X, aa.pack(up, Wg), aa.pack(up, Wu), aa.pack(down, Wd), H, Y, None, pos)
    torch.cuda.synchronize()
    return X, Wg, Wu, H


@pytest.mark.parametrize("law,q,M,b_in,b_out,kind,pos", CASES)
@pytest.mark.parametrize("h_dt", ["bf16", "f32"])
def test_tile32_gate_up_matches_oracle(law, q, M, b_in, b_out, kind, pos, h_dt, monkeypatch):
    say("tile32 gate/up", law, q, M, b_in, b_out, kind, pos, h_dt)
    seed = 700 + 13 * q + b_in
    X, Wg, Wu, H = _gate_up(law, q, M, b_in, b_out, kind, pos, h_dt, seed, monkeypatch)
    types = oracle.types_block_rows(M, q) if kind == "block_rows" else oracle.types_pos_mod(M, q, pos)
    Href = oracle.silu(oracle.project(host(X), host(Wg), law, q, types)) * oracle.project(host(X), host(Wu), law, q, types)
    h = host(H)
    assert np.isfinite(h).all(), "rows or columns left unwritten"
    assert_parity(h, Href, h_dt == "bf16", "tile32 H")
    # the 16 x 16 tile kernel on the same inputs, where it applies (b_in a multiple of 64)
    if b_in % 64 == 0:
        _, _, _, H16 = _gate_up(law, q, M, b_in, b_out, kind, pos, h_dt, seed, monkeypatch, tile="501")
        assert_parity(host(H16), Href, h_dt == "bf16", "16x16 tile H")
