"""The FFN stack of the 110M pilot model decoded one token at a time (the
fixed-length generation timing the [review] page suggests for isolating the
layer's effect, here without attention): 12 SwiGLU blocks of width 768 and
hidden width 1536 under the Q2 x Q2 law, context 1536, each token through
every layer in turn.  Every test needs an MI355X and goes through the C ABI.
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
LAYERS, D, F, Q, PERIOD = 12, 768, 1536, 4, 1536


@pytest.fixture(scope="module")
def stack():
    assert torch.cuda.is_available()
    aa.load()
    up = aa.aa_plan_create("Q2xQ2", Q, D, F, "pos_mod", PERIOD, "bf16", "bf16")
    down = aa.aa_plan_create("Q2xQ2", Q, F, D, "pos_mod", PERIOD, "bf16", "bf16")
    raw = [(inp.gaussian((D, F), 300 + 3 * l, D ** -0.5, torch.bfloat16, DEV),
            inp.gaussian((D, F), 301 + 3 * l, D ** -0.5, torch.bfloat16, DEV),
            inp.gaussian((F, D), 302 + 3 * l, F ** -0.5, torch.bfloat16, DEV)) for l in range(LAYERS)]
    packed = [(aa.pack(up, g), aa.pack(up, u), aa.pack(down, d)) for g, u, d in raw]
    return up, down, raw, packed


def _bf16(a):
    """Round to bf16 (nearest even), as the library stores H and each layer's
    output; done on the host with torch's CPU conversion."""
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def _run_tokens(up, down, packed, x, H, Ys, pos0):
    """Token j (position pos0 + j) through every layer, one call per token
    and layer, as generation issues them."""
    for j in range(x.shape[0]):
        src = x[j:j + 1]
        for l, (g, u, d) in enumerate(packed):
            aa.aa_swiglu_ffn_fwd(up, down, src, g, u, d, H[j:j + 1], Ys[l][j:j + 1], None, pos0 + j)
            src = Ys[l][j:j + 1]


def test_stack_matches_oracle_chain(stack):
    """Three tokens across the context wrap (positions 1534, 1535, 1536: types
    2, 3, 0) through the 12 layers.  The oracle chain rounds H and every
    layer's output to bf16 where the library stores them in bf16."""
    up, down, raw, packed = stack
    n, pos0 = 3, PERIOD - 2
    say("ffn stack", LAYERS, D, F, n, pos0)
    x = inp.gaussian((n, D), 311, 1.0, torch.bfloat16, DEV)
    H = torch.empty(n, F, dtype=torch.bfloat16, device=DEV)
    Ys = [torch.empty(n, D, dtype=torch.bfloat16, device=DEV) for _ in range(LAYERS)]
    _run_tokens(up, down, packed, x, H, Ys, pos0)
    torch.cuda.synchronize()
    types = oracle.types_pos_mod(n, Q, pos0, PERIOD)
    assert list(types) == [2, 3, 0]
    h = host(x)
    for l, (g, u, d) in enumerate(raw):
        G = oracle.project(h, host(g), "Q2xQ2", Q, types)
        U = oracle.project(h, host(u), "Q2xQ2", Q, types)
        Hl = _bf16(oracle.silu(G) * U)
        Yl = oracle.project(Hl, host(d), "Q2xQ2", Q, types)
        assert_parity(host(Ys[l]), Yl, True, f"layer {l}")
        h = _bf16(Yl)


def test_stack_graph_replays_match_eager(stack):
    """q consecutive tokens through the 12 layers captured in one HIP graph
    (96 launches): every replay, with eager work and synchronisations between
    replays, equals the eager calls bit for bit."""
    up, down, raw, packed = stack
    say("ffn stack graph", LAYERS, Q)
    x = inp.gaussian((Q, D), 312, 1.0, torch.bfloat16, DEV)
    H = torch.empty(Q, F, dtype=torch.bfloat16, device=DEV)
    Ye = [torch.empty(Q, D, dtype=torch.bfloat16, device=DEV) for _ in range(LAYERS)]
    Yg = [torch.empty(Q, D, dtype=torch.bfloat16, device=DEV) for _ in range(LAYERS)]
    _run_tokens(up, down, packed, x, H, Ye, 0)
    torch.cuda.synchronize()
    _run_tokens(up, down, packed, x, H, Yg, 0)   # warm the graph's calls once
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run_tokens(up, down, packed, x, H, Yg, 0)
    other = torch.empty(64, D, dtype=torch.bfloat16, device=DEV)
    for r in range(3):
        for y in Yg:
            y.fill_(float("nan"))
        g.replay()
        aa.aa_project_fwd(down, inp.gaussian((64, F), 320 + r, 1.0, torch.bfloat16, DEV), packed[0][2], other)
        torch.cuda.synchronize()
        for l in range(LAYERS):
            assert torch.equal(Yg[l], Ye[l]), (r, l)
