"""Plans whose weight blocks are not multiples of the 16-wide MFMA fragment:
packed layout 2 and the small-block kernel, through the C ABI, against the
fp64 oracle.  The Qwen3-32B row of the review's projection table (M = 32768,
5120 -> 25600, q = 256) has 20 x 100 blocks.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

import aa_inputs as inp
import associative_algebra_block_amd as aa
import oracle
from tests._gpu_util import MAX_RMS, REL_FRO, assert_parity, bf16_floor, host, metrics, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available()
    aa.load()


def _layout2(W, q):
    """The packed layout-2 order of a row-major weight, stated on the host:
    blocks in row-major block order; inside a block, runs of 4 rows of one
    column, 16 columns at a time (kq-major, then column), the last fragment
    narrower."""
    d_in, d_out = W.shape
    bi, bo = d_in // q, d_out // q
    nfull, w = bo // 16, bo % 16
    out = []
    for j in range(q):
        for k in range(q):
            B = W[j * bi:(j + 1) * bi, k * bo:(k + 1) * bo]
            for f in range(nfull):
                for kq in range(bi // 4):
                    for n in range(16):
                        out.append(B[4 * kq:4 * kq + 4, 16 * f + n])
            for kq in range(bi // 4):
                for n in range(w):
                    out.append(B[4 * kq:4 * kq + 4, 16 * nfull + n])
    return np.concatenate(out)


@pytest.mark.parametrize("q,d_in,d_out", [(3, 36, 60), (8, 160, 800), (2, 128, 248), (5, 20, 20)])
def test_pack_layout2_roundtrip_and_order(q, d_in, d_out):
    say("pack layout 2", q, d_in, d_out)
    plan = aa.aa_plan_create("Qq", q, d_in, d_out, "pos_mod", 0, "bf16", "bf16")
    assert aa.aa_packed_layout_version(plan) == 2
    W = inp.gaussian((d_in, d_out), 91, 1.0, torch.bfloat16, DEV)
    P = aa.pack(plan, W)
    back = torch.empty_like(W)
    aa.aa_unpack_weights(plan, P, back)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), W.view(torch.int16))
    want = _layout2(W.view(torch.int16).cpu().numpy(), q)
    assert np.array_equal(P.view(torch.int16).cpu().numpy(), want)


def _int_case(law, q, M, d_in, d_out, kind, out_dt, seed, edges=None):
    if edges is None:
        plan = aa.aa_plan_create(law, q, d_in, d_out, kind, 0, "bf16", out_dt)
    else:
        plan = aa.aa_plan_create_digraph(q, edges, d_in, d_out, kind, 0, "bf16", out_dt)
    X = inp.small_integers((M, d_in), seed + 1, dtype=torch.bfloat16, device=DEV)
    W = inp.small_integers((d_in, d_out), seed + 2, dtype=torch.bfloat16, device=DEV)
    bi, bo = d_in // q, d_out // q
    scale = torch.tensor([[2.0 ** ((5 * j + 3 * k) % 7) for k in range(q)] for j in range(q)], device=DEV)
    W = (W.float().view(q, bi, q, bo) * scale.view(q, 1, q, 1)).view(d_in, d_out).to(torch.bfloat16)
    return plan, X, W


@pytest.mark.parametrize("q,M,d_in,d_out,kind,pos", [
    (3, 301, 36, 60, "pos_mod", 2),        # 12 x 20 blocks, ragged rows
    (8, 1000, 160, 800, "pos_mod", 5),     # 20 x 100 blocks (the Qwen3-32B block shape)
    (5, 77, 20, 20, "pos_mod", 0),         # 4 x 4 blocks
    (4, 256, 96, 144, "block_rows", 0),    # 24 x 36 blocks, block-row typing
    (1, 33, 20, 12, "pos_mod", 0),         # q = 1: a plain product
    (4, 300, 512, 80, "pos_mod", 1),       # 128 x 20 blocks: 256-wide leaves
    (2, 200, 128, 248, "pos_mod", 1),      # 64 x 124 blocks: fragments over two launch rows
    (4, 150, 128, 384, "pos_mod", 1),      # 32 x 96 blocks: four weight runs a thread in the LDS-staged kernel
])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_layout2_integer_exact(q, M, d_in, d_out, kind, pos, out_dt):
    """Small integers with a distinct power-of-two scale per weight block,
    every sum exact in fp32: the GPU equals the oracle bit for bit."""
    say("layout2 int-exact", q, M, d_in, d_out, kind, pos, out_dt)
    plan, X, W = _int_case("Qq", q, M, d_in, d_out, kind, out_dt, 17 * q + M)
    Y = torch.full((M, d_out), float("nan"), dtype=TD[out_dt], device=DEV)
    aa.aa_project_fwd(plan, X, aa.pack(plan, W), Y, None, pos)
    torch.cuda.synchronize()
    types = oracle.types_block_rows(M, q) if kind == "block_rows" else oracle.types_pos_mod(M, q, pos)
    ref = oracle.project(host(X), host(W), "Qq", q, types)
    assert np.abs(ref).max() < 2 ** 24
    want = torch.from_numpy(ref).float().to(TD[out_dt])
    iv = torch.int16 if out_dt == "bf16" else torch.int32
    assert torch.equal(Y.cpu().view(iv), want.view(iv))


def _three_paths(q, M, d_in, d_out, pos, X, W, out_dt, monkeypatch):
    """Y from each kernel a plain layout-2 call can take: the default, the
    16 x 16 LDS-staged kernel (AA_TILE=611) and the per-wave register kernel
    (AA_TILE=610).  Plans read AA_TILE when they are created."""
    outs = []
    for tile in (None, "611", "610"):
        if tile is None:
            monkeypatch.delenv("AA_TILE", raising=False)
        else:
            monkeypatch.setenv("AA_TILE", tile)
        plan = aa.aa_plan_create("Qq", q, d_in, d_out, "pos_mod", 0, "bf16", out_dt)
        Y = torch.full((M, d_out), float("nan"), dtype=TD[out_dt], device=DEV)
        aa.aa_project_fwd(plan, X, aa.pack(plan, W), Y, None, pos)
        outs.append(Y)
    monkeypatch.delenv("AA_TILE", raising=False)
    torch.cuda.synchronize()
    return outs


SHAPES_3 = [
    (8, 1000, 160, 800, 5),   # 20 x 100 blocks (the Qwen3-32B block shape): 32 x 32 fragments by default
    (3, 301, 36, 252, 2),     # 12 x 84: 32 x 32 fragments, one k-step pair
    (4, 150, 96, 480, 3),     # 24 x 120
    (1, 70, 20, 100, 0),      # q = 1
    (8, 5, 160, 800, 3),      # fewer rows than types: most types empty
    (3, 301, 36, 60, 2),      # 12 x 20: the 16 x 16 LDS kernel by default
    (4, 150, 96, 240, 3),     # 24 x 60
]


@pytest.mark.parametrize("q,M,d_in,d_out,pos", SHAPES_3)
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_layout2_kernels_integer_exact(q, M, d_in, d_out, pos, out_dt, monkeypatch):
    """Small integers (every sum exact in fp32) through all three kernels:
    each equals the oracle bit for bit."""
    say("layout2 three kernels int-exact", q, M, d_in, d_out, pos, out_dt)
    X = inp.small_integers((M, d_in), 61 + q, dtype=torch.bfloat16, device=DEV)
    W = inp.small_integers((d_in, d_out), 62 + q, dtype=torch.bfloat16, device=DEV)
    ref = oracle.project(host(X), host(W), "Qq", q, oracle.types_pos_mod(M, q, pos))
    want = torch.from_numpy(ref).float().to(TD[out_dt])
    iv = torch.int16 if out_dt == "bf16" else torch.int32
    for Y in _three_paths(q, M, d_in, d_out, pos, X, W, out_dt, monkeypatch):
        assert torch.equal(Y.cpu().view(iv), want.view(iv))


@pytest.mark.parametrize("q,M,d_in,d_out,pos", SHAPES_3)
def test_layout2_kernels_float_parity(q, M, d_in, d_out, pos, monkeypatch):
    """Gaussian inputs through all three kernels, fp32 output: each within the
    parity bounds of the oracle; the register and 16 x 16 LDS kernels sum the
    same products in the same order, so those two agree bit for bit."""
    say("layout2 three kernels parity", q, M, d_in, d_out, pos)
    X = inp.gaussian((M, d_in), 41 + q, 1.0, torch.bfloat16, DEV)
    W = inp.gaussian((d_in, d_out), 42 + q, d_in ** -0.5, torch.bfloat16, DEV)
    ref = oracle.project(host(X), host(W), "Qq", q, oracle.types_pos_mod(M, q, pos))
    Yd, Yl, Yr = _three_paths(q, M, d_in, d_out, pos, X, W, "f32", monkeypatch)
    assert torch.equal(Yl.view(torch.int32), Yr.view(torch.int32))
    for name, Y in (("default", Yd), ("lds16", Yl), ("register", Yr)):
        assert_parity(host(Y), ref, False, f"layout2 {name} q={q} {d_in}->{d_out}")


@pytest.mark.parametrize("q,M,d_in,d_out,out_dt", [(8, 560, 160, 800, "bf16"), (8, 560, 160, 800, "f32"),
                                                   (3, 201, 36, 252, "bf16")])
def test_layout2_block_rows_integer_exact(q, M, d_in, d_out, out_dt):
    """Block-row typing on the default kernels (the 32 x 32 fragment kernel
    for bf16 20 x 100 and 12 x 84 blocks; fp32 20 x 100 outputs need more LDS
    and take the 16 x 16 kernel): contiguous rows per type, ragged m-tiles
    (70 and 67 rows per type)."""
    say("layout2 block rows", q, M, d_in, d_out, out_dt)
    plan, X, W = _int_case("Qq", q, M, d_in, d_out, "block_rows", out_dt, 29)
    Y = torch.full((M, d_out), float("nan"), dtype=TD[out_dt], device=DEV)
    aa.aa_project_fwd(plan, X, aa.pack(plan, W), Y, None, 0)
    torch.cuda.synchronize()
    ref = oracle.project(host(X), host(W), "Qq", q, oracle.types_block_rows(M, q))
    want = torch.from_numpy(ref).float().to(TD[out_dt])
    iv = torch.int16 if out_dt == "bf16" else torch.int32
    assert torch.equal(Y.cpu().view(iv), want.view(iv))


@pytest.mark.parametrize("q,M,d_in,d_out", [(6, 250, 48, 168), (4, 300, 64, 400)])
def test_layout2_digraph_integer_exact(q, M, d_in, d_out):
    """Digraph tables with 8 x 28 and 16 x 100 blocks (the second on the 32 x
    32 fragment kernel): non-edge output groups are zero."""
    edges = inp.random_edges(q, 0.4, 23)
    say("layout2 digraph", q, M, d_in, d_out, len(edges))
    plan, X, W = _int_case(None, q, M, d_in, d_out, "pos_mod", "f32", 5, edges)
    assert aa.aa_packed_layout_version(plan) == 2
    Y = torch.full((M, d_out), float("nan"), dtype=torch.float32, device=DEV)
    aa.aa_project_fwd(plan, X, aa.pack(plan, W), Y, None, 4)
    torch.cuda.synchronize()
    ref = oracle.project(host(X), host(W), oracle.Digraph(q, edges), q, oracle.types_pos_mod(M, q, 4))
    assert np.array_equal(host(Y), ref)


@pytest.mark.parametrize("q,M,d_in,d_out", [(8, 999, 160, 800), (4, 2050, 400, 80), (16, 700, 512, 1984)])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_layout2_float_parity(q, M, d_in, d_out, out_dt):
    """Gaussian inputs: 20 x 100 blocks, 100 x 20 (a down projection's
    shape: 200-wide leaves) and 32 x 124 blocks, ragged rows."""
    say("layout2 parity", q, M, d_in, d_out, out_dt)
    plan = aa.aa_plan_create("Qq", q, d_in, d_out, "pos_mod", 0, "bf16", out_dt)
    X = inp.gaussian((M, d_in), 301 + q, 1.0, torch.bfloat16, DEV)
    W = inp.gaussian((d_in, d_out), 302 + q, d_in ** -0.5, torch.bfloat16, DEV)
    Y = torch.empty(M, d_out, dtype=TD[out_dt], device=DEV)
    aa.aa_project_fwd(plan, X, aa.pack(plan, W), Y, None, 7)
    torch.cuda.synchronize()
    ref = oracle.project(host(X), host(W), "Qq", q, oracle.types_pos_mod(M, q, 7))
    assert_parity(host(Y), ref, out_dt == "bf16", f"layout2 q={q} {d_in}->{d_out}")


def test_qwen3_32b_projection_full_size():
    """M = 32768, 5120 -> 25600, q = 256 (20 x 100 blocks), the benchmark's
    launch configuration, fp32 and bf16 output.  fp32 at the plain bounds on
    two rows of every row type and on all rows of three types; bf16 on the same
    rows (output floor); over all 2^29.6 outputs, the bf16 result equals the
    fp32 result rounded to bf16."""
    M, D, F, q = 32768, 5120, 25600, 256
    say("qwen3-32b projection", M, D, F, q)
    planf = aa.aa_plan_create("Qq", q, D, F, "pos_mod", 0, "bf16", "f32")
    planb = aa.aa_plan_create("Qq", q, D, F, "pos_mod", 0, "bf16", "bf16")
    X = inp.gaussian((M, D), inp.seed_for(inp.ROLE_X, 8), 1.0, torch.bfloat16, DEV)
    W = inp.gaussian((D, F), inp.seed_for(inp.ROLE_W, 8), D ** -0.5, torch.bfloat16, DEV)
    Wp = aa.pack(planf, W)
    Yf = torch.empty(M, F, dtype=torch.float32, device=DEV)
    aa.aa_project_fwd(planf, X, Wp, Yf)
    Yb = torch.empty(M, F, dtype=torch.bfloat16, device=DEV)
    aa.aa_project_fwd(planb, X, Wp, Yb)
    torch.cuda.synchronize()
    mism = 0
    for r0 in range(0, M, 4096):
        mism += int((Yf[r0:r0 + 4096].to(torch.bfloat16).view(torch.int16) != Yb[r0:r0 + 4096].view(torch.int16)).sum())
    say(f"qwen3-32b: bf16 outputs differing from bf16(fp32 outputs): {mism}")
    assert mism == 0
    rng = np.random.default_rng(32)
    rows = [i + q * rng.choice(M // q, 2, replace=False) for i in range(q)]
    rows += [np.arange(t, M, q) for t in (0, 101, 255)]
    rows = np.unique(np.concatenate(rows))
    idx = torch.from_numpy(rows).to(DEV)
    ref = oracle.project(host(X[idx]), host(W), "Qq", q, oracle.types_pos_mod(M, q)[rows])
    assert_parity(host(Yf[idx]), ref, False, f"qwen3-32b fp32 ({rows.size} rows, every type)")
    assert_parity(host(Yb[idx]), ref, True, f"qwen3-32b bf16 ({rows.size} rows, every type)")


@pytest.mark.parametrize("M,pos", [(300, 0), (5, 32771), (1, 9)])
def test_qwen3_32b_swiglu(M, pos):
    """SwiGLU FFN at the Qwen3-32B widths (5120 -> 25600 -> 5120, q = 256; gate
    and up 20 x 100 blocks, down 100 x 20): H against the oracle (bf16 floor)
    and Y against the oracle's down projection of the GPU's own H."""
    D, F, q = 5120, 25600, 256
    say("qwen3-32b swiglu", M, pos)
    up = aa.aa_plan_create("Qq", q, D, F, "pos_mod", 0, "bf16", "bf16")
    down = aa.aa_plan_create("Qq", q, F, D, "pos_mod", 0, "bf16", "f32")
    X = inp.gaussian((M, D), 811, 1.0, torch.bfloat16, DEV)
    Wg = inp.gaussian((D, F), 812, D ** -0.5, torch.bfloat16, DEV)
    Wu = inp.gaussian((D, F), 813, D ** -0.5, torch.bfloat16, DEV)
    Wd = inp.gaussian((F, D), 814, F ** -0.5, torch.bfloat16, DEV)
    H = torch.empty(M, F, dtype=torch.bfloat16, device=DEV)
    Y = torch.empty(M, D, dtype=torch.float32, device=DEV)
    aa.aa_swiglu_ffn_fwd(up, down, X, aa.pack(up, Wg), aa.pack(up, Wu), aa.pack(down, Wd), H, Y, None, pos)
    torch.cuda.synchronize()
    types = oracle.types_pos_mod(M, q, pos)
    Href, _ = oracle.swiglu_ffn(host(X), host(Wg), host(Wu), host(Wd), "Qq", q, types)
    assert_parity(host(H), Href, True, "qwen3-32b H")
    assert_parity(host(Y), oracle.project(host(H), host(Wd), "Qq", q, types), False, "qwen3-32b Y")


@pytest.mark.parametrize("n", [1, 5])
def test_qwen3_32b_decode(n):
    """Decode of n new tokens on a layout-2 plan (the projection of the new
    rows) against the oracle's decode."""
    D, F, q = 5120, 25600, 256
    say("qwen3-32b decode", n)
    plan = aa.aa_plan_create("Qq", q, D, F, "pos_mod", 0, "bf16", "f32")
    x = inp.gaussian((n, D), 821, 1.0, torch.bfloat16, DEV)
    W = inp.gaussian((D, F), 822, D ** -0.5, torch.bfloat16, DEV)
    y = torch.empty(n, F, dtype=torch.float32, device=DEV)
    aa.aa_decode_gemv(plan, x, aa.pack(plan, W), y, None, 40000)
    torch.cuda.synchronize()
    assert_parity(host(y), oracle.decode(host(x), host(W), "Qq", q, 40000 + np.arange(n)), False, "decode")
