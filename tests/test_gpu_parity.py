"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every test here needs an MI355X.  Inputs are seeded (aa_inputs); the oracle
gets exact host copies of the same bf16/fp32 values the GPU reads.  Each case
prints its name and shape before its first GPU call.
"""
import os

import numpy as np
import pytest
import torch

import aa_inputs as inp
import associative_algebra_block_amd as aa
import oracle
from tests._gpu_util import MAX_RMS, REL_FRO, LazyRows, assert_parity, bf16_floor, host, metrics, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available()
    aa.load()   # fails loudly when libaa.so is missing
    say("device", torch.cuda.get_device_name(0))


def _types(kind, M, q, pos_offset=0, period=0):
    if kind == "block_rows":
        return oracle.types_block_rows(M, q)
    return oracle.types_pos_mod(M, q, pos_offset, period)


def _make(law, q, M, d_in, d_out, in_dt="bf16", out_dt="f32", kind="pos_mod", period=0, seed=0, int_exact=False):
    plan = aa.aa_plan_create(law, q, d_in, d_out, kind, period, in_dt, out_dt)
    if int_exact:
        X = inp.small_integers((M, d_in), seed + 1, dtype=TD[in_dt], device=DEV)
        W = inp.small_integers((d_in, d_out), seed + 2, dtype=TD[in_dt], device=DEV)
        # a distinct power-of-two scale per weight block, so a block read from
        # the wrong place changes the result
        bi, bo = d_in // q, d_out // q
        scale = torch.empty(q, q, device=DEV)
        for j in range(q):
            for k in range(q):
                scale[j, k] = 2.0 ** ((5 * j + 3 * k) % 7)
        W = (W.float().view(q, bi, q, bo) * scale.view(q, 1, q, 1)).view(d_in, d_out).to(TD[in_dt])
    else:
        X = inp.gaussian((M, d_in), seed + 1, 1.0, TD[in_dt], DEV)
        W = inp.gaussian((d_in, d_out), seed + 2, d_in ** -0.5, TD[in_dt], DEV)
    return plan, X, W


def _run_project(plan, X, W, pos_offset=0, row_types=None):
    Wp = aa.pack(plan, W)
    Y = torch.empty(X.shape[0], plan.d_out, dtype=plan.out_torch_dtype, device=DEV)
    aa.aa_project_fwd(plan, X, Wp, Y, None, pos_offset, row_types)
    torch.cuda.synchronize()
    return Y


# ------------------------------------------------------------- packing ---

@pytest.mark.parametrize("law,q,d_in,d_out,dt", [
    ("Qq", 2, 64, 64, "f32"), ("Qq", 32, 4096, 12288, "bf16"), ("Qq", 16, 768, 2048, "bf16"),
    ("Qq", 16, 2048, 768, "bf16"), ("Q2xQ2", 4, 768, 1536, "bf16"), ("Qq", 3, 96, 144, "f32")])
def test_pack_roundtrip_and_layout(law, q, d_in, d_out, dt):
    say("pack", law, q, d_in, d_out, dt)
    plan = aa.aa_plan_create(law, q, d_in, d_out, "pos_mod", 0, dt, dt)
    W = inp.gaussian((d_in, d_out), 77, 1.0, TD[dt], DEV)
    P = aa.pack(plan, W)
    back = torch.empty_like(W)
    aa.aa_unpack_weights(plan, P, back)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16 if dt == "bf16" else torch.int32),
                       W.view(torch.int16 if dt == "bf16" else torch.int32))
    # the documented layout, element by element, on a sample of runs
    bi, bo = d_in // q, d_out // q
    Wh, Ph = W.float().cpu().numpy(), P.float().cpu().numpy()
    rng = np.random.default_rng(0)
    runs = rng.integers(0, d_in * d_out // 8, 4000)
    for c in runs:
        blk, w = divmod(int(c), bi * bo // 8)
        j, k = divmod(blk, q)
        nt, rr = divmod(w, 2 * bi)
        kf, ln = divmod(rr, 64)
        row = j * bi + kf * 32 + (ln // 16) * 8
        col = k * bo + nt * 16 + ln % 16
        assert np.array_equal(Ph[c * 8:(c + 1) * 8], Wh[row:row + 8, col]), (c, j, k, nt, kf, ln)


# ------------------------------------------------- integer-exact routing ---

@pytest.mark.parametrize("law,q,M,d_in,d_out,kind,in_dt", [
    ("Qq", 32, 96, 4096, 12288, "pos_mod", "bf16"),     # q = 32 blocks 128 x 384, 3 rows per type
    ("Qq", 16, 272, 2048, 768, "pos_mod", "bf16"),      # narrow 128 x 48 blocks, ragged
    ("Qq", 16, 272, 768, 2048, "pos_mod", "bf16"),      # 48 x 128 blocks (odd multiple of 16)
    ("Q2xQ2", 4, 520, 768, 1536, "pos_mod", "bf16"),
    ("Q2xQ2", 4, 2100, 768, 1536, "pos_mod", "bf16"),  # 525 rows per type: large tiles, ragged
    ("Qq", 4, 2048, 512, 448, "block_rows", "bf16"),   # 512 rows per type, ragged output strips
    ("Qq", 8, 1024, 256, 256, "block_rows", "bf16"),
    ("Qq", 2, 256, 64, 64, "pos_mod", "f32"),
    ("Qq", 1, 40, 64, 48, "pos_mod", "bf16"),
    ("Qq", 3, 700, 384, 576, "pos_mod", "bf16"),       # q = 3 (a law the pages plan next)
    ("Qq", 5, 333, 320, 160, "pos_mod", "bf16"),       # q = 5, 64 x 32 blocks
    ("Qq", 16, 1599, 1024, 3072, "pos_mod", "bf16"),   # 64 x 192 blocks on the persistent kernel, ragged m-tiles
])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_integer_exact(law, q, M, d_in, d_out, kind, in_dt, out_dt):
    say("int-exact", law, q, M, d_in, d_out, kind, in_dt, out_dt)
    plan, X, W = _make(law, q, M, d_in, d_out, in_dt, out_dt, kind, seed=11, int_exact=True)
    Y = _run_project(plan, X, W, pos_offset=3 if kind == "pos_mod" else 0)
    ref = oracle.project(host(X), host(W), law, q, _types(kind, M, q, 3 if kind == "pos_mod" else 0))
    assert np.abs(ref).max() < 2 ** 24
    want = torch.from_numpy(ref).float()
    if out_dt == "bf16":
        want = want.to(torch.bfloat16)
    got = Y.cpu()
    assert torch.equal(got.view(torch.int16 if out_dt == "bf16" else torch.int32),
                       want.view(torch.int16 if out_dt == "bf16" else torch.int32))


# ---------------------------------------------- projection parity (float) ---

@pytest.mark.parametrize("law,q,M,d_in,d_out,kind", [
    ("Qq", 8, 1000, 512, 768, "pos_mod"),        # several tiles and a ragged tail
    ("Qq", 4, 1, 256, 128, "pos_mod"),           # a single token
    ("Qq", 32, 2048, 4096, 12288, "pos_mod"),    # the Qwen3-8B-shaped projection, full size
    ("Qq", 32, 2048, 2048, 6144, "pos_mod"),     # the Qwen3-1.7B-shaped projection (64 x 192 blocks)
    ("Q2xQ2", 4, 4100, 768, 1536, "pos_mod"),
    ("Qq", 64, 8192, 8192, 8192, "block_rows"),  # full product, 128 x 128 blocks
    ("Qq", 3, 3000, 768, 2304, "pos_mod"),       # q = 3: 256 x 768 blocks, 1000 rows per type
    ("Qq", 4, 2050, 1024, 4096, "pos_mod"),      # q = 4: 256 x 1024 blocks
])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_project_parity(law, q, M, d_in, d_out, kind, out_dt):
    say("project", law, q, M, d_in, d_out, kind, out_dt)
    plan, X, W = _make(law, q, M, d_in, d_out, "bf16", out_dt, kind, seed=21)
    Y = _run_project(plan, X, W, pos_offset=5 if kind == "pos_mod" else 0)
    ref = oracle.project(host(X), host(W), law, q, _types(kind, M, q, 5 if kind == "pos_mod" else 0))
    assert_parity(host(Y), ref, out_dt == "bf16", f"project {law} q={q} M={M}")


def test_every_tile_variant_agrees():
    """The tuning override picks each kernel variant in turn; all must match."""
    law, q, M, d_in, d_out = "Qq", 8, 700, 1024, 1536
    say("variants", law, q, M, d_in, d_out)
    ref = None
    for v in list(range(9)) + [100 + j for j in range(9)] + [200, 201] + [300 + j for j in range(7)] + [400 + j for j in range(5)] + [500]:
        os.environ["AA_TILE"] = str(v)
        try:
            plan, X, W = _make(law, q, M, d_in, d_out, "bf16", "f32", seed=31)
        finally:
            del os.environ["AA_TILE"]
        Y = _run_project(plan, X, W, pos_offset=2)
        if ref is None:
            ref = oracle.project(host(X), host(W), law, q, _types("pos_mod", M, q, 2))
        assert_parity(host(Y), ref, False, f"variant {v}")


@pytest.mark.parametrize("q,M,d_in,d_out,kind", [
    (8, 20, 1024, 1536, "pos_mod"),        # fewer tiles than pipeline stages
    (16, 2048, 2048, 768, "pos_mod"),      # 48-wide output blocks (ragged strips)
    (64, 8192, 8192, 8192, "block_rows"),  # several m-tiles per leaf
    (16, 2048, 2048, 6144, "block_rows"),  # jobs of 11 and 10 workgroups over 2 m-tiles: both tile splits
])
def test_job_kernel_variants(q, M, d_in, d_out, kind):
    """Each pipelined job-kernel variant, bf16 output, against the oracle."""
    say("job variants", q, M, d_in, d_out, kind)
    off = 3 if kind == "pos_mod" else 0
    ref = None
    for v in range(300, 307):
        os.environ["AA_TILE"] = str(v)
        try:
            plan, X, W = _make("Qq", q, M, d_in, d_out, "bf16", "bf16", kind, seed=37)
        finally:
            del os.environ["AA_TILE"]
        Y = _run_project(plan, X, W, pos_offset=off)
        if ref is None:
            ref = oracle.project(host(X), host(W), "Qq", q, _types(kind, M, q, off))
        assert_parity(host(Y), ref, True, f"job variant {v}")


@pytest.mark.parametrize("q,M,d_in,d_out,kind,out_dt", [
    (8, 500, 3072, 1024, "pos_mod", "bf16"),      # 384-wide input groups (six K steps)
    (8, 500, 1536, 1024, "pos_mod", "f32"),       # 192-wide input groups
    (16, 40, 2048, 768, "pos_mod", "bf16"),       # ragged strips, fewer steps than stages
    (32, 8192, 4096, 4096, "block_rows", "bf16"), # several m-tiles per leaf
])
def test_kstream_kernel_variants(q, M, d_in, d_out, kind, out_dt):
    """Each K-stream variant whose K chunk divides the input group, against the oracle."""
    say("kstream variants", q, M, d_in, d_out, kind, out_dt)
    off = 7 if kind == "pos_mod" else 0
    ref = None
    for v in range(400, 407):   # every K-stream variant (override 400 + id)
        os.environ["AA_TILE"] = str(v)
        try:
            plan, X, W = _make("Qq", q, M, d_in, d_out, "bf16", out_dt, kind, seed=41)
        finally:
            del os.environ["AA_TILE"]
        Y = _run_project(plan, X, W, pos_offset=off)
        if ref is None:
            ref = oracle.project(host(X), host(W), "Qq", q, _types(kind, M, q, off))
        assert_parity(host(Y), ref, out_dt == "bf16", f"kstream variant {v}")


def test_kstream_swiglu_matches_oracle():
    """The fused SwiGLU gate/up through the K-stream kernel (384-wide groups)."""
    q, M, D, F = 8, 300, 3072, 1536
    say("kstream swiglu", q, M, D, F)
    os.environ["AA_TILE"] = "402"
    try:
        up = aa.aa_plan_create("Qq", q, D, F, "pos_mod", 0, "bf16", "bf16")
    finally:
        del os.environ["AA_TILE"]
    down = aa.aa_plan_create("Qq", q, F, D, "pos_mod", 0, "bf16", "f32")
    X = inp.gaussian((M, D), 51, 1.0, torch.bfloat16, DEV)
    Wg = inp.gaussian((D, F), 52, D ** -0.5, torch.bfloat16, DEV)
    Wu = inp.gaussian((D, F), 53, D ** -0.5, torch.bfloat16, DEV)
    Wd = inp.gaussian((F, D), 54, F ** -0.5, torch.bfloat16, DEV)
    H = torch.empty(M, F, dtype=torch.bfloat16, device=DEV)
    Y = torch.empty(M, D, dtype=torch.float32, device=DEV)
    aa.aa_swiglu_ffn_fwd(up, down, X, aa.pack(up, Wg), aa.pack(up, Wu), aa.pack(down, Wd), H, Y, None, 3)
    torch.cuda.synchronize()
    types = oracle.types_pos_mod(M, q, 3)
    Href, Yref = oracle.swiglu_ffn(host(X), host(Wg), host(Wu), host(Wd), "Qq", q, types)
    assert_parity(host(H), Href, True, "kstream swiglu H")
    # Y is computed from the GPU's bf16 H; compare it with the oracle applied to that H
    assert_parity(host(Y), oracle.project(host(H), host(Wd), "Qq", q, types), False, "kstream swiglu Y")


@pytest.mark.parametrize("kind,q,M,D,F,off", [
    ("pos_mod", 8, 999, 1024, 2048, 5),       # ragged second m-tile, two 128-wide n-tiles
    ("pos_mod", 8, 520, 1024, 3072, 0),       # three n-tiles per leaf (the Qwen3-8B gate/up layout)
    ("block_rows", 4, 4 * 100, 512, 512, 0),  # block-row typing, 100 rows per type
])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_kstream_gateup_128_wide(kind, q, M, D, F, off, out_dt):
    """SwiGLU gate/up of 128-wide input blocks whose output blocks 128 divides
    takes the K-stream kernel with 128-wide tiles and 32-wide K chunks by
    default; its H and the down projection against the oracle."""
    say("kstream gate/up 128-wide", kind, q, M, D, F, off, out_dt)
    up = aa.aa_plan_create("Qq", q, D, F, kind, 0, "bf16", "bf16")
    down = aa.aa_plan_create("Qq", q, F, D, kind, 0, "bf16", out_dt)
    X = inp.gaussian((M, D), 61, 1.0, torch.bfloat16, DEV)
    Wg = inp.gaussian((D, F), 62, D ** -0.5, torch.bfloat16, DEV)
    Wu = inp.gaussian((D, F), 63, D ** -0.5, torch.bfloat16, DEV)
    Wd = inp.gaussian((F, D), 64, F ** -0.5, torch.bfloat16, DEV)
    H = torch.empty(M, F, dtype=torch.bfloat16, device=DEV)
    Y = torch.empty(M, D, dtype=TD[out_dt], device=DEV)
    aa.aa_swiglu_ffn_fwd(up, down, X, aa.pack(up, Wg), aa.pack(up, Wu), aa.pack(down, Wd), H, Y, None, off)
    torch.cuda.synchronize()
    types = _types(kind, M, q, off)
    Href, _ = oracle.swiglu_ffn(host(X), host(Wg), host(Wu), host(Wd), "Qq", q, types)
    # H is stored in bf16: the rounding floor is allowed on top of the bound
    assert_parity(host(H), Href, True, "kstream gate/up H")
    # Y from the GPU's own H, against the oracle's down projection of that H
    assert_parity(host(Y), oracle.project(host(H), host(Wd), "Qq", q, types), out_dt == "bf16", "kstream gate/up Y")


def test_decode_single_tokens_in_a_graph_replay():
    """Single-token decode calls captured in one HIP graph: every replay,
    with eager work and synchronisations between replays, equals the eager
    calls bit for bit, and the eager calls match the oracle."""
    q, D, F, n = 8, 1024, 1536, 8
    say("decode graph", q, D, F, n)
    plan = aa.aa_plan_create("Qq", q, D, F, "pos_mod", 0, "bf16", "f32")
    x = inp.gaussian((n, D), 61, 1.0, torch.bfloat16, DEV)
    W = inp.gaussian((D, F), 62, D ** -0.5, torch.bfloat16, DEV)
    Wp = aa.pack(plan, W)
    y_eager = torch.empty(n, F, dtype=torch.float32, device=DEV)
    y_graph = torch.empty(n, F, dtype=torch.float32, device=DEV)
    pos0 = 1000
    for j in range(n):
        aa.aa_decode_gemv(plan, x[j:j + 1], Wp, y_eager[j:j + 1], None, pos0 + j)
    torch.cuda.synchronize()
    ref = oracle.decode(host(x), host(W), "Qq", q, np.arange(pos0, pos0 + n))
    assert_parity(host(y_eager), ref, False, "decode eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in range(n):
            aa.aa_decode_gemv(plan, x[j:j + 1], Wp, y_graph[j:j + 1], None, pos0 + j)
    other = aa.aa_plan_create("Qq", q, D, F, "pos_mod", 0, "bf16", "bf16")
    Y_other = torch.empty(300, F, dtype=torch.bfloat16, device=DEV)
    for r in range(4):
        y_graph.fill_(float("nan"))
        g.replay()
        # eager work between replays
        aa.aa_project_fwd(other, inp.gaussian((300, D), 70 + r, 1.0, torch.bfloat16, DEV), Wp, Y_other)
        torch.cuda.synchronize()
        assert torch.equal(y_graph, y_eager), f"replay {r}"


def test_step_in_a_graph_replay():
    """The Qwen3-8B-shaped step (projection, SwiGLU FFN, a 32-token decode)
    captured in one HIP graph: the persistent, K-stream and decode kernels
    replay with eager work and synchronisations between replays, and every
    replay equals the eager calls bit for bit."""
    q, M, D, F = 32, 2048, 4096, 12288
    say("step graph", q, M, D, F)
    up = aa.aa_plan_create("Qq", q, D, F, "pos_mod", 0, "bf16", "bf16")
    down = aa.aa_plan_create("Qq", q, F, D, "pos_mod", 0, "bf16", "bf16")
    X = inp.gaussian((M, D), 91, 1.0, torch.bfloat16, DEV)
    Wp = aa.pack(up, inp.gaussian((D, F), 92, D ** -0.5, torch.bfloat16, DEV))
    Wg = aa.pack(up, inp.gaussian((D, F), 93, D ** -0.5, torch.bfloat16, DEV))
    Wu = aa.pack(up, inp.gaussian((D, F), 94, D ** -0.5, torch.bfloat16, DEV))
    Wd = aa.pack(down, inp.gaussian((F, D), 95, F ** -0.5, torch.bfloat16, DEV))
    x = X[:32].clone()

    def outs():
        return (torch.empty(M, F, dtype=torch.bfloat16, device=DEV), torch.empty(M, F, dtype=torch.bfloat16, device=DEV),
                torch.empty(M, D, dtype=torch.bfloat16, device=DEV), torch.empty(32, F, dtype=torch.bfloat16, device=DEV))

    def step(o):
        aa.aa_project_fwd(up, X, Wp, o[0])
        aa.aa_swiglu_ffn_fwd(up, down, X, Wg, Wu, Wd, o[1], o[2])
        aa.aa_decode_gemv(up, x, Wp, o[3], None, 4096)

    eager, graph = outs(), outs()
    step(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(graph)
    Y_other = torch.empty(M, F, dtype=torch.bfloat16, device=DEV)
    for r in range(3):
        for t in graph:
            t.fill_(float("nan"))
        g.replay()
        aa.aa_project_fwd(up, inp.gaussian((M, D), 96 + r, 1.0, torch.bfloat16, DEV), Wg, Y_other)
        torch.cuda.synchronize()
        for a, b in zip(eager, graph):
            assert torch.equal(a, b), f"replay {r}"


def test_config1_q2_f32_full_product_and_associativity():
    """Q_2 in fp32: row-typed projection, the full 64 x 64 product, and
    (X * W1) * W2 == X * (W1 * W2) computed on the GPU."""
    wl = inp.WORKLOADS[1]
    say("config1", wl)
    plan = aa.aa_plan_create("Qq", 2, 64, 64, "pos_mod", 0, "f32", "f32")
    full = aa.aa_plan_create("Qq", 2, 64, 64, "block_rows", 0, "f32", "f32")
    X = inp.gaussian((256, 64), inp.seed_for(inp.ROLE_X, 1), 1.0, torch.float32, DEV)
    W1 = inp.gaussian((64, 64), inp.seed_for(inp.ROLE_W, 1), 64 ** -0.5, torch.float32, DEV)
    W2 = inp.gaussian((64, 64), inp.seed_for(inp.ROLE_W2, 1), 64 ** -0.5, torch.float32, DEV)
    Y = _run_project(plan, X, W1)
    assert_parity(host(Y), oracle.project(host(X), host(W1), "Qq", 2, oracle.types_pos_mod(256, 2)), False,
                  "config1 project")
    Xs = X[:64].contiguous()
    XW = _run_project(full, Xs, W1)
    assert_parity(host(XW), oracle.star(host(Xs), host(W1), "Qq", 2), False, "config1 X*W")
    lhs = _run_project(full, XW, W2)
    W12 = _run_project(full, W1, W2)
    rhs = _run_project(full, Xs, W12)
    ref = oracle.star(oracle.star(host(Xs), host(W1), "Qq", 2), host(W2), "Qq", 2)
    assert_parity(host(lhs), ref, False, "config1 (X*W1)*W2")
    assert_parity(host(rhs), ref, False, "config1 X*(W1*W2)")
    # the two GPU sides agree with each other to fp32 rounding
    assert np.max(np.abs(host(lhs) - host(rhs))) <= 1e-4 * np.sqrt(np.mean(ref ** 2))


# ------------------------------------------------------------ properties ---

def test_deterministic_and_pos_shift():
    law, q, M, d_in, d_out = "Qq", 16, 1024, 2048, 2048
    say("determinism", law, q, M)
    plan, X, W = _make(law, q, M, d_in, d_out, "bf16", "bf16", seed=41)
    Wp = aa.pack(plan, W)
    outs = []
    for off in (7, 7, 7 + q, 8):
        Y = torch.empty(M, d_out, dtype=torch.bfloat16, device=DEV)
        aa.aa_project_fwd(plan, X, Wp, Y, None, off)
        outs.append(Y)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])         # bitwise deterministic
    assert torch.equal(outs[0], outs[2])         # a shift by q changes no type
    assert not torch.equal(outs[0], outs[3])     # a shift by 1 changes every type
    ref = oracle.project(host(X), host(W), law, q, oracle.types_pos_mod(M, q, 8))
    assert_parity(host(outs[3]), ref, True, "shift by one")


def test_kernel_events_time_the_dispatch():
    """aa_set_kernel_events: the events are recorded by the kernel's own
    dispatch, so the time is positive and no longer than marker events around
    the call; switching them off leaves later calls untimed; results do not
    change."""
    law, q, M, d_in, d_out = "Qq", 32, 2048, 4096, 12288
    say("kernel events", law, q, M, d_in, d_out)
    plan, X, W = _make(law, q, M, d_in, d_out, "bf16", "bf16", seed=71)
    Wp = aa.pack(plan, W)
    Ys = [torch.empty(M, d_out, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    aa.aa_project_fwd(plan, X, Wp, Ys[0])
    ks, ke, a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(5))
    ks.record()
    ke.record()
    torch.cuda.synchronize()
    a.record()
    aa.aa_set_kernel_events(ks, ke)
    aa.aa_project_fwd(plan, X, Wp, Ys[1])
    aa.aa_set_kernel_events(None, None)
    b.record()
    aa.aa_project_fwd(plan, X, Wp, Ys[2])
    c.record()
    torch.cuda.synchronize()
    tk, tm, tm2 = ks.elapsed_time(ke), a.elapsed_time(b), a.elapsed_time(c)
    say("kernel events ms", tk, tm, tm2)
    assert 0.0 < tk <= tm + 1e-3, (tk, tm)
    assert tk < 0.75 * tm2, (tk, tm2)
    assert torch.equal(Ys[0], Ys[1]) and torch.equal(Ys[0], Ys[2])


def test_period_and_empty():
    law, q, M, d_in, d_out = "Q2xQ2", 4, 3 * 24, 256, 512
    say("period", law, q, M)
    plan = aa.aa_plan_create(law, q, d_in, d_out, "pos_mod", 24, "bf16", "f32")
    _, X, W = _make(law, q, M, d_in, d_out, "bf16", "f32", seed=51)
    Y = _run_project(plan, X, W, pos_offset=4)
    ref = oracle.project(host(X), host(W), law, q, oracle.types_pos_mod(M, q, 4, 24))
    assert_parity(host(Y), ref, False, "period 24")
    E = torch.empty(0, d_in, dtype=torch.bfloat16, device=DEV)
    Yo = torch.empty(0, d_out, dtype=torch.float32, device=DEV)
    aa.aa_project_fwd(plan, E, aa.pack(plan, W), Yo)
    torch.cuda.synchronize()


def test_explicit_types():
    law, q, M, d_in, d_out = "Qq", 8, 333, 512, 256
    say("explicit", law, q, M)
    plan = aa.aa_plan_create(law, q, d_in, d_out, "explicit", 0, "bf16", "f32")
    _, X, W = _make(law, q, M, d_in, d_out, "bf16", "f32", seed=61)
    types = inp.random_types(M, q, 62, DEV)
    Y = _run_project(plan, X, W, row_types=types)
    ref = oracle.project(host(X), host(W), law, q, types.cpu().numpy())
    assert_parity(host(Y), ref, False, "explicit")


def test_row_locality():
    law, q, M, d_in, d_out = "Qq", 4, 64, 256, 256
    say("row locality", law, q, M)
    plan, X, W = _make(law, q, M, d_in, d_out, "bf16", "f32", seed=71)
    Y1 = _run_project(plan, X, W)
    X2 = X.clone()
    X2[::3] = inp.gaussian((X2[::3].shape[0], d_in), 72, 1.0, torch.bfloat16, DEV)
    Y2 = _run_project(plan, X2, W)
    keep = [t for t in range(M) if t % 3]
    assert torch.equal(Y1[keep], Y2[keep])


# ---------------------------------------------------------------- decode ---

@pytest.mark.parametrize("law,q,d_in,d_out,n,dt", [
    ("Qq", 32, 4096, 12288, 32, "bf16"), ("Qq", 32, 4096, 12288, 1, "bf16"),
    ("Q2xQ2", 4, 768, 1536, 7, "bf16"), ("Qq", 16, 768, 2048, 20, "bf16"),
    ("Qq", 32, 12288, 4096, 5, "bf16"), ("Qq", 2, 64, 64, 9, "f32"), ("Qq", 4, 320, 64, 6, "bf16"),
    ("Qq", 8, 1024, 1536, 2, "bf16"), ("Q2xQ2", 4, 768, 1536, 1, "bf16"), ("Qq", 16, 6144, 2048, 2, "bf16"),
    # one token per workgroup: a half-width last slab (b_in = 80), q = 1, 384-wide blocks, Q2 x Q2 tails
    ("Qq", 4, 320, 64, 1, "bf16"), ("Qq", 1, 64, 48, 1, "bf16"), ("Qq", 32, 12288, 4096, 1, "bf16"),
    ("Q2xQ2", 4, 320, 512, 3, "bf16"), ("Q2xQ2", 4, 1536, 768, 2, "f32"),
    # many tokens: from 2q (by position) and 8q (explicit types) on, the leaf kernels
    ("Qq", 8, 1024, 1536, 64, "bf16"), ("Qq", 32, 4096, 12288, 300, "bf16"), ("Q2xQ2", 4, 768, 1536, 40, "bf16"),
    # input blocks wider than the matrix-vector kernels take (b_in = 768): the leaf kernels at any count
    ("Qq", 16, 12288, 4096, 1, "bf16"), ("Qq", 16, 12288, 4096, 3, "f32")])
def test_decode_matches_oracle_and_prefill(law, q, d_in, d_out, n, dt):
    say("decode", law, q, d_in, d_out, n, dt)
    plan, X, W = _make(law, q, max(64, n), d_in, d_out, dt, "f32", seed=81)
    Wp = aa.pack(plan, W)
    pos0 = 1000 + 3
    x = X[:n].contiguous()
    y = torch.empty(n, d_out, dtype=torch.float32, device=DEV)
    aa.aa_decode_gemv(plan, x, Wp, y, None, pos0)
    # prefill of the same rows at the same positions through the leaf kernel
    Yp = torch.empty(n, d_out, dtype=torch.float32, device=DEV)
    aa.aa_project_fwd(plan, x, Wp, Yp, None, pos0)
    torch.cuda.synchronize()
    ref = oracle.decode(host(x), host(W), law, q, pos0 + np.arange(n))
    assert_parity(host(y), ref, False, "decode")
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(host(y) - host(Yp))) <= 1e-4 * rms
    # explicit per-token types (mixed positions)
    types = inp.random_types(n, q, 82, DEV)
    aa.aa_decode_gemv(plan, x, Wp, y, None, 0, types)
    torch.cuda.synchronize()
    assert_parity(host(y), oracle.project(host(x), host(W), law, q, types.cpu().numpy()), False, "decode explicit")


# ---------------------------------------------------------------- SwiGLU ---

def _swiglu_case(law, q, M, D, F, out_dt, seed, pos_offset=0, period=0):
    up = aa.aa_plan_create(law, q, D, F, "pos_mod", period, "bf16", "bf16")
    down = aa.aa_plan_create(law, q, F, D, "pos_mod", period, "bf16", out_dt)
    X = inp.gaussian((M, D), seed + 1, 1.0, torch.bfloat16, DEV)
    Wg = inp.gaussian((D, F), seed + 2, D ** -0.5, torch.bfloat16, DEV)
    Wu = inp.gaussian((D, F), seed + 3, D ** -0.5, torch.bfloat16, DEV)
    Wd = inp.gaussian((F, D), seed + 4, F ** -0.5, torch.bfloat16, DEV)
    H = torch.empty(M, F, dtype=torch.bfloat16, device=DEV)
    Y = torch.empty(M, D, dtype=TD[out_dt], device=DEV)
    aa.aa_swiglu_ffn_fwd(up, down, X, aa.pack(up, Wg), aa.pack(up, Wu), aa.pack(down, Wd), H, Y, None, pos_offset)
    torch.cuda.synchronize()
    types = oracle.types_pos_mod(M, q, pos_offset, period)
    Href, Yref = oracle.swiglu_ffn(host(X), host(Wg), host(Wu), host(Wd), law, q, types)
    return H, Y, Href, Yref


@pytest.mark.parametrize("name,law,q,M,D,F,period", [
    ("small ragged", "Qq", 8, 999, 512, 1024, 0),
    ("pilot Q2xQ2 FFN (full)", "Q2xQ2", 4, 8 * 1536, 768, 1536, 1536),
    ("Qwen3-8B SwiGLU (full)", "Qq", 32, 2048, 4096, 12288, 0),
    ("Qwen3-30B-A3B expert (full)", "Qq", 16, 2048, 2048, 768, 0),
])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_swiglu_parity(name, law, q, M, D, F, period, out_dt):
    say("swiglu", name, law, q, M, D, F, out_dt)
    H, Y, Href, Yref = _swiglu_case(law, q, M, D, F, out_dt, 1000 * q + M % 97, 0, period)
    assert_parity(host(H), Href, True, f"{name} H")
    assert_parity(host(Y), Yref, out_dt == "bf16", f"{name} Y")


@pytest.mark.parametrize("name,law,q,M,D,F,period,pos_offset,out_dt", [
    ("Qwen3-8B one token", "Qq", 32, 1, 4096, 12288, 0, 4101, "bf16"),
    ("Qwen3-8B two tokens across the wrap", "Qq", 32, 2, 4096, 12288, 0, 31, "f32"),
    ("Qwen3-8B one token per type", "Qq", 32, 32, 4096, 12288, 0, 7, "bf16"),
    ("pilot Q2xQ2 one token", "Q2xQ2", 4, 1, 768, 1536, 1536, 1535, "f32"),
    ("pilot Q2xQ2 three tokens", "Q2xQ2", 4, 3, 768, 1536, 1536, 2, "bf16"),
    ("Qwen3-30B-A3B expert, five tokens", "Qq", 16, 5, 2048, 768, 0, 13, "bf16"),
    # the Qwen3-8B widths at q = 16: gate/up blocks 256 wide (matrix-vector),
    # down blocks 768 wide (leaf kernels)
    ("Qwen3-8B widths at q = 16, one token", "Qq", 16, 1, 4096, 12288, 0, 9, "bf16"),
    ("Qwen3-8B widths at q = 16, one token per type", "Qq", 16, 16, 4096, 12288, 0, 3, "f32"),
])
def test_swiglu_few_tokens_matches_oracle(name, law, q, M, D, F, period, pos_offset, out_dt):
    """At most q tokens: the FFN runs as a fused gate/up matrix-vector kernel
    (silu(x Wg) * (x Wu) per token) followed by the down matrix-vector kernel."""
    say("swiglu decode", name, law, q, M, D, F, pos_offset, out_dt)
    H, Y, Href, Yref = _swiglu_case(law, q, M, D, F, out_dt, 2000 + 7 * M + q, pos_offset, period)
    assert_parity(host(H), Href, True, f"{name} H")
    assert_parity(host(Y), Yref, out_dt == "bf16", f"{name} Y")


def test_swiglu_few_tokens_explicit_types():
    """Explicit per-token types, some outside [0, q): those rows of H and Y
    are left as they were; the others match the oracle."""
    q, M, D, F = 8, 7, 1024, 1536
    say("swiglu decode explicit", q, M, D, F)
    up = aa.aa_plan_create("Qq", q, D, F, "explicit", 0, "bf16", "bf16")
    down = aa.aa_plan_create("Qq", q, F, D, "explicit", 0, "bf16", "f32")
    X = inp.gaussian((M, D), 91, 1.0, torch.bfloat16, DEV)
    Wg = inp.gaussian((D, F), 92, D ** -0.5, torch.bfloat16, DEV)
    Wu = inp.gaussian((D, F), 93, D ** -0.5, torch.bfloat16, DEV)
    Wd = inp.gaussian((F, D), 94, F ** -0.5, torch.bfloat16, DEV)
    types = torch.tensor([5, -1, 0, 7, q, 3, 5], dtype=torch.int32, device=DEV)
    H = torch.full((M, F), 3.0, dtype=torch.bfloat16, device=DEV)
    Y = torch.full((M, D), 3.0, dtype=torch.float32, device=DEV)
    aa.aa_swiglu_ffn_fwd(up, down, X, aa.pack(up, Wg), aa.pack(up, Wu), aa.pack(down, Wd), H, Y, None, 0, types)
    torch.cuda.synchronize()
    t = types.cpu().numpy()
    live = (t >= 0) & (t < q)
    Href, Yref = oracle.swiglu_ffn(host(X)[live], host(Wg), host(Wu), host(Wd), "Qq", q, t[live])
    assert_parity(host(H)[live], Href, True, "explicit H")
    assert_parity(host(Y)[live], Yref, False, "explicit Y")
    assert np.all(host(H)[~live] == 3.0) and np.all(host(Y)[~live] == 3.0)


def test_swiglu_single_token_in_a_graph_replay():
    """One-token FFN calls captured in a HIP graph replay bit for bit like the
    eager calls, with eager work between replays."""
    q, D, F, n = 32, 4096, 12288, 4
    say("swiglu decode graph", q, D, F, n)
    up = aa.aa_plan_create("Qq", q, D, F, "pos_mod", 0, "bf16", "bf16")
    down = aa.aa_plan_create("Qq", q, F, D, "pos_mod", 0, "bf16", "bf16")
    X = inp.gaussian((n, D), 95, 1.0, torch.bfloat16, DEV)
    Wg, Wu = (aa.pack(up, inp.gaussian((D, F), s, D ** -0.5, torch.bfloat16, DEV)) for s in (96, 97))
    Wd = aa.pack(down, inp.gaussian((F, D), 98, F ** -0.5, torch.bfloat16, DEV))
    He, Ye = torch.empty(n, F, dtype=torch.bfloat16, device=DEV), torch.empty(n, D, dtype=torch.bfloat16, device=DEV)
    Hg, Yg = torch.empty_like(He), torch.empty_like(Ye)
    pos0 = 77
    for j in range(n):
        aa.aa_swiglu_ffn_fwd(up, down, X[j:j + 1], Wg, Wu, Wd, He[j:j + 1], Ye[j:j + 1], None, pos0 + j)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in range(n):
            aa.aa_swiglu_ffn_fwd(up, down, X[j:j + 1], Wg, Wu, Wd, Hg[j:j + 1], Yg[j:j + 1], None, pos0 + j)
    for r in range(3):
        Yg.fill_(float("nan"))
        Hg.fill_(float("nan"))
        g.replay()
        aa.aa_swiglu_ffn_fwd(up, down, X, Wg, Wu, Wd, He.clone(), Ye.clone(), None, 5)   # eager work
        torch.cuda.synchronize()
        assert torch.equal(Hg, He) and torch.equal(Yg, Ye), f"replay {r}"


# ------------------------------------------------- full square product ---

def test_square_product_full_size():
    """n = 32768, b = 128, q = 256: the whole X * W on the GPU in the
    benchmark's launch configuration, with fp32 and with bf16 output.

    fp32 output, at the plain bounds: three whole block-rows (first, middle,
    last) and four seeded rows of every other block-row against the oracle,
    which reads only the weight blocks the row's type names.  bf16 output: the
    same rows against the oracle (bf16 output floor), and, over all 2^30
    outputs, equality with the fp32 result rounded to bf16 (both outputs come
    from the same summation; only the final conversion differs)."""
    n, q = 32768, 256
    b = n // q
    say("square", n, q)
    planf = aa.aa_plan_create("Qq", q, n, n, "block_rows", 0, "bf16", "f32")
    planb = aa.aa_plan_create("Qq", q, n, n, "block_rows", 0, "bf16", "bf16")
    X = inp.gaussian((n, n), inp.seed_for(inp.ROLE_X, 5), 1.0, torch.bfloat16, DEV)
    W = inp.gaussian((n, n), inp.seed_for(inp.ROLE_W, 5), n ** -0.5, torch.bfloat16, DEV)
    Wp = aa.pack(planf, W)
    Yf = torch.empty(n, n, dtype=torch.float32, device=DEV)
    aa.aa_project_fwd(planf, X, Wp, Yf)
    Yb = torch.empty(n, n, dtype=torch.bfloat16, device=DEV)
    aa.aa_project_fwd(planb, X, Wp, Yb)
    torch.cuda.synchronize()
    del Wp
    mism = 0
    for r0 in range(0, n, 4096):
        mism += int((Yf[r0:r0 + 4096].to(torch.bfloat16).view(torch.int16) !=
                     Yb[r0:r0 + 4096].view(torch.int16)).sum())
    say(f"square: bf16 outputs differing from bf16(fp32 outputs): {mism}")
    assert mism == 0
    Wl = LazyRows(W.cpu())
    rng = np.random.default_rng(5)
    worst_f = worst_b = 0.0
    for i in range(q):
        if i in (0, 137, 255):
            rows = np.arange(i * b, (i + 1) * b)
        else:
            rows = i * b + np.sort(rng.choice(b, 4, replace=False))
        idx = torch.from_numpy(rows).to(DEV)
        ref = oracle.project_block_row(host(X[idx]), Wl, "Qq", q, i)
        got_f, got_b = host(Yf[idx]), host(Yb[idx])
        if rows.size == b:
            assert_parity(got_f, ref, False, f"square block-row {i} (whole, fp32)")
            assert_parity(got_b, ref, True, f"square block-row {i} (whole, bf16)")
        rel_f, max_f = metrics(got_f, ref)
        rel_b, max_b = metrics(got_b, ref)
        floor = bf16_floor(ref)
        assert rel_f <= REL_FRO and max_f <= MAX_RMS, (i, rel_f, max_f)
        assert rel_b <= REL_FRO and max_b <= MAX_RMS + floor, (i, rel_b, max_b, floor)
        worst_f, worst_b = max(worst_f, max_f), max(worst_b, max_b)
    say(f"square: 256 block-rows checked; worst max/rms fp32 {worst_f:.3e}, bf16 {worst_b:.3e}")
