"""Parity of the gradient kernels (aa_project_bwd_data, aa_project_bwd_weight)
with the fp64 oracle, through the C ABI.  Every test needs an MI355X.

dW is produced in the packed layout; it is unpacked on the GPU with
aa_unpack_weights (a bit-exact permutation, checked elsewhere) before it is
compared with the oracle's row-major dW.
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


def _types(kind, M, q, pos_offset, period):
    if kind == "block_rows":
        return oracle.types_block_rows(M, q)
    return oracle.types_pos_mod(M, q, pos_offset, period)


def _unpack(plan, dWp):
    """Row-major copy of a packed gradient of the plan's output dtype."""
    up = aa.aa_plan_create(plan.law, plan.q, plan.d_in, plan.d_out, "pos_mod", 0, plan.out_dtype, plan.out_dtype)
    out = torch.empty(plan.d_in, plan.d_out, dtype=plan.out_torch_dtype, device=DEV)
    aa.aa_unpack_weights(up, dWp, out)
    return out


def _run(law, q, M, d_in, d_out, out_dt="f32", kind="pos_mod", pos_offset=0, period=0, seed=0, ints=False):
    plan = aa.aa_plan_create(law, q, d_in, d_out, kind, period, "bf16", out_dt)
    if ints:
        X = inp.small_integers((M, d_in), seed + 1, dtype=torch.bfloat16, device=DEV)
        W = inp.small_integers((d_in, d_out), seed + 2, dtype=torch.bfloat16, device=DEV)
        dY = inp.small_integers((M, d_out), seed + 3, dtype=torch.bfloat16, device=DEV)
    else:
        X = inp.gaussian((M, d_in), seed + 1, 1.0, torch.bfloat16, DEV)
        W = inp.gaussian((d_in, d_out), seed + 2, d_in ** -0.5, torch.bfloat16, DEV)
        dY = inp.gaussian((M, d_out), seed + 3, 1.0, torch.bfloat16, DEV)
    Wp = aa.pack(plan, W)
    dX = torch.full((M, d_in), float("nan"), dtype=TD[out_dt], device=DEV)
    dWp = torch.full((d_in * d_out,), float("nan"), dtype=TD[out_dt], device=DEV)
    nd, nw = aa.aa_project_bwd_workspace(plan, M)
    wsd = torch.empty(max(nd, 1), dtype=torch.uint8, device=DEV)
    wsw = torch.empty(max(nw, 1), dtype=torch.uint8, device=DEV)
    aa.aa_project_bwd_data(plan, dY, Wp, dX, None, pos_offset, None, wsd if nd else None, nd)
    aa.aa_project_bwd_weight(plan, X, dY, dWp, None, pos_offset, None, wsw if nw else None, nw)
    torch.cuda.synchronize()
    dW = _unpack(plan, dWp)
    torch.cuda.synchronize()
    types = _types(kind, M, q, pos_offset, period)
    return (host(dX), host(dW), oracle.project_grad_input(host(dY), host(W), law, q, types),
            oracle.project_grad_weight(host(X), host(dY), law, q, types))


@pytest.mark.parametrize("name,law,q,M,d_in,d_out,kind,pos_offset,period", [
    ("small ragged", "Qq", 8, 999, 512, 1024, "pos_mod", 3, 0),
    ("odd strips (b_out 48)", "Qq", 16, 700, 2048, 768, "pos_mod", 5, 0),
    ("narrow input blocks (b_in 48)", "Qq", 16, 600, 768, 2048, "pos_mod", 0, 0),
    ("fewer rows than types", "Qq", 8, 5, 512, 512, "pos_mod", 6, 0),
    ("block rows", "Qq", 4, 512, 256, 512, "block_rows", 0, 0),
    ("q = 2", "Qq", 2, 300, 128, 64, "pos_mod", 1, 0),
    ("Q2xQ2 gate/up shape", "Q2xQ2", 4, 3000, 768, 1536, "pos_mod", 0, 1536),
    ("Q2xQ2 down shape", "Q2xQ2", 4, 1100, 1536, 768, "pos_mod", 2, 1536),
    ("Q2xQ2 block rows", "Q2xQ2", 4, 256, 256, 128, "block_rows", 0, 0),
    ("wide input blocks (b_in 384)", "Qq", 32, 900, 12288, 4096, "pos_mod", 9, 0),
    ("q = 1 (dense gradients)", "Qq", 1, 300, 64, 96, "pos_mod", 0, 0),
    ("one row", "Qq", 8, 1, 512, 512, "pos_mod", 11, 0),
    ("b = 16, q = 256 block rows", "Qq", 256, 2048, 4096, 4096, "block_rows", 0, 0),
    ("q = 3", "Qq", 3, 700, 384, 576, "pos_mod", 1, 0),
    ("Qwen3-30B-A3B expert gate", "Qq", 16, 2048, 2048, 768, "pos_mod", 0, 0),
])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_gradients_match_oracle(name, law, q, M, d_in, d_out, kind, pos_offset, period, out_dt):
    say("bwd", name, law, q, M, d_in, d_out, kind, pos_offset, period, out_dt)
    dX, dW, dX_ref, dW_ref = _run(law, q, M, d_in, d_out, out_dt, kind, pos_offset, period, seed=17 * q + M % 31)
    assert_parity(dX, dX_ref, out_dt == "bf16", f"{name} dX")
    assert_parity(dW, dW_ref, out_dt == "bf16", f"{name} dW")


@pytest.mark.parametrize("law,q,M,d_in,d_out,kind", [
    ("Qq", 4, 300, 256, 192, "pos_mod"),
    ("Qq", 8, 130, 1024, 384, "pos_mod"),
    ("Q2xQ2", 4, 200, 768, 256, "pos_mod"),
    ("Qq", 4, 128, 512, 256, "block_rows"),
])
def test_gradients_integer_exact(law, q, M, d_in, d_out, kind):
    """Small integers, exact in bf16 and in fp32 sums: bit for bit."""
    say("bwd int", law, q, M, d_in, d_out, kind)
    dX, dW, dX_ref, dW_ref = _run(law, q, M, d_in, d_out, "f32", kind, 7 if kind == "pos_mod" else 0, 0, seed=5,
                                  ints=True)
    assert np.array_equal(dX, dX_ref), np.max(np.abs(dX - dX_ref))
    assert np.array_equal(dW, dW_ref), np.max(np.abs(dW - dW_ref))


@pytest.mark.parametrize("path", ["630", "631"])
@pytest.mark.parametrize("q,M,d_in,d_out,kind", [
    (4, 300, 256, 192, "pos_mod"),
    (8, 130, 1024, 384, "pos_mod"),
    (4, 128, 512, 256, "block_rows"),
    (32, 700, 2048, 4096, "pos_mod"),
    (8, 5, 512, 512, "pos_mod"),
])
def test_weight_gradient_walk_and_parts_integer_exact(path, q, M, d_in, d_out, kind, monkeypatch):
    """Q_q dW takes one of two kernels: the walk over the row types (one
    workgroup per 64 x 64 tile of a group, no partial sums) or the parts of
    the diagonal blocks' rows with a reduction.  AA_TILE=630 / 631 force each
    on every shape; small integers make both exact, bit for bit."""
    monkeypatch.setenv("AA_TILE", path)
    say("bwd dW path", path, q, M, d_in, d_out, kind)
    _, dW, _, dW_ref = _run("Qq", q, M, d_in, d_out, "f32", kind, 7 if kind == "pos_mod" else 0, 0, seed=9,
                            ints=True)
    assert np.array_equal(dW, dW_ref), np.max(np.abs(dW - dW_ref))


@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
def test_grad_input_widest_blocks(out_dt):
    """dX at the widest input blocks it takes (b_in = 512; dW stops at 384)."""
    q, M, d_in, d_out = 8, 1000, 4096, 1024
    say("bwd dX b_in 512", q, M, d_in, d_out, out_dt)
    plan = aa.aa_plan_create("Qq", q, d_in, d_out, "pos_mod", 0, "bf16", out_dt)
    W = inp.gaussian((d_in, d_out), 402, d_in ** -0.5, torch.bfloat16, DEV)
    dY = inp.gaussian((M, d_out), 403, 1.0, torch.bfloat16, DEV)
    Wp = aa.pack(plan, W)
    dX = torch.full((M, d_in), float("nan"), dtype=TD[out_dt], device=DEV)
    nd, _ = aa.aa_project_bwd_workspace(plan, M)
    wsd = torch.empty(max(nd, 1), dtype=torch.uint8, device=DEV)
    aa.aa_project_bwd_data(plan, dY, Wp, dX, None, 5, None, wsd if nd else None, nd)
    torch.cuda.synchronize()
    ref = oracle.project_grad_input(host(dY), host(W), "Qq", q, oracle.types_pos_mod(M, q, 5))
    assert_parity(host(dX), ref, out_dt == "bf16", "dX b_in 512")


def test_gradients_qwen3_8b_shape():
    """M = 2048, 4096 -> 12288, Q_32, bf16 outputs: the benchmark's launch configuration."""
    say("bwd qwen3-8b")
    dX, dW, dX_ref, dW_ref = _run("Qq", 32, 2048, 4096, 12288, "bf16", seed=inp.seed_for(inp.ROLE_X, 3))
    assert_parity(dX, dX_ref, True, "qwen3 dX")
    assert_parity(dW, dW_ref, True, "qwen3 dW")


def test_gradient_adjoint_identity_on_gpu():
    """<X * W, dY> = <X, dX> = <W, dW> with the forward, dX and dW all from the GPU."""
    q, M, d_in, d_out = 16, 1024, 2048, 768
    say("bwd adjoint", q, M, d_in, d_out)
    plan = aa.aa_plan_create("Qq", q, d_in, d_out, "pos_mod", 0, "bf16", "f32")
    X = inp.gaussian((M, d_in), 301, 1.0, torch.bfloat16, DEV)
    W = inp.gaussian((d_in, d_out), 302, d_in ** -0.5, torch.bfloat16, DEV)
    dY = inp.gaussian((M, d_out), 303, 1.0, torch.bfloat16, DEV)
    Wp = aa.pack(plan, W)
    Y = torch.empty(M, d_out, dtype=torch.float32, device=DEV)
    aa.aa_project_fwd(plan, X, Wp, Y)
    dX = torch.empty(M, d_in, dtype=torch.float32, device=DEV)
    nd, nw = aa.aa_project_bwd_workspace(plan, M)
    wsd = torch.empty(max(nd, 1), dtype=torch.uint8, device=DEV)
    wsw = torch.empty(max(nw, 1), dtype=torch.uint8, device=DEV)
    aa.aa_project_bwd_data(plan, dY, Wp, dX, None, 0, None, wsd, nd)
    dWp = torch.empty(d_in * d_out, dtype=torch.float32, device=DEV)
    aa.aa_project_bwd_weight(plan, X, dY, dWp, None, 0, None, wsw, nw)
    dW = _unpack(plan, dWp)
    torch.cuda.synchronize()
    v = float((Y.double() * dY.double()).sum())
    a = float((X.double() * dX.double()).sum())
    b = float((W.double() * dW.double()).sum())
    scale = float(torch.linalg.norm(Y.double()) * torch.linalg.norm(dY.double()))
    assert abs(a - v) <= 1e-4 * scale and abs(b - v) <= 1e-4 * scale, (v, a, b, scale)
