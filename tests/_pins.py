"""Pins of the oracle against what the pages and the mathematics fix.

Each pin takes an oracle module `orc` and raises AssertionError when it
disagrees.  They are written against facts that do not come from the oracle
itself: worked examples derived by hand from the pages' rule (tests/golden),
counts the pages print, closed forms through a plain library matrix product,
the structure of a tensor-product algebra (numpy.kron), associativity, the
unit, and composition.  test_oracle_pins.py runs them on the real oracle and
on copies of it with planted mistakes, each of which some pin must catch.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-11


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, tol=TOL):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"max abs err {err} > {tol * scale}"


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- golden ---

def pin_golden_q2(orc):
    g = _load("q2_hand_examples.json")
    ex = g["scalar_full_product"]
    _close(orc.star(ex["X"], ex["W"], ex["law"], ex["q"]), ex["star"], 0)
    dense = np.asarray(ex["X"], float) @ np.asarray(ex["W"], float)
    _close(dense, ex["dense"], 0)
    ex = g["rowtyped_rectangular"]
    _close(orc.project(ex["X"], ex["W"], ex["law"], ex["q"], ex["types"]), ex["Y"], 0)
    ex = g["decode_positions"]
    _close(orc.decode(ex["x"], ex["W"], ex["law"], ex["q"], ex["positions"]), ex["y"], 0)


def pin_golden_q2xq2_triples(orc):
    g = _load("q2xq2_triples.json")
    for t in g["triples"]:
        got = orc.in_table("Q2xQ2", 4, t["g"], t["g1"], t["g2"])
        assert got == t["kept"], t
        got4 = orc.in_table("Qq", 4, t["g"], t["g1"], t["g2"])
        assert got4 == t["q4_kept"], t


def pin_counts(orc):
    c = _load("page_counts.json")
    assert orc.count_block_products("Qq", 2) == c["q2_block_products"]
    assert orc.count_block_products("Qq", 2) < c["q2_dense_block_products"]
    for q in c["rank_formula_qs"]:
        assert orc.count_block_products("Qq", q) == 2 * q * q - q, q
        for i in range(min(q, 8)):
            assert Fraction(orc.count_row_block_products("Qq", q, i), q * q) == Fraction(2 * q - 1, q * q)
    assert orc.count_block_products("Q2xQ2", 4) == c["q2xq2_block_products"]
    # 16 coordinates = a 4x4 grid of groups
    assert 4 * 4 == c["q2xq2_coordinates"]
    r = Fraction(*c["q2xq2_ffn_mac_ratio"])
    for i in range(4):
        assert Fraction(orc.count_row_block_products("Q2xQ2", 4, i), 16) == r
    # not isomorphic to Q4: a different number of structure constants
    assert orc.count_block_products("Qq", 4) == 28 != c["q2xq2_block_products"]
    # projection share of one pilot decoder block: four dense d x d attention
    # projections plus three FFN projections at the law's MAC ratio
    d, F = c["pilot_width"], c["pilot_ffn_width"]
    share = (4 * d * d + r * 3 * d * F) / Fraction(4 * d * d + 3 * d * F)
    assert share == Fraction(*c["pilot_block_projection_share"])


# ---------------------------------------------------- library reductions ---

def pin_q1_is_matmul(orc):
    rng = _rng(1)
    A = rng.standard_normal((5, 7))
    B = rng.standard_normal((7, 3))
    _close(orc.star(A, B, "Qq", 1), A @ B)
    _close(orc.project(A, B, "Qq", 1, np.zeros(5, int)), A @ B)


def _off_qq(A, q):
    """Zero the diagonal blocks of a q x q block matrix (rectangular blocks)."""
    A = np.array(A, dtype=np.float64)
    r, c = A.shape[0] // q, A.shape[1] // q
    for i in range(q):
        A[i * r:(i + 1) * r, i * c:(i + 1) * c] = 0
    return A


def pin_closed_form_qq(orc):
    # The edge-times-edge products are exactly off(A) off(B), so the algebra
    # product is the ordinary product minus that.
    rng = _rng(2)
    for q, (ra, ca, cb) in [(2, (3, 2, 4)), (3, (2, 3, 2)), (4, (1, 2, 3)), (5, (2, 1, 1))]:
        A = rng.standard_normal((q * ra, q * ca))
        B = rng.standard_normal((q * ca, q * cb))
        _close(orc.star(A, B, "Qq", q), A @ B - _off_qq(A, q) @ _off_qq(B, q))
        # row-typed: y_t = x_t W - off_tau(x_t) off(W), off_tau zeroing group tau
        M = 11
        X = rng.standard_normal((M, q * ca))
        types = rng.integers(0, q, M)
        ref = X @ B
        offB = _off_qq(B, q)
        for t in range(M):
            xo = X[t].copy()
            xo[types[t] * ca:(types[t] + 1) * ca] = 0
            ref[t] -= xo @ offB
        _close(orc.project(X, B, "Qq", q, types), ref)


def _proj_q2xq2(A, keep):
    """Keep the blocks (g, g') of a 4 x 4 block matrix where keep(a, b, a1, b1)."""
    A = np.array(A, dtype=np.float64)
    r, c = A.shape[0] // 4, A.shape[1] // 4
    out = np.zeros_like(A)
    for g in range(4):
        for g1 in range(4):
            a, b = divmod(g, 2)
            a1, b1 = divmod(g1, 2)
            if keep(a, b, a1, b1):
                out[g * r:(g + 1) * r, g1 * c:(g1 + 1) * c] = A[g * r:(g + 1) * r, g1 * c:(g1 + 1) * c]
    return out


def pin_closed_form_q2xq2(orc):
    # Inclusion-exclusion: a triple is dropped when the first factor's middle
    # index leaves {a, a''} or the second factor's leaves {b, b''}.
    rng = _rng(3)
    Pa = lambda A: _proj_q2xq2(A, lambda a, b, a1, b1: a != a1)
    Pb = lambda A: _proj_q2xq2(A, lambda a, b, a1, b1: b != b1)
    Pab = lambda A: _proj_q2xq2(A, lambda a, b, a1, b1: a != a1 and b != b1)
    for (ra, ca, cb) in [(1, 1, 1), (2, 3, 2), (3, 2, 1)]:
        A = rng.standard_normal((4 * ra, 4 * ca))
        B = rng.standard_normal((4 * ca, 4 * cb))
        ref = A @ B - Pa(A) @ Pa(B) - Pb(A) @ Pb(B) + Pab(A) @ Pab(B)
        _close(orc.star(A, B, "Q2xQ2", 4), ref)


def pin_kronecker_q2xq2(orc):
    # The tensor square of Q2: (P1 (x) P2) * (R1 (x) R2) = (P1 *2 R1) (x) (P2 *2 R2)
    # with g = 2a + b, which is numpy.kron's index order.  The second factor may
    # carry matrix blocks.
    rng = _rng(4)
    for b in (1, 2, 3):
        P1, R1 = rng.standard_normal((2, 2)), rng.standard_normal((2, 2))
        P2, R2 = rng.standard_normal((2 * b, 2 * b)), rng.standard_normal((2 * b, 2 * b))
        lhs = orc.star(np.kron(P1, P2), np.kron(R1, R2), "Q2xQ2", 4)
        rhs = np.kron(orc.star(P1, R1, "Qq", 2), orc.star(P2, R2, "Qq", 2))
        _close(lhs, rhs)


def pin_basis_products_qq(orc):
    # Structure constants at block size 1 for q = 3: e_ij * e_lk is e_ik when
    # l == j and j is i or k, else 0.  The matrix-unit product in star must
    # follow that orientation (rows of A, columns of B).
    q = 3
    E = lambda i, j: np.eye(q)[:, [i]] @ np.eye(q)[[j], :]
    for i in range(q):
        for j in range(q):
            for l in range(q):
                for k in range(q):
                    got = orc.star(E(i, j), E(l, k), "Qq", q)
                    want = E(i, k) if (l == j and j in (i, k)) else np.zeros((q, q))
                    _close(got, want, 0)


# ------------------------------------------------------------- algebra ---

def pin_associativity(orc):
    rng = _rng(5)
    for law, q in [("Qq", 2), ("Qq", 3), ("Qq", 4), ("Q2xQ2", 4)]:
        for (r0, r1, r2, r3) in [(1, 1, 1, 1), (2, 3, 1, 2)]:
            A = rng.standard_normal((q * r0, q * r1))
            B = rng.standard_normal((q * r1, q * r2))
            C = rng.standard_normal((q * r2, q * r3))
            _close(orc.star(orc.star(A, B, law, q), C, law, q), orc.star(A, orc.star(B, C, law, q), law, q), 1e-10)


def pin_unit(orc):
    rng = _rng(6)
    for law, q in [("Qq", 2), ("Qq", 5), ("Q2xQ2", 4)]:
        A = rng.standard_normal((2 * q, 2 * q))
        I = np.eye(2 * q)
        _close(orc.star(I, A, law, q), A)
        _close(orc.star(A, I, law, q), A)


def pin_composition(orc):
    # Phi_W2(Phi_W1(X)) = Phi_{W1 * W2}(X) for row-typed inputs.
    rng = _rng(7)
    for law, q in [("Qq", 2), ("Qq", 4), ("Q2xQ2", 4)]:
        d0, d1, d2 = 3 * q, 2 * q, 5 * q
        X = rng.standard_normal((13, d0))
        W1 = rng.standard_normal((d0, d1))
        W2 = rng.standard_normal((d1, d2))
        types = orc.types_pos_mod(13, q, 3)
        lhs = orc.project(orc.project(X, W1, law, q, types), W2, law, q, types)
        rhs = orc.project(X, orc.star(W1, W2, law, q), law, q, types)
        _close(lhs, rhs, 1e-10)


def pin_rowtyped_equals_full_rows(orc):
    rng = _rng(8)
    for law, q in [("Qq", 2), ("Qq", 3), ("Q2xQ2", 4)]:
        A = rng.standard_normal((2 * q, 3 * q))
        B = rng.standard_normal((3 * q, 2 * q))
        _close(orc.project(A, B, law, q, orc.types_block_rows(2 * q, q)), orc.star(A, B, law, q))
        # a single token of type i equals the matching row of a full product
        # whose block-row i holds it
        x = rng.standard_normal((1, 3 * q))
        for i in range(q):
            Asq = np.zeros((q, 3 * q))
            Asq[i] = x[0]
            full = orc.star(Asq, B, law, q)
            _close(orc.project(x, B, law, q, [i]), full[[i]])


def pin_project_block_row(orc):
    # Block-row i of a full product A * B, computed from that block-row of A
    # alone, equals block-row i of the product given by the closed forms
    # through library matrix products (Q_q: A B - off(A) off(B); Q2 x Q2: the
    # inclusion-exclusion form).  The weight may also be any 2-D sliceable
    # (the tests pass a lazy view of a device tensor).
    rng = _rng(31)
    Pa = lambda A: _proj_q2xq2(A, lambda a, b, a1, b1: a != a1)
    Pb = lambda A: _proj_q2xq2(A, lambda a, b, a1, b1: b != b1)
    Pab = lambda A: _proj_q2xq2(A, lambda a, b, a1, b1: a != a1 and b != b1)
    for law, q, (ra, ca, cb) in [("Qq", 3, (2, 2, 3)), ("Qq", 5, (1, 3, 2)), ("Q2xQ2", 4, (3, 2, 2))]:
        A = rng.standard_normal((q * ra, q * ca))
        B = rng.standard_normal((q * ca, q * cb))
        if law == "Qq":
            full = A @ B - _off_qq(A, q) @ _off_qq(B, q)
        else:
            full = A @ B - Pa(A) @ Pa(B) - Pb(A) @ Pb(B) + Pab(A) @ Pab(B)
        for i in range(q):
            rows = slice(i * ra, (i + 1) * ra)
            _close(orc.project_block_row(A[rows], B, law, q, i), full[rows])
            # a subset of the block-row's rows (one row, in the middle)
            r = i * ra + ra // 2
            _close(orc.project_block_row(A[r:r + 1], B, law, q, i), full[r:r + 1])


def pin_row_locality(orc):
    rng = _rng(9)
    q = 4
    X = rng.standard_normal((9, 8))
    W = rng.standard_normal((8, 12))
    types = orc.types_pos_mod(9, q)
    Y = orc.project(X, W, "Qq", q, types)
    X2 = X.copy()
    X2[[0, 2, 5]] = rng.standard_normal((3, 8))
    Y2 = orc.project(X2, W, "Qq", q, types)
    keep = [1, 3, 4, 6, 7, 8]
    _close(Y[keep], Y2[keep])


def pin_types(orc):
    q = 4
    t0 = orc.types_pos_mod(10, q, 5)
    assert list(t0) == [(5 + t) % 4 for t in range(10)]
    assert list(orc.types_pos_mod(10, q, 5 + q)) == list(t0)
    assert list(orc.types_pos_mod(10, q, 6)) == list(t0[1:]) + [(6 + 9) % 4]
    # two sequences of length 8 laid end to end: positions restart
    assert list(orc.types_pos_mod(16, q, 0, 8)) == [p % 4 for p in list(range(8)) * 2]
    assert list(orc.types_pos_mod(12, 3, 0, 6)) == [0, 1, 2] * 4
    # a sequence length that q does not divide: types restart with each sequence
    assert list(orc.types_pos_mod(12, 4, 0, 6)) == [0, 1, 2, 3, 0, 1] * 2
    assert list(orc.types_pos_mod(6, 4, 4, 6)) == [0, 1, 0, 1, 2, 3]
    assert list(orc.types_block_rows(8, 4)) == [0, 0, 1, 1, 2, 2, 3, 3]


def pin_decode(orc):
    rng = _rng(10)
    for law, q in [("Qq", 4), ("Q2xQ2", 4)]:
        X = rng.standard_normal((12, 8))
        W = rng.standard_normal((8, 16))
        full = orc.project(X, W, law, q, orc.types_pos_mod(12, q, 7))
        for t in (0, 5, 11):
            _close(orc.decode(X[[t]], W, law, q, [7 + t]), full[[t]])


def pin_swiglu(orc):
    # silu against the library logistic function
    g = np.linspace(-30, 30, 241)
    _close(orc.silu(g), g * expit(g))
    # hand example (one feature, q = 1): G = ln 3, U = 2, H = ln3 * (3/4) * 2,
    # Y = 4 H = 6 ln 3
    ln3 = math.log(3.0)
    H, Y = orc.swiglu_ffn([[1.0]], [[ln3]], [[2.0]], [[4.0]], "Qq", 1, [0])
    _close(H, [[1.5 * ln3]])
    _close(Y, [[6.0 * ln3]])
    # q = 1 is the ordinary SwiGLU FFN
    rng = _rng(11)
    X = rng.standard_normal((6, 4))
    Wg, Wu, Wd = rng.standard_normal((4, 5)), rng.standard_normal((4, 5)), rng.standard_normal((5, 4))
    Gd = X @ Wg
    H, Y = orc.swiglu_ffn(X, Wg, Wu, Wd, "Qq", 1, np.zeros(6, int))
    _close(H, Gd * expit(Gd) * (X @ Wu))
    _close(Y, (Gd * expit(Gd) * (X @ Wu)) @ Wd)


# ------------------------------------------------------------- gradients ---

def pin_grad_golden_q2(orc):
    g = _load("q2_grad_hand_example.json")
    _close(orc.project(g["X"], g["W"], g["law"], g["q"], g["types"]), g["Y"], 0)
    _close(orc.project_grad_input(g["dY"], g["W"], g["law"], g["q"], g["types"]), g["dX"], 0)
    _close(orc.project_grad_weight(g["X"], g["dY"], g["law"], g["q"], g["types"]), g["dW"], 0)
    _close(orc.project_grad_weight(g["X"][:1], g["dY"][:1], g["law"], g["q"], g["types"][:1]), g["dW_type0"], 0)


def _torch_grads(fwd, X, W, dY):
    """dX, dW of sum(fwd(X, W) * dY) by torch autograd on the CPU in float64."""
    import torch
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    (fwd(torch, Xt, Wt) * torch.tensor(dY, dtype=torch.float64)).sum().backward()
    return Xt.grad.numpy(), Wt.grad.numpy()


def pin_grad_q1_is_dense(orc):
    # q = 1: the gradients of an ordinary matrix product
    rng = _rng(21)
    X, W, dY = rng.standard_normal((6, 5)), rng.standard_normal((5, 3)), rng.standard_normal((6, 3))
    gX, gW = _torch_grads(lambda torch, x, w: x @ w, X, W, dY)
    z = np.zeros(6, int)
    _close(orc.project_grad_input(dY, W, "Qq", 1, z), gX)
    _close(orc.project_grad_weight(X, dY, "Qq", 1, z), gW)
    _close(gX, dY @ W.T)
    _close(gW, X.T @ dY)


def _group_mask(q, width, keep):
    """0/1 vector over q groups of `width` features: 1 where keep(group)."""
    return np.repeat(np.array([1.0 if keep(g) else 0.0 for g in range(q)]), width)


def pin_grad_closed_form_qq(orc):
    # Autograd through the closed form y_t = x_t W - off_tau(x_t) off(W)
    # (library products only), rectangular blocks, every type present.
    rng = _rng(22)
    for q, bi, bo, M in [(2, 3, 2, 7), (3, 2, 3, 9), (5, 1, 2, 13)]:
        X = rng.standard_normal((M, q * bi))
        W = rng.standard_normal((q * bi, q * bo))
        dY = rng.standard_normal((M, q * bo))
        types = np.concatenate([np.arange(q), rng.integers(0, q, M - q)])
        keep_off = np.stack([_group_mask(q, bi, lambda g, t=t: g != t) for t in types])
        mask_off = _off_qq(np.ones_like(W), q)

        def fwd(torch, x, w):
            return x @ w - (x * torch.tensor(keep_off)) @ (w * torch.tensor(mask_off))

        gX, gW = _torch_grads(fwd, X, W, dY)
        _close(orc.project_grad_input(dY, W, "Qq", q, types), gX)
        _close(orc.project_grad_weight(X, dY, "Qq", q, types), gW)


def pin_grad_closed_form_q2xq2(orc):
    # Autograd through the row-typed inclusion-exclusion form of the tensor
    # square: y_t = x_t W - Pa_t(x_t) Pa(W) - Pb_t(x_t) Pb(W) + Pab_t(x_t) Pab(W),
    # where Pa(W) keeps blocks (g, g'') whose first factors differ and Pa_t
    # keeps the groups of x_t whose first factor differs from the type's.
    rng = _rng(23)
    for bi, bo, M in [(1, 1, 6), (2, 3, 9), (3, 1, 8)]:
        X = rng.standard_normal((M, 4 * bi))
        W = rng.standard_normal((4 * bi, 4 * bo))
        dY = rng.standard_normal((M, 4 * bo))
        types = np.concatenate([np.arange(4), rng.integers(0, 4, M - 4)])
        ones = np.ones_like(W)
        mPa = _proj_q2xq2(ones, lambda a, b, a1, b1: a != a1)
        mPb = _proj_q2xq2(ones, lambda a, b, a1, b1: b != b1)
        mPab = _proj_q2xq2(ones, lambda a, b, a1, b1: a != a1 and b != b1)
        ka = np.stack([_group_mask(4, bi, lambda g, t=t: g // 2 != t // 2) for t in types])
        kb = np.stack([_group_mask(4, bi, lambda g, t=t: g % 2 != t % 2) for t in types])
        kab = ka * kb

        def fwd(torch, x, w):
            T = lambda a: torch.tensor(a, dtype=torch.float64)
            return (x @ w - (x * T(ka)) @ (w * T(mPa)) - (x * T(kb)) @ (w * T(mPb))
                    + (x * T(kab)) @ (w * T(mPab)))

        gX, gW = _torch_grads(fwd, X, W, dY)
        _close(orc.project_grad_input(dY, W, "Q2xQ2", 4, types), gX)
        _close(orc.project_grad_weight(X, dY, "Q2xQ2", 4, types), gW)


def pin_grad_adjoint(orc):
    # Y is linear in X and in W, so <X * W, dY> = <X, dX> = <W, dW>.
    rng = _rng(24)
    for law, q, bi, bo, M in [("Qq", 4, 3, 2, 17), ("Qq", 7, 1, 3, 30), ("Q2xQ2", 4, 2, 5, 19)]:
        X = rng.standard_normal((M, q * bi))
        W = rng.standard_normal((q * bi, q * bo))
        dY = rng.standard_normal((M, q * bo))
        types = rng.integers(0, q, M)
        v = float(np.sum(orc.project(X, W, law, q, types) * dY))
        _close(np.sum(X * orc.project_grad_input(dY, W, law, q, types)), v)
        _close(np.sum(W * orc.project_grad_weight(X, dY, law, q, types)), v)


def pin_executed_flops(orc):
    for q in (2, 4, 32):
        M, d_in, d_out = 4 * q, 2 * q, 3 * q
        per = [M // q] * q
        assert orc.executed_flops(per, d_in, d_out, "Qq", q) == Fraction(2 * M * d_in * d_out * (2 * q - 1), q * q)
    assert orc.executed_flops([4] * 4, 8, 8, "Q2xQ2", 4) == Fraction(2 * 16 * 8 * 8 * 9, 16)


# ------------------------------------------------------------- digraphs ---
#
# [review], multiplication-table paragraph: the table of a directed graph
# keeps the vertex slots and the edge slots, edge times edge is zero, and the
# complete graph is Q_q.

def _upper(A, q):
    """Zero the blocks below the block diagonal."""
    A = np.array(A, dtype=np.float64)
    r, c = A.shape[0] // q, A.shape[1] // q
    for i in range(q):
        for k in range(i):
            A[i * r:(i + 1) * r, k * c:(k + 1) * c] = 0
    return A


def _support(C, q, edges):
    """Keep the diagonal blocks and the blocks of the edges; zero the rest."""
    C = np.array(C, dtype=np.float64)
    r, c = C.shape[0] // q, C.shape[1] // q
    for i in range(q):
        for k in range(q):
            if i != k and (i, k) not in edges:
                C[i * r:(i + 1) * r, k * c:(k + 1) * c] = 0
    return C


def pin_digraph_two_vertex_chain(orc):
    """One edge 0 -> 1 on two vertices: the algebra of block upper-triangular
    matrices, whose product is the ordinary matrix product."""
    g = orc.Digraph(2, [(0, 1)])
    rng = _rng(31)
    A, B = rng.standard_normal((6, 4)), rng.standard_normal((4, 10))
    _close(orc.star(A, B, g, 2), _upper(A, 2) @ _upper(B, 2))
    X, W = rng.standard_normal((7, 4)), rng.standard_normal((4, 10))
    types = np.array([0, 1, 1, 0, 1, 0, 0])
    Y = orc.project(X, W, g, 2, types)
    Wu = _upper(W, 2)
    for t in range(7):
        x = X[t].copy()
        if types[t] == 1:
            x[:2] = 0                 # a type-1 row has only its own group ...
        y = x @ Wu
        if types[t] == 1:
            y[:5] = 0                 # ... and nothing in output group 0
        _close(Y[t], y)


def pin_digraph_masked_closed_form(orc):
    """A digraph product is Q_q's closed form A B - off(A) off(B) restricted
    to the vertex and edge slots; a row of type i is x W - off_i(x) off(W) with
    the groups k of non-edges (i, k) set to zero."""
    q = 5
    rng = _rng(32)
    edges = {(i, k) for i in range(q) for k in range(q) if i != k and rng.random() < 0.45}
    g = orc.Digraph(q, edges)
    A, B = rng.standard_normal((10, 15)), rng.standard_normal((15, 20))
    want = _support(A @ B - _off_qq(A, q) @ _off_qq(B, q), q, edges)
    _close(orc.star(A, B, g, q), want)
    X, W = rng.standard_normal((23, 15)), rng.standard_normal((15, 20))
    types = rng.integers(0, q, 23)
    Y = orc.project(X, W, g, q, types)
    offW = _off_qq(W, q)
    for t in range(23):
        i = int(types[t])
        xo = X[t].copy()
        xo[i * 3:(i + 1) * 3] = 0
        y = X[t] @ W - xo @ offW
        for k in range(q):
            if k != i and (i, k) not in edges:
                y[k * 4:(k + 1) * 4] = 0
        _close(Y[t], y)


def pin_digraph_special_cases(orc):
    """The empty graph gives the block-diagonal product, the complete graph
    Q_q; one full product has q + 2 |E| block products."""
    q = 4
    rng = _rng(33)
    A, B = rng.standard_normal((8, 8)), rng.standard_normal((8, 12))
    bd = np.zeros((8, 12))
    for i in range(q):
        bd[2 * i:2 * i + 2, 3 * i:3 * i + 3] = A[2 * i:2 * i + 2, 2 * i:2 * i + 2] @ B[2 * i:2 * i + 2, 3 * i:3 * i + 3]
    _close(orc.star(A, B, orc.Digraph(q, []), q), bd)
    full = orc.Digraph(q, [(i, k) for i in range(q) for k in range(q)])
    _close(orc.star(A, B, full, q), A @ B - _off_qq(A, q) @ _off_qq(B, q))
    edges = [(0, 1), (1, 2), (2, 0), (3, 1), (0, 3)]
    assert orc.count_block_products(orc.Digraph(q, edges), q) == q + 2 * len(edges)


def pin_digraph_associativity(orc):
    q = 4
    rng = _rng(34)
    g = orc.Digraph(q, [(0, 1), (1, 2), (0, 2), (3, 0), (2, 3)])
    A, B, C = (rng.standard_normal((8, 8)) for _ in range(3))
    _close(orc.star(orc.star(A, B, g, q), C, g, q), orc.star(A, orc.star(B, C, g, q), g, q), 1e-10)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
