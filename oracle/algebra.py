"""Plain fp64 CPU oracle for the row-typed associative-algebra projection Y = X * W.

TEST INFRASTRUCTURE. This module is the checker, not the product: only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it.  It
shares no code with the HIP library and imports nothing from it.

Sources (the pages are web pages about the preprint "Change the Product, Keep
the Parameters: Associative Algebra Layers for Transformers", Koziev and
Oseledets):
  [review]   agihunt.info review of the preprint, the only page that states the
             construction: the paragraph on the graph multiplication table, the
             rank paragraph, the composition paragraph, the row-typing
             paragraph and the pilot-law paragraph (tensor square of Q2).
  [summary]  hotpaper.ai summary, "technical approach" list (6 block GEMMs for
             Q2; row types use (A,U) and (V,D)).
  [post]     the authors' post on feed.hirify.me, part one (bilinear operator,
             rank 6 for q = 2).

Everything is computed in float64 from whatever values the caller passes (the
tests pass the same bf16-rounded numbers the GPU receives).  Loops are plain
block loops over the interaction table; the only library primitive is the
matrix product of two blocks.  Nothing is blocked, fused or reordered beyond
the definition.

Readings taken where the pages are silent:
  * feature groups are contiguous and of equal width;
  * the row type of the token at absolute position p is p mod q;
  * a token's own (diagonal) group is the group whose index equals its type;
  * coordinates of the tensor-square law are Kronecker-ordered, g = 2a + b;
  * SwiGLU is silu(g) * u with no biases.
"""
from __future__ import annotations

import numpy as np

LAW_QQ = "Qq"
LAW_Q2XQ2 = "Q2xQ2"
LAWS = (LAW_QQ, LAW_Q2XQ2)


class Digraph:
    """The multiplication table of a directed graph on q vertices.

    [review], multiplication-table paragraph: the table comes from a directed
    graph whose vertices are the diagonal slots and whose edges are the kept
    off-diagonal slots; a product of two edges is zero, and the complete graph
    gives Q_q.  So with an edge set E (pairs (i, k), i != k):
        C_ii = A_ii B_ii,  C_ik = A_ii B_ik + A_ik B_kk for (i, k) in E,
    and a slot (i, k) that is not an edge holds nothing: C_ik = 0, and the
    blocks A_ik, B_ik of such slots take part in no product.
    An instance is passed wherever a law is expected.
    """

    def __init__(self, q: int, edges):
        self.q = int(q)
        es = set()
        for i, k in edges:
            i, k = int(i), int(k)
            if not (0 <= i < self.q and 0 <= k < self.q):
                raise ValueError("edge outside the vertex range")
            if i != k:
                es.add((i, k))
        self.edges = frozenset(es)

    def has(self, i: int, k: int) -> bool:
        return (i, k) in self.edges

    def __repr__(self) -> str:
        return f"Digraph({self.q}, {sorted(self.edges)})"


# --------------------------------------------------------------------------
# The interaction table
# --------------------------------------------------------------------------

def _check_law(law, q: int) -> None:
    if isinstance(law, Digraph):
        if law.q != q:
            raise ValueError("the digraph has a different number of vertices")
        return
    if law not in LAWS:
        raise ValueError(f"unknown law {law!r}")
    if q < 1:
        raise ValueError("q must be >= 1")
    if law == LAW_Q2XQ2 and q != 4:
        raise ValueError("the tensor square of Q2 has exactly 4 groups")


def in_table(law: str, q: int, i: int, j: int, k: int) -> bool:
    """True when row type i lets input group j reach output group k.

    Q_q ([review], multiplication-table paragraph): for the complete graph on q
    vertices the diagonal block of the product takes only its own diagonal
    pair, C_ii = A_ii B_ii, and an off-diagonal block is the source diagonal
    times the edge plus the edge times the target diagonal,
    C_ik = A_ii B_ik + A_ik B_kk.  Written as a set of index triples
    (i, j, k) with C_ik = sum over j of A_ij B_jk, that is: j == i or j == k.
    An edge times an edge (j differing from both i and k) is zero.

    Q2 (x) Q2 ([review], pilot-law paragraph): the tensor square of Q2.  Group
    g stands for the pair (a, b) with g = 2a + b; a triple of pairs is kept when
    it is kept in each factor separately.
    """
    _check_law(law, q)
    if isinstance(law, Digraph):
        # vertex slot: its own diagonal pair; edge slot: source diagonal times
        # the edge, edge times target diagonal; any other slot: nothing
        if k == i:
            return j == i
        return law.has(i, k) and (j == i or j == k)
    if law == LAW_QQ:
        return j == i or j == k
    a, b = divmod(i, 2)
    a1, b1 = divmod(j, 2)
    a2, b2 = divmod(k, 2)
    return (a1 == a or a1 == a2) and (b1 == b or b1 == b2)


def leaf_groups(law: str, q: int, i: int, k: int) -> list[int]:
    """Input groups j that feed output group k for a row of type i."""
    return [j for j in range(q) if in_table(law, q, i, j, k)]


def count_block_products(law: str, q: int) -> int:
    """Number of block products A_ij B_jk in one full algebra product."""
    return sum(len(leaf_groups(law, q, i, k)) for i in range(q) for k in range(q))


def count_row_block_products(law: str, q: int, i: int) -> int:
    """Number of block products one row of type i performs (one table row)."""
    return sum(len(leaf_groups(law, q, i, k)) for k in range(q))


# --------------------------------------------------------------------------
# Row types
# --------------------------------------------------------------------------

def types_pos_mod(M: int, q: int, pos_offset: int = 0, period: int = 0) -> np.ndarray:
    """Row type from absolute position ([review], row-typing paragraph).

    Row t of the batch sits at position pos_offset + t, taken modulo `period`
    when the batch is several sequences of that length laid end to end; its
    type is that position modulo q.
    """
    pos = pos_offset + np.arange(M, dtype=np.int64)
    if period:
        pos = pos % period
    return (pos % q).astype(np.int64)


def types_block_rows(M: int, q: int) -> np.ndarray:
    """Block-row typing for a full algebra product: row r of block-row i has type i."""
    if M % q:
        raise ValueError("block-row typing needs q | M")
    return (np.arange(M, dtype=np.int64) // (M // q)).astype(np.int64)


# --------------------------------------------------------------------------
# Products
# --------------------------------------------------------------------------

def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def star(A, B, law: str, q: int) -> np.ndarray:
    """Full algebra product C = A * B of two q x q block matrices.

    C_ik = sum over j with (i, j, k) in the table of A_ij B_jk.  A is split
    into q block-rows and q block-columns, B into q block-rows (matching A's
    block-columns) and q block-columns.  Rectangular blocks are allowed.
    """
    _check_law(law, q)
    A = _f64(A)
    B = _f64(B)
    mA, nA = A.shape
    nB_rows, nB = B.shape
    if nA != nB_rows:
        raise ValueError("inner sizes differ")
    if mA % q or nA % q or nB % q:
        raise ValueError("q must divide every side")
    ra, ca, cb = mA // q, nA // q, nB // q
    C = np.zeros((mA, nB), dtype=np.float64)
    for i in range(q):
        for k in range(q):
            acc = np.zeros((ra, cb), dtype=np.float64)
            for j in leaf_groups(law, q, i, k):
                acc += A[i * ra:(i + 1) * ra, j * ca:(j + 1) * ca] @ B[j * ca:(j + 1) * ca, k * cb:(k + 1) * cb]
            C[i * ra:(i + 1) * ra, k * cb:(k + 1) * cb] = acc
    return C


def project(X, W, law: str, q: int, types) -> np.ndarray:
    """Row-typed projection Y = X * W ([review], row-typing paragraph).

    Each token (row t of X) computes only the table row of its type tau(t):
    Y[t, group k] = sum over j with (tau(t), j, k) in the table of
    X[t, group j] @ W_jk.  X is M x d_in, W is d_in x d_out, q divides both.
    """
    _check_law(law, q)
    # Anything with .shape and 2-D slicing will do for W (only the blocks the
    # table names are read); lists are converted.
    X = X if hasattr(X, "shape") else np.asarray(X)
    W = W if hasattr(W, "shape") else np.asarray(W)
    types = np.asarray(types, dtype=np.int64)
    M, d_in = X.shape
    if W.shape[0] != d_in:
        raise ValueError("X and W disagree on d_in")
    d_out = W.shape[1]
    if d_in % q or d_out % q:
        raise ValueError("q must divide d_in and d_out")
    if types.shape != (M,):
        raise ValueError("one type per row")
    if M and (types.min() < 0 or types.max() >= q):
        raise ValueError("row type out of range")
    bi, bo = d_in // q, d_out // q
    Y = np.zeros((M, d_out), dtype=np.float64)
    for i in range(q):
        rows = np.nonzero(types == i)[0]
        if rows.size == 0:
            continue
        Xi = _f64(X[rows])
        for k in range(q):
            acc = np.zeros((rows.size, bo), dtype=np.float64)
            for j in leaf_groups(law, q, i, k):
                acc += Xi[:, j * bi:(j + 1) * bi] @ _f64(W[j * bi:(j + 1) * bi, k * bo:(k + 1) * bo])
            Y[rows, k * bo:(k + 1) * bo] = acc
    return Y


def project_block_row(X_rows, W, law: str, q: int, i: int) -> np.ndarray:
    """Row-typed projection of a set of rows that all have type i.

    The same definition as `project`, for callers that hold only some rows
    (for example one block-row of a large full product).  Only the weight
    blocks the table row of type i names are read.
    """
    X_rows = X_rows if hasattr(X_rows, "shape") else np.asarray(X_rows)
    return project(X_rows, W, law, q, np.full(X_rows.shape[0], i, dtype=np.int64))


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU, g * sigmoid(g), in float64."""
    return g / (1.0 + np.exp(-g))


def swiglu_ffn(X, Wg, Wu, Wd, law: str, q: int, types) -> tuple[np.ndarray, np.ndarray]:
    """SwiGLU feed-forward whose three projections use the algebra product.

    The pilot model's FFN is SwiGLU ([post], part three; [review], model
    paragraph) and only its projections change.  Reading: no biases,
    H = silu(X * Wg) elementwise-times (X * Wu), Y = H * Wd, with the same row
    types in all three products.  Returns (H, Y), both float64.
    """
    G = project(X, Wg, law, q, types)
    U = project(X, Wu, law, q, types)
    H = silu(G) * U
    Y = project(H, Wd, law, q, types)
    return H, Y


def decode(x, W, law: str, q: int, positions) -> np.ndarray:
    """Decode step: each new token computes only its own table row.

    [review], row-typing paragraph: at generation time only the new position's
    row is computed.  x holds one row per new token, positions[r] is the
    absolute position of row r, and its type is positions[r] mod q.
    """
    positions = np.asarray(positions, dtype=np.int64)
    return project(x, W, law, q, positions % q)


# --------------------------------------------------------------------------
# Gradients of the row-typed projection
# --------------------------------------------------------------------------
#
# The pages report a backward pass for the projection (authors' measurements
# of forward plus gradient on the Qwen3-30B-A3B expert shape, [review] kernel
# paragraph) without writing it out.  Reading: the backward is the exact
# gradient of the bilinear map Y = X * W defined by `project`.  With
# T the interaction table and tau(t) the type of row t,
#     Y[t, k] = sum over j with (tau(t), j, k) in T of X[t, j] W_jk,
# so for an upstream gradient dY
#     dX[t, j] = sum over k with (tau(t), j, k) in T of dY[t, k] W_jk^T,
#     dW_jk    = sum over rows t with (tau(t), j, k) in T of X[t, j]^T dY[t, k].
# Both are written out below as block loops over the same table.

def project_grad_input(dY, W, law: str, q: int, types) -> np.ndarray:
    """dX of the row-typed projection for upstream gradient dY (M x d_out).

    Row t of type i receives, in input group j, dY[t, k] W_jk^T summed over
    the output groups k whose table entry (i, j, k) is kept.  Under Q_q that
    is every k for j == i and only k == j otherwise.
    """
    _check_law(law, q)
    dY = _f64(dY)
    W = _f64(W)
    types = np.asarray(types, dtype=np.int64)
    M, d_out = dY.shape
    d_in = W.shape[0]
    if W.shape[1] != d_out:
        raise ValueError("dY and W disagree on d_out")
    if d_in % q or d_out % q:
        raise ValueError("q must divide d_in and d_out")
    if types.shape != (M,):
        raise ValueError("one type per row")
    if M and (types.min() < 0 or types.max() >= q):
        raise ValueError("row type out of range")
    bi, bo = d_in // q, d_out // q
    dX = np.zeros((M, d_in), dtype=np.float64)
    for i in range(q):
        rows = np.nonzero(types == i)[0]
        if rows.size == 0:
            continue
        dYi = dY[rows]
        for j in range(q):
            acc = np.zeros((rows.size, bi), dtype=np.float64)
            for k in range(q):
                if in_table(law, q, i, j, k):
                    acc += dYi[:, k * bo:(k + 1) * bo] @ W[j * bi:(j + 1) * bi, k * bo:(k + 1) * bo].T
            dX[rows, j * bi:(j + 1) * bi] = acc
    return dX


def project_grad_weight(X, dY, law: str, q: int, types) -> np.ndarray:
    """dW (d_in x d_out, row-major) of the row-typed projection.

    Block W_jk collects X[t, j]^T dY[t, k] over the rows t whose type i keeps
    the entry (i, j, k).  Under Q_q an off-diagonal block W_jk (j != k) is
    reached only by rows of type j; a diagonal block W_kk by rows of every
    type.  Blocks no row reaches get zero.
    """
    _check_law(law, q)
    X = _f64(X)
    dY = _f64(dY)
    types = np.asarray(types, dtype=np.int64)
    M, d_in = X.shape
    if dY.shape[0] != M:
        raise ValueError("X and dY disagree on M")
    d_out = dY.shape[1]
    if d_in % q or d_out % q:
        raise ValueError("q must divide d_in and d_out")
    if types.shape != (M,):
        raise ValueError("one type per row")
    if M and (types.min() < 0 or types.max() >= q):
        raise ValueError("row type out of range")
    bi, bo = d_in // q, d_out // q
    dW = np.zeros((d_in, d_out), dtype=np.float64)
    for i in range(q):
        rows = np.nonzero(types == i)[0]
        if rows.size == 0:
            continue
        Xi, dYi = X[rows], dY[rows]
        for k in range(q):
            for j in leaf_groups(law, q, i, k):
                dW[j * bi:(j + 1) * bi, k * bo:(k + 1) * bo] += Xi[:, j * bi:(j + 1) * bi].T @ dYi[:, k * bo:(k + 1) * bo]
    return dW


# --------------------------------------------------------------------------
# Arithmetic counts
# --------------------------------------------------------------------------

def executed_flops(M_per_type, d_in: int, d_out: int, law: str, q: int) -> int:
    """Multiply-add FLOPs (2 per MAC) a row-typed projection executes.

    M_per_type[i] rows of type i each perform count_row_block_products(i)
    products of a 1 x b_in row with a b_in x b_out block.
    """
    bi, bo = d_in // q, d_out // q
    return int(sum(2 * int(m) * bi * bo * count_row_block_products(law, q, i)
                   for i, m in enumerate(M_per_type)))
