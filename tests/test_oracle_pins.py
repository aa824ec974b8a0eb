"""The oracle against its pins, and planted mistakes that the pins must catch.

CPU only.  A planted mistake is a copy of oracle/algebra.py with one edit,
loaded as a separate module; the real oracle is never modified.
"""
import os
import types

import pytest

import oracle
from tests import _pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "algebra.py")


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


# Each entry: (name, text in the oracle, replacement).  Every one is a
# plausible mistake: a dropped or extra term, a wrong index, a transposed
# operand, a swapped argument, an off-by-one.
MUTANTS = [
    ("qq_drops_edge_term", "return j == i or j == k", "return j == i"),
    ("qq_drops_diag_term", "return j == i or j == k", "return j == k"),
    ("qq_is_dense", "return j == i or j == k", "return True"),
    ("qq_keeps_edge_edge", "return j == i or j == k", "return j == i or j == k or (i != k and j == (i + 1) % q)"),
    ("q2xq2_or_instead_of_and", "return (a1 == a or a1 == a2) and (b1 == b or b1 == b2)",
     "return (a1 == a or a1 == a2) or (b1 == b or b1 == b2)"),
    ("q2xq2_mixed_factors", "return (a1 == a or a1 == a2) and (b1 == b or b1 == b2)",
     "return (a1 == a or b1 == a2) and (b1 == b or a1 == b2)"),
    ("q2xq2_drops_second_factor", "return (a1 == a or a1 == a2) and (b1 == b or b1 == b2)",
     "return (a1 == a or a1 == a2)"),
    ("star_transposed_A_block", "acc += A[i * ra:(i + 1) * ra, j * ca:(j + 1) * ca]",
     "acc += A[j * ra:(j + 1) * ra, i * ca:(i + 1) * ca]"),
    ("star_transposed_B_block", "@ B[j * ca:(j + 1) * ca, k * cb:(k + 1) * cb]",
     "@ B[k * ca:(k + 1) * ca, j * cb:(j + 1) * cb]"),
    ("project_transposed_W_block", "_f64(W[j * bi:(j + 1) * bi, k * bo:(k + 1) * bo])",
     "_f64(W[k * bi:(k + 1) * bi, j * bo:(j + 1) * bo])"),
    ("project_wrong_x_group", "acc += Xi[:, j * bi:(j + 1) * bi]", "acc += Xi[:, k * bi:(k + 1) * bi]"),
    ("project_sign", "acc += Xi[:, j * bi:(j + 1) * bi]", "acc -= Xi[:, j * bi:(j + 1) * bi]"),
    ("types_off_by_one", "pos = pos_offset + np.arange(M, dtype=np.int64)",
     "pos = pos_offset + 1 + np.arange(M, dtype=np.int64)"),
    ("types_period_ignored", "        pos = pos % period\n", "        pass\n"),
    ("block_rows_interleaved", "return (np.arange(M, dtype=np.int64) // (M // q)).astype(np.int64)",
     "return (np.arange(M, dtype=np.int64) % q).astype(np.int64)"),
    ("swiglu_gate_up_swapped", "H = silu(G) * U", "H = silu(U) * G"),
    ("silu_sign", "return g / (1.0 + np.exp(-g))", "return g / (1.0 + np.exp(g))"),
    ("decode_type_from_row_index", "return project(x, W, law, q, positions % q)",
     "return project(x, W, law, q, np.arange(len(positions)) % q)"),
    ("flops_missing_factor_two", "sum(2 * int(m) * bi * bo", "sum(int(m) * bi * bo"),
    ("grad_input_untransposed_table", "if in_table(law, q, i, j, k):", "if in_table(law, q, i, k, j):"),
    ("grad_input_wrong_dy_group", "acc += dYi[:, k * bo:(k + 1) * bo] @ W", "acc += dYi[:, j * bo:(j + 1) * bo] @ W"),
    ("grad_input_transposed_block", "@ W[j * bi:(j + 1) * bi, k * bo:(k + 1) * bo].T",
     "@ W[k * bi:(k + 1) * bi, j * bo:(j + 1) * bo].T"),
    ("grad_input_only_own_group", "if in_table(law, q, i, j, k):", "if j == i:"),
    ("grad_weight_wrong_x_group", "+= Xi[:, j * bi:(j + 1) * bi].T @ dYi", "+= Xi[:, k * bi:(k + 1) * bi].T @ dYi"),
    ("grad_weight_overwrites", "dW[j * bi:(j + 1) * bi, k * bo:(k + 1) * bo] += Xi", "dW[j * bi:(j + 1) * bi, k * bo:(k + 1) * bo] = Xi"),
    ("grad_weight_dense", "for j in leaf_groups(law, q, i, k):\n                dW", "for j in range(q):\n                dW"),
    ("digraph_keeps_every_slot", "return law.has(i, k) and (j == i or j == k)", "return j == i or j == k"),
    ("digraph_edge_drops_target_diag", "return law.has(i, k) and (j == i or j == k)", "return law.has(i, k) and j == i"),
    ("block_row_next_type", "np.full(X_rows.shape[0], i, dtype=np.int64)",
     "np.full(X_rows.shape[0], (i + 1) % q, dtype=np.int64)"),
    ("block_row_type_zero", "np.full(X_rows.shape[0], i, dtype=np.int64)",
     "np.zeros(X_rows.shape[0], dtype=np.int64)"),
    ("digraph_reversed_edges", "return law.has(i, k) and (j == i or j == k)", "return law.has(k, i) and (j == i or j == k)"),
]


def _load_mutant(old, new):
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    mut = _load_mutant(old, new)
    caught = []
    for pin in _pins.ALL_PINS:
        try:
            pin(mut)
        except Exception as e:  # AssertionError or a crash both count
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches the planted mistake {name}"
