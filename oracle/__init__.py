"""fp64 CPU oracle (test infrastructure only; see oracle/algebra.py)."""
from .algebra import (  # noqa: F401
    LAW_QQ, LAW_Q2XQ2, LAWS, Digraph, in_table, leaf_groups, count_block_products,
    count_row_block_products, types_pos_mod, types_block_rows, star, project,
    project_block_row, silu, swiglu_ffn, decode, executed_flops,
    project_grad_input, project_grad_weight,
)
