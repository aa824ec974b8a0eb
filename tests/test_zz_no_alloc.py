"""The allocation-free SwiGLU call (aa_swiglu_ffn_fwd_noalloc) against the
call with a caller-owned hidden buffer (aa_swiglu_ffn_fwd), through the C ABI.

Both run the same kernels in the same order, so their outputs must agree bit
for bit.  Two calls in a row, the second with fewer tokens (another kernel
route: matrix-vector instead of leaf GEMMs), so that the second reads a
scratch array the first has filled.  Needs an MI355X.
"""
import pytest
import torch

import aa_inputs as inp
import associative_algebra_block_amd as aa
from tests._gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_noalloc_swiglu_equals_workspace_call():
    assert torch.cuda.is_available()
    aa.load()
    q, D, F = 32, 4096, 12288   # Qwen3-8B widths, Q_32
    up = aa.aa_plan_create("Qq", q, D, F, "pos_mod", 0, "bf16", "bf16")
    down = aa.aa_plan_create("Qq", q, F, D, "pos_mod", 0, "bf16", "f32")
    Wg, Wu = (aa.pack(up, inp.gaussian((D, F), s, D ** -0.5, torch.bfloat16, DEV)) for s in (702, 703))
    Wd = aa.pack(down, inp.gaussian((F, D), 704, F ** -0.5, torch.bfloat16, DEV))
    for M, pos in ((2048, 0), (20, 4101)):
        say("noalloc swiglu", q, D, F, M, pos)
        X = inp.gaussian((M, D), 701 + M, 1.0, torch.bfloat16, DEV)
        H = torch.empty(M, F, dtype=torch.bfloat16, device=DEV)
        Y_ref = torch.empty(M, D, dtype=torch.float32, device=DEV)
        aa.aa_swiglu_ffn_fwd(up, down, X, Wg, Wu, Wd, H, Y_ref, None, pos)
        Y = torch.full((M, D), float("nan"), dtype=torch.float32, device=DEV)
        aa.aa_swiglu_ffn_fwd_noalloc(up, down, X, Wg, Wu, Wd, Y, None, pos)
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_ref), float((Y - Y_ref).abs().max())
    # over the scratch size: refused before anything is launched, Y untouched
    M = aa.AA_NOALLOC_SCRATCH_BYTES // (2 * F) + 1
    X = torch.zeros(M, D, dtype=torch.bfloat16, device=DEV)
    Y = torch.full((M, D), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(aa.AAError) as e:
        aa.aa_swiglu_ffn_fwd_noalloc(up, down, X, Wg, Wu, Wd, Y)
    assert e.value.status == aa.AA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())
