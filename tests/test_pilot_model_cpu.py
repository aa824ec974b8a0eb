"""CPU checks of the pilot-shaped decoder stack's definition (no GPU)."""
import torch

from associative_algebra_block_amd.pilot_stack import PilotConfig, make_weights


def test_parameter_count_is_the_pages():
    """agihunt.info review, model paragraph: 110,631,168 parameters.  The
    configuration's count and the tensors make_weights creates (the tied LM
    head's transposed copy is storage, not a parameter) both give it."""
    cfg = PilotConfig()
    assert cfg.parameter_count() == 110_631_168
    w = make_weights(cfg, 0, "cpu")
    n = sum(t.numel() for k, t in w.items() if k not in ("layers", "E_T"))
    n += sum(t.numel() for lw in w["layers"] for t in lw.values())
    assert n == 110_631_168
    assert torch.equal(w["E_T"], w["E"].t())
