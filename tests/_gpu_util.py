"""Helpers for the GPU parity tests: tolerances, metrics, host copies."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances for floating-point outputs against the fp64 oracle on the same
# bf16-rounded inputs: relative Frobenius error and max |err| relative to the
# rms of the reference.
REL_FRO = 5e-3
MAX_RMS = 2e-2


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    """Exact float32 host copy of a bf16/fp32 device tensor."""
    return t.detach().float().cpu().numpy()


def metrics(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = got - ref
    nref = float(np.linalg.norm(ref))
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    rel_fro = float(np.linalg.norm(err)) / nref if nref else float(np.linalg.norm(err))
    max_rms = float(np.max(np.abs(err))) / rms if rms else float(np.max(np.abs(err), initial=0.0))
    return rel_fro, max_rms


def bf16_floor(ref) -> float:
    """max |bf16(ref) - ref| / rms(ref): what rounding the exact result to bf16 costs."""
    ref = np.asarray(ref, dtype=np.float64)
    r = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(r - ref))) / rms if rms else 0.0


def assert_parity(got, ref, out_bf16: bool, what: str = ""):
    """fp32 output: rel Frobenius <= 5e-3 and max|err| <= 2e-2 rms.  bf16
    output: the same Frobenius bound, and max|err| <= 2e-2 rms plus the cost
    of rounding the exact result to bf16 (the output format's own floor)."""
    rel_fro, max_rms = metrics(got, ref)
    floor = bf16_floor(ref) if out_bf16 else 0.0
    say(f"{what}: rel_fro={rel_fro:.3e} max/rms={max_rms:.3e} floor={floor:.3e}")
    assert rel_fro <= REL_FRO, (what, rel_fro)
    assert max_rms <= MAX_RMS + floor, (what, max_rms, floor)


class LazyRows:
    """2-D slicing view of a device tensor that copies only the requested
    slice to the host (as float32).  Lets the oracle read a few weight blocks
    of a multi-GB weight without a full host copy."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        return self.t[idx].float().cpu().numpy()
