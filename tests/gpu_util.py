"""Shared helpers of the GPU parity tests: moving seeded inputs to the device
and the comparison rules (tolerances, Top-K near-tie rule)."""
import os
import sys

import numpy as np
import pytest
import torch

GAP_TIE = 1e-4        # Top-K boundary gap below which either choice is accepted
TOL_OUT = {"f32": 1e-5, "bf16": 2e-2}     # max-abs on attention outputs
TOL_F32_OUT = {"f32": 1e-5, "bf16": 1e-4}  # fp32 outputs of fp32 math (lse, scores, log_gate)
TOL_GRAD_REL = 3e-2   # per-tensor relative L2 on gradients

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(arr: np.ndarray, dtype: str = None) -> torch.Tensor:
    """Host array -> contiguous GPU tensor (uint16 bf16 bits become bfloat16)."""
    if arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)


def idx_dev(idx: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(idx.astype(np.int32))).cuda()


def lg_dev(lg: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(lg.astype(np.float32))).cuda()


def check_selection_row(gidx, glg, scores, oidx, gap, k, lse, tol_lg):
    """One (sequence, group, row) selection against the oracle.

    gidx/glg: the GPU's idx and log_gate rows; scores: the oracle's float64
    score row; oidx: the oracle's idx row; gap: oracle k-th/(k+1)-th gap.
    Returns True when the row matched bit-exactly."""
    C = len(scores)
    kk = min(k, C)
    g = [int(x) for x in gidx[:kk]]
    assert all(int(x) == -1 for x in gidx[kk:]), gidx
    assert all(np.isneginf(glg[kk:])), glg
    assert g == sorted(g) and len(set(g)) == kk and all(0 <= m < C for m in g), g
    exact = g == [int(x) for x in oidx[:kk]]
    if not exact:
        assert gap <= GAP_TIE, f"indices differ with gap {gap}: {g} vs {list(oidx[:kk])}"
        # near tie: the GPU's set must still be a valid Top-K up to the tie band
        sel = np.zeros(C, bool)
        sel[g] = True
        if kk < C:
            assert scores[sel].min() >= scores[~sel].max() - GAP_TIE
    for slot, m in enumerate(g):
        assert abs(glg[slot] - (scores[m] - lse)) <= tol_lg, (slot, m, glg[slot], scores[m] - lse)
    return exact


def rel_l2(x, ref):
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-30))
