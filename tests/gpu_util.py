"""Helpers for the GPU tests: move synthetic inputs to the device and compare
results with the oracle.  Holds no DyRA arithmetic."""
import numpy as np

from structured_rank_matmul_amd import synth

TOL = {"bf16": 1e-2, "f32": 1e-5}     # relative Frobenius error vs the float64 oracle
OWN_ERR_TOL = 0.01                      # relative difference of ||XW - Y||/||XW||


def to_device(acts: synth.Activations, device="cuda:0"):
    import torch
    if acts.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(acts.data).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(acts.data)).to(device)


def weight_to_device(W: np.ndarray, dtype: str, device="cuda:0"):
    """W [c1, c2] float32 -> device Wt [c2, c1] rounded to dtype (round to nearest even)."""
    acts = synth.round_activations(np.ascontiguousarray(W.T, dtype=np.float64), dtype)
    return to_device(acts, device), acts.exact.T


def to_host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel(a, b) -> float:
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def own_error_gap(y_gpu, y_orc, exact) -> float:
    """|e_gpu - e_orc| / e_orc for e = ||XW - Y||_F / ||XW||_F.

    Where the method is exact (e_orc at float64 rounding level, e.g. a
    correction whose rank covers the instance) the relative gap is undefined;
    the absolute e_gpu is returned instead, to be held to the parity tolerance.
    """
    e_gpu = rel(y_gpu, exact)
    e_orc = rel(y_orc, exact)
    if e_orc < 1e-9:
        return e_gpu / 2.0
    return abs(e_gpu - e_orc) / e_orc
