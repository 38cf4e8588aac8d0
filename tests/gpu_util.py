"""Helpers for the GPU tests: move synthetic inputs to the device and compare
results with the oracle.  Holds no DyRA arithmetic."""
import numpy as np

from structured_rank_matmul_amd import synth

TOL = {"bf16": 1e-2, "f32": 1e-5}     # relative Frobenius error vs the float64 oracle
OWN_ERR_TOL = 0.01                      # relative difference of ||XW - Y||/||XW||
# A single token row is held to this multiple of the tolerance: a row's error
# is a sum over fewer output elements than the whole, so it spreads more (the
# bf16 rounding of Y alone puts about 2e-3 into every row); a wrong instance
# boundary, a raced statistic or a dropped correction puts 1e-1 or more into
# the rows it touches.
ROW_MULT = 4.0


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


def check_parity(y, ref, n, dtype, label=""):
    """Asserts the parity bar three ways and returns (whole, worst instance,
    worst row): the relative Frobenius error of the whole output, of every
    instance (blocks of n rows) on its own, both <= TOL, and of every row on
    its own, <= ROW_MULT * TOL.  Rows whose reference is zero must come out
    exactly zero."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    tol = TOL[dtype]
    whole = rel(y, ref)
    d = y - ref
    inst_err = np.sqrt((d.reshape(-1, n, y.shape[1]) ** 2).sum(axis=(1, 2)))
    inst_ref = np.sqrt((ref.reshape(-1, n, y.shape[1]) ** 2).sum(axis=(1, 2)))
    row_err = np.sqrt((d ** 2).sum(axis=1))
    row_ref = np.sqrt((ref ** 2).sum(axis=1))
    zero_rows = row_ref == 0
    assert np.all(row_err[zero_rows] == 0), f"{label}: rows with a zero reference are not zero"
    inst = np.where(inst_ref > 0, inst_err / np.where(inst_ref > 0, inst_ref, 1), 0)
    rows = np.where(zero_rows, 0, row_err / np.where(zero_rows, 1, row_ref))
    worst_inst, worst_row = float(inst.max()), float(rows.max())
    assert whole <= tol, f"{label}: parity {whole:.3e} > {tol}"
    assert worst_inst <= tol, f"{label}: instance {int(inst.argmax())} parity {worst_inst:.3e} > {tol}"
    assert worst_row <= ROW_MULT * tol, f"{label}: row {int(rows.argmax())} parity {worst_row:.3e} > {ROW_MULT * tol}"
    return whole, worst_inst, worst_row


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
