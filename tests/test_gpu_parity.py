"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Bar: relative Frobenius error <= 1e-2 (bf16) / 1e-5 (fp32) against the
oracle's output, and the approximation's own error ||XW - Y||/||XW|| within 1%
(relative) of the oracle's.  Small shapes span several tiles with ragged
tails; the workload shapes run at full size.
"""
import numpy as np
import pytest

import oracle as orc
from structured_rank_matmul_amd import dyra, synth

from gpu_util import OWN_ERR_TOL, TOL, own_error_gap, rel, to_device, to_host, weight_to_device

pytestmark = pytest.mark.gpu

_PLANS = {}


def oracle_plan(W, r, k, lam):
    key = (W.tobytes().__hash__(), W.shape, r, k, lam)
    if key not in _PLANS:
        _PLANS[key] = orc.offline_preparation(W.astype(np.float64), r, k, lam)
    return _PLANS[key]


def run_case(W, X, B, n, r, k, lam, dtype, check_own=True):
    import torch
    plan = dyra.dyra_prepare(W, r, k, lam, dtype, 0)
    xd = to_device(X)
    Y = dyra.dyra_forward(xd, B, n, plan)
    torch.cuda.synchronize()
    y = to_host(Y)
    op = oracle_plan(W, r, k, lam)
    ref = orc.inference(X.exact, B, n, op)
    err = rel(y, ref)
    assert err <= TOL[dtype], f"parity {err:.3e} > {TOL[dtype]}"
    if check_own:
        exact = X.exact @ W.astype(np.float64)
        gap = own_error_gap(y, ref, exact)
        assert gap <= OWN_ERR_TOL, f"own-error gap {gap:.3e}"
    plan.close()
    return err


# ------------------------------------------------------------------ dense reference

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,c1,c2", [(300, 96, 160), (129, 64, 64), (1, 32, 32), (517, 256, 384)])
def test_dense_ref_matches_exact(dtype, N, c1, c2):
    import torch
    W = synth.random_weight(c1, c2, 3)
    X = synth.random_matrix(N, c1, 4, dtype)
    Wt, W_exact = weight_to_device(W, dtype)
    Y = dyra.dyra_dense_ref(to_device(X), Wt)
    torch.cuda.synchronize()
    ref = X.exact @ W_exact
    assert rel(to_host(Y), ref) <= TOL[dtype]
    # agrees with the vendor GEMM to output rounding
    Yt = to_device(X).float() @ Wt.float().T
    assert rel(to_host(Y), to_host(Yt)) <= (5e-3 if dtype == "bf16" else 1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,c1,c2", [(8192, 352, 4096), (8192, 352, 3072), (25600, 352, 320)])
def test_dense_ref_k_tail_on_large_tiles(dtype, N, c1, c2):
    """K = 352 is 5.5 slices of 64 bf16 elements: the last slice is short.
    These sizes select the 256 x 256, 256 x 128 and 256 x 160 tiles."""
    test_dense_ref_matches_exact(dtype, N, c1, c2)


def _random_gemm_shapes(count=12, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        N = int(rng.integers(1, 3000))
        c1 = 32 * int(rng.integers(1, 24))   # odd multiples of 32 leave a short last slice
        c2 = 32 * int(rng.integers(1, 80))
        out.append((N, c1, c2))
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,c1,c2", _random_gemm_shapes())
def test_dense_ref_random_shapes(dtype, N, c1, c2):
    """Seeded random shapes: ragged rows and columns against every tile size,
    K an odd or even multiple of 32."""
    test_dense_ref_matches_exact(dtype, N, c1, c2)


def test_dense_ref_empty_is_noop():
    import torch
    Wt = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda:0")
    X = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    Y = dyra.dyra_dense_ref(X, Wt)
    assert Y.shape == (0, 64)


# ------------------------------------------------------------------ forward, small shapes

SMALL = [
    # B, n, c1, c2, r, k
    (5, 37, 192, 320, 40, 12),     # tiles straddle several instances, ragged rows
    (3, 150, 256, 288, 64, 16),    # instances longer than a 128-row tile
    (2, 300, 128, 416, 20, 32),    # ragged output columns (416 = 3*128 + 32)
    (1, 64, 64, 96, 8, 8),
    (7, 16, 96, 128, 30, 16),      # n = k = 16: taken by the dual form
    (6, 32, 96, 128, 30, 16),      # n = 2k: smallest primal case here
    (2, 17, 128, 96, 24, 16),      # 17 tokens: primal just above the dual range
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", SMALL)
def test_forward_small(dtype, case):
    B, n, c1, c2, r, k = case
    W = synth.random_weight(c1, c2, 11 + c1, p=0.5)
    X = synth.random_matrix(B * n, c1, 12 + n, dtype)
    run_case(W, X, B, n, r, k, 0.0, dtype)


def test_forward_k_tail_on_large_tiles():
    """32 instances of 201 tokens into 4096 outputs select the 256 x 256
    output tiles with correction slices; r = 96 leaves a short last static
    slice there (K = 96) and c1 = 352 one in the left pass."""
    B, n, c1, c2, r, k = 32, 201, 352, 4096, 96, 64
    W = synth.random_weight(c1, c2, 61, p=0.6)
    X = synth.random_matrix(B * n, c1, 62, "bf16")
    run_case(W, X, B, n, r, k, 0.0, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("lam", [1e-2, 5.0])
def test_forward_ridge(dtype, lam):
    B, n, c1, c2, r, k = 4, 50, 128, 192, 16, 16
    W = synth.random_weight(c1, c2, 21, p=0.5)
    X = synth.random_matrix(B * n, c1, 22, dtype)
    run_case(W, X, B, n, r, k, lam, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_weight_only_and_exact(dtype):
    B, n, c1, c2 = 3, 40, 96, 160
    W = synth.random_weight(c1, c2, 31, p=0.5)
    X = synth.random_matrix(B * n, c1, 32, dtype)
    run_case(W, X, B, n, 24, 0, 0.0, dtype)          # k = 0: X A_s V_s^T only
    err = run_case(W, X, B, n, 96, 0, 0.0, dtype, check_own=False)   # full rank: X W
    assert err <= TOL[dtype]


def test_forward_empty_batch_is_noop():
    import torch
    W = synth.random_weight(64, 64, 41)
    plan = dyra.dyra_prepare(W, 8, 8, 0.0, "bf16", 0)
    X = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    Y = dyra.dyra_forward(X, 0, 5, plan)
    assert Y.shape == (0, 64)


def test_failed_solve_is_flagged():
    """lambda = 0 and an all-zero instance: L1 = 0, the Gram matrix is singular;
    that instance is flagged and gets no correction (its exact output is 0)."""
    import torch
    B, n, c1, c2, r, k = 4, 20, 64, 96, 8, 8
    W = synth.random_weight(c1, c2, 42)
    X = synth.random_matrix(B * n, c1, 43, "bf16")
    X.data[n:2 * n] = 0
    X.data[3 * n:] = 0
    plan = dyra.dyra_prepare(W, r, k, 0.0, "bf16", 0)
    ws = dyra.alloc_workspace(plan, B, n)
    Y = dyra.dyra_forward(to_device(X), B, n, plan, workspace=ws)
    assert dyra.dyra_forward_status(plan, B, n, ws) == 2
    y = to_host(Y)
    assert np.all(y[n:2 * n] == 0) and np.all(y[3 * n:] == 0)
    ref = orc.inference(X.exact[:n], 1, n, oracle_plan(W, r, k, 0.0))
    assert rel(y[:n], ref) <= TOL["bf16"]
    torch.cuda.synchronize()


# ------------------------------------------------------------------ fewer tokens than the correction rank

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,n,lam", [(1, 1, 0.0), (16, 1, 0.0), (64, 1, 0.0), (5, 1, 0.3), (6, 3, 0.2),
                                     (4, 5, 0.0), (9, 15, 0.05)])
def test_forward_dual_form(dtype, B, n, lam):
    c1, c2, r, k = 256, 320, 32, 16
    W = synth.random_weight(c1, c2, 51, p=0.5)
    X = synth.random_matrix(B * n, c1, 52 + B * n, dtype)
    run_case(W, X, B, n, r, k, lam, dtype, check_own=(lam > 0 or n > 1))


# ------------------------------------------------------------------ workload shapes

def _workload_case(wname, lname, sample=None):
    import torch
    w = synth.WORKLOADS[wname]
    spec = w.layer(lname)
    W, _ = synth.make_weight(w, spec)
    X = synth.make_activations(w, spec)
    plan = dyra.dyra_prepare(W, spec.r, spec.k, 0.0, w.dtype, 0)
    Y = dyra.dyra_forward(to_device(X), w.B, w.n, plan)
    torch.cuda.synchronize()
    y = to_host(Y)
    op = oracle_plan(W, spec.r, spec.k, 0.0)
    idx = range(w.B) if sample is None else sample
    rows = np.concatenate([np.arange(b * w.n, (b + 1) * w.n) for b in idx])
    Xs = X.exact[rows]
    ref = orc.inference(Xs, len(idx), w.n, op)
    err = rel(y[rows], ref)
    exact = Xs @ W.astype(np.float64)
    gap = own_error_gap(y[rows], ref, exact)
    e_w = rel(orc.weight_only(Xs, op), exact)
    print(f"{wname}/{lname}: parity {err:.3e}  own-error gap {gap:.3e}  "
          f"e_dyra {rel(ref, exact):.4f}  e_weight_only {e_w:.4f}", flush=True)
    assert err <= TOL[w.dtype]
    assert gap <= OWN_ERR_TOL
    plan.close()


def test_workload_linear384_fp32():
    _workload_case("linear384_fp32", "linear")


def test_workload_vitb_fc1():
    _workload_case("vitb_fc1", "fc1")


@pytest.mark.parametrize("layer", ["qkv", "fc1", "fc2"])
def test_workload_vitl_block(layer):
    _workload_case("vitl_block", layer)


@pytest.mark.parametrize("layer", ["fc1", "fc2"])
def test_workload_whisper_mlp(layer):
    _workload_case("whisper_mlp", layer, sample=[0, 7, 15])
