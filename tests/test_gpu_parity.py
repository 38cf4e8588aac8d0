"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Bar: relative Frobenius error <= 1e-2 (bf16) / 1e-5 (fp32) against the
oracle's output, for the whole output and for every instance on its own,
every token row within ROW_MULT times that (gpu_util.check_parity), and the
approximation's own error ||XW - Y||/||XW|| within 1% (relative) of the
oracle's.  Small shapes span several tiles with ragged tails; the workload
shapes run at full size, on every instance or on sampled ones.
"""
import numpy as np
import pytest

import oracle as orc
from structured_rank_matmul_amd import dyra, synth

from gpu_util import OWN_ERR_TOL, TOL, check_parity, own_error_gap, rel, to_device, to_host, weight_to_device

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
    err, _, _ = check_parity(y, ref, n, dtype, f"B={B} n={n} r={r} k={k} lambda={lam} {dtype}")
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
    check_parity(to_host(Y), ref, N, dtype, f"dense {N}x{c1}x{c2}")
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


LARGE_K = [
    # B, n, c1, c2, r, k: correction ranks above 64 (blocked Cholesky,
    # several 32-wide panels; G in the workspace above 128; M' in passes of 64)
    (4, 300, 512, 640, 64, 128),
    (3, 400, 512, 512, 32, 256),
    (2, 260, 384, 512, 40, 200),    # padded to 208: panels past the real rank
    (5, 150, 256, 384, 48, 80),     # n < 2k, tiles straddle instances
]


@pytest.mark.parametrize("case", LARGE_K, ids=lambda c: f"B{c[0]}n{c[1]}-{c[2]}x{c[3]}-r{c[4]}k{c[5]}")
def test_forward_large_correction_rank(case):
    B, n, c1, c2, r, k = case
    W = synth.random_weight(c1, c2, 13 + k, p=0.5)
    X = synth.random_matrix(B * n, c1, 14 + n, "bf16")
    X = synth.round_activations(X.exact * np.exp(synth.random_matrix(1, c1, 15, "f32").exact), "bf16")
    run_case(W, X, B, n, r, k, 0.0, "bf16")


@pytest.mark.parametrize("k", [128, 192])
def test_vitl_qkv_large_correction_rank(k):
    """The ViT-L qkv layer (128 x 201 tokens, 1024 -> 3072, r = 256) with a
    correction rank of 128 and 192, three instances against the oracle."""
    import torch
    w = synth.WORKLOADS["vitl_block"]
    spec = w.layer("qkv")
    W, _ = synth.make_weight(w, spec)
    X = synth.make_activations(w, spec)
    plan = dyra.dyra_prepare(W, spec.r, k, 0.0, "bf16", 0)
    Y = dyra.dyra_forward(to_device(X), w.B, w.n, plan)
    torch.cuda.synchronize()
    sample = [0, 63, 127]
    rows = np.concatenate([np.arange(b * w.n, (b + 1) * w.n) for b in sample])
    Xs = X.exact[rows]
    op = oracle_plan(W, spec.r, k, 0.0)
    ref = orc.inference(Xs, len(sample), w.n, op)
    y = to_host(Y)[rows]
    err, wi, wr = check_parity(y, ref, w.n, "bf16", f"vitl qkv k={k}")
    exact = Xs @ W.astype(np.float64)
    gap = own_error_gap(y, ref, exact)
    e_orc = rel(ref, exact)
    print(f"vitl qkv k={k}: parity {err:.3e} (instance {wi:.3e}, row {wr:.3e})  own-error gap {gap:.3e}  "
          f"e_dyra {e_orc:.4f}", flush=True)
    # the output's own rounding adds to the approximation error in
    # quadrature, e_gpu^2 ~ e_orc^2 + err^2, so the 1% bar on the own error
    # is reachable only where e_orc >= 7 err (k = 192 leaves e_dyra near 0.02,
    # within 6x of the bf16 rounding of Y: parity is the measure there)
    if e_orc >= 7 * err:
        assert gap <= OWN_ERR_TOL
    plan.close()


PANELS = [
    # B, n, c1, c2, r, k, lambda: instance boundaries against the GEMMs' row
    # tiles, a static rank that fills whole 32-wide K slices, a ragged last tile
    (5, 37, 384, 512, 256, 64, 0.3),     # several instances per tile (n < k: ridge)
    (3, 201, 384, 768, 240, 64, 0.0),    # r = 240 padded to 256; instances straddle tiles
    (4, 64, 512, 512, 256, 64, 0.0),     # instances aligned with 64-row blocks
    (2, 100, 320, 512, 240, 50, 0.5),    # k = 50 padded to 64, with a ridge
    (3, 90, 320, 512, 256, 0, 0.0),      # static path: no correction
    (1, 1000, 448, 1024, 256, 64, 0.0),  # one long instance, ragged last tile
]


@pytest.mark.parametrize("case", PANELS, ids=lambda c: f"B{c[0]}n{c[1]}-{c[2]}x{c[3]}-r{c[4]}k{c[5]}-lam{c[6]}")
def test_forward_instance_boundaries(case):
    B, n, c1, c2, r, k, lam = case
    W = synth.random_weight(c1, c2, 141 + n, p=0.6)
    X = synth.random_matrix(B * n, c1, 142 + n, "bf16")
    run_case(W, X, B, n, r, k, lam, "bf16", check_own=k > 0)


def test_forward_ex_bias_alpha_full_static_slices():
    import torch
    B, n, c1, c2, r, k = 4, 70, 384, 512, 256, 64
    W = synth.random_weight(c1, c2, 151, p=0.6)
    X = synth.random_matrix(B * n, c1, 152, "bf16")
    bias = synth.random_matrix(1, c2, 153, "bf16", scale=2.0)
    plan = dyra.dyra_prepare(W, r, k, 0.0, "bf16", 0)
    Y = dyra.dyra_forward_ex(to_device(X), B, n, plan, bias=to_device(bias)[0], alpha=-0.5)
    torch.cuda.synchronize()
    ref = orc.inference(X.exact, B, n, oracle_plan(W, r, k, 0.0), bias=bias.exact[0], alpha=-0.5)
    check_parity(to_host(Y), ref, n, "bf16", "bias/alpha r = 256")
    plan.close()


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


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_failed_solve_is_flagged(dtype):
    """lambda = 0 and an all-zero instance: L1 = 0, the Gram matrix is singular;
    that instance is flagged and gets no correction (its exact output is 0)."""
    import torch
    B, n, c1, c2, r, k = 4, 20, 64, 96, 8, 8
    W = synth.random_weight(c1, c2, 42)
    X = synth.random_matrix(B * n, c1, 43, dtype)
    X.data[n:2 * n] = 0
    X.data[3 * n:] = 0
    plan = dyra.dyra_prepare(W, r, k, 0.0, dtype, 0)
    ws = dyra.alloc_workspace(plan, B, n)
    Y = dyra.dyra_forward(to_device(X), B, n, plan, workspace=ws)
    assert dyra.dyra_forward_status(plan, B, n, ws) == 2
    y = to_host(Y)
    assert np.all(y[n:2 * n] == 0) and np.all(y[3 * n:] == 0)
    ref = orc.inference(X.exact, B, n, oracle_plan(W, r, k, 0.0))
    check_parity(y, ref, n, dtype, "zero instances")
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


# ------------------------------------------------------------------ 16 < n < k

@pytest.mark.parametrize("dtype", ["bf16"])
@pytest.mark.parametrize("B,n,c1,c2,r,k", [(6, 20, 256, 320, 32, 32), (4, 40, 256, 384, 48, 64),
                                           (3, 63, 256, 256, 32, 64), (2, 50, 512, 512, 64, 128),
                                           (5, 17, 128, 192, 16, 48)])
def test_forward_fewer_tokens_than_rank_no_ridge(dtype, B, n, c1, c2, r, k):
    """lambda = 0 and 16 < n < k: the dual form with the projector onto
    range(L1_b); with independent token rows that projector is the identity and
    the output is X W up to the plan's rounding."""
    W = synth.random_weight(c1, c2, 101 + n, p=0.5)
    X = synth.random_matrix(B * n, c1, 102 + n, dtype)
    run_case(W, X, B, n, r, k, 0.0, dtype, check_own=False)


def test_forward_fewer_tokens_than_rank_rank_deficient():
    """lambda = 0, 16 < n < k, instances whose L1 rows are dependent: repeated
    tokens (rank 10 of 30) and an all-zero instance.  The projector is then
    onto a proper subspace; it must still match the oracle's minimum-norm
    least-squares result."""
    B, n, c1, c2, r, k = 3, 30, 256, 320, 32, 64
    W = synth.random_weight(c1, c2, 111, p=0.5)
    X = synth.random_matrix(B * n, c1, 112, "bf16")
    X.data[n:2 * n] = np.tile(X.data[n:n + 10], (3, 1))   # instance 1: 10 distinct rows, each 3 times
    X.data[2 * n:] = 0                                    # instance 2: zero
    run_case(W, X, B, n, r, k, 0.0, "bf16", check_own=False)


@pytest.mark.parametrize("B,n,c1,c2,r,k,lam", [(4, 40, 256, 384, 48, 64, 0.5), (3, 100, 512, 512, 64, 128, 0.1)])
def test_forward_fewer_tokens_than_rank_with_ridge(B, n, c1, c2, r, k, lam):
    """lambda > 0 and 16 < n < k: the primal form (L1^T L1 + lambda I is
    positive definite)."""
    W = synth.random_weight(c1, c2, 121 + n, p=0.5)
    X = synth.random_matrix(B * n, c1, 122 + n, "bf16")
    run_case(W, X, B, n, r, k, lam, "bf16")


def test_forward_refuses_long_instances_below_rank_without_ridge():
    """lambda = 0 with 64 < n < k has no supported form."""
    import torch
    W = synth.random_weight(512, 512, 131)
    plan = dyra.dyra_prepare(W, 32, 128, 0.0, "bf16", 0)
    X = torch.zeros((2 * 100, 512), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(dyra.DyraError) as e:
        dyra.dyra_forward(X, 2, 100, plan)
    assert e.value.status == 2
    plan.close()


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
    err, worst_inst, worst_row = check_parity(y[rows], ref, w.n, w.dtype, f"{wname}/{lname}")
    exact = Xs @ W.astype(np.float64)
    gap = own_error_gap(y[rows], ref, exact)
    e_w = rel(orc.weight_only(Xs, op), exact)
    print(f"{wname}/{lname}: parity {err:.3e} (worst instance {worst_inst:.3e}, worst row {worst_row:.3e}) over "
          f"{len(idx)} instances  own-error gap {gap:.3e}  e_dyra {rel(ref, exact):.4f}  e_weight_only {e_w:.4f}",
          flush=True)
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
    """Every instance: each spans six 256-token blocks."""
    _workload_case("whisper_mlp", layer)


def test_many_long_instances():
    """96 instances of 2048 tokens: the per-instance statistics span eight
    256-token blocks per instance and the launches far more workgroups than
    are resident at once, so an instance's Gram matrix must be complete before
    any of its rows is rewritten.  Every instance is checked on its own."""
    B, n, c1, c2, r, k = 96, 2048, 512, 512, 128, 64
    W = synth.random_weight(c1, c2, 71, p=0.6)
    X = synth.random_matrix(B * n, c1, 72, "bf16")
    run_case(W, X, B, n, r, k, 0.0, "bf16")
