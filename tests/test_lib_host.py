"""CPU-side tests of libdyra: the C ABI loads and exports every declared symbol,
argument checks fail cleanly before any GPU work, and the host factorisation
(Algorithm 1 Offline Preparation) agrees with the oracle and with weights of
known SVD."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as orc
from structured_rank_matmul_amd import dyra, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dyra.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dyra_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = dyra.load()
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(L, name), name
    assert sorted(dyra.EXPORTED) == names


def test_status_strings():
    for s in range(0, 11):
        assert dyra.status_str(s) not in ("", "unknown status")
    assert dyra.status_str(1234) == "unknown status"


# ------------------------------------------------------------------ argument checks (no GPU needed)

def _prepare_status(W, c1, c2, r, k, lam=0.0, dtype=1, device=0):
    h = ctypes.c_void_p()
    ptr = W.ctypes.data if W is not None else None
    return dyra.load().dyra_prepare(ptr, c1, c2, r, k, lam, dtype, device, ctypes.byref(h))


def test_prepare_rejects_bad_arguments():
    W = np.zeros((64, 64), np.float32)
    assert _prepare_status(None, 64, 64, 8, 8) == 1           # null W
    assert _prepare_status(W, 64, 64, 40, 30) == 1             # r + k > min(c1, c2)
    assert _prepare_status(W, 64, 64, -1, 8) == 1              # negative rank
    assert _prepare_status(W, 64, 64, 8, 8, lam=-1.0) == 1     # negative lambda
    assert _prepare_status(W, 64, 64, 8, 8, lam=float("nan")) == 1
    assert _prepare_status(W, 64, 64, 8, 8, dtype=7) == 3      # dtype
    W2 = np.zeros((48, 64), np.float32)
    assert _prepare_status(W2, 48, 64, 8, 8) == 2              # c1 not a multiple of 32
    W3 = np.zeros((512, 512), np.float32)
    assert _prepare_status(W3, 512, 512, 8, 264) == 2          # correction rank above 256
    assert _prepare_status(W3, 512, 512, 8, 80, dtype=0) == 2  # float32 plans: correction rank above 64


def test_forward_and_dense_ref_reject_bad_arguments():
    L = dyra.load()
    # null plan
    assert L.dyra_forward(16, 1, 4, None, 16, 16, 1 << 20, None) == 1
    assert L.dyra_forward_ex(16, 1, 4, None, None, 1.0, 16, 16, 1 << 20, None) == 1
    assert L.dyra_workspace_bytes(None, 1, 4) == 0
    # dense ref: shape, dtype and alignment are checked before any launch
    assert L.dyra_dense_ref(16, 16, 8, 48, 64, 1, 16, None) == 2
    assert L.dyra_dense_ref(16, 16, 8, 64, 64, 5, 16, None) == 3
    assert L.dyra_dense_ref(18, 16, 8, 64, 64, 1, 16, None) == 4
    assert L.dyra_dense_ref(None, 16, 8, 64, 64, 1, 16, None) == 1
    assert L.dyra_dense_ref(16, 16, 0, 64, 64, 1, 16, None) == 0   # empty is a no-op
    fails = ctypes.c_int32()
    assert L.dyra_forward_status(None, 1, 1, 16, None, ctypes.byref(fails)) == 1
    assert L.dyra_stage_name(None, 1, 0) is None
    # the allocation-free forward: null plan, bad shape; its scratch size
    assert L.dyra_forward_noalloc(16, 1, 4, None, 16, None) == 1
    assert L.dyra_noalloc_scratch_bytes() == 128 << 20


def test_factorize_rejects_non_finite_weight():
    W = np.ones((32, 32), np.float32)
    W[3, 4] = np.inf
    with pytest.raises(dyra.DyraError) as e:
        dyra.dyra_factorize_host(W, 4, 4)
    assert e.value.status == 5


# ------------------------------------------------------------------ host factorisation vs oracle

def _known(c1, c2, s, seed):
    rng = synth.rng_for(seed, 88, c1 * 1000 + c2, 0)
    m = min(c1, c2)
    q1 = synth.haar_orthogonal(rng, c1, m)
    q2 = synth.haar_orthogonal(rng, c2, m)
    return ((q1 * s) @ q2.T).astype(np.float32), q1, q2


@pytest.mark.parametrize("c1,c2", [(96, 64), (64, 96), (128, 128)])
@pytest.mark.parametrize("lam", [0.0, 0.05])
def test_factorize_matches_oracle(c1, c2, lam):
    r, k = 12, 6
    W = synth.random_weight(c1, c2, 5, p=0.6)
    f = dyra.dyra_factorize_host(W, r, k, lam)
    plan = orc.offline_preparation(W.astype(np.float64), r, k, lam)
    sv = np.linalg.svd(W.astype(np.float64), compute_uv=False)
    np.testing.assert_allclose(f["sigma"], sv[:r + k], rtol=1e-10)
    np.testing.assert_allclose(f["A_s"] @ f["V_s"].T, plan.W_hat, atol=1e-10 * sv[0])
    # R0 spans the same subspace and the precomputed left factor agrees on it
    np.testing.assert_allclose(f["R0"].T @ f["R0"], plan.R0.T @ plan.R0, atol=1e-9)
    np.testing.assert_allclose(f["P_L"] @ f["R0"], plan.P_L @ plan.R0, atol=1e-9 * sv[0])
    np.testing.assert_allclose(f["R0"] @ f["R0"].T, np.eye(k), atol=1e-12)


def test_factorize_known_spectrum_and_vectors():
    c1, c2, r, k = 160, 96, 10, 8
    s = np.arange(96, 0, -1, dtype=float) ** 1.5 / 96 ** 1.5 + 0.01
    W, q1, q2 = _known(c1, c2, s, 3)
    f = dyra.dyra_factorize_host(W, r, k)
    sv = np.linalg.svd(W.astype(np.float64), compute_uv=False)
    np.testing.assert_allclose(f["sigma"], sv[:r + k], rtol=1e-10)
    np.testing.assert_allclose(f["sigma"], s[:r + k], rtol=1e-5)        # float32 rounding of W
    Vt = q2[:, r:r + k].T
    np.testing.assert_allclose(f["R0"].T @ f["R0"], Vt.T @ Vt, atol=1e-4)


def test_factorize_generated_workload_spectrum():
    w = synth.WORKLOADS["linear384_fp32"]
    W, s = synth.make_weight(w, w.layers[0])
    f = dyra.dyra_factorize_host(W, 96, 16)
    np.testing.assert_allclose(f["sigma"], s[:112], rtol=2e-5)


def test_factorize_exact_low_rank_and_edge_ranks():
    c1, c2 = 64, 96
    s = np.zeros(64)
    s[:7] = [5, 4, 3, 2.5, 2, 1.5, 1]
    W, _, _ = _known(c1, c2, s, 9)
    f = dyra.dyra_factorize_host(W, 3, 4)
    W64 = W.astype(np.float64)
    # W is exactly rank 7 only up to its float32 rounding (~1e-8 here)
    np.testing.assert_allclose(f["A_s"] @ f["V_s"].T + f["P_L"] @ f["R0"], W64, atol=1e-6)
    f0 = dyra.dyra_factorize_host(W, 0, 5)
    assert f0["A_s"].shape == (64, 0)
    plan = orc.offline_preparation(W64, 0, 5)
    np.testing.assert_allclose(f0["R0"].T @ f0["R0"], plan.R0.T @ plan.R0, atol=1e-9)
    fk = dyra.dyra_factorize_host(W, 64, 0)
    np.testing.assert_allclose(fk["A_s"] @ fk["V_s"].T, W64, atol=1e-9)


def test_factorize_vit_shape_against_oracle():
    """A full ViT-B-sized layer (768 -> 3072): subspaces at both cuts match LAPACK."""
    w = synth.WORKLOADS["vitb_fc1"]
    spec = w.layers[0]
    W, s = synth.make_weight(w, spec)
    f = dyra.dyra_factorize_host(W, spec.r, spec.k)
    plan = orc.offline_preparation(W.astype(np.float64), spec.r, spec.k)
    assert np.abs(f["A_s"] @ f["V_s"].T - plan.W_hat).max() < 1e-9 * s[0]
    assert np.abs(f["P_L"] @ f["R0"] - plan.P_L @ plan.R0).max() < 1e-9 * s[0]


# ------------------------------------------------------------------ BLAST preparation (host part)

def _blast_status(W, c1, c2, nb, rb, U, S, V, k, lam=0.0, dtype=1, device=0):
    h = ctypes.c_void_p()
    ptr = lambda a: a.ctypes.data if a is not None else None
    return dyra.load().dyra_prepare_blast(ptr(W), c1, c2, nb, rb, ptr(U), ptr(S), ptr(V), k, lam, dtype, device,
                                          ctypes.byref(h))


def test_prepare_blast_rejects_bad_arguments():
    c1, c2, nb, rb = 256, 128, 4, 8
    b = synth.random_blast_weight(c1, c2, nb, rb, 3)
    W, U, S, V = b.W, b.U, b.S, b.V
    assert _blast_status(None, c1, c2, nb, rb, U, S, V, 8) == 1        # null W
    assert _blast_status(W, c1, c2, nb, rb, None, S, V, 8) == 1        # null U
    assert _blast_status(W, c1, c2, 0, rb, U, S, V, 8) == 1            # no blocks
    assert _blast_status(W, c1, c2, nb, 0, U, S, V, 8) == 1            # rank 0
    assert _blast_status(W, c1, c2, nb, rb, U, S, V, -1) == 1          # negative k
    assert _blast_status(W, c1, c2, nb, rb, U, S, V, 8, lam=-1.0) == 1
    assert _blast_status(W, c1, c2, nb, rb, U, S, V, 8, dtype=9) == 3
    assert _blast_status(W, c1, c2, 8, rb, U, S, V, 8) == 2            # more than 4 blocks
    assert _blast_status(W, c1, c2, nb, rb, U, S, V, 80, dtype=0) == 2  # float32: k above 64
    W2 = np.zeros((192, 128), np.float32)
    assert _blast_status(W2, 192, 128, nb, rb, U, S, V, 8) == 2        # c1 not a multiple of 32 nb
    big = np.zeros((c1, 2080), np.float32)
    assert _blast_status(W, c1, c2, nb, 2080, big, S, V, 8) == 2       # rank past the mix kernel's row


def test_factorize_blast_host_matches_oracle():
    c1, c2, nb, rb, k = 96, 64, 2, 6, 5
    b = synth.random_blast_weight(c1, c2, nb, rb, 21)
    for lam in (0.0, 0.25):
        got = dyra.dyra_factorize_blast_host(b.W, b.U, b.S, b.V, nb, k, lam)
        ref = orc.offline_preparation_blast(b.W, b.U, b.S, b.V, nb, k, lam)
        assert np.allclose(got["W_res"], ref.W_res, atol=1e-12 * np.abs(ref.W_res).max())
        # R0 is fixed up to signs (and rotations within ties); P_L R0 is not
        assert np.allclose(got["P_L"] @ got["R0"], ref.P_L @ ref.R0, atol=1e-9)
        assert np.allclose(got["R0"] @ got["R0"].T, np.eye(k), atol=1e-10)


def test_factorize_blast_host_rejects_non_finite_factors():
    b = synth.random_blast_weight(64, 64, 2, 4, 22)
    U = b.U.copy()
    U[3, 1] = np.nan
    with pytest.raises(dyra.DyraError):
        dyra.dyra_factorize_blast_host(b.W, U, b.S, b.V, 2, 4)
