"""Pins of the CPU oracle against what the DyRA paper and linear algebra fix.

Each test ties the oracle (oracle/dyra_oracle.py) to something other than its
own formulas: a hand-worked example, a closed form printed by the paper
(Proposition 1 / Eq. 8 / Eq. 16), a theorem (Eckart-Young, least-squares
optimality), a known construction (W with a prescribed SVD) or brute force on
tiny shapes.  The checks are chosen so that a dropped ridge term, a wrong R0
slice, a swapped operand or a wrong sign fails at least one of them.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc
from structured_rank_matmul_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers

def known_svd_weight(c1, c2, s, seed):
    """W = Q1 diag(s) Q2^T with known Haar factors (independent of any SVD routine)."""
    rng = synth.rng_for(seed, 77, c1 * 1000 + c2, 0)
    m = min(c1, c2)
    q1 = synth.haar_orthogonal(rng, c1, m)
    q2 = synth.haar_orthogonal(rng, c2, m)
    return (q1 * s) @ q2.T, q1, q2


def gaussian(shape, seed, scale=1.0):
    rng = synth.rng_for(seed, 78, shape[0] * 1000 + shape[1], 1)
    return scale * rng.standard_normal(shape)


def qr_lstsq(A, B):
    """Least squares min ||A Z - B||_F via Householder QR (numpy.linalg.qr) and back-substitution."""
    Q, R = np.linalg.qr(A, mode="reduced")
    rhs = Q.T @ B
    n = R.shape[1]
    Z = np.zeros((n, B.shape[1]))
    for i in range(n - 1, -1, -1):
        Z[i] = (rhs[i] - R[i, i + 1:] @ Z[i + 1:]) / R[i, i]
    return Z


def read_golden(name):
    blocks, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0].isalpha() or "_" in tok[0]:
                key = tok[0]
                if len(tok) == 2:
                    blocks[key] = int(tok[1])
                    cur = None
                else:
                    blocks[key] = []
                    cur = key
            else:
                blocks[cur].append([Fraction(t) for t in tok])
    return {k: (np.array([[float(x) for x in row] for row in v]) if isinstance(v, list) else v)
            for k, v in blocks.items()}


# ------------------------------------------------------------------ golden hand example

@pytest.mark.parametrize("lam,key", [(0.0, "Y_lam0"), (1.0, "Y_lam1")])
def test_hand_worked_example(lam, key):
    g = read_golden("hand_permuted3.txt")
    plan = orc.offline_preparation(g["W"], g["r_w"], g["r_c"], lam)
    Y = orc.inference(g["X"], 1, 2, plan)
    np.testing.assert_allclose(Y, g[key], rtol=0, atol=1e-13)
    np.testing.assert_allclose(orc.dense_product(g["X"], g["W"]), g["XW"], atol=0)
    if lam == 0.0:
        assert abs(np.linalg.norm(Y - g["XW"]) - np.sqrt(2.0)) < 1e-13


# ------------------------------------------------------------------ P1 full rank

@pytest.mark.parametrize("c1,c2", [(7, 5), (5, 7), (12, 12)])
def test_full_rank_static_is_exact(c1, c2):
    W = gaussian((c1, c2), 1)
    X = gaussian((9, c1), 2)
    plan = orc.offline_preparation(W, min(c1, c2), 0)
    Y = orc.inference(X, 3, 3, plan)
    assert orc.rel_fro(Y, X @ W) < 1e-13


# ------------------------------------------------------------------ P2 isotropic / Eq. 16

@pytest.mark.parametrize("c1,c2,r_w,r_c", [(8, 10, 2, 3), (10, 6, 1, 2), (12, 12, 4, 4)])
def test_isotropic_input_reduces_to_static_rank_sum(c1, c2, r_w, r_c):
    """Proposition 1, isotropic case (App. C Eq. 16): X^T X = I gives R1 = V_{k+1:k+r}^T,
    so DyRA equals the static rank-(r_w + r_c) truncated SVD."""
    m = min(c1, c2)
    s = np.arange(m, 0, -1, dtype=float) + 0.5
    W, q1, q2 = known_svd_weight(c1, c2, s, 3)
    X = np.linalg.qr(gaussian((20, c1), 4))[0]        # orthonormal columns, X^T X = I
    plan = orc.offline_preparation(W, r_w, r_c, 0.0)
    L1, R1 = orc.factors_instance(X, plan)
    V_next = q2[:, r_w:r_w + r_c].T
    # R1 equals V_{r_w+1:r_w+r_c}^T row by row up to the sign of each singular pair
    for i in range(r_c):
        assert min(np.abs(R1[i] - V_next[i]).max(), np.abs(R1[i] + V_next[i]).max()) < 1e-10
    W_sum = (q1[:, :r_w + r_c] * s[:r_w + r_c]) @ q2[:, :r_w + r_c].T
    np.testing.assert_allclose(orc.inference(X, 1, 20, plan), X @ W_sum, atol=1e-10)


# ------------------------------------------------------------------ P3 Eq. 8 closed form

@pytest.mark.parametrize("lam_zero", [True])
@pytest.mark.parametrize("n,c1,c2,r_w,r_c", [(30, 12, 9, 3, 2), (16, 10, 14, 2, 4)])
def test_prop1_closed_form(n, c1, c2, r_w, r_c, lam_zero):
    """Proposition 1, Eq. 8: one-step DyRA = X [A_k, A_r][V_k^T; R1] with
    R1 = (A_r^T X^T X A_r)^-1 A_r^T X^T X W_res and A_r = U_{k+1:k+r} S_{k+1:k+r}."""
    m = min(c1, c2)
    s = 2.0 ** (-np.arange(m) / 2.0)
    W, q1, q2 = known_svd_weight(c1, c2, s, 5)
    X = gaussian((n, c1), 6) * np.exp(gaussian((1, c1), 7))
    A_k = q1[:, :r_w] * s[:r_w]
    A_r = q1[:, r_w:r_w + r_c] * s[r_w:r_w + r_c]
    W_res = (q1[:, r_w:] * s[r_w:]) @ q2[:, r_w:].T
    XtX = X.T @ X
    R1 = np.linalg.inv(A_r.T @ XtX @ A_r) @ (A_r.T @ XtX @ W_res)
    Y_closed = X @ np.hstack([A_k, A_r]) @ np.vstack([q2[:, :r_w].T, R1])
    plan = orc.offline_preparation(W, r_w, r_c, 0.0)
    np.testing.assert_allclose(orc.inference(X, 1, n, plan), Y_closed, rtol=0,
                               atol=1e-10 * np.abs(Y_closed).max())


# ------------------------------------------------------------------ P4 Eckart-Young

def _floor_eigh(P, r):
    """Best rank-r error of P from the eigenvalues of P^T P (an independent routine)."""
    ev = np.sort(np.clip(np.linalg.eigvalsh(P.T @ P), 0, None))[::-1]
    return np.sqrt(np.sum(ev[r:]))


@pytest.mark.parametrize("lam", [0.0, 0.3])
def test_correction_never_beats_eckart_young(lam):
    c1, c2, r_w, r_c, B, n = 16, 20, 4, 3, 5, 12
    W = synth.random_weight(c1, c2, 11).astype(np.float64)
    X = synth.x_logcols(synth.rng_for(0, 79, 0, 1), B * n, c1)
    plan = orc.offline_preparation(W, r_w, r_c, lam)
    for b in range(B):
        Xb = X[b * n:(b + 1) * n]
        P = Xb @ plan.W_res
        L1, R1 = orc.factors_instance(Xb, plan)
        err = np.linalg.norm(P - L1 @ R1)
        assert err >= _floor_eigh(P, r_c) * (1 - 1e-12) - 1e-12
        # the whole output is rank <= r_w + r_c: it cannot beat that floor for X W either
        Yb = orc.inference_instance(Xb, plan)
        assert np.linalg.norm(Xb @ W - Yb) >= _floor_eigh(Xb @ W, r_w + r_c) * (1 - 1e-12) - 1e-12


def test_oracle_floor_matches_independent_routine():
    P = gaussian((13, 9), 12)
    for r in range(0, 9):
        assert abs(orc.optimal_rank_error(P, r) - _floor_eigh(P, r)) < 1e-10


def test_als_error_is_monotone_and_approaches_floor():
    """Each ALS half-step is an exact least-squares minimisation at lambda = 0,
    so the error cannot increase; with enough steps it reaches the rank-r_c
    floor (Fig. 2 / App. E.3 behaviour, here on synthetic data)."""
    c1, c2, r_w, r_c, n = 24, 30, 6, 4, 40
    W = synth.random_weight(c1, c2, 13).astype(np.float64)
    X = gaussian((n, c1), 14) * np.exp(2 * gaussian((1, c1), 15))
    plan = orc.offline_preparation(W, r_w, r_c, 0.0)
    P = X @ plan.W_res
    errs = []
    for h in range(2, 41, 2):
        L, R = orc.als(X, plan.W_res, plan.R0, 0.0, h)
        errs.append(np.linalg.norm(P - L @ R))
    assert all(b <= a * (1 + 1e-10) for a, b in zip(errs, errs[1:]))
    assert errs[-1] <= _floor_eigh(P, r_c) * (1 + 1e-3)
    # one ALS iteration (two half-steps) is exactly what Inference computes
    L, R = orc.als(X, plan.W_res, plan.R0, 0.0, 2)
    np.testing.assert_allclose(orc.inference_instance(X, plan), X @ plan.W_hat + L @ R, atol=1e-10)


# ------------------------------------------------------------------ P5 never worse than weight-only

@pytest.mark.parametrize("lam", [0.0, 1e-3, 1.0, 100.0])
@pytest.mark.parametrize("seed", [0, 1])
def test_dyra_not_worse_than_weight_only(lam, seed):
    c1, c2, r_w, r_c, B, n = 32, 24, 5, 4, 4, 10
    W = synth.random_weight(c1, c2, 20 + seed).astype(np.float64)
    X = gaussian((B * n, c1), 21 + seed) * np.exp(gaussian((1, c1), 22))
    plan = orc.offline_preparation(W, r_w, r_c, lam)
    XW = X @ W
    for b in range(B):
        rows = slice(b * n, (b + 1) * n)
        e_dyra = np.linalg.norm(XW[rows] - orc.inference_instance(X[rows], plan))
        e_w = np.linalg.norm(XW[rows] - orc.weight_only(X[rows], plan))
        assert e_dyra <= e_w * (1 + 1e-12)


# ------------------------------------------------------------------ P6 single token

@pytest.mark.parametrize("lam", [0.0, 0.5])
def test_single_token_sherman_morrison(lam):
    c1, c2, r_w, r_c = 20, 14, 3, 5
    W = synth.random_weight(c1, c2, 30).astype(np.float64)
    x = gaussian((1, c1), 31)
    plan = orc.offline_preparation(W, r_w, r_c, lam)
    l = x @ plan.P_L
    ll = (l @ l.T).item()
    s = ll / (lam + ll)
    expect = x @ plan.W_hat + s * (x @ plan.W_res)
    np.testing.assert_allclose(orc.inference_instance(x, plan), expect, atol=1e-12)
    if lam == 0.0:  # the correction restores the exact product
        np.testing.assert_allclose(orc.inference_instance(x, plan), x @ W, atol=1e-12)


# ------------------------------------------------------------------ P7 fewer tokens than rank: dual form

@pytest.mark.parametrize("n", [2, 3, 5])
def test_primal_equals_push_through_dual(n):
    c1, c2, r_w, r_c, lam = 18, 16, 3, 6, 0.25
    W = synth.random_weight(c1, c2, 40).astype(np.float64)
    X = gaussian((n, c1), 41 + n)
    plan = orc.offline_preparation(W, r_w, r_c, lam)
    L1 = X @ plan.P_L
    dual = L1 @ L1.T @ np.linalg.inv(L1 @ L1.T + lam * np.eye(n)) @ (X @ plan.W_res)
    np.testing.assert_allclose(orc.inference_instance(X, plan), X @ plan.W_hat + dual, atol=1e-11)


def test_lambda_zero_underdetermined_is_projection():
    """lambda = 0, n < r_c: L1 R1 is the projection of X W_res onto span(L1) (min-norm LS)."""
    c1, c2, r_w, r_c, n = 18, 16, 3, 6, 4
    W = synth.random_weight(c1, c2, 42).astype(np.float64)
    X = gaussian((n, c1), 43)
    plan = orc.offline_preparation(W, r_w, r_c, 0.0)
    L1 = X @ plan.P_L
    Q = np.linalg.qr(L1)[0]
    proj = Q @ (Q.T @ (X @ plan.W_res))
    np.testing.assert_allclose(orc.inference_instance(X, plan), X @ plan.W_hat + proj, atol=1e-11)


# ------------------------------------------------------------------ P8 exact low-rank W

def test_exact_when_rank_equals_r_w_plus_r_c():
    c1, c2, r_w, r_c = 14, 11, 3, 4
    s = np.zeros(11)
    s[:r_w + r_c] = np.linspace(5, 1, r_w + r_c)
    W, _, _ = known_svd_weight(c1, c2, s, 50)
    X = gaussian((3 * 9, c1), 51)
    plan = orc.offline_preparation(W, r_w, r_c, 0.0)
    assert orc.rel_fro(orc.inference(X, 3, 9, plan), X @ W) < 1e-12


# ------------------------------------------------------------------ P9 invariants

def test_instances_independent_and_equivariant():
    c1, c2, r_w, r_c, B, n = 16, 12, 3, 2, 3, 7
    W = synth.random_weight(c1, c2, 60).astype(np.float64)
    X = gaussian((B * n, c1), 61)
    plan = orc.offline_preparation(W, r_w, r_c, 0.0)
    Y = orc.inference(X, B, n, plan)
    X2 = X.copy()
    X2[n:2 * n] = gaussian((n, c1), 62)                      # change instance 1 only
    Y2 = orc.inference(X2, B, n, plan)
    np.testing.assert_array_equal(Y[:n], Y2[:n])
    np.testing.assert_array_equal(Y[2 * n:], Y2[2 * n:])
    perm = np.random.default_rng(0).permutation(n)
    Yp = orc.inference(X[perm], 1, n, plan)
    np.testing.assert_allclose(Yp, Y[:n][perm], atol=1e-12)
    np.testing.assert_allclose(orc.inference(3.5 * X, B, n, plan), 3.5 * Y, rtol=1e-11, atol=1e-11)
    plan2 = orc.offline_preparation(-2.0 * W, r_w, r_c, 0.0)
    np.testing.assert_allclose(orc.inference(X, B, n, plan2), -2.0 * Y, rtol=1e-10, atol=1e-10)


def test_r0_rotation_and_sign_invariance():
    """Only the row space of R0 matters: a rotation of R0 (any invertible mix) leaves Y unchanged."""
    c1, c2, r_w, r_c, n = 16, 12, 3, 3, 9
    W = synth.random_weight(c1, c2, 63).astype(np.float64)
    X = gaussian((n, c1), 64)
    plan = orc.offline_preparation(W, r_w, r_c, 0.0)
    Q = np.linalg.qr(gaussian((r_c, r_c), 65))[0]
    plan_rot = orc.offline_preparation(W, r_w, r_c, 0.0, R0=Q @ plan.R0)
    np.testing.assert_allclose(orc.inference(X, 1, n, plan_rot), orc.inference(X, 1, n, plan), atol=1e-11)


# ------------------------------------------------------------------ P10 known spectrum

def test_generated_weight_has_prescribed_spectrum():
    w = synth.WORKLOADS["linear384_fp32"]
    spec = w.layers[0]
    W32, s = synth.make_weight(w, spec)
    sv = np.linalg.svd(W32.astype(np.float64), compute_uv=False)
    np.testing.assert_allclose(sv, s, rtol=2e-5, atol=1e-6 * s[0])
    np.testing.assert_allclose(s, np.arange(1, 385) ** -0.7)


def test_static_factor_matches_known_construction():
    c1, c2, r_w = 40, 30, 7
    s = 1.0 / np.arange(1, 31)
    W, q1, q2 = known_svd_weight(c1, c2, s, 70)
    plan = orc.offline_preparation(W, r_w, 2, 0.0)
    np.testing.assert_allclose(plan.W_hat, (q1[:, :r_w] * s[:r_w]) @ q2[:, :r_w].T, atol=1e-12)
    # R0 spans the next two right singular vectors of W
    P = plan.R0.T @ plan.R0
    np.testing.assert_allclose(P, q2[:, r_w:r_w + 2] @ q2[:, r_w:r_w + 2].T, atol=1e-10)


# ------------------------------------------------------------------ P11 brute force, tiny shapes

def _tiny_cases():
    out = []
    for (c1, c2) in [(4, 6), (6, 4), (5, 5), (8, 3)]:
        m = min(c1, c2)
        for r_w in range(0, m):
            for r_c in range(1, m - r_w + 1):
                for n in (r_c, 6):
                    out.append((c1, c2, r_w, r_c, n))
    return out


@pytest.mark.parametrize("lam", [0.0, 0.7])
def test_brute_force_tiny(lam):
    """Form X W_res explicitly and solve both ridge least-squares half-steps by QR of
    the stacked systems [R0^T; sqrt(lam) I] and [L1; sqrt(lam) I]."""
    count = 0
    for (c1, c2, r_w, r_c, n) in _tiny_cases():
        seed = c1 * 1000 + c2 * 100 + r_w * 10 + r_c + n
        W = gaussian((c1, c2), seed)
        X = gaussian((n, c1), seed + 1)
        plan = orc.offline_preparation(W, r_w, r_c, lam)
        P = X @ plan.W_res
        # L step: min ||P - L R0||^2 + lam ||L||^2  ->  stacked LS for L^T
        A = np.vstack([plan.R0.T, np.sqrt(lam) * np.eye(r_c)])
        L = qr_lstsq(A, np.vstack([P.T, np.zeros((r_c, n))])).T
        np.testing.assert_allclose(L, X @ plan.P_L, atol=1e-10)
        # R step: min ||P - L R||^2 + lam ||R||^2
        if lam == 0.0 and np.linalg.matrix_rank(L) < r_c:
            LR = L @ np.linalg.pinv(L) @ P
        else:
            A = np.vstack([L, np.sqrt(lam) * np.eye(r_c)])
            LR = L @ qr_lstsq(A, np.vstack([P, np.zeros((r_c, c2))]))
        Y = orc.inference_instance(X, plan)
        np.testing.assert_allclose(Y, X @ plan.W_hat + LR, atol=1e-9 * max(1.0, np.abs(Y).max()))
        # no random perturbation of R1 lowers the ridge objective
        L1, R1 = orc.factors_instance(X, plan)
        obj = np.linalg.norm(P - L1 @ R1) ** 2 + lam * np.linalg.norm(R1) ** 2
        rng = np.random.default_rng(seed)
        for _ in range(5):
            D = 1e-3 * rng.standard_normal(R1.shape)
            obj2 = np.linalg.norm(P - L1 @ (R1 + D)) ** 2 + lam * np.linalg.norm(R1 + D) ** 2
            assert obj2 >= obj - 1e-12 * max(1.0, obj)
        count += 1
    assert count > 40


def test_rank_arguments_validated():
    W = gaussian((5, 4), 90)
    with pytest.raises(ValueError):
        orc.offline_preparation(W, 3, 2)
    with pytest.raises(ValueError):
        orc.inference(gaussian((5, 5), 91), 2, 3, orc.offline_preparation(W, 1, 1))


# ------------------------------------------------------------------ §2.4 fused output: bias and alpha

@pytest.mark.parametrize("c1,c2", [(7, 5), (6, 9)])
def test_fused_bias_full_rank_is_exact_affine(c1, c2):
    """§2.4's fused linear layer at full static rank without correction is the
    plain affine map X W + b (P1 with a bias)."""
    W = gaussian((c1, c2), 100)
    X = gaussian((8, c1), 101)
    b = gaussian((1, c2), 102)[0]
    plan = orc.offline_preparation(W, min(c1, c2), 0)
    Y = orc.inference(X, 2, 4, plan, bias=b)
    assert orc.rel_fro(Y, X @ W + b[None, :]) < 1e-13


def test_fused_alpha_zero_is_weight_only_plus_bias():
    """alpha = 0 leaves the static product X W_hat plus the bias, with W_hat the
    rank-r_w truncated SVD formed here from numpy's SVD of W directly."""
    W = gaussian((12, 10), 103)
    X = gaussian((15, 12), 104)
    b = gaussian((1, 10), 105)[0]
    plan = orc.offline_preparation(W, 3, 4)
    U, S, Vt = np.linalg.svd(W)
    W_hat = (U[:, :3] * S[:3]) @ Vt[:3]
    Y = orc.inference(X, 3, 5, plan, bias=b, alpha=0.0)
    np.testing.assert_allclose(Y, X @ W_hat + b[None, :], atol=1e-12)


@pytest.mark.parametrize("alpha", [0.5, -1.25, 3.0])
def test_fused_alpha_scales_only_the_correction(alpha):
    """Y(alpha) - Y(0) = alpha (Y(1) - Y(0)), and the bias shifts every row of
    every instance by b: the static part is neither scaled nor biased twice."""
    W = gaussian((16, 11), 106)
    X = gaussian((18, 16), 107)
    b = gaussian((1, 11), 108)[0]
    plan = orc.offline_preparation(W, 4, 3, 0.05)
    y0 = orc.inference(X, 3, 6, plan, alpha=0.0)
    y1 = orc.inference(X, 3, 6, plan)
    ya = orc.inference(X, 3, 6, plan, alpha=alpha)
    np.testing.assert_allclose(ya - y0, alpha * (y1 - y0), atol=1e-12)
    yb = orc.inference(X, 3, 6, plan, bias=b, alpha=alpha)
    np.testing.assert_allclose(yb - ya, np.broadcast_to(b, ya.shape), atol=1e-12)
    # the correction really is there: alpha changes the output
    assert orc.rel_fro(y1, y0) > 1e-3


# ------------------------------------------------------------------ §3.3 further ALS steps, Gaussian R0

def _proj(A):
    """Orthogonal projector onto the column space of A (full column rank), by QR."""
    Qm, _ = np.linalg.qr(A)
    return Qm @ Qm.T


@pytest.mark.parametrize("half_steps", [2, 3, 4, 5, 6])
@pytest.mark.parametrize("gaussian_r0", [False, True])
def test_als_steps_are_block_power_iteration(half_steps, gaussian_r0):
    """At lambda = 0 every ALS update is an exact least-squares fit, so with
    P = X W_res the alternation from R0 is block power iteration: after 2h
    updates L R is P projected onto the columns of (P P^T)^(h-1) P R0^T, after
    2h + 1 updates P projected on the right onto the columns of (P^T P)^h R0^T.
    The projectors come from QR here, not from the oracle's solves."""
    c1, c2, r_w, r_c, n = 14, 17, 3, 4, 12
    W = synth.random_weight(c1, c2, 110).astype(np.float64)
    X = gaussian((n, c1), 111) * np.exp(gaussian((1, c1), 112))
    R0 = gaussian((r_c, c2), 113) if gaussian_r0 else None
    plan = orc.offline_preparation(W, r_w, r_c, 0.0, R0=R0)
    P = X @ plan.W_res
    R0 = plan.R0
    h = half_steps // 2
    if half_steps % 2 == 0:
        K = np.linalg.matrix_power(P @ P.T, h - 1) @ P @ R0.T
        corr = _proj(K) @ P
    else:
        K = np.linalg.matrix_power(P.T @ P, h) @ R0.T
        corr = P @ _proj(K)
    Y = orc.inference(X, 1, n, plan, half_steps=half_steps)
    np.testing.assert_allclose(Y - X @ plan.W_hat, corr, atol=1e-8 * np.linalg.norm(P))


def test_more_als_steps_never_increase_the_error_and_reach_the_floor_from_gaussian_r0():
    """Fig. 2 / Appendix E.3 setting: Gaussian R^(0); at lambda = 0 the error of
    the correction falls with every update and approaches the Eckart-Young floor
    of the realised residual product, at the rate of block power iteration (the
    ratio of the (r_c+1)-th to the r_c-th singular value per two updates; 0.66 to
    0.89 for these instances, so 80 updates)."""
    c1, c2, r_w, r_c, B, n = 20, 26, 4, 3, 3, 15
    W = synth.random_weight(c1, c2, 114).astype(np.float64)
    X = gaussian((B * n, c1), 115) * np.exp(gaussian((1, c1), 116))
    plan = orc.offline_preparation(W, r_w, r_c, 0.0, R0=gaussian((r_c, c2), 117))
    for b in range(B):
        Xb = X[b * n:(b + 1) * n]
        P = Xb @ plan.W_res
        errs = [np.linalg.norm(orc.inference(Xb, 1, n, plan, half_steps=h) - Xb @ plan.W_hat - P)
                for h in range(2, 81)]
        assert all(e2 <= e1 * (1 + 1e-9) for e1, e2 in zip(errs, errs[1:]))
        assert errs[-1] <= orc.optimal_rank_error(P, r_c) * (1 + 1e-6)
        assert errs[0] > orc.optimal_rank_error(P, r_c) * (1 + 1e-3)   # one step is not yet optimal


def test_half_steps_with_ridge_differ_from_plain_and_keep_bias_alpha_semantics():
    """With lambda > 0 the extra updates still change the result, and bias and
    alpha act on the final product exactly as for one step."""
    c1, c2, r_w, r_c, n = 16, 12, 3, 3, 10
    W = synth.random_weight(c1, c2, 118).astype(np.float64)
    X = gaussian((2 * n, c1), 119) * np.exp(gaussian((1, c1), 120))
    b = gaussian((1, c2), 121)[0]
    plan = orc.offline_preparation(W, r_w, r_c, 0.3)
    y2 = orc.inference(X, 2, n, plan)
    y4 = orc.inference(X, 2, n, plan, half_steps=4)
    assert orc.rel_fro(y4, y2) > 1e-6
    y0 = orc.inference(X, 2, n, plan, alpha=0.0)
    y4ab = orc.inference(X, 2, n, plan, bias=b, alpha=0.5, half_steps=4)
    np.testing.assert_allclose(y4ab - b[None, :] - y0, 0.5 * (y4 - y0), atol=1e-11)


# ------------------------------------------------------------------ §2.4 Newton-Schulz SPD solve

def _ns_scalar(mu, iters):
    """The coupled iteration on one eigenvalue mu of G / c: y_0 = mu, z_0 = 1,
    t = (3 - z y) / 2, y <- y t, z <- t z."""
    y, z = mu, 1.0
    for _ in range(iters):
        t = 0.5 * (3.0 - z * y)
        y, z = y * t, t * z
    return z


@pytest.mark.parametrize("iters", [0, 1, 3, 8, 20])
def test_newton_schulz_acts_eigenvalue_by_eigenvalue(iters):
    """Every iterate is a polynomial in G, so the matrix iteration is the scalar
    recurrence applied to each eigenvalue of G / ||G||_F (eigenvectors from
    numpy's eigh, not from the iteration)."""
    A = gaussian((30, 9), 122) * np.exp(gaussian((1, 9), 123))
    G = A.T @ A + 0.01 * np.eye(9)
    lam, V = np.linalg.eigh(G)
    c = np.linalg.norm(G)
    expect = (V * np.array([_ns_scalar(m / c, iters) for m in lam])) @ V.T / np.sqrt(c)
    np.testing.assert_allclose(orc.newton_schulz_inv_sqrt(G, iters), expect, atol=1e-10 * np.abs(expect).max())


def test_newton_schulz_converges_to_the_cholesky_solution():
    """Enough steps reach G^-1/2 (eigh) and the correction equals the one of the
    Cholesky / LU solve of Eq. 5; few steps do not."""
    c1, c2, r_w, r_c, n = 18, 14, 3, 5, 25
    W = synth.random_weight(c1, c2, 124).astype(np.float64)
    X = gaussian((2 * n, c1), 125) * np.exp(gaussian((1, c1), 126))
    plan = orc.offline_preparation(W, r_w, r_c, 0.0)
    y_exact = orc.inference(X, 2, n, plan)
    y_ns = orc.inference(X, 2, n, plan, ns_iters=40)
    assert orc.rel_fro(y_ns, y_exact) < 1e-10
    assert orc.rel_fro(orc.inference(X, 2, n, plan, ns_iters=2), y_exact) > 1e-4
    L1 = X[:n] @ plan.P_L
    G = L1.T @ L1
    lam, V = np.linalg.eigh(G)
    np.testing.assert_allclose(orc.newton_schulz_inv_sqrt(G, 40), (V / np.sqrt(lam)) @ V.T, rtol=1e-9, atol=1e-12)


def test_rel_fro_hand_values():
    """The metric's relative Frobenius error, ||A - B||_F / ||B||_F, against
    values worked by hand: the reference is the second argument (swapping the
    two changes the value), the norm runs over every entry of the matrix (not a
    row or column), and it is a ratio of norms, not of squared norms."""
    A = np.array([[3.0, 4.0], [0.0, 1.0]])
    B = np.array([[3.0, 4.0], [0.0, 0.0]])
    assert orc.rel_fro(A, B) == pytest.approx(1.0 / 5.0, rel=1e-15)          # ||(0,0,0,1)|| / ||(3,4,0,0)||
    assert orc.rel_fro(B, A) == pytest.approx(1.0 / np.sqrt(26.0), rel=1e-15)
    C = np.array([[1.0, 2.0], [2.0, 4.0]])
    D = np.array([[1.0, 0.0], [0.0, 2.0]])
    # ||(0,2,2,2)|| / ||(1,0,0,2)|| = sqrt(12) / sqrt(5)
    assert orc.rel_fro(C, D) == pytest.approx(np.sqrt(12.0 / 5.0), rel=1e-15)
    assert orc.rel_fro(D, D) == 0.0
