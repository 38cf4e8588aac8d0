"""CPU oracle for DyRA's one-step dynamic residual approximation (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The product path
(the HIP library and its Python binding) never calls it and shares no code
with it.

Source: "DyRA: Dynamic Residual Approximation for Efficient Matrix
Multiplication in DNNs" (Chae, Chung, Lee, Kim).  Every function below follows
one passage of that paper, cited by section / equation / algorithm.  The code
is deliberately plain: each step of the algorithm is one numpy expression in
the paper's order, in float64, with no blocking or fusion, so that it can be
checked against the paper by eye.  Library routines (SVD, linear solve,
least squares) serve as single steps.

Notation (the paper's §2.2-2.4 / Algorithm 1 letters):
    X      [n, c1]   activations of one instance (n tokens)
    W      [c1, c2]  dense weight, product X @ W
    W_hat            structured (here: rank-r_w truncated SVD) approximation of W
    W_res            W - W_hat
    R0     [r_c, c2] fixed initial right factor R^(0)
    P_L    [c1, r_c] precomputed left projection (Eq. 7)
    L1, R1           the one-step ALS factors L^(1), R^(1)
The static rank is called ``r_w`` here and the correction rank ``r_c``; the
paper's §2.2-2.4 calls the correction rank r, and Proposition 1 calls the
static rank k.

Readings taken where the paper is silent (all listed with the design notes):
  * The structured approximation is the truncated SVD W_hat = U_r S_r V_r^T
    (Appendix B, low-rank case); Sigma is folded into the left factor.
  * R^(0) is the top-r_c right singular vectors of W_res (Appendix D default),
    obtained here from an SVD of W_res itself.
  * One lambda >= 0 per layer, used in both ridge Gram matrices (§2.2
    footnote 2; Algorithm 1 lines 5 and 12).
  * Where lambda = 0 and L^(1)'s Gram is singular (fewer tokens than the
    correction rank), L^(1) R^(1) is taken as its lambda -> 0+ limit, the
    minimum-norm least-squares solution, which is unique as a product.
  * BLAST as the structured approximation (Appendix B, BLAST): the page prints
    the block coupling S_ij as an r x r matrix, but the BLAST ranks swept in
    Appendix D reach the FLOPs reductions of Fig. 4 only with a diagonal
    coupling (an r x r one would cost more than the dense product at the
    larger ranks), so S_ij = diag(s_ij) is taken.  The paper leaves the fit of
    the factors open; they are inputs here.
  * Eq. 6 and Algorithm 1 carry no bias and no scale.  §2.4's fused linear
    layer adds a bias b and weights the correction by alpha; both are optional
    arguments here, and alpha = 1 without a bias is Eq. 6.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass
class OraclePlan:
    """Output of Algorithm 1's Offline Preparation for one layer (float64)."""
    W: np.ndarray        # [c1, c2] the dense weight, as given (upcast)
    W_hat: np.ndarray    # [c1, c2] structured approximation
    W_res: np.ndarray    # [c1, c2] residual weight W - W_hat
    A_s: np.ndarray      # [c1, r_w] left static factor U_r S_r
    V_s: np.ndarray      # [c2, r_w] right static factor V_r
    R0: np.ndarray       # [r_c, c2] fixed initial right factor
    P_L: np.ndarray      # [c1, r_c] precomputed left projection
    lam: float
    r_w: int
    r_c: int
    nb: int = 0          # BLAST blocks per side (0: the truncated-SVD W_hat)


def truncated_svd(W: np.ndarray, r: int):
    """Rank-r truncated SVD of W as (L, R) = (U_r S_r, V_r^T).

    DyRA paper, Appendix B (Low-Rank Approximation): W_hat = U_r S_r V_r^T,
    the best rank-r approximation in Frobenius norm, with L = U_r S_r and
    R = V_r^T.
    """
    U, S, Vt = np.linalg.svd(np.asarray(W, dtype=np.float64), full_matrices=False)
    return U[:, :r] * S[:r], Vt[:r, :]


def offline_preparation(W: np.ndarray, r_w: int, r_c: int, lam: float = 0.0,
                        R0: Optional[np.ndarray] = None) -> OraclePlan:
    """Algorithm 1, procedure Offline Preparation(W, k, r, lambda).

    1. structured approximation W_hat of W (Appendix B truncated SVD, rank r_w);
    2. W_res <- W - W_hat                                   (§2.1 Eq. 1);
    3. fix R^(0): by default the top-r_c right singular vectors of W_res
       (Appendix D); a caller may pass another R^(0) (§2.2 uses a Gaussian one);
    4. P_L <- (W_res R0^T)(R0 R0^T + lambda I)^-1           (Eq. 7, Alg. 1 l.5).
    """
    W = np.asarray(W, dtype=np.float64)
    c1, c2 = W.shape
    if not (r_w >= 0 and r_c >= 0 and r_w + r_c <= min(c1, c2)):
        raise ValueError("ranks out of range")
    if r_w > 0:
        A_s, Vt_s = truncated_svd(W, r_w)
    else:
        A_s, Vt_s = np.zeros((c1, 0)), np.zeros((0, c2))
    W_hat = A_s @ Vt_s
    W_res, R0, P_L = _residual_projection(W, W_hat, r_c, lam, R0)
    return OraclePlan(W=W, W_hat=W_hat, W_res=W_res, A_s=A_s, V_s=Vt_s.T.copy(), R0=R0,
                      P_L=P_L, lam=float(lam), r_w=r_w, r_c=r_c)


def _residual_projection(W: np.ndarray, W_hat: np.ndarray, r_c: int, lam: float,
                         R0: Optional[np.ndarray]):
    """Algorithm 1 Offline Preparation after the structured approximation:
    W_res <- W - W_hat (Eq. 1); R^(0) (default: top-r_c right singular vectors
    of W_res, Appendix D); P_L <- (W_res R0^T)(R0 R0^T + lambda I)^-1 (Eq. 7)."""
    c1, c2 = W.shape
    W_res = W - W_hat
    if R0 is None:
        if r_c > 0:
            _, _, Vt_res = np.linalg.svd(W_res, full_matrices=False)
            R0 = Vt_res[:r_c, :]
        else:
            R0 = np.zeros((0, c2))
    R0 = np.asarray(R0, dtype=np.float64)
    gram = R0 @ R0.T + lam * np.eye(r_c)
    # P_L = (W_res R0^T) gram^-1, written as a solve against gram^T = gram
    P_L = np.linalg.solve(gram.T, (W_res @ R0.T).T).T if r_c > 0 else np.zeros((c1, 0))
    return W_res, R0, P_L


def blast_matrix(U: np.ndarray, S: np.ndarray, V: np.ndarray, nb: int) -> np.ndarray:
    """The BLAST structured matrix W_hat [c1, c2] from its factors (Appendix B, BLAST).

    W is cut into an nb x nb grid of p x q blocks (p = c1 / nb, q = c2 / nb).
    Block (i, j) is U_i diag(s_ij) V_j^T, where U_i [p, r] (rows i p .. i p + p - 1
    of U [c1, r]) is shared by block row i, V_j [q, r] (rows of V [c2, r]) by
    block column j, and s_ij = S[i, j] [r] is the block's own coupling.
    """
    U = np.asarray(U, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    c1, r = U.shape
    c2 = V.shape[0]
    if nb < 1 or c1 % nb or c2 % nb or V.shape[1] != r or S.shape != (nb, nb, r):
        raise ValueError("BLAST factor shapes do not match")
    p, q = c1 // nb, c2 // nb
    W_hat = np.zeros((c1, c2))
    for i in range(nb):
        for j in range(nb):
            U_i = U[i * p:(i + 1) * p]
            V_j = V[j * q:(j + 1) * q]
            W_hat[i * p:(i + 1) * p, j * q:(j + 1) * q] = (U_i * S[i, j]) @ V_j.T
    return W_hat


def offline_preparation_blast(W: np.ndarray, U: np.ndarray, S: np.ndarray, V: np.ndarray, nb: int,
                              r_c: int, lam: float = 0.0, R0: Optional[np.ndarray] = None) -> OraclePlan:
    """Algorithm 1 Offline Preparation with a BLAST W_hat (Appendix B; §1 and
    §2.3 pair DyRA with any structured approximation).

    1. W_hat <- the BLAST matrix of the given factors (their fit is the
       caller's: the paper obtains them by minimising ||W - W_hat||);
    2-4. as for the truncated SVD: W_res, R^(0), P_L (Eq. 1, Appendix D, Eq. 7).
    """
    W = np.asarray(W, dtype=np.float64)
    c1, c2 = W.shape
    r = np.asarray(U).shape[1]
    if not (r_c >= 0 and r_c <= min(c1, c2)):
        raise ValueError("ranks out of range")
    W_hat = blast_matrix(U, S, V, nb)
    W_res, R0, P_L = _residual_projection(W, W_hat, r_c, lam, R0)
    return OraclePlan(W=W, W_hat=W_hat, W_res=W_res, A_s=np.zeros((c1, 0)), V_s=np.zeros((c2, 0)),
                      R0=R0, P_L=P_L, lam=float(lam), r_w=r, r_c=r_c, nb=nb)


def right_factor(L1: np.ndarray, X: np.ndarray, W_res: np.ndarray, lam: float) -> np.ndarray:
    """R^(1) <- (L1^T L1 + lambda I)^-1 (L1^T X) W_res   (Eq. 5, Alg. 1 line 12).

    The product (L1^T X) W_res is formed in the algorithm's order (the input is
    first projected onto L1, then multiplied by W_res; §2.2).  For lambda = 0
    and a singular Gram matrix the minimum-norm least-squares solution of
    min ||X W_res - L1 R|| is returned (the lambda -> 0+ limit).
    """
    r_c = L1.shape[1]
    gram = L1.T @ L1 + lam * np.eye(r_c)
    rhs = (L1.T @ X) @ W_res
    if lam == 0.0 and np.linalg.matrix_rank(L1) < r_c:
        return np.linalg.lstsq(L1, X @ W_res, rcond=None)[0]
    return np.linalg.solve(gram, rhs)


def newton_schulz_inv_sqrt(G: np.ndarray, iters: int) -> np.ndarray:
    """G^-1/2 of an SPD matrix by the coupled Newton-Schulz iteration.

    §2.4 names a Newton-Schulz iterative solver for the r x r SPD system when r
    is large (matrix products instead of a sequential factorisation) and fixes
    nothing else.  Reading taken: the coupled iteration for the inverse square
    root, scaled by the Frobenius norm c = ||G||_F so that G / c has its
    eigenvalues in (0, 1]:
        Y_0 = G / c,  Z_0 = I,
        T_k = (3 I - Z_k Y_k) / 2,  Y_{k+1} = Y_k T_k,  Z_{k+1} = T_k Z_k,
    Z_k -> (G / c)^-1/2, returned as Z_iters / sqrt(c).  Any F with F F^T = G^-1
    gives the same correction L F F^T L^T X W_res as the solve of Eq. 5.
    """
    G = np.asarray(G, dtype=np.float64)
    k = G.shape[0]
    c = np.linalg.norm(G)
    Y = G / c
    Z = np.eye(k)
    for _ in range(iters):
        Tk = 0.5 * (3.0 * np.eye(k) - Z @ Y)
        Y, Z = Y @ Tk, Tk @ Z
    return Z / np.sqrt(c)


def right_factor_ns(L1: np.ndarray, X: np.ndarray, W_res: np.ndarray, lam: float, iters: int) -> np.ndarray:
    """R^(1) of Eq. 5 with G^-1 replaced by F F, F the Newton-Schulz G^-1/2
    after `iters` steps (newton_schulz_inv_sqrt); (L1^T X) W_res in the
    algorithm's order."""
    r_c = L1.shape[1]
    F = newton_schulz_inv_sqrt(L1.T @ L1 + lam * np.eye(r_c), iters)
    return F @ (F @ ((L1.T @ X) @ W_res))


def inference_instance(X: np.ndarray, plan: OraclePlan, bias: Optional[np.ndarray] = None,
                       alpha: float = 1.0, half_steps: int = 2, ns_iters: int = 0) -> np.ndarray:
    """Algorithm 1, procedure Inference, for one instance X [n, c1].

    line 10: Y_base <- X W_hat
    line 11: L1 <- X P_L                             (Eq. 7)
    line 12: R1 <- (L1^T L1 + lambda I)^-1 (L1^T X) W_res   (Eq. 5)
    line 13: Y <- Y_base + L1 R1                     (Eq. 6)
    With §2.4's fused linear layer, line 13 becomes Y <- Y_base + b + alpha L1 R1
    (bias b [c2] added to every token row; alpha weights the correction only).
    half_steps > 2 continues the alternation of Eq. 4 / Eq. 5 from there (the
    §3.3 ablation over the iteration count: 3 = t 1.5, 4 = t 2) and uses the
    product of the last L and the last R.  ns_iters > 0 solves line 12 with the
    Newton-Schulz G^-1/2 of §2.4 instead (one ALS step only).
    """
    X = np.asarray(X, dtype=np.float64)
    Y_base = X @ plan.W_hat
    if bias is not None:
        Y_base = Y_base + np.asarray(bias, dtype=np.float64)[None, :]
    if plan.r_c == 0:
        return Y_base
    if ns_iters > 0:
        if half_steps != 2:
            raise ValueError("the Newton-Schulz solve is taken for one ALS step only")
        L1 = X @ plan.P_L
        return Y_base + alpha * (L1 @ right_factor_ns(L1, X, plan.W_res, plan.lam, ns_iters))
    if half_steps == 2:
        L1 = X @ plan.P_L
        R1 = right_factor(L1, X, plan.W_res, plan.lam)
        return Y_base + alpha * (L1 @ R1)
    L, R = als(X, plan.W_res, plan.R0, plan.lam, half_steps)
    return Y_base + alpha * (L @ R)


def inference(X: np.ndarray, B: int, n: int, plan: OraclePlan, bias: Optional[np.ndarray] = None,
              alpha: float = 1.0, half_steps: int = 2, ns_iters: int = 0) -> np.ndarray:
    """Algorithm 1 Inference over B independent instances of n tokens.

    X is [B*n, c1] with instance b in rows [b*n, (b+1)*n).  The paper solves the
    r x r system "for each batch instance" (§2.4), so every instance gets its
    own L1, R1.  bias / alpha: §2.4's fused output; half_steps: further ALS
    updates; ns_iters: the Newton-Schulz solve (see inference_instance).
    """
    X = np.asarray(X, dtype=np.float64)
    if X.shape[0] != B * n:
        raise ValueError("X rows must equal B*n")
    if half_steps < 2:
        raise ValueError("half_steps must be >= 2")
    Y = np.empty((B * n, plan.W.shape[1]))
    for b in range(B):
        rows = slice(b * n, (b + 1) * n)
        Y[rows] = inference_instance(X[rows], plan, bias, alpha, half_steps, ns_iters)
    return Y


def factors_instance(X: np.ndarray, plan: OraclePlan):
    """(L1, R1) of one instance, for tests that look inside the correction."""
    X = np.asarray(X, dtype=np.float64)
    L1 = X @ plan.P_L
    return L1, right_factor(L1, X, plan.W_res, plan.lam)


def als(X: np.ndarray, W_res: np.ndarray, R0: np.ndarray, lam: float, half_steps: int):
    """Alternating least squares on min ||X W_res - L R||_F^2 (Eq. 3-5).

    Starting from R^(0), alternate the L update (Eq. 4) and the R update
    (Eq. 5), each with the ridge term of footnote 2; ``half_steps`` counts
    single updates, so 2 = one ALS iteration (t = 1), 3 = t 1.5 (L, R, L),
    4 = t 2 (§3.3 ablation).  Returns (L, R) after the last update; R is the
    last R computed (R^(0) if none).
    """
    X = np.asarray(X, dtype=np.float64)
    r_c = R0.shape[0]
    R = np.asarray(R0, dtype=np.float64)
    L = None
    for h in range(half_steps):
        if h % 2 == 0:
            gram = R @ R.T + lam * np.eye(r_c)
            L = X @ np.linalg.solve(gram.T, (W_res @ R.T).T).T
        else:
            R = right_factor(L, X, W_res, lam)
    return L, R


def dense_product(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """The exact product X W that DyRA approximates (§2.1 Eq. 2)."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64)


def rel_fro(A: np.ndarray, B: np.ndarray) -> float:
    """||A - B||_F / ||B||_F (the normalised Frobenius error of §2.3 / App. E.4)."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    return float(np.linalg.norm(A - B) / np.linalg.norm(B))


def weight_only(X: np.ndarray, plan: OraclePlan) -> np.ndarray:
    """The static approximation X W_hat alone (§2.1, conventional methods)."""
    return np.asarray(X, dtype=np.float64) @ plan.W_hat


def optimal_rank_error(P: np.ndarray, r: int) -> float:
    """||P - [P]_r||_F for the best rank-r approximation [P]_r (Eckart-Young, §2.2).

    The optimum of Eq. 3 is the truncated SVD of the realised product; its
    error is the root-sum-square of the discarded singular values.
    """
    s = np.linalg.svd(np.asarray(P, dtype=np.float64), compute_uv=False)
    return float(np.sqrt(np.sum(s[r:] ** 2)))
