"""Exact floating-point operation counts of one DyRA layer call, for the
FLOPs-matched static baseline.

"DyRA: Dynamic Residual Approximation for Efficient Matrix Multiplication in
DNNs", §2.3 (Computational Cost; FLOPs-Matched Comparison, footnote 4) and
Appendix E.4: the static baseline raises the truncated-SVD rank from r (the
paper's k) to r + k + r' so that its exact FLOPs count equals DyRA's, the
correction included; r' absorbs every constant and lower-order term.

Counting convention: a multiply-add is 2 FLOPs (a product [m, p] x [p, q] is
2 m p q), and a lone addition, division or square root is 1.  The count
follows Algorithm 1's Inference in the order the paper writes it, per
instance of n tokens:

    line 10  Y_base = (X A_s) V_s^T          2 n c1 r + 2 n r c2
    line 11  L1 = X P_L                      2 n c1 k
    line 12  G = L1^T L1 + lambda I          2 n k^2 + k
             M = L1^T X                      2 n k c1
             P = M W_res                     2 k c1 c2
             R1 = G^-1 P  (Cholesky, then two triangular solves on c2 columns)
                                             k (k + 1)(2k + 1) / 6 + 2 k^2 c2
    line 13  Y = Y_base + L1 R1              2 n k c2 + n c2

The library evaluates the same product in a different but equivalent order
(Q = L1 C^-T, then (Q^T X) W_res); the baseline is matched to the algorithm,
not to one implementation of it.
"""
from __future__ import annotations


def cholesky_flops(k: int) -> int:
    """Column j of C: j multiply-adds and one square root or division per entry,
    k - j entries: sum over j of (k - j)(2 j + 1) = k (k + 1)(2k + 1) / 6."""
    return k * (k + 1) * (2 * k + 1) // 6


def dyra_flops(n: int, c1: int, c2: int, r: int, k: int) -> int:
    """Exact FLOPs of Algorithm 1 Inference for one instance of n tokens."""
    f = 2 * n * c1 * r + 2 * n * r * c2
    if k == 0:
        return f
    f += 2 * n * c1 * k                       # L1
    f += 2 * n * k * k + k                    # G and its ridge
    f += 2 * n * k * c1                       # M
    f += 2 * k * c1 * c2                      # M W_res
    f += cholesky_flops(k) + 2 * k * k * c2   # G^-1 (M W_res)
    f += 2 * n * k * c2 + n * c2              # L1 R1 and the sum
    return f


def static_flops(n: int, c1: int, c2: int, s: int) -> int:
    """Exact FLOPs of the weight-only rank-s product (X A_s) V_s^T for n tokens."""
    return 2 * n * s * (c1 + c2)


def flops_matched_rank(n: int, c1: int, c2: int, r: int, k: int) -> int:
    """Largest static rank s <= min(c1, c2) whose FLOPs do not exceed DyRA's at
    (r, k) for instances of n tokens (the r + k + r' of §2.3)."""
    budget = dyra_flops(n, c1, c2, r, k)
    s = budget // (2 * n * (c1 + c2))
    return int(min(s, min(c1, c2)))
