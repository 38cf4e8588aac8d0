"""Parity of DyRA with a BLAST static approximation (Appendix B) against the
oracle, through the C ABI (dyra_prepare_blast / dyra_forward[_ex]).

Shapes span several GEMM tiles with ragged rows, instances that straddle
tiles, 1 to 4 blocks per side, BLAST ranks that are not multiples of 32 (the
library pads them), the static-only case, bias and alpha, a ridge term with
fewer tokens than the correction rank, and the ViT-L block at full size on
sampled instances.
"""
import numpy as np
import pytest

import oracle as orc
from structured_rank_matmul_amd import dyra, synth

from gpu_util import OWN_ERR_TOL, check_parity, own_error_gap, rel, to_device, to_host

pytestmark = pytest.mark.gpu

CASES = [
    # B, n, c1, c2, nb, rb, k
    (5, 70, 256, 384, 4, 40, 24),     # rank 40 -> 64 padded; 350 rows: ragged 256-row tiles
    (3, 150, 256, 256, 2, 64, 16),    # instances longer than a 128-row tile
    (2, 201, 288, 192, 3, 20, 32),    # three blocks, 96 x 64 each
    (4, 33, 128, 320, 1, 48, 16),     # one block: a diagonal-coupled low-rank product
    (6, 80, 512, 256, 4, 100, 64),    # k = 64 (four correction slices)
    (3, 90, 384, 256, 4, 64, 16),     # grouped block-row product with K = 96: a short last slice
]


def _run(b, X, B, n, k, lam, dtype, bias=None, alpha=1.0):
    import torch
    plan = dyra.dyra_prepare_blast(b.W, b.U, b.S, b.V, b.nb, k, lam, dtype, 0)
    x = to_device(X)
    if bias is None and alpha == 1.0:
        Y = dyra.dyra_forward(x, B, n, plan)
    else:
        bt = None
        if bias is not None:
            bt = to_device(synth.round_activations(bias[None, :].astype(np.float64), dtype))[0].contiguous()
        Y = dyra.dyra_forward_ex(x, B, n, plan, bias=bt, alpha=alpha)
    torch.cuda.synchronize()
    plan.close()
    return to_host(Y)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES)
def test_blast_forward_matches_oracle(dtype, case):
    B, n, c1, c2, nb, rb, k = case
    print(f"blast case B={B} n={n} {c1}->{c2} nb={nb} rb={rb} k={k} {dtype}", flush=True)
    b = synth.random_blast_weight(c1, c2, nb, rb, 31 + c1 + nb)
    X = synth.random_matrix(B * n, c1, 32 + n, dtype)
    y = _run(b, X, B, n, k, 0.0, dtype)
    op = orc.offline_preparation_blast(b.W, b.U, b.S, b.V, nb, k, 0.0)
    ref = orc.inference(X.exact, B, n, op)
    exact = X.exact @ b.W.astype(np.float64)
    check_parity(y, ref, n, dtype, f"blast B={B} n={n} nb={nb} rb={rb} k={k} {dtype}")
    assert own_error_gap(y, ref, exact) <= OWN_ERR_TOL
    # the correction is doing its job: the result is closer than the static part alone
    assert rel(y, exact) < rel(orc.weight_only(X.exact, op), exact)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_blast_static_only(dtype):
    B, n, c1, c2, nb, rb = 3, 90, 256, 128, 4, 24
    b = synth.random_blast_weight(c1, c2, nb, rb, 41)
    X = synth.random_matrix(B * n, c1, 42, dtype)
    y = _run(b, X, B, n, 0, 0.0, dtype)
    ref = X.exact @ orc.blast_matrix(b.U, b.S, b.V, nb)
    check_parity(y, ref, n, dtype, "blast static only")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_blast_bias_alpha(dtype):
    B, n, c1, c2, nb, rb, k = 4, 60, 256, 256, 2, 32, 16
    b = synth.random_blast_weight(c1, c2, nb, rb, 43)
    X = synth.random_matrix(B * n, c1, 44, dtype)
    bias = synth.random_matrix(1, c2, 45, dtype).exact[0]
    alpha = 0.75
    y = _run(b, X, B, n, k, 0.0, dtype, bias=bias, alpha=alpha)
    op = orc.offline_preparation_blast(b.W, b.U, b.S, b.V, nb, k, 0.0)
    ref = orc.inference(X.exact, B, n, op, bias=bias, alpha=alpha)
    check_parity(y, ref, n, dtype, "blast bias/alpha")


def test_blast_ridge_with_few_tokens():
    # n < k: singular without a ridge term (rejected), solvable with one
    B, n, c1, c2, nb, rb, k = 6, 12, 128, 256, 2, 32, 32
    b = synth.random_blast_weight(c1, c2, nb, rb, 46)
    X = synth.random_matrix(B * n, c1, 47, "bf16")
    plan = dyra.dyra_prepare_blast(b.W, b.U, b.S, b.V, nb, k, 0.0, "bf16", 0)
    with pytest.raises(dyra.DyraError):
        dyra.dyra_forward(to_device(X), B, n, plan)
    plan.close()
    lam = 0.5
    y = _run(b, X, B, n, k, lam, "bf16")
    op = orc.offline_preparation_blast(b.W, b.U, b.S, b.V, nb, k, lam)
    check_parity(y, orc.inference(X.exact, B, n, op), n, "bf16", "blast ridge n < k")


def test_blast_stage_names():
    b = synth.random_blast_weight(128, 128, 2, 16, 48)
    plan = dyra.dyra_prepare_blast(b.W, b.U, b.S, b.V, 2, 16, 0.0, "bf16", 0)
    assert dyra.stage_names(plan, 40) == ["left", "blast_mix", "gram_q", "mprime", "right", "output"]
    plan.close()
    plan = dyra.dyra_prepare_blast(b.W, b.U, b.S, b.V, 2, 0, 0.0, "bf16", 0)
    assert dyra.stage_names(plan, 40) == ["left", "blast_mix", "output"]
    plan.close()


@pytest.mark.parametrize("layer", ["qkv", "fc1", "fc2"])
def test_blast_vitl_block_full_size(layer):
    # the ViT-L block workload (128 x 201 tokens, bf16) with a 4 x 4 BLAST
    # static part of rank 256 and k = 64; three sampled instances checked
    import torch
    w = synth.WORKLOADS["vitl_block"]
    spec = w.layer(layer)
    b = synth.make_blast_weight(w, spec, 4, 256)
    X = synth.make_activations(w, spec)
    print(f"blast vitl_block/{layer}", flush=True)
    plan = dyra.dyra_prepare_blast(b.W, b.U, b.S, b.V, 4, spec.k, 0.0, w.dtype, 0)
    Y = dyra.dyra_forward(to_device(X), w.B, w.n, plan)
    torch.cuda.synchronize()
    plan.close()
    y = to_host(Y)
    idx = [0, 64, 127]
    rows = np.concatenate([np.arange(i * w.n, (i + 1) * w.n) for i in idx])
    Xs = X.exact[rows]
    op = orc.offline_preparation_blast(b.W, b.U, b.S, b.V, 4, spec.k, 0.0)
    ref = orc.inference(Xs, len(idx), w.n, op)
    exact = Xs @ b.W.astype(np.float64)
    err, _, _ = check_parity(y[rows], ref, w.n, "bf16", f"blast vitl {layer}")
    gap = own_error_gap(y[rows], ref, exact)
    print(f"  parity {err:.3e} gap {gap:.3e} e_dyra {rel(ref, exact):.4f} "
          f"e_weight {rel(orc.weight_only(Xs, op), exact):.4f}", flush=True)
    assert gap <= OWN_ERR_TOL
