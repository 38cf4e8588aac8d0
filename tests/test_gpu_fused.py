"""§2.4's fused linear layer through the C ABI (dyra_forward_ex):
Y = X A_s V_s^T + b + alpha L1 R1, against the float64 oracle with the same bias
and alpha, on the primal, dual (fewer tokens than the correction rank) and
static (k = 0) paths, in bf16 and float32."""
import numpy as np
import pytest

import oracle as orc
from structured_rank_matmul_amd import dyra, synth

from gpu_util import check_parity, to_device, to_host

pytestmark = pytest.mark.gpu

FUSED = [
    # B, n, c1, c2, r, k, lambda, dtype, alpha
    (5, 37, 192, 320, 40, 12, 0.0, "bf16", 0.5),     # primal; tiles straddle instances
    (3, 150, 256, 288, 64, 16, 0.0, "f32", -1.5),    # primal, float32, negative weight
    (2, 300, 128, 416, 20, 32, 0.0, "bf16", 0.0),    # alpha 0: static product plus bias
    (16, 1, 256, 320, 40, 16, 0.0, "bf16", 0.75),    # dual form, one token per instance
    (4, 8, 128, 160, 16, 24, 1e-2, "f32", 2.0),      # dual form, n < k, ridge
    (3, 40, 192, 224, 48, 0, 0.0, "bf16", 1.0),      # static path (k = 0) with bias
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: f"B{c[0]}n{c[1]}-{c[2]}x{c[3]}-r{c[4]}k{c[5]}-{c[7]}-a{c[8]}")
def test_forward_ex_bias_alpha(case):
    import torch
    B, n, c1, c2, r, k, lam, dtype, alpha = case
    W = synth.random_weight(c1, c2, 61)
    X = synth.random_matrix(B * n, c1, 62, dtype)
    bias = synth.random_matrix(1, c2, 63, dtype, scale=3.0)
    plan = dyra.dyra_prepare(W, r, k, lam, dtype, 0)
    Y = dyra.dyra_forward_ex(to_device(X), B, n, plan, bias=to_device(bias)[0], alpha=alpha)
    torch.cuda.synchronize()
    op = orc.offline_preparation(W.astype(np.float64), r, k, lam)
    ref = orc.inference(X.exact, B, n, op, bias=bias.exact[0], alpha=alpha)
    err, _, _ = check_parity(to_host(Y), ref, n, dtype, f"fused {case}")
    print(f"fused case {case}: parity {err:.3e}", flush=True)
    plan.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_ex_defaults_equal_forward_bitwise(dtype):
    """No bias and alpha = 1 is Eq. 6: the same kernels, the same bits."""
    import torch
    B, n, c1, c2, r, k = 4, 53, 128, 192, 24, 16
    W = synth.random_weight(c1, c2, 64)
    X = synth.random_matrix(B * n, c1, 65, dtype)
    plan = dyra.dyra_prepare(W, r, k, 0.0, dtype, 0)
    xd = to_device(X)
    Y0 = dyra.dyra_forward(xd, B, n, plan)
    Y1 = dyra.dyra_forward_ex(xd, B, n, plan, bias=None, alpha=1.0)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1)
    plan.close()


def test_forward_ex_rejects_non_finite_alpha():
    W = synth.random_weight(64, 64, 66)
    X = synth.random_matrix(8, 64, 67, "bf16")
    plan = dyra.dyra_prepare(W, 8, 8, 0.0, "bf16", 0)
    for a in (float("nan"), float("inf")):
        with pytest.raises(dyra.DyraError) as e:
            dyra.dyra_forward_ex(to_device(X), 2, 4, plan, alpha=a)
        assert e.value.status == 1
    plan.close()
