"""Further ALS steps (the §3.3 ablation over the iteration count t; Eq. 4 L
updates between Eq. 5 R updates) and a Gaussian R^(0) (§2.2 Fig. 2, Appendix
E.3), through the C ABI (dyra_prepare_ex), against the float64 oracle."""
import numpy as np
import pytest

import oracle as orc
from structured_rank_matmul_amd import dyra, synth

from gpu_util import OWN_ERR_TOL, check_parity, own_error_gap, rel, to_device, to_host

pytestmark = pytest.mark.gpu

CASES = [
    # B, n, c1, c2, r, k, lambda, dtype, half_steps, gaussian R0
    (4, 60, 192, 320, 40, 16, 0.0, "bf16", 3, False),    # t 1.5: ends on an L update
    (4, 60, 192, 320, 40, 16, 0.0, "bf16", 4, True),     # t 2 from a Gaussian R0
    (3, 150, 256, 288, 64, 32, 0.1, "f32", 4, True),     # ridge, float32
    (2, 100, 128, 224, 24, 40, 0.0, "f32", 5, False),    # k = 40 padded to 48
    (5, 37, 128, 160, 16, 12, 0.05, "bf16", 6, True),    # k = 12 padded to 16, instances straddle tiles
    (3, 201, 256, 512, 64, 64, 0.0, "bf16", 4, False),   # full correction width
]


def _r0(k, c2, seed):
    return synth.random_matrix(k, c2, seed, "f32")


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}n{c[1]}-{c[2]}x{c[3]}-r{c[4]}k{c[5]}-lam{c[6]}-{c[7]}"
                                                     f"-h{c[8]}{'-gauss' if c[9] else ''}")
def test_als_steps_match_oracle(case):
    import torch
    B, n, c1, c2, r, k, lam, dtype, hs, gauss = case
    W = synth.random_weight(c1, c2, 71)
    X = synth.random_matrix(B * n, c1, 72, dtype)
    X = synth.round_activations(X.exact * np.exp(synth.random_matrix(1, c1, 73, "f32").exact), dtype)
    R0 = _r0(k, c2, 74) if gauss else None
    plan = dyra.dyra_prepare_ex(W, r, k, lam, dtype, 0, R0=None if R0 is None else R0.data, als_half_steps=hs)
    names = dyra.stage_names(plan, n)
    assert names[0] == "left" and names[-1] == "output"
    assert names.count("als_lupdate") == (hs - 1) // 2 and names.count("right") == hs // 2
    Y = dyra.dyra_forward(to_device(X), B, n, plan)
    torch.cuda.synchronize()
    y = to_host(Y)
    op = orc.offline_preparation(W.astype(np.float64), r, k, lam, R0=None if R0 is None else R0.exact)
    ref = orc.inference(X.exact, B, n, op, half_steps=hs)
    exact = X.exact @ W.astype(np.float64)
    err, _, _ = check_parity(y, ref, n, dtype, f"als {case}")
    gap = own_error_gap(y, ref, exact)
    one = orc.inference(X.exact, B, n, op)
    print(f"als case {case}: parity {err:.3e}  own-error gap {gap:.3e}  e(t) {rel(ref, exact):.4f}  "
          f"e(t=1) {rel(one, exact):.4f}", flush=True)
    assert gap <= OWN_ERR_TOL
    plan.close()


@pytest.mark.parametrize("hs", [3, 4])
def test_als_steps_with_bias_and_alpha(hs):
    import torch
    B, n, c1, c2, r, k = 3, 45, 128, 192, 16, 16
    W = synth.random_weight(c1, c2, 75)
    X = synth.random_matrix(B * n, c1, 76, "bf16")
    bias = synth.random_matrix(1, c2, 77, "bf16", scale=2.0)
    plan = dyra.dyra_prepare_ex(W, r, k, 0.0, "bf16", 0, als_half_steps=hs)
    Y = dyra.dyra_forward_ex(to_device(X), B, n, plan, bias=to_device(bias)[0], alpha=-0.75)
    torch.cuda.synchronize()
    op = orc.offline_preparation(W.astype(np.float64), r, k, 0.0)
    ref = orc.inference(X.exact, B, n, op, bias=bias.exact[0], alpha=-0.75, half_steps=hs)
    check_parity(to_host(Y), ref, n, "bf16", f"als bias/alpha h={hs}")
    plan.close()


def test_als_steps_on_a_vitl_layer():
    """ViT-L qkv (128 x 201 tokens, 1024 -> 3072, r = 256, k = 64) at t = 2,
    sampled instances against the oracle."""
    import torch
    w = synth.WORKLOADS["vitl_block"]
    spec = w.layer("qkv")
    W, _ = synth.make_weight(w, spec)
    X = synth.make_activations(w, spec)
    plan = dyra.dyra_prepare_ex(W, spec.r, spec.k, 0.0, "bf16", 0, als_half_steps=4)
    Y = dyra.dyra_forward(to_device(X), w.B, w.n, plan)
    torch.cuda.synchronize()
    sample = [0, 77, 127]
    rows = np.concatenate([np.arange(b * w.n, (b + 1) * w.n) for b in sample])
    Xs = X.exact[rows]
    op = orc.offline_preparation(W.astype(np.float64), spec.r, spec.k, 0.0)
    ref = orc.inference(Xs, len(sample), w.n, op, half_steps=4)
    y = to_host(Y)[rows]
    exact = Xs @ W.astype(np.float64)
    err, _, _ = check_parity(y, ref, w.n, "bf16", "vitl qkv t=2")
    gap = own_error_gap(y, ref, exact)
    print(f"vitl qkv t=2: parity {err:.3e}  own-error gap {gap:.3e}  e(t=2) {rel(ref, exact):.4f}  "
          f"e(t=1) {rel(orc.inference(Xs, len(sample), w.n, op), exact):.4f}", flush=True)
    assert gap <= OWN_ERR_TOL
    plan.close()


def test_als_steps_reject_the_dual_form_and_bad_counts():
    W = synth.random_weight(64, 96, 78)
    X = synth.random_matrix(8, 64, 79, "bf16")
    plan = dyra.dyra_prepare_ex(W, 8, 16, 0.0, "bf16", 0, als_half_steps=4)
    with pytest.raises(dyra.DyraError) as e:
        dyra.dyra_forward(to_device(X), 8, 1, plan)      # one token per instance: dual form
    assert e.value.status == 2
    plan.close()
    for hs in (1, 9):
        with pytest.raises(dyra.DyraError) as e:
            dyra.dyra_prepare_ex(W, 8, 16, 0.0, "bf16", 0, als_half_steps=hs)
        assert e.value.status == 1
