"""The FLOPs-matched static baseline (§2.3 FLOPs-Matched Comparison, Appendix
E.4) through the C ABI: the weight-only truncated SVD at the rank whose exact
FLOPs equal DyRA's (the k = 0 path), against the oracle's static product at
that rank, on workload shapes and sampled instances."""
import numpy as np
import pytest

import oracle as orc
from structured_rank_matmul_amd import costs, dyra, synth

from gpu_util import OWN_ERR_TOL, check_parity, own_error_gap, rel, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wname,lname,sample", [("vitb_fc1", "fc1", [0, 31, 63]), ("linear384_fp32", "linear", None),
                                                ("vitl_block", "fc2", [5, 127])])
def test_flops_matched_static_matches_oracle(wname, lname, sample):
    import torch
    w = synth.WORKLOADS[wname]
    spec = w.layer(lname)
    s = costs.flops_matched_rank(w.n, spec.c1, spec.c2, spec.r, spec.k)
    W, _ = synth.make_weight(w, spec)
    X = synth.make_activations(w, spec)
    plan = dyra.dyra_prepare(W, s, 0, 0.0, w.dtype, 0)
    assert dyra.stage_names(plan, w.n) == ["left", "output"]
    Y = dyra.dyra_forward(to_device(X), w.B, w.n, plan)
    torch.cuda.synchronize()
    idx = range(w.B) if sample is None else sample
    rows = np.concatenate([np.arange(b * w.n, (b + 1) * w.n) for b in idx])
    Xs = X.exact[rows]
    op = orc.offline_preparation(W.astype(np.float64), s, 0)
    ref = orc.weight_only(Xs, op)
    y = to_host(Y)[rows]
    exact = Xs @ W.astype(np.float64)
    err, _, _ = check_parity(y, ref, w.n, w.dtype, f"{wname}/{lname} static rank {s}")
    gap = own_error_gap(y, ref, exact)
    print(f"{wname}/{lname}: FLOPs-matched static rank {s}: parity {err:.3e}  own-error gap {gap:.3e}  "
          f"e_static {rel(ref, exact):.4f}", flush=True)
    assert gap <= OWN_ERR_TOL
    plan.close()
