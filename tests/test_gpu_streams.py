"""Repeatability and stream safety of dyra_forward (through the C ABI).

The plan is immutable after preparation, so forwards that use separate
workspaces and outputs may run at once on different streams.  The kernels
reduce in a fixed order, so the same input gives bitwise the same output on
every call.  Both properties are checked here on a shape that spans several
tiles and instances, with the results also held to the oracle bar.
"""
import numpy as np
import pytest

import oracle as orc
from structured_rank_matmul_amd import dyra, synth

from gpu_util import check_parity, to_device, to_host

pytestmark = pytest.mark.gpu

B, N_TOK, C1, C2, R, K = 6, 150, 256, 384, 64, 32


def test_forward_is_repeatable_and_stream_safe():
    import torch
    W = synth.random_weight(C1, C2, 51, p=0.5)
    Xa = synth.random_matrix(B * N_TOK, C1, 52, "bf16")
    Xb = synth.random_matrix(B * N_TOK, C1, 53, "bf16")
    plan = dyra.dyra_prepare(W, R, K, 0.0, "bf16", 0)
    xa, xb = to_device(Xa), to_device(Xb)

    # one stream: repeated calls agree bit for bit
    ya0 = dyra.dyra_forward(xa, B, N_TOK, plan)
    ya1 = dyra.dyra_forward(xa, B, N_TOK, plan)
    yb0 = dyra.dyra_forward(xb, B, N_TOK, plan)
    torch.cuda.synchronize()
    assert torch.equal(ya0, ya1)

    # both inputs meet the oracle bar, so the comparison below is against
    # correct results
    op = orc.offline_preparation(W.astype(np.float64), R, K, 0.0)
    check_parity(to_host(ya0), orc.inference(Xa.exact, B, N_TOK, op), N_TOK, "bf16", "stream a")
    check_parity(to_host(yb0), orc.inference(Xb.exact, B, N_TOK, op), N_TOK, "bf16", "stream b")

    # two default-priority streams, separate workspaces and outputs, several
    # forwards each in flight at once
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    ya, yb = torch.empty_like(ya0), torch.empty_like(yb0)
    wa, wb = dyra.alloc_workspace(plan, B, N_TOK), dyra.alloc_workspace(plan, B, N_TOK)
    s1.wait_stream(cur)
    s2.wait_stream(cur)
    for _ in range(4):
        dyra.dyra_forward(xa, B, N_TOK, plan, Y=ya, workspace=wa, stream=s1)
        dyra.dyra_forward(xb, B, N_TOK, plan, Y=yb, workspace=wb, stream=s2)
    torch.cuda.synchronize()
    assert torch.equal(ya, ya0)
    assert torch.equal(yb, yb0)

    # a side stream with the output and workspace allocated by the binding:
    # they are marked as used on that stream, so the allocator does not hand
    # their memory to the next allocation before the stream is done with it
    s1.wait_stream(cur)
    outs = [dyra.dyra_forward(xa, B, N_TOK, plan, stream=s1) for _ in range(3)]
    filler = [torch.full_like(ya0, 7.0) for _ in range(3)]  # allocations on the current stream meanwhile
    torch.cuda.synchronize()
    for y in outs:
        assert torch.equal(y, ya0)
    del filler
    plan.close()
