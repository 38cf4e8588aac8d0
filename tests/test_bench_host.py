"""Host-side pieces of bench.py: workload lookup, the dual-form rule and the
algorithmic FLOP and byte counts its roofline record uses."""
import dataclasses

import pytest

import bench
from structured_rank_matmul_amd import synth


def test_workload_lookup():
    assert synth.workload("vitl_block") is synth.WORKLOADS["vitl_block"]
    w = synth.workload("llama_decode_m16")
    assert (w.B, w.n) == (16, 1)
    assert [s.name for s in w.layers] == [s.name for s in synth.WORKLOADS["llama_prefill"].layers]
    for bad in ("llama_decode_m0", "llama_decode_mx", "nope"):
        with pytest.raises(KeyError):
            synth.workload(bad)


def test_dual_form_rule():
    # the library takes the n x n form at n <= 16 tokens or n < k
    spec = synth.WORKLOADS["vitl_block"].layers[0]          # k = 64
    assert bench.dual_form(spec, 1) and bench.dual_form(spec, 16) and bench.dual_form(spec, 63)
    assert not bench.dual_form(spec, 64) and not bench.dual_form(spec, 201)
    small_k = dataclasses.replace(spec, k=8)
    assert bench.dual_form(small_k, 16) and not bench.dual_form(small_k, 17)
    assert not bench.dual_form(dataclasses.replace(spec, k=0), 1)   # k = 0: static path


def test_decode_counts():
    # decode FLOPs: 2N c1 (r+k) + 2N c1 c2 + 2N r c2 plus the n x n terms
    spec = synth.workload("llama_decode_m1").layers[0]
    N = 1
    expect = 2 * N * spec.c1 * (spec.r + spec.k) + 2 * N * spec.c1 * spec.c2 + 2 * N * spec.r * spec.c2
    got = bench.dyra_flops(spec, 1, 1)
    assert expect <= got <= expect * 1.001
    # the dominant bytes are W_res and V_s streamed once
    by = bench.stage_bytes(spec, 1, 1, 2)["decode_output"]
    assert by >= 2 * (spec.c1 * spec.c2 + spec.c2 * spec.r)
    # the primal count is the stage sum of its five kernels
    v = synth.WORKLOADS["vitl_block"].layers[1]
    fl = bench.stage_flops(v, 128, 201)
    assert bench.dyra_flops(v, 128, 201) == sum(fl[s] for s in bench.PRIMAL_STAGES)


def test_cpu_baseline_cycles_to_budget():
    # a batch that finishes well inside the budget is taken again from the first
    # instance, at most 8 passes; the rate counts every instance done
    import types

    import numpy as np

    import oracle as orc
    W = np.random.default_rng(3).standard_normal((16, 24))
    plan = orc.offline_preparation(W, 4, 2, 0.0)
    X = np.random.default_rng(4).standard_normal((2 * 5, 16))
    w = types.SimpleNamespace(B=2, n=5, layers=[None])
    r = bench.cpu_baseline(w, [plan], [X], budget_s=60.0)
    assert r["kind"] == "oracle" and r["value"] > 0
    assert r["sample"].startswith("8.00 passes over the 2 instances (80 tokens)")
    r = bench.cpu_baseline(w, [plan], [X], budget_s=0.0)
    assert r["sample"].startswith("1 of 2 instances (5 tokens)")


def test_oracle_leg_fills_parity_and_baseline():
    # library outputs equal to the oracle's on the sampled rows: parity 0, the
    # own-error gap 0, and the oracle's error and the static part's filled in
    import types

    import numpy as np

    import oracle as orc
    spec = synth.LayerSpec("t", 64, 96, r=8, k=4, p=0.7, kaiming=False, x_kind="gaussian")
    w = types.SimpleNamespace(B=3, n=10, layers=[spec])
    W = synth.random_weight(64, 96, 5)
    X = synth.random_matrix(30, 64, 6, "f32")
    sample = [0, 1, 2]
    rows = np.arange(30)
    op = orc.offline_preparation(W.astype(np.float64), 8, 4, 0.0)
    y_rows = orc.inference(X.exact[rows], 3, 10, op)
    layers = [dict(spec=spec, W=W, X=X, y_rows=y_rows)]
    parity = {"t": {"e_dyra": 0.0}, "sample_instances": sample}
    args = types.SimpleNamespace(no_parity=False, cpu_budget=0.0)
    cpu = bench.oracle_leg(w, layers, None, [], parity, args)
    assert parity["t"]["rel_fro_vs_oracle"] == 0.0
    assert parity["worst_rel_fro"] == 0.0 and parity["worst_own_error_gap"] == 0.0
    exact = X.exact @ W.astype(np.float64)
    assert abs(parity["t"]["e_dyra_oracle"] - bench.rel_err(y_rows, exact)) < 1e-5
    assert parity["t"]["e_weight_only"] >= parity["t"]["e_dyra_oracle"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0


@pytest.mark.parametrize("wname", ["vitl_block", "whisper_mlp", "llama_prefill", "llama_decode_m16"])
def test_algorithmic_bytes_count_each_layer_array_once(wname):
    # over the stages of one layer call, the algorithmic bytes are X, Y and
    # the plan's factors ([A_s | P_L], V_s, W_res), each exactly once; the
    # intermediates appear only in the operand bytes
    w = synth.workload(wname)
    for spec in w.layers:
        es = 2
        N = w.B * w.n
        stages = bench.DUAL_STAGES if bench.dual_form(spec, w.n) else bench.PRIMAL_STAGES
        by = bench.stage_bytes(spec, w.B, w.n, es)
        total = sum(by[s] for s in stages)
        c1, c2, r, k = spec.c1, spec.c2, spec.r, spec.k
        assert total == es * (N * c1 + N * c2 + (r + k) * c1 + c2 * r + c1 * c2)
        op = bench.stage_operand_bytes(spec, w.B, w.n, es)
        assert all(op[s] >= by[s] for s in stages)

