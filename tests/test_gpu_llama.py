"""Parity at the Llama-class MLP shapes: gate 4096 -> 14336 and down 14336 -> 4096,
r = 1024, k = 64, bf16.  Prefill (8 instances of 2048 tokens) and decode (m
sequences of one token, m = 1, 16, 64: the dual form), every instance against
the oracle, each instance and each row on its own (gpu_util.check_parity).

Each layer is prepared once per module: the host factorisation and the oracle's
float64 SVD of a 4096 x 14336 weight take tens of seconds each."""
import numpy as np
import pytest

import oracle as orc
from gpu_util import OWN_ERR_TOL, check_parity, own_error_gap, rel, to_device, to_host
from structured_rank_matmul_amd import dyra, synth

pytestmark = pytest.mark.gpu


def _prepare(lname):
    w = synth.WORKLOADS["llama_prefill"]
    spec = w.layer(lname)
    W, _ = synth.make_weight(w, spec)
    plan = dyra.dyra_prepare(W, spec.r, spec.k, 0.0, "bf16", 0)
    op = orc.offline_preparation(W.astype(np.float64), spec.r, spec.k, 0.0)
    return w, spec, W, plan, op


@pytest.fixture(scope="module")
def gate():
    w, spec, W, plan, op = _prepare("gate")
    yield w, spec, W, plan, op
    plan.close()


@pytest.fixture(scope="module")
def down():
    w, spec, W, plan, op = _prepare("down")
    yield w, spec, W, plan, op
    plan.close()


def _check(w, spec, W, plan, op, X, B, n, sample, label):
    import torch
    Y = dyra.dyra_forward(to_device(X), B, n, plan)
    torch.cuda.synchronize()
    y = to_host(Y)
    rows = np.concatenate([np.arange(b * n, (b + 1) * n) for b in sample])
    Xs = X.exact[rows]
    ref = orc.inference(Xs, len(sample), n, op)
    exact = Xs @ W.astype(np.float64)
    assert np.isfinite(y).all()
    err, worst_inst, worst_row = check_parity(y[rows], ref, n, "bf16", label)
    gap = own_error_gap(y[rows], ref, exact)
    e_w = rel(orc.weight_only(Xs, op), exact)
    print(f"{label}: parity {err:.3e} (worst instance {worst_inst:.3e}, worst row {worst_row:.3e})  "
          f"own-error gap {gap:.3e}  e_dyra {rel(ref, exact):.4f}  e_weight_only {e_w:.4f}", flush=True)
    assert gap <= OWN_ERR_TOL


def test_llama_prefill_gate(gate):
    w, spec, W, plan, op = gate
    X = synth.make_activations(w, spec)
    _check(w, spec, W, plan, op, X, w.B, w.n, list(range(w.B)), "llama prefill gate")


@pytest.mark.parametrize("m", synth.DECODE_TOKENS)
def test_llama_decode_gate(gate, m):
    w, spec, W, plan, op = gate
    wd = synth.llama_decode(m)
    X = synth.make_activations(wd, spec)
    _check(wd, spec, W, plan, op, X, m, 1, list(range(m)), f"llama decode m={m} gate")


def test_llama_prefill_down(down):
    w, spec, W, plan, op = down
    X = synth.make_activations(w, spec)
    _check(w, spec, W, plan, op, X, w.B, w.n, list(range(w.B)), "llama prefill down")


@pytest.mark.parametrize("m", synth.DECODE_TOKENS)
def test_llama_decode_down(down, m):
    w, spec, W, plan, op = down
    wd = synth.llama_decode(m)
    X = synth.make_activations(wd, spec)
    _check(wd, spec, W, plan, op, X, m, 1, list(range(m)), f"llama decode m={m} down")
