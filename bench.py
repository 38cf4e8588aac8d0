#!/usr/bin/env python3
"""Benchmark of the DyRA layer forward on one MI355X.

One step = dyra_forward over every layer of the workload (default: the
DINOv3-ViT-L-like block, qkv 1024->3072, fc1 1024->4096, fc2 4096->1024 on
128 images x 201 tokens, r = 256, k = 64, bf16) with inputs resident in HBM.
Prints one JSON line with tokens/s, the speedup over a dense bf16 GEMM of the
same shapes (hipBLASLt through torch), the relative Frobenius error against
the float64 oracle on sampled instances, the roofline of the dominant kernel
and the oracle's own throughput on the host cores.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s
PEAK_FP32 = 157.3e12    # MI355X fp32 matrix, FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E, B/s


def stage_flops(spec, B, n):
    """Algorithmic FLOPs of each kernel for one layer call: the primal path's
    stages and the dual (n x n) form's, keyed by the library's stage names."""
    N = B * n
    c1, c2, r, k = spec.c1, spec.c2, spec.r, spec.k
    return {
        # one pass over X gives X A_s and L1 = X P_L
        "left": 2.0 * N * c1 * (r + k),
            # G = L1^T L1 and Q = L1 C^-T per instance
        "gram_q": 2.0 * N * k * k + 1.0 * N * k * k,
        "mprime": 2.0 * N * k * c1,
        "right": 2.0 * B * k * c1 * c2,
        "output": 2.0 * N * (r + k) * c2,
        # dual form: [X A_s | L1], the n x n Gram L1 L1^T per instance, then
        # Y = T_s V_s^T + blockdiag(C) X W_res with W_res streamed once
        "decode_project": 2.0 * N * c1 * (r + k),
        "decode_coef": 2.0 * N * n * k,
        "decode_output": 2.0 * N * r * c2 + 2.0 * N * c1 * c2 + 2.0 * N * n * c2,
    }


def stage_bytes(spec, B, n, es):
    """Algorithmic HBM bytes of each kernel for one layer call.  The layer's
    algorithmic bytes are X, Y and the plan's factors ([A_s | P_L], V_s,
    W_res), each moved once in the element size es; each is counted at the
    kernel that must move it.  The intermediates (T = [X A_s | L1], Q, M', R1)
    and a second read of X are practical extra traffic, reported by
    stage_operand_bytes and the counters, not here."""
    N = B * n
    c1, c2, r, k = spec.c1, spec.c2, spec.r, spec.k
    return {
        "left": es * (N * c1 + (r + k) * c1),
        "gram_q": 0,
        "mprime": 0,
        "right": es * (c1 * c2),
        "output": es * (c2 * r + N * c2),
        "decode_project": es * (N * c1 + (r + k) * c1),
        "decode_coef": 0,
        "decode_output": es * (c2 * r + c1 * c2 + N * c2),
    }


def stage_operand_bytes(spec, B, n, es):
    """Bytes each kernel reads and writes at the least, intermediates
    included (every operand read once, every result written once)."""
    N = B * n
    c1, c2, r, k = spec.c1, spec.c2, spec.r, spec.k
    return {
        "left": es * (N * c1 + (r + k) * c1 + N * (r + k)),
        "gram_q": es * (3 * N * k),
        "mprime": es * (N * c1 + N * k + B * k * c1),
        "right": es * (B * k * c1 + c1 * c2 + B * k * c2),
        "output": es * (N * (r + k) + c2 * r + B * k * c2 + N * c2),
        "decode_project": es * (N * c1 + (r + k) * c1 + N * (r + k)),
        "decode_coef": es * (N * k),
        "decode_output": es * (N * r + c2 * r + c1 * c2 + N * c1 + N * c2),
    }


def dual_form(spec, n):
    """True when the library takes the n x n dual form for n tokens per instance
    (at most 16 tokens, or fewer tokens than the correction rank)."""
    return spec.k > 0 and (n <= 16 or n < spec.k)


# kernel behind each stage of the primal path (for the roofline record)
STAGE_KERNEL = {
    "left": "gemm_kernel (T = X [A_s | P_L])",
    "gram_q": "gram_chol_kernel (+ q_apply_kernel for n > 256 or k > 64)",
    "mprime": "mprime_tr_kernel",
    "right": "gemm_kernel (R1 = M' W_res, R1t store)",
    "output": "gemm_kernel with correction slices (Y = T_s V_s^T + Q R1_b)",
    "decode_project": "decode_project_kernel ([X A_s | L1], split-K)",
    "decode_coef": "decode_coef_kernel (n x n Gram and eigen-solve per instance)",
    "decode_output": "decode_z_kernel + decode_output_kernel (Y = T_s V_s^T + blockdiag(C) X W_res)",
}
TRAFFIC_FILE = {"output": "profiles/output_gemm_{workload}_traffic.txt"}


PRIMAL_STAGES = ("left", "gram_q", "mprime", "right", "output")
DUAL_STAGES = ("decode_project", "decode_coef", "decode_output")


def dyra_flops(spec, B, n):
    fl = stage_flops(spec, B, n)
    return sum(fl[st] for st in (DUAL_STAGES if dual_form(spec, n) else PRIMAL_STAGES))


def rel_err(a, b) -> float:
    """||a - b||_F / ||b||_F in float64 (the relative Frobenius error of the metric)."""
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


def time_loop(fn, steps, warmup, stream, per_step=False):
    """Mean seconds per step over `steps` timed steps (events on `stream`);
    with per_step, also the list of single-step durations."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if per_step else 2)]
    evs[0].record(stream)
    for i in range(steps):
        fn()
        if per_step:
            evs[i + 1].record(stream)
    if not per_step:
        evs[1].record(stream)
    torch.cuda.synchronize()
    total = evs[0].elapsed_time(evs[-1]) / 1e3
    if not per_step:
        return total / steps
    return total / steps, [evs[i].elapsed_time(evs[i + 1]) / 1e3 for i in range(steps)]


def cpu_baseline(workload, plans_orc, X_host, budget_s):
    """Oracle inference, instance by instance through every layer, until ~budget_s of CPU time.

    When the whole batch takes less than the budget the instances are taken again
    from the first, so that the sample is long enough to time; at most 8 passes."""
    import oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    n = workload.n
    done, t_total = 0, 0.0
    while done < 8 * workload.B:
        b = done % workload.B
        t0 = time.perf_counter()
        for li, spec in enumerate(workload.layers):
            Xb = X_host[li][b * n:(b + 1) * n]
            orc.inference(Xb, 1, n, plans_orc[li])
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    tokens = done * n
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:  # pragma: no cover
        pass
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    if done <= workload.B:
        what = f"{done} of {workload.B} instances"
    else:
        what = f"{done / workload.B:.2f} passes over the {workload.B} instances"
    return {"value": tokens / t_total, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas, "numpy": np.__version__,
            "sample": f"{what} ({tokens} tokens) through all {len(workload.layers)} "
                      f"layers, float64 numpy, {t_total:.1f} s"}


def oracle_leg(w, layers, blast, blast_legs, parity, args):
    """The CPU leg: the oracle's Offline Preparation per layer, its Inference
    on the sampled instances compared with the library's outputs (filled into
    the parity and BLAST records), then the timed CPU baseline."""
    import oracle as orc
    n = w.n
    plans = [orc.offline_preparation(L["W"].astype(np.float64), L["spec"].r, L["spec"].k, 0.0) for L in layers]
    if not args.no_parity and parity:
        sample = parity["sample_instances"]
        rows = np.concatenate([np.arange(b * n, (b + 1) * n) for b in sample])
        worst, worst_gap = 0.0, None

        def compare(rec, y, Xs, W, op):
            nonlocal worst, worst_gap
            ref = orc.inference(Xs, len(sample), n, op)
            exact = Xs @ W.astype(np.float64)
            err, e_gpu, e_orc = rel_err(y, ref), rel_err(y, exact), rel_err(ref, exact)
            rec.update({"rel_fro_vs_oracle": float(f"{err:.3e}"), "e_dyra_oracle": round(e_orc, 5),
                        "e_weight_only": round(rel_err(orc.weight_only(Xs, op), exact), 5)})
            worst = max(worst, err)
            # where the method is exact (one token with lambda = 0: the
            # correction reaches X W) the relative gap is undefined; parity
            # against the oracle is the measure there
            if e_orc > 1e-9:
                gap = abs(e_gpu - e_orc) / e_orc
                worst_gap = gap if worst_gap is None else max(worst_gap, gap)

        for L, op in zip(layers, plans):
            compare(parity[L["spec"].name], L["y_rows"], L["X"].exact[rows], L["W"], op)
        for G in blast_legs:
            if "y_rows" not in G:
                continue
            bw = G["bw"]
            op = orc.offline_preparation_blast(bw.W, bw.U, bw.S, bw.V, bw.nb, G["spec"].k, 0.0)
            compare(blast["layers"][G["spec"].name], G["y_rows"], G["X"].exact[rows], bw.W, op)
        parity["worst_rel_fro"] = float(f"{worst:.3e}")
        parity["worst_own_error_gap"] = None if worst_gap is None else float(f"{worst_gap:.3e}")
    return cpu_baseline(w, plans, [L["X"].exact for L in layers], args.cpu_budget)


def blast_record(w, layers, args, stream, reps, t_dense, log):
    """DyRA with a BLAST W_hat: per-layer plans on BLAST-structured stand-in
    weights, the whole-step time, the per-stage times, the mix kernel's
    bandwidth, and parity and error on sampled instances."""
    import torch
    from structured_rank_matmul_amd import dyra, synth
    B, n, N = w.B, w.n, w.B * w.n
    nb = args.blast_blocks
    es = 2 if w.dtype == "bf16" else 4
    legs = []
    for L in layers:
        spec = L["spec"]
        bw = synth.make_blast_weight(w, spec, nb, spec.r)
        t0 = time.perf_counter()
        plan = dyra.dyra_prepare_blast(bw.W, bw.U, bw.S, bw.V, nb, spec.k, 0.0, w.dtype, 0)
        log(f"prepared BLAST {spec.name} in {time.perf_counter() - t0:.1f} s")
        legs.append(dict(spec=spec, bw=bw, plan=plan, ws=dyra.alloc_workspace(plan, B, n),
                         y=torch.empty_like(L["y"]), xd=L["xd"], X=L["X"]))

    def step():
        for G in legs:
            dyra.dyra_forward(G["xd"], B, n, G["plan"], G["y"], G["ws"], stream)

    t_blast = time_loop(step, args.steps, args.warmup, stream)
    rec = {"blocks": nb, "ms_per_step": round(t_blast * 1e3, 4), "speedup_vs_dense": round(t_dense / t_blast, 4),
           "layers": {}}
    mix_bytes, mix_t = 0.0, 0.0
    sample = [0, B // 2, B - 1]
    rows = np.concatenate([np.arange(b * n, (b + 1) * n) for b in sample])
    for G in legs:
        spec = G["spec"]
        names = dyra.stage_names(G["plan"], n)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        acc = np.zeros(len(names))
        for it in range(reps + 1):
            dyra.dyra_forward_timed(G["xd"], B, n, G["plan"], G["y"], G["ws"], evs, stream)
            torch.cuda.synchronize()
            if it:
                acc += [evs[i].elapsed_time(evs[i + 1]) / 1e3 for i in range(len(names))]
        per = {nm: acc[i] / reps for i, nm in enumerate(names)}
        rbp = -(-spec.r // 32) * 32
        mix_bytes += 2.0 * N * nb * rbp * es          # Z read, H written
        mix_t += per["blast_mix"]
        lrec = {"rank": spec.r, "k": spec.k, "stage_us": {k_: round(v * 1e6, 2) for k_, v in per.items()}}
        if not args.no_parity:
            Xs = G["X"].exact[rows]
            G["y_rows"] = G["y"].float().cpu().numpy().astype(np.float64)[rows]
            lrec["e_dyra"] = round(rel_err(G["y_rows"], Xs @ G["bw"].W.astype(np.float64)), 5)
        rec["layers"][spec.name] = lrec
        log(f"BLAST {spec.name}: " + "  ".join(f"{k_} {v * 1e6:.1f}us" for k_, v in per.items()))
        G["plan"].close()
    rec["blast_mix_gbps"] = round(mix_bytes / mix_t / 1e9, 1)
    rec["sample_instances"] = sample
    return rec, legs


def solve_scaling_record(w, layers, args, stream, log):
    """The two SPD solves of §2.4 side by side as the correction rank and the
    number of instances grow: stage time of the Cholesky solve (gram_q) and of
    the Newton-Schulz one (ns_factor + ns_apply, ns_iters steps), and the whole
    layer call, on the first layer's weight with n = 320 tokens per instance
    (rows of the workload's own activations) and B = 1, 8, 64."""
    import torch
    from structured_rank_matmul_amd import dyra
    L = layers[0]
    spec = L["spec"]
    n = 320
    iters = args.ns_scaling_iters
    rec = {"layer": spec.name, "tokens_per_instance": n, "ns_iters": iters, "points": []}
    for k in (64, 128, 256):
        if spec.r + k > min(spec.c1, spec.c2):
            continue
        plans = {"cholesky": dyra.dyra_prepare(L["W"], spec.r, k, 0.0, w.dtype, 0),
                 "newton_schulz": dyra.dyra_prepare_ex(L["W"], spec.r, k, 0.0, w.dtype, 0, ns_iters=iters)}
        for B in (1, 8, 64):
            if B * n > w.B * w.n:
                continue
            xd = L["xd"][:B * n]
            y = torch.empty((B * n, spec.c2), dtype=xd.dtype, device=xd.device)
            pt = {"k": k, "instances": B}
            for name, plan in plans.items():
                ws = dyra.alloc_workspace(plan, B, n)
                names = dyra.stage_names(plan, n)
                evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
                acc = np.zeros(len(names))
                reps = 5
                for it in range(reps + 1):
                    dyra.dyra_forward_timed(xd, B, n, plan, y, ws, evs, stream)
                    torch.cuda.synchronize()
                    if it:
                        acc += [evs[i].elapsed_time(evs[i + 1]) / 1e3 for i in range(len(names))]
                per = {nm: acc[i] / reps for i, nm in enumerate(names)}
                solve = sum(v for nm, v in per.items() if nm in ("gram_q", "ns_factor", "ns_apply"))
                pt[name] = {"solve_us": round(solve * 1e6, 2), "layer_us": round(sum(per.values()) * 1e6, 2)}
            rec["points"].append(pt)
            log(f"solve scaling k={k} B={B}: cholesky {pt['cholesky']['solve_us']} us, "
                f"newton-schulz {pt['newton_schulz']['solve_us']} us")
        for plan in plans.values():
            plan.close()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="vitl_block")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time on the host")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-flops-matched", action="store_true",
                    help="skip the FLOPs-matched static baseline (a second prepare and timing per layer)")
    ap.add_argument("--no-als-steps", action="store_true",
                    help="skip the t = 1.5 / t = 2 ALS measurement (two more prepares and timings per layer)")
    ap.add_argument("--no-ns", action="store_true",
                    help="skip the Newton-Schulz SPD-solve measurement (two more prepares and timings per layer)")
    ap.add_argument("--no-blast", action="store_true",
                    help="skip the BLAST static-approximation measurement (a second weight and plan per layer)")
    ap.add_argument("--blast-blocks", type=int, default=4, help="BLAST blocks per side")
    ap.add_argument("--no-solve-scaling", action="store_true",
                    help="skip the Cholesky vs Newton-Schulz solve record over k = 64, 128, 256 and B = 1, 8, 64")
    ap.add_argument("--ns-scaling-iters", type=int, default=12, help="Newton-Schulz steps in that record")
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run three forward steps and a calibration copy only (for rocprofv3 --pmc runs)")
    ap.add_argument("--layers", default="", help="with --traffic-probe: comma-separated layer names to run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the DyRA layer path here is a "
              f"single-GPU kernel path and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    import torch.nn.functional as F

    from structured_rank_matmul_amd import costs, dyra, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.workload(args.workload)
    if args.layers:
        # a subset of the workload's layers (profiling runs only: the bench
        # line's step is every layer)
        keep = [x for x in args.layers.split(",") if x]
        w = dataclasses.replace(w, layers=tuple(spec for spec in w.layers if spec.name in keep))
        if not args.traffic_probe:
            ap.error("--layers is for --traffic-probe runs only")
    dual = any(dual_form(spec, w.n) for spec in w.layers)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    B, n, N = w.B, w.n, w.B * w.n
    log = (lambda *a: print(*a, file=sys.stderr, flush=True)) if args.verbose else (lambda *a: None)

    layers = []
    for spec in w.layers:
        W, _ = synth.make_weight(w, spec)
        X = synth.make_activations(w, spec)
        t0 = time.perf_counter()
        plan = dyra.dyra_prepare(W, spec.r, spec.k, 0.0, w.dtype, 0)
        log(f"prepared {spec.name} in {time.perf_counter() - t0:.1f} s")
        if w.dtype == "bf16":
            xd = torch.from_numpy(np.ascontiguousarray(X.data).view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            xd = torch.from_numpy(X.data).to(dev)
        Wd = torch.from_numpy(W).to(dev).to(tdt)           # [c1, c2]
        Wt = Wd.t().contiguous()                             # [c2, c1], nn.Linear layout
        layers.append(dict(spec=spec, W=W, X=X, plan=plan, xd=xd, Wd=Wd.contiguous(), Wt=Wt,
                           y=torch.empty((N, spec.c2), dtype=tdt, device=dev),
                           yd=torch.empty((N, spec.c2), dtype=tdt, device=dev),
                           ws=dyra.alloc_workspace(plan, B, n)))
    stream = torch.cuda.current_stream()

    def dyra_step():
        for L in layers:
            dyra.dyra_forward(L["xd"], B, n, L["plan"], L["y"], L["ws"], stream)

    def dense_linear():
        for L in layers:
            torch.matmul(L["xd"], L["Wd"], out=L["yd"])

    def dense_nt():
        for L in layers:
            F.linear(L["xd"], L["Wt"])

    def dense_ref():
        for L in layers:
            dyra.dyra_dense_ref(L["xd"], L["Wt"], L["yd"], stream)

    if args.traffic_probe:
        # three forwards, then a plain copy of known size that calibrates the
        # FETCH_SIZE / WRITE_SIZE counters (torch.neg: reads and writes COPY bytes)
        for _ in range(3):
            dyra_step()
        copy_bytes = 1 << 30
        src = torch.ones(copy_bytes // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": True, "copy_bytes": copy_bytes, "workload": w.name}))
        return

    t_dyra, step_times = time_loop(dyra_step, args.steps, args.warmup, stream, per_step=True)
    t_dense_nn = time_loop(dense_linear, args.steps, args.warmup, stream)
    t_dense_nt = time_loop(dense_nt, args.steps, args.warmup, stream)
    t_dense = min(t_dense_nn, t_dense_nt)
    t_dense_ref = time_loop(dense_ref, max(5, args.steps // 5), 2, stream)
    log(f"t_dyra {t_dyra * 1e6:.1f} us  dense nn {t_dense_nn * 1e6:.1f} us  nt {t_dense_nt * 1e6:.1f} us  "
        f"dense_ref {t_dense_ref * 1e6:.1f} us")

    # ---- achievable peaks on this GPU, for context beside the published ones:
    # a streaming copy (reads and writes 1 GiB) and a large hipBLASLt bf16 GEMM
    copy_n = (1 << 30) // 2
    src = torch.ones(copy_n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    t_copy = time_loop(lambda: dst.copy_(src), 10, 3, stream)
    del src, dst
    ga = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    gb = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    gc = torch.empty_like(ga)
    t_gemm = time_loop(lambda: torch.matmul(ga, gb, out=gc), 10, 3, stream)
    del ga, gb, gc
    achievable = {"copy_gbs": round(2.0 * copy_n * 2 / t_copy / 1e9, 1),
                  "gemm_bf16_tflops": round(2.0 * 8192 ** 3 / t_gemm / 1e12, 1),
                  "copy": "torch copy_ of 1 GiB bf16 (read + write)", "gemm": "torch.matmul 8192^3 bf16"}
    log(f"achievable: copy {achievable['copy_gbs']} GB/s, bf16 GEMM {achievable['gemm_bf16_tflops']} TFLOP/s")

    # ---- per-kernel durations with events on the launch stream
    reps = max(5, args.steps // 5)
    stage_time, stage_fl = {}, {}
    for L in layers:
        names = dyra.stage_names(L["plan"], n)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        acc = np.zeros(len(names))
        for it in range(reps + 1):
            dyra.dyra_forward_timed(L["xd"], B, n, L["plan"], L["y"], L["ws"], evs, stream)
            torch.cuda.synchronize()
            if it == 0:
                continue
            acc += [evs[i].elapsed_time(evs[i + 1]) / 1e3 for i in range(len(names))]
        fl = stage_flops(L["spec"], B, n)
        per = {}
        for i, nm in enumerate(names):
            d = acc[i] / reps
            per[nm] = d
            stage_time[nm] = stage_time.get(nm, 0.0) + d
            stage_fl[nm] = stage_fl.get(nm, 0.0) + fl.get(nm, 0.0)
        L["stages"] = per
        log(f"{L['spec'].name}: " + "  ".join(f"{k} {v * 1e6:.1f}us" for k, v in per.items()))
    # ---- roofline of the dominant kernel: its algorithmic FLOPs and bytes
    # per launch (the layer's X, Y and factors counted at the kernel that must
    # move them) against the MFMA and HBM peaks; the larger ideal time is the
    # bound.  The bytes it moves including intermediates are reported beside.
    dom = max(stage_time, key=stage_time.get)
    es = 2 if w.dtype == "bf16" else 4
    launches = len(layers)
    dom_fl = sum(stage_flops(L["spec"], B, n)[dom] for L in layers)
    dom_by = sum(stage_bytes(L["spec"], B, n, es)[dom] for L in layers)
    dom_op = sum(stage_operand_bytes(L["spec"], B, n, es)[dom] for L in layers)
    peak = PEAK_BF16 if w.dtype == "bf16" else PEAK_FP32
    t_dom = stage_time[dom]
    if dom_by / PEAK_HBM > dom_fl / peak:
        bound, achieved, pk, unit = "hbm", dom_by / t_dom / 1e9, PEAK_HBM / 1e9, "GB/s"
    else:
        bound, achieved, pk, unit = "mfma", dom_fl / t_dom / 1e12, peak / 1e12, "TFLOP/s"
    traffic = None
    if dom in TRAFFIC_FILE:
        from structured_rank_matmul_amd import profiling
        traffic = profiling.read_traffic(os.path.join(ROOT, TRAFFIC_FILE[dom].format(workload=w.name)))
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": pk, "unit": unit,
                "frac": round(achieved / pk, 4),
                "traffic": None if traffic is None else round(traffic, 0),
                "kernel": STAGE_KERNEL.get(dom, dom), "stage": dom, "launches_per_step": launches,
                "avg_launch_us": round(t_dom / launches * 1e6, 2),
                "algorithmic_bytes_per_launch": round(dom_by / launches, 0),
                "algorithmic_flops_per_launch": round(dom_fl / launches, 0),
                "operand_bytes_per_launch": round(dom_op / launches, 0),
                "mfma_frac": round(dom_fl / t_dom / peak, 4),
                "hbm_frac": round(dom_by / t_dom / PEAK_HBM, 4),
                "frac_of_achievable": round(achieved / (achievable["copy_gbs"] if bound == "hbm"
                                                        else achievable["gemm_bf16_tflops"]), 4)
                if w.dtype == "bf16" or bound == "hbm" else None}
    # every stage on the same accounting (summed over the step's launches)
    stage_roofline = {}
    for nm, t in stage_time.items():
        fl = sum(stage_flops(L["spec"], B, n).get(nm, 0.0) for L in layers)
        by = sum(stage_bytes(L["spec"], B, n, es).get(nm, 0.0) for L in layers)
        b_ = "hbm" if by / PEAK_HBM > fl / peak else "mfma"
        stage_roofline[nm] = {"bound": b_, "us_per_step": round(t * 1e6, 2),
                              "frac": round((by / PEAK_HBM if b_ == "hbm" else fl / peak) / t, 4)}

    # ---- the metric's error on sampled instances: ||Y - X W|| / ||X W|| with
    # the exact product in float64 (the oracle comparison is made in the CPU
    # leg below)
    parity = {}
    if not args.no_parity:
        sample = [0, B // 2, B - 1]
        rows = np.concatenate([np.arange(b * n, (b + 1) * n) for b in sample])
        for L in layers:
            L["y_rows"] = L["y"].float().cpu().numpy().astype(np.float64)[rows]
            exact = L["X"].exact[rows] @ L["W"].astype(np.float64)
            parity[L["spec"].name] = {"e_dyra": round(rel_err(L["y_rows"], exact), 5)}
        parity["sample_instances"] = sample

    # ---- FLOPs-matched static baseline (§2.3 FLOPs-Matched Comparison,
    # Appendix E.4): the truncated SVD at the rank whose exact FLOPs equal
    # DyRA's, run through the same library (the k = 0 path), timed and scored
    # on the same sampled instances against the exact product X W
    # (the FLOPs-matched, ALS and Newton-Schulz records are for the primal
    # path: the dual form at decode has one ALS step and no k x k solve)
    matched = None
    if not args.no_flops_matched and not dual:
        matched = {}
        sample = [0, B // 2, B - 1]
        rows = np.concatenate([np.arange(b * n, (b + 1) * n) for b in sample])
        for L in layers:
            spec = L["spec"]
            s = costs.flops_matched_rank(n, spec.c1, spec.c2, spec.r, spec.k)
            plan_s = dyra.dyra_prepare(L["W"], s, 0, 0.0, w.dtype, 0)
            ws_s = dyra.alloc_workspace(plan_s, B, n)
            ys = torch.empty_like(L["y"])
            t_s = time_loop(lambda: dyra.dyra_forward(L["xd"], B, n, plan_s, ys, ws_s, stream), reps, 3, stream)
            t_d = time_loop(lambda: dyra.dyra_forward(L["xd"], B, n, L["plan"], L["y"], L["ws"], stream), reps, 3,
                            stream)
            Xs = L["X"].exact[rows]
            exact = Xs @ L["W"].astype(np.float64)
            e_s = rel_err(ys.float().cpu().numpy().astype(np.float64)[rows], exact)
            e_d = rel_err(L["y"].float().cpu().numpy().astype(np.float64)[rows], exact)
            matched[spec.name] = {"static_rank": s, "e_dyra": round(e_d, 5), "e_static": round(e_s, 5),
                                  "t_dyra_us": round(t_d * 1e6, 2), "t_static_us": round(t_s * 1e6, 2),
                                  "flops_dyra": costs.dyra_flops(n, spec.c1, spec.c2, spec.r, spec.k) * B,
                                  "flops_static": costs.static_flops(n, spec.c1, spec.c2, s) * B}
            log(f"{spec.name}: FLOPs-matched static rank {s}: e_static {e_s:.4f} vs e_dyra {e_d:.4f}; "
                f"t_static {t_s * 1e6:.1f} us vs t_dyra {t_d * 1e6:.1f} us")
            plan_s.close()
        matched["sample_instances"] = sample

    # ---- further ALS steps (§3.3 ablation over t): error and time of the same
    # layers at t = 1 (Algorithm 1), 1.5 and 2, same sampled instances
    als_steps = None
    if not args.no_als_steps and not dual:
        als_steps = {}
        sample = [0, B // 2, B - 1]
        rows = np.concatenate([np.arange(b * n, (b + 1) * n) for b in sample])
        for L in layers:
            spec = L["spec"]
            Xs = L["X"].exact[rows]
            exact = Xs @ L["W"].astype(np.float64)
            rec = {}
            for hs in (2, 3, 4):
                plan_h = L["plan"] if hs == 2 else dyra.dyra_prepare_ex(L["W"], spec.r, spec.k, 0.0, w.dtype, 0,
                                                                        als_half_steps=hs)
                ws_h = L["ws"] if hs == 2 else dyra.alloc_workspace(plan_h, B, n)
                yh = torch.empty_like(L["y"])
                t_h = time_loop(lambda: dyra.dyra_forward(L["xd"], B, n, plan_h, yh, ws_h, stream), reps, 3, stream)
                e_h = rel_err(yh.float().cpu().numpy().astype(np.float64)[rows], exact)
                rec[f"t={hs / 2:g}"] = {"half_steps": hs, "e": round(e_h, 5), "t_us": round(t_h * 1e6, 2)}
                if hs != 2:
                    plan_h.close()
            als_steps[spec.name] = rec
            log(f"{spec.name}: ALS steps " + "  ".join(f"{k_}: e {v['e']:.4f} t {v['t_us']:.1f} us"
                                                      for k_, v in rec.items()))
        als_steps["sample_instances"] = sample

    # ---- §2.4's Newton-Schulz SPD solve in place of the Cholesky one: error
    # and time at 12 and 24 steps, same sampled instances
    ns = None
    if not args.no_ns and not dual:
        ns = {}
        sample = [0, B // 2, B - 1]
        rows = np.concatenate([np.arange(b * n, (b + 1) * n) for b in sample])
        for L in layers:
            spec = L["spec"]
            Xs = L["X"].exact[rows]
            exact = Xs @ L["W"].astype(np.float64)
            rec = {}
            for it in (12, 24):
                plan_h = dyra.dyra_prepare_ex(L["W"], spec.r, spec.k, 0.0, w.dtype, 0, ns_iters=it)
                ws_h = dyra.alloc_workspace(plan_h, B, n)
                yh = torch.empty_like(L["y"])
                t_h = time_loop(lambda: dyra.dyra_forward(L["xd"], B, n, plan_h, yh, ws_h, stream), reps, 3, stream)
                e_h = rel_err(yh.float().cpu().numpy().astype(np.float64)[rows], exact)
                rec[f"ns_iters={it}"] = {"e": round(e_h, 5), "t_us": round(t_h * 1e6, 2)}
                plan_h.close()
            ns[spec.name] = rec
            log(f"{spec.name}: Newton-Schulz " + "  ".join(f"{k_}: e {v['e']:.4f} t {v['t_us']:.1f} us"
                                                         for k_, v in rec.items()))
        ns["sample_instances"] = sample

    # ---- BLAST static approximation (Appendix B) in place of the truncated
    # SVD: an nb x nb block grid of the same static rank r (so the static
    # FLOPs match the low-rank path's, plus the mix), on a BLAST-structured
    # stand-in weight of each layer; step time, stages and error on the same
    # sampled instances
    blast, blast_legs = None, []
    if not args.no_blast and not dual:
        blast, blast_legs = blast_record(w, layers, args, stream, reps, t_dense, log)

    # ---- §2.4's two SPD solves as k and B grow
    solve_scaling = None
    if not args.no_solve_scaling and not dual and w.dtype == "bf16":
        solve_scaling = solve_scaling_record(w, layers, args, stream, log)

    # ---- the CPU leg, the one place this script runs the oracle: its float64
    # result on the sampled instances set beside the library's (parity, the
    # oracle's own error, the static part alone), and its throughput on the
    # host cores
    cpu = None
    if not args.no_cpu_baseline:
        cpu = oracle_leg(w, layers, blast, blast_legs, parity, args)

    flops = sum(dyra_flops(L["spec"], B, n) for L in layers)
    dense_flops = sum(2.0 * N * L["spec"].c1 * L["spec"].c2 for L in layers)
    out = {
        "metric": "DyRA layer tokens/s, speedup vs dense bf16 GEMM, rel. Frobenius error",
        "value": round(N / t_dyra, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_dyra * 1e3, 4),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_times, q)) * 1e3, 4) for q in (10, 50, 90)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; shapes and value distributions of the workload, no dataset or trained weights)",
        "config": {"workload": w.name, "description": w.description, "instances": B, "tokens_per_instance": n,
                   "layers": {L["spec"].name: [L["spec"].c1, L["spec"].c2, L["spec"].r, L["spec"].k]
                              for L in layers}},
        "speedup_vs_dense": round(t_dense / t_dyra, 4),
        "dense_ms_per_step": round(t_dense * 1e3, 4),
        "dense_ref_ms_per_step": round(t_dense_ref * 1e3, 4),
        "dyra_tflops": round(flops / t_dyra / 1e12, 1),
        "dense_tflops": round(dense_flops / t_dense / 1e12, 1),
        "stage_us": {L["spec"].name: {k: round(v * 1e6, 2) for k, v in L["stages"].items()} for L in layers},
        "rel_fro_error": parity,
        "flops_matched_static": matched,
        "als_steps": als_steps,
        "newton_schulz": ns,
        "solve_scaling": solve_scaling,
        "blast": blast,
        "roofline": roofline,
        "stage_roofline": stage_roofline,
        "achievable_peaks": achievable,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
