#!/usr/bin/env python3
"""Benchmark of the MoE-layer forward on one MI355X.

Prints ONE JSON line: whole-layer forward throughput (tokens/s) on the
Mixtral-shaped workload (T=4096, d_model=4096, 8 SwiGLU experts of
d_hidden=14336, top-2 softmax, dropless, bf16), with inputs resident in HBM,
plus
  * ``roofline``: the grouped SwiGLU step (gate/up GEMM + down GEMM, the
    dominant work) timed with HIP events on its stream inside the timed
    region, against the bf16 dense MFMA peak; ``traffic`` comes from the
    committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary when it was taken on the
    current kernel source, else null;
  * ``cpu_baseline``: the float64 CPU oracle on a bounded sample of tokens of
    the same workload, on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/s; grouped-GEMM TFLOP/s as % bf16 MFMA peak (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3         # MI355X fp32 (vector)
PEAK_HBM_GBS = 8000.0
GEMM_SRC = os.path.join(ROOT, "mixture_experts_layer_21_amd", "csrc", "grouped_swiglu.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_swiglu_traffic_{workload}.md")


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_8x_top2")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    return ap.parse_args()


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _source_hash():
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(workload, n_launch_units):
    """HBM bytes per launch of the grouped SwiGLU step from the committed
    rocprofv3 counter summary, or None if absent or taken on other source."""
    path = TRAFFIC_FILE.format(workload=workload)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", txt)
    m_bytes = re.search(r"hbm_bytes_per_step:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_bytes or m_hash.group(1) != _source_hash():
        return None
    return float(m_bytes.group(1))


def _cpu_baseline(w, inp, target_s):
    """The float64 oracle on a sample of tokens: routing of every token (the
    capacity rule needs all of them) and the expert work of the sample."""
    import numpy as np
    import torch

    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    _log("[cpu] converting inputs to float64")
    oi = {}
    for k, v in inp.items():
        if k in ("w_gate", "w_up", "w_down"):
            oi[k] = [v[e].to("cpu").to(torch.float64).numpy() for e in range(v.shape[0])]
        else:
            oi[k] = W.to_f64(v)

    def run(n):
        toks = np.linspace(0, w.T - 1, n).astype(np.int64)
        t0 = time.perf_counter()
        oracle.forward(oi, top_k=w.top_k, score=w.score, renormalize=w.renormalize,
                       route_scale=w.route_scale, n_groups=w.n_groups,
                       topk_groups=w.topk_groups, group_rule=w.group_rule,
                       capacity_factor=w.capacity_factor, tokens=toks)
        return time.perf_counter() - t0

    n = min(16, w.T)
    dt = run(n)
    _log(f"[cpu] calibration: {n} tokens in {dt:.2f}s")
    while dt < target_s / 3 and n < w.T:
        n = int(min(w.T, max(2 * n, n * target_s / max(dt, 1e-3))))
        dt = run(n)
        _log(f"[cpu] calibration: {n} tokens in {dt:.2f}s")
    reps, total = 1, dt
    while total < target_s and reps < 20:   # whole workload is quick: repeat it
        total += run(n)
        reps += 1
    dt = total / reps
    _log(f"[cpu] oracle: {n} tokens in {dt:.2f}s (mean of {reps})")
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} of {w.T} tokens (evenly spaced); routing of all {w.T} tokens "
                      f"included; float64 NumPy; mean of {reps} run(s), {dt:.2f} s each"}


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs on a single MI355X; sharding is described in DESIGN.md).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_layer_21_amd as moe
    import workloads as W

    w = W.WORKLOADS[args.workload]
    assert torch.cuda.is_available(), "bench.py needs a visible MI355X"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    _log(f"[bench] {w.name}: drawing inputs")
    gen_dev = "cpu" if w.act_dtype == "f32" else "cuda"
    inp = {k: v.to(dev) for k, v in W.make_inputs(w, gen_dev, seed=args.seed).items()}
    cfg = moe.make_config(w.T, w.D, w.H, w.E, w.top_k, H_shared=w.H_shared,
                          act_dtype=w.act_dtype, router_dtype=w.router_dtype, score=w.score,
                          renormalize=w.renormalize, route_scale=w.route_scale,
                          n_groups=w.n_groups, topk_groups=w.topk_groups,
                          group_rule=w.group_rule, capacity_factor=w.capacity_factor)
    ws = moe.new_workspace(cfg, dev)
    out = torch.empty(w.T, w.D, dtype=W.torch_dtype(w.act_dtype), device=dev)
    ids = torch.empty(w.T, w.top_k, dtype=torch.int32, device=dev)
    gw = torch.empty(w.T, w.top_k, dtype=torch.float32, device=dev)
    counts = torch.empty(w.E, dtype=torch.int32, device=dev)
    aux = torch.empty(2, dtype=torch.float32, device=dev)

    def forward():
        moe.moe_forward(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                        inp["w_down"], logit_bias=inp.get("logit_bias"),
                        select_bias=inp.get("select_bias"), ws_gate=inp.get("ws_gate"),
                        ws_up=inp.get("ws_up"), ws_down=inp.get("ws_down"), out=out,
                        expert_ids=ids, gate_w=gw, counts=counts, aux=aux, workspace=ws)

    _log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        forward()
    torch.cuda.synchronize()
    _log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        forward()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = w.T / (elapsed / args.steps)
    _log(f"[bench] {ms_per_step:.3f} ms/step, {tokens_per_s:.4g} tokens/s")

    # Stage-wise timing with HIP events on the launch stream: the same routing
    # and permutation as the forward, each stage through its own entry point.
    stream = torch.cuda.current_stream()
    cap = moe.capacity(cfg) if w.capacity_factor is not None else 0
    r = moe.moe_route(cfg, inp["x"], inp["w_router"], inp.get("logit_bias"),
                      inp.get("select_bias"), workspace=ws)
    perm = moe.moe_permute(cfg, r["expert_ids"], cap, workspace=ws)
    n_kept = int(perm["n_kept"].item())
    rows_bound = moe.max_rows(cfg)
    y = torch.empty(max(rows_bound, 1), w.D, dtype=out.dtype, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    stage_ms = np.zeros(4)
    shared_y = torch.empty_like(out) if w.H_shared else None
    for it in range(args.warmup + args.steps):
        ev[0].record(stream)
        moe.moe_route(cfg, inp["x"], inp["w_router"], inp.get("logit_bias"),
                      inp.get("select_bias"), expert_ids=r["expert_ids"], gate_w=r["gate_w"],
                      counts=r["counts"], aux=r["aux"], mean_prob=r["mean_prob"], workspace=ws)
        ev[1].record(stream)
        moe.moe_permute(cfg, r["expert_ids"], cap, workspace=ws)
        ev[2].record(stream)
        moe.moe_grouped_swiglu(cfg, inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"],
                               row_to_assign=perm["row_to_assign"],
                               expert_offsets=perm["expert_offsets"], max_rows_bound=rows_bound,
                               gate_w=r["gate_w"], y_rows=y, workspace=ws, validate=False)
        if w.H_shared:
            moe.moe_grouped_swiglu(cfg, inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"],
                                   y_rows=shared_y, workspace=ws, validate=False)
        ev[3].record(stream)
        moe.moe_combine(cfg, y, perm["assign_to_row"], shared_y, validate=False)
        ev[4].record(stream)
        ev[4].synchronize()
        if it >= args.warmup:
            stage_ms += [ev[i].elapsed_time(ev[i + 1]) for i in range(4)]
    stage_ms /= args.steps
    _log("[bench] stages ms: route %.4f permute %.4f grouped_swiglu %.4f combine %.4f"
         % tuple(stage_ms))

    # Algorithmic work of the grouped SwiGLU step: 2*D*H FLOP for each of the
    # gate, up and down products per kept row (plus the shared expert on T rows).
    bf16 = w.act_dtype == "bf16"
    flops = 6.0 * w.D * w.H * n_kept + 6.0 * w.D * w.H_shared * w.T
    achieved = flops / (stage_ms[2] * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    traffic = _traffic(w.name, 1)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": "grouped_swiglu step (gate/up GEMM + down GEMM)",
                "algorithmic_flop_per_launch": flops,
                "launch_ms": round(float(stage_ms[2]), 4)}

    result = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if bf16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d_model": w.D, "d_hidden": w.H,
                   "experts": w.E, "top_k": w.top_k, "shared_d_hidden": w.H_shared,
                   "capacity_factor": w.capacity_factor, "kept_rows": n_kept,
                   "parallelism": "none (1 GPU)"},
        "stages_ms": {k: round(float(v), 4) for k, v in
                      zip(("route", "permute", "grouped_swiglu", "combine"), stage_ms)},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
