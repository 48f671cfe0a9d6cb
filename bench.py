#!/usr/bin/env python3
"""Benchmark of the MoE-layer forward on one MI355X.

Prints ONE JSON line: whole-layer forward throughput (tokens/s) on the
Mixtral-shaped workload (T=4096, d_model=4096, 8 SwiGLU experts of
d_hidden=14336, top-2 softmax, dropless, bf16), with inputs resident in HBM,
plus
  * ``roofline``: the grouped SwiGLU step (gate/up GEMM + down GEMM, the
    dominant work) timed with HIP events on its stream.  Its bound is the
    one its algorithmic intensity selects: FLOP (6*D*H per kept row) per
    algorithmic byte (the weights of every expert that keeps a row, the
    gathered input rows and the output rows) against the ridge of the bf16
    MFMA peak over the HBM peak.  ``traffic`` comes from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summary when it was taken on the current
    kernel source, else null;
  * ``cpu_baseline``: the float64 CPU oracle on a bounded sample of tokens of
    the same workload, on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       python bench.py --pmc-summary FETCH_DB WRITE_DB --workload NAME
       python bench.py --trace-summary KERNEL_TRACE_CSV --workload NAME [--steps K --warmup W]
The second form turns two rocprofv3 counter databases (one FETCH_SIZE pass,
one WRITE_SIZE pass, each of a run with --copy-calibration) into the traffic
summary that the first form reads; the third turns the kernel trace of a
first-form run into per-kernel durations, with the mean over the dispatches of
the timed steps beside the mean over all of them.
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
# The grouped SwiGLU kernels' source: the traffic summaries record its hash.
GEMM_SRC = [os.path.join(ROOT, "mixture_experts_layer_21_amd", "csrc", f)
            for f in ("grouped_swiglu.hip", "dma_gemm.hpp")]
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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB read + 1 GiB write kernel (torch.neg on "
                         "fp32), the reference that scales the HBM byte counters")
    ap.add_argument("--backward", action="store_true",
                    help="also time moe_backward (beside the forward step) and report it")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="summarise two rocprofv3 counter databases and exit")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="summarise a rocprofv3 kernel trace (CSV) of a run with the same "
                         "--workload, --steps and --warmup, and exit")
    ap.add_argument("--mfma-summary", metavar="DB",
                    help="summarise a rocprofv3 database of SQ_VALU_MFMA_BUSY_CYCLES, "
                         "SQ_BUSY_CYCLES and GRBM_GUI_ACTIVE and exit")
    return ap.parse_args()


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _source_hash():
    h = hashlib.sha256()
    for path in GEMM_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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


CALIB_BYTES = 1 << 30           # bytes read (and written) by the calibration kernel


def _copy_calibration(dev):
    """A plain streaming kernel of known size: torch.neg over 2^28 fp32 values
    reads 1 GiB and writes 1 GiB.  Its FETCH_SIZE / WRITE_SIZE readings give
    the factor that turns counter units into bytes."""
    import torch
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _pmc_means(db):
    """Mean counter value per dispatch for each kernel of one rocprofv3 DB."""
    import collections
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select name, dispatch_id, counter_name, counter_value, duration "
                       "from pmc_events").fetchall()
    per = collections.defaultdict(float)
    dur = {}
    for name, did, cn, v, d in rows:
        per[(name, did, cn)] += v     # summed over hardware instances
        dur[(name, did)] = d
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for (name, did, cn), v in per.items():
        out[name][cn].append(v)
        out[name].setdefault("_dur", []).append(dur[(name, did)])
    res = {n: {c: sum(v) / len(v) for c, v in d.items()} for n, d in out.items()}
    for n, d in out.items():
        res[n]["_n"] = len(d["_dur"])
    return res


def _short(name):
    name = re.sub(r"\(anonymous namespace\)::", "", name).replace("void ", "")
    return re.sub(r"\(moe::\w+Params(, int)?\)", "", name)


def _pmc_summary(fetch_db, write_db, workload):
    fetch, write = _pmc_means(fetch_db), _pmc_means(write_db)
    calib = [n for n in fetch if "neg_kernel" in n]
    assert calib, "no calibration kernel in the FETCH_SIZE run (use --copy-calibration)"
    calib_w = [n for n in write if "neg_kernel" in n]
    f_cal = fetch[calib[0]]["FETCH_SIZE"]
    w_cal = write[calib_w[0]]["WRITE_SIZE"]
    f_scale = CALIB_BYTES / f_cal
    w_scale = CALIB_BYTES / w_cal
    lines = [f"# HBM traffic of the MoE kernels: {workload}", "",
             f"source_sha256_16: {_source_hash()}", "",
             "FETCH_SIZE and WRITE_SIZE (rocprofv3, one pass each) per dispatch, scaled by",
             "the readings of a plain torch.neg over 2^28 fp32 values (1 GiB read, 1 GiB",
             f"written): FETCH_SIZE {f_cal:.6g} -> {f_scale:.4f} B per unit, "
             f"WRITE_SIZE {w_cal:.6g} -> {w_scale:.4f} B per unit.  The calibration kernel "
             f"itself moves 2 GiB in {fetch[calib[0]]['_dur'] / 1e3:.1f} us "
             f"({2 * CALIB_BYTES / fetch[calib[0]]['_dur']:.0f} GB/s).", "",
             "Commands (one MI355X; the counter passes, then this summary):", "", "```",
             "cd /tmp && export TMPDIR=/tmp",
             *(f"rocprofv3 --kernel-include-regex 'moe::|neg_kernel' --pmc {c} -d /tmp/t_{c} "
               f"-o {workload} -- python3 /root/repo/bench.py --workload {workload} --steps 2 "
               f"--warmup 1 --no-cpu-baseline --copy-calibration"
               for c in ("FETCH_SIZE", "WRITE_SIZE")),
             f"python3 /root/repo/bench.py --pmc-summary /tmp/t_FETCH_SIZE/{workload}_results.db "
             f"/tmp/t_WRITE_SIZE/{workload}_results.db --workload {workload}",
             "```", "",
             "| kernel | dispatches | avg duration (us) | read (MB) | written (MB) | GB/s |",
             "|---|---:|---:|---:|---:|---:|"]
    step = 0.0
    for name in sorted(n for n in fetch if "moe::" in n):
        f = fetch[name]
        wr = write.get(name, {})
        rd = f["FETCH_SIZE"] * f_scale
        wb = wr.get("WRITE_SIZE", 0.0) * w_scale
        us = f["_dur"] / 1e3
        lines.append(f"| `{_short(name)}` | {f['_n']} | {us:.1f} | {rd / 1e6:.1f} | "
                     f"{wb / 1e6:.1f} | {(rd + wb) / us / 1e3:.0f} |")
        if "gemm" in name:
            step += rd + wb
    lines += ["", "Grouped SwiGLU step (every gemm kernel above once per forward):", "",
              f"hbm_bytes_per_step: {step:.6g}", ""]
    return "\n".join(lines)


def _trace_summary(csv_path, workload, steps, warmup):
    """Per-kernel durations from a rocprofv3 kernel trace of
    `bench.py --workload W --steps K --warmup W0 --no-cpu-baseline`.  Each
    warm-up round runs one staged step and one moe_forward, then the K timed
    staged steps run, then K moe_forward calls; a kernel with p launches per
    step therefore has 2*(W0+K)*p dispatches, and the timed steps' ones are
    dispatches [2*W0*p, (2*W0+K)*p) in start order."""
    import collections
    import csv
    import statistics
    rows = list(csv.DictReader(open(csv_path)))
    key = lambda *names: next(k for k in rows[0] if k in names)
    kn, ks, ke = (key("Kernel_Name", "Name"), key("Start_Timestamp", "Start"),
                  key("End_Timestamp", "End"))
    per = collections.defaultdict(list)
    for r in rows:
        if "moe::" in r[kn]:
            per[r[kn]].append((int(r[ks]), int(r[ke]) - int(r[ks])))
    cmd = (f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --kernel-include-regex "
           f"'moe::' --output-format csv -d /tmp/kt_{workload} -o run -- python3 "
           f"/root/repo/bench.py --workload {workload} --steps {steps} --warmup {warmup} "
           f"--no-cpu-baseline")
    lines = [f"# Kernel trace of the MoE forward: {workload}", "",
             "Per-dispatch durations from a rocprofv3 kernel trace (the library's kernels",
             f"only) of bench.py on one MI355X: {warmup} warm-up rounds (a staged step and a",
             f"`moe_forward` each), {steps} timed staged steps, then {steps} `moe_forward`",
             "calls, plus the route/permute calls of the set-up.  \"timed steps\" is the mean",
             "per step over the dispatches of the timed staged steps (the region bench.py",
             "times with HIP events), for kernels whose dispatch count is a whole number",
             "of launches per step; \"all\" is the mean over every dispatch, warm-up included.",
             "", "Commands:", "", "```", cmd,
             f"python3 /root/repo/bench.py --trace-summary "
             f"$(find /tmp/kt_{workload} -name run_kernel_trace.csv) "
             f"--workload {workload} --steps {steps} --warmup {warmup}", "```", "",
             "| kernel | dispatches | launches per step | timed steps, per step (us) | "
             "all: mean (us) | median (us) | min (us) | max (us) |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    rounds = 2 * (warmup + steps)
    step_sum = 0.0
    for name in sorted(per):
        d = sorted(per[name])
        us = [x[1] / 1e3 for x in d]
        p = len(d) // rounds if len(d) % rounds == 0 else 0
        if p:
            timed = sum(us[2 * warmup * p:(2 * warmup + steps) * p]) / steps
            tcol = f"{timed:.1f}"
            if "gemm" in name:
                step_sum += timed
        else:
            tcol = "-"
        lines.append(f"| `{_short(name)}` | {len(d)} | {p or '-'} | {tcol} | "
                     f"{sum(us) / len(us):.1f} | {statistics.median(us):.1f} | "
                     f"{min(us):.1f} | {max(us):.1f} |")
    lines += ["", "Grouped SwiGLU step (every gemm kernel, timed steps): "
              f"{step_sum:.1f} us per step.", ""]
    return "\n".join(lines)


def _time_backward(moe, w, cfg, inp, r, n_kept, steps, stream):
    """moe_backward on the forward's routes with a seeded dout, timed with HIP
    events on the launch stream.  Algorithmic FLOP: the input-gradient and
    weight-gradient products of every kept row (2 x the forward's 6*D*H per
    row, plus the shared expert on T rows) and of the router (2 x 2*T*D*E)."""
    import torch
    if w.act_dtype != "bf16":
        return {"skipped": "the backward covers bf16 activations"}
    gen = torch.Generator(device=inp["x"].device)
    gen.manual_seed(1)
    dout = torch.randn(w.T, w.D, generator=gen, device=inp["x"].device).to(inp["x"].dtype)
    ws = torch.empty(moe.backward_workspace_bytes(cfg), dtype=torch.uint8,
                     device=inp["x"].device)

    def bwd():
        return moe.moe_backward(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                                inp["w_down"], r["expert_ids"], r["gate_w"], dout,
                                logit_bias=inp.get("logit_bias"), ws_gate=inp.get("ws_gate"),
                                ws_up=inp.get("ws_up"), ws_down=inp.get("ws_down"),
                                balance_coef=0.01, z_coef=0.001, workspace=ws)
    bwd()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        bwd()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    flops = (12.0 * w.D * w.H * n_kept + 12.0 * w.D * w.H_shared * w.T
             + 4.0 * w.T * w.D * w.E)
    _log(f"[bench] moe_backward: {ms:.3f} ms/step, {flops / ms / 1e9:.1f} TFLOP/s")

    # The same step with the SwiGLU state saved by the forward: the forward
    # writes two more bf16 [rows, H] arrays, the backward skips the gate/up
    # recompute.
    saved = moe.new_saved(cfg, inp["x"].device)
    fws = moe.new_workspace(cfg, inp["x"].device)

    def fwd(save):
        return moe.moe_forward(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                               inp["w_down"], logit_bias=inp.get("logit_bias"),
                               select_bias=inp.get("select_bias"), ws_gate=inp.get("ws_gate"),
                               ws_up=inp.get("ws_up"), ws_down=inp.get("ws_down"),
                               workspace=fws, saved=saved if save else None)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(steps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / steps

    f_plain = timed(lambda: fwd(False))
    f_save = timed(lambda: fwd(True))

    def bwd_saved():
        return moe.moe_backward(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                                inp["w_down"], r["expert_ids"], r["gate_w"], dout,
                                logit_bias=inp.get("logit_bias"), ws_gate=inp.get("ws_gate"),
                                ws_up=inp.get("ws_up"), ws_down=inp.get("ws_down"),
                                balance_coef=0.01, z_coef=0.001, workspace=ws, saved=saved)
    ms_saved = timed(bwd_saved)
    _log(f"[bench] with saved state: forward {f_plain:.3f} -> {f_save:.3f} ms, backward "
         f"{ms:.3f} -> {ms_saved:.3f} ms")
    return {"ms_per_step": round(ms, 4), "algorithmic_flop": flops,
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "with_saved_state": {"forward_ms": round(f_save, 4),
                                 "forward_without_saving_ms": round(f_plain, 4),
                                 "backward_ms": round(ms_saved, 4),
                                 "saved_bytes": moe.saved_bytes(cfg)}}


SIMDS = 256 * 4  # MI355X: 256 compute units of four SIMDs


def _mfma_summary(db, workload):
    """Clock and MFMA utilisation per kernel from one rocprofv3 counter pass:
    clock = GRBM_GUI_ACTIVE / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES
    (summed over the SIMDs) / (SIMDS * GRBM_GUI_ACTIVE)."""
    import collections
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select name, dispatch_id, counter_name, counter_value, duration "
                       "from pmc_events").fetchall()
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = {}
    for name, did, cn, v, d in rows:
        per[(name, did)][cn].append(v)
        dur[(name, did)] = d
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for (name, did), cs in per.items():
        if "moe::" not in name:
            continue
        for cn, vals in cs.items():  # GRBM: one clock for the chip; SQ: summed
            agg[name][cn].append(max(vals) if cn.startswith("GRBM") else sum(vals))
        agg[name]["_dur"].append(dur[(name, did)])
    cmd = (f"rocprofv3 --kernel-include-regex 'moe::' --pmc SQ_VALU_MFMA_BUSY_CYCLES "
           f"SQ_BUSY_CYCLES GRBM_GUI_ACTIVE -d /tmp/t_mfma -o {workload} -- python3 "
           f"/root/repo/bench.py --workload {workload} --steps 2 --warmup 1 --no-cpu-baseline")
    lines = [f"# Clock and MFMA utilisation of the MoE kernels: {workload}", "",
             f"source_sha256_16: {_source_hash()}", "",
             "One rocprofv3 counter pass.  clock = GRBM_GUI_ACTIVE / duration;",
             f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / ({SIMDS} SIMDs x GRBM_GUI_ACTIVE),",
             "the fraction of SIMD cycles in which the matrix core is busy.  At the",
             "nominal 2.4 GHz a fully busy matrix core gives the 2.5 PFLOP/s bf16 peak.",
             "Kernels under 100 us are listed without either figure: GRBM_GUI_ACTIVE",
             "then counts more cycles than the kernel runs.", "",
             "Commands (one MI355X):", "", "```", "cd /tmp && export TMPDIR=/tmp", cmd,
             f"python3 /root/repo/bench.py --mfma-summary /tmp/t_mfma/{workload}_results.db "
             f"--workload {workload}", "```", "",
             "| kernel | dispatches | avg duration (us) | clock (GHz) | MFMA busy |",
             "|---|---:|---:|---:|---:|"]
    for name in sorted(agg):
        d = agg[name]
        us = sum(d["_dur"]) / len(d["_dur"]) / 1e3
        g = sum(d.get("GRBM_GUI_ACTIVE", [0])) / max(len(d.get("GRBM_GUI_ACTIVE", [])), 1)
        m = sum(d.get("SQ_VALU_MFMA_BUSY_CYCLES", [0])) / max(
            len(d.get("SQ_VALU_MFMA_BUSY_CYCLES", [])), 1)
        if us < 100.0 or not g:  # the counter window outlasts short kernels
            lines.append(f"| `{_short(name)}` | {len(d['_dur'])} | {us:.1f} | - | - |")
            continue
        lines.append(f"| `{_short(name)}` | {len(d['_dur'])} | {us:.1f} | "
                     f"{g / (us * 1e3):.2f} | {100 * m / (SIMDS * g):.1f}% |")
    return "\n".join(lines) + "\n"


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
    if args.pmc_summary:
        print(_pmc_summary(*args.pmc_summary, args.workload))
        return
    if args.mfma_summary:
        print(_mfma_summary(args.mfma_summary, args.workload))
        return
    if args.trace_summary:
        print(_trace_summary(args.trace_summary, args.workload, args.steps, args.warmup))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs on a single MI355X; it shards by expert across GPUs).",
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

    if args.copy_calibration:
        _copy_calibration(dev)
    # One step = one pass of the whole hot path through the C-ABI entry points
    # (route, permute, grouped SwiGLU (+ shared expert), combine), with HIP
    # events recorded between the stages on the launch stream.  The kernels and
    # their order are those of moe_forward; the fused entry is timed after it
    # as a cross-check.
    stream = torch.cuda.current_stream()
    cap = moe.capacity(cfg) if w.capacity_factor is not None else 0
    r = moe.moe_route(cfg, inp["x"], inp["w_router"], inp.get("logit_bias"),
                      inp.get("select_bias"), workspace=ws)
    perm = moe.moe_permute(cfg, r["expert_ids"], cap, workspace=ws)
    n_kept = int(perm["n_kept"].item())
    rows_bound = moe.max_rows(cfg)
    y = torch.empty(max(rows_bound, 1), w.D, dtype=out.dtype, device=dev)
    shared_y = torch.empty_like(out) if w.H_shared else None

    def step(ev):
        ev[0].record(stream)
        moe.moe_route(cfg, inp["x"], inp["w_router"], inp.get("logit_bias"),
                      inp.get("select_bias"), expert_ids=r["expert_ids"], gate_w=r["gate_w"],
                      counts=r["counts"], aux=r["aux"], mean_prob=r["mean_prob"], workspace=ws)
        ev[1].record(stream)
        moe.moe_permute(cfg, r["expert_ids"], cap, workspace=ws, **perm)
        ev[2].record(stream)
        moe.moe_grouped_swiglu(cfg, inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"],
                               row_to_assign=perm["row_to_assign"],
                               expert_offsets=perm["expert_offsets"], max_rows_bound=rows_bound,
                               gate_w=r["gate_w"], y_rows=y, workspace=ws, validate=False)
        if w.H_shared:
            moe.moe_grouped_swiglu(cfg, inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"],
                                   y_rows=shared_y, workspace=ws, validate=False)
        ev[3].record(stream)
        moe.moe_combine(cfg, y, perm["assign_to_row"], shared_y, out=out, validate=False)
        ev[4].record(stream)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
              for _ in range(args.steps)]
    _log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        step(events[i % args.steps])
        forward()
    torch.cuda.synchronize()
    _log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = w.T / (elapsed / args.steps)
    stage_ms = np.array([[ev[i].elapsed_time(ev[i + 1]) for i in range(4)]
                         for ev in events]).mean(axis=0)
    # each timed step on the device clock (HIP events around the step)
    step_dev = np.array([ev[0].elapsed_time(ev[4]) for ev in events])
    _log(f"[bench] {ms_per_step:.3f} ms/step, {tokens_per_s:.4g} tokens/s")
    _log("[bench] stages ms: route %.4f permute %.4f grouped_swiglu %.4f combine %.4f"
         % tuple(stage_ms))
    t0 = time.perf_counter()
    for _ in range(args.steps):
        forward()
    torch.cuda.synchronize()
    fwd_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    _log(f"[bench] moe_forward: {fwd_ms:.3f} ms/step")

    # A step beside the layer, timed on its own (not part of the step above):
    # the RMSNorm pre-norm of the residual stream.  Algorithmic bytes: x read
    # once, the normalised rows written once, the weight vector.
    xn = torch.empty_like(inp["x"])
    nw = torch.ones(w.D, dtype=torch.float32, device=dev)
    moe.moe_rmsnorm(cfg, inp["x"], nw, out=xn)
    rev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    rev[0].record(stream)
    for _ in range(args.steps):
        moe.moe_rmsnorm(cfg, inp["x"], nw, out=xn)
    rev[1].record(stream)
    torch.cuda.synchronize()
    rms_ms = rev[0].elapsed_time(rev[1]) / args.steps
    esz_x = 2 if w.act_dtype == "bf16" else 4
    rms_bytes = 2.0 * w.T * w.D * esz_x + 4.0 * w.D

    # Algorithmic work of the grouped SwiGLU step: 2*D*H FLOP for each of the
    # gate, up and down products per kept row (plus the shared expert on T
    # rows); algorithmic bytes: the three weight matrices of every expert that
    # keeps at least one row, the gathered input rows and the output rows.
    bf16 = w.act_dtype == "bf16"
    esz = 2 if bf16 else 4
    kept = np.diff(perm["expert_offsets"].cpu().numpy())
    touched = int((kept > 0).sum())
    flops = 6.0 * w.D * w.H * n_kept + 6.0 * w.D * w.H_shared * w.T
    nbytes = (3.0 * w.D * w.H * touched * esz + 2.0 * n_kept * w.D * esz
              + (3.0 * w.D * w.H_shared + 2.0 * w.T * w.D) * esz * (w.H_shared > 0))
    sec = stage_ms[2] * 1e-3
    peak_f = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    traffic = _traffic(w.name, 1)
    mfma_bound = flops / nbytes >= peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        achieved, peak, unit = flops / sec / 1e12, peak_f, "TFLOP/s"
    else:
        achieved, peak, unit = nbytes / sec / 1e9, PEAK_HBM_GBS, "GB/s"
    roofline = {"bound": "mfma" if mfma_bound else "hbm", "achieved": round(achieved, 2),
                "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": traffic,
                "kernel": "grouped_swiglu step (gate/up GEMM + down GEMM)",
                "algorithmic_flop_per_launch": flops,
                "algorithmic_bytes_per_launch": nbytes,
                "experts_with_rows": touched,
                "tflops": round(flops / sec / 1e12, 2),
                "hbm_gbs": round(nbytes / sec / 1e9, 1),
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
        "moe_forward_ms_per_step": round(fwd_ms, 4),
        "step_ms_device": {"median": round(float(np.median(step_dev)), 4),
                           "min": round(float(step_dev.min()), 4),
                           "p90": round(float(np.percentile(step_dev, 90)), 4)},
        "stages_ms": {k: round(float(v), 4) for k, v in
                      zip(("route", "permute", "grouped_swiglu", "combine"), stage_ms)},
        "roofline": roofline,
        "beside_the_step": {"rmsnorm_ms": round(rms_ms, 4),
                            "rmsnorm_gbs": round(rms_bytes / (rms_ms * 1e-3) / 1e9, 1)},
    }
    if args.backward:
        result["backward"] = _time_backward(moe, w, cfg, inp, r, n_kept, args.steps, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
