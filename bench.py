#!/usr/bin/env python3
"""Benchmark of the MoE-layer forward on one MI355X.

Prints ONE JSON line.  By default all five workloads run in one process (the
tiny fp32 layer, the Switch-style capacity layer, the Mixtral-shaped layer,
the DeepSeek-V3-shaped layer and the decode-shaped layer); the headline
fields (value, roofline, cpu_baseline, ...) are those of the Mixtral-shaped
workload (T=4096, d_model=4096, 8 SwiGLU experts of d_hidden=14336, top-2
softmax, dropless, bf16), the configuration the metric is quoted on, and
``configs`` carries every workload's tokens/s, stages, rooflines and CPU
baseline.  Inputs are resident in HBM when timing starts.
  * ``value``: tokens/s of the whole hot path, one ``moe_forward`` call per
    step, K steps between two synchronisations.  The same path as its four
    stage calls (route, permute, grouped SwiGLU, combine) gives ``stages_ms``
    from HIP events; ``moe_forward_graph_ms_per_step`` is the forward
    captured once into a HIP graph and replayed;
  * ``roofline``: the grouped SwiGLU step (gate/up GEMM + down GEMM, the
    dominant work), K calls back to back between two HIP events on its
    stream (so the device never waits on the host).  Its bound is the
    one its algorithmic intensity selects: FLOP (6*D*H per kept row) per
    algorithmic byte (the weights of every expert that keeps a row, x read
    once, the output written once) against the ridge of the bf16 MFMA peak
    over the HBM peak.  ``traffic`` comes from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary when it was taken on the current kernel
    source, else null;
  * ``layer``: the whole step (route, permute, grouped SwiGLU, combine)
    against both peaks (the router GEMM and weights added);
  * ``cpu_baseline``: the float64 CPU oracle on the same workload (whole
    layer, or a bounded sample of it), on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]
       python bench.py --pmc-summary FETCH_DB WRITE_DB --workload NAME
       python bench.py --mfma-summary DB --workload NAME
       python bench.py --stall-summary DB --workload NAME
       python bench.py --trace-summary KERNEL_TRACE_CSV --workload NAME [--steps K --warmup W]
The summary forms turn rocprofv3 counter databases of single-workload runs
(the FETCH_SIZE and WRITE_SIZE passes with --copy-calibration; the MFMA pass;
the wait/LDS pass) into the summaries under profiles/; the last turns the
kernel trace of a single-workload run into per-kernel durations, with the
mean over the dispatches of the timed steps beside the mean over all of them.
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
    ap.add_argument("--workload", default="all",
                    help="one workload, or 'all' (default): the five in one run, the "
                         "headline fields from the Mixtral-shaped layer")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of moe_forward")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
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
    ap.add_argument("--stall-summary", metavar="DB",
                    help="summarise a rocprofv3 database of SQ_WAIT_ANY, SQ_WAVE_CYCLES, "
                         "SQ_LDS_BANK_CONFLICT, SQ_INSTS_LDS and GRBM_GUI_ACTIVE and exit")
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


# Steps of the counter runs: each warm-up round and each timed round runs one
# staged step and one moe_forward, and the grouped SwiGLU stage then runs
# K + 1 more times on its own (the back-to-back timing), so a grouped GEMM
# kernel with p launches per step has gemm_rounds(W, K) * p dispatches and
# any other kernel of the step 2 * (W + K) * p.
PMC_STEPS, PMC_WARMUP = 2, 1


def gemm_rounds(warmup, steps):
    return 2 * (warmup + steps) + steps + 1


def _rounds_of(name, warmup, steps):
    return gemm_rounds(warmup, steps) if "gemm" in name else 2 * (warmup + steps)


def _pmc_dispatches(db, grbm_max=False):
    """Per kernel: the dispatches of one rocprofv3 DB in dispatch order, each
    as (counter -> value summed over hardware instances, duration in ns);
    with grbm_max the GRBM counters (one clock for the chip) take the largest
    instance instead."""
    import collections
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select name, dispatch_id, counter_name, counter_value, duration "
                       "from pmc_events").fetchall()
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    dur = {}
    for name, did, cn, v, d in rows:
        if grbm_max and cn.startswith("GRBM"):
            per[(name, did)][cn] = max(per[(name, did)][cn], v)
        else:
            per[(name, did)][cn] += v
        dur[(name, did)] = d
    out = collections.defaultdict(list)
    for (name, did) in sorted(per, key=lambda k: k[1]):
        out[name].append((dict(per[(name, did)]), dur[(name, did)]))
    return out


def _mean(vals):
    return sum(vals) / len(vals) if vals else 0.0


def _short(name):
    name = re.sub(r"\(anonymous namespace\)::", "", name).replace("void ", "")
    return re.sub(r"\(moe::\w+Params(, int)?\)", "", name)


def _pmc_summary(fetch_db, write_db, workload):
    fetch, write = _pmc_dispatches(fetch_db), _pmc_dispatches(write_db)
    calib = [n for n in fetch if "neg_kernel" in n]
    assert calib, "no calibration kernel in the FETCH_SIZE run (use --copy-calibration)"
    calib_w = [n for n in write if "neg_kernel" in n]
    f_cal = _mean([c["FETCH_SIZE"] for c, _ in fetch[calib[0]]])
    w_cal = _mean([c["WRITE_SIZE"] for c, _ in write[calib_w[0]]])
    cal_us = _mean([d for _, d in fetch[calib[0]]]) / 1e3
    f_scale = CALIB_BYTES / f_cal
    w_scale = CALIB_BYTES / w_cal
    rounds = gemm_rounds(PMC_WARMUP, PMC_STEPS)
    lines = [f"# HBM traffic of the MoE kernels: {workload}", "",
             f"source_sha256_16: {_source_hash()}", "",
             "FETCH_SIZE and WRITE_SIZE (rocprofv3, one pass each) per dispatch, scaled by",
             "the readings of a plain torch.neg over 2^28 fp32 values (1 GiB read, 1 GiB",
             f"written): FETCH_SIZE {f_cal:.6g} -> {f_scale:.4f} B per unit, "
             f"WRITE_SIZE {w_cal:.6g} -> {w_scale:.4f} B per unit.  The calibration kernel "
             f"itself moves 2 GiB in {cal_us:.1f} us ({2 * CALIB_BYTES / (cal_us * 1e3):.0f} GB/s).",
             "",
             "A grouped GEMM kernel that runs p times per step (the routed experts, then",
             "the shared expert) has one row per launch: the i-th dispatch of every step",
             "goes to row i.  The step's bytes add every launch of every gemm kernel.", "",
             "Commands (one MI355X; the counter passes, then this summary):", "", "```",
             "cd /tmp && export TMPDIR=/tmp",
             *(f"rocprofv3 --kernel-include-regex 'moe::|neg_kernel' --pmc {c} -d /tmp/t_{c} "
               f"-o {workload} -- python3 /root/repo/bench.py --workload {workload} "
               f"--steps {PMC_STEPS} --warmup {PMC_WARMUP} --no-cpu-baseline --no-graph "
               f"--copy-calibration"
               for c in ("FETCH_SIZE", "WRITE_SIZE")),
             f"python3 /root/repo/bench.py --pmc-summary /tmp/t_FETCH_SIZE/{workload}_results.db "
             f"/tmp/t_WRITE_SIZE/{workload}_results.db --workload {workload}",
             "```", "",
             "| kernel | launch | dispatches | avg duration (us) | read (MB) | written (MB) "
             "| GB/s |",
             "|---|---|---:|---:|---:|---:|---:|"]
    step = 0.0
    for name in sorted(n for n in fetch if "moe::" in n):
        fd, wd = fetch[name], write.get(name, [])
        n = len(fd)
        p = n // rounds if ("gemm" in name and n % rounds == 0 and len(wd) == n) else 1
        for i in range(p):
            f_i = fd[i::p] if p > 1 else fd
            w_i = wd[i::p] if p > 1 else wd
            rd = _mean([c.get("FETCH_SIZE", 0.0) for c, _ in f_i]) * f_scale
            wb = _mean([c.get("WRITE_SIZE", 0.0) for c, _ in w_i]) * w_scale
            us = _mean([d for _, d in f_i]) / 1e3
            launch = f"{i + 1} of {p}" if p > 1 else "all"
            lines.append(f"| `{_short(name)}` | {launch} | {len(f_i)} | {us:.1f} | "
                         f"{rd / 1e6:.1f} | {wb / 1e6:.1f} | {(rd + wb) / us / 1e3:.0f} |")
            if "gemm" in name:
                step += rd + wb
    lines += ["", "Grouped SwiGLU step (every launch of every gemm kernel above, per step):",
              "", f"hbm_bytes_per_step: {step:.6g}", ""]
    return "\n".join(lines)


def _trace_summary(csv_path, workload, steps, warmup):
    """Per-kernel durations from a rocprofv3 kernel trace of
    `bench.py --workload W --steps K --warmup W0 --no-cpu-baseline --no-graph`.
    Each warm-up round runs one staged step and one moe_forward, then the K
    timed moe_forward steps run, then K staged steps; a kernel with p launches
    per step therefore has 2*(W0+K)*p dispatches (gemm kernels K+1 more
    rounds: the back-to-back stage timing), and the timed steps' ones are
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
           f"--no-cpu-baseline --no-graph")
    lines = [f"# Kernel trace of the MoE forward: {workload}", "",
             "Per-dispatch durations from a rocprofv3 kernel trace (the library's kernels",
             f"only) of bench.py on one MI355X: {warmup} warm-up rounds (a staged step and a",
             f"`moe_forward` each), {steps} timed `moe_forward` steps, then {steps} staged",
             f"steps and {steps + 1} more calls of the grouped SwiGLU stage alone, plus the",
             "route/permute calls of the set-up.  \"timed steps\" is the mean",
             "per step over the dispatches of the timed `moe_forward` steps (the region",
             "bench.py times), for kernels whose dispatch count is a whole number of",
             "launches per step; \"all\" is the mean over every dispatch, warm-up included.",
             "", "Commands:", "", "```", cmd,
             f"python3 /root/repo/bench.py --trace-summary "
             f"$(find /tmp/kt_{workload} -name run_kernel_trace.csv) "
             f"--workload {workload} --steps {steps} --warmup {warmup}", "```", "",
             "| kernel | dispatches | launches per step | timed steps, per step (us) | "
             "all: mean (us) | median (us) | min (us) | max (us) |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    step_sum = 0.0
    for name in sorted(per):
        d = sorted(per[name])
        us = [x[1] / 1e3 for x in d]
        rounds = _rounds_of(name, warmup, steps)
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


def _launch_rows(disp):
    """Dispatch lists of each kernel split per launch of a step (see
    _pmc_summary): [(kernel, launch label, dispatches)]."""
    rounds = gemm_rounds(PMC_WARMUP, PMC_STEPS)
    out = []
    for name in sorted(n for n in disp if "moe::" in n):
        d = disp[name]
        p = len(d) // rounds if ("gemm" in name and len(d) % rounds == 0) else 1
        for i in range(p):
            out.append((name, f"{i + 1} of {p}" if p > 1 else "all", d[i::p] if p > 1 else d))
    return out


def _counter_table(db, workload, kind):
    """Per kernel launch, from one rocprofv3 counter pass over
    `bench.py --steps PMC_STEPS --warmup PMC_WARMUP`: clock = GRBM_GUI_ACTIVE
    / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES (summed over the SIMDs)
    / (SIMDS * GRBM_GUI_ACTIVE) (kind "mfma"); or the fraction of wave cycles
    spent waiting (waitcnt and barrier), SQ_WAIT_ANY / SQ_WAVE_CYCLES, and
    the LDS bank-conflict cycles per LDS instruction (kind "stall")."""
    counters = {"mfma": "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
                "stall": "SQ_WAIT_ANY SQ_WAVE_CYCLES SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS "
                         "GRBM_GUI_ACTIVE"}[kind]
    disp = _pmc_dispatches(db, grbm_max=True)
    cmd = (f"rocprofv3 --kernel-include-regex 'moe::' --pmc {counters} -d /tmp/t_{kind} "
           f"-o {workload} -- python3 /root/repo/bench.py --workload {workload} "
           f"--steps {PMC_STEPS} --warmup {PMC_WARMUP} --no-cpu-baseline --no-graph")
    title = {"mfma": "Clock and MFMA utilisation", "stall": "Wait and LDS-conflict cycles"}[kind]
    lines = [f"# {title} of the MoE kernels: {workload}", "",
             f"source_sha256_16: {_source_hash()}", "",
             "One rocprofv3 counter pass.  clock = GRBM_GUI_ACTIVE / duration."]
    if kind == "mfma":
        lines += [f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / ({SIMDS} SIMDs x GRBM_GUI_ACTIVE),",
                  "the fraction of SIMD cycles in which the matrix core is busy.  At the",
                  "nominal 2.4 GHz a fully busy matrix core gives the 2.5 PFLOP/s bf16 peak."]
        head = "| kernel | launch | dispatches | avg duration (us) | clock (GHz) | MFMA busy |"
        sep = "|---|---|---:|---:|---:|---:|"
    else:
        lines += ["wait = SQ_WAIT_ANY / SQ_WAVE_CYCLES: the share of the waves' cycles spent",
                  "in s_waitcnt or at a barrier; LDS conflicts = SQ_LDS_BANK_CONFLICT cycles",
                  "per LDS instruction (SQ_INSTS_LDS)."]
        head = ("| kernel | launch | dispatches | avg duration (us) | clock (GHz) | wait | "
                "LDS conflict cycles / LDS instruction |")
        sep = "|---|---|---:|---:|---:|---:|---:|"
    lines += ["Kernels under 100 us are listed without these figures: GRBM_GUI_ACTIVE",
              "then counts more cycles than the kernel runs.  A grouped GEMM kernel that",
              "runs p times per step (routed experts, then the shared expert) has one row",
              "per launch.", "", "Commands (one MI355X):", "", "```",
              "cd /tmp && export TMPDIR=/tmp", cmd,
              f"python3 /root/repo/bench.py --{kind}-summary /tmp/t_{kind}/{workload}_results.db "
              f"--workload {workload}", "```", "", head, sep]
    for name, launch, d in _launch_rows(disp):
        us = _mean([x[1] for x in d]) / 1e3
        c = {k: _mean([x[0].get(k, 0.0) for x in d]) for k in counters.split()}
        g = c["GRBM_GUI_ACTIVE"]
        if us < 100.0 or not g:  # the counter window outlasts short kernels
            lines.append(f"| `{_short(name)}` | {launch} | {len(d)} | {us:.1f} | - | - |"
                         + (" - |" if kind == "stall" else ""))
            continue
        clock = g / (us * 1e3)
        if kind == "mfma":
            lines.append(f"| `{_short(name)}` | {launch} | {len(d)} | {us:.1f} | {clock:.2f} | "
                         f"{100 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (SIMDS * g):.1f}% |")
        else:
            wait = c["SQ_WAIT_ANY"] / max(c["SQ_WAVE_CYCLES"], 1.0)
            conf = c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_INSTS_LDS"], 1.0)
            lines.append(f"| `{_short(name)}` | {launch} | {len(d)} | {us:.1f} | {clock:.2f} | "
                         f"{100 * wait:.1f}% | {conf:.3f} |")
    return "\n".join(lines) + "\n"


class _F64Experts:
    """Stacked expert weights as the oracle reads them, w[e] -> float64,
    upcast from the stored bf16/fp32 tensor once per expert and kept."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            import torch
            self.cache[e] = self.t[e].to("cpu").to(torch.float64).numpy()
        return self.cache[e]

    def prefetch(self, experts):
        for e in experts:
            self[e]


CPU_F64_CAP = 12e9   # host bytes of float64 expert weights the CPU baseline keeps


def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        info = [d for d in threadpool_info() if d.get("user_api") == "blas"] or threadpool_info()
        d = max(info, key=lambda d: d.get("num_threads", 1))
        return int(d.get("num_threads", 1)), f"{d.get('internal_api')} {d.get('version')}"
    except Exception:  # pragma: no cover
        return os.cpu_count(), "unknown"


def _cpu_baseline(w, inp, target_s):
    """The float64 CPU oracle on the same workload, on this host's cores.

    Inputs are upcast to float64 first (outside the timing): the oracle's
    input format.  When the float64 weights of every expert that keeps a row
    fit in CPU_F64_CAP bytes, the whole layer (oracle.forward) is timed,
    repeated up to ~target_s.  Otherwise (the 256-expert layer: 90 GB in
    float64) the oracle's steps are timed on a bounded sample: routing,
    capacity and permutation of every token; the expert FFNs of an evenly
    spaced sample of the experts with rows, each on all its kept rows; the
    shared expert and the combine on a sample of tokens; each part scaled to
    the whole layer."""
    import numpy as np

    import oracle
    import workloads as W
    threads, blas = _blas_info()
    cores = {"cores": threads, "host_cpus": os.cpu_count(), "blas": blas}
    oi = {k: (_F64Experts(v) if k in ("w_gate", "w_up", "w_down") else W.to_f64(v))
          for k, v in inp.items()}
    kw = dict(top_k=w.top_k, score=w.score, renormalize=w.renormalize,
              route_scale=w.route_scale, n_groups=w.n_groups, topk_groups=w.topk_groups,
              group_rule=w.group_rule)
    t0 = time.perf_counter()
    r = oracle.route(oi["x"], oi["w_router"], w.top_k, score=w.score,
                     renormalize=w.renormalize, route_scale=w.route_scale,
                     logit_bias=oi.get("logit_bias"), select_bias=oi.get("select_bias"),
                     n_groups=w.n_groups, topk_groups=w.topk_groups, group_rule=w.group_rule)
    cap = oracle.capacity(w.capacity_factor, w.T, w.top_k, w.E)
    keep = oracle.first_within_capacity(r["ids"], w.E, cap)
    offsets, r2a, _ = oracle.permutation(r["ids"], keep, w.E)
    t_route = time.perf_counter() - t0
    with_rows = [e for e in range(w.E) if offsets[e + 1] > offsets[e]]
    per_expert = 3.0 * w.D * w.H * 8
    if per_expert * len(with_rows) <= CPU_F64_CAP:
        _log(f"[cpu] upcasting {len(with_rows)} experts to float64")
        for k in ("w_gate", "w_up", "w_down"):
            oi[k].prefetch(with_rows)
        runs = []
        while sum(runs) < target_s and len(runs) < 20:
            t0 = time.perf_counter()
            oracle.forward(oi, capacity_factor=w.capacity_factor, **kw)
            runs.append(time.perf_counter() - t0)
        dt = sum(runs) / len(runs)
        _log(f"[cpu] oracle: whole layer in {dt:.2f}s (mean of {len(runs)})")
        return {"value": w.T / dt, "unit": "tokens/s", **cores, "kind": "oracle",
                "sample": f"the whole layer ({w.T} tokens, {len(with_rows)} experts with "
                          f"rows), oracle.forward in float64, mean of {len(runs)} run(s) of "
                          f"{dt:.2f} s; inputs upcast to float64 beforehand"}
    # bounded sample of the experts, every kept row of each
    n_s = max(1, min(len(with_rows), int(CPU_F64_CAP // per_expert), 32))
    pick = [with_rows[i] for i in np.linspace(0, len(with_rows) - 1, n_s).round().astype(int)]
    pick = sorted(set(pick))
    _log(f"[cpu] upcasting a sample of {len(pick)} of {len(with_rows)} experts to float64")
    for k in ("w_gate", "w_up", "w_down"):
        oi[k].prefetch(pick)
    t0 = time.perf_counter()
    for e in pick:
        a = r2a[offsets[e]:offsets[e + 1]]
        t, sl = a // w.top_k, a % w.top_k
        y = oracle.swiglu_ffn(oi["x"][t], oi["w_gate"][e], oi["w_up"][e], oi["w_down"][e])
        y = r["weights"][t, sl][:, None] * y
    t_exp = time.perf_counter() - t0
    n_tok = min(w.T, 1024)
    toks = np.linspace(0, w.T - 1, n_tok).round().astype(np.int64)
    t0 = time.perf_counter()
    sh = oracle.shared_expert(oi["x"][toks], oi)
    Y = np.zeros((n_tok, w.top_k, w.D))
    oracle.combine(Y, sh)
    t_tok = time.perf_counter() - t0
    dt = t_route + t_exp * len(with_rows) / len(pick) + t_tok * w.T / n_tok
    _log(f"[cpu] oracle: routing {t_route:.2f}s, {len(pick)} experts {t_exp:.2f}s, "
         f"{n_tok} tokens of shared expert + combine {t_tok:.2f}s -> layer {dt:.2f}s")
    return {"value": w.T / dt, "unit": "tokens/s", **cores, "kind": "oracle",
            "sample": f"routing, capacity and permutation of all {w.T} tokens "
                      f"({t_route:.2f} s); the expert FFNs of {len(pick)} evenly spaced of the "
                      f"{len(with_rows)} experts with rows, on all their kept rows "
                      f"({t_exp:.2f} s, scaled by {len(with_rows)}/{len(pick)}); shared expert "
                      f"and combine on {n_tok} evenly spaced tokens ({t_tok:.2f} s, scaled by "
                      f"{w.T}/{n_tok}); float64, inputs upcast beforehand; layer estimate "
                      f"{dt:.2f} s"}


ORDER = ["tiny_dropless_fp32", "switch_top1_capacity", "mixtral_8x_top2",
         "deepseek_v3_256x_top8_grouped", "decode_128x_top8"]
HEADLINE = "mixtral_8x_top2"     # the workload the metric is quoted on


def _bench_workload(w, args, moe, dev):
    """Time W warm-up and K timed steps of workload w; returns its result."""
    import numpy as np
    import torch

    import workloads as W

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
    # One step = one pass of the whole hot path: moe_forward (routing with its
    # auxiliary sums, permutation, grouped SwiGLU (+ shared expert), combine)
    # on inputs resident in HBM; W warm-up steps, then K timed steps between
    # two synchronisations.  The same path is then run as its four C-ABI stage
    # calls (route, permute, grouped SwiGLU, combine) with HIP events recorded
    # between them on the launch stream, for the per-stage times and the
    # roofline of the grouped SwiGLU stage; those calls do a little more than
    # moe_forward (the route call finishes its own counts and losses, the
    # permute call builds its own histogram from the expert IDs).
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
    _log(f"[bench] {w.name}: warmup {args.warmup}")
    for i in range(args.warmup):
        step(events[i % args.steps])
        forward()
    torch.cuda.synchronize()
    _log(f"[bench] {w.name}: timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        forward()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = w.T / (elapsed / args.steps)
    _log(f"[bench] {w.name}: moe_forward {ms_per_step:.3f} ms/step, {tokens_per_s:.4g} tokens/s")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    staged_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    stage_ms = np.array([[ev[i].elapsed_time(ev[i + 1]) for i in range(4)]
                         for ev in events]).mean(axis=0)
    # each staged step on the device clock (HIP events around the step)
    step_dev = np.array([ev[0].elapsed_time(ev[4]) for ev in events])
    _log(f"[bench] {w.name}: staged {staged_ms:.3f} ms/step; stages ms: route %.4f permute %.4f "
         "grouped_swiglu %.4f combine %.4f" % tuple(stage_ms))

    # The grouped SwiGLU stage's launch duration for the roofline: K calls
    # back to back between two events on the launch stream, so the device
    # never waits on the host between them (the per-step events above also
    # hold whatever time the host took to marshal the call's arguments while
    # the device sat idle).  The inter-kernel gaps inside the stage count.
    def gemm_stage():
        moe.moe_grouped_swiglu(cfg, inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"],
                               row_to_assign=perm["row_to_assign"],
                               expert_offsets=perm["expert_offsets"], max_rows_bound=rows_bound,
                               gate_w=r["gate_w"], y_rows=y, workspace=ws, validate=False)
        if w.H_shared:
            moe.moe_grouped_swiglu(cfg, inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"],
                                   y_rows=shared_y, workspace=ws, validate=False)

    bev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    gemm_stage()
    torch.cuda.synchronize()
    bev[0].record(stream)
    for _ in range(args.steps):
        gemm_stage()
    bev[1].record(stream)
    torch.cuda.synchronize()
    gemm_b2b_ms = bev[0].elapsed_time(bev[1]) / args.steps
    _log(f"[bench] {w.name}: grouped_swiglu back to back {gemm_b2b_ms:.4f} ms/launch")
    graph_ms = _graph_ms(forward, args) if not args.no_graph else None
    if graph_ms is not None:
        _log(f"[bench] {w.name}: moe_forward as a replayed HIP graph {graph_ms:.3f} ms/step")

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
    bf16 = w.act_dtype == "bf16"
    esz = 2 if bf16 else 4
    rms_bytes = 2.0 * w.T * w.D * esz + 4.0 * w.D

    # Algorithmic work of the grouped SwiGLU step: 2*D*H FLOP for each of the
    # gate, up and down products per kept row (plus the shared expert on T
    # rows); algorithmic bytes: the three weight matrices of every expert that
    # keeps at least one row (and of the shared expert), x read once and the
    # output written once.  The rows the implementation gathers, its hidden
    # rows and its weighted expert rows are reported beside them.
    kept = np.diff(perm["expert_offsets"].cpu().numpy())
    touched = int((kept > 0).sum())
    flops = 6.0 * w.D * w.H * n_kept + 6.0 * w.D * w.H_shared * w.T
    weight_bytes = 3.0 * w.D * (w.H * touched + w.H_shared) * esz
    nbytes = weight_bytes + 2.0 * w.T * w.D * esz
    inter = {"gathered_rows": n_kept * w.D * esz,
             "hidden_rows_written_and_read": 2.0 * (n_kept * w.H + w.T * w.H_shared) * esz,
             "expert_rows_written_and_read": 2.0 * (n_kept + w.T * (w.H_shared > 0)) * w.D * esz}
    sec = gemm_b2b_ms * 1e-3
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
                "kernel": "grouped_swiglu step (gate/up GEMM + down GEMM"
                          + (", routed and shared expert)" if w.H_shared else ")"),
                "algorithmic_flop_per_launch": flops,
                "algorithmic_bytes_per_launch": nbytes,
                "intermediate_bytes_per_launch": inter,
                "experts_with_rows": touched,
                "tflops": round(flops / sec / 1e12, 2),
                "frac_of_mfma_peak": round(flops / sec / 1e12 / peak_f, 4),
                "hbm_gbs": round(nbytes / sec / 1e9, 1),
                "frac_of_hbm_peak": round(nbytes / sec / 1e9 / PEAK_HBM_GBS, 4),
                "launch_ms": round(gemm_b2b_ms, 4),
                "launch_ms_timing": "mean of K back-to-back calls between two HIP events",
                "staged_step_stage_ms": round(float(stage_ms[2]), 4)}
    # The whole layer (route, permute, grouped SwiGLU, combine): the router
    # GEMM joins the FLOP, its weights the bytes.
    rsz = 4 if w.router_dtype == "f32" else 2
    l_flops = flops + 2.0 * w.T * w.D * w.E
    l_bytes = nbytes + 1.0 * w.E * w.D * rsz
    l_sec = ms_per_step * 1e-3
    layer = {"ms_per_step": round(l_sec * 1e3, 4),
             "algorithmic_flop": l_flops, "algorithmic_bytes": l_bytes,
             "tflops": round(l_flops / l_sec / 1e12, 2),
             "frac_of_mfma_peak": round(l_flops / l_sec / 1e12 / peak_f, 4),
             "hbm_gbs": round(l_bytes / l_sec / 1e9, 1),
             "frac_of_hbm_peak": round(l_bytes / l_sec / 1e9 / PEAK_HBM_GBS, 4)}

    result = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if bf16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d_model": w.D, "d_hidden": w.H,
                   "experts": w.E, "top_k": w.top_k, "shared_d_hidden": w.H_shared,
                   "capacity_factor": w.capacity_factor, "kept_rows": n_kept,
                   "parallelism": "none (1 GPU)"},
        "staged_ms_per_step": round(staged_ms, 4),
        "moe_forward_graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "staged_step_ms_device": {"median": round(float(np.median(step_dev)), 4),
                           "min": round(float(step_dev.min()), 4),
                           "p90": round(float(np.percentile(step_dev, 90)), 4)},
        "stages_ms": {k: round(float(v), 4) for k, v in
                      zip(("route", "permute", "grouped_swiglu", "combine"), stage_ms)},
        "roofline": roofline,
        "layer": layer,
        "beside_the_step": {"rmsnorm_ms": round(rms_ms, 4),
                            "rmsnorm_gbs": round(rms_bytes / (rms_ms * 1e-3) / 1e9, 1)},
    }
    if args.backward:
        result["backward"] = _time_backward(moe, w, cfg, inp, r, n_kept, args.steps, stream)
    del ws, y, shared_y, xn
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(w, inp, args.cpu_seconds)
    del inp
    torch.cuda.empty_cache()
    return result


def _graph_ms(forward, args):
    """ms per step of moe_forward captured once into a HIP graph and replayed
    (the serving form: the same kernels, without the per-launch host work).
    W warm-up replays, then K timed replays between two synchronisations.
    None if the capture fails (the eager figures stand alone then)."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            forward()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            forward()
        for _ in range(max(args.warmup, 1)):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        del g
        return ms
    except Exception as e:  # noqa: BLE001 - report and go on with the eager figures
        _log(f"[bench] HIP graph capture of moe_forward failed: {e}")
        torch.cuda.synchronize()
        return None


def _entry(res):
    """The per-workload summary carried in the headline line."""
    e = {k: res[k] for k in ("value", "unit", "ms_per_step", "staged_ms_per_step",
                             "moe_forward_graph_ms_per_step", "dtype", "stages_ms", "layer")}
    e["tokens_per_s"] = e.pop("value")
    rf = res["roofline"]
    e["grouped_swiglu"] = {k: rf[k] for k in ("bound", "achieved", "unit", "frac", "tflops",
                                              "frac_of_mfma_peak", "hbm_gbs",
                                              "frac_of_hbm_peak", "launch_ms", "traffic",
                                              "experts_with_rows")}
    e["kept_rows"] = res["config"]["kept_rows"]
    if "cpu_baseline" in res:
        e["cpu_baseline"] = res["cpu_baseline"]
    return e


def main():
    args = _parse()
    if args.pmc_summary:
        print(_pmc_summary(*args.pmc_summary, args.workload))
        return
    if args.mfma_summary:
        print(_counter_table(args.mfma_summary, args.workload, "mfma"))
        return
    if args.stall_summary:
        print(_counter_table(args.stall_summary, args.workload, "stall"))
        return
    if args.trace_summary:
        print(_trace_summary(args.trace_summary, args.workload, args.steps, args.warmup))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs on a single MI355X; it shards by expert across GPUs).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_layer_21_amd as moe
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a visible MI355X"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload != "all":
        print(json.dumps(_bench_workload(W.WORKLOADS[args.workload], args, moe, dev)),
              flush=True)
        return
    # Every workload in one process; the headline fields are the Mixtral-shaped
    # layer's, the metric's own configuration.
    results = {}
    for name in ORDER:
        results[name] = _bench_workload(W.WORKLOADS[name], args, moe, dev)
    head = dict(results[HEADLINE])
    head["configs"] = {name: _entry(res) for name, res in results.items()}
    print(json.dumps(head), flush=True)


if __name__ == "__main__":
    main()
