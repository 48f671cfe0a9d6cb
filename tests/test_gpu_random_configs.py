"""Seeded random layer configurations through the whole forward, against the
oracle.

Each configuration draws its expert count, top-k, widths, batch, score
function, renormalisation, group limit, capacity factor, shared expert,
biases and router dtype from a fixed-seed generator, with the batch chosen
so that the average rows per expert fall in each of the grouped GEMM's row
bands (decode-sized, 64-191 and 192 or more).  The forward is compared as in
the other parity tests: expert IDs bit-exact outside the oracle's flagged
near ties, gate weights within 1e-5, counts exact, and every comparable
token's output within the bf16 tolerance ("Lab: build a tiny MoE in
PyTorch", "Required correctness tests").  The configurations themselves are
checked on the CPU against the library's host-side validation."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import workloads as W
from tests import parity as P


def _configs(n=48, seed=1204, act="bf16"):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 40, 64, 96, 128, 160, 200, 256]))
        k = int(rng.integers(1, min(E, 8) + 1))
        if act == "bf16":  # the bf16 path takes widths in multiples of 64
            D = int(rng.choice([64, 128, 192, 256, 512]))
            H = int(rng.choice([64, 128, 192, 320, 512]))
        else:
            D = int(rng.choice([48, 80, 96, 144, 256]))
            H = int(rng.choice([32, 48, 112, 128, 200]))
        rows_per_expert = int(rng.choice([8, 40, 100, 160, 300]))
        T = int(np.clip(rows_per_expert * E // k + rng.integers(-7, 8), 1, 3000))
        while T > 1 and T * k * D * H > 3e8:  # keeps the float64 oracle to about a second
            T //= 2
        score = str(rng.choice(["softmax", "sigmoid", "sqrtsoftplus"]))
        renorm = bool(rng.integers(0, 2)) if score == "softmax" else True
        n_groups, topk_groups = 1, 1
        if E % 8 == 0 and E >= 32 and rng.random() < 0.5:
            n_groups = 8
            lo = -(-k // (E // 8))  # enough groups to hold k experts
            topk_groups = int(rng.integers(lo, 9))
        cf = None if rng.random() < 0.5 else float(rng.choice([0.5, 1.0, 1.25, 2.0]))
        Hs = 0 if rng.random() < 0.7 else int(rng.choice([64, 128]))
        out.append(W.Workload(
            f"random{i}" if act == "bf16" else f"random_f32_{i}", batch=1, seq=T, D=D, H=H,
            E=E, top_k=k, act_dtype=act,
            router_dtype="f32" if rng.random() < 0.25 else "bf16", score=score,
            renormalize=renorm, route_scale=1.0 if score == "softmax" else 2.5,
            n_groups=n_groups, topk_groups=topk_groups,
            group_rule=str(rng.choice(["top2sum", "max"])), capacity_factor=cf, H_shared=Hs,
            logit_bias=str(rng.choice(["none", "gauss", "zipf"])), gauss_sigma=0.5,
            select_bias_sigma=0.05 if rng.random() < 0.4 else 0.0))
    return out


# bf16 layers first (the forward, backward and variant tests index these),
# then fp32 layers (forward only: the backward is bf16).
CONFIGS = _configs() + _configs(12, seed=1205, act="f32")
N_BF16 = 48


def _describe(w):
    return (f"T={w.T} D={w.D} H={w.H} E={w.E} k={w.top_k} {w.score} renorm={w.renormalize} "
            f"groups={w.n_groups}/{w.topk_groups} cf={w.capacity_factor} Hs={w.H_shared} "
            f"router={w.router_dtype} bias={w.logit_bias} sel={w.select_bias_sigma}")


def test_random_configs_are_valid():
    import mixture_experts_layer_21_amd as moe
    bands = set()
    for w in CONFIGS:
        moe.check_config(P.config_of(w))
        rows = w.T * w.top_k / w.E
        bands.add(0 if rows < 64 else 1 if rows < 192 else 2)
    assert bands == {0, 1, 2}, "the configurations cover every row band"


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(len(CONFIGS)))
def test_random_config(i):
    import mixture_experts_layer_21_amd as moe
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    w = CONFIGS[i]
    print(f"[random] {w.name}: {_describe(w)}", file=sys.stderr, flush=True)
    inp = W.make_inputs(w, "cpu", seed=100 + i)
    d = {kk: v.to("cuda") for kk, v in inp.items()}
    cfg = P.config_of(w)
    ids = torch.empty(w.T, w.top_k, dtype=torch.int32, device="cuda")
    gw = torch.empty(w.T, w.top_k, dtype=torch.float32, device="cuda")
    out = moe.moe_forward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                          logit_bias=d.get("logit_bias"), select_bias=d.get("select_bias"),
                          ws_gate=d.get("ws_gate"), ws_up=d.get("ws_up"),
                          ws_down=d.get("ws_down"), expert_ids=ids, gate_w=gw)
    g = moe.moe_route(cfg, d["x"], d["w_router"], d.get("logit_bias"), d.get("select_bias"))
    torch.cuda.synchronize()
    assert torch.equal(g["expert_ids"], ids) and torch.equal(g["gate_w"], gw)
    oi = P.oracle_inputs(inp)
    r = P.oracle_route(w, oi)
    nflag, ndiff = P.compare_route(w, r, g)
    f = P.oracle_forward(w, oi)
    err, scale = P.compare_tokens(out, f["out"], P.comparable_tokens(w, r["ids"], ids),
                                  w.act_dtype, f"{w.name} forward")
    print(f"  near ties {nflag} (differing {ndiff}), max|err| {err:.3g} max|ref| {scale:.3g}",
          file=sys.stderr, flush=True)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(0, N_BF16, 2))
def test_random_config_backward(i):
    """Every gradient of every other configuration above (the device on the
    oracle's routes), every element, at the layer's bf16 tolerance ("Lab:
    build a tiny MoE in PyTorch", "Smoke test and backward pass")."""
    import mixture_experts_layer_21_amd as moe
    from tests.test_gpu_backward import GRADS, SHARED, _compare, _run
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    w = CONFIGS[i]
    print(f"[random-backward] {w.name}: {_describe(w)}", file=sys.stderr, flush=True)
    g, ref = _run(moe, w, seed=200 + i)
    names = GRADS + (SHARED if w.H_shared else ())
    _compare(g, ref, names + ("d_gate_w",), w.name)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(1, N_BF16, 2))
def test_random_config_variants(i):
    """The other half of the configurations with a seeded choice of the
    forward's variants: a token (padding) mask, the SwiGLU clamp, the
    residual add, the RMSNorm pre-norm and the gated shared expert ([NEMO]
    ``token_mask``, ``swiglu_limit``, ``shared_expert_gate``; "Lab: build a
    tiny MoE in PyTorch", "Put the MoE into a decoder block")."""
    import mixture_experts_layer_21_amd as moe
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    w = CONFIGS[i]
    rng = np.random.default_rng(500 + i)
    use_mask = bool(rng.random() < 0.5)
    limit = float(rng.choice([0.0, 0.05, 0.5]))
    use_res = bool(rng.random() < 0.5)
    use_pre = bool(rng.random() < 0.4)
    use_gate = bool(w.H_shared > 0 and rng.random() < 0.6)
    print(f"[random-variants] {w.name}: {_describe(w)} mask={use_mask} limit={limit} "
          f"residual={use_res} pre_norm={use_pre} shared_gate={use_gate}",
          file=sys.stderr, flush=True)
    inp = W.make_inputs(w, "cpu", seed=300 + i)
    if use_gate:
        gen = torch.Generator().manual_seed(300 + i)
        inp["ws_sgate"] = (torch.randn(w.D, generator=gen) / w.D ** 0.5).to(
            W.torch_dtype(w.act_dtype))
    d = {kk: v.to("cuda") for kk, v in inp.items()}
    cfg = P.config_of(w, swiglu_limit=limit)
    mask = None
    kw = {}
    if use_mask:
        mask = rng.random(w.T) >= 0.3
        kw["token_mask"] = torch.from_numpy(mask).cuda()
    if use_res:
        kw["residual"] = d["x"]
    nw = None
    if use_pre:
        cfg.pre_norm, cfg.norm_eps = 1, 1e-5
        nw = torch.rand(w.D, generator=torch.Generator().manual_seed(400 + i)) + 0.5
        kw["norm_weight"] = nw.cuda()
    if use_gate:
        kw["shared_expert_gate"] = d["ws_sgate"]
    ids = torch.empty(w.T, w.top_k, dtype=torch.int32, device="cuda")
    gw = torch.empty(w.T, w.top_k, dtype=torch.float32, device="cuda")
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    aux = torch.empty(2, dtype=torch.float32, device="cuda")
    out = moe.moe_forward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                          logit_bias=d.get("logit_bias"), select_bias=d.get("select_bias"),
                          ws_gate=d.get("ws_gate"), ws_up=d.get("ws_up"),
                          ws_down=d.get("ws_down"), expert_ids=ids, gate_w=gw, counts=counts,
                          aux=aux, **kw)
    x_dev = moe.moe_rmsnorm(cfg, d["x"], nw.cuda()) if use_pre else d["x"]
    g = moe.moe_route(cfg, x_dev, d["w_router"], d.get("logit_bias"), d.get("select_bias"),
                      token_mask=kw.get("token_mask"))
    torch.cuda.synchronize()
    assert torch.equal(g["expert_ids"], ids) and torch.equal(g["gate_w"], gw)
    oi = P.oracle_inputs(inp)
    pre = None
    x_route = oi["x"]
    if use_pre:
        pre = (nw.to(torch.float64).numpy(), float(np.float32(1e-5)), w.act_dtype)
        x_route = P.oracle.rms_norm(oi["x"], *pre)
    r = P.oracle_route(w, dict(oi, x=x_route), token_mask=mask)
    nflag, ndiff = P.compare_route(w, r, {"expert_ids": ids, "gate_w": gw, "counts": counts,
                                          "aux": aux, "mean_prob": g["mean_prob"]})
    f = P.oracle_forward(w, oi, token_mask=mask, swiglu_limit=limit,
                         residual=oi["x"] if use_res else None, pre_norm=pre)
    err, scale = P.compare_tokens(out, f["out"], P.comparable_tokens(w, r["ids"], ids),
                                  w.act_dtype, f"{w.name} forward variants")
    print(f"  near ties {nflag} (differing {ndiff}), max|err| {err:.3g} max|ref| {scale:.3g}",
          file=sys.stderr, flush=True)
