"""GPU parity of the backward pass (moe_backward) against the oracle's float64
gradients of <dout, out> + alpha * balance + beta * z.  The device gets the
oracle's own routes and gate weights, so both sides differentiate the same
routed layer.  On the reduced workloads every element of every gradient is
compared; at full size, sampled tokens and sampled weight-gradient rows.  The
bar is the layer's bf16 tolerance (max|err| <= 2e-2 * max|ref|)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

GRADS = ("dx", "dw_router", "dw_gate", "dw_up", "dw_down")
SHARED = ("dws_gate", "dws_up", "dws_down")


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_layer_21_amd as m
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return m


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _run(moe, w, seed, aux=(0.3, 0.2), token_mask=None, swiglu_limit=0.0, pre_norm=None,
         mutate=None, workspace=None):
    """``pre_norm`` = (norm weight [D] f32 CPU tensor or None, eps): the layer
    takes RMSNorm(x) and x is the input before the norm.  ``mutate`` edits the
    drawn inputs in place before either side sees them."""
    inp = W.make_inputs(w, "cpu", seed=seed)
    if mutate is not None:
        mutate(inp)
    oi = P.oracle_inputs(inp)
    x_route = oi["x"]
    if pre_norm is not None:
        nw, eps = pre_norm
        pre = (np.ones(w.D) if nw is None else nw.to(torch.float64).numpy(),
               float(np.float32(eps)), w.act_dtype)
        x_route = P.oracle.rms_norm(oi["x"], *pre)
    dout = torch.randn(w.T, w.D, generator=torch.Generator().manual_seed(seed + 1)).to(
        W.torch_dtype(w.act_dtype))
    fw = dict(top_k=w.top_k, score=w.score, renormalize=w.renormalize,
              route_scale=w.route_scale, n_groups=w.n_groups, topk_groups=w.topk_groups,
              group_rule=w.group_rule, capacity_factor=w.capacity_factor,
              token_mask=token_mask, swiglu_limit=swiglu_limit)
    ref = P.oracle.backward(oi, dout.to(torch.float64).numpy(), aux_coef=aux,
                            pre_norm=None if pre_norm is None else pre, **fw)
    r = P.oracle.route(x_route, oi["w_router"], w.top_k, score=w.score,
                       renormalize=w.renormalize, route_scale=w.route_scale,
                       logit_bias=oi.get("logit_bias"), select_bias=oi.get("select_bias"),
                       n_groups=w.n_groups, topk_groups=w.topk_groups,
                       group_rule=w.group_rule, token_mask=token_mask)
    d = {k: v.to("cuda") for k, v in inp.items()}
    cfg = P.config_of(w, swiglu_limit=swiglu_limit)
    nw_dev = None
    if pre_norm is not None:
        cfg.pre_norm, cfg.norm_eps = 1, eps
        nw_dev = None if nw is None else nw.cuda()
    ids = torch.from_numpy(r["ids"].astype(np.int32)).cuda()
    gw = torch.from_numpy(r["weights"].astype(np.float32)).cuda()
    _say(f"[backward] {w.name} T={w.T} E={w.E} k={w.top_k} aux={aux} limit={swiglu_limit} "
         f"pre_norm={pre_norm is not None}")
    g = moe.moe_backward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"], ids,
                         gw, dout.cuda(), logit_bias=d.get("logit_bias"),
                         ws_gate=d.get("ws_gate"), ws_up=d.get("ws_up"),
                         ws_down=d.get("ws_down"), balance_coef=aux[0], z_coef=aux[1],
                         d_gate_w=True, norm_weight=nw_dev,
                         shared_expert_gate=d.get("ws_sgate"), workspace=workspace)
    torch.cuda.synchronize()
    return g, ref


def _compare(g, ref, names, what):
    for n in names:
        err, scale = P.compare_rows(g[n], ref[n], "bf16", f"{what} {n}")
        _say(f"  {n}: max|err| {err:.3g} max|ref| {scale:.3g}")


@pytest.mark.parametrize("name", ["mixtral_small", "deepseek_small", "switch_small",
                                  "decode_small"])
def test_backward_matches_oracle(moe, name):
    w = W.SMALL[name]
    g, ref = _run(moe, w, seed=30)
    names = GRADS + (SHARED if w.H_shared else ())
    _compare(g, ref, names + ("d_gate_w",), name)
    g2, _ = _run(moe, w, seed=30)
    for n in names:  # deterministic: a second call gives the same bits
        assert torch.equal(g[n], g2[n]), n


def test_backward_256_experts(moe):
    """256 experts, the most the library takes: the padded offsets of the
    ragged-K weight-gradient GEMMs have 257 entries, one more than the
    threads of the kernel that writes them.  On a zero-filled workspace a
    missing last entry would leave the last expert without gradient."""
    w = W.Workload("bwd_256", 1, 600, D=192, H=128, E=256, top_k=4)
    cfg = P.config_of(w)
    ws = torch.zeros(moe.backward_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    g, ref = _run(moe, w, seed=33, workspace=ws)
    _compare(g, ref, GRADS + ("d_gate_w",), "256 experts")


def test_backward_without_aux_terms(moe):
    """alpha = beta = 0: the router gradient comes from the gate weights only."""
    w = W.SMALL["mixtral_small"]
    g, ref = _run(moe, w, seed=31, aux=(0.0, 0.0))
    _compare(g, ref, GRADS, "no aux")


def test_backward_token_mask_and_clamp(moe):
    """Masked tokens (IDs -1) get no expert or router gradient; the SwiGLU
    clamp passes gradient only inside its limits."""
    w = W.SMALL["deepseek_small"]
    mask = np.random.default_rng(32).random(w.T) >= 0.3
    g, ref = _run(moe, w, seed=32, token_mask=mask, swiglu_limit=0.05)
    _compare(g, ref, GRADS + SHARED + ("d_gate_w",), "masked, clamped")
    assert (g["d_gate_w"].cpu().numpy()[~mask] == 0).all()


@pytest.mark.parametrize("name,unit_weight", [("mixtral_small", False),
                                              ("deepseek_small", False),
                                              ("decode_small", True)])
def test_backward_pre_norm(moe, name, unit_weight):
    """Backward of MoE(RMSNorm(x)): every gradient, and dL/d norm weight,
    through the norm against the oracle's chain rule; deterministic."""
    w = W.SMALL[name]
    nw = None if unit_weight else \
        torch.rand(w.D, generator=torch.Generator().manual_seed(34)) + 0.5
    g, ref = _run(moe, w, seed=34, pre_norm=(nw, 1e-5))
    names = GRADS + (SHARED if w.H_shared else ()) + ("d_gate_w", "d_norm_weight")
    _compare(g, ref, names, f"{name} pre-norm")
    g2, _ = _run(moe, w, seed=34, pre_norm=(nw, 1e-5))
    for n in names:
        assert torch.equal(g[n], g2[n]), n


def test_norm_weight_needs_pre_norm_backward(moe):
    w = W.SMALL["mixtral_small"]
    d = {k: v.to("cuda") for k, v in W.make_inputs(w, "cpu", seed=35).items()}
    ids = torch.zeros(w.T, w.top_k, dtype=torch.int32, device="cuda")
    ids[:, 1] = 1
    gw = torch.full((w.T, w.top_k), 0.5, device="cuda")
    with pytest.raises(moe.MoeError, match="pre_norm"):
        moe.moe_backward(P.config_of(w), d["x"], d["w_router"], d["w_gate"], d["w_up"],
                         d["w_down"], ids, gw, d["x"], norm_weight=torch.ones(w.D, device="cuda"))


def test_backward_single_token(moe):
    w = W.Workload("one", 1, 1, D=128, H=64, E=8, top_k=3)
    g, ref = _run(moe, w, seed=36)
    _compare(g, ref, GRADS + ("d_gate_w",), "single token")


def test_backward_zero_router_leaves_experts_empty(moe):
    """A zero router sends every token to experts 0..k-1 (ties to the lower
    index): the other experts get exactly zero weight gradients."""
    w = W.Workload("zero", 1, 70, D=128, H=64, E=8, top_k=3)
    g, ref = _run(moe, w, seed=37, mutate=lambda inp: inp["w_router"].zero_())
    _compare(g, ref, GRADS + ("d_gate_w",), "zero router")
    for n in ("dw_gate", "dw_up", "dw_down"):
        assert not g[n][3:].any(), n


def test_backward_dense_limit(moe):
    """top_k = E: every expert sees every token."""
    w = W.Workload("dense", 1, 45, D=64, H=128, E=4, top_k=4, w_std=0.1)
    g, ref = _run(moe, w, seed=38)
    _compare(g, ref, GRADS + ("d_gate_w",), "top_k = E")


def test_backward_all_tokens_masked(moe):
    """No valid token: no expert row, no auxiliary term; every gradient is
    exactly zero on both sides."""
    w = W.SMALL["mixtral_small"]
    mask = np.zeros(w.T, dtype=bool)
    g, ref = _run(moe, w, seed=39, token_mask=mask)
    for n in GRADS + ("d_gate_w",):
        assert not np.abs(ref[n]).any(), n
        assert not g[n].any(), n


@pytest.mark.parametrize("T,E,k", [(2000, 4, 2), (1111, 2, 1)])
def test_backward_large_ragged_tiles(moe, T, E, k):
    """Hundreds of rows per expert with ragged tails: several 256-row tiles
    and 64-row k blocks per expert in every backward GEMM."""
    w = W.Workload("ragged", 1, T, D=256, H=192, E=E, top_k=k, w_std=0.05)
    g, ref = _run(moe, w, seed=40)
    _compare(g, ref, GRADS + ("d_gate_w",), f"T={T} E={E} k={k}")


def _with_shared_gate(seed):
    def mutate(inp):
        g = torch.Generator().manual_seed(seed)
        inp["ws_sgate"] = (torch.randn(inp["x"].shape[1], generator=g) * 0.05).to(
            inp["x"].dtype)
    return mutate


@pytest.mark.parametrize("pre_norm", [False, True])
def test_backward_gated_shared_expert(moe, pre_norm):
    """Shared expert scaled by sigmoid(x . w_sg): every gradient, and
    dL/dw_sg, against the oracle; with the pre-norm the gate sees the
    normalised rows."""
    w = W.SMALL["deepseek_small"]
    nw = torch.rand(w.D, generator=torch.Generator().manual_seed(41)) + 0.5
    g, ref = _run(moe, w, seed=41, mutate=_with_shared_gate(42),
                  pre_norm=(nw, 1e-5) if pre_norm else None)
    names = GRADS + SHARED + ("d_gate_w", "d_shared_gate") + (
        ("d_norm_weight",) if pre_norm else ())
    _compare(g, ref, names, "gated shared expert")


@pytest.mark.parametrize("name", ["mixtral_small", "deepseek_small", "switch_small",
                                  "decode_small"])
def test_backward_with_saved_state(moe, name):
    """moe_forward(saved=...) keeps the SwiGLU state and moe_backward(saved=...)
    skips the gate/up recompute: the forward output is unchanged by saving,
    and the gradients still match the oracle.  (The device's routes equal the
    oracle's at this seed, so the saved rows are the oracle's rows.)"""
    w = W.SMALL[name]
    inp = W.make_inputs(w, "cpu", seed=43)
    oi = P.oracle_inputs(inp)
    r = P.oracle_route(w, oi)
    d = {k: v.to("cuda") for k, v in inp.items()}
    cfg = P.config_of(w)
    ids = torch.empty(w.T, w.top_k, dtype=torch.int32, device="cuda")
    gw = torch.empty(w.T, w.top_k, dtype=torch.float32, device="cuda")
    kw = dict(logit_bias=d.get("logit_bias"), select_bias=d.get("select_bias"),
              ws_gate=d.get("ws_gate"), ws_up=d.get("ws_up"), ws_down=d.get("ws_down"))
    saved = moe.new_saved(cfg)
    _say(f"[saved state] {name}: forward with and without saving")
    out = moe.moe_forward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                          expert_ids=ids, gate_w=gw, saved=saved, **kw)
    plain = moe.moe_forward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                            **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    assert (ids.cpu().numpy() == r["ids"]).all()
    dout = torch.randn(w.T, w.D, generator=torch.Generator().manual_seed(44)).to(
        W.torch_dtype(w.act_dtype))
    aux = (0.3, 0.2)
    fw = dict(top_k=w.top_k, score=w.score, renormalize=w.renormalize,
              route_scale=w.route_scale, n_groups=w.n_groups, topk_groups=w.topk_groups,
              group_rule=w.group_rule, capacity_factor=w.capacity_factor)
    ref = P.oracle.backward(oi, dout.to(torch.float64).numpy(), aux_coef=aux, **fw)
    _say(f"[saved state] {name}: backward on the saved state")
    g = moe.moe_backward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                         torch.from_numpy(r["ids"].astype(np.int32)).cuda(),
                         torch.from_numpy(r["weights"].astype(np.float32)).cuda(), dout.cuda(),
                         logit_bias=d.get("logit_bias"), ws_gate=d.get("ws_gate"),
                         ws_up=d.get("ws_up"), ws_down=d.get("ws_down"), balance_coef=aux[0],
                         z_coef=aux[1], d_gate_w=True, saved=saved)
    torch.cuda.synchronize()
    names = GRADS + (SHARED if w.H_shared else ()) + ("d_gate_w",)
    _compare(g, ref, names, f"{name} with saved state")


def test_backward_saved_state_clamp_gate_pre_norm(moe):
    """Saved state with the SwiGLU clamp (the forward's epilogues then store
    the clamped factors), the gated shared expert and the pre-norm together."""
    w = W.SMALL["deepseek_small"]
    limit, eps = 0.05, 1e-5
    inp = W.make_inputs(w, "cpu", seed=45)
    _with_shared_gate(46)(inp)
    nw = torch.rand(w.D, generator=torch.Generator().manual_seed(47)) + 0.5
    oi = P.oracle_inputs(inp)
    pre = (nw.to(torch.float64).numpy(), float(np.float32(eps)), w.act_dtype)
    r = P.oracle_route(w, dict(oi, x=P.oracle.rms_norm(oi["x"], *pre)))
    d = {k: v.to("cuda") for k, v in inp.items()}
    cfg = P.config_of(w, swiglu_limit=limit)
    cfg.pre_norm, cfg.norm_eps = 1, eps
    ids = torch.empty(w.T, w.top_k, dtype=torch.int32, device="cuda")
    kw = dict(logit_bias=d.get("logit_bias"), ws_gate=d["ws_gate"], ws_up=d["ws_up"],
              ws_down=d["ws_down"])
    saved = moe.new_saved(cfg)
    moe.moe_forward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                    select_bias=d.get("select_bias"), expert_ids=ids, saved=saved,
                    norm_weight=nw.cuda(), shared_expert_gate=d["ws_sgate"], **kw)
    torch.cuda.synchronize()
    assert (ids.cpu().numpy() == r["ids"]).all()
    dout = torch.randn(w.T, w.D, generator=torch.Generator().manual_seed(48)).to(
        W.torch_dtype(w.act_dtype))
    aux = (0.3, 0.2)
    fw = dict(top_k=w.top_k, score=w.score, renormalize=w.renormalize,
              route_scale=w.route_scale, n_groups=w.n_groups, topk_groups=w.topk_groups,
              group_rule=w.group_rule, capacity_factor=w.capacity_factor, swiglu_limit=limit)
    ref = P.oracle.backward(oi, dout.to(torch.float64).numpy(), aux_coef=aux, pre_norm=pre, **fw)
    g = moe.moe_backward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                         torch.from_numpy(r["ids"].astype(np.int32)).cuda(),
                         torch.from_numpy(r["weights"].astype(np.float32)).cuda(), dout.cuda(),
                         balance_coef=aux[0], z_coef=aux[1], d_gate_w=True, saved=saved,
                         norm_weight=nw.cuda(), shared_expert_gate=d["ws_sgate"], **kw)
    torch.cuda.synchronize()
    _compare(g, ref, GRADS + SHARED + ("d_gate_w", "d_shared_gate", "d_norm_weight"),
             "saved state, clamp, gate, pre-norm")


def test_backward_dropped_slots(moe):
    """Capacity drops: a dropped slot's dL/dw is exactly 0."""
    w = W.SMALL["switch_small"]
    g, ref = _run(moe, w, seed=33)
    keep = P.oracle.forward(P.oracle_inputs(W.make_inputs(w, "cpu", seed=33)),
                            top_k=w.top_k, score=w.score, renormalize=w.renormalize,
                            capacity_factor=w.capacity_factor)["keep"]
    assert (~keep).any()
    assert (g["d_gate_w"].cpu().numpy()[~keep] == 0).all()


# ------------------------------------------------------------- full size ---

def _sampled_weight_rows(g, r, keep, oi, do, w, rng, what, n_experts=3):
    """Rows h of dW_gate/dW_up and columns h of dW_down of sampled experts
    from the one-unit FFN of h over all of the expert's kept rows."""
    kept_rows = [np.nonzero((r["ids"] == e) & keep) for e in range(w.E)]
    with_rows = [e for e in range(w.E) if kept_rows[e][0].size]
    pick = rng.choice(with_rows, size=min(n_experts, len(with_rows)), replace=False)
    for e in pick:
        t, s_ = kept_rows[e]
        dF = r["weights"][t, s_][:, None] * do[t]
        for h in rng.choice(w.H, size=2, replace=False):
            _, dwg, dwu, dwd, _ = P.oracle.swiglu_ffn_backward(
                oi["x"][t], oi["w_gate"][e][h:h + 1], oi["w_up"][e][h:h + 1],
                oi["w_down"][e][:, h:h + 1], dF)
            tag = f"{what} expert {e} unit {h}"
            P.compare_rows(g["dw_gate"][e, h], dwg[0], "bf16", tag + " dW_gate row")
            P.compare_rows(g["dw_up"][e, h], dwu[0], "bf16", tag + " dW_up row")
            P.compare_rows(g["dw_down"][e, :, h], dwd[:, 0], "bf16", tag + " dW_down column")
    return kept_rows, with_rows, pick


def test_backward_beyond_32bit_offsets(moe):
    """Backward of a layer whose input passes 2 GB (most operands beyond the
    32-bit buffer offsets: the register-staged GEMM path): dx on sampled
    tokens and sampled weight-gradient rows."""
    w = W.Workload("beyond_2gb", 1, 262144, D=4096, H=64, E=8, top_k=2)
    _say(f"[backward beyond 2 GB] T={w.T}: drawing inputs")
    inp = {k: v.to("cuda") for k, v in W.make_inputs(w, "cuda", seed=23).items()}
    oi = P.oracle_inputs(inp)
    r = P.oracle_route(w, oi)
    keep = r["ids"] >= 0
    gen = torch.Generator(device="cuda")
    gen.manual_seed(24)
    dout = torch.randn(w.T, w.D, generator=gen, device="cuda").to(torch.bfloat16)
    aux = (0.01, 0.001)
    g = moe.moe_backward(P.config_of(w), inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                         inp["w_down"], torch.from_numpy(r["ids"].astype(np.int32)).cuda(),
                         torch.from_numpy(r["weights"].astype(np.float32)).cuda(), dout,
                         balance_coef=aux[0], z_coef=aux[1], d_gate_w=True)
    torch.cuda.synchronize()
    do = dout.to(torch.float64).cpu().numpy()
    rng = np.random.default_rng(25)
    toks = np.unique(np.concatenate([rng.choice(w.T, 12, replace=False), [0, w.T - 1]]))
    dx = np.zeros((toks.size, w.D))
    dgw = np.zeros_like(r["weights"])
    for i, t in enumerate(toks):
        for s_ in range(w.top_k):
            e = r["ids"][t, s_]
            dz, _, _, _, F = P.oracle.swiglu_ffn_backward(
                oi["x"][t:t + 1], oi["w_gate"][e], oi["w_up"][e], oi["w_down"][e],
                r["weights"][t, s_] * do[t:t + 1])
            dx[i] += dz[0]
            dgw[t, s_] = float(np.sum(do[t] * F[0]))
    dx += P.oracle.router_backward(r, dgw, top_k=w.top_k, aux_coef=aux, tokens=toks) @ \
        oi["w_router"]
    sel = torch.from_numpy(toks).cuda()
    P.compare_rows(g["dx"][sel], dx, "bf16", "beyond 2 GB dx on sampled tokens")
    P.compare_rows(g["d_gate_w"][sel], dgw[toks], "bf16", "beyond 2 GB dL/dw")
    _sampled_weight_rows(g, r, keep, oi, do, w, rng, "beyond 2 GB", n_experts=2)


FULL = ["mixtral_8x_top2", "switch_top1_capacity", "decode_128x_top8",
        "deepseek_v3_256x_top8_grouped"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_backward(moe, name):
    """Full-size workload as bench.py draws it, on the oracle's routes: dx and
    dL/dw on sampled tokens, and whole weight-gradient rows for sampled
    (expert, hidden unit) pairs.  A SwiGLU FFN is a sum over its hidden units,
    so the one-unit FFN of unit h gives exactly row h of dW_gate and dW_up and
    column h of dW_down from all of the expert's rows."""
    w = W.WORKLOADS[name]
    _say(f"[full backward] {name}: drawing inputs")
    inp = {k: v.to("cuda") for k, v in W.make_inputs(w, "cuda", seed=0).items()}
    oi = P.oracle_inputs(inp)
    aux = (0.01, 0.001)
    _say(f"[full backward] {name}: oracle routing")
    r = P.oracle_route(w, oi)
    cap = P.oracle.capacity(w.capacity_factor, w.T, w.top_k, w.E)
    keep = P.oracle.first_within_capacity(r["ids"], w.E, cap)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    dout = torch.randn(w.T, w.D, generator=gen, device="cuda").to(torch.bfloat16)
    cfg = P.config_of(w)
    _say(f"[full backward] {name}: moe_backward")
    g = moe.moe_backward(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                         inp["w_down"], torch.from_numpy(r["ids"].astype(np.int32)).cuda(),
                         torch.from_numpy(r["weights"].astype(np.float32)).cuda(), dout,
                         logit_bias=inp.get("logit_bias"), ws_gate=inp.get("ws_gate"),
                         ws_up=inp.get("ws_up"), ws_down=inp.get("ws_down"),
                         balance_coef=aux[0], z_coef=aux[1], d_gate_w=True)
    torch.cuda.synchronize()
    x, do = oi["x"], dout.to(torch.float64).cpu().numpy()
    experts = {}  # float64 weights of each expert the samples reach, converted once

    def expert(e):
        if e not in experts:
            experts[e] = (oi["w_gate"][e], oi["w_up"][e], oi["w_down"][e])
        return experts[e]
    # sampled tokens: experts' input gradients, dL/dw, and the router's share
    rng = np.random.default_rng(3)
    toks = np.unique(np.concatenate([rng.choice(w.T, 16, replace=False), [0, w.T - 1],
                                     np.nonzero(~keep.any(1))[0][:4]]))
    _say(f"[full backward] {name}: oracle on {toks.size} tokens")
    dx = np.zeros((toks.size, w.D))
    dgw = np.zeros_like(r["weights"])
    for i, t in enumerate(toks):
        for s_ in range(w.top_k):
            if not keep[t, s_]:
                continue
            e = r["ids"][t, s_]
            dz, _, _, _, F = P.oracle.swiglu_ffn_backward(x[t:t + 1], *expert(e),
                                                          r["weights"][t, s_] * do[t:t + 1])
            dx[i] += dz[0]
            dgw[t, s_] = float(np.sum(do[t] * F[0]))
    if w.H_shared:  # the ungated shared expert sees every token with weight 1
        dz, _, _, _, _ = P.oracle.swiglu_ffn_backward(x[toks], oi["ws_gate"], oi["ws_up"],
                                                      oi["ws_down"], do[toks])
        dx += dz
    dh = P.oracle.router_backward(r, dgw, top_k=w.top_k, score=w.score,
                                  renormalize=w.renormalize, route_scale=w.route_scale,
                                  aux_coef=aux, tokens=toks)
    dx += dh @ oi["w_router"]
    sel = torch.from_numpy(toks).cuda()
    P.compare_rows(g["dx"][sel], dx, "bf16", f"{name} dx on sampled tokens")
    P.compare_rows(g["d_gate_w"][sel], dgw[toks], "bf16", f"{name} dL/dw on sampled tokens")
    assert (g["d_gate_w"].cpu().numpy()[~keep] == 0).all()
    # weight-gradient rows of sampled experts and hidden units
    kept_rows = [np.nonzero((r["ids"] == e) & keep) for e in range(w.E)]
    with_rows = [e for e in range(w.E) if kept_rows[e][0].size]
    pick = rng.choice(with_rows, size=min(3, len(with_rows)), replace=False)
    for e in pick:
        t, s_ = kept_rows[e]
        dF = r["weights"][t, s_][:, None] * do[t]
        for h in rng.choice(w.H, size=2, replace=False):
            _, dwg, dwu, dwd, _ = P.oracle.swiglu_ffn_backward(
                x[t], oi["w_gate"][e][h:h + 1], oi["w_up"][e][h:h + 1],
                oi["w_down"][e][:, h:h + 1], dF)
            what = f"{name} expert {e} unit {h}"
            P.compare_rows(g["dw_gate"][e, h], dwg[0], "bf16", what + " dW_gate row")
            P.compare_rows(g["dw_up"][e, h], dwu[0], "bf16", what + " dW_up row")
            P.compare_rows(g["dw_down"][e, :, h], dwd[:, 0], "bf16", what + " dW_down column")
    for e in range(w.E):
        if not kept_rows[e][0].size:  # an expert without rows gets exactly zero
            assert not g["dw_gate"][e].any() and not g["dw_down"][e].any()
            break
    if w.H_shared:  # whole weight-gradient rows of sampled shared-expert units
        for h in rng.choice(w.H_shared, size=2, replace=False):
            _, dwg, dwu, dwd, _ = P.oracle.swiglu_ffn_backward(
                x, oi["ws_gate"][h:h + 1], oi["ws_up"][h:h + 1], oi["ws_down"][:, h:h + 1], do)
            what = f"{name} shared expert unit {h}"
            P.compare_rows(g["dws_gate"][h], dwg[0], "bf16", what + " dW_gate row")
            P.compare_rows(g["dws_up"][h], dwu[0], "bf16", what + " dW_up row")
            P.compare_rows(g["dws_down"][:, h], dwd[:, 0], "bf16", what + " dW_down column")
    _say(f"[full backward] {name}: {len(with_rows)} experts with rows; checked {list(pick)}")
