"""GPU parity of the forward variants named on the NeMo AutoModel MoE page:
score functions (sqrt-softplus; softmax with a selection bias; softmax-then-
top-k without renormalisation for k > 1), the token (padding) mask, the
clamped SwiGLU (swiglu_limit) and the gated shared expert, and the steps on
either side of the layer (RMSNorm pre-norm, residual add, bias update), each
against the CPU oracle on the reduced workloads (every output element
compared)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_layer_21_amd as m
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return m


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _to_dev(inp):
    return {k: v.to("cuda") for k, v in inp.items()}


def _mask(T, seed, frac=0.3):
    g = np.random.default_rng(seed)
    m = g.random(T) >= frac
    m[0] = False           # the first token of the first tile is padding
    return m


def _forward(moe, w, cfg, d, **kw):
    ids = torch.empty(w.T, w.top_k, dtype=torch.int32, device="cuda")
    gw = torch.empty(w.T, w.top_k, dtype=torch.float32, device="cuda")
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    aux = torch.empty(2, dtype=torch.float32, device="cuda")
    out = moe.moe_forward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                          logit_bias=d.get("logit_bias"), select_bias=d.get("select_bias"),
                          ws_gate=d.get("ws_gate"), ws_up=d.get("ws_up"),
                          ws_down=d.get("ws_down"), expert_ids=ids, gate_w=gw, counts=counts,
                          aux=aux, **kw)
    torch.cuda.synchronize()
    return out, ids, gw, counts, aux


SCORE_CASES = [
    # workload, score, renormalize, selection bias sigma, k override
    ("mixtral_small", "sqrtsoftplus", True, 0.0, None),
    ("deepseek_small", "sqrtsoftplus", True, 0.01, None),
    ("decode_small", "softmax", False, 0.0, 4),
    ("mixtral_small", "softmax", True, 0.01, None),
    ("switch_small", "sqrtsoftplus", False, 0.0, None),
]


@pytest.mark.parametrize("name,score,renorm,sb,k", SCORE_CASES)
def test_route_score_variants(moe, name, score, renorm, sb, k):
    w = W.SMALL[name].with_(score=score, renormalize=renorm, select_bias_sigma=sb,
                            top_k=k or W.SMALL[name].top_k)
    _say(f"[score] {name} {score} renorm={renorm} sb={sb} k={w.top_k}")
    inp = W.make_inputs(w, "cpu", seed=11)
    d = _to_dev(inp)
    cfg = P.config_of(w)
    g = moe.moe_route(cfg, d["x"], d["w_router"], d.get("logit_bias"), d.get("select_bias"))
    torch.cuda.synchronize()
    r = P.oracle_route(w, P.oracle_inputs(inp))
    nflag, ndiff = P.compare_route(w, r, g)
    _say(f"  near ties flagged {nflag}, differing {ndiff}")
    if not renorm and score == "softmax":
        assert (g["gate_w"].sum(1) < 1.0).all()


@pytest.mark.parametrize("name", sorted(W.SMALL))
def test_forward_token_mask(moe, name):
    w = W.SMALL[name]
    _say(f"[mask] {name}")
    inp = W.make_inputs(w, "cpu", seed=12)
    d = _to_dev(inp)
    cfg = P.config_of(w)
    mask = _mask(w.T, 12)
    out, ids, gw, counts, aux = _forward(moe, w, cfg, d,
                                         token_mask=torch.from_numpy(mask).cuda())
    oi = P.oracle_inputs(inp)
    r = P.oracle_route(w, oi, token_mask=mask)
    ids_h = ids.cpu().numpy()
    assert (ids_h[~mask] == -1).all() and (gw.cpu().numpy()[~mask] == 0).all()
    P.compare_route(w, r, {"expert_ids": ids, "gate_w": gw, "counts": counts, "aux": aux,
                           "mean_prob": moe.moe_route(cfg, d["x"], d["w_router"],
                                                      d.get("logit_bias"), d.get("select_bias"),
                                                      token_mask=torch.from_numpy(mask).cuda())
                           ["mean_prob"]})
    f = P.oracle_forward(w, oi, token_mask=mask)
    err, scale = P.compare_tokens(out, f["out"], P.comparable_tokens(w, r["ids"], ids_h),
                                  w.act_dtype, f"{name} masked forward")
    _say(f"  max|err| {err:.3g} max|ref| {scale:.3g}")


def test_all_tokens_masked(moe):
    w = W.SMALL["deepseek_small"]
    inp = W.make_inputs(w, "cpu", seed=13)
    d = _to_dev(inp)
    cfg = P.config_of(w)
    mask = torch.zeros(w.T, dtype=torch.bool, device="cuda")
    out, ids, gw, counts, aux = _forward(moe, w, cfg, d, token_mask=mask)
    assert (ids == -1).all() and (counts == 0).all() and (aux == 0).all()
    oi = P.oracle_inputs(inp)
    shared = P.oracle.shared_expert(oi["x"], oi)
    P.compare_rows(out, shared, w.act_dtype, "all masked: shared expert only")


LIMIT_CASES = [("mixtral_small", 0.2), ("decode_small", 0.2), ("tiny", 0.1),
               ("deepseek_small", 0.05), ("switch_small", 0.2)]


@pytest.mark.parametrize("name,limit", LIMIT_CASES)
def test_forward_swiglu_limit(moe, name, limit):
    w = W.SMALL[name]
    _say(f"[swiglu_limit] {name} L={limit}")
    inp = W.make_inputs(w, "cpu", seed=14)
    d = _to_dev(inp)
    cfg = P.config_of(w, swiglu_limit=limit)
    out, ids, gw, _, _ = _forward(moe, w, cfg, d)
    oi = P.oracle_inputs(inp)
    f = P.oracle_forward(w, oi, swiglu_limit=limit)
    same = P.comparable_tokens(w, f["route"]["ids"], ids)
    err, scale = P.compare_tokens(out, f["out"], same, w.act_dtype, f"{name} clamped forward")
    plain = P.oracle_forward(w, oi)["out"]
    assert np.abs(plain - f["out"]).max() > 10 * (err + 1e-12), "the clamp changed nothing"
    _say(f"  max|err| {err:.3g} max|ref| {scale:.3g}")


@pytest.mark.parametrize("name", ["deepseek_small", "decode_small"])
def test_forward_shared_expert_gate(moe, name):
    w = W.SMALL[name].with_(H_shared=W.SMALL[name].H_shared or 256)
    _say(f"[shared gate] {name}")
    inp = W.make_inputs(w, "cpu", seed=15)
    gen = torch.Generator().manual_seed(15)
    inp["ws_sgate"] = (torch.randn(w.D, generator=gen) / w.D ** 0.5).to(
        W.torch_dtype(w.act_dtype))
    d = _to_dev(inp)
    cfg = P.config_of(w)
    out, ids, gw, _, _ = _forward(moe, w, cfg, d, shared_expert_gate=d["ws_sgate"])
    oi = P.oracle_inputs(inp)
    f = P.oracle_forward(w, oi)
    err, scale = P.compare_tokens(out, f["out"], P.comparable_tokens(w, f["route"]["ids"], ids),
                                  w.act_dtype, f"{name} gated shared expert")
    _say(f"  max|err| {err:.3g} max|ref| {scale:.3g}")


def test_shared_gate_needs_shared_expert(moe):
    w = W.SMALL["mixtral_small"]
    d = _to_dev(W.make_inputs(w, "cpu", seed=16))
    cfg = P.config_of(w)
    with pytest.raises(moe.MoeError, match="shared_expert_gate"):
        moe.moe_forward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                        shared_expert_gate=torch.zeros(w.D, dtype=torch.bfloat16,
                                                       device="cuda"))


def test_residual_add(moe):
    """out = x + MoE(x) when the residual is x itself, and in place into x."""
    w = W.SMALL["deepseek_small"]
    inp = W.make_inputs(w, "cpu", seed=17)
    d = _to_dev(inp)
    cfg = P.config_of(w)
    out, ids, gw, _, _ = _forward(moe, w, cfg, d, residual=d["x"])
    oi = P.oracle_inputs(inp)
    f = P.oracle_forward(w, oi, residual=oi["x"])
    same = P.comparable_tokens(w, f["route"]["ids"], ids)
    P.compare_tokens(out, f["out"], same, w.act_dtype, "residual forward")
    # combine in place (residual and out the same buffer), on the oracle's routes
    base = P.oracle_forward(w, oi)
    rids = torch.from_numpy(base["route"]["ids"].astype(np.int32)).cuda()
    rgw = torch.from_numpy(base["route"]["weights"].astype(np.float32)).cuda()
    y = torch.zeros(moe.max_rows(cfg), w.D, dtype=torch.bfloat16, device="cuda")
    r = moe.moe_permute(cfg, rids, 0)
    moe.moe_grouped_swiglu(cfg, d["x"], d["w_gate"], d["w_up"], d["w_down"],
                           row_to_assign=r["row_to_assign"], expert_offsets=r["expert_offsets"],
                           gate_w=rgw, y_rows=y)
    sy = moe.moe_grouped_swiglu(cfg, d["x"], d["ws_gate"], d["ws_up"], d["ws_down"])
    acc = d["x"].clone()
    moe.moe_combine(cfg, y, r["assign_to_row"], sy, out=acc, residual=acc)
    P.compare_rows(acc, base["out"] + oi["x"], w.act_dtype, "in-place residual combine")


@pytest.mark.parametrize("E,gamma", [(8, 0.01), (64, 0.125), (256, 1e-3)])
def test_update_bias(moe, E, gamma):
    """One balancer step on the device equals the oracle's (one fp32 rounding
    of bias + gamma * sign), including experts exactly at the mean."""
    w = W.SMALL["deepseek_small"].with_(E=E, n_groups=1, topk_groups=1)
    cfg = P.config_of(w)
    g = np.random.default_rng(E)
    counts = g.integers(0, 50, size=E).astype(np.int32)
    counts[: E // 4] = int(round(counts.mean()))  # some at (or near) the mean
    bias = (g.normal(size=E) * 0.1).astype(np.float32)
    dev_bias = torch.from_numpy(bias).cuda()
    moe.moe_update_bias(cfg, torch.from_numpy(counts).cuda(), gamma, dev_bias)
    torch.cuda.synchronize()
    ref = P.oracle.update_bias(bias.astype(np.float64), counts, np.float32(gamma))
    got = dev_bias.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2.0 ** -23 * np.maximum(np.abs(ref), 1e-30) + 1e-12)
    step = np.sign(counts.sum() - E * counts.astype(np.int64))
    assert (np.sign(got - bias.astype(np.float64)) == step).all()


def _near_rounding_tie(exact, act, rel=1e-12):
    """Elements whose exact value lies within ``rel`` of a rounding tie of the
    activation dtype: there the last fp64 bits of a differently ordered sum
    may pick either neighbour, so both are correct."""
    lo, hi = exact * (1 - rel), exact * (1 + rel)
    if act == "bf16":
        return P.oracle.round_to_bf16(lo) != P.oracle.round_to_bf16(hi)
    return lo.astype(np.float32) != hi.astype(np.float32)


RMS_CASES = [
    # act, T, D, weight, scale of x
    ("bf16", 301, 4096, True, 1.0),
    ("bf16", 67, 64, False, 1e3),
    ("bf16", 5, 7168, True, 1e-3),
    ("f32", 129, 48, True, 1.0),
    ("f32", 33, 4096, False, 10.0),
]


@pytest.mark.parametrize("act,T,D,wt,scale", RMS_CASES)
def test_rmsnorm_correctly_rounded(moe, act, T, D, wt, scale):
    """moe_rmsnorm returns the oracle's float64 RMSNorm rounded once to the
    activation dtype, bit for bit (ties within 1e-12 excepted), also in place;
    a zero row stays zero."""
    _say(f"[rmsnorm] {act} T={T} D={D} weight={wt} scale={scale}")
    dt = W.torch_dtype(act)
    g = torch.Generator().manual_seed(T * D)
    x = (torch.randn(T, D, generator=g) * scale).to(dt)
    x[min(3, T - 1)] = 0
    nw = (torch.rand(D, generator=g) * 1.5 + 0.25) if wt else None
    eps = 1e-6
    cfg = moe.make_config(T, D, 64, 4, 2, act_dtype=act, router_dtype=act, norm_eps=eps)
    xd = x.cuda()
    got = moe.moe_rmsnorm(cfg, xd, None if nw is None else nw.cuda())
    torch.cuda.synchronize()
    x64 = x.to(torch.float64).numpy()
    w64 = None if nw is None else nw.to(torch.float64).numpy()
    eps64 = float(np.float32(eps))
    ref = P.oracle.rms_norm(x64, w64, eps64, act=act)
    near = _near_rounding_tie(P.oracle.rms_norm(x64, w64, eps64, act=None), act)
    g64 = got.cpu().to(torch.float64).numpy()
    bad = (g64 != ref) & ~near
    assert not bad.any(), f"{int(bad.sum())} elements differ, e.g. {np.argwhere(bad)[:3]}"
    _say(f"  {int(near.sum())} elements within 1e-12 of a tie")
    assert (g64[min(3, T - 1)] == 0).all()
    moe.moe_rmsnorm(cfg, xd, None if nw is None else nw.cuda(), out=xd)
    torch.cuda.synchronize()
    assert torch.equal(xd, got), "in-place result differs"


@pytest.mark.parametrize("name", ["mixtral_small", "deepseek_small", "decode_small", "tiny"])
def test_forward_pre_norm(moe, name):
    """out = x + MoE(RMSNorm(x)) in one moe_forward call: routing of the
    normalised rows bit-exact, the output within the layer tolerance."""
    w = W.SMALL[name]
    _say(f"[pre-norm] {name}")
    inp = W.make_inputs(w, "cpu", seed=18)
    d = _to_dev(inp)
    cfg = P.config_of(w)
    cfg.pre_norm, cfg.norm_eps = 1, 1e-5
    nw = torch.rand(w.D, generator=torch.Generator().manual_seed(18)) + 0.5
    out, ids, gw, counts, aux = _forward(moe, w, cfg, d, residual=d["x"], norm_weight=nw.cuda())
    oi = P.oracle_inputs(inp)
    pre = (nw.to(torch.float64).numpy(), float(np.float32(1e-5)), w.act_dtype)
    xn = P.oracle.rms_norm(oi["x"], *pre)
    r = P.oracle_route(w, dict(oi, x=xn))
    xn_dev = moe.moe_rmsnorm(cfg, d["x"], nw.cuda())
    g = moe.moe_route(cfg, xn_dev, d["w_router"], d.get("logit_bias"), d.get("select_bias"))
    torch.cuda.synchronize()
    assert torch.equal(g["expert_ids"], ids) and torch.equal(g["gate_w"], gw)
    nflag, ndiff = P.compare_route(w, r, {"expert_ids": ids, "gate_w": gw, "counts": counts,
                                          "aux": aux, "mean_prob": g["mean_prob"]})
    f = P.oracle_forward(w, oi, residual=oi["x"], pre_norm=pre)
    err, scale = P.compare_tokens(out, f["out"], P.comparable_tokens(w, r["ids"], ids),
                                  w.act_dtype, f"{name} pre-norm forward")
    _say(f"  near ties {nflag} (differing {ndiff}); max|err| {err:.3g} max|ref| {scale:.3g}")


def test_norm_weight_needs_pre_norm(moe):
    w = W.SMALL["mixtral_small"]
    d = _to_dev(W.make_inputs(w, "cpu", seed=19))
    cfg = P.config_of(w)
    with pytest.raises(moe.MoeError, match="pre_norm"):
        moe.moe_forward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                        norm_weight=torch.ones(w.D, device="cuda"))
