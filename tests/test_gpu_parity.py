"""GPU parity: every entry point of the C ABI against the CPU oracle.

Stage-wise (each stage fed identical inputs) and end to end, on reduced
workloads whose every output element the oracle computes, on edge cases, and
on the full-size workloads in the launch configuration the benchmark times
(sampled rows there).  Integer results are compared bit for bit; routing
excludes only tokens the oracle flags as near ties (score gap < 1e-5), and the
downstream stages are then fed the device's own routing, so nothing else is
excluded."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
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


def _route(moe, w, cfg, d):
    return moe.moe_route(cfg, d["x"], d["w_router"], d.get("logit_bias"), d.get("select_bias"))


def _cap_int(w):
    c = oracle.capacity(w.capacity_factor, w.T, w.top_k, w.E)
    return 0 if c is None else c


def _check_permute(moe, w, cfg, ids, cap):
    """The device permutation of the routes ``ids`` (the oracle's, or a
    test's own) against the oracle's, bit for bit."""
    ids = np.asarray(ids).astype(np.int64)
    keep = oracle.first_within_capacity(ids, w.E, cap if cap > 0 else None)
    off, r2a, a2r = oracle.permutation(ids, keep, w.E)
    g = moe.moe_permute(cfg, torch.from_numpy(ids.astype(np.int32)).cuda(), cap)
    n = int(g["n_kept"].item())
    assert n == int(keep.sum())
    assert (g["expert_offsets"].cpu().numpy() == off).all()
    assert (g["row_to_assign"][:n].cpu().numpy() == r2a).all()
    assert (g["assign_to_row"].cpu().numpy() == a2r).all()
    return g, keep


def _reference_rows(w, oi, ids, gw, keep, r2a, rows=None):
    """Weighted expert rows in expert-major order: gw[t,s] * FFN_e(x_t)."""
    k = w.top_k
    r2a = np.asarray(r2a)
    if rows is not None:
        r2a = r2a[rows]
    toks = np.unique(r2a // k)
    Y = oracle.expert_outputs(oi["x"], ids, gw, keep, oi["w_gate"], oi["w_up"], oi["w_down"],
                              tokens=toks)
    pos = {t: i for i, t in enumerate(toks)}
    return np.stack([Y[pos[a // k], a % k] for a in r2a]) if r2a.size else np.zeros((0, w.D))


# --------------------------------------------------------- reduced sizes ---

SMALL = sorted(W.SMALL)


@pytest.mark.parametrize("name", SMALL)
def test_route_small(moe, name):
    w = W.SMALL[name]
    _say(f"[route] {name} T={w.T} E={w.E} k={w.top_k}")
    inp = W.make_inputs(w, "cpu", seed=0)
    cfg = P.config_of(w)
    g = _route(moe, w, cfg, _to_dev(inp))
    torch.cuda.synchronize()
    r = P.oracle_route(w, P.oracle_inputs(inp))
    nflag, ndiff = P.compare_route(w, r, g)
    _say(f"  near ties flagged {nflag}, differing {ndiff}")


# Group-limit shapes: group sizes 2..32 (segmented in-wave reduction), 64 and
# 12 (the general path), both group rules, and softmax as well as sigmoid.
# With softmax the top-2 group sum is over probabilities, which the sum of
# two logits does not order alike once the logits spread out (x_std 4 and no
# selection bias: the last two cases, one per group path).
GROUP_CASES = [
    # E, n_groups, topk_groups, k, rule, score, x_std, selection-bias sigma
    (64, 32, 8, 6, "top2sum", "sigmoid", 1.0, 0.01),
    (64, 16, 4, 8, "top2sum", "sigmoid", 1.0, 0.01),
    (128, 8, 3, 8, "top2sum", "softmax", 1.0, 0.01),
    (256, 8, 4, 8, "max", "sigmoid", 1.0, 0.01),
    (256, 4, 2, 8, "top2sum", "sigmoid", 1.0, 0.01),
    (48, 4, 2, 6, "top2sum", "sigmoid", 1.0, 0.01),
    (96, 3, 1, 4, "max", "softmax", 1.0, 0.01),
    (64, 8, 5, 8, "top2sum", "softmax", 4.0, 0.0),
    (96, 8, 3, 6, "top2sum", "softmax", 4.0, 0.0),
]


@pytest.mark.parametrize("E,ng,tg,k,rule,score,x_std,sel", GROUP_CASES)
def test_route_group_limits(moe, E, ng, tg, k, rule, score, x_std, sel):
    w = W.SMALL["deepseek_small"].with_(
        seq=173, E=E, top_k=k, n_groups=ng, topk_groups=tg, group_rule=rule, score=score,
        route_scale=2.5 if score == "sigmoid" else 1.0, H_shared=0, x_std=x_std,
        select_bias_sigma=sel)
    _say(f"[route-groups] E={E} groups={ng} keep={tg} k={k} {rule} {score}")
    inp = W.make_inputs(w, "cpu", seed=3)
    cfg = P.config_of(w)
    g = _route(moe, w, cfg, _to_dev(inp))
    torch.cuda.synchronize()
    r = P.oracle_route(w, P.oracle_inputs(inp))
    nflag, ndiff = P.compare_route(w, r, g)
    _say(f"  near ties flagged {nflag}, differing {ndiff}")


# Shapes that take the LDS-tiled router GEMM (bf16, E >= 128, T >= 1024):
# ragged token and expert tiles, E below and at one 256-wide tile.
TILED_ROUTER_CASES = [(1100, 160, 6, "softmax"), (2048, 256, 8, "sigmoid"), (1031, 128, 4, "softmax")]


@pytest.mark.parametrize("T,E,k,score", TILED_ROUTER_CASES)
def test_route_tiled_router_gemm(moe, T, E, k, score):
    w = W.SMALL["decode_small"].with_(batch=1, seq=T, D=768, E=E, top_k=k, score=score,
                                      H=128, route_scale=2.5 if score == "sigmoid" else 1.0)
    _say(f"[route-tiled] T={T} E={E} k={k} {score}")
    inp = W.make_inputs(w, "cpu", seed=5)
    cfg = P.config_of(w)
    g = _route(moe, w, cfg, _to_dev(inp))
    torch.cuda.synchronize()
    r = P.oracle_route(w, P.oracle_inputs(inp))
    nflag, ndiff = P.compare_route(w, r, g)
    _say(f"  near ties flagged {nflag}, differing {ndiff}")


@pytest.mark.parametrize("name", SMALL)
def test_route_deterministic(moe, name):
    w = W.SMALL[name]
    d = _to_dev(W.make_inputs(w, "cpu", seed=1))
    cfg = P.config_of(w)
    a, b = _route(moe, w, cfg, d), _route(moe, w, cfg, d)
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("name", SMALL)
def test_capacity_matches_oracle(moe, name):
    w = W.SMALL[name].with_(capacity_factor=W.SMALL[name].capacity_factor or 1.25)
    cfg = P.config_of(w)
    assert moe.capacity(cfg) == oracle.capacity(w.capacity_factor, w.T, w.top_k, w.E)


@pytest.mark.parametrize("name", SMALL)
def test_permute_small(moe, name):
    w = W.SMALL[name]
    _say(f"[permute] {name}")
    cfg = P.config_of(w)
    r = P.oracle_route(w, P.oracle_inputs(W.make_inputs(w, "cpu", seed=0)))
    _check_permute(moe, w, cfg, r["ids"], _cap_int(w))
    # also with a tight capacity, so that drops happen on every workload
    tight = max(1, (w.T * w.top_k) // (4 * w.E))
    _check_permute(moe, w, cfg, r["ids"], tight)


# Shapes past the one-workgroup permutation (more than 4096 assignments):
# the per-expert scans and the per-tile scatter, with one to 256 experts, E
# not a power of two, k up to 8, and capacity limits; the last two keep
# 8-token routing tiles (T <= 1024) and leave the scatter's last block with
# a single tile.
LARGE_PERMUTE_CASES = [
    # T, E, k, capacity (0: dropless)
    (3001, 8, 3, 0), (8192, 64, 1, 160), (4100, 5, 2, 0), (2048, 256, 8, 0),
    (5000, 3, 3, 2000), (1500, 130, 4, 10), (16384, 1, 1, 0), (3000, 2, 2, 0),
    (1000, 256, 8, 0), (777, 97, 6, 20),
]


@pytest.mark.parametrize("T,E,k,cap", LARGE_PERMUTE_CASES)
def test_permute_large_shapes(moe, T, E, k, cap):
    w = W.Workload("perm_large", 1, T, D=64, H=64, E=E, top_k=k)
    _say(f"[permute-large] T={T} E={E} k={k} cap={cap}")
    cfg = P.config_of(w)
    rng = np.random.default_rng(T * 131 + E)
    # skewed, distinct experts per token (as a top-k gives)
    pref = rng.permutation(E)
    ids = np.stack([pref[np.sort(rng.choice(E, size=k, replace=False,
                                            p=np.linspace(2.0, 1.0, E) / np.linspace(2.0, 1.0, E).sum()))]
                    for _ in range(T)])
    _check_permute(moe, w, cfg, ids, cap)


@pytest.mark.parametrize("name", SMALL)
def test_grouped_swiglu_small(moe, name):
    w = W.SMALL[name]
    _say(f"[grouped_swiglu] {name}")
    inp = W.make_inputs(w, "cpu", seed=0)
    d = _to_dev(inp)
    cfg = P.config_of(w)
    oi = P.oracle_inputs(inp)
    r = P.oracle_route(w, oi)  # the oracle's routes and weights go in
    perm, keep = _check_permute(moe, w, cfg, r["ids"], _cap_int(w))
    n = int(perm["n_kept"].item())
    y = moe.moe_grouped_swiglu(cfg, d["x"], d["w_gate"], d["w_up"], d["w_down"],
                               row_to_assign=perm["row_to_assign"],
                               expert_offsets=perm["expert_offsets"],
                               max_rows_bound=moe.max_rows(cfg),
                               gate_w=torch.from_numpy(r["weights"].astype(np.float32)).cuda())
    torch.cuda.synchronize()
    ref = _reference_rows(w, oi, r["ids"], r["weights"], keep,
                          perm["row_to_assign"][:n].cpu().numpy())
    P.compare_rows(y[:n], ref, w.act_dtype, f"{name} expert rows")


def test_shared_expert_identity_rows(moe):
    w = W.SMALL["deepseek_small"]
    inp = W.make_inputs(w, "cpu", seed=0)
    d = _to_dev(inp)
    cfg = P.config_of(w)
    y = moe.moe_grouped_swiglu(cfg, d["x"], d["ws_gate"], d["ws_up"], d["ws_down"])
    oi = P.oracle_inputs(inp)
    ref = oracle.swiglu_ffn(oi["x"], oi["ws_gate"], oi["ws_up"], oi["ws_down"])
    P.compare_rows(y, ref, w.act_dtype, "shared expert")


@pytest.mark.parametrize("name", SMALL)
def test_combine_small(moe, name):
    w = W.SMALL[name]
    inp = W.make_inputs(w, "cpu", seed=0)
    d = _to_dev(inp)
    cfg = P.config_of(w)
    r = P.oracle_route(w, P.oracle_inputs(inp))
    perm, keep = _check_permute(moe, w, cfg, r["ids"], _cap_int(w))
    n = int(perm["n_kept"].item())
    dt = W.torch_dtype(w.act_dtype)
    gen = torch.Generator().manual_seed(5)
    rows = torch.randn(max(n, 1), w.D, generator=gen).to(dt)
    shared = torch.randn(w.T, w.D, generator=gen).to(dt) if w.H_shared else None
    out = moe.moe_combine(cfg, rows.cuda(), perm["assign_to_row"],
                          None if shared is None else shared.cuda())
    a2r = perm["assign_to_row"].cpu().numpy().reshape(w.T, w.top_k)
    R = rows.to(torch.float64).numpy()
    Y = np.zeros((w.T, w.top_k, w.D))
    for s in range(w.top_k):
        m = a2r[:, s] >= 0
        Y[m, s] = R[a2r[m, s]]
    ref = oracle.combine(Y, None if shared is None else shared.to(torch.float64).numpy())
    got = out.cpu().to(torch.float64).numpy()
    # one rounding of an exactly representable fp32 sum of at most k+1 terms
    rel = 2.0 ** -8 if w.act_dtype == "bf16" else 2.0 ** -22
    assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 1e-30)


@pytest.mark.parametrize("shared,residual", [(False, False), (True, True)])
def test_combine_wide(moe, shared, residual):
    """The combine at a batch of 256K row chunks, where each thread sums four
    chunks of its token (capacity drops, a shared row and the residual)."""
    w = W.Workload("combine_wide", 1, 2048, D=1024, H=64, E=8, top_k=3)
    _say(f"[combine-wide] shared={shared} residual={residual}")
    cfg = P.config_of(w)
    rng = np.random.default_rng(17)
    ids = np.stack([rng.choice(w.E, size=w.top_k, replace=False) for _ in range(w.T)])
    perm, keep = _check_permute(moe, w, cfg, ids, 600)
    n = int(perm["n_kept"].item())
    gen = torch.Generator().manual_seed(9)
    rows = torch.randn(max(n, 1), w.D, generator=gen).to(torch.bfloat16)
    sh = torch.randn(w.T, w.D, generator=gen).to(torch.bfloat16) if shared else None
    res = torch.randn(w.T, w.D, generator=gen).to(torch.bfloat16) if residual else None
    out = moe.moe_combine(cfg, rows.cuda(), perm["assign_to_row"],
                          None if sh is None else sh.cuda(),
                          residual=None if res is None else res.cuda())
    a2r = perm["assign_to_row"].cpu().numpy().reshape(w.T, w.top_k)
    R = rows.to(torch.float64).numpy()
    Y = np.zeros((w.T, w.top_k, w.D))
    for s_ in range(w.top_k):
        m = a2r[:, s_] >= 0
        Y[m, s_] = R[a2r[m, s_]]
    ref = oracle.combine(Y, None if sh is None else sh.to(torch.float64).numpy(),
                         residual=None if res is None else res.to(torch.float64).numpy())
    got = out.cpu().to(torch.float64).numpy()
    # fp32 sum of at most k+2 terms (error at most (k+1) 2^-24 of the sum of
    # their magnitudes), then one rounding to bf16 (2^-9 of the value)
    mag = np.abs(Y).sum(1)
    mag += 0.0 if sh is None else np.abs(sh.to(torch.float64).numpy())
    mag += 0.0 if res is None else np.abs(res.to(torch.float64).numpy())
    fp32_err = (w.top_k + 1) * 2.0 ** -24 * mag
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * (np.abs(ref) + fp32_err) + fp32_err)


@pytest.mark.parametrize("name", SMALL)
def test_forward_small(moe, name):
    w = W.SMALL[name]
    _say(f"[forward] {name}")
    inp = W.make_inputs(w, "cpu", seed=0)
    d = _to_dev(inp)
    cfg = P.config_of(w)
    ids = torch.empty(w.T, w.top_k, dtype=torch.int32, device="cuda")
    gw = torch.empty(w.T, w.top_k, dtype=torch.float32, device="cuda")
    out = moe.moe_forward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                          logit_bias=d.get("logit_bias"), select_bias=d.get("select_bias"),
                          ws_gate=d.get("ws_gate"), ws_up=d.get("ws_up"),
                          ws_down=d.get("ws_down"), expert_ids=ids, gate_w=gw)
    torch.cuda.synchronize()
    g = _route(moe, w, cfg, d)
    assert torch.equal(g["expert_ids"], ids) and torch.equal(g["gate_w"], gw)
    oi = P.oracle_inputs(inp)
    r = P.oracle_route(w, oi)
    P.compare_route(w, r, g)
    f = P.oracle_forward(w, oi)
    err, scale = P.compare_tokens(out, f["out"], P.comparable_tokens(w, r["ids"], ids),
                                  w.act_dtype, f"{name} forward")
    _say(f"  max|err| {err:.3g} max|ref| {scale:.3g}")


@pytest.mark.parametrize("name", SMALL)
def test_forward_deterministic(moe, name):
    w = W.SMALL[name]
    d = _to_dev(W.make_inputs(w, "cpu", seed=2))
    cfg = P.config_of(w)
    args = (cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"])
    kw = dict(logit_bias=d.get("logit_bias"), select_bias=d.get("select_bias"),
              ws_gate=d.get("ws_gate"), ws_up=d.get("ws_up"), ws_down=d.get("ws_down"))
    assert torch.equal(moe.moe_forward(*args, **kw), moe.moe_forward(*args, **kw))


# ------------------------------------------------------------ edge cases ---

def _fwd(moe, w, inp):
    d = _to_dev(inp)
    cfg = P.config_of(w)
    ids = torch.empty(w.T, w.top_k, dtype=torch.int32, device="cuda")
    gw = torch.empty(w.T, w.top_k, dtype=torch.float32, device="cuda")
    out = moe.moe_forward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                          logit_bias=d.get("logit_bias"), select_bias=d.get("select_bias"),
                          ws_gate=d.get("ws_gate"), ws_up=d.get("ws_up"),
                          ws_down=d.get("ws_down"), expert_ids=ids, gate_w=gw)
    torch.cuda.synchronize()
    return out, ids, gw


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token(moe, dtype):
    w = W.Workload("one", 1, 1, D=128, H=64, E=8, top_k=3, act_dtype=dtype, router_dtype=dtype)
    inp = W.make_inputs(w, "cpu", seed=3)
    out, ids, gw = _fwd(moe, w, inp)
    oi = P.oracle_inputs(inp)
    f = P.oracle_forward(w, oi)
    P.compare_tokens(out, f["out"], P.comparable_tokens(w, f["route"]["ids"], ids, 1.0), dtype,
                     "single token")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_router_picks_first_k(moe, dtype):
    w = W.Workload("zero", 1, 70, D=64, H=64, E=8, top_k=3, act_dtype=dtype, router_dtype=dtype)
    inp = W.make_inputs(w, "cpu", seed=4)
    inp["w_router"].zero_()
    out, ids, gw = _fwd(moe, w, inp)
    assert (ids.cpu() == torch.arange(3, dtype=torch.int32)).all()
    assert torch.allclose(gw.cpu(), torch.full_like(gw.cpu(), 1.0 / 3), atol=1e-7)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_limit_topk_equals_E(moe, dtype):
    w = W.Workload("dense", 1, 45, D=64, H=128, E=4, top_k=4, act_dtype=dtype,
                   router_dtype=dtype, w_std=0.1)
    inp = W.make_inputs(w, "cpu", seed=5)
    inp["w_router"].zero_()
    out, ids, gw = _fwd(moe, w, inp)
    oi = P.oracle_inputs(inp)
    mean = sum(oracle.swiglu_ffn(oi["x"], oi["w_gate"][e], oi["w_up"][e], oi["w_down"][e])
               for e in range(4)) / 4.0
    P.compare_rows(out, mean, dtype, "top_k = E with a zero router")


def test_identical_experts_are_dense(moe):
    w = W.Workload("same", 2, 77, D=128, H=192, E=6, top_k=2, w_std=0.05)
    inp = W.make_inputs(w, "cpu", seed=6)
    for key in ("w_gate", "w_up", "w_down"):
        inp[key][:] = inp[key][:1].clone()
    out, _, _ = _fwd(moe, w, inp)
    oi = P.oracle_inputs(inp)
    dense = oracle.swiglu_ffn(oi["x"], oi["w_gate"][0], oi["w_up"][0], oi["w_down"][0])
    P.compare_rows(out, dense, "bf16", "identical experts")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forced_routes_with_empty_experts(moe, dtype):
    """Forced IDs that leave most experts empty, through permute, grouped
    SwiGLU and combine."""
    w = W.Workload("forced", 1, 50, D=64, H=64, E=7, top_k=2, act_dtype=dtype,
                   router_dtype=dtype, w_std=0.1)
    inp = W.make_inputs(w, "cpu", seed=7)
    d = _to_dev(inp)
    cfg = P.config_of(w)
    ids = torch.tensor([[4, 1]] * 30 + [[1, 4]] * 20, dtype=torch.int32)
    gw = torch.tensor([[0.75, 0.25]] * 50, dtype=torch.float32)
    perm, keep = _check_permute(moe, w, cfg, ids.numpy(), 0)
    assert perm["expert_offsets"].cpu().tolist() == [0, 0, 50, 50, 50, 100, 100, 100]
    y = moe.moe_grouped_swiglu(cfg, d["x"], d["w_gate"], d["w_up"], d["w_down"],
                               row_to_assign=perm["row_to_assign"],
                               expert_offsets=perm["expert_offsets"], gate_w=gw.cuda())
    out = moe.moe_combine(cfg, y, perm["assign_to_row"])
    oi = P.oracle_inputs(inp)
    ref = oracle.brute_force_forward(oi, ids.numpy(), gw.numpy().astype(np.float64))
    P.compare_rows(out, ref, dtype, "forced routes")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_capacity_drops_everything_but_one(moe, dtype):
    """Capacity 1: each expert keeps only its first assignment; tokens with
    every slot dropped get exactly zero."""
    w = W.Workload("cap1", 1, 90, D=64, H=64, E=4, top_k=1, act_dtype=dtype,
                   router_dtype=dtype, renormalize=False, capacity_factor=0.01)
    inp = W.make_inputs(w, "cpu", seed=8)
    out, ids, gw = _fwd(moe, w, inp)
    oi = P.oracle_inputs(inp)
    f = P.oracle_forward(w, oi)
    assert f["capacity"] == 1 and f["n_kept"] <= 4
    same = P.comparable_tokens(w, f["route"]["ids"], ids)
    P.compare_tokens(out, f["out"], same, dtype, "capacity 1")
    dropped = ~f["keep"][:, 0] & same
    assert (out.cpu()[torch.from_numpy(dropped)] == 0).all()


@pytest.mark.parametrize("T,E,k", [(2000, 4, 2), (1111, 2, 1), (3001, 8, 3)])
def test_large_tile_path(moe, T, E, k):
    """Enough rows per expert for the 256-row direct-to-LDS kernels, with
    ragged last tiles: every output row against the oracle."""
    w = W.Workload("large_tiles", 1, T, D=512, H=384, E=E, top_k=k, w_std=0.05)
    _say(f"[large tiles] T={T} E={E} k={k}")
    inp = W.make_inputs(w, "cpu", seed=9)
    out, ids, gw = _fwd(moe, w, inp)
    oi = P.oracle_inputs(inp)
    f = P.oracle_forward(w, oi)
    err, scale = P.compare_tokens(out, f["out"], P.comparable_tokens(w, f["route"]["ids"], ids),
                                  "bf16", "large-tile forward")
    _say(f"  max|err| {err:.3g} max|ref| {scale:.3g}")


# x of exactly 2^31 bytes: past the 32-bit buffer offsets of the
# direct-to-LDS kernels, so the grouped GEMMs take the register-staged path.
BEYOND_2GB = W.Workload("beyond_2gb", 1, 262144, D=4096, H=64, E=8, top_k=2)


def test_forward_beyond_32bit_offsets(moe):
    """A layer whose input passes 2 GB: routing of every token bit-exact and
    sampled outputs against the oracle on its own routes."""
    w = BEYOND_2GB
    _say(f"[beyond 2 GB] T={w.T} D={w.D}: drawing inputs")
    inp = W.make_inputs(w, "cuda", seed=21)
    assert inp["x"].numel() * 2 >= 1 << 31
    out, ids, gw = _fwd(moe, w, inp)
    _say("[beyond 2 GB] oracle routing")
    oi = P.oracle_inputs(inp)
    r = P.oracle_route(w, oi)
    P.compare_route(w, r, dict(_route(moe, w, P.config_of(w), inp), expert_ids=ids, gate_w=gw))
    toks = _sample_tokens(w.T, 24, seed=22)
    f = P.oracle_forward(w, oi, tokens=toks)
    same = P.comparable_tokens(w, r["ids"], ids)[toks]
    err, scale = P.compare_tokens(out[torch.from_numpy(toks).cuda()], f["out"], same, "bf16",
                                  "beyond 2 GB sampled outputs")
    _say(f"  max|err| {err:.3g} max|ref| {scale:.3g}")


def test_errors_are_reported(moe):
    w = W.SMALL["mixtral_small"]
    d = _to_dev(W.make_inputs(w, "cpu", seed=0))
    cfg = P.config_of(w)
    small_ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError, match="WORKSPACE"):
        moe.moe_forward(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"],
                        workspace=small_ws)
    bad = moe.make_config(w.T, w.D, w.H, w.E, w.E + 1)
    with pytest.raises(moe.MoeError, match="INVALID_ARG"):
        moe.moe_route(bad, d["x"], d["w_router"])


# ------------------------------------------------------------- full size ---

FULL = ["tiny_dropless_fp32", "switch_top1_capacity", "mixtral_8x_top2",
        "deepseek_v3_256x_top8_grouped", "decode_128x_top8"]


def _sample_tokens(T, n, seed):
    r = np.random.default_rng(seed)
    pick = set(r.choice(T, size=min(n, T), replace=False).tolist())
    pick.update({0, T - 1})
    return np.array(sorted(pick))


@pytest.mark.parametrize("name", FULL)
def test_full_size_forward(moe, name):
    """Full-size workload exactly as the benchmark draws and launches it:
    routing on every token, permutation bit-exact, outputs on sampled tokens
    (with a capacity limit: on every token that keeps a slot)."""
    w = W.WORKLOADS[name]
    _say(f"[full] {name}: drawing inputs")
    dev = "cpu" if w.act_dtype == "f32" else "cuda"
    inp = {k: v.to("cuda") for k, v in W.make_inputs(w, dev, seed=0).items()}
    cfg = P.config_of(w)
    ids = torch.empty(w.T, w.top_k, dtype=torch.int32, device="cuda")
    gw = torch.empty(w.T, w.top_k, dtype=torch.float32, device="cuda")
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    aux = torch.empty(2, dtype=torch.float32, device="cuda")
    _say(f"[full] {name}: forward")
    out = moe.moe_forward(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                          inp["w_down"], logit_bias=inp.get("logit_bias"),
                          select_bias=inp.get("select_bias"), ws_gate=inp.get("ws_gate"),
                          ws_up=inp.get("ws_up"), ws_down=inp.get("ws_down"), expert_ids=ids,
                          gate_w=gw, counts=counts, aux=aux)
    torch.cuda.synchronize()
    _say(f"[full] {name}: oracle routing")
    oi = P.oracle_inputs(inp)
    r = P.oracle_route(w, oi)
    g = {"expert_ids": ids, "gate_w": gw, "counts": counts, "aux": aux,
         "mean_prob": _route(moe, w, cfg, inp)["mean_prob"]}
    nflag, ndiff = P.compare_route(w, r, g)
    _say(f"  near ties flagged {nflag}, differing {ndiff}")
    _check_permute(moe, w, cfg, r["ids"], _cap_int(w))
    # Sampled tokens; the Mixtral-shaped layer (8 experts, each upcast once)
    # takes 256 of them.
    nsample = 256 if w.E <= 8 else 24
    toks = _sample_tokens(w.T, nsample if w.T > 1024 else w.T, seed=11)
    if w.capacity_factor is not None:
        # Every token that keeps a slot (the capacity-limited layer keeps few
        # rows, so each of them is compared), and 64 dropped ones.
        keep = oracle.first_within_capacity(r["ids"], w.E,
                                            oracle.capacity(w.capacity_factor, w.T, w.top_k, w.E))
        toks = np.unique(np.concatenate([toks, np.nonzero(keep.any(1))[0],
                                         np.nonzero(~keep.any(1))[0][:64]]))
    _say(f"[full] {name}: oracle outputs on {toks.size} tokens")
    f = P.oracle_forward(w, oi, tokens=toks)
    same = P.comparable_tokens(w, r["ids"], ids)[toks]
    err, scale = P.compare_tokens(out[torch.from_numpy(toks).cuda()], f["out"], same,
                                  w.act_dtype, f"{name} sampled outputs")
    _say(f"  max|err| {err:.3g} max|ref| {scale:.3g}")


@pytest.mark.parametrize("name,n_pick", [("deepseek_v3_256x_top8_grouped", 16),
                                         ("mixtral_8x_top2", 8)])
def test_full_size_expert_rows(moe, name, n_pick):
    """Every row of whole experts of the full-size grouped SwiGLU stage (all
    their row tiles, partial ones and split-K tail pieces included), on the
    oracle's routes, weights and permutation: every expert of the
    Mixtral-shaped layer (the whole stage), and 16 of the DeepSeek-shaped
    layer's, from the fewest rows to the most."""
    w = W.WORKLOADS[name]
    _say(f"[full-rows] {name}: drawing inputs")
    inp = {k: v.to("cuda") for k, v in W.make_inputs(w, "cuda", seed=0).items()}
    cfg = P.config_of(w)
    oi = P.oracle_inputs(inp)
    r = P.oracle_route(w, oi)
    cap = _cap_int(w)
    keep = oracle.first_within_capacity(r["ids"], w.E, cap if cap > 0 else None)
    off, r2a, _ = oracle.permutation(r["ids"], keep, w.E)
    ids = torch.from_numpy(r["ids"].astype(np.int32)).cuda()
    gw = torch.from_numpy(r["weights"].astype(np.float32)).cuda()
    perm = moe.moe_permute(cfg, ids, cap)
    assert np.array_equal(perm["expert_offsets"].cpu().numpy(), off)
    rows = moe.max_rows(cfg)
    y = torch.empty(max(rows, 1), w.D, dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_swiglu(cfg, inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"],
                           row_to_assign=perm["row_to_assign"],
                           expert_offsets=perm["expert_offsets"], max_rows_bound=rows,
                           gate_w=gw, y_rows=y)
    torch.cuda.synchronize()
    n = np.diff(off)
    with_rows = np.nonzero(n)[0]
    by_size = with_rows[np.argsort(n[with_rows], kind="stable")]
    picks = sorted(set(int(by_size[j]) for j in
                       np.linspace(0, by_size.size - 1, n_pick).round().astype(int)))
    for e in picks:
        a = np.asarray(r2a[off[e]:off[e + 1]])
        t, s = a // w.top_k, a % w.top_k
        ref = r["weights"][t, s][:, None] * oracle.swiglu_ffn(
            oi["x"][t], oi["w_gate"][e], oi["w_up"][e], oi["w_down"][e])
        err, scale = P.compare_rows(y[off[e]:off[e + 1]], ref, w.act_dtype,
                                    f"{name} expert {e} ({a.size} rows)")
        _say(f"  expert {e}: {a.size} rows, max|err| {err:.3g} max|ref| {scale:.3g}")
