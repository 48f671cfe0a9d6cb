"""Pins for the CPU oracle: facts fixed by the pages or by mathematics.

Each ``pin_*`` function takes the oracle module ``o`` and raises
AssertionError when ``o`` disagrees with a value the pages print, a closed
form, an identity, a special case or a brute-force loop.  The same functions
run against the real oracle (``test_oracle_pins.py``) and against copies of it
with a planted mistake (``test_oracle_mutants.py``), which must each fail at
least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sig(v):
    return 1.0 / (1.0 + math.exp(-v))


def _rng(seed):
    return np.random.default_rng(seed)


def _tiny_inputs(seed, T=9, D=6, H=5, E=4, shared=False, std=0.5):
    r = _rng(seed)
    inp = {
        "x": r.normal(size=(T, D)),
        "w_router": r.normal(size=(E, D)) * std,
        "w_gate": r.normal(size=(E, H, D)) * std,
        "w_up": r.normal(size=(E, H, D)) * std,
        "w_down": r.normal(size=(E, D, H)) * std,
    }
    if shared:
        inp["ws_gate"] = r.normal(size=(H + 1, D)) * std
        inp["ws_up"] = r.normal(size=(H + 1, D)) * std
        inp["ws_down"] = r.normal(size=(D, H + 1)) * std
    return inp


def _route_logits(o, logits, k, **kw):
    """Route tokens whose logits are given directly (x = h, W_r = I)."""
    h = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    return o.route(h, np.eye(h.shape[1]), k, **kw)


# ------------------------------------------------------------- routing -----

def pin_worked_example_ids(o):
    """Both conventions pick experts [5, 0] for the printed 8-expert logits."""
    g = _golden("worked_routing_example.json")
    for renorm in (True, False):
        r = _route_logits(o, g["logits"], g["k"], renormalize=renorm)
        assert r["ids"][0].tolist() == g["expected_ids"], r["ids"]


def pin_worked_example_renorm_closed_form(o):
    """Renormalised weights are exp(3)/(exp(3)+exp(2)) = sigmoid(1) and sigmoid(-1)."""
    g = _golden("worked_routing_example.json")
    r = _route_logits(o, g["logits"], g["k"], renormalize=True)
    assert np.allclose(r["weights"][0], [_sig(1.0), _sig(-1.0)], rtol=0, atol=1e-15)


def pin_worked_example_switch_ratio(o):
    """Without renormalisation the two kept probabilities keep the ratio
    exp(h5 - h0) = e, and all E probabilities add to 1."""
    g = _golden("worked_routing_example.json")
    r = _route_logits(o, g["logits"], g["k"], renormalize=False)
    w = r["weights"][0]
    assert abs(w[0] / w[1] - math.e) < 1e-13
    assert w.sum() < 1.0
    rall = _route_logits(o, g["logits"], 8, renormalize=False)
    assert abs(rall["weights"][0].sum() - 1.0) < 1e-15


def pin_renorm_is_topk_then_softmax(o):
    """Softmax-then-top-k with renormalisation equals top-k-then-softmax over the
    k selected logits (the book's Mixtral-style route) for any logits."""
    h = _rng(1).normal(size=(40, 12)) * 2.0
    k = 3
    r = _route_logits(o, h, k, renormalize=True)
    top = np.sort(h, axis=1)[:, ::-1][:, :k]
    alt = np.exp(top - top[:, :1])
    alt = alt / alt.sum(axis=1, keepdims=True)
    assert np.allclose(r["weights"], alt, rtol=0, atol=1e-14)
    assert (np.take_along_axis(h, r["ids"], 1) == top).all()


def pin_zero_router_picks_first_k(o):
    """A zero router gives equal scores, so top-k picks experts 0..k-1 with
    equal weights (book, 'Sparse upcycling')."""
    inp = _tiny_inputs(2, E=6)
    for k in (1, 2, 4):
        r = o.route(inp["x"], np.zeros((6, inp["x"].shape[1])), k)
        assert (r["ids"] == np.arange(k)[None, :]).all()
        assert np.allclose(r["weights"], 1.0 / k, rtol=0, atol=1e-15)
        assert r["near_tie"].all()


def pin_weight_sums(o):
    """Renormalised weights sum to 1 (lab smoke test); with route_scale they sum
    to route_scale; the un-renormalised top-1 weight lies in (1/E, 1]."""
    inp = _tiny_inputs(3, T=30, E=8)
    r = o.route(inp["x"], inp["w_router"], 3)
    assert np.allclose(r["weights"].sum(1), 1.0, rtol=0, atol=1e-14)
    r = o.route(inp["x"], inp["w_router"], 3, score="sigmoid", route_scale=2.5)
    assert np.allclose(r["weights"].sum(1), 2.5, rtol=0, atol=1e-13)
    r = o.route(inp["x"], inp["w_router"], 1, renormalize=False)
    assert ((r["weights"] > 1.0 / 8) & (r["weights"] <= 1.0)).all()


def pin_slots_descending(o):
    """Slot j holds the j-th largest selection score."""
    inp = _tiny_inputs(4, T=25, E=10)
    for score in ("softmax", "sigmoid"):
        r = o.route(inp["x"], inp["w_router"], 4, score=score)
        v = np.take_along_axis(r["scores"], r["ids"], 1)
        assert (np.diff(v, axis=1) <= 0).all()
        rest = r["scores"].copy()
        np.put_along_axis(rest, r["ids"], -np.inf, 1)
        assert (v[:, -1] >= rest.max(1)).all()


def pin_sigmoid_closed_form(o):
    """Sigmoid weights with renormalisation for a token with logits 0 and ln 3:
    scores 1/2 and 3/4, weights 2.5*(2/5) and 2.5*(3/5)."""
    h = np.array([[0.0, math.log(3.0), -5.0, -6.0]])
    r = _route_logits(o, h, 2, score="sigmoid", route_scale=2.5)
    assert r["ids"][0].tolist() == [1, 0]
    assert np.allclose(r["weights"][0], [1.5, 1.0], rtol=0, atol=1e-14)


def pin_selection_only_bias(o):
    """A selection bias changes which experts win but the weights still come
    from the unbiased scores (book exercise 6; DeepSeek-V3 paragraph)."""
    inp = _tiny_inputs(5, T=20, E=8)
    x, w = inp["x"], inp["w_router"]
    r0 = o.route(x, w, 2, score="sigmoid")
    rz = o.route(x, w, 2, score="sigmoid", select_bias=np.zeros(8))
    assert (r0["ids"] == rz["ids"]).all() and np.allclose(r0["weights"], rz["weights"])
    b = np.zeros(8)
    b[6] = 10.0
    rb = o.route(x, w, 2, score="sigmoid", select_bias=b)
    assert (rb["ids"][:, 0] == 6).all()
    s = 1.0 / (1.0 + np.exp(-(x @ w.T)))
    chosen = np.take_along_axis(s, rb["ids"], 1)
    assert np.allclose(rb["weights"], chosen / chosen.sum(1, keepdims=True), atol=1e-15)


def pin_group_limit_hand_built(o):
    """Hand-worked group-limited selection for both group rules."""
    g = _golden("group_limit_hand_built.json")
    sel = np.array([g["sel"]])
    # sigmoid^-1 of the wanted scores gives logits whose sigmoid is `sel`
    # exactly enough; feed the scores through the bias with zero logits
    # instead: s = 1/2 everywhere, bias = sel - 1/2.
    E = sel.shape[1]
    for rule, key in (("top2sum", "expected_ids_top2sum"), ("max", "expected_ids_max")):
        r = o.route(np.zeros((1, E)), np.eye(E), g["k"], score="sigmoid",
                    select_bias=sel[0] - 0.5, n_groups=g["n_groups"],
                    topk_groups=g["topk_groups"], group_rule=rule)
        assert r["ids"][0].tolist() == g[key], (rule, r["ids"])


def pin_group_limit_invariants(o):
    """No token uses more than topk_groups groups; one group, or keeping every
    group, is plain top-k."""
    inp = _tiny_inputs(6, T=40, E=16)
    x, w = inp["x"], inp["w_router"]
    r = o.route(x, w, 4, score="sigmoid", n_groups=4, topk_groups=2)
    assert max(len(set((r["ids"][t] // 4).tolist())) for t in range(40)) <= 2
    plain = o.route(x, w, 4, score="sigmoid")
    for ng, tg in ((1, 1), (4, 4)):
        rr = o.route(x, w, 4, score="sigmoid", n_groups=ng, topk_groups=tg)
        assert (rr["ids"] == plain["ids"]).all()


def pin_logit_bias_is_an_extra_feature(o):
    """An additive per-expert logit bias b routes exactly like a router with
    one more input feature fixed at 1 whose weight column is b (a Linear with
    bias written as a bias-free Linear); z-loss and weights included."""
    inp = _tiny_inputs(19, T=15, E=6)
    b = _rng(20).normal(size=6) * 2.0
    xa = np.concatenate([inp["x"], np.ones((15, 1))], axis=1)
    wa = np.concatenate([inp["w_router"], b[:, None]], axis=1)
    for score, renorm in (("softmax", False), ("softmax", True), ("sigmoid", True)):
        r1 = o.route(inp["x"], inp["w_router"], 2, score=score, renormalize=renorm,
                     logit_bias=b)
        r2 = o.route(xa, wa, 2, score=score, renormalize=renorm)
        assert (r1["ids"] == r2["ids"]).all()
        assert np.allclose(r1["weights"], r2["weights"], rtol=0, atol=1e-14)
        assert abs(r1["z"] - r2["z"]) < 1e-12
    r0 = o.route(inp["x"], inp["w_router"], 2)
    r1 = o.route(inp["x"], inp["w_router"], 2, logit_bias=b)
    assert not (r0["ids"] == r1["ids"]).all()


def pin_near_tie_flag(o):
    """Exact ties are flagged; well separated scores are not."""
    h = np.array([[1.0, 1.0, 0.0, -1.0], [3.0, 0.0, -3.0, -6.0]])
    r = _route_logits(o, h, 1)
    assert r["near_tie"].tolist() == [True, False]


def pin_group_near_tie_flag(o):
    """Hand-worked group-limited tokens: a gap below 1e-5 between the last
    kept group and the first dropped one is flagged even when the chosen
    experts are well separated; the same gap at 1e-3, or a near tie between
    two dropped groups, is not; a near tie between the kept groups is."""
    g = _golden("group_near_tie_hand_built.json")
    s = np.array(g["sel"])
    h = np.log(s / (1.0 - s))  # sigmoid(h) = s
    r = _route_logits(o, h, g["k"], score="sigmoid", n_groups=g["n_groups"],
                      topk_groups=g["topk_groups"])
    assert r["ids"].tolist() == g["expected_ids"], r["ids"]
    assert r["near_tie"].tolist() == g["expected_near_tie"], r["margin"]


# ------------------------------------------------------------- aux ---------

def pin_balance_uniform_is_one(o):
    """Balance loss is exactly 1 at uniform assignment and uniform mean
    probability (lab, 'Read the loss values correctly')."""
    E = 6
    base = np.array([1.3, -0.2, 0.7, 0.1, -1.1, 0.4])
    h = np.stack([np.roll(base, t) for t in range(E)])   # each expert wins once
    r = _route_logits(o, h, 1)
    assert (np.bincount(r["ids"][:, 0], minlength=E) == 1).all()
    assert abs(r["balance"] - 1.0) < 1e-14


def pin_balance_collapsed_is_E(o):
    """A fully collapsed router gives balance = E (book, aux-loss section)."""
    E = 5
    h = np.tile(np.array([200.0, 0.0, 0.0, 0.0, 0.0]), (7, 1))
    r = _route_logits(o, h, 1)
    assert abs(r["balance"] - E) < 1e-12


def pin_z_constant_logits(o):
    """For constant logits c over E experts, logsumexp = c + ln E, so the
    z-loss is (c + ln E)^2."""
    for c, E in ((0.0, 4), (1.5, 8), (-2.0, 3)):
        r = _route_logits(o, np.full((3, E), c), 1)
        assert abs(r["z"] - (c + math.log(E)) ** 2) < 1e-13


def pin_counts_sum(o):
    """Counts sum to T*k, also when a capacity later drops assignments."""
    inp = _tiny_inputs(7, T=33, E=5)
    for k in (1, 2, 5):
        r = o.route(inp["x"], inp["w_router"], k)
        assert int(r["counts"].sum()) == 33 * k
        f = o.forward(inp, top_k=k, capacity_factor=0.5)
        assert int(f["route"]["counts"].sum()) == 33 * k
        assert f["n_kept"] == int(np.minimum(f["route"]["counts"], f["capacity"]).sum())


# ------------------------------------------------------------- capacity ----

def pin_capacity_exercise(o):
    """Book exercise 2: capacity 768, 132 dropped when 900 tokens pick one expert."""
    g = _golden("capacity_exercise.json")
    ex = g["expected"]
    E, k, N, cf = g["E"], g["k"], g["N"], g["capacity_factor"]
    assert N * k // E == ex["avg_tokens_per_expert"]
    C = o.capacity(cf, N, k, E)
    assert C == ex["capacity"]
    ids = np.zeros((g["hot_expert_tokens"], 1), dtype=np.int64)
    keep = o.first_within_capacity(ids, E, C)
    assert int((~keep).sum()) == ex["dropped_at_hot_expert"]
    assert E * 2 * g["d_model"] * g["d_ff"] == ex["total_expert_params_two_matrix"]
    assert k * 2 * g["d_model"] * g["d_ff"] == ex["active_expert_params_per_token"]


def pin_capacity_small_cases(o):
    """ceil and the floor of 1: 1.25*8192/64 = 160 exactly; tiny batches get 1."""
    assert o.capacity(1.25, 8192, 1, 64) == 160
    assert o.capacity(1.0, 10, 1, 4) == 3
    assert o.capacity(0.01, 3, 1, 64) == 1
    assert o.capacity(None, 10, 2, 4) is None


def pin_capacity_hand_built(o):
    """The hand-built keep mask, offsets and row order."""
    g = _golden("capacity_hand_built.json")
    ids = np.array(g["ids"])
    keep = o.first_within_capacity(ids, g["E"], g["capacity"])
    assert keep.tolist() == g["expected_keep"]
    assert int((~keep).sum()) == g["expected_dropped"]
    off, r2a, a2r = o.permutation(ids, keep, g["E"])
    assert off.tolist() == g["expected_expert_offsets"]
    assert r2a.tolist() == g["expected_row_to_assign"]
    assert a2r.tolist() == g["expected_assign_to_row"]


def pin_drop_is_rank_in_token_order(o):
    """An assignment is dropped exactly when at least C earlier tokens chose
    the same expert (a counting restatement of the first-come walk)."""
    r = _rng(8)
    E, T, k, C = 5, 60, 2, 9
    ids = np.stack([r.choice(E, size=k, replace=False, p=[.4, .3, .1, .1, .1])
                    for _ in range(T)])
    keep = o.first_within_capacity(ids, E, C)
    for t in range(T):
        for s in range(k):
            earlier = int((ids[:t] == ids[t, s]).sum())
            assert keep[t, s] == (earlier < C)


def pin_permutation_inverse(o):
    """Permute then inverse-permute restores token order; rows are sorted by
    (expert, token) and cover every kept assignment once."""
    r = _rng(9)
    E, T, k = 7, 50, 3
    ids = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)])
    keep = o.first_within_capacity(ids, E, 12)
    off, r2a, a2r = o.permutation(ids, keep, E)
    payload = np.arange(T * k) * 10 + 3
    rows = payload[r2a]
    back = np.full(T * k, -1)
    back[r2a] = rows
    assert (back[keep.reshape(-1)] == payload[keep.reshape(-1)]).all()
    assert sorted(r2a.tolist()) == np.nonzero(keep.reshape(-1))[0].tolist()
    e_of_row = ids.reshape(-1)[r2a]
    t_of_row = r2a // k
    assert all((e_of_row[i], t_of_row[i]) < (e_of_row[i + 1], t_of_row[i + 1])
               for i in range(len(r2a) - 1))
    for e in range(E):
        assert (e_of_row[off[e]:off[e + 1]] == e).all()
    assert ((a2r >= 0) == keep.reshape(-1)).all()


def pin_empty_experts(o):
    """Forced routes that leave experts empty run and give empty groups."""
    inp = _tiny_inputs(10, T=6, E=5)
    ids = np.array([[3, 1]] * 6)
    w = np.full((6, 2), 0.5)
    f = o.forward(inp, top_k=2, routing={"ids": ids, "weights": w})
    off = f["expert_offsets"]
    assert off.tolist() == [0, 0, 6, 6, 12, 12]
    ref = o.brute_force_forward(inp, ids, w)
    assert np.allclose(f["out"], ref, rtol=0, atol=1e-13)


# ------------------------------------------------------------- experts -----

def pin_swiglu_scalar_closed_form(o):
    """D = H = 1: FFN(z) = wd * (wg z) sigmoid(wg z) * (wu z)."""
    for z, wg, wu, wd in ((2.0, 1.0, 1.0, 1.0), (-0.7, 1.9, -0.4, 2.2)):
        y = o.swiglu_ffn(np.array([[z]]), np.array([[wg]]), np.array([[wu]]),
                         np.array([[wd]]))
        want = wd * (wg * z) / (1.0 + math.exp(-wg * z)) * (wu * z)
        assert abs(y[0, 0] - want) < 1e-15


def pin_swiglu_loops(o):
    """Matrix form equals explicit sums over the Linear layout W[out, in]."""
    r = _rng(11)
    D, H = 4, 3
    z = r.normal(size=(2, D))
    wg, wu, wd = r.normal(size=(H, D)), r.normal(size=(H, D)), r.normal(size=(D, H))
    y = o.swiglu_ffn(z, wg, wu, wd)
    for n in range(2):
        for d in range(D):
            acc = 0.0
            for j in range(H):
                g = sum(wg[j, i] * z[n, i] for i in range(D))
                u = sum(wu[j, i] * z[n, i] for i in range(D))
                acc += wd[d, j] * (g / (1.0 + math.exp(-g))) * u
            assert abs(y[n, d] - acc) < 1e-13


def pin_identical_experts_are_dense(o):
    """Identical experts with weights summing to 1 reproduce one dense FFN
    (lab required test; book 'Sparse upcycling' at zero jitter), with or
    without a shared expert added on top."""
    inp = _tiny_inputs(12, T=11, E=4, shared=True)
    for key in ("w_gate", "w_up", "w_down"):
        inp[key] = np.repeat(inp[key][:1], 4, axis=0)
    inp["w_router"] = _rng(13).normal(size=inp["w_router"].shape) * 1e-3
    dense = o.swiglu_ffn(inp["x"], inp["w_gate"][0], inp["w_up"][0], inp["w_down"][0])
    shared = o.swiglu_ffn(inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"])
    f = o.forward(inp, top_k=2)
    assert np.allclose(f["out"], dense + shared, rtol=0, atol=1e-13)
    no_shared = {k: v for k, v in inp.items() if not k.startswith("ws_")}
    f = o.forward(no_shared, top_k=3)
    assert np.allclose(f["out"], dense, rtol=0, atol=1e-13)


def pin_dense_limit_mean(o):
    """top_k = E with a zero router weights every expert 1/E: the output is the
    mean of the E experts (the dense mixture of the book's first section)."""
    inp = _tiny_inputs(14, T=5, E=4)
    inp["w_router"] = np.zeros_like(inp["w_router"])
    f = o.forward(inp, top_k=4)
    each = [o.swiglu_ffn(inp["x"], inp["w_gate"][e], inp["w_up"][e], inp["w_down"][e])
            for e in range(4)]
    assert np.allclose(f["out"], sum(each) / 4.0, rtol=0, atol=1e-14)


def pin_forward_matches_brute_force(o):
    """Dispatch/combine equals the token-by-token loop and the all-experts-then-
    mask form on tiny shapes (lab 'Trace one token by hand')."""
    for seed, k, shared in ((15, 2, False), (16, 3, True)):
        inp = _tiny_inputs(seed, T=13, E=5, shared=shared)
        f = o.forward(inp, top_k=k)
        r = f["route"]
        bf = o.brute_force_forward(inp, r["ids"], r["weights"])
        assert np.allclose(f["out"], bf, rtol=0, atol=1e-12)
        if not shared:
            am = o.all_experts_then_mask(inp, r["ids"], r["weights"])
            assert np.allclose(f["out"], am, rtol=0, atol=1e-12)


def pin_dropped_tokens_get_zero(o):
    """With a capacity, a token whose every slot is dropped gets exactly zero
    from the routed branch; kept slots match the brute-force loop."""
    inp = _tiny_inputs(17, T=20, E=3)
    f = o.forward(inp, top_k=1, capacity_factor=0.3)
    keep = f["keep"]
    assert (~keep).any()
    bf = o.brute_force_forward(inp, f["route"]["ids"], f["route"]["weights"], keep)
    assert np.allclose(f["out"], bf, rtol=0, atol=1e-13)
    assert (f["out"][~keep[:, 0]] == 0).all()


def pin_subset_tokens(o):
    """Evaluating a subset of tokens gives the same rows as the full forward."""
    inp = _tiny_inputs(18, T=17, E=4, shared=True)
    full = o.forward(inp, top_k=2, capacity_factor=0.8)
    sub = o.forward(inp, top_k=2, capacity_factor=0.8, tokens=[16, 3, 0])
    assert np.allclose(sub["out"], full["out"][[16, 3, 0]], rtol=0, atol=1e-15)


# ------------------------------------------- forward variants (NeMo flags) --


def pin_sqrtsoftplus_closed_form(o):
    """score_func 'sqrtsoftplus': s = sqrt(ln(1 + e^h)) per expert, written out
    with math on scalars; renormalised weights s_i / sum s times route_scale."""
    h = [1.5, -0.25, 3.0, -4.0, 0.0]
    r = _route_logits(o, [h], 2, score="sqrtsoftplus", route_scale=2.0)
    s = [math.sqrt(math.log(1.0 + math.exp(v))) for v in h]
    assert np.allclose(r["scores"][0], s, rtol=0, atol=1e-14)
    assert r["ids"][0].tolist() == [2, 0]
    assert np.allclose(r["weights"][0], [2.0 * s[2] / (s[2] + s[0]), 2.0 * s[0] / (s[2] + s[0])],
                       rtol=0, atol=1e-14)
    # large logits do not overflow: softplus(h) -> h
    r2 = _route_logits(o, [[800.0, 0.0]], 1, score="sqrtsoftplus", renormalize=False)
    assert abs(r2["weights"][0, 0] - math.sqrt(800.0)) < 1e-12


def pin_sqrtsoftplus_selects_like_logits(o):
    """sqrt(softplus(.)) is strictly increasing, so without a bias it selects
    exactly the experts softmax selects, in the same slot order."""
    inp = _tiny_inputs(31, T=40, E=7)
    a = o.route(inp["x"], inp["w_router"], 3, score="sqrtsoftplus")
    b = o.route(inp["x"], inp["w_router"], 3, score="softmax")
    assert (a["ids"] == b["ids"]).all()


def pin_softmax_then_topk_without_renorm(o):
    """GShard/Switch convention for k > 1 (book 'The Router'): the kept weights
    are the slice of the full softmax and do not sum to 1."""
    h = [2.0, 1.0, 0.0, -1.0]
    r = _route_logits(o, [h], 2, renormalize=False)
    e = [math.exp(v) for v in h]
    assert np.allclose(r["weights"][0], [e[0] / sum(e), e[1] / sum(e)], rtol=0, atol=1e-15)
    assert r["weights"][0].sum() < 1.0


def pin_token_mask_routing(o):
    """Masked tokens are not routed: IDs -1, weights 0, no load, and the aux
    means run over the unmasked tokens only (a masked copy of a routed batch
    gives the balance and z of the unmasked part)."""
    inp = _tiny_inputs(32, T=12, E=5)
    x, w = inp["x"], inp["w_router"]
    mask = np.array([1, 0, 1, 1, 0, 0, 1, 1, 1, 0, 1, 1], dtype=bool)
    r = o.route(x, w, 2, token_mask=mask)
    sub = o.route(x[mask], w, 2)
    assert (r["ids"][~mask] == -1).all() and (r["weights"][~mask] == 0).all()
    assert (r["ids"][mask] == sub["ids"]).all()
    assert (r["counts"] == sub["counts"]).all() and r["counts"].sum() == 2 * mask.sum()
    assert abs(r["balance"] - sub["balance"]) < 1e-14 and abs(r["z"] - sub["z"]) < 1e-14
    assert np.allclose(r["mean_prob"], sub["mean_prob"], rtol=0, atol=1e-15)
    none = o.route(x, w, 2, token_mask=np.zeros(12, dtype=bool))
    assert none["counts"].sum() == 0 and none["balance"] == 0 and none["z"] == 0


def pin_token_mask_forward(o):
    """Masked tokens get no routed output (only the shared expert), take no
    capacity, and the unmasked tokens match the layer run on them alone."""
    inp = _tiny_inputs(33, T=14, E=3, shared=True)
    mask = np.ones(14, dtype=bool)
    mask[[0, 5, 6, 13]] = False
    f = o.forward(inp, top_k=2, capacity_factor=0.7, token_mask=mask)
    sub_inp = dict(inp, x=inp["x"][mask])
    T_sub = int(mask.sum())
    # same C as the masked run (C counts the configured T, not the unmasked)
    cap = o.capacity(0.7, 14, 2, 3)
    r_sub = o.route(sub_inp["x"], inp["w_router"], 2)
    keep_sub = o.first_within_capacity(r_sub["ids"], 3, cap)
    assert (f["keep"][mask] == keep_sub).all() and not f["keep"][~mask].any()
    Y = o.expert_outputs(sub_inp["x"], r_sub["ids"], r_sub["weights"], keep_sub,
                         inp["w_gate"], inp["w_up"], inp["w_down"])
    shared = o.swiglu_ffn(inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"])
    assert np.allclose(f["out"][mask], Y.sum(1) + shared[mask], rtol=0, atol=1e-13)
    assert np.allclose(f["out"][~mask], shared[~mask], rtol=0, atol=1e-14)
    assert T_sub == 10


def pin_swiglu_limit_closed_form(o):
    """Clamped SwiGLU: both projections clamped to [-L, L] (scalars worked by
    hand), a limit above every projection changes nothing, 0 means off."""
    L = 0.5
    z = np.array([[1.0]])
    for g, u in ((2.0, 3.0), (-2.0, 0.25), (0.3, -4.0)):
        out = o.swiglu_ffn(z, [[g]], [[u]], [[1.0]], limit=L)[0, 0]
        gc, uc = max(-L, min(L, g)), max(-L, min(L, u))
        assert abs(out - gc * _sig(gc) * uc) < 1e-15
    inp = _tiny_inputs(34, T=6, E=3)
    a = o.forward(inp, top_k=2)["out"]
    b = o.forward(inp, top_k=2, swiglu_limit=1e9)["out"]
    c = o.forward(inp, top_k=2, swiglu_limit=0.0)["out"]
    assert np.array_equal(a, b) and np.array_equal(a, c)
    d = o.forward(inp, top_k=2, swiglu_limit=0.05)["out"]
    assert not np.allclose(a, d)


def pin_shared_expert_gate(o):
    """A zero gate vector halves the shared output (sigmoid(0) = 1/2); a gate
    vector along x with a large norm passes it through; the token loop agrees."""
    inp = _tiny_inputs(35, T=7, E=3, shared=True)
    base = o.forward(inp, top_k=1)
    plain = o.shared_expert(inp["x"], inp)
    half = o.forward(dict(inp, ws_sgate=np.zeros(inp["x"].shape[1])), top_k=1)
    assert np.allclose(half["out"], base["out"] - 0.5 * plain, rtol=0, atol=1e-13)
    big = o.forward(dict(inp, ws_sgate=50.0 * np.ones(inp["x"].shape[1])), top_k=1)
    s = inp["x"].sum(1)
    g = 1.0 / (1.0 + np.exp(-50.0 * s))
    assert np.allclose(big["out"], base["out"] - plain + g[:, None] * plain, rtol=0, atol=1e-12)
    r = big["route"]
    bf = o.brute_force_forward(dict(inp, ws_sgate=50.0 * np.ones(inp["x"].shape[1])),
                               r["ids"], r["weights"])
    assert np.allclose(big["out"], bf, rtol=0, atol=1e-12)


def pin_update_bias_rule(o):
    """Hand-worked step: counts (5, 1, 2, 0) have mean 2, so expert 0 goes
    down, experts 1 and 3 go up and expert 2 (at the mean) stays."""
    b = o.update_bias([0.5, -0.25, 0.0, 1.0], [5, 1, 2, 0], 0.125)
    assert b.tolist() == [0.375, -0.125, 0.0, 1.125]
    assert o.update_bias([0.1, 0.2], [7, 7], 1.0).tolist() == [0.1, 0.2]


def pin_update_bias_balances(o):
    """The book's demonstration: a router that favours one expert, corrected by
    repeated select-with-bias steps, ends far more uniform, with a negative
    bias on the favourite (selection on logits + bias, renormalised softmax of
    the unbiased logits, as in the exercise)."""
    r = np.random.default_rng(36)
    h = r.normal(size=(1024, 8))
    h[:, 0] += 3.0
    bias = np.zeros(8)
    first = None
    for _ in range(200):
        rr = _route_logits(o, h + bias[None, :], 2)
        counts = rr["counts"]
        first = counts if first is None else first
        bias = o.update_bias(bias, counts, 1e-2)
    assert counts.max() / max(counts.min(), 1) < first.max() / max(first.min(), 1) / 4
    assert bias[0] < 0 and bias[0] == bias.min()


def pin_residual_is_added(o):
    """The residual stream adds to the layer output exactly."""
    inp = _tiny_inputs(37, T=8, E=3, shared=True)
    res = _rng(38).normal(size=inp["x"].shape)
    a = o.forward(inp, top_k=2)["out"]
    b = o.forward(inp, top_k=2, residual=res)["out"]
    assert np.allclose(b, a + res, rtol=0, atol=1e-15)


def pin_bf16_rounding_ties_and_library(o):
    """Rounding to bfloat16 (8 significant bits): exact ties go to the even
    neighbour, anything past a tie goes up, and float32 inputs (exact in
    float64) round as torch's own float32 -> bfloat16 conversion does."""
    u = 2.0 ** -7                                 # bf16 spacing in [1, 2)
    cases = {1.0: 1.0, 1.0 + u: 1.0 + u, 1.0 + u / 2: 1.0, 1.0 + 3 * u / 2: 1.0 + 2 * u,
             1.0 + u / 2 + 2.0 ** -40: 1.0 + u, 1.0 + u / 2 - 2.0 ** -40: 1.0,
             -(1.0 + 3 * u / 2): -(1.0 + 2 * u), 2.0 - 3 * u / 4: 2.0 - u, 2.0 - u / 4: 2.0,
             2.0 - u / 2: 2.0,
             3.0 * 2.0 ** -20: 3.0 * 2.0 ** -20}
    got = o.round_to_bf16(np.array(list(cases)))
    assert np.array_equal(got, np.array(list(cases.values()))), got
    import torch
    v32 = (_rng(41).normal(size=4000) * np.exp(_rng(42).uniform(-8, 8, 4000))).astype(np.float32)
    lib = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(o.round_to_bf16(v32.astype(np.float64)), lib)


def pin_rms_norm_loops_and_library(o):
    """RMSNorm against a pure-Python loop on a tiny matrix and against
    torch.nn.functional.rms_norm in float64; unit mean square with w = 1 and
    eps = 0; a constant row c gives w * c / sqrt(c^2 + eps)."""
    r = _rng(43)
    x = r.normal(size=(4, 7)) * 3.0
    w = r.uniform(0.5, 2.0, size=7)
    eps = 0.25
    got = o.rms_norm(x, w, eps, act=None)
    for t in range(4):
        ms = sum(v * v for v in x[t]) / 7
        for d in range(7):
            assert abs(got[t, d] - x[t, d] / math.sqrt(ms + eps) * w[d]) < 1e-14
    import torch
    lib = torch.nn.functional.rms_norm(torch.from_numpy(x), (7,), torch.from_numpy(w), eps)
    assert np.allclose(got, lib.numpy(), rtol=1e-14, atol=0)
    y = o.rms_norm(x, None, 0.0, act=None)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-14)
    c = np.full((1, 5), -0.5)
    assert np.allclose(o.rms_norm(c, w[:5], 0.75, act=None), w[:5] * -0.5 / 1.0, rtol=1e-15)


def pin_rms_norm_rounds_once(o):
    """The normalised rows are the float64 values rounded once to the
    activation dtype."""
    x = _rng(44).normal(size=(6, 33))
    exact = o.rms_norm(x, None, 1e-6, act=None)
    assert np.array_equal(o.rms_norm(x, None, 1e-6, act="bf16"), o.round_to_bf16(exact))
    assert np.array_equal(o.rms_norm(x, None, 1e-6, act="f32"),
                          exact.astype(np.float32).astype(np.float64))


def pin_pre_norm_layer_is_scale_free(o):
    """With eps = 0 the pre-normed layer cannot see the scale of its input:
    x and 4x (a power of two, so every rounding is the same) give the same
    routes and outputs; the router and experts take the normalised rows."""
    inp = _tiny_inputs(45, T=10, E=4, shared=True)
    w = _rng(46).uniform(0.5, 1.5, size=inp["x"].shape[1])
    a = o.forward(inp, top_k=2, pre_norm=(w, 0.0, "bf16"))
    big = dict(inp, x=inp["x"] * 4.0)
    b = o.forward(big, top_k=2, pre_norm=(w, 0.0, "bf16"))
    assert np.array_equal(a["route"]["ids"], b["route"]["ids"])
    assert np.allclose(a["out"], b["out"], rtol=0, atol=1e-14)
    normed = dict(inp, x=o.rms_norm(inp["x"], w, 0.0, "bf16"))
    c = o.forward(normed, top_k=2)
    assert np.allclose(a["out"], c["out"], rtol=0, atol=1e-14)
    raw = o.forward(inp, top_k=2)
    assert not np.allclose(a["out"], raw["out"], rtol=0, atol=1e-6)


GRAD_OF = {"x": "dx", "w_router": "dw_router", "w_gate": "dw_gate", "w_up": "dw_up",
           "w_down": "dw_down", "ws_gate": "dws_gate", "ws_up": "dws_up", "ws_down": "dws_down",
           "ws_sgate": "d_shared_gate"}


def _fd_agrees(o, inp, seed, aux, **fw):
    """Central finite differences of the loss along random directions, one per
    parameter, against the analytic gradient.  The step is small enough that
    no route or drop changes (checked)."""
    r = _rng(seed)
    dout = r.normal(size=inp["x"].shape)
    g = o.backward(inp, dout, aux_coef=aux, **fw)
    base = o.forward(inp, **fw)
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        if inp.get(name) is None:
            continue
        V = r.normal(size=np.shape(inp[name]))
        lp, fp = o.loss(dict(inp, **{name: inp[name] + eps * V}), dout, aux, **fw)
        lm, fm = o.loss(dict(inp, **{name: inp[name] - eps * V}), dout, aux, **fw)
        for ff in (fp, fm):
            assert np.array_equal(ff["route"]["ids"], base["route"]["ids"]), "route moved"
            assert np.array_equal(ff["keep"], base["keep"]), "drops moved"
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(g[gname] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
        assert abs(an) > 1e-3, (name, an)  # the direction exercises the gradient


def pin_backward_fd_softmax_capacity_shared(o):
    """Softmax, renormalised top-2, capacity drops, shared expert, both aux terms."""
    inp = _tiny_inputs(51, T=12, E=4, shared=True)
    _fd_agrees(o, inp, 52, (0.3, 0.2), top_k=2, capacity_factor=0.75)


def pin_backward_fd_gated_shared_expert(o):
    """The shared expert scaled per token by sigmoid(x . w_sg): central
    differences for w_sg, x and the shared weights."""
    inp = _tiny_inputs(60, T=9, E=4, shared=True)
    inp["ws_sgate"] = _rng(61).normal(size=inp["x"].shape[1]) * 0.5
    _fd_agrees(o, inp, 62, (0.1, 0.05), top_k=2)


def pin_backward_fd_sigmoid_groups_scale(o):
    """Sigmoid scores with a selection bias, group limit, route_scale 2.5."""
    inp = _tiny_inputs(53, T=10, E=8)
    inp["select_bias"] = _rng(54).normal(size=8) * 0.1
    _fd_agrees(o, inp, 55, (0.5, 0.1), top_k=3, score="sigmoid", route_scale=2.5,
               n_groups=4, topk_groups=2)


def pin_backward_fd_switch_top1(o):
    """Switch top-1: raw softmax weight (no renorm) times a route scale, logit
    bias, capacity."""
    inp = _tiny_inputs(56, T=14, E=4)
    inp["logit_bias"] = -1.1 * np.log(np.arange(1, 5))
    _fd_agrees(o, inp, 57, (0.2, 0.05), top_k=1, renormalize=False, capacity_factor=1.0,
               route_scale=1.7)


def pin_backward_fd_sqrtsoftplus_mask_limit(o):
    """sqrt-softplus scores, a token mask and the SwiGLU clamp."""
    inp = _tiny_inputs(58, T=11, E=5, std=0.8)
    mask = np.ones(11, dtype=bool)
    mask[[0, 4, 5]] = False
    _fd_agrees(o, inp, 59, (0.4, 0.3), top_k=2, score="sqrtsoftplus", token_mask=mask,
               swiglu_limit=0.6)


def pin_backward_zero_router_grad_top1_renorm(o):
    """Renormalised top-1 weights are exactly 1, so without aux terms the
    router gets no gradient ([LAB] "Ablation 2: top-1 versus top-2")."""
    inp = _tiny_inputs(60, T=9, E=4)
    g = o.backward(inp, _rng(61).normal(size=inp["x"].shape), top_k=1)
    assert np.abs(g["dw_gate"]).max() > 0.1
    assert np.abs(g["dw_router"]).max() < 1e-12


def pin_router_backward_rows(o):
    """The router gradient of a subset of tokens equals those rows of the
    full one (the balance and z terms use every token's counts)."""
    inp = _tiny_inputs(62, T=12, E=5)
    r = o.route(inp["x"], inp["w_router"], 2)
    dgw = _rng(63).normal(size=(12, 2))
    full = o.router_backward(r, dgw, top_k=2, aux_coef=(0.3, 0.2))
    sub = o.router_backward(r, dgw, top_k=2, aux_coef=(0.3, 0.2), tokens=[1, 4, 11])
    assert np.array_equal(sub, full[[1, 4, 11]])


def pin_backward_fd_pre_norm(o):
    """The pre-normed layer (without the rounding of the normalised rows):
    central differences for x, the norm weight and the experts; dx then
    includes the norm's own Jacobian."""
    inp = _tiny_inputs(64, T=10, E=4, shared=True)
    r = _rng(65)
    nw = r.uniform(0.5, 1.5, size=inp["x"].shape[1])
    dout = r.normal(size=inp["x"].shape)
    aux = (0.2, 0.1)
    fw = dict(top_k=2)
    g = o.backward(inp, dout, aux_coef=aux, pre_norm=(nw, 0.05, None), **fw)
    eps = 1e-6
    base = o.forward(inp, pre_norm=(nw, 0.05, None), **fw)
    for name in ("x", "w_gate", "w_router", "norm"):
        V = r.normal(size=nw.shape if name == "norm" else np.shape(inp[name]))
        vals = []
        for sgn in (1, -1):
            if name == "norm":
                lv, f = o.loss(inp, dout, aux, pre_norm=(nw + sgn * eps * V, 0.05, None), **fw)
            else:
                lv, f = o.loss(dict(inp, **{name: inp[name] + sgn * eps * V}), dout, aux,
                               pre_norm=(nw, 0.05, None), **fw)
            assert np.array_equal(f["route"]["ids"], base["route"]["ids"]), "route moved"
            vals.append(lv)
        fd = (vals[0] - vals[1]) / (2 * eps)
        an = float(np.sum((g["d_norm_weight"] if name == "norm" else g[GRAD_OF[name]]) * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def pin_rms_norm_backward_loops(o):
    """The RMSNorm gradients against a pure-Python loop of the chain rule."""
    r = _rng(66)
    x, w, dy = r.normal(size=(3, 5)), r.uniform(0.5, 2, 5), r.normal(size=(3, 5))
    dx, dw = o.rms_norm_backward(x, w, 0.3, dy)
    for t in range(3):
        s = math.sqrt(sum(v * v for v in x[t]) / 5 + 0.3)
        for d in range(5):
            ref = 0.0
            for j in range(5):  # d y_tj / d x_td
                dyj_dxd = (w[j] / s) * ((1.0 if j == d else 0.0) - x[t, j] * x[t, d] / (5 * s * s))
                ref += dy[t, j] * dyj_dxd
            assert abs(dx[t, d] - ref) < 1e-13
    for d in range(5):
        assert abs(dw[d] - sum(dy[t, d] * x[t, d] / math.sqrt(np.mean(x[t] ** 2) + 0.3)
                               for t in range(3))) < 1e-13


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
