"""Plain, slow, float64 CPU oracle for the top-k token-choice MoE-layer forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.  It shares
no code with the HIP library; both sides only consume the same seeded inputs.

Sources (the pages this follows; section names as printed on each page):
  [LAB]  "Lab: build a tiny MoE in PyTorch" (open-llm-engineering), sections
         "The contract", "Full implementation", "Smoke test and backward pass",
         "Trace one token by hand", "Read the loss values correctly",
         "Ablation 2: top-1 versus top-2", "Add a capacity limit",
         "Add a shared expert", "Required correctness tests", "Lab extensions".
  [BOOK] "2.9 Mixture-of-Experts (MoE) Architectures" (llm-stack-book), sections
         "From One FFN to a Bank of Experts", "The Router: Gating, Top-k, and the
         Softmax-Then-Select Question", "A Toy MoE Layer From Scratch",
         "The auxiliary load-balancing loss", "Capacity Factor, Token Dropping,
         and the Worked Numbers", "DeepSeek-MoE and the fine-grained +
         shared-expert idea", "Sparse upcycling", "Exercises".
  [ST]   "st-moe-pytorch" API reference, "rms-norm" (RMSNorm before the MoE
         inside ``SparseMoEBlock``; the prenormalisation pattern).
  [NEMO] "nemo_automodel.components.moe.layers" (NeMo AutoModel v0.4 API):
         class ``Gate`` attributes ``score_func``, ``n_groups``, ``topk_groups``,
         ``norm_topk_prob``, ``route_scale``; class ``MLP`` (SwiGLU, no bias).

Precision: every floating-point step runs in float64 on the exact stored input
values (bf16 or fp32 upcast without rounding).

Readings taken where the pages are silent or garbled:
  * top-k ties go to the lower expert index; slot j holds the j-th largest
    selection score (the tie rule is what makes a zero router pick experts
    0..k-1, as [BOOK] "Sparse upcycling" states);
  * capacity drops are first-come in token order, slot order inside a token
    ([LAB] "Add a capacity limit"); counts and the balance loss use the
    pre-drop assignments; surviving weights are not renormalised;
  * sigmoid scoring adds the per-expert correction bias to the scores for
    selection only; gate weights use the unbiased scores ([BOOK] "The Router",
    noisy/top-k gating paragraph; [NEMO] ``score_func`` 'sigmoid');
  * group-limited routing ranks each contiguous group by the sum of its two
    largest biased scores (``group_rule='top2sum'``) or by its maximum
    (``'max'``).  PARITY UNPINNED: the pages name ``n_groups``/``topk_groups``
    but define no group score;
  * for sigmoid scoring the balance loss uses P_e = mean_t s_te / sum_e' s_te'.
    PARITY UNPINNED: the pages give no formula for this case.
  * ``score='sqrtsoftplus'`` ([NEMO] ``score_func``): s = sqrt(softplus(h)),
    normalised like sigmoid.  The pages only name it; the score is read from
    the name (pinned by its closed form and by selecting exactly what the
    logits select);
  * a token mask ([NEMO] ``Gate.forward(x, token_mask)``, ``MoE.forward``'s
    ``padding_mask``): masked tokens are not routed (IDs -1, weights 0), take
    no capacity, contribute no routed output, and are left out of counts and
    of the means in P_e and z; the shared expert still applies to them;
  * ``swiglu_limit`` ([NEMO] ``MLP``, ``_clamped_swiglu_act``): the gate and
    up projections are each clamped to [-limit, limit] before silu(g) * u;
    0 means no clamp.  PARITY UNPINNED: the pages name the clamp, not its form;
  * a shared-expert gate ([NEMO] ``MoE.shared_expert_gate``): the shared
    output is scaled per token by sigmoid(x . w_sg).  PARITY UNPINNED: the
    pages name the gate, not its form;
  * the backward pass: gradients of <dout, out> + alpha * balance + beta * z
    ([LAB] "Smoke test and backward pass") with the selected IDs, the drops
    and the counts f held constant ([BOOK] "The Router": top-k is a stop-
    gradient on the index decision; "The auxiliary load-balancing loss": f is
    detached); the SwiGLU clamp passes gradient strictly inside the limits;
  * the pre-norm ([LAB] "Put the MoE into a decoder block", where the MoE
    branch takes the RMS-normalised residual stream; [ST] the RMSNorm of
    ``SparseMoEBlock``): y = x * w / sqrt(mean(x^2) + eps) per token, computed
    in float64 and rounded once to the activation dtype (bfloat16: nearest,
    ties to even), because the layer receives a tensor of that dtype.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "NEAR_TIE", "router_logits", "softmax", "sigmoid", "softplus", "logsumexp",
    "route", "capacity", "first_within_capacity", "permutation",
    "swiglu_ffn", "expert_outputs", "shared_expert", "combine", "forward", "update_bias",
    "round_to_bf16", "rms_norm", "rms_norm_backward", "loss", "backward", "router_backward",
    "swiglu_ffn_backward",
    "brute_force_forward", "all_experts_then_mask",
]

# Tokens whose top-(k+1) selection scores (or top group scores) sit closer than
# this are "near ties": a last-bit difference may flip the choice.
NEAR_TIE = 1e-5


# ---------------------------------------------------------------- router ---

def router_logits(x, w_router, logit_bias=None):
    """h[t, e] = sum_d x[t, d] * W_r[e, d]  (+ logit_bias[e]).

    The router is a bias-free Linear(d_model, E) ([LAB] "Full implementation",
    ``self.router``); its math is done in high precision ([LAB] comment on
    router math in float32; here float64).  ``logit_bias`` is an additive
    per-expert logit offset ([NEMO] score function 'softmax_with_bias')."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float64)
    h = x @ w.T
    if logit_bias is not None:
        h = h + np.asarray(logit_bias, dtype=np.float64)[None, :]
    return h


def softmax(h):
    """Softmax over experts with the maximum subtracted ([LAB] ``F.softmax``)."""
    m = h.max(axis=-1, keepdims=True)
    e = np.exp(h - m)
    return e / e.sum(axis=-1, keepdims=True)


def sigmoid(h):
    """Logistic score 1/(1+exp(-h)) ([NEMO] ``score_func`` 'sigmoid')."""
    return 1.0 / (1.0 + np.exp(-h))


def softplus(h):
    """log(1 + e^h), evaluated without overflow."""
    h = np.asarray(h, dtype=np.float64)
    return np.maximum(h, 0.0) + np.log1p(np.exp(-np.abs(h)))


def logsumexp(h):
    m = h.max(axis=-1)
    return m + np.log(np.exp(h - m[:, None]).sum(axis=-1))


def _order_desc(v):
    """Indices sorting each row of ``v`` by descending value, equal values
    in ascending index order (a stable sort of the negated values)."""
    return np.argsort(-v, axis=-1, kind="stable")


def _group_limit(sel, n_groups, topk_groups, group_rule):
    """Mask experts outside each token's ``topk_groups`` best groups.

    Experts form ``n_groups`` contiguous groups of E/n_groups ([NEMO]
    ``n_groups``/``topk_groups``; [LAB] "Lab extensions": no token may touch
    more groups than allowed).  Returns (masked selection scores, group scores,
    kept-group indices)."""
    T, E = sel.shape
    gs = E // n_groups
    grouped = sel.reshape(T, n_groups, gs)
    if group_rule == "top2sum":
        srt = -np.sort(-grouped, axis=-1)
        gscore = srt[..., 0] + srt[..., 1]
    elif group_rule == "max":
        gscore = grouped.max(axis=-1)
    else:
        raise ValueError(f"unknown group rule {group_rule!r}")
    keep_groups = _order_desc(gscore)[:, :topk_groups]
    allowed = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(allowed, keep_groups, True, axis=1)
    allowed_e = np.repeat(allowed, gs, axis=1)
    masked = np.where(allowed_e, sel, -np.inf)
    return masked, gscore, keep_groups


def _min_adjacent_gap(sorted_desc, n):
    """Smallest gap between neighbours among the first ``n`` sorted values
    (inf where there are fewer than two finite values)."""
    v = sorted_desc[:, :n]
    if v.shape[1] < 2:
        return np.full(v.shape[0], np.inf)
    with np.errstate(invalid="ignore"):
        g = v[:, :-1] - v[:, 1:]
    g = np.where(np.isfinite(g), g, np.inf)
    return g.min(axis=1)


def route(x, w_router, top_k, *, score="softmax", renormalize=True, route_scale=1.0,
          logit_bias=None, select_bias=None, n_groups=1, topk_groups=1,
          group_rule="top2sum", token_mask=None):
    """Routing step of the layer, in the pages' order.

    1. logits h = x W_r^T (+ logit bias)                  [LAB] "Full implementation"
    2. scores: softmax over all E ([LAB]) or sigmoid ([NEMO] ``score_func``)
    3. selection score = score (+ selection-only bias)   [BOOK] "The Router"
    4. optional group limit (contiguous groups)          [NEMO] ``n_groups``
    5. top-k IDs, descending                             [LAB] ``topk``
    6. weights: renormalised over the k selected scores  [LAB]; ``norm_topk_prob``
       or the raw top score (Switch top-1)               [LAB] "Ablation 2"
       times ``route_scale``                              [NEMO] ``route_scale``
    7. counts, f, P, balance = E sum f P, z = mean lse^2  [LAB]; [BOOK] aux loss
       over the unmasked tokens                           [NEMO] ``token_mask``

    Returns a dict with ``ids`` [T,k] int64 (-1 for masked tokens),
    ``weights`` [T,k], ``counts`` [E], ``mean_prob`` [E], ``balance``, ``z``,
    ``margin`` [T] and ``near_tie`` [T]."""
    h = router_logits(x, w_router, logit_bias)
    T, E = h.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, n_experts]")
    if score == "softmax":
        sc = softmax(h)
        prob_for_P = sc
    elif score == "sigmoid":
        sc = sigmoid(h)
        prob_for_P = sc / sc.sum(axis=-1, keepdims=True)
    elif score == "sqrtsoftplus":
        sc = np.sqrt(softplus(h))
        prob_for_P = sc / sc.sum(axis=-1, keepdims=True)
    else:
        raise ValueError(f"unknown score {score!r}")
    sel = sc.copy()
    if select_bias is not None:
        sel = sel + np.asarray(select_bias, dtype=np.float64)[None, :]
    group_margin = np.full(T, np.inf)
    if n_groups > 1:
        if E % n_groups or topk_groups < 1 or topk_groups > n_groups:
            raise ValueError("bad group configuration")
        if top_k > topk_groups * (E // n_groups):
            raise ValueError("top_k exceeds the experts of the allowed groups")
        sel, gscore, _ = _group_limit(sel, n_groups, topk_groups, group_rule)
        gsorted = -np.sort(-gscore, axis=1)
        group_margin = _min_adjacent_gap(gsorted, min(topk_groups + 1, n_groups))
    order = _order_desc(sel)
    ids = order[:, :top_k]
    chosen = np.take_along_axis(sc, ids, axis=1)
    if renormalize:
        weights = chosen / chosen.sum(axis=1, keepdims=True)
    else:
        weights = chosen.copy()
    weights = weights * route_scale
    sel_sorted = np.take_along_axis(sel, order[:, :min(top_k + 1, E)], axis=1)
    margin = np.minimum(_min_adjacent_gap(sel_sorted, min(top_k + 1, E)), group_margin)
    valid = np.ones(T, dtype=bool) if token_mask is None else np.asarray(token_mask, dtype=bool)
    ids = np.where(valid[:, None], ids, -1)
    weights = np.where(valid[:, None], weights, 0.0)
    margin = np.where(valid, margin, np.inf)
    n_valid = int(valid.sum())
    counts = np.bincount(ids[valid].reshape(-1), minlength=E)
    if n_valid:
        f = counts / float(n_valid * top_k)
        P = prob_for_P[valid].mean(axis=0)
        z = float(np.mean(logsumexp(h[valid]) ** 2))
    else:
        f, P, z = np.zeros(E), np.zeros(E), 0.0
    balance = E * float(np.sum(f * P))
    return {
        "logits": h, "scores": sc, "ids": ids.astype(np.int64), "weights": weights,
        "counts": counts.astype(np.int64), "mean_prob": P, "balance": balance,
        "z": z, "margin": margin, "near_tie": margin < NEAR_TIE,
    }


# -------------------------------------------------------------- capacity ---

def capacity(capacity_factor, T, top_k, E):
    """C = max(1, ceil(cf * T*k / E)); None (no limit) when dropless.

    [LAB] "Add a capacity limit" (ceil of factor * assignments / experts);
    [BOOK] "A Toy MoE Layer From Scratch" (at least 1).  Evaluated in that
    operand order in double precision."""
    if capacity_factor is None or capacity_factor <= 0:
        return None
    return max(1, math.ceil(capacity_factor * (T * top_k) / E))


def first_within_capacity(ids, E, cap):
    """Keep mask [T,k]: walk tokens in order, slots in order, and keep an
    assignment while its expert has taken fewer than ``cap`` assignments
    ([LAB] "Add a capacity limit", first-come policy).  ``cap=None`` keeps all."""
    ids = np.asarray(ids)
    T, k = ids.shape
    keep = np.zeros((T, k), dtype=bool)
    if cap is None:
        keep[:] = ids >= 0
        return keep
    used = [0] * E
    for t in range(T):
        for s in range(k):
            e = int(ids[t, s])
            if e < 0:  # masked token: not routed
                continue
            if used[e] < cap:
                keep[t, s] = True
                used[e] += 1
    return keep


def permutation(ids, keep, E):
    """Canonical expert-major order of the kept assignments.

    Kept assignments a = t*k + s are listed by (expert ascending, token
    ascending), the sorted expert-major token list a grouped GEMM consumes
    ([BOOK] "MoE in Practice", serving paragraph).  It is unique because a
    token picks an expert at most once.  Returns ``expert_offsets`` [E+1],
    ``row_to_assign`` [n_kept] and ``assign_to_row`` [T*k] (-1 = dropped)."""
    ids = np.asarray(ids)
    T, k = ids.shape
    flat_e = ids.reshape(-1)
    flat_keep = np.asarray(keep).reshape(-1)
    a = np.nonzero(flat_keep)[0]
    tok = a // k
    order = np.lexsort((tok, flat_e[a]))
    row_to_assign = a[order]
    kept_counts = np.bincount(flat_e[a], minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept_counts)
    assign_to_row = np.full(T * k, -1, dtype=np.int64)
    assign_to_row[row_to_assign] = np.arange(row_to_assign.size)
    return offsets, row_to_assign.astype(np.int64), assign_to_row


# --------------------------------------------------------------- experts ---

def swiglu_ffn(z, w_gate, w_up, w_down, limit=0.0):
    """FFN(z) = W_down (silu(W_gate z) * (W_up z)), silu(u) = u sigmoid(u).

    [LAB] ``SwiGLUExpert`` (three bias-free Linears); weights in Linear layout:
    w_gate, w_up [H, D]; w_down [D, H].  ``z`` is [n, D].  ``limit`` > 0
    clamps both projections to [-limit, limit] first ([NEMO] ``swiglu_limit``)."""
    z = np.asarray(z, dtype=np.float64)
    g = z @ np.asarray(w_gate, dtype=np.float64).T
    u = z @ np.asarray(w_up, dtype=np.float64).T
    if limit > 0:
        g = np.clip(g, -limit, limit)
        u = np.clip(u, -limit, limit)
    act = g * sigmoid(g) * u
    return act @ np.asarray(w_down, dtype=np.float64).T


def expert_outputs(x, ids, weights, keep, w_gate, w_up, w_down, tokens=None, limit=0.0):
    """Weighted expert output per (token, slot): Y[t, s] = w_ts FFN_{e_ts}(x_t)
    for kept slots, 0 for dropped ones ([LAB] "Full implementation", the
    per-expert gather / run / scale step).  Only tokens in ``tokens`` (default:
    all) are evaluated; returns [len(tokens), k, D]."""
    ids = np.asarray(ids)
    T, k = ids.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    D = np.asarray(x).shape[1]
    Y = np.zeros((tokens.size, k, D))
    sub_ids = ids[tokens]
    sub_keep = np.asarray(keep)[tokens]
    for e in np.unique(sub_ids):
        r, s = np.nonzero((sub_ids == e) & sub_keep)
        if e < 0 or r.size == 0:
            continue
        out = swiglu_ffn(np.asarray(x, dtype=np.float64)[tokens[r]], w_gate[e], w_up[e],
                         w_down[e], limit)
        Y[r, s] = np.asarray(weights)[tokens[r], s][:, None] * out
    return Y


def combine(Y, shared=None, residual=None):
    """out_t = sum over slots (in slot order) of the weighted expert outputs,
    plus the always-on shared expert ([LAB] ``index_add_`` combine and
    "Add a shared expert"), plus the residual stream when given (the block's
    skip connection around the layer, [BOOK] "From One FFN to a Bank of
    Experts": the MoE layer replaces the FFN of a transformer block)."""
    out = np.zeros(Y.shape[::2])
    for s in range(Y.shape[1]):
        out = out + Y[:, s]
    if shared is not None:
        out = out + shared
    if residual is not None:
        out = out + np.asarray(residual, dtype=np.float64)
    return out


def shared_expert(x, inputs, limit=0.0):
    """Always-on shared expert ([LAB] "Add a shared expert"; [BOOK]
    DeepSeek-MoE), scaled per token by sigmoid(x . w_sg) when ``ws_sgate``
    [D] is given ([NEMO] ``shared_expert_gate``); None without one."""
    if inputs.get("ws_gate") is None:
        return None
    x = np.asarray(x, dtype=np.float64)
    s = swiglu_ffn(x, inputs["ws_gate"], inputs["ws_up"], inputs["ws_down"], limit)
    if inputs.get("ws_sgate") is not None:
        s = sigmoid(x @ np.asarray(inputs["ws_sgate"], dtype=np.float64))[:, None] * s
    return s


def forward(inputs, *, top_k, score="softmax", renormalize=True, route_scale=1.0,
            n_groups=1, topk_groups=1, group_rule="top2sum", capacity_factor=None,
            tokens=None, routing=None, token_mask=None, swiglu_limit=0.0, residual=None,
            pre_norm=None):
    """The whole layer forward on float64 arrays.

    ``inputs`` holds x [T,D], w_router [E,D], w_gate/w_up [E,H,D], w_down
    [E,D,H], optional ws_gate/ws_up [Hs,D], ws_down [D,Hs], ws_sgate [D],
    logit_bias [E], select_bias [E].  ``token_mask`` [T] (True = valid) and
    ``swiglu_limit`` are the [NEMO] switches read in the module docstring.
    ``pre_norm`` = (weight or None, eps, act) runs ``rms_norm`` on x first;
    router, experts and shared expert then all take the normalised rows, and
    the residual (if any) is added as given.  ``tokens`` limits the expert/combine work to a subset of
    tokens (routing and capacity are always computed for all tokens, because
    drops depend on every earlier token).  ``routing`` may supply precomputed
    ``ids``/``weights`` (e.g. those of the device, to compare the downstream
    steps on identical routes)."""
    x = inputs["x"]
    if pre_norm is not None:
        x = rms_norm(x, pre_norm[0], pre_norm[1], pre_norm[2])
    T, D = x.shape
    E = inputs["w_router"].shape[0]
    r = route(x, inputs["w_router"], top_k, score=score, renormalize=renormalize,
              route_scale=route_scale, logit_bias=inputs.get("logit_bias"),
              select_bias=inputs.get("select_bias"), n_groups=n_groups,
              topk_groups=topk_groups, group_rule=group_rule, token_mask=token_mask)
    if routing is not None:
        r = dict(r)
        r["ids"] = np.asarray(routing["ids"], dtype=np.int64)
        r["weights"] = np.asarray(routing["weights"], dtype=np.float64)
        r["counts"] = np.bincount(r["ids"][r["ids"] >= 0].reshape(-1), minlength=E)
    cap = capacity(capacity_factor, T, top_k, E)
    keep = first_within_capacity(r["ids"], E, cap)
    offsets, row_to_assign, assign_to_row = permutation(r["ids"], keep, E)
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    Y = expert_outputs(x, r["ids"], r["weights"], keep, inputs["w_gate"],
                       inputs["w_up"], inputs["w_down"], tokens=tok, limit=swiglu_limit)
    shared = shared_expert(np.asarray(x, dtype=np.float64)[tok], inputs, swiglu_limit)
    out = combine(Y, shared, None if residual is None else np.asarray(residual)[tok])
    return {
        "out": out, "tokens": tok, "route": r, "capacity": cap, "keep": keep,
        "expert_offsets": offsets, "row_to_assign": row_to_assign,
        "assign_to_row": assign_to_row, "n_kept": int(keep.sum()), "x_in": x,
    }


# -------------------------------------------------------------- pre-norm ---

def round_to_bf16(v):
    """Nearest bfloat16 value of each float64 in ``v`` (ties to even), as
    float64.  bfloat16 is the upper 16 bits of an IEEE single: 8 significant
    bits and the single's exponent range.  The rounding is taken once, on the
    float64 bit pattern (52 fraction bits, of which the lowest 45 go), so no
    intermediate float32 rounding can shift a tie.  Finite, normal inputs."""
    v = np.asarray(v, dtype=np.float64)
    bits = v.view(np.uint64).copy()
    drop = np.uint64(45)
    keep_lsb = (bits >> drop) & np.uint64(1)
    bits = bits + (np.uint64((1 << 44) - 1) + keep_lsb)
    bits = bits & ~np.uint64((1 << 45) - 1)
    return bits.view(np.float64)


def rms_norm(x, weight=None, eps=1e-6, act="bf16"):
    """RMSNorm of every token row: y = x * w / sqrt(mean_d x_d^2 + eps)
    ([LAB] "Put the MoE into a decoder block"; [ST] "rms-norm"), w = 1 when
    ``weight`` is None.  float64, then one rounding to the activation dtype
    ``act`` ('bf16', 'f32', or None for no rounding)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)[None, :]
    if act == "bf16":
        return round_to_bf16(y)
    if act == "f32":
        return y.astype(np.float32).astype(np.float64)
    return y


def rms_norm_backward(x, weight, eps, dy):
    """Gradients of sum(dy * rms_norm(x, weight, eps, act=None)): returns
    (dx, dweight).  With s_t = sqrt(mean_d x_td^2 + eps):
    dx_td = w_d dy_td / s_t - x_td sum_j(dy_tj w_j x_tj) / (D s_t^3) and
    dweight_d = sum_t dy_td x_td / s_t (w = 1 when ``weight`` is None)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    D = x.shape[1]
    w = np.ones(D) if weight is None else np.asarray(weight, dtype=np.float64)
    s = np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    g = dy * w[None, :]
    dx = g / s - x * np.sum(g * x, axis=1, keepdims=True) / (D * s ** 3)
    return dx, np.sum(dy * x / s, axis=0)


# ------------------------------------------------ bias-adjustment balancer ---

def update_bias(bias, counts, gamma):
    """One step of the auxiliary-loss-free balancer ([BOOK] "DeepSeek-MoE and
    the fine-grained + shared-expert idea" and "Exercises" 6; [NEMO]
    ``Gate.update_bias``): every expert above the mean load has its selection
    bias lowered by ``gamma``, every expert below it raised, an expert exactly
    at the mean left alone.  The comparison count_e <> mean(counts) is taken
    exactly, as E * count_e <> sum(counts) on integers."""
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.size
    total = int(counts.sum())
    step = np.sign(total - E * counts).astype(np.float64)
    return np.asarray(bias, dtype=np.float64) + gamma * step


# -------------------------------------------------------------- backward ---
#
# The training objective of [LAB] "Smoke test and backward pass": a task loss
# plus alpha * balance + beta * z.  Here the task term is <dout, out> (dout is
# the gradient the rest of the network sends back).  As in [BOOK] "The
# Router" (top-k is a stop-gradient on the index decision) and "The auxiliary
# load-balancing loss" (f is detached), the selected IDs, the capacity drops
# and the counts f are constants; gradients reach the router through the gate
# weights of the kept slots, through P_e and through z.

def loss(inputs, dout, aux_coef=(0.0, 0.0), **fw):
    """L = <dout, out> + alpha * balance + beta * z for the forward ``fw``."""
    f = forward(inputs, **fw)
    a, b = aux_coef
    return (float(np.sum(np.asarray(dout, dtype=np.float64) * f["out"]))
            + a * f["route"]["balance"] + b * f["route"]["z"]), f


def _dsilu(v):
    s = sigmoid(v)
    return s + v * s * (1.0 - s)


def swiglu_ffn_backward(z, w_gate, w_up, w_down, dF, limit=0.0):
    """Gradients of sum(dF * FFN(z)) for FFN of ``swiglu_ffn``: returns
    (dz [n,D], dW_gate [H,D], dW_up [H,D], dW_down [D,H], F [n,D]).  The clamp
    passes gradient where |g| < limit (resp. |u|) and none outside."""
    z = np.asarray(z, dtype=np.float64)
    wg, wu, wd = (np.asarray(w, dtype=np.float64) for w in (w_gate, w_up, w_down))
    g, u = z @ wg.T, z @ wu.T
    gc, uc = (np.clip(g, -limit, limit), np.clip(u, -limit, limit)) if limit > 0 else (g, u)
    act = gc * sigmoid(gc) * uc
    F = act @ wd.T
    da = dF @ wd
    dWd = dF.T @ act
    dgc = da * uc * _dsilu(gc)
    duc = da * gc * sigmoid(gc)
    if limit > 0:
        dgc = dgc * (np.abs(g) < limit)
        duc = duc * (np.abs(u) < limit)
    dz = dgc @ wg + duc @ wu
    return dz, dgc.T @ z, duc.T @ z, dWd, F


def router_backward(r, d_gate_w, *, top_k, score="softmax", renormalize=True,
                    route_scale=1.0, aux_coef=(0.0, 0.0), tokens=None):
    """dL/dh [T,E] (or the rows of ``tokens``) of ``loss`` for the routing
    ``r`` of ``route`` and dL/dw per slot ``d_gate_w`` (zero for dropped
    slots): through the kept gate weights (renormalised or raw, times
    route_scale), P_e of the balance term (f held constant) and z."""
    # router: gate weights -> chosen scores
    ids = r["ids"]
    T, k = ids.shape
    E = r["logits"].shape[1]
    sc, h = r["scores"], r["logits"]
    valid = ids[:, 0] >= 0
    dsc = np.zeros((T, E))
    rows = np.nonzero(valid)[0] if tokens is None else [t for t in tokens if valid[t]]
    for t in rows:  # (d_gate_w is read on these rows only)
        c = sc[t, ids[t]]
        if renormalize:
            S = c.sum()
            dc = route_scale / S * (d_gate_w[t] - np.sum(d_gate_w[t] * c) / S)
        else:
            dc = route_scale * d_gate_w[t]
        np.add.at(dsc[t], ids[t], dc)
    # balance = E * sum_e f_e P_e, P_e = mean over valid tokens of q_te
    alpha, beta = aux_coef
    n_valid = int(valid.sum())
    if n_valid and alpha:
        f_e = r["counts"] / float(n_valid * top_k)
        dq = np.where(valid[:, None], alpha * E * f_e[None, :] / n_valid, 0.0)
        if score == "softmax":
            dsc += dq
        else:  # q = s / sum_e s
            ssum = sc.sum(axis=1, keepdims=True)
            q = sc / ssum
            dsc += (dq - np.sum(dq * q, axis=1, keepdims=True)) / ssum
    # scores -> logits
    if score == "softmax":
        dh = sc * (dsc - np.sum(dsc * sc, axis=1, keepdims=True))
    elif score == "sigmoid":
        dh = dsc * sc * (1.0 - sc)
    else:  # s = sqrt(softplus(h)): ds/dh = sigmoid(h) / (2 s)
        dh = dsc * sigmoid(h) / (2.0 * sc)
    # z = mean over valid tokens of lse(h_t)^2
    if n_valid and beta:
        lse = logsumexp(h)
        dh += np.where(valid[:, None], beta * 2.0 * lse[:, None] * softmax(h) / n_valid, 0.0)
    dh = np.where(valid[:, None], dh, 0.0)
    return dh if tokens is None else dh[np.asarray(tokens)]


def backward(inputs, dout, *, top_k, score="softmax", renormalize=True, route_scale=1.0,
             n_groups=1, topk_groups=1, group_rule="top2sum", capacity_factor=None,
             token_mask=None, swiglu_limit=0.0, aux_coef=(0.0, 0.0), pre_norm=None):
    """Gradients of ``loss`` with respect to x, W_r and every expert weight
    (float64).  With ``pre_norm`` = (weight, eps, act) the layer takes
    rms_norm(x) (rounded to ``act``; the rounding passes gradients through
    unchanged) and the result also holds d_norm_weight.  Returns dx, dw_router, dw_gate, dw_up, dw_down (+ dws_gate,
    dws_up, dws_down with a shared expert, + d_shared_gate with its gate), and
    the intermediates d_gate_w [T,k] (dL/dw per slot) and d_logits [T,E].

    The gated shared expert adds g_t S(x_t) with g_t = sigmoid(x_t . w_sg):
    S sees g_t dout_t, and the gate's logit gets g_t (1 - g_t) <dout_t, S(x_t)>,
    which reaches w_sg (times x_t) and x_t (times w_sg)."""
    fw = dict(top_k=top_k, score=score, renormalize=renormalize, route_scale=route_scale,
              n_groups=n_groups, topk_groups=topk_groups, group_rule=group_rule,
              capacity_factor=capacity_factor, token_mask=token_mask,
              swiglu_limit=swiglu_limit)
    if pre_norm is not None:
        x_raw = np.asarray(inputs["x"], dtype=np.float64)
        inner = backward(dict(inputs, x=rms_norm(x_raw, *pre_norm)), dout, aux_coef=aux_coef,
                         **fw)
        inner["dx"], inner["d_norm_weight"] = rms_norm_backward(
            x_raw, pre_norm[0], pre_norm[1], inner["dx"])
        return inner
    f = forward(inputs, **fw)
    r = f["route"]
    x = np.asarray(inputs["x"], dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    T, D = x.shape
    E = inputs["w_router"].shape[0]
    ids, keep, wts = r["ids"], f["keep"], r["weights"]
    k = ids.shape[1]
    dx = np.zeros((T, D))
    grads = {n: np.zeros(np.shape(inputs[n])) for n in ("w_gate", "w_up", "w_down")}
    d_gate_w = np.zeros((T, k))
    # experts: each kept slot sends w_ts * dout_t into FFN_e; dL/dw_ts = <dout_t, FFN_e(x_t)>
    for e in range(E):
        t, s = np.nonzero((ids == e) & keep)
        if t.size == 0:
            continue
        dF = wts[t, s][:, None] * dout[t]
        dz, dwg, dwu, dwd, F = swiglu_ffn_backward(x[t], inputs["w_gate"][e], inputs["w_up"][e],
                                                   inputs["w_down"][e], dF, swiglu_limit)
        np.add.at(dx, t, dz)
        grads["w_gate"][e] += dwg
        grads["w_up"][e] += dwu
        grads["w_down"][e] += dwd
        d_gate_w[t, s] = np.sum(dout[t] * F, axis=1)
    out = {"dw_gate": grads["w_gate"], "dw_up": grads["w_up"], "dw_down": grads["w_down"]}
    if inputs.get("ws_gate") is not None:
        wsg = inputs.get("ws_sgate")
        g = np.ones(T) if wsg is None else sigmoid(x @ np.asarray(wsg, dtype=np.float64))
        dz, dwg, dwu, dwd, S = swiglu_ffn_backward(x, inputs["ws_gate"], inputs["ws_up"],
                                                   inputs["ws_down"], g[:, None] * dout,
                                                   swiglu_limit)
        dx += dz
        out.update(dws_gate=dwg, dws_up=dwu, dws_down=dwd)
        if wsg is not None:
            dlogit = g * (1.0 - g) * np.sum(dout * S, axis=1)
            dx += dlogit[:, None] * np.asarray(wsg, dtype=np.float64)[None, :]
            out["d_shared_gate"] = dlogit @ x
    dh = router_backward(r, d_gate_w, top_k=top_k, score=score, renormalize=renormalize,
                         route_scale=route_scale, aux_coef=aux_coef)
    wr = np.asarray(inputs["w_router"], dtype=np.float64)
    dx += dh @ wr
    out.update(dx=dx, dw_router=dh.T @ x, d_gate_w=d_gate_w, d_logits=dh)
    return out


# ------------------------------------------- second implementations (tiny) ---

def brute_force_forward(inputs, ids, weights, keep=None, limit=0.0):
    """Token-by-token, slot-by-slot loop in pure Python ([LAB] "Trace one token
    by hand"): out_t = sum_s w_ts FFN_{e_ts}(x_t) (+ shared, times its gate).
    For tiny shapes; IDs < 0 (masked tokens) are skipped."""
    x = np.asarray(inputs["x"], dtype=np.float64)
    T, D = x.shape
    k = ids.shape[1]
    out = np.zeros((T, D))
    for t in range(T):
        for s in range(k):
            if keep is not None and not keep[t, s]:
                continue
            e = int(ids[t, s])
            if e < 0:
                continue
            out[t] += weights[t, s] * swiglu_ffn(x[t:t + 1], inputs["w_gate"][e],
                                                 inputs["w_up"][e], inputs["w_down"][e],
                                                 limit)[0]
        if inputs.get("ws_gate") is not None:
            sh = swiglu_ffn(x[t:t + 1], inputs["ws_gate"], inputs["ws_up"],
                            inputs["ws_down"], limit)[0]
            if inputs.get("ws_sgate") is not None:
                dot = sum(float(a) * float(b) for a, b in zip(x[t], inputs["ws_sgate"]))
                sh = sh / (1.0 + math.exp(-dot))
            out[t] += sh
    return out


def all_experts_then_mask(inputs, ids, weights):
    """Run every expert on every token and keep only the selected ones
    ([BOOK] "A Toy MoE Layer From Scratch", second approach; unit tests only)."""
    x = np.asarray(inputs["x"], dtype=np.float64)
    T, D = x.shape
    E = inputs["w_gate"].shape[0]
    dense = np.stack([swiglu_ffn(x, inputs["w_gate"][e], inputs["w_up"][e],
                                 inputs["w_down"][e]) for e in range(E)], axis=1)
    gate = np.zeros((T, E))
    ids = np.asarray(ids)
    for t in range(T):
        for s in range(ids.shape[1]):
            if ids[t, s] >= 0:
                gate[t, ids[t, s]] += weights[t, s]
    return np.einsum("te,ted->td", gate, dense)
