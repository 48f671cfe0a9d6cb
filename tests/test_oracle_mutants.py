"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
every one of them breaks at least one pin.  This shows that the pins constrain
each step: a dropped term, a wrong sign or index, a swapped operand or a wrong
order would not go unnoticed."""
import importlib.util
import os

import pytest

from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "moe_oracle.py")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("tie_to_higher_index",
     'return np.argsort(-v, axis=-1, kind="stable")',
     'return (v.shape[-1] - 1) - np.argsort(-v[..., ::-1], axis=-1, kind="stable")'),
    ("no_renormalisation",
     "weights = chosen / chosen.sum(axis=1, keepdims=True)",
     "weights = chosen.copy()"),
    ("route_scale_ignored",
     "weights = weights * route_scale",
     "weights = weights * 1.0"),
    ("softmax_without_max_shift_sign",
     "e = np.exp(h - m)",
     "e = np.exp(m - h)"),
    ("selection_bias_in_weights",
     "chosen = np.take_along_axis(sc, ids, axis=1)",
     "chosen = np.take_along_axis(sel, ids, axis=1)"),
    ("group_rule_max_for_top2sum",
     "gscore = srt[..., 0] + srt[..., 1]",
     "gscore = srt[..., 0]"),
    ("group_ascending",
     "keep_groups = _order_desc(gscore)[:, :topk_groups]",
     "keep_groups = _order_desc(-gscore)[:, :topk_groups]"),
    ("balance_without_E",
     "balance = E * float(np.sum(f * P))",
     "balance = float(np.sum(f * P))"),
    ("z_without_square",
     "z = float(np.mean(logsumexp(h[valid]) ** 2))",
     "z = float(np.mean(logsumexp(h[valid])))"),
    ("lse_missing_max",
     "return m + np.log(np.exp(h - m[:, None]).sum(axis=-1))",
     "return np.log(np.exp(h - m[:, None]).sum(axis=-1))"),
    ("capacity_floor",
     "return max(1, math.ceil(capacity_factor * (T * top_k) / E))",
     "return max(1, math.floor(capacity_factor * (T * top_k) / E))"),
    ("capacity_off_by_one",
     "if used[e] < cap:",
     "if used[e] <= cap:"),
    ("slot_major_priority",
     "    for t in range(T):\n        for s in range(k):\n            e = int(ids[t, s])\n            if e < 0",
     "    for s in range(k):\n        for t in range(T):\n            e = int(ids[t, s])\n            if e < 0"),
    ("permutation_token_major",
     "order = np.lexsort((tok, flat_e[a]))",
     "order = np.lexsort((flat_e[a], tok))"),
    ("silu_missing_gate_factor",
     "act = g * sigmoid(g) * u",
     "act = sigmoid(g) * u"),
    ("gate_and_up_swapped_roles",
     "act = g * sigmoid(g) * u",
     "act = u * sigmoid(u) * g"),
    ("down_transposed",
     "return act @ np.asarray(w_down, dtype=np.float64).T",
     "return act @ np.asarray(w_down, dtype=np.float64).reshape(-1, np.asarray(w_down).shape[0])"),
    ("weight_not_applied",
     "Y[r, s] = np.asarray(weights)[tokens[r], s][:, None] * out",
     "Y[r, s] = out"),
    ("shared_expert_dropped",
     "    if shared is not None:\n        out = out + shared",
     "    if shared is not None:\n        out = out + 0.0 * shared"),
    ("sqrtsoftplus_without_sqrt",
     "sc = np.sqrt(softplus(h))",
     "sc = softplus(h)"),
    ("softplus_sign",
     "return np.maximum(h, 0.0) + np.log1p(np.exp(-np.abs(h)))",
     "return np.maximum(h, 0.0) + np.log1p(np.exp(np.abs(h)))"),
    ("mask_still_counted",
     "counts = np.bincount(ids[valid].reshape(-1), minlength=E)",
     "counts = np.bincount(np.where(ids < 0, 0, ids).reshape(-1), minlength=E)"),
    ("mask_mean_over_all_tokens",
     "P = prob_for_P[valid].mean(axis=0)",
     "P = prob_for_P[valid].sum(axis=0) / T"),
    ("mask_takes_capacity",
     "            if e < 0:  # masked token: not routed\n                continue\n",
     "            if e < 0:  # masked token: not routed\n                used[0] += 1\n                continue\n"),
    ("clamp_gate_only",
     "        u = np.clip(u, -limit, limit)",
     "        u = u"),
    ("clamp_one_sided",
     "        g = np.clip(g, -limit, limit)",
     "        g = np.minimum(g, limit)"),
    ("shared_gate_not_applied",
     "        s = sigmoid(x @ np.asarray(inputs[\"ws_sgate\"], dtype=np.float64))[:, None] * s",
     "        s = s"),
    ("bias_update_sign_flipped",
     "step = np.sign(total - E * counts).astype(np.float64)",
     "step = np.sign(E * counts - total).astype(np.float64)"),
    ("bias_update_against_max",
     "step = np.sign(total - E * counts).astype(np.float64)",
     "step = np.sign(counts.max() - counts).astype(np.float64)"),
    ("residual_dropped",
     "        out = out + np.asarray(residual, dtype=np.float64)",
     "        out = out + 0.0"),
    ("rms_eps_dropped",
     "y = x / np.sqrt(ms + eps)",
     "y = x / np.sqrt(ms)"),
    ("rms_sum_not_mean",
     "ms = np.mean(x * x, axis=1, keepdims=True)",
     "ms = np.sum(x * x, axis=1, keepdims=True)"),
    ("rms_over_tokens",
     "ms = np.mean(x * x, axis=1, keepdims=True)",
     "ms = np.mean(x * x, axis=0, keepdims=True)"),
    ("rms_weight_not_applied",
     "y = y * np.asarray(weight, dtype=np.float64)[None, :]",
     "y = y * 1.0"),
    ("bf16_ties_away",
     "bits = bits + (np.uint64((1 << 44) - 1) + keep_lsb)",
     "bits = bits + np.uint64(1 << 44)"),
    ("bf16_truncates",
     "bits = bits + (np.uint64((1 << 44) - 1) + keep_lsb)",
     "bits = bits + np.uint64(0)"),
    ("bf16_keeps_a_bit_too_many",
     "drop = np.uint64(45)",
     "drop = np.uint64(44)"),
    ("pre_norm_ignored",
     "        x = rms_norm(x, pre_norm[0], pre_norm[1], pre_norm[2])",
     "        x = x"),
    ("bwd_dsilu_missing_term",
     "return s + v * s * (1.0 - s)",
     "return s"),
    ("bwd_up_grad_without_gate",
     "duc = da * gc * sigmoid(gc)",
     "duc = da * sigmoid(gc)"),
    ("bwd_gate_weight_not_in_dF",
     "dF = wts[t, s][:, None] * dout[t]",
     "dF = dout[t]"),
    ("bwd_renorm_jacobian_no_subtract",
     "dc = route_scale / S * (d_gate_w[t] - np.sum(d_gate_w[t] * c) / S)",
     "dc = route_scale / S * d_gate_w[t]"),
    ("bwd_route_scale_dropped",
     "dc = route_scale * d_gate_w[t]",
     "dc = d_gate_w[t]"),
    ("bwd_balance_without_f",
     "dq = np.where(valid[:, None], alpha * E * f_e[None, :] / n_valid, 0.0)",
     "dq = np.where(valid[:, None], alpha * E / E + 0 * f_e[None, :] / n_valid, 0.0)"),
    ("bwd_normalised_q_jacobian",
     "dsc += (dq - np.sum(dq * q, axis=1, keepdims=True)) / ssum",
     "dsc += dq / ssum"),
    ("bwd_softmax_jacobian_sign",
     "dh = sc * (dsc - np.sum(dsc * sc, axis=1, keepdims=True))",
     "dh = sc * (dsc + np.sum(dsc * sc, axis=1, keepdims=True))"),
    ("bwd_sigmoid_derivative",
     "dh = dsc * sc * (1.0 - sc)",
     "dh = dsc * sc"),
    ("bwd_sqrtsoftplus_half",
     "dh = dsc * sigmoid(h) / (2.0 * sc)",
     "dh = dsc * sigmoid(h) / sc"),
    ("bwd_z_without_2",
     "beta * 2.0 * lse[:, None]",
     "beta * lse[:, None]"),
    ("bwd_router_dx_missing",
     "dx += dh @ wr",
     "dx += 0.0 * (dh @ wr)"),
    ("bwd_clamp_passes_gradient",
     "dgc = dgc * (np.abs(g) < limit)",
     "dgc = dgc * 1.0"),
    ("bwd_shared_expert_dx_missing",
     "        dx += dz\n        out.update(dws_gate=dwg",
     "        dx += 0 * dz\n        out.update(dws_gate=dwg"),
    ("rms_bwd_projection_dropped",
     "dx = g / s - x * np.sum(g * x, axis=1, keepdims=True) / (D * s ** 3)",
     "dx = g / s"),
    ("rms_bwd_wrong_power",
     "dx = g / s - x * np.sum(g * x, axis=1, keepdims=True) / (D * s ** 3)",
     "dx = g / s - x * np.sum(g * x, axis=1, keepdims=True) / (D * s ** 2)"),
    ("rms_bwd_weight_grad_unnormalised",
     "return dx, np.sum(dy * x / s, axis=0)",
     "return dx, np.sum(dy * x, axis=0)"),
    ("shared_gate_bwd_no_sigmoid_slope",
     "dlogit = g * (1.0 - g) * np.sum(dout * S, axis=1)",
     "dlogit = np.sum(dout * S, axis=1)"),
    ("shared_gate_bwd_ungated_branch",
     "inputs[\"ws_down\"], g[:, None] * dout,",
     "inputs[\"ws_down\"], dout,"),
    ("shared_gate_bwd_no_dx_term",
     "dx += dlogit[:, None] * np.asarray(wsg, dtype=np.float64)[None, :]",
     "dx += 0.0"),
    ("group_margin_over_all_groups",
     "group_margin = _min_adjacent_gap(gsorted, min(topk_groups + 1, n_groups))",
     "group_margin = _min_adjacent_gap(gsorted, n_groups)"),
    ("group_margin_kept_groups_only",
     "group_margin = _min_adjacent_gap(gsorted, min(topk_groups + 1, n_groups))",
     "group_margin = _min_adjacent_gap(gsorted, topk_groups)"),
    ("group_margin_dropped",
     "margin = np.minimum(_min_adjacent_gap(sel_sorted, min(top_k + 1, E)), group_margin)",
     "margin = _min_adjacent_gap(sel_sorted, min(top_k + 1, E))"),
    ("router_bias_ignored",
     "h = h + np.asarray(logit_bias, dtype=np.float64)[None, :]",
     "h = h + 0.0"),
]


def _load_mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site not unique/present: {old!r}"
    spec = importlib.util.spec_from_loader("oracle_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _failing_pins(mod):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:  # AssertionError or a crash both count as caught
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _load_mutant(old, new)
    assert _failing_pins(mod), f"planted mistake {name!r} passed every pin"


def test_unmutated_copy_passes():
    with open(SRC) as f:
        src = f.read()
    spec = importlib.util.spec_from_loader("oracle_copy", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src, "oracle_copy", "exec"), mod.__dict__)
    assert _failing_pins(mod) == []
