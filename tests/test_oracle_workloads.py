"""The oracle on the seeded workloads (CPU): invariants that hold at any size."""
import numpy as np
import pytest

import oracle
import workloads as W


def _f64(inp):
    return {k: W.to_f64(v) for k, v in inp.items()}


def _run(w, inp, **kw):
    return oracle.forward(inp, top_k=w.top_k, score=w.score, renormalize=w.renormalize,
                          route_scale=w.route_scale, n_groups=w.n_groups,
                          topk_groups=w.topk_groups, group_rule=w.group_rule,
                          capacity_factor=w.capacity_factor, **kw)


@pytest.mark.parametrize("name", sorted(W.SMALL))
def test_small_workload_invariants(name):
    w = W.SMALL[name]
    inp = _f64(W.make_inputs(w, "cpu", seed=0))
    f = _run(w, inp)
    r = f["route"]
    T, k, E = w.T, w.top_k, w.E
    assert f["out"].shape == (T, w.D)
    assert int(r["counts"].sum()) == T * k
    ws = r["weights"].sum(1)
    if w.renormalize:
        assert np.allclose(ws, w.route_scale, atol=1e-12)
    else:
        assert (ws <= 1.0 + 1e-15).all()
    if w.n_groups > 1:
        gs = E // w.n_groups
        assert max(len(set((r["ids"][t] // gs).tolist())) for t in range(T)) <= w.topk_groups
    if w.capacity_factor is not None:
        assert f["n_kept"] == int(np.minimum(r["counts"], f["capacity"]).sum())
    else:
        assert f["n_kept"] == T * k
    # a few tokens by the slow per-token loop
    toks = [0, T // 2, T - 1]
    bf = oracle.brute_force_forward(inp, r["ids"], r["weights"], f["keep"])
    assert np.allclose(f["out"][toks], bf[toks], rtol=0, atol=1e-12)


def test_tiny_workload_shapes_and_dtypes():
    inp = W.make_inputs(W.TINY, "cpu", seed=0)
    assert inp["x"].shape == (256, 64) and str(inp["x"].dtype) == "torch.float32"
    assert inp["w_gate"].shape == (4, 128, 64) and inp["w_down"].shape == (4, 64, 128)
    inp2 = W.make_inputs(W.TINY, "cpu", seed=0)
    assert all((inp[k] == inp2[k]).all() for k in inp)


def test_switch_reading_skews_load():
    """The Zipf logit bias concentrates load on low-index experts, so a
    capacity factor of 1.25 drops assignments."""
    w = W.SMALL["switch_small"]
    inp = _f64(W.make_inputs(w, "cpu", seed=0))
    f = _run(w, inp)
    c = f["route"]["counts"]
    assert c[0] == c.max() and f["n_kept"] < w.T
