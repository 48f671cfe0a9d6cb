"""moe_forward_noalloc (the forward on the library's static scratch) against
moe_forward (the same forward on a caller workspace), through the C ABI.

Two calls in a row on one GPU share the static scratch, the second with a
smaller input, and each must agree with moe_forward on the same inputs:
routing results bit for bit, outputs within the layer's tolerance."""
from __future__ import annotations

import sys

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


def _both(moe, w, d, T):
    """moe_forward and moe_forward_noalloc on the first T tokens of d."""
    w = w.with_(batch=1, seq=T)
    cfg = P.config_of(w)
    x = d["x"][:T].contiguous()
    kw = dict(logit_bias=d.get("logit_bias"), select_bias=d.get("select_bias"),
              ws_gate=d.get("ws_gate"), ws_up=d.get("ws_up"), ws_down=d.get("ws_down"))
    res = []
    for fn in (moe.moe_forward, moe.moe_forward_noalloc):
        out = torch.empty(T, w.D, dtype=x.dtype, device="cuda")
        ids = torch.empty(T, w.top_k, dtype=torch.int32, device="cuda")
        gw = torch.empty(T, w.top_k, dtype=torch.float32, device="cuda")
        counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
        aux = torch.empty(2, dtype=torch.float32, device="cuda")
        fn(cfg, x, d["w_router"], d["w_gate"], d["w_up"], d["w_down"], out=out,
           expert_ids=ids, gate_w=gw, counts=counts, aux=aux, **kw)
        res.append((out, ids, gw, counts, aux))
    torch.cuda.synchronize()
    return w, res


def _agree(w, res, what):
    (o0, i0, g0, c0, a0), (o1, i1, g1, c1, a1) = res
    assert torch.equal(i0, i1), f"{what}: expert IDs differ"
    assert torch.equal(g0, g1), f"{what}: gate weights differ"
    assert torch.equal(c0, c1), f"{what}: counts differ"
    assert torch.equal(a0, a1), f"{what}: aux losses differ"
    err, scale = P.compare_rows(o1, o0.double().cpu().numpy(), w.act_dtype, what)
    _say(f"  {what}: max|err| {err:.3g} max|ref| {scale:.3g} "
         f"(bit-identical: {torch.equal(o0, o1)})")


# (workload, first T, second T): the decode-shaped layer at its full size and
# reduced shapes that take the 32-row, 128-row and 256-row GEMM tiles, the
# shared expert and a capacity limit.
CASES = [("decode_128x_top8", 64, 23), ("decode_small", 37, 5), ("switch_band", 1600, 901),
         ("mixtral_small", 778, 300), ("deepseek_small", 517, 130), ("tiny", 256, 77)]


@pytest.mark.parametrize("name,t1,t2", CASES)
def test_noalloc_matches_forward_twice(moe, name, t1, t2):
    w = W.WORKLOADS.get(name) or W.SMALL[name]
    _say(f"[noalloc] {name}: T={t1}, then T={t2}")
    dev = "cuda" if w.T * w.D > (1 << 22) else "cpu"
    d = {k: v.to("cuda") for k, v in W.make_inputs(w, dev, seed=31).items()}
    wa, ra = _both(moe, w, d, t1)
    _agree(wa, ra, f"{name} T={t1}")
    wb, rb = _both(moe, w, d, t2)
    _agree(wb, rb, f"{name} T={t2}")


def test_noalloc_rejects_a_layer_beyond_its_scratch(moe):
    w = W.SMALL["mixtral_small"].with_(batch=1, seq=16384)  # Hb and Y rows exceed 64 MiB
    cfg = P.config_of(w)
    d = {k: v.to("cuda") for k, v in W.make_inputs(w, "cpu", seed=32).items()}
    out = torch.empty(w.T, w.D, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError, match="UNSUPPORTED.*scratch"):
        moe.moe_forward_noalloc(cfg, d["x"], d["w_router"], d["w_gate"], d["w_up"],
                                d["w_down"], out=out)


@pytest.mark.parametrize("i", range(0, 60, 3))
def test_noalloc_random_configs(moe, i):
    """Every third seeded random configuration (bf16 and fp32 layers of 1 to
    256 experts), one after another on the same static scratch."""
    from tests.test_gpu_random_configs import CONFIGS
    w = CONFIGS[i]
    _say(f"[noalloc-random] {w.name}: T={w.T} D={w.D} H={w.H} E={w.E} k={w.top_k}")
    d = {k: v.to("cuda") for k, v in W.make_inputs(w, "cpu", seed=600 + i).items()}
    wa, ra = _both(moe, w, d, w.T)
    _agree(wa, ra, f"{w.name} T={w.T}")
