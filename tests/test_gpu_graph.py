"""The forward under HIP graph capture: moe_forward (caller's workspace) and
moe_forward_noalloc (static scratch) record only kernel launches, so a
captured forward replays.  Each graph is replayed several times with other
eager work of the program and synchronisations between the replays; every
replay must reproduce the eager forward bit for bit (the kernels are
deterministic: fixed reduction orders, no float atomics)."""
from __future__ import annotations

import sys

import pytest
import torch

import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu

# 32-row GEMM tiles (decode_small, switch_small, deepseek_small), the 128-row
# band with its split-K tail (switch_band, mixtral_band), the 256-row tiles
# (mixtral_small) and the fp32 path (tiny).
NAMES = ["decode_small", "switch_small", "deepseek_small", "tiny", "switch_band",
         "mixtral_band", "mixtral_small"]


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_layer_21_amd as m
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return m


def _outputs(w, dev):
    dt = W.torch_dtype(w.act_dtype)
    return {"out": torch.empty(w.T, w.D, dtype=dt, device=dev),
            "expert_ids": torch.empty(w.T, w.top_k, dtype=torch.int32, device=dev),
            "gate_w": torch.empty(w.T, w.top_k, dtype=torch.float32, device=dev),
            "counts": torch.empty(w.E, dtype=torch.int32, device=dev),
            "aux": torch.empty(2, dtype=torch.float32, device=dev)}


@pytest.mark.parametrize("noalloc", [False, True], ids=["moe_forward", "moe_forward_noalloc"])
@pytest.mark.parametrize("name", NAMES)
def test_captured_forward_replays_bit_exact(moe, name, noalloc):
    w = W.SMALL[name]
    print(f"[graph] {name} noalloc={noalloc} T={w.T}", file=sys.stderr, flush=True)
    dev = torch.device("cuda")
    d = {k: v.to(dev) for k, v in W.make_inputs(w, "cpu", seed=7).items()}
    other = {k: v.to(dev) for k, v in W.make_inputs(w, "cpu", seed=8).items()}
    cfg = P.config_of(w)
    ws = None if noalloc else moe.new_workspace(cfg, dev)

    def fwd(inp, o):
        kw = dict(logit_bias=inp.get("logit_bias"), select_bias=inp.get("select_bias"),
                  ws_gate=inp.get("ws_gate"), ws_up=inp.get("ws_up"), ws_down=inp.get("ws_down"),
                  **o)
        if noalloc:
            moe.moe_forward_noalloc(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                                    inp["w_down"], **kw)
        else:
            moe.moe_forward(cfg, inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"],
                            inp["w_down"], workspace=ws, **kw)

    ref = _outputs(w, dev)
    fwd(d, ref)                      # eager reference (and first-call set-up)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items()}

    o = _outputs(w, dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(d, o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(d, o)
    torch.cuda.synchronize()

    o2 = _outputs(w, dev)
    for rep in range(3):
        for v in o.values():
            v.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(o[k], ref[k]), f"replay {rep}: {k} differs from the eager forward"
        # eager work of the program between replays: a forward on other inputs
        # (on the same workspace or static scratch), then a synchronisation
        fwd(other, o2)
        torch.cuda.synchronize()
