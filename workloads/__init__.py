"""Seeded synthetic workloads for the MoE-layer forward.

This module only *describes* workloads (shapes, dtypes, routing switches) and
*draws* their inputs from a seeded generator.  It contains none of the layer's
arithmetic: no routing, capacity, permutation, expert FFN or combine.  Both the
GPU path (through the Python binding) and the CPU oracle consume what it draws.

Input recipe (the same for every workload):
  * one ``torch.Generator`` seeded with ``seed`` on the device the tensors are
    drawn on; tensors are drawn in a fixed order: x, W_router, W_gate, W_up,
    W_down, shared W_gate/W_up/W_down, then the bias vectors;
  * every tensor is drawn as float32 N(0, 1) scaled by its standard deviation
    and then rounded once to its storage dtype (round-to-nearest-even);
  * expert weights use the nn.Linear layout per expert: gate/up ``[E, H, D]``,
    down ``[E, D, H]``; the router is ``[E, D]`` (Linear(D, E, bias=False)).

The five named workloads follow the shapes of the dense Mixtral-like and the
fine-grained DeepSeek-like layers the pages describe ("2.9 Mixture-of-Experts
(MoE) Architectures", sections "Mixtral 8x7B" and "DeepSeek-MoE and the
fine-grained + shared-expert idea"), a Switch-style top-1 layer with a
capacity factor (same page, "Capacity Factor, Token Dropping, and the Worked
Numbers") and the dropless lab layer ("Lab: build a tiny MoE in PyTorch").
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int
    D: int
    H: int
    E: int
    top_k: int
    act_dtype: str = "bf16"          # dtype of x, expert weights and the output
    router_dtype: str = "bf16"       # dtype of W_router
    score: str = "softmax"           # "softmax" | "sigmoid"
    renormalize: bool = True
    route_scale: float = 1.0
    n_groups: int = 1
    topk_groups: int = 1
    group_rule: str = "top2sum"      # "top2sum" | "max"
    capacity_factor: Optional[float] = None   # None: dropless
    H_shared: int = 0
    x_std: float = 1.0
    w_std: float = 0.02
    logit_bias: str = "none"         # "none" | "zipf" | "gauss"
    zipf_s: float = 1.1
    gauss_sigma: float = 1.0
    select_bias_sigma: float = 0.0   # > 0: per-expert selection-only bias ~ N(0, sigma)

    @property
    def T(self) -> int:
        return self.batch * self.seq

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, in the order they are listed in the benchmark description.
TINY = Workload("tiny_dropless_fp32", batch=2, seq=128, D=64, H=128, E=4, top_k=2,
                act_dtype="f32", router_dtype="f32")
SWITCH = Workload("switch_top1_capacity", batch=8, seq=1024, D=1024, H=2816, E=64,
                  top_k=1, router_dtype="f32", renormalize=False,
                  capacity_factor=1.25, logit_bias="zipf", zipf_s=1.1)
MIXTRAL = Workload("mixtral_8x_top2", batch=4, seq=1024, D=4096, H=14336, E=8, top_k=2)
DEEPSEEK = Workload("deepseek_v3_256x_top8_grouped", batch=1, seq=8192, D=7168, H=2048,
                    E=256, top_k=8, score="sigmoid", route_scale=2.5, n_groups=8,
                    topk_groups=4, H_shared=2048, w_std=0.006, select_bias_sigma=0.01)
DECODE = Workload("decode_128x_top8", batch=1, seq=64, D=4096, H=1536, E=128, top_k=8,
                  logit_bias="gauss", gauss_sigma=1.0)

WORKLOADS = {w.name: w for w in (TINY, SWITCH, MIXTRAL, DEEPSEEK, DECODE)}

# Reduced shapes with the same routing structure as the big workloads.  They
# span several kernel tiles and end in ragged tails, and the oracle runs them
# in seconds, so every output element can be compared.
SMALL = {
    "tiny": TINY,
    "switch_small": SWITCH.with_(name="switch_small", batch=3, seq=331, D=256, H=320,
                                 E=16),
    "mixtral_small": MIXTRAL.with_(name="mixtral_small", batch=2, seq=389, D=512,
                                   H=448, E=8),
    "deepseek_small": DEEPSEEK.with_(name="deepseek_small", batch=1, seq=517, D=384,
                                     H=192, E=64, n_groups=8, topk_groups=4, top_k=6,
                                     H_shared=256),
    "decode_small": DECODE.with_(name="decode_small", batch=1, seq=37, D=512, H=384,
                                 E=32, top_k=8),
    # 64-191 rows per expert on average, the band of the full Switch-shaped
    # layer (8192 rows over 64 experts): a capacity-limited Zipf-skewed layer
    # (C = 125) and a dropless top-2 one (about 150 rows per expert).
    "switch_band": SWITCH.with_(name="switch_band", batch=1, seq=1600, D=256, H=320, E=16),
    "mixtral_band": MIXTRAL.with_(name="mixtral_band", batch=1, seq=601, D=256, H=320, E=8),
}

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def _draw(shape, std, dtype, gen, device, chunks=1):
    """float32 N(0,1)*std rounded once to ``dtype``; drawn in ``chunks`` slices
    along dim 0 to bound the float32 temporary."""
    out = torch.empty(shape, dtype=dtype, device=device)
    n = shape[0]
    step = max(1, math.ceil(n / chunks))
    for i in range(0, n, step):
        sub = (min(step, n - i),) + tuple(shape[1:])
        out[i:i + sub[0]] = (torch.randn(sub, generator=gen, device=device,
                                          dtype=torch.float32) * std).to(dtype)
    return out


def make_inputs(w: Workload, device="cpu", seed: int = 0) -> dict:
    """Draw every input tensor of workload ``w`` on ``device``."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    act = torch_dtype(w.act_dtype)
    T, D, H, E = w.T, w.D, w.H, w.E
    big = E * H * D > (1 << 26)
    inp = {}
    inp["x"] = _draw((T, D), w.x_std, act, gen, device)
    inp["w_router"] = _draw((E, D), w.w_std, torch_dtype(w.router_dtype), gen, device)
    inp["w_gate"] = _draw((E, H, D), w.w_std, act, gen, device, chunks=E if big else 1)
    inp["w_up"] = _draw((E, H, D), w.w_std, act, gen, device, chunks=E if big else 1)
    inp["w_down"] = _draw((E, D, H), w.w_std, act, gen, device, chunks=E if big else 1)
    if w.H_shared:
        Hs = w.H_shared
        inp["ws_gate"] = _draw((Hs, D), w.w_std, act, gen, device)
        inp["ws_up"] = _draw((Hs, D), w.w_std, act, gen, device)
        inp["ws_down"] = _draw((D, Hs), w.w_std, act, gen, device)
    if w.logit_bias == "zipf":
        # log of the unnormalised Zipf(s) pmf over expert rank r = e + 1; the
        # normalising constant is dropped because softmax ignores a shift.
        r = torch.arange(1, E + 1, dtype=torch.float64)
        inp["logit_bias"] = (-w.zipf_s * torch.log(r)).to(torch.float32).to(device)
    elif w.logit_bias == "gauss":
        inp["logit_bias"] = torch.randn(E, generator=gen, device=device,
                                        dtype=torch.float32) * w.gauss_sigma
    if w.select_bias_sigma > 0:
        inp["select_bias"] = torch.randn(E, generator=gen, device=device,
                                         dtype=torch.float32) * w.select_bias_sigma
    return inp


def to_f64(t: torch.Tensor):
    """Exact upcast of stored values (bf16 or fp32) to a float64 NumPy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
