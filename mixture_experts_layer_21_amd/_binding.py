"""ctypes binding over ``libmoe.so``: argument marshalling only.

Every function here checks that the tensors it is given have the shapes,
dtypes and devices the C entry point of the same name expects (so no kernel
ever runs past a buffer), passes their device pointers and the current HIP
stream, and raises ``MoeError`` on a non-OK status.  All compute runs in the
HIP kernels; there is no fallback path.  PyTorch is used for device memory
and streams only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python mixture_experts_layer_21_amd/build.py` "
        "(gfx950 HIP library, no CPU fallback exists)")
_lib = ctypes.CDLL(LIB_PATH)

# ------------------------------------------------------------------ enums ---
MOE_OK = 0
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_NULL_PTR",
          3: "MOE_ERR_UNSUPPORTED", 4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_DEVICE",
          6: "MOE_ERR_HIP"}
DTYPES = {"f32": 0, "bf16": 1}
SCORES = {"softmax": 0, "sigmoid": 1, "sqrtsoftplus": 2}
GROUP_RULES = {"top2sum": 0, "max": 1}
_TORCH = {0: torch.float32, 1: torch.bfloat16}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _lib.moe_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


class MoeConfig(ctypes.Structure):
    """Mirror of ``moe_config`` in include/moe.h."""
    _fields_ = [
        ("T", ctypes.c_int32), ("D", ctypes.c_int32), ("H", ctypes.c_int32),
        ("E", ctypes.c_int32), ("top_k", ctypes.c_int32), ("H_shared", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32), ("router_dtype", ctypes.c_int32),
        ("score_func", ctypes.c_int32), ("renormalize", ctypes.c_int32),
        ("route_scale", ctypes.c_float), ("n_groups", ctypes.c_int32),
        ("topk_groups", ctypes.c_int32), ("group_rule", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double), ("swiglu_limit", ctypes.c_float),
        ("pre_norm", ctypes.c_int32), ("norm_eps", ctypes.c_float),
    ]

    @property
    def act_torch_dtype(self):
        return _TORCH[self.act_dtype]

    @property
    def router_torch_dtype(self):
        return _TORCH[self.router_dtype]


def make_config(T, D, H, E, top_k, *, H_shared=0, act_dtype="bf16", router_dtype="bf16",
                score="softmax", renormalize=True, route_scale=1.0, n_groups=1,
                topk_groups=1, group_rule="top2sum", capacity_factor=None,
                swiglu_limit=0.0, pre_norm=False, norm_eps=1e-6) -> MoeConfig:
    return MoeConfig(T=T, D=D, H=H, E=E, top_k=top_k, H_shared=H_shared,
                     act_dtype=DTYPES[act_dtype], router_dtype=DTYPES[router_dtype],
                     score_func=SCORES[score], renormalize=int(bool(renormalize)),
                     route_scale=route_scale, n_groups=n_groups, topk_groups=topk_groups,
                     group_rule=GROUP_RULES[group_rule],
                     capacity_factor=0.0 if capacity_factor is None else capacity_factor,
                     swiglu_limit=float(swiglu_limit), pre_norm=int(bool(pre_norm)),
                     norm_eps=float(norm_eps))


_P = ctypes.c_void_p
_CFG = ctypes.POINTER(MoeConfig)
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_sigs = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_check_config": (ctypes.c_int, [_CFG]),
    "moe_capacity": (_I32, [_CFG]),
    "moe_max_rows": (_I32, [_CFG]),
    "moe_workspace_bytes": (_SZ, [_CFG]),
    "moe_route": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute": (ctypes.c_int, [_CFG, _P, _I32, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_swiglu": (ctypes.c_int, [_CFG, _I32, _I32, _P, _P, _P, _I32, _P, _P, _P,
                                          _P, _P, _P, _SZ, _P]),
    "moe_combine": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_forward": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_forward_noalloc": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_saved_bytes": (ctypes.c_size_t, [_CFG]),
    "moe_rmsnorm": (ctypes.c_int, [_CFG, _P, _P, _P, _P]),
    "moe_backward_workspace_bytes": (_SZ, [_CFG]),
    "moe_backward": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, ctypes.c_float, ctypes.c_float, _P, _P, _P, _P, _P, _P,
                                    _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_update_bias": (ctypes.c_int, [_CFG, _P, ctypes.c_float, _P, _P]),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sigs)


# --------------------------------------------------------------- helpers ---

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _mask(token_mask, T):
    """A [T] token mask as contiguous uint8 (nonzero = valid), or None."""
    if token_mask is None:
        return None
    if not token_mask.is_cuda or tuple(token_mask.shape) != (T,):
        raise ValueError(f"token_mask must be a device tensor of shape ({T},)")
    if token_mask.dtype not in (torch.bool, torch.uint8):
        raise ValueError("token_mask must be bool or uint8")
    return token_mask.to(torch.uint8).contiguous()


def _expect(t: Optional[torch.Tensor], name: str, shape, dtype, required=True):
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def check_config(cfg: MoeConfig):
    _check(_lib.moe_check_config(ctypes.byref(cfg)), "moe_check_config")


def capacity(cfg: MoeConfig) -> int:
    return _lib.moe_capacity(ctypes.byref(cfg))


def max_rows(cfg: MoeConfig) -> int:
    return _lib.moe_max_rows(ctypes.byref(cfg))


def workspace_bytes(cfg: MoeConfig) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(cfg))


def status_string(s: int) -> str:
    return _lib.moe_status_string(s).decode()


def new_workspace(cfg: MoeConfig, device="cuda") -> torch.Tensor:
    n = workspace_bytes(cfg)
    if n == 0:
        check_config(cfg)
    return torch.empty(n, dtype=torch.uint8, device=device)


# ---------------------------------------------------------- entry points ---

def moe_route(cfg, x, w_router, logit_bias=None, select_bias=None, *, token_mask=None,
              expert_ids=None, gate_w=None, counts=None, aux=None, mean_prob=None,
              workspace=None):
    """Routing (see ``moe_route`` in include/moe.h).  ``token_mask`` [T]
    (bool or uint8, nonzero = valid) leaves padding tokens unrouted.  Returns
    a dict of the output tensors (allocated here when not given)."""
    check_config(cfg)
    T, D, E, k = cfg.T, cfg.D, cfg.E, cfg.top_k
    dev = x.device
    _expect(x, "x", (T, D), cfg.act_torch_dtype)
    _expect(w_router, "w_router", (E, D), cfg.router_torch_dtype)
    _expect(logit_bias, "logit_bias", (E,), torch.float32, required=False)
    _expect(select_bias, "select_bias", (E,), torch.float32, required=False)
    token_mask = _mask(token_mask, T)
    expert_ids = torch.empty(T, k, dtype=torch.int32, device=dev) if expert_ids is None else expert_ids
    gate_w = torch.empty(T, k, dtype=torch.float32, device=dev) if gate_w is None else gate_w
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    aux = torch.empty(2, dtype=torch.float32, device=dev) if aux is None else aux
    mean_prob = torch.empty(E, dtype=torch.float32, device=dev) if mean_prob is None else mean_prob
    _expect(expert_ids, "expert_ids", (T, k), torch.int32)
    _expect(gate_w, "gate_w", (T, k), torch.float32)
    _expect(counts, "counts", (E,), torch.int32)
    _expect(aux, "aux", (2,), torch.float32)
    _expect(mean_prob, "mean_prob", (E,), torch.float32)
    ws = new_workspace(cfg, dev) if workspace is None else workspace
    _check(_lib.moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(logit_bias),
                          _ptr(select_bias), _ptr(token_mask), _ptr(expert_ids), _ptr(gate_w),
                          _ptr(counts),
                          _ptr(aux), _ptr(mean_prob), _ptr(ws), ws.numel(), _stream()),
           "moe_route")
    return {"expert_ids": expert_ids, "gate_w": gate_w, "counts": counts, "aux": aux,
            "mean_prob": mean_prob}


def moe_permute(cfg, expert_ids, capacity_limit: int = 0, *, expert_offsets=None,
                row_to_assign=None, assign_to_row=None, n_kept=None, workspace=None):
    """Dispatch bookkeeping (see ``moe_permute``).  ``capacity_limit`` <= 0 is
    dropless.  Returns expert_offsets, row_to_assign, assign_to_row, n_kept
    (allocated here when not given; a row_to_assign allocated here starts as
    -1, so rows past n_kept read -1)."""
    check_config(cfg)
    T, E, k = cfg.T, cfg.E, cfg.top_k
    dev = expert_ids.device
    _expect(expert_ids, "expert_ids", (T, k), torch.int32)
    rows = T * k
    _expect(expert_offsets, "expert_offsets", (E + 1,), torch.int32, required=False)
    _expect(row_to_assign, "row_to_assign", (rows,), torch.int32, required=False)
    _expect(assign_to_row, "assign_to_row", (rows,), torch.int32, required=False)
    _expect(n_kept, "n_kept", (1,), torch.int32, required=False)
    offsets = (torch.empty(E + 1, dtype=torch.int32, device=dev)
               if expert_offsets is None else expert_offsets)
    r2a = (torch.full((rows,), -1, dtype=torch.int32, device=dev)
           if row_to_assign is None else row_to_assign)
    a2r = torch.empty(rows, dtype=torch.int32, device=dev) if assign_to_row is None else assign_to_row
    n_kept = torch.empty(1, dtype=torch.int32, device=dev) if n_kept is None else n_kept
    ws = new_workspace(cfg, dev) if workspace is None else workspace
    _check(_lib.moe_permute(ctypes.byref(cfg), _ptr(expert_ids), int(capacity_limit),
                            _ptr(offsets), _ptr(r2a), _ptr(a2r), _ptr(n_kept), _ptr(ws),
                            ws.numel(), _stream()), "moe_permute")
    return {"expert_offsets": offsets, "row_to_assign": r2a, "assign_to_row": a2r,
            "n_kept": n_kept}


def moe_grouped_swiglu(cfg, x, w_gate, w_up, w_down, *, row_to_assign=None,
                       expert_offsets=None, max_rows_bound=None, gate_w=None, y_rows=None,
                       workspace=None, validate=True):
    """Grouped SwiGLU experts (see ``moe_grouped_swiglu``).  Without
    ``row_to_assign`` the call is the identity-row (shared expert) form.
    ``validate`` copies the offsets and row map to the host (a synchronisation)
    to check that every row the kernels will read is in bounds."""
    check_config(cfg)
    T, D = cfg.T, cfg.D
    G, hidden = w_gate.shape[0], w_gate.shape[1]
    dt = cfg.act_torch_dtype
    _expect(x, "x", (T, D), dt)
    identity = row_to_assign is None
    if identity:
        if w_gate.dim() == 2:
            G, hidden = 1, w_gate.shape[0]
            w_gate, w_up, w_down = (w.unsqueeze(0) for w in (w_gate, w_up, w_down))
        rows = T
    else:
        rows = int(max_rows_bound if max_rows_bound is not None else row_to_assign.numel())
        if rows > row_to_assign.numel():
            raise ValueError("max_rows_bound exceeds row_to_assign")
        _expect(expert_offsets, "expert_offsets", (G + 1,), torch.int32)
        _expect(gate_w, "gate_w", (T, cfg.top_k), torch.float32, required=False)
        if row_to_assign.dtype != torch.int32 or not row_to_assign.is_contiguous():
            raise ValueError("row_to_assign must be contiguous int32")
        if validate:
            off = expert_offsets.cpu()
            if off[0] != 0 or bool((off[1:] < off[:-1]).any()) or int(off[-1]) > rows:
                raise ValueError("expert_offsets must be non-decreasing from 0 to <= max_rows")
            used = row_to_assign[:int(off[-1])].cpu()
            if used.numel() and (int(used.min()) < 0 or int(used.max()) >= T * cfg.top_k):
                raise ValueError("row_to_assign entries must be assignment indices < T*top_k")
    _expect(w_gate, "w_gate", (G, hidden, D), dt)
    _expect(w_up, "w_up", (G, hidden, D), dt)
    _expect(w_down, "w_down", (G, D, hidden), dt)
    y_rows = torch.empty(max(rows, 1), D, dtype=dt, device=x.device) if y_rows is None else y_rows
    if y_rows.shape[0] < rows or y_rows.shape[1] != D or y_rows.dtype != dt or not y_rows.is_contiguous():
        raise ValueError("y_rows must be contiguous [>= max_rows, D] of the activation dtype")
    ws = new_workspace(cfg, x.device) if workspace is None else workspace
    need = rows * hidden * (2 if dt == torch.bfloat16 else 4)
    if ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(_lib.moe_grouped_swiglu(ctypes.byref(cfg), G, hidden, _ptr(x), _ptr(row_to_assign),
                                   _ptr(expert_offsets), rows, _ptr(gate_w), _ptr(w_gate),
                                   _ptr(w_up), _ptr(w_down), _ptr(y_rows), _ptr(ws),
                                   ws.numel(), _stream()), "moe_grouped_swiglu")
    return y_rows


def moe_combine(cfg, y_rows, assign_to_row, shared_rows=None, out=None, validate=True, *,
                x=None, shared_expert_gate=None, residual=None):
    """Combine (see ``moe_combine``).  Every non-negative entry of
    ``assign_to_row`` must index a row of ``y_rows``; ``validate`` checks that
    on the host (a synchronisation)."""
    check_config(cfg)
    T, D, k = cfg.T, cfg.D, cfg.top_k
    dt = cfg.act_torch_dtype
    if y_rows.dim() != 2 or y_rows.shape[1] != D or y_rows.dtype != dt or not y_rows.is_contiguous():
        raise ValueError("y_rows must be contiguous [rows, D] of the activation dtype")
    _expect(assign_to_row, "assign_to_row", (T * k,), torch.int32)
    if validate and int(assign_to_row.max()) >= y_rows.shape[0]:
        raise ValueError("assign_to_row indexes past the end of y_rows")
    _expect(shared_rows, "shared_rows", (T, D), dt, required=False)
    _expect(x, "x", (T, D), dt, required=False)
    _expect(shared_expert_gate, "shared_expert_gate", (D,), dt, required=False)
    _expect(residual, "residual", (T, D), dt, required=False)
    out = torch.empty(T, D, dtype=dt, device=y_rows.device) if out is None else out
    _expect(out, "out", (T, D), dt)
    _check(_lib.moe_combine(ctypes.byref(cfg), _ptr(y_rows), _ptr(assign_to_row),
                            _ptr(shared_rows), _ptr(x), _ptr(shared_expert_gate),
                            _ptr(residual), _ptr(out), _stream()), "moe_combine")
    return out


def _forward_args(cfg, x, w_router, w_gate, w_up, w_down, logit_bias, select_bias, ws_gate,
                  ws_up, ws_down, out, expert_ids, gate_w, counts, aux, token_mask,
                  shared_expert_gate, residual, norm_weight, saved):
    """Checked pointer arguments of moe_forward / moe_forward_noalloc up to
    ``saved`` (the output is allocated here when ``out`` is None), with the
    output and the token mask actually passed."""
    check_config(cfg)
    T, D, H, E, k, Hs = cfg.T, cfg.D, cfg.H, cfg.E, cfg.top_k, cfg.H_shared
    dt = cfg.act_torch_dtype
    _expect(x, "x", (T, D), dt)
    _expect(w_router, "w_router", (E, D), cfg.router_torch_dtype)
    _expect(w_gate, "w_gate", (E, H, D), dt)
    _expect(w_up, "w_up", (E, H, D), dt)
    _expect(w_down, "w_down", (E, D, H), dt)
    _expect(logit_bias, "logit_bias", (E,), torch.float32, required=False)
    _expect(select_bias, "select_bias", (E,), torch.float32, required=False)
    if Hs:
        _expect(ws_gate, "ws_gate", (Hs, D), dt)
        _expect(ws_up, "ws_up", (Hs, D), dt)
        _expect(ws_down, "ws_down", (D, Hs), dt)
    _expect(shared_expert_gate, "shared_expert_gate", (D,), dt, required=False)
    _expect(residual, "residual", (T, D), dt, required=False)
    _expect(norm_weight, "norm_weight", (D,), torch.float32, required=False)
    token_mask = _mask(token_mask, T)
    out = torch.empty(T, D, dtype=dt, device=x.device) if out is None else out
    _expect(out, "out", (T, D), dt)
    _expect(expert_ids, "expert_ids", (T, k), torch.int32, required=False)
    _expect(gate_w, "gate_w", (T, k), torch.float32, required=False)
    _expect(counts, "counts", (E,), torch.int32, required=False)
    _expect(aux, "aux", (2,), torch.float32, required=False)
    # token_mask may be a converted copy: it rides along in the tuple so that
    # it stays alive until the call has been enqueued
    return out, token_mask, (ctypes.byref(cfg), _ptr(x), _ptr(norm_weight), _ptr(w_router),
                 _ptr(logit_bias), _ptr(select_bias), _ptr(token_mask), _ptr(w_gate),
                 _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down),
                 _ptr(shared_expert_gate), _ptr(residual), _ptr(out), _ptr(expert_ids),
                 _ptr(gate_w), _ptr(counts), _ptr(aux), _ptr(saved))


def moe_forward(cfg, x, w_router, w_gate, w_up, w_down, *, logit_bias=None, select_bias=None,
                ws_gate=None, ws_up=None, ws_down=None, out=None, expert_ids=None, gate_w=None,
                counts=None, aux=None, workspace=None, token_mask=None,
                shared_expert_gate=None, residual=None, norm_weight=None, saved=None):
    """The whole layer forward (see ``moe_forward``); with ``cfg.pre_norm``
    the layer takes RMSNorm(x) (``norm_weight`` [D] f32 or None).  ``saved``
    (uint8 device tensor of ``saved_bytes(cfg)``, see ``new_saved``) receives
    the SwiGLU state that ``moe_backward(saved=...)`` then reuses."""
    out, _keep, args = _forward_args(cfg, x, w_router, w_gate, w_up, w_down, logit_bias,
                                     select_bias, ws_gate, ws_up, ws_down, out, expert_ids,
                                     gate_w, counts, aux, token_mask, shared_expert_gate,
                                     residual, norm_weight, saved)
    ws = new_workspace(cfg, x.device) if workspace is None else workspace
    _check(_lib.moe_forward(*args, _ptr(ws), ws.numel(), _stream()), "moe_forward")
    return out


def moe_forward_noalloc(cfg, x, w_router, w_gate, w_up, w_down, *, out, logit_bias=None,
                        select_bias=None, ws_gate=None, ws_up=None, ws_down=None,
                        expert_ids=None, gate_w=None, counts=None, aux=None, token_mask=None,
                        shared_expert_gate=None, residual=None, norm_weight=None, saved=None):
    """``moe_forward`` on the library's static scratch (see
    ``moe_forward_noalloc``): no workspace, and the caller passes ``out`` so
    that the call allocates nothing."""
    out, _keep, args = _forward_args(cfg, x, w_router, w_gate, w_up, w_down, logit_bias,
                                     select_bias, ws_gate, ws_up, ws_down, out, expert_ids,
                                     gate_w, counts, aux, token_mask, shared_expert_gate,
                                     residual, norm_weight, saved)
    _check(_lib.moe_forward_noalloc(*args, _stream()), "moe_forward_noalloc")
    return out


def moe_rmsnorm(cfg, x, norm_weight=None, out=None):
    """RMSNorm of x [T, D] (see ``moe_rmsnorm``): x / sqrt(mean(x^2) +
    cfg.norm_eps) * norm_weight, in act dtype; ``out`` may be ``x``."""
    check_config(cfg)
    dt = cfg.act_torch_dtype
    _expect(x, "x", (cfg.T, cfg.D), dt)
    _expect(norm_weight, "norm_weight", (cfg.D,), torch.float32, required=False)
    out = torch.empty_like(x) if out is None else out
    _expect(out, "out", (cfg.T, cfg.D), dt)
    _check(_lib.moe_rmsnorm(ctypes.byref(cfg), _ptr(x), _ptr(norm_weight), _ptr(out),
                            _stream()), "moe_rmsnorm")
    return out


def backward_workspace_bytes(cfg) -> int:
    return int(_lib.moe_backward_workspace_bytes(ctypes.byref(cfg)))


def saved_bytes(cfg):
    """Bytes of the forward's saved SwiGLU state (0: not bf16)."""
    return int(_lib.moe_saved_bytes(ctypes.byref(cfg)))


def new_saved(cfg, device="cuda"):
    n = saved_bytes(cfg)
    if n == 0:
        raise ValueError("saved SwiGLU state needs bf16 activations")
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_backward(cfg, x, w_router, w_gate, w_up, w_down, expert_ids, gate_w, dout, *,
                 logit_bias=None, ws_gate=None, ws_up=None, ws_down=None, balance_coef=0.0,
                 z_coef=0.0, workspace=None, d_gate_w=False, norm_weight=None,
                 shared_expert_gate=None, saved=None):
    """Gradients of <dout, out> + balance_coef*balance + z_coef*z (see
    ``moe_backward``).  Returns a dict with dx (act dtype) and the fp32
    weight gradients dw_router, dw_gate, dw_up, dw_down (+ dws_* with a shared
    expert, + d_gate_w [T,k] when asked, + d_norm_weight [D] with the
    pre-norm, + d_shared_gate [D] with ``shared_expert_gate``).  ``saved``:
    the state ``moe_forward(saved=...)`` kept for these inputs and routes
    (the gate/up GEMMs are then not recomputed).  With
    ``cfg.pre_norm``, ``x`` is the input before the norm and ``norm_weight``
    [D] f32 (None: unit weight) its weight."""
    check_config(cfg)
    T, D, H, E, k, Hs = cfg.T, cfg.D, cfg.H, cfg.E, cfg.top_k, cfg.H_shared
    dt = cfg.act_torch_dtype
    _expect(x, "x", (T, D), dt)
    _expect(w_router, "w_router", (E, D), cfg.router_torch_dtype)
    _expect(w_gate, "w_gate", (E, H, D), dt)
    _expect(w_up, "w_up", (E, H, D), dt)
    _expect(w_down, "w_down", (E, D, H), dt)
    _expect(logit_bias, "logit_bias", (E,), torch.float32, required=False)
    _expect(expert_ids, "expert_ids", (T, k), torch.int32)
    _expect(gate_w, "gate_w", (T, k), torch.float32)
    _expect(dout, "dout", (T, D), dt)
    _expect(norm_weight, "norm_weight", (D,), torch.float32, required=False)
    _expect(shared_expert_gate, "shared_expert_gate", (D,), dt, required=False)
    if Hs:
        _expect(ws_gate, "ws_gate", (Hs, D), dt)
        _expect(ws_up, "ws_up", (Hs, D), dt)
        _expect(ws_down, "ws_down", (D, Hs), dt)
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"dx": torch.empty(T, D, dtype=dt, device=dev),
         "dw_router": torch.empty(E, D, **f32), "dw_gate": torch.empty(E, H, D, **f32),
         "dw_up": torch.empty(E, H, D, **f32), "dw_down": torch.empty(E, D, H, **f32)}
    if Hs:
        g.update(dws_gate=torch.empty(Hs, D, **f32), dws_up=torch.empty(Hs, D, **f32),
                 dws_down=torch.empty(D, Hs, **f32))
    if d_gate_w:
        g["d_gate_w"] = torch.empty(T, k, **f32)
    if cfg.pre_norm:
        g["d_norm_weight"] = torch.empty(D, **f32)
    if shared_expert_gate is not None and Hs:
        g["d_shared_gate"] = torch.empty(D, **f32)
    nbytes = backward_workspace_bytes(cfg)  # 0: not covered, the library says why
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws = workspace
    _check(_lib.moe_backward(ctypes.byref(cfg), _ptr(x), _ptr(norm_weight), _ptr(w_router),
                             _ptr(logit_bias),
                             _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(ws_gate), _ptr(ws_up),
                             _ptr(ws_down), _ptr(shared_expert_gate), _ptr(expert_ids),
                             _ptr(gate_w), _ptr(dout),
                             float(balance_coef), float(z_coef), _ptr(g["dx"]),
                             _ptr(g["dw_router"]), _ptr(g["dw_gate"]), _ptr(g["dw_up"]),
                             _ptr(g["dw_down"]), _ptr(g.get("dws_gate")), _ptr(g.get("dws_up")),
                             _ptr(g.get("dws_down")), _ptr(g.get("d_shared_gate")),
                             _ptr(g.get("d_gate_w")),
                             _ptr(g.get("d_norm_weight")), _ptr(saved), _ptr(ws),
                             0 if ws is None else ws.numel(), _stream()), "moe_backward")
    return g


def moe_update_bias(cfg, counts, gamma, select_bias):
    """Auxiliary-loss-free balancer step on ``select_bias`` [E] f32, in place
    (see ``moe_update_bias``); ``counts`` [E] int32 as returned by routing."""
    check_config(cfg)
    _expect(counts, "counts", (cfg.E,), torch.int32)
    _expect(select_bias, "select_bias", (cfg.E,), torch.float32)
    _check(_lib.moe_update_bias(ctypes.byref(cfg), _ptr(counts), float(gamma),
                                _ptr(select_bias), _stream()), "moe_update_bias")
    return select_bias
