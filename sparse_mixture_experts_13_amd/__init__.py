"""Sparse Mixture-of-Experts layer forward on one AMD MI355X (gfx950).

Thin Python binding over libmoe.so (include/moe.h).  Every step of the layer
runs in the library's HIP kernels; this module only marshals arguments:
torch tensors supply device memory and the current HIP stream supplies the
stream.  Function names and argument orders follow the C ABI.

    cfg = make_config(T=8192, d_model=768, d_ff=3072, E=128, k=1,
                      capacity_factor=1.0, act="relu", dtype="bf16")
    ws = alloc_workspace(cfg)
    forward(cfg, x, w_r, None, None, w1, w2, y, ws)
"""
from __future__ import annotations

import ctypes
from typing import Optional

from ._lib import ACT, DTYPE, EXPORTS, REGION, ROUTE, MoeConfig, load  # noqa: F401

__all__ = ["MoeConfig", "MoeError", "make_config", "config_for", "capacity", "workspace_bytes",
           "workspace_offset", "alloc_workspace", "workspace_view", "router", "router_aux", "dispatch",
           "expert_ffn", "expert_ffn_fused", "expert_up", "expert_down", "combine", "forward", "forward_noalloc",
           "NOALLOC_SCRATCH_BYTES", "backward_workspace_bytes", "alloc_backward_workspace",
           "backward", "sparse_clip", "version", "load"]


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"moe status {status}: {message}")
        self.status = status


def make_config(T: int, d_model: int, d_ff: int, E: int, k: int, capacity_factor: float,
                act: str = "relu", dtype: str = "bf16", route: str = "topk",
                n_groups: int = 1, rre_seed: int = 0) -> MoeConfig:
    return MoeConfig(T=T, d_model=d_model, d_ff=d_ff, E=E, k=k,
                     capacity_factor=float(capacity_factor), route=ROUTE[route],
                     n_groups=n_groups, rre_seed=rre_seed, act=ACT[act], dtype=DTYPE[dtype])


def config_for(wl) -> MoeConfig:
    """Configuration of a workload record (moe_workloads.Workload or alike); a record
    with a true ``glu`` field selects the GLU form of its activation."""
    act = {"relu": "reglu", "gelu": "geglu"}[wl.act] if getattr(wl, "glu", False) else wl.act
    return make_config(wl.T, wl.d_model, wl.d_ff, wl.E, wl.k, wl.capacity_factor, act,
                       wl.dtype, wl.route, wl.n_groups, wl.rre_seed)


def _status(rc: int) -> None:
    if rc != 0:
        raise MoeError(rc, load().moe_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor arguments must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr() or None


def _stream(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream or None


def capacity(cfg: MoeConfig) -> int:
    c = load().moe_capacity(ctypes.byref(cfg))
    if c < 0:
        _status(int(c))
    return int(c)


def workspace_bytes(cfg: MoeConfig) -> int:
    n = load().moe_workspace_bytes(ctypes.byref(cfg))
    if n < 0:
        _status(int(n))
    return int(n)


def workspace_offset(cfg: MoeConfig, region: str) -> int:
    o = load().moe_workspace_offset(ctypes.byref(cfg), REGION[region])
    if o < 0:
        _status(int(o))
    return int(o)


def alloc_workspace(cfg: MoeConfig, device="cuda"):
    import torch
    return torch.empty(workspace_bytes(cfg), dtype=torch.uint8, device=device)


def workspace_view(ws, cfg: MoeConfig, region: str):
    """A typed view of one region of the workspace that ``forward`` fills."""
    import torch
    elem = torch.bfloat16 if cfg.dtype == DTYPE["bf16"] else torch.float32
    C = capacity(cfg)
    T, k, E = cfg.T, cfg.k, cfg.E
    spec = {"expert_idx": (torch.int32, (T, k)), "gate": (torch.float32, (T, k)),
            "slot": (torch.int32, (T, k)), "expert_count": (torch.int32, (E,)),
            "slot_token": (torch.int32, (E, C)), "x_e": (elem, (E, C, cfg.d_model)),
            "hidden": (elem, (E, C, cfg.d_ff)), "y_e": (elem, (E, C, cfg.d_model))}
    dt, shape = spec[region]
    n = 1
    for s in shape:
        n *= s
    off = workspace_offset(cfg, region)
    nbytes = n * torch.tensor([], dtype=dt).element_size()
    return ws[off:off + nbytes].view(dt).view(shape)


def router(cfg, x, w_r, bias, group_id, expert_idx, gate, ws, stream=None) -> None:
    _status(load().moe_router(ctypes.byref(cfg), _ptr(x), _ptr(w_r), _ptr(bias), _ptr(group_id),
                              _ptr(expert_idx), _ptr(gate), _ptr(ws), _stream(stream)))


def router_aux(cfg, x, w_r, bias, expert_idx, gate, alpha, aux, ws, stream=None) -> None:
    _status(load().moe_router_aux(ctypes.byref(cfg), _ptr(x), _ptr(w_r), _ptr(bias),
                                  _ptr(expert_idx), _ptr(gate), float(alpha), _ptr(aux), _ptr(ws),
                                  _stream(stream)))


def dispatch(cfg, x, expert_idx, slot, expert_count, slot_token, x_e, ws, stream=None) -> None:
    _status(load().moe_dispatch(ctypes.byref(cfg), _ptr(x), _ptr(expert_idx), _ptr(slot),
                                _ptr(expert_count), _ptr(slot_token), _ptr(x_e), _ptr(ws),
                                _stream(stream)))


def expert_ffn(cfg, x_e, expert_count, w1, w2, y_e, ws, stream=None) -> None:
    _status(load().moe_expert_ffn(ctypes.byref(cfg), _ptr(x_e), _ptr(expert_count), _ptr(w1),
                                  _ptr(w2), _ptr(y_e), _ptr(ws), _stream(stream)))


def expert_ffn_fused(cfg, x_e, expert_count, w1, w2, y_e, stream=None) -> None:
    _status(load().moe_expert_ffn_fused(ctypes.byref(cfg), _ptr(x_e), _ptr(expert_count),
                                        _ptr(w1), _ptr(w2), _ptr(y_e), _stream(stream)))


def expert_up(cfg, x_e, expert_count, w1, hidden, stream=None) -> None:
    _status(load().moe_expert_up(ctypes.byref(cfg), _ptr(x_e), _ptr(expert_count), _ptr(w1),
                                 _ptr(hidden), _stream(stream)))


def expert_down(cfg, hidden, expert_count, w2, y_e, stream=None) -> None:
    _status(load().moe_expert_down(ctypes.byref(cfg), _ptr(hidden), _ptr(expert_count), _ptr(w2),
                                   _ptr(y_e), _stream(stream)))


def combine(cfg, y_e, expert_idx, slot, gate, y, stream=None) -> None:
    _status(load().moe_combine(ctypes.byref(cfg), _ptr(y_e), _ptr(expert_idx), _ptr(slot),
                               _ptr(gate), _ptr(y), _stream(stream)))


def backward_workspace_bytes(cfg: MoeConfig) -> int:
    n = load().moe_backward_workspace_bytes(ctypes.byref(cfg))
    if n < 0:
        _status(int(n))
    return int(n)


def alloc_backward_workspace(cfg, device="cuda"):
    """A uint8 device tensor of moe_backward_workspace_bytes(cfg) bytes."""
    import torch
    return torch.empty(max(backward_workspace_bytes(cfg), 1), dtype=torch.uint8, device=device)


def backward(cfg, x, w_r, bias, w1, w2, dy, dx, dw_r, dbias, dw1, dw2, ws, bws, stream=None) -> None:
    _status(load().moe_backward(ctypes.byref(cfg), _ptr(x), _ptr(w_r), _ptr(bias), _ptr(w1), _ptr(w2),
                                _ptr(dy), _ptr(dx), _ptr(dw_r), _ptr(dbias), _ptr(dw1), _ptr(dw2),
                                _ptr(ws), _ptr(bws), _stream(stream)))


def sparse_clip(cfg, dw_r, dbias, dw1, dw2, max_norm, norm_coef, bws, stream=None) -> None:
    _status(load().moe_sparse_clip(ctypes.byref(cfg), _ptr(dw_r), _ptr(dbias), _ptr(dw1), _ptr(dw2),
                                   float(max_norm), _ptr(norm_coef), _ptr(bws), _stream(stream)))


def forward(cfg, x, w_r, bias, group_id, w1, w2, y, ws, stream=None) -> None:
    _status(load().moe_forward(ctypes.byref(cfg), _ptr(x), _ptr(w_r), _ptr(bias), _ptr(group_id),
                               _ptr(w1), _ptr(w2), _ptr(y), _ptr(ws), _stream(stream)))


def forward_noalloc(cfg, x, w_r, bias, group_id, w1, w2, y, stream=None) -> None:
    """moe_forward on the library's static per-GPU scratch (no workspace argument)."""
    _status(load().moe_forward_noalloc(ctypes.byref(cfg), _ptr(x), _ptr(w_r), _ptr(bias), _ptr(group_id),
                                       _ptr(w1), _ptr(w2), _ptr(y), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 80 << 20


def version() -> str:
    return load().moe_version().decode()
