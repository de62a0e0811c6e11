"""Device-side containers for the binding: upload of storage arrays into HBM and the descriptor /
weight structs the C ABI takes.  Pure marshalling; no arithmetic of the layer happens here."""
from __future__ import annotations

import numpy as np
import torch

from . import (MOE_FMT_F32, MOE_ROUTER_BIAS, MOE_ROUTER_NORM, moe_desc_t, moe_dispatch_t, moe_weights_t,
               moe_workspace_bytes)
from . import synth


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Storage array -> device tensor with the same bytes (bf16 for uint16 storage)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def desc_of(cfg: synth.LayerConfig, max_tokens: int = None, layer: "DeviceLayer" = None) -> moe_desc_t:
    """The C descriptor of a layer configuration; the router prologue tensors come from `layer`."""
    flags = (MOE_ROUTER_NORM if cfg.router_norm else 0) | (MOE_ROUTER_BIAS if cfg.router_bias else 0)
    d = moe_desc_t(cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter, cfg.shared_inter,
                   max_tokens or cfg.M, cfg.act_fmt, cfg.weight_fmt, flags, cfg.norm_eps)
    if flags:
        if layer is None:
            raise ValueError("%s has a router prologue: pass its DeviceLayer" % cfg.name)
        d.norm_weight = layer.t["norm_w"].data_ptr() if cfg.router_norm else None
        d.router_bias = layer.t["router_bias"].data_ptr() if cfg.router_bias else None
    return d


class DeviceLayer:
    """One layer's weights in HBM (keeps the tensors alive while the struct points at them)."""

    def __init__(self, layer: synth.Layer, device="cuda"):
        self.cfg = layer.cfg
        self.t = {"router": to_device(layer.router, device)}
        if getattr(layer, "norm_w", None) is not None:
            self.t["norm_w"] = to_device(layer.norm_w, device)
        if getattr(layer, "router_bias", None) is not None:
            self.t["router_bias"] = to_device(layer.router_bias, device)
        for name in ("gate", "up", "down"):
            data, sc = layer.stacks[name]
            self.t[name] = to_device(data, device)
            if sc is not None:
                self.t[name + "_s"] = to_device(sc, device)
        if layer.shared is not None:
            for name in ("gate", "up", "down"):
                data, sc = layer.shared[name]
                self.t["sh_" + name] = to_device(data, device)
                if sc is not None:
                    self.t["sh_" + name + "_s"] = to_device(sc, device)

    @classmethod
    def from_tensors(cls, cfg, tensors: dict):
        obj = cls.__new__(cls)
        obj.cfg = cfg
        obj.t = dict(tensors)
        return obj

    def clone(self) -> "DeviceLayer":
        """A copy at distinct device addresses with the same values."""
        return DeviceLayer.from_tensors(self.cfg, {k: v.clone() for k, v in self.t.items()})

    @property
    def router(self) -> torch.Tensor:
        return self.t["router"]

    def weights(self) -> moe_weights_t:
        g = lambda n: self.t[n].data_ptr() if n in self.t else None  # noqa: E731
        return moe_weights_t(g("gate"), g("up"), g("down"), g("gate_s"), g("up_s"), g("down_s"),
                             g("sh_gate"), g("sh_up"), g("sh_down"), g("sh_gate_s"), g("sh_up_s"), g("sh_down_s"))

    def nbytes(self) -> int:
        return sum(v.numel() * v.element_size() for v in self.t.values())


def workspace(desc: moe_desc_t, device="cuda") -> torch.Tensor:
    n = moe_workspace_bytes(desc)
    if n == 0:
        raise ValueError("invalid layer description")
    return torch.zeros(n, dtype=torch.uint8, device=device)


class DispatchOut:
    """Device buffers receiving the optional dispatch description of a call."""

    def __init__(self, M: int, k: int, E: int, R: int = 0, device="cuda"):
        nu = min(M * k, E)
        self.unit_count = torch.zeros(1, dtype=torch.int32, device=device)
        self.unit_expert = torch.full((nu + 1,), -1, dtype=torch.int32, device=device)
        self.unit_off = torch.full((nu + 2,), -1, dtype=torch.int32, device=device)
        self.row_token = torch.full((M * k + M,), -1, dtype=torch.int32, device=device)
        self.row_slot = torch.full((M * k + M,), -1, dtype=torch.int32, device=device)
        self.row_weight = torch.full((M * k + M,), -1.0, dtype=torch.float32, device=device)
        self.req_unique = torch.full((max(R, 1),), -1, dtype=torch.int32, device=device) if R else None

    def struct(self) -> moe_dispatch_t:
        p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
        return moe_dispatch_t(p(self.unit_count), p(self.unit_expert), p(self.unit_off), p(self.row_token),
                              p(self.row_slot), p(self.row_weight), p(self.req_unique))


def act_dtype(cfg) -> torch.dtype:
    return torch.float32 if cfg.act_fmt == MOE_FMT_F32 else torch.bfloat16
