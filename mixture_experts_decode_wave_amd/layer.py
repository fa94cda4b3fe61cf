"""Device set-up of one MoE layer for the library, and thin calls of its
entry points on torch tensors.

A layer's tensors (router, expert matrices and scales, shared expert, token
rows) already live on the GPU; this module only builds the pointer tables
and the shared-expert struct the C ABI takes, allocates a zero-filled
workspace, and allocates the output tensors of a call.  Every step of the
layer runs in libmoewave.so.

`li` is any object with the fields of a layer's inputs: spec (hidden,
num_experts, top_k, inter, shared_inter, scoring, norm_topk, routed_scaling,
act_dtype, expert_dtype), x, router, bias, gate / up / down and sh_gate /
sh_up / sh_down (each with stacked weights .w and scales .s), sgate.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Any, Optional

import torch

from . import (ExpertTables, SharedExpert, alloc_workspace, make_cfg, moe_cfg,
               moe_experts_forward, moe_layer_forward, moe_route)


def cfg_of(spec) -> moe_cfg:
    return make_cfg(spec.hidden, spec.num_experts, spec.top_k, spec.inter, spec.shared_inter,
                    spec.scoring, spec.norm_topk, spec.routed_scaling, spec.act_dtype,
                    spec.expert_dtype, getattr(spec, "zero_experts", 0))


def _width(spec) -> int:
    """Logits per row: the real experts, then the zero-computation experts."""
    return spec.num_experts + getattr(spec, "zero_experts", 0)


@dataclass
class DeviceLayer:
    li: Any
    cfg: moe_cfg
    tables: ExpertTables
    shared: Optional[SharedExpert]
    ws: torch.Tensor
    max_n: int

    @property
    def spec(self):
        return self.li.spec


def device_layer(li, max_n: int = 256) -> DeviceLayer:
    """Pointer tables and a workspace for a layer whose tensors live on a GPU."""
    cfg = cfg_of(li.spec)
    g, u, d = li.gate, li.up, li.down
    tables = ExpertTables.from_stacked(g.w, u.w, d.w, g.s, u.s, d.s)
    shared = None
    if li.sh_gate is not None:
        shared = SharedExpert(li.sh_gate.w[0], li.sh_up.w[0], li.sh_down.w[0],
                              None if li.sh_gate.s is None else li.sh_gate.s[0],
                              None if li.sh_up.s is None else li.sh_up.s[0],
                              None if li.sh_down.s is None else li.sh_down.s[0],
                              li.sgate)
    ws = alloc_workspace(cfg, max_n, li.x.device)
    return DeviceLayer(li, cfg, tables, shared, ws, max_n)


def run_layer(dl: DeviceLayer, n: int, x: Optional[torch.Tensor] = None, stream=None):
    """moe_layer_forward on the first n rows of x; returns device tensors."""
    spec = dl.spec
    x = (dl.li.x if x is None else x)[:n].contiguous()
    dev = x.device
    out = torch.empty(n, spec.hidden, dtype=x.dtype, device=dev)
    logits = torch.empty(n, _width(spec), dtype=torch.float32, device=dev)
    idx = torch.empty(n, spec.top_k, dtype=torch.int32, device=dev)
    w = torch.empty(n, spec.top_k, dtype=torch.float32, device=dev)
    moe_layer_forward(dl.cfg, x, dl.li.router, dl.li.bias, dl.tables, dl.shared, out, dl.ws,
                      logits=logits, topk_idx=idx, topk_w=w, stream=stream)
    return {"out": out, "logits": logits, "idx": idx, "w": w}


def run_route(dl: DeviceLayer, n: int, x: Optional[torch.Tensor] = None):
    """moe_route on the first n rows of x: logits, idx and w."""
    spec = dl.spec
    x = (dl.li.x if x is None else x)[:n].contiguous()
    dev = x.device
    logits = torch.empty(n, _width(spec), dtype=torch.float32, device=dev)
    idx = torch.empty(n, spec.top_k, dtype=torch.int32, device=dev)
    w = torch.empty(n, spec.top_k, dtype=torch.float32, device=dev)
    moe_route(dl.cfg, x, dl.li.router, dl.li.bias, idx, w, dl.ws, logits=logits)
    return {"logits": logits, "idx": idx, "w": w}


def run_experts(dl: DeviceLayer, n: int, idx, w, x: Optional[torch.Tensor] = None):
    """moe_experts_forward on the first n rows of x under a given routing."""
    spec = dl.spec
    x = (dl.li.x if x is None else x)[:n].contiguous()
    out = torch.empty(n, spec.hidden, dtype=x.dtype, device=x.device)
    idx = torch.as_tensor(idx, dtype=torch.int32).to(x.device).contiguous()
    w = torch.as_tensor(w, dtype=torch.float32).to(x.device).contiguous()
    moe_experts_forward(dl.cfg, x, dl.tables, dl.shared, idx, w, out, dl.ws)
    return out
