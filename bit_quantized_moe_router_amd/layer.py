"""Device-memory plumbing around the C ABI: upload canonical weights with
torch, pack them once, and hold the workspace.  No arithmetic of the layer
happens here; every step of the layer runs in libmoe.so's HIP kernels."""
from __future__ import annotations

import numpy as np
import torch

from . import (make_desc, moe_forward_decode, moe_forward_prefill, moe_max_tiles, moe_pack_weights,
               moe_packed_bytes, moe_route, moe_workspace_bytes)


def to_dev(a: np.ndarray, device) -> torch.Tensor:
    """Copy a numpy array to the device, keeping its bytes (uint16 travels as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class MoELayer:
    """Packed weights and workspace for one layer on one device."""

    def __init__(self, w: dict, k: int, device="cuda", max_tokens=2048, max_chunk=2048, tile_rows=0,
                 gemv_max_rows=-1, keep_canonical=False):
        self.device = torch.device(device)
        self.H, self.E, self.I, self.Is, self.k = w["H"], w["E"], w["I"], w["Is"], k
        self.desc = make_desc(self.H, self.E, k, self.I, self.Is, gemv_max_rows=gemv_max_rows,
                              max_chunk=max_chunk, tile_rows=tile_rows)
        self.router_w = to_dev(w["router_w"], self.device)

        def qm(m):
            return None if m is None else tuple(to_dev(m[a], self.device) for a in ("codes", "scales", "biases"))

        mats = [qm(w["gate"]), qm(w["up"]), qm(w["down"])]
        mats += [qm(w.get("sh_gate")), qm(w.get("sh_up")), qm(w.get("sh_down"))] if self.Is else [None] * 3
        self.packed = torch.empty(moe_packed_bytes(self.desc), dtype=torch.uint8, device=self.device)
        moe_pack_weights(self.desc, *mats, self.packed)
        self.canonical = mats if keep_canonical else None
        self.max_tokens = max_tokens
        self.ws = torch.empty(moe_workspace_bytes(self.desc, max_tokens), dtype=torch.uint8, device=self.device)

    def set_desc(self, **kw):
        for key, v in kw.items():
            setattr(self.desc, key, v)
        need = moe_workspace_bytes(self.desc, self.max_tokens)
        if need > self.ws.numel():
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)

    def forward_prefill(self, x: torch.Tensor, bias=None, y=None) -> torch.Tensor:
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.H), dtype=torch.float32, device=self.device)
        moe_forward_prefill(self.desc, self.packed, self.router_w, bias, x, T, y, self.ws)
        return y

    def forward_decode(self, x: torch.Tensor, bias=None, y=None) -> torch.Tensor:
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.H), dtype=torch.float32, device=self.device)
        moe_forward_decode(self.desc, self.packed, self.router_w, bias, x, T, y, self.ws)
        return y

    def route(self, x: torch.Tensor, bias=None) -> dict:
        T = x.shape[0]
        dev, k, E = self.device, self.k, self.E
        mt = moe_max_tiles(self.desc, T)
        r = dict(topk_ids=torch.full((T, k), -1, dtype=torch.int32, device=dev),
                 topk_weights=torch.zeros((T, k), dtype=torch.float32, device=dev),
                 expert_counts=torch.full((E,), -1, dtype=torch.int32, device=dev),
                 expert_offsets=torch.full((E + 1,), -1, dtype=torch.int32, device=dev),
                 sorted_assign=torch.full((T * k,), -1, dtype=torch.int32, device=dev),
                 tile_map=torch.full((mt, 3), -1, dtype=torch.int32, device=dev),
                 n_tiles=torch.full((1,), -1, dtype=torch.int32, device=dev))
        moe_route(self.desc, x, T, self.router_w, bias, r, self.ws)
        return r
