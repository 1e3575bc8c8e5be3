"""A layer on the GPU: packs and uploads expert blobs into torch device memory
and calls the C ABI.  Marshalling only; the computation is in the kernels."""
from __future__ import annotations

import numpy as np

from . import binding as B


class DeviceLayer:
    """One MoE layer with every expert resident in HBM.

    Expert blobs live in one device tensor [E + S, expert_bytes] (rows stay
    256-byte aligned because expert_bytes is a multiple of 256)."""

    def __init__(self, weights, max_T: int = 1, device: str = "cuda:0"):
        import torch

        cfg = weights.cfg
        self.cfg = cfg
        self.device = device
        self.expert_bytes = nb = B.moe_expert_bytes(cfg)
        if nb == 0:
            raise B.MoeError(B.MOE_EINVAL, B.last_error())
        n_all = cfg.n_total_experts
        self.blobs = torch.empty((n_all, nb), dtype=torch.uint8, device=device)
        host = np.empty(nb, np.uint8)
        for e in range(n_all):
            B.moe_expert_pack(cfg, *weights.expert_arrays(e), host)
            self.blobs[e].copy_(torch.from_numpy(host))
        self.router_w = torch.from_numpy(np.ascontiguousarray(weights.router_w)).to(device)
        self.bias = torch.from_numpy(np.ascontiguousarray(weights.bias)).to(device)
        shared = [self.blobs[cfg.n_experts + s] for s in range(cfg.n_shared)]
        self.handle = B.moe_layer_create(cfg, self.router_w, self.bias, shared)
        self.max_T = max_T
        self.ws_bytes = B.moe_workspace_bytes(cfg, max_T)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        torch.cuda.synchronize(device)
        B.moe_layer_set_workspace(self.handle, self.ws, self.ws_bytes, max_T)
        B.moe_layer_set_experts(self.handle, [self.blobs[e] for e in range(cfg.n_experts)])

    def close(self):
        if getattr(self, "handle", None):
            B.moe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def to_device_bf16(x_bits: np.ndarray, device: str = "cuda:0"):
        import torch
        return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(device).view(torch.bfloat16)

    def forward(self, x, y=None, ids=None, w=None, stream=None):
        """x: device bf16 [T, H].  Returns (y fp32 [T,H], ids int32 [T,k], w fp32 [T,k])."""
        import torch
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.cfg.hidden), dtype=torch.float32, device=self.device)
        if ids is None:
            ids = torch.empty((T, self.cfg.top_k), dtype=torch.int32, device=self.device)
        if w is None:
            w = torch.empty((T, self.cfg.top_k), dtype=torch.float32, device=self.device)
        B.moe_layer_forward(self.handle, x, T, y, ids, w, stream)
        return y, ids, w

    def router_topk(self, x, stream=None):
        import torch
        T = x.shape[0]
        ids = torch.empty((T, self.cfg.top_k), dtype=torch.int32, device=self.device)
        w = torch.empty((T, self.cfg.top_k), dtype=torch.float32, device=self.device)
        B.moe_router_topk(self.handle, x, T, ids, w, stream)
        return ids, w
