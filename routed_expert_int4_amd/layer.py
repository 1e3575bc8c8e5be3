"""A layer on the GPU: packs and uploads expert blobs into torch device memory
and calls the C ABI.  Marshalling only; the computation is in the kernels."""
from __future__ import annotations

import numpy as np

from . import binding as B


def pack_expert(weights, e: int, out: np.ndarray | None = None) -> np.ndarray:
    """Packed device blob of expert e (routed 0..E-1, shared at E..)."""
    nb = B.moe_expert_bytes(weights.cfg)
    if out is None:
        out = np.empty(nb, np.uint8)
    B.moe_expert_pack(weights.cfg, *weights.expert_arrays(e), out)
    return out


def _hip_runtime():
    """The HIP runtime library (for exact-size pinned host allocations)."""
    import ctypes
    global _HIP
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
        _HIP.hipHostMalloc.restype = ctypes.c_int
        _HIP.hipHostFree.argtypes = [ctypes.c_void_p]
        _HIP.hipHostFree.restype = ctypes.c_int
    return _HIP


_HIP = None


class HostExpertStore:
    """Packed blobs of one layer's routed experts in pinned host memory
    [E, expert_bytes], the store an expert cache copies from.  Allocated
    with hipHostMalloc at its exact size (a caching pinned allocator would
    round each multi-GB store up to a power of two)."""

    def __init__(self, weights):
        import ctypes

        cfg = weights.cfg
        self.nb = nb = B.moe_expert_bytes(cfg)
        self.n = cfg.n_experts
        ptr = ctypes.c_void_p()
        rc = _hip_runtime().hipHostMalloc(ctypes.byref(ptr), self.n * nb, 0)
        if rc != 0 or not ptr.value:
            raise MemoryError(f"hipHostMalloc of {self.n * nb} bytes failed (error {rc})")
        self.base = ptr.value
        view = np.ctypeslib.as_array((ctypes.c_uint8 * (self.n * nb)).from_address(self.base)).reshape(self.n, nb)
        for e in range(cfg.n_experts):
            pack_expert(weights, e, view[e])

    def ptr(self, e: int) -> int:
        return self.base + e * self.nb

    def close(self) -> None:
        if getattr(self, "base", None):
            _hip_runtime().hipHostFree(self.base)
            self.base = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class ExpertCache:
    """Device slot pool, copy stream and the library's cache handle for
    n_layers layers of one shape."""

    def __init__(self, cfg, n_layers: int, slots: int, device: str = "cuda:0"):
        import torch

        self.cfg = cfg
        self.n_layers, self.slots = n_layers, slots
        self.nb = nb = B.moe_expert_bytes(cfg)
        self.pool = torch.empty(n_layers * slots * nb, dtype=torch.uint8, device=device)
        self.copy_stream = torch.cuda.Stream(device=device)
        self.handle = B.expert_cache_create(cfg, n_layers, slots, self.pool, self.pool.numel(), self.copy_stream)
        self.stores = {}

    def register(self, layer: int, store: HostExpertStore) -> None:
        for e in range(self.cfg.n_experts):
            B.expert_cache_register(self.handle, layer, e, store.ptr(e), store.nb)
        self.stores[layer] = store  # keeps the pinned blobs alive

    def prefetch(self, layer: int, experts) -> None:
        B.expert_cache_prefetch(self.handle, layer, experts)

    def evict(self, layer: int, expert: int) -> None:
        B.expert_cache_evict(self.handle, layer, expert)

    def stats(self, layer: int) -> dict:
        return B.expert_cache_stats(self.handle, layer)

    def usage(self, layer: int):
        return B.expert_cache_usage(self.handle, layer, self.cfg.n_experts)

    def pin(self, layer: int, experts) -> None:
        B.expert_cache_pin(self.handle, layer, experts)

    def unpin(self, layer: int, experts) -> None:
        B.expert_cache_unpin(self.handle, layer, experts)

    def autopin(self, layer: int, n: int) -> None:
        B.expert_cache_autopin(self.handle, layer, n)

    def timeline(self, enable: bool, max_marks: int = 0) -> None:
        B.expert_cache_timeline(self.handle, enable, max_marks)

    def timeline_read(self) -> dict:
        return B.expert_cache_timeline_read(self.handle)

    def close(self) -> None:
        if getattr(self, "handle", None):
            B.expert_cache_destroy(self.handle)
            self.handle = None
        for store in self.stores.values():
            store.close()
        self.stores = {}

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DeviceLayer:
    """One MoE layer on the GPU.

    With resident=True every expert blob lives in one device tensor
    [E + S, expert_bytes] (rows stay 256-byte aligned because expert_bytes is
    a multiple of 256).  With resident=False only the shared expert(s) are
    uploaded and the routed experts come from an attached ExpertCache."""

    def __init__(self, weights, max_T: int = 1, device: str = "cuda:0", resident: bool = True):
        import torch

        cfg = weights.cfg
        self.cfg = cfg
        self.device = device
        self.expert_bytes = nb = B.moe_expert_bytes(cfg)
        if nb == 0:
            raise B.MoeError(B.MOE_EINVAL, B.last_error())
        first = 0 if resident else cfg.n_experts
        n_all = cfg.n_total_experts
        self.blobs = torch.empty((cfg.n_experts if resident else 0) + cfg.n_shared, nb, dtype=torch.uint8,
                                 device=device)
        host = np.empty(nb, np.uint8)
        for e in range(first, n_all):
            pack_expert(weights, e, host)
            self.blobs[e - first].copy_(torch.from_numpy(host))
        self.router_w = torch.from_numpy(np.ascontiguousarray(weights.router_w)).to(device)
        self.bias = torch.from_numpy(np.ascontiguousarray(weights.bias)).to(device)
        shared = [self.blobs[cfg.n_experts - first + s] for s in range(cfg.n_shared)]
        self.handle = B.moe_layer_create(cfg, self.router_w, self.bias, shared)
        self.max_T = max_T
        self.ws_bytes = B.moe_workspace_bytes(cfg, max_T)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        torch.cuda.synchronize(device)
        B.moe_layer_set_workspace(self.handle, self.ws, self.ws_bytes, max_T)
        if resident:
            B.moe_layer_set_experts(self.handle, [self.blobs[e] for e in range(cfg.n_experts)])

    def attach_cache(self, cache: "ExpertCache", layer_id: int) -> None:
        B.moe_layer_attach_cache(self.handle, cache.handle, layer_id)
        self.cache = cache  # the cache outlives the layer's use of it

    def set_next(self, next_layer: "DeviceLayer | None", max_prefetch: int = 0) -> None:
        """Speculative prefetch of next_layer's experts on this layer's input
        (None: off)."""
        B.moe_layer_set_next(self.handle, next_layer.handle if next_layer is not None else None, max_prefetch)
        self.next_layer = next_layer  # kept alive while linked

    def close(self):
        if getattr(self, "handle", None):
            B.moe_layer_destroy(self.handle)
            self.handle = None
        self.next_layer = None

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

    def forward_each(self, x, y=None, ids=None, w=None, stream=None):
        """Like forward, as T separate one-token calls (the decode path):
        token t's call reads x[t] and writes y[t], ids[t], w[t]."""
        import torch
        T, H, k = x.shape[0], self.cfg.hidden, self.cfg.top_k
        if y is None:
            y = torch.empty((T, H), dtype=torch.float32, device=self.device)
        if ids is None:
            ids = torch.empty((T, k), dtype=torch.int32, device=self.device)
        if w is None:
            w = torch.empty((T, k), dtype=torch.float32, device=self.device)
        px, py, pi, pw = x.data_ptr(), y.data_ptr(), ids.data_ptr(), w.data_ptr()
        st = B._stream_handle(stream)
        for t in range(T):
            B.moe_layer_forward(self.handle, px + 2 * H * t, 1, py + 4 * H * t, pi + 4 * k * t, pw + 4 * k * t, st)
        return y, ids, w

    def router_topk(self, x, stream=None):
        import torch
        T = x.shape[0]
        ids = torch.empty((T, self.cfg.top_k), dtype=torch.int32, device=self.device)
        w = torch.empty((T, self.cfg.top_k), dtype=torch.float32, device=self.device)
        B.moe_router_topk(self.handle, x, T, ids, w, stream)
        return ids, w
