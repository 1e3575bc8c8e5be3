"""ctypes binding of libmoe_int4.so (include/moe.h), same names as the C ABI.

Argument marshalling only: every step of the layer runs in the HIP kernels.
Device buffers are torch tensors (torch supplies memory and streams); they
are passed as raw pointers.  Loading fails loudly if the library is missing:
there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_int4.so")

MOE_OK, MOE_EINVAL, MOE_ENOSLOT, MOE_EHIP, MOE_EUNSUPPORTED = 0, -1, -2, -3, -4

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("hidden", _i), ("inter", _i), ("n_experts", _i), ("n_groups", _i), ("topk_group", _i),
        ("top_k", _i), ("n_shared", _i), ("routed_scaling_factor", ctypes.c_float), ("top_p", ctypes.c_float),
        ("codec", _i),
    ]

    @classmethod
    def from_cfg(cls, cfg) -> "MoeConfig":
        return cls(cfg.hidden, cfg.inter, cfg.n_experts, cfg.n_groups, cfg.topk_group, cfg.top_k, cfg.n_shared,
                   float(cfg.routed_scaling_factor), float(getattr(cfg, "top_p", 1.0)),
                   CODECS[getattr(cfg, "codec", "int4")])


class MoeCacheStats(ctypes.Structure):
    _fields_ = [("hits", ctypes.c_uint64), ("misses", ctypes.c_uint64), ("h2d_bytes", ctypes.c_uint64),
                ("evictions", ctypes.c_uint64), ("prefetches", ctypes.c_uint64), ("pinned", ctypes.c_uint64),
                ("prefetch_hits", ctypes.c_uint64), ("predicted_uses", ctypes.c_uint64),
                ("predicted_hits", ctypes.c_uint64)]


class MoeCacheTimeline(ctypes.Structure):
    _fields_ = [("copy_ms", ctypes.c_double), ("kernel_ms", ctypes.c_double), ("overlap_ms", ctypes.c_double),
                ("span_ms", ctypes.c_double), ("copies", ctypes.c_uint64), ("kernels", ctypes.c_uint64),
                ("truncated", ctypes.c_int)]


MOE_CODEC_INT4, MOE_CODEC_MXFP4, MOE_CODEC_INT8, MOE_CODEC_INT2 = 0, 1, 2, 3
CODECS = {"int4": MOE_CODEC_INT4, "mxfp4": MOE_CODEC_MXFP4, "int8": MOE_CODEC_INT8, "int2": MOE_CODEC_INT2}


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moe error {code}: {msg}")
        self.code = code


_lib = None

_SIGNATURES = {
    "moe_last_error": ([], ctypes.c_char_p),
    "moe_expert_bytes": ([ctypes.POINTER(MoeConfig)], _sz),
    "moe_expert_pack": ([ctypes.POINTER(MoeConfig)] + [_vp] * 7, _i),
    "moe_workspace_bytes": ([ctypes.POINTER(MoeConfig), _i], _sz),
    "moe_layer_create": ([ctypes.POINTER(MoeConfig), _vp, _vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp)], _i),
    "moe_layer_set_workspace": ([_vp, _vp, _sz, _i], _i),
    "moe_layer_set_experts": ([_vp, ctypes.POINTER(_vp)], _i),
    "moe_layer_destroy": ([_vp], None),
    "moe_router_topk": ([_vp, _vp, _i, _vp, _vp, _vp], _i),
    "moe_layer_forward": ([_vp, _vp, _i, _vp, _vp, _vp, _vp], _i),
    "moe_layer_forward_noalloc": ([_vp, _vp, _i, _vp, _vp, _vp, _vp], _i),
    "moe_layer_profile": ([_vp, _i], _i),
    "moe_layer_set_decode": ([_vp, _i, ctypes.c_uint], _i),
    "moe_layer_profile_read": ([_vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_uint64)], _i),
    "moe_dispatch": ([_vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp], _i),
    "moe_hbm_read_probe": ([_vp, _sz, _vp, _i, _vp], _i),
    "expert_cache_create": ([ctypes.POINTER(MoeConfig), _i, _i, _vp, _sz, _vp, ctypes.POINTER(_vp)], _i),
    "expert_cache_register": ([_vp, _i, _i, _vp, _sz], _i),
    "expert_cache_prefetch": ([_vp, _i, _vp, _i], _i),
    "expert_cache_evict": ([_vp, _i, _i], _i),
    "expert_cache_stats": ([_vp, _i, ctypes.POINTER(MoeCacheStats)], _i),
    "expert_cache_destroy": ([_vp], None),
    "moe_layer_attach_cache": ([_vp, _vp, _i], _i),
    "expert_cache_usage": ([_vp, _i, _vp], _i),
    "expert_cache_pin": ([_vp, _i, _vp, _i], _i),
    "expert_cache_unpin": ([_vp, _i, _vp, _i], _i),
    "expert_cache_autopin": ([_vp, _i, _i], _i),
    "expert_cache_replay": ([_i, _i, _i, _vp, _i, _vp, _i, ctypes.POINTER(ctypes.c_uint64),
                             ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64)], _i),
    "moe_layer_set_next": ([_vp, _vp, _i], _i),
    "expert_cache_replay_prefetch": ([_i, _i, _i, _vp, _vp, _i, _i, _vp, _i, ctypes.POINTER(ctypes.c_uint64)], _i),
    "expert_cache_timeline": ([_vp, _i, _i], _i),
    "expert_cache_timeline_read": ([_vp, ctypes.POINTER(MoeCacheTimeline)], _i),
}


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m routed_expert_int4_amd.build` "
                               "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def last_error() -> str:
    return lib().moe_last_error().decode()


def check(code: int) -> None:
    if code != MOE_OK:
        raise MoeError(code, last_error())


def _ptr(t) -> int | None:
    """Raw address of a torch tensor / numpy array / int address (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream_handle(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ----------------------------------------------------------------- 1:1 wrappers
def moe_expert_bytes(cfg) -> int:
    c = MoeConfig.from_cfg(cfg)
    return lib().moe_expert_bytes(ctypes.byref(c))


def moe_expert_pack(cfg, gate_q, gate_s, up_q, up_s, down_q, down_s, dst: np.ndarray) -> None:
    c = MoeConfig.from_cfg(cfg)
    arrs = [np.ascontiguousarray(a) for a in (gate_q, gate_s, up_q, up_s, down_q, down_s)]
    assert dst.flags["C_CONTIGUOUS"] and dst.nbytes >= moe_expert_bytes(cfg)
    check(lib().moe_expert_pack(ctypes.byref(c), *[a.ctypes.data for a in arrs], dst.ctypes.data))


def moe_workspace_bytes(cfg, max_T: int) -> int:
    c = MoeConfig.from_cfg(cfg)
    return lib().moe_workspace_bytes(ctypes.byref(c), int(max_T))


def moe_layer_create(cfg, d_router_w, d_bias, d_shared_blobs) -> int:
    c = MoeConfig.from_cfg(cfg)
    arr = (_vp * max(1, len(d_shared_blobs)))(*[_ptr(b) for b in d_shared_blobs])
    out = _vp()
    check(lib().moe_layer_create(ctypes.byref(c), _ptr(d_router_w), _ptr(d_bias), arr, ctypes.byref(out)))
    return out.value


def moe_layer_set_workspace(layer: int, d_ws, nbytes: int, max_T: int) -> None:
    check(lib().moe_layer_set_workspace(layer, _ptr(d_ws), int(nbytes), int(max_T)))


def moe_layer_set_experts(layer: int, d_blobs) -> None:
    arr = (_vp * len(d_blobs))(*[_ptr(b) for b in d_blobs])
    check(lib().moe_layer_set_experts(layer, arr))


def moe_layer_destroy(layer: int) -> None:
    lib().moe_layer_destroy(layer)


def moe_router_topk(layer: int, d_x, T: int, d_ids, d_w, stream=None) -> None:
    check(lib().moe_router_topk(layer, _ptr(d_x), int(T), _ptr(d_ids), _ptr(d_w), _stream_handle(stream)))


def moe_layer_forward(layer: int, d_x, T: int, d_y, d_ids=None, d_w=None, stream=None) -> None:
    check(lib().moe_layer_forward(layer, _ptr(d_x), int(T), _ptr(d_y), _ptr(d_ids), _ptr(d_w),
                                  _stream_handle(stream)))


def moe_layer_forward_noalloc(layer: int, d_x, T: int, d_y, d_ids=None, d_w=None, stream=None) -> None:
    check(lib().moe_layer_forward_noalloc(layer, _ptr(d_x), int(T), _ptr(d_y), _ptr(d_ids), _ptr(d_w),
                                          _stream_handle(stream)))


def moe_dispatch(layer: int, d_ids, T: int, d_counts, d_offsets, d_perm, d_distinct, d_n_distinct,
                 stream=None) -> None:
    check(lib().moe_dispatch(layer, _ptr(d_ids), int(T), _ptr(d_counts), _ptr(d_offsets), _ptr(d_perm),
                             _ptr(d_distinct), _ptr(d_n_distinct), _stream_handle(stream)))


def moe_hbm_read_probe(d_buf, nbytes: int, d_sink, blocks: int, stream=None) -> None:
    check(lib().moe_hbm_read_probe(_ptr(d_buf), int(nbytes), _ptr(d_sink), int(blocks), _stream_handle(stream)))


def moe_layer_profile(layer: int, enable: bool) -> None:
    check(lib().moe_layer_profile(layer, 1 if enable else 0))


def moe_layer_set_decode(layer: int, launches: int, spin_limit: int = 0) -> None:
    check(lib().moe_layer_set_decode(layer, int(launches), int(spin_limit)))


def moe_layer_profile_read(layer: int):
    """-> (total_ms[9], launches[9]) for router, gate/up + SwiGLU, down + combine, fused one-token launch,
    batched grouped gate/up kernel, batched grouped down kernel, batched gate/up and down of single-entry
    experts, one-token gate/up + down launch."""
    ms = (ctypes.c_double * 9)()
    n = (ctypes.c_uint64 * 9)()
    check(lib().moe_layer_profile_read(layer, ms, n))
    return [float(v) for v in ms], [int(v) for v in n]


def expert_cache_create(cfg, n_layers: int, slots_per_layer: int, d_pool, pool_bytes: int, copy_stream) -> int:
    c = MoeConfig.from_cfg(cfg)
    out = _vp()
    check(lib().expert_cache_create(ctypes.byref(c), int(n_layers), int(slots_per_layer), _ptr(d_pool),
                                    int(pool_bytes), _stream_handle(copy_stream), ctypes.byref(out)))
    return out.value


def expert_cache_register(cache: int, layer: int, expert: int, h_pinned_blob, nbytes: int) -> None:
    check(lib().expert_cache_register(cache, int(layer), int(expert), _ptr(h_pinned_blob), int(nbytes)))


def expert_cache_prefetch(cache: int, layer: int, experts) -> None:
    a = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
    check(lib().expert_cache_prefetch(cache, int(layer), a.ctypes.data, int(a.size)))


def expert_cache_evict(cache: int, layer: int, expert: int) -> None:
    check(lib().expert_cache_evict(cache, int(layer), int(expert)))


def expert_cache_stats(cache: int, layer: int) -> dict:
    s = MoeCacheStats()
    check(lib().expert_cache_stats(cache, int(layer), ctypes.byref(s)))
    return {k: int(getattr(s, k)) for k, _ in MoeCacheStats._fields_}


def expert_cache_usage(cache: int, layer: int, n_experts: int) -> np.ndarray:
    out = np.zeros(int(n_experts), np.uint64)
    check(lib().expert_cache_usage(cache, int(layer), out.ctypes.data))
    return out


def expert_cache_pin(cache: int, layer: int, experts) -> None:
    a = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
    check(lib().expert_cache_pin(cache, int(layer), a.ctypes.data, int(a.size)))


def expert_cache_unpin(cache: int, layer: int, experts) -> None:
    a = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
    check(lib().expert_cache_unpin(cache, int(layer), a.ctypes.data, int(a.size)))


def expert_cache_autopin(cache: int, layer: int, n: int) -> None:
    check(lib().expert_cache_autopin(cache, int(layer), int(n)))


def expert_cache_destroy(cache: int) -> None:
    lib().expert_cache_destroy(cache)


def moe_layer_attach_cache(layer: int, cache: int, layer_id: int) -> None:
    check(lib().moe_layer_attach_cache(layer, cache, int(layer_id)))


def expert_cache_replay(n_experts: int, slots: int, top_k: int, trace: np.ndarray, pinned=()):
    t = np.ascontiguousarray(trace, dtype=np.int32)
    p = np.ascontiguousarray(np.asarray(pinned, dtype=np.int32))
    h, m, e = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    check(lib().expert_cache_replay(int(n_experts), int(slots), int(top_k), t.ctypes.data, int(t.shape[0]),
                                    p.ctypes.data if p.size else None, int(p.size), ctypes.byref(h), ctypes.byref(m),
                                    ctypes.byref(e)))
    return int(h.value), int(m.value), int(e.value)


def moe_layer_set_next(layer: int, next_layer, max_prefetch: int = 0) -> None:
    check(lib().moe_layer_set_next(layer, next_layer, int(max_prefetch)))


REPLAY_PREFETCH_KEYS = ("hits", "misses", "evictions", "prefetches", "prefetch_hits", "predicted_uses",
                        "predicted_hits")


def expert_cache_replay_prefetch(n_experts: int, slots: int, top_k: int, trace: np.ndarray, predicted: np.ndarray,
                                 max_prefetch: int = 0, pinned=()) -> dict:
    t = np.ascontiguousarray(trace, dtype=np.int32)
    q = np.ascontiguousarray(predicted, dtype=np.int32)
    assert t.shape == q.shape
    p = np.ascontiguousarray(np.asarray(pinned, dtype=np.int32))
    out = (ctypes.c_uint64 * 7)()
    check(lib().expert_cache_replay_prefetch(int(n_experts), int(slots), int(top_k), t.ctypes.data, q.ctypes.data,
                                             int(t.shape[0]), int(max_prefetch), p.ctypes.data if p.size else None,
                                             int(p.size), out))
    return {k: int(out[i]) for i, k in enumerate(REPLAY_PREFETCH_KEYS)}


def expert_cache_timeline(cache: int, enable: bool, max_marks: int = 0) -> None:
    check(lib().expert_cache_timeline(cache, int(bool(enable)), int(max_marks)))


def expert_cache_timeline_read(cache: int) -> dict:
    t = MoeCacheTimeline()
    check(lib().expert_cache_timeline_read(cache, ctypes.byref(t)))
    return {k: (float(getattr(t, k)) if k.endswith("_ms") else int(getattr(t, k))) for k, _ in MoeCacheTimeline._fields_}
