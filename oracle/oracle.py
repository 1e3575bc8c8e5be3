"""ctypes wrapper of the CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg.  The GPU library never imports it.  It takes the
public-layout arrays produced by ``routed_expert_int4_amd.synth`` and returns
fp64 results.  See moe_oracle.c for what is computed and which page passage
each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_d = ctypes.POINTER(ctypes.c_double)
_i32 = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p


def build() -> str:
    """Compile the oracle with gcc (-O2 -fopenmp, no fast-math)."""
    subprocess.run(["sh", os.path.join(_HERE, "build.sh")], check=True)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(
            os.path.join(_HERE, "moe_oracle.c")
        ):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_expert_ffn.argtypes = [ctypes.c_int] * 3 + [_vp] * 6 + [_d, _d, _d]
        L.oracle_expert_ffn.restype = None
        L.oracle_matvec.argtypes = [ctypes.c_int, _vp, _vp, ctypes.c_int, ctypes.c_int, _d, _d]
        L.oracle_matvec.restype = None
        L.oracle_router_scores.argtypes = [ctypes.c_int, ctypes.c_int, _vp, _vp, _d, _d, _d, _d]
        L.oracle_router_scores.restype = None
        L.oracle_select.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double, ctypes.c_double, _d, _d, _i32, _d, _d, _d]
        L.oracle_select.restype = ctypes.c_int
        L.oracle_layer_forward.argtypes = (
            [ctypes.c_int] * 8 + [ctypes.c_double, ctypes.c_double, _vp, _vp] + [_vp] * 6
            + [_vp, ctypes.c_int, _vp, _d, _i32, _d, _d, _d, _vp, ctypes.c_int]
        )
        L.oracle_layer_forward.restype = ctypes.c_int
        L.oracle_route.argtypes = [ctypes.c_int] * 5 + [ctypes.c_double, ctypes.c_double, _vp, _vp, _vp, ctypes.c_int,
                                                         _i32, _d, _d, _d, ctypes.c_int]
        L.oracle_route.restype = ctypes.c_int
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _dptr(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_d)


def max_threads() -> int:
    return lib().oracle_max_threads()


CODECS = {"int4": 0, "mxfp4": 1, "int8": 2, "int2": 3}
CODES_PER_BYTE = {"int4": 2, "mxfp4": 2, "int8": 1, "int2": 4}


def _scale_dtype(codec: str):
    return np.uint8 if codec == "mxfp4" else np.uint16


def expert_ffn(hidden, inter, gate_q, gate_s, up_q, up_s, down_q, down_s, x: np.ndarray, codec: str = "int4"):
    """One expert on one fp64 token vector x[hidden] -> (d[hidden], h[inter])."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    d = np.empty(hidden, np.float64)
    h = np.empty(inter, np.float64)
    arrs = [np.ascontiguousarray(a) for a in (gate_q, gate_s, up_q, up_s, down_q, down_s)]
    for a in arrs[1::2]:
        assert a.dtype == _scale_dtype(codec), "scale dtype does not match the codec"
    lib().oracle_expert_ffn(CODECS[codec], hidden, inter, *[_ptr(a) for a in arrs], _dptr(x), _dptr(d), _dptr(h))
    return d, h


def matvec(q: np.ndarray, s: np.ndarray, x: np.ndarray, codec: str = "int4") -> np.ndarray:
    """y = W x for one quantised matrix: codes q [rows, cols/codes per byte],
    scales s [rows, cols/32] (fp16 bits for int4, int8 and int2, E8M0 bytes
    for mxfp4)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=_scale_dtype(codec))
    rows, cols = q.shape[0], CODES_PER_BYTE[codec] * q.shape[1]
    assert s.shape == (rows, cols // 32)
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(rows, np.float64)
    lib().oracle_matvec(CODECS[codec], _ptr(q), _ptr(s), rows, cols, _dptr(x), _dptr(y))
    return y


def router_scores(router_w: np.ndarray, bias: np.ndarray, x: np.ndarray):
    """(logit, s, sb) of one fp64 token vector."""
    e, hidden = router_w.shape
    rw = np.ascontiguousarray(router_w, dtype=np.float32)
    b = np.ascontiguousarray(bias, dtype=np.float32)
    x = np.ascontiguousarray(x, dtype=np.float64)
    lg, s, sb = (np.empty(e, np.float64) for _ in range(3))
    lib().oracle_router_scores(hidden, e, _ptr(rw), _ptr(b), _dptr(x), _dptr(lg), _dptr(s), _dptr(sb))
    return lg, s, sb


def select(n_groups, topk_group, top_k, rsf, s: np.ndarray, sb: np.ndarray, top_p: float = 1.0,
           with_pgap: bool = False):
    """Group-limited top-k of one token (adaptive top-p when top_p < 1) ->
    (ids, w, gap) or, with with_pgap, (ids, w, gap, pgap)."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    sb = np.ascontiguousarray(sb, dtype=np.float64)
    ids = np.empty(top_k, np.int32)
    w = np.empty(top_k, np.float64)
    gap = np.empty(1, np.float64)
    pgap = np.empty(1, np.float64)
    rc = lib().oracle_select(
        len(s), n_groups, topk_group, top_k, float(rsf), float(top_p), _dptr(s), _dptr(sb),
        ids.ctypes.data_as(_i32), _dptr(w), _dptr(gap), _dptr(pgap),
    )
    if rc != 0:
        raise ValueError("oracle_select: inconsistent arguments")
    if with_pgap:
        return ids, w, float(gap[0]), float(pgap[0])
    return ids, w, float(gap[0])


def layer_forward(weights, x_bf16: np.ndarray, forced_ids=None, n_threads: int = 0, want_logits=False):
    """Full layer on tokens x_bf16 [T, H] (bf16 bits).

    Returns dict(y [T,H] f64, ids [T,k] i32 (-1: slot dropped by top-p),
    w [T,k] f64, gap [T] f64, pgap [T] f64 (top-p decision margin, inf
    without top-p), logits [T,E] f64 or None)."""
    cfg = weights.cfg
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    T = x.shape[0]
    k = cfg.top_k
    y = np.empty((T, cfg.hidden), np.float64)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    gap = np.empty(T, np.float64)
    pgap = np.empty(T, np.float64)
    logits = np.empty((T, cfg.n_experts), np.float64) if want_logits else None
    fid = None
    if forced_ids is not None:
        fid = np.ascontiguousarray(forced_ids, dtype=np.int32)
        assert fid.shape == (T, k)
    wt = weights
    codec = getattr(cfg, "codec", "int4")
    for a in (weights.gate_s, weights.up_s, weights.down_s):
        assert a.dtype == _scale_dtype(codec), "scale dtype does not match the codec"
    rc = lib().oracle_layer_forward(
        CODECS[codec], cfg.hidden, cfg.inter, cfg.n_experts, cfg.n_groups, cfg.topk_group, k, cfg.n_shared,
        float(cfg.routed_scaling_factor), float(getattr(cfg, "top_p", 1.0)),
        _ptr(wt.router_w), _ptr(wt.bias),
        _ptr(wt.gate_q), _ptr(wt.gate_s), _ptr(wt.up_q), _ptr(wt.up_s), _ptr(wt.down_q), _ptr(wt.down_s),
        _ptr(x), T, _ptr(fid) if fid is not None else None,
        _dptr(y), ids.ctypes.data_as(_i32), _dptr(w), _dptr(gap), _dptr(pgap),
        logits.ctypes.data_as(ctypes.c_void_p) if logits is not None else None,
        int(n_threads),
    )
    if rc != 0:
        raise ValueError("oracle_layer_forward: bad arguments")
    return {"y": y, "ids": ids, "w": w, "gap": gap, "pgap": pgap, "logits": logits}


def route(weights, x_bf16: np.ndarray, n_threads: int = 0, with_pgap: bool = False):
    """Router + selection for tokens x_bf16 [T, H] -> (ids [T,k], w [T,k], gap [T])
    or, with with_pgap, (ids, w, gap, pgap [T])."""
    cfg = weights.cfg
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    T = x.shape[0]
    ids = np.empty((T, cfg.top_k), np.int32)
    w = np.empty((T, cfg.top_k), np.float64)
    gap = np.empty(T, np.float64)
    pgap = np.empty(T, np.float64)
    rc = lib().oracle_route(
        cfg.hidden, cfg.n_experts, cfg.n_groups, cfg.topk_group, cfg.top_k, float(cfg.routed_scaling_factor),
        float(getattr(cfg, "top_p", 1.0)), _ptr(weights.router_w), _ptr(weights.bias), _ptr(x), T,
        ids.ctypes.data_as(_i32), _dptr(w), _dptr(gap), _dptr(pgap), int(n_threads))
    if rc != 0:
        raise ValueError("oracle_route: bad arguments")
    if with_pgap:
        return ids, w, gap, pgap
    return ids, w, gap
