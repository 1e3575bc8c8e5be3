"""Seeded synthetic inputs for the routed int4 MoE layer.

This module draws random numbers and rounds them to the storage formats of the
public weight layout; it contains none of the layer's arithmetic (no routing,
no dequantisation, no expert math). Both the CPU oracle and the GPU path
consume exactly the arrays produced here.

Public layout of one layer (row-major, little-endian):

* ``router_w``  float32 ``[E, H]``
* ``bias``      float32 ``[E]`` (the expert-score correction bias)
* per expert ``e`` in ``0..E-1`` followed by the shared expert(s) at index ``E``:
  ``gate_q`` uint8 ``[I, H/2]``, ``gate_s`` float16 bits ``[I, H/32]``,
  ``up_q``/``up_s`` likewise, ``down_q`` uint8 ``[H, I/2]``, ``down_s`` float16
  bits ``[H, I/32]``.  A code byte holds two int4 values in two's complement,
  the even column in the low nibble; one scale covers 32 consecutive input
  columns.
* activations: bfloat16 bits ``[T, H]``.

With ``codec="mxfp4"`` the codes are MXFP4 elements (E2M1 nibbles, same
packing) and every scale array is uint8 E8M0 bytes (one per 32 inputs).
With ``codec="int8"`` every code is one two's complement byte (code arrays
``[I, H]`` and ``[H, I]``) with the same fp16 scales; with ``codec="int2"``
a byte holds four two's complement 2-bit codes, column 4j + t in bits
[2t, 2t + 2) of byte j (code arrays ``[I, H/4]`` and ``[H, I/4]``).

Value distributions follow the GLM-5.2-shaped layer described on the pages
(routed experts 256, top-8, ~19 MB of int4 codes per expert): codes are uniform
random bytes (so both nibbles are independent and uniform over [-8, 7]),
scales are exp(N(-4, 0.5)) rounded to fp16, the router weight is N(0, 0.02) in
fp32, the bias N(0, 0.01) in fp32 and the activations N(0, 1) rounded to bf16.
MXFP4 layers draw their codes the same way (uniform bytes: every E2M1 code
equally likely, rms element 2.93) and E8M0 scale bytes 127 + round(N(-5, 0.75))
(about 2^-5, so the weights have the int4 layer's magnitude).  Int8 layers
draw uniform code bytes and scales exp(N(-6.77, 0.5)) (the int4 scale times
4.64 / 73.9, the ratio of the codes' rms values); int2 layers uniform code
bytes and scales exp(N(-2.66, 0.5)) (ratio 4.64 / 1.22).
Streams: SeedSequence(seed).spawn(1 + E + S); the first child draws the
router weight then the bias; child 1 + e draws expert e (routed experts
first, shared last) in the order gate codes, gate scales, up codes, up
scales, down codes, down scales.  Activations come from their own seed.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    hidden: int
    inter: int
    n_experts: int
    n_groups: int
    topk_group: int
    top_k: int
    n_shared: int = 1
    routed_scaling_factor: float = 2.5
    top_p: float = 1.0  # adaptive expert top-p over the selected experts (1: plain top-k)
    codec: str = "int4"  # "int4", "int8", "int2" (fp16 scales) or "mxfp4" (E2M1 codes, E8M0 scales)

    @property
    def n_total_experts(self) -> int:
        return self.n_experts + self.n_shared

    @property
    def scale_bytes(self) -> int:
        return 1 if self.codec == "mxfp4" else 2

    @property
    def codes_per_byte(self) -> int:
        return {"int8": 1, "int2": 4}.get(self.codec, 2)

    def expert_bytes(self) -> int:
        """Bytes of one expert in the public layout (codes + scales)."""
        h, i = self.hidden, self.inter
        return 3 * (h * i // self.codes_per_byte) + 3 * (h * i // 32) * self.scale_bytes


# Tiny layer: hidden 256, intermediate 128, 16 experts in 4 groups, top-4 of 2 groups.
TINY = LayerConfig(hidden=256, inter=128, n_experts=16, n_groups=4, topk_group=2, top_k=4)
# GLM-5.2-shaped layer: hidden 6144, intermediate 2048, 256 experts in 8 groups, top-8 of 4 groups.
GLM = LayerConfig(hidden=6144, inter=2048, n_experts=256, n_groups=8, topk_group=4, top_k=8)


@dataclasses.dataclass
class LayerWeights:
    cfg: LayerConfig
    router_w: np.ndarray  # float32 [E, H]
    bias: np.ndarray      # float32 [E]
    gate_q: np.ndarray    # uint8  [E+S, I, H/2]
    gate_s: np.ndarray    # uint16 [E+S, I, H/32] (fp16 bits; uint8 E8M0 for mxfp4)
    up_q: np.ndarray
    up_s: np.ndarray
    down_q: np.ndarray    # uint8  [E+S, H, I/2]
    down_s: np.ndarray    # uint16 [E+S, H, I/32]

    def expert_arrays(self, e: int):
        return (self.gate_q[e], self.gate_s[e], self.up_q[e], self.up_s[e], self.down_q[e], self.down_s[e])


def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (storage format)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform random bytes (two independent uniform int4 codes each)."""
    n = int(np.prod(shape))
    assert n % 8 == 0
    return rng.bit_generator.random_raw(n // 8).view(np.uint8).reshape(shape)


def _scales(rng: np.random.Generator, shape) -> np.ndarray:
    """exp(N(-4, 0.5)) rounded to fp16 (bits)."""
    z = rng.standard_normal(size=shape, dtype=np.float32)
    return np.exp(z * np.float32(0.5) - np.float32(4.0)).astype(np.float16).view(np.uint16)


def _int8_scales(rng: np.random.Generator, shape) -> np.ndarray:
    """exp(N(-6.77, 0.5)) rounded to fp16 (bits)."""
    z = rng.standard_normal(size=shape, dtype=np.float32)
    return np.exp(z * np.float32(0.5) - np.float32(6.77)).astype(np.float16).view(np.uint16)


def _int2_scales(rng: np.random.Generator, shape) -> np.ndarray:
    """exp(N(-2.66, 0.5)) rounded to fp16 (bits)."""
    z = rng.standard_normal(size=shape, dtype=np.float32)
    return np.exp(z * np.float32(0.5) - np.float32(2.66)).astype(np.float16).view(np.uint16)


def _e8m0_scales(rng: np.random.Generator, shape) -> np.ndarray:
    """E8M0 bytes 127 + round(N(-5, 0.75))."""
    z = rng.standard_normal(size=shape, dtype=np.float32)
    return (np.rint(z * np.float32(0.75) - np.float32(5.0)) + 127).astype(np.uint8)


def gen_router(cfg: LayerConfig, seed: int):
    """The router weight and bias of gen_layer(cfg, seed), without the experts."""
    child = np.random.SeedSequence(seed).spawn(1 + cfg.n_total_experts)[0]
    rng = np.random.Generator(np.random.PCG64(child))
    router_w = rng.normal(0.0, 0.02, size=(cfg.n_experts, cfg.hidden)).astype(np.float32)
    bias = rng.normal(0.0, 0.01, size=(cfg.n_experts,)).astype(np.float32)
    return router_w, bias


def gen_layer(cfg: LayerConfig, seed: int, workers: int | None = None) -> LayerWeights:
    """One layer from `seed`.  SeedSequence(seed) spawns one child stream for
    the router (weight, then bias) and one per expert (routed 0..E-1, then
    shared), so experts can be drawn in parallel threads."""
    import concurrent.futures
    import os

    h, i, e_all = cfg.hidden, cfg.inter, cfg.n_total_experts
    children = np.random.SeedSequence(seed).spawn(1 + e_all)
    router_w, bias = gen_router(cfg, seed)
    sdt, scales = {"mxfp4": (np.uint8, _e8m0_scales), "int8": (np.uint16, _int8_scales),
                   "int2": (np.uint16, _int2_scales)}.get(
        cfg.codec, (np.uint16, _scales))
    cpb = cfg.codes_per_byte
    gq = np.empty((e_all, i, h // cpb), np.uint8)
    gs = np.empty((e_all, i, h // 32), sdt)
    uq = np.empty_like(gq)
    us = np.empty_like(gs)
    dq = np.empty((e_all, h, i // cpb), np.uint8)
    ds = np.empty((e_all, h, i // 32), sdt)

    def draw(e):
        r = np.random.Generator(np.random.PCG64(children[1 + e]))
        gq[e] = _codes(r, gq.shape[1:])
        gs[e] = scales(r, gs.shape[1:])
        uq[e] = _codes(r, uq.shape[1:])
        us[e] = scales(r, us.shape[1:])
        dq[e] = _codes(r, dq.shape[1:])
        ds[e] = scales(r, ds.shape[1:])

    n_workers = workers or min(16, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(max_workers=n_workers) as ex:
        list(ex.map(draw, range(e_all)))
    return LayerWeights(cfg, router_w, bias, gq, gs, uq, us, dq, ds)


def gen_tokens(cfg: LayerConfig, n_tokens: int, seed: int, std: float = 1.0) -> np.ndarray:
    """bf16 bits [T, H] of N(0, std^2) activations."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.normal(0.0, std, size=(n_tokens, cfg.hidden)).astype(np.float32)
    return round_to_bf16_bits(x)


def gen_noise(cfg: LayerConfig, n_tokens: int, seed: int, std: float) -> np.ndarray:
    """float32 [T, H] of N(0, std^2) noise (used between stacked layers)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.normal(0.0, std, size=(n_tokens, cfg.hidden)).astype(np.float32)
