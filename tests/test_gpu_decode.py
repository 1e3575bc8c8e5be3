"""GPU parity of the decode path (one-token calls) with the oracle.

Every GPU test calls the library through the C ABI (ctypes binding) and
compares element by element with the fp64 CPU oracle on the same seeded
inputs: routed ids bit-exact unless the oracle's selection gap is below 1e-6
(then the outputs are checked against the oracle forced onto the GPU's ids),
weights within 1e-6 * rsf, outputs within 2e-3 * max|ref| per token.
"""
import dataclasses
import sys

import numpy as np
import pytest

from oracle import oracle
from routed_expert_int4_amd import binding as B
from routed_expert_int4_amd import synth
from tests.helpers import MID_A, MID_B, MID_C, MID_D, check_layer, check_routing

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()  # fails loudly if the HIP library is missing
    return torch


def run_layer(torch, weights, x_bits, max_T=None):
    from routed_expert_int4_amd.layer import DeviceLayer
    T = x_bits.shape[0]
    layer = DeviceLayer(weights, max_T=max_T or max(T, 1))
    x = DeviceLayer.to_device_bf16(x_bits)
    y, ids, w = layer.forward_each(x)
    torch.cuda.synchronize()
    return layer, y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("cfg_name", ["TINY", "MID_A", "MID_B", "MID_C", "MID_D"])
def test_layer_parity(torch_cuda, cfg_name):
    cfg = {"TINY": synth.TINY, "MID_A": MID_A, "MID_B": MID_B, "MID_C": MID_C, "MID_D": MID_D}[cfg_name]
    say(f"[gpu] layer parity {cfg_name} {cfg}")
    weights = synth.gen_layer(cfg, seed=0)
    T = 4 if cfg.hidden * cfg.inter > 2 ** 24 else 13
    x = synth.gen_tokens(cfg, T, seed=1)
    layer, y, ids, w = run_layer(torch_cuda, weights, x)
    res = check_layer(weights, x, y, ids, w)
    say(f"[gpu] {cfg_name}: worst rel err {res['worst_rel']:.3g}, excused {res['excused']}")
    layer.close()


def test_tiny_router_topk_matches_oracle(torch_cuda):
    say("[gpu] tiny router_topk")
    weights = synth.gen_layer(synth.TINY, seed=0)
    x = synth.gen_tokens(synth.TINY, 64, seed=2)
    from routed_expert_int4_amd.layer import DeviceLayer
    layer = DeviceLayer(weights, max_T=64)
    ids, w = layer.router_topk(DeviceLayer.to_device_bf16(x))
    torch_cuda.cuda.synchronize()
    ids_ref, w_ref, gap = oracle.route(weights, x)
    check_routing(synth.TINY, ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, gap)
    layer.close()


@pytest.mark.parametrize("std", [1e-3, 1.0, 300.0])
def test_activation_scale_range(torch_cuda, std):
    """Inputs far from unit scale keep full accuracy (power-of-two range scaling)."""
    say(f"[gpu] tiny activation std {std}")
    weights = synth.gen_layer(synth.TINY, seed=0)
    x = synth.gen_tokens(synth.TINY, 8, seed=3, std=std)
    layer, y, ids, w = run_layer(torch_cuda, weights, x)
    check_layer(weights, x, y, ids, w)
    layer.close()


def test_zero_input_gives_shared_only_output(torch_cuda):
    """x = 0: weights rsf/k exactly, routing on the bias alone, y = 0."""
    say("[gpu] tiny zero input")
    weights = synth.gen_layer(synth.TINY, seed=0)
    x = np.zeros((3, synth.TINY.hidden), np.uint16)
    layer, y, ids, w = run_layer(torch_cuda, weights, x)
    ref_ids, _, _ = oracle.route(weights, x)
    np.testing.assert_array_equal(ids, ref_ids)
    assert np.all(w == np.float32(synth.TINY.routed_scaling_factor / synth.TINY.top_k))
    assert np.all(y == 0.0)
    layer.close()


def test_routed_off_gives_shared_expert(torch_cuda):
    say("[gpu] tiny routed experts zeroed")
    w0 = synth.gen_layer(synth.TINY, seed=0)
    E = synth.TINY.n_experts
    wz = dataclasses.replace(w0, gate_q=w0.gate_q.copy(), up_q=w0.up_q.copy(), down_q=w0.down_q.copy())
    wz.gate_q[:E] = 0
    wz.up_q[:E] = 0
    wz.down_q[:E] = 0
    x = synth.gen_tokens(synth.TINY, 5, seed=4)
    layer, y, ids, w = run_layer(torch_cuda, wz, x)
    check_layer(wz, x, y, ids, w)
    layer.close()


def test_empty_call_and_errors(torch_cuda):
    say("[gpu] T=0 and argument errors")
    weights = synth.gen_layer(synth.TINY, seed=0)
    from routed_expert_int4_amd.layer import DeviceLayer
    layer = DeviceLayer(weights, max_T=2)
    x = DeviceLayer.to_device_bf16(synth.gen_tokens(synth.TINY, 3, seed=1))
    y = torch_cuda.full((3, synth.TINY.hidden), 7.0, device="cuda:0")
    B.moe_layer_forward(layer.handle, x, 0, y)
    torch_cuda.cuda.synchronize()
    assert torch_cuda.all(y == 7.0)
    with pytest.raises(B.MoeError) as e:
        B.moe_layer_forward(layer.handle, x, 3, y)  # T above max_T
    assert e.value.code == B.MOE_EINVAL and "max_T" in B.last_error()
    with pytest.raises(B.MoeError):
        B.moe_layer_forward(layer.handle, None, 1, y)
    layer.close()


def test_repeatable_and_batch_independent(torch_cuda):
    """Two runs are bit-identical; a token's result does not depend on the
    other tokens of the call."""
    say("[gpu] determinism / batch independence")
    weights = synth.gen_layer(MID_A, seed=0)
    x = synth.gen_tokens(MID_A, 9, seed=5)
    layer, y1, ids1, w1 = run_layer(torch_cuda, weights, x)
    from routed_expert_int4_amd.layer import DeviceLayer
    y2, ids2, w2 = layer.forward_each(DeviceLayer.to_device_bf16(x))
    np.testing.assert_array_equal(y1, y2.cpu().numpy())
    np.testing.assert_array_equal(ids1, ids2.cpu().numpy())
    for t in (0, 4, 8):
        y3, _, _ = layer.forward(DeviceLayer.to_device_bf16(x[t:t + 1]))
        np.testing.assert_array_equal(y1[t], y3.cpu().numpy()[0])
    layer.close()


# ---------------------------------------------------------------- GLM-5.2 shape
@pytest.fixture(scope="module")
def glm(torch_cuda):
    say("[gpu] generating the GLM-shaped layer (seed 0)")
    weights = synth.gen_layer(synth.GLM, seed=0)
    from routed_expert_int4_amd.layer import DeviceLayer
    layer = DeviceLayer(weights, max_T=1)
    yield weights, layer
    layer.close()


def test_glm_decode_1000_tokens(torch_cuda, glm):
    """The benchmark's workload: 1,000 independent tokens at batch 1.  Routing
    of all 1,000 tokens against the oracle; full outputs on a sample of tokens
    (the first, the last, a spread, and the smallest-gap ones)."""
    weights, layer = glm
    say("[gpu] GLM 1000-token decode")
    x = synth.gen_tokens(synth.GLM, 1000, seed=1)
    from routed_expert_int4_amd.layer import DeviceLayer
    y, ids, w = layer.forward_each(DeviceLayer.to_device_bf16(x))
    torch_cuda.cuda.synchronize()
    y, ids, w = y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    ids_ref, w_ref, gap = oracle.route(weights, x)
    excused = check_routing(synth.GLM, ids, w, ids_ref, w_ref, gap)
    say(f"[gpu] GLM routing: {len(excused)} tokens excused by the 1e-6 gap rule, min gap {gap.min():.3g}")
    np.testing.assert_allclose(w.sum(axis=1), synth.GLM.routed_scaling_factor, rtol=1e-6)
    rows = sorted(set([0, 1, 137, 500, 998, 999] + list(np.argsort(gap)[:2])))
    res = check_layer(weights, x, y, ids, w, rows=rows)
    say(f"[gpu] GLM sampled outputs: worst rel err {res['worst_rel']:.3g}")
    assert np.all(np.isfinite(y))


def test_glm_zero_token_and_repeat(torch_cuda, glm):
    weights, layer = glm
    say("[gpu] GLM zero token + repeat")
    x = synth.gen_tokens(synth.GLM, 3, seed=7)
    x[1] = 0
    from routed_expert_int4_amd.layer import DeviceLayer
    xd = DeviceLayer.to_device_bf16(x)
    y1, ids1, w1 = layer.forward_each(xd)
    y2, ids2, w2 = layer.forward_each(xd)
    torch_cuda.cuda.synchronize()
    assert torch_cuda.equal(y1, y2) and torch_cuda.equal(ids1, ids2)
    y1 = y1.cpu().numpy()
    assert np.all(y1[1] == 0.0)
    assert np.all(w1.cpu().numpy()[1] == np.float32(synth.GLM.routed_scaling_factor / synth.GLM.top_k))
    check_layer(weights, x, y1, ids1.cpu().numpy(), w1.cpu().numpy(), rows=[0, 2])


# ---------------------------------------------------------------- adaptive top-p
def with_top_p(weights, top_p):
    return dataclasses.replace(weights, cfg=dataclasses.replace(weights.cfg, top_p=top_p))


@pytest.mark.parametrize("cfg_name,top_p", [("TINY", 0.5), ("MID_A", 0.8), ("MID_B", 0.6), ("MID_D", 0.3)])
def test_top_p_layer_parity(torch_cuda, cfg_name, top_p):
    """One-token calls with the top-p cut: ids (-1 where dropped), weights
    and outputs against the oracle; tokens whose top-p margin is below 1e-6
    are excused and re-checked with the oracle forced onto the GPU's ids."""
    cfg = {"TINY": synth.TINY, "MID_A": MID_A, "MID_B": MID_B, "MID_D": MID_D}[cfg_name]
    say(f"[gpu] top-p {top_p} layer parity {cfg_name}")
    weights = with_top_p(synth.gen_layer(cfg, seed=0), top_p)
    x = synth.gen_tokens(cfg, 13, seed=2)
    layer, y, ids, w = run_layer(torch_cuda, weights, x)
    res = check_layer(weights, x, y, ids, w)
    dropped = int((ids < 0).sum())
    say(f"[gpu] {cfg_name} top-p {top_p}: dropped {dropped} of {ids.size} choices, "
        f"worst rel err {res['worst_rel']:.3g}, excused {res['excused']}")
    assert dropped > 0, "the cut dropped nothing: the case does not exercise top-p"
    assert np.all(w[ids < 0] == 0.0)
    kept = ids >= 0
    np.testing.assert_allclose((w * kept).sum(axis=1), cfg.routed_scaling_factor, rtol=1e-6)
    layer.close()


def test_top_p_tiny_cut_keeps_one_expert(torch_cuda):
    """top_p far below every share: only the choice with the largest
    affinity survives, with the whole weight rsf."""
    cfg = MID_A
    say("[gpu] top-p 1e-4 keeps the top expert")
    weights = with_top_p(synth.gen_layer(cfg, seed=0), 1e-4)
    x = synth.gen_tokens(cfg, 5, seed=3)
    layer, y, ids, w = run_layer(torch_cuda, weights, x)
    assert np.all((ids >= 0).sum(axis=1) == 1)
    np.testing.assert_allclose(w.max(axis=1), cfg.routed_scaling_factor, rtol=1e-6)
    check_layer(weights, x, y, ids, w)
    layer.close()


def test_top_p_one_is_plain_top_k(torch_cuda):
    """top_p = 1 routes and computes exactly as the plain top-k layer."""
    say("[gpu] top-p 1.0 equals plain top-k")
    base = synth.gen_layer(MID_A, seed=0)
    x = synth.gen_tokens(MID_A, 6, seed=4)
    l1, y1, ids1, w1 = run_layer(torch_cuda, base, x)
    l2, y2, ids2, w2 = run_layer(torch_cuda, with_top_p(base, 1.0), x)
    np.testing.assert_array_equal(ids1, ids2)
    np.testing.assert_array_equal(w1, w2)
    np.testing.assert_array_equal(y1, y2)
    l1.close()
    l2.close()


def test_glm_top_p_decode(torch_cuda, glm):
    """GLM-shaped layer, top_p 0.7, 200 one-token calls: routing of every
    token against the oracle, outputs on a sample."""
    weights, _ = glm
    say("[gpu] GLM top-p 0.7 decode, 200 tokens")
    from routed_expert_int4_amd.layer import DeviceLayer
    wp = with_top_p(weights, 0.7)
    layer = DeviceLayer(wp, max_T=1)
    x = synth.gen_tokens(synth.GLM, 200, seed=9)
    y, ids, w = layer.forward_each(DeviceLayer.to_device_bf16(x))
    torch_cuda.cuda.synchronize()
    y, ids, w = y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    ids_ref, w_ref, gap, pgap = oracle.route(wp, x, with_pgap=True)
    excused = check_routing(wp.cfg, ids, w, ids_ref, w_ref, gap, pgap)
    kept = (ids >= 0).sum(axis=1)
    say(f"[gpu] GLM top-p: kept {kept.mean():.2f} of 8 experts per token, {len(excused)} excused")
    assert kept.min() >= 1 and kept.mean() < 8
    rows = sorted(set([0, 1, 99, 199] + list(np.argsort(np.minimum(gap, pgap))[:2])))
    res = check_layer(wp, x, y, ids, w, rows=rows)
    say(f"[gpu] GLM top-p sampled outputs: worst rel err {res['worst_rel']:.3g}")
    layer.close()


# ---------------------------------------------------------------- MXFP4 codec
def with_codec(cfg, codec="mxfp4"):
    return dataclasses.replace(cfg, codec=codec)


@pytest.mark.parametrize("codec", ["mxfp4", "int8", "int2"])
@pytest.mark.parametrize("cfg_name", ["TINY", "MID_A", "MID_B", "MID_C", "MID_D"])
def test_codec_layer_parity(torch_cuda, cfg_name, codec):
    """One-token calls of MXFP4 (E2M1 codes, E8M0 scales), int8 and int2
    layers against the oracle, every lane mapping of the kernels."""
    cfg = with_codec({"TINY": synth.TINY, "MID_A": MID_A, "MID_B": MID_B, "MID_C": MID_C, "MID_D": MID_D}[cfg_name],
                     codec)
    say(f"[gpu] {codec} layer parity {cfg_name}")
    weights = synth.gen_layer(cfg, seed=0)
    T = 4 if cfg.hidden * cfg.inter > 2 ** 24 else 13
    x = synth.gen_tokens(cfg, T, seed=1)
    layer, y, ids, w = run_layer(torch_cuda, weights, x)
    res = check_layer(weights, x, y, ids, w)
    say(f"[gpu] {codec} {cfg_name}: worst rel err {res['worst_rel']:.3g}, excused {res['excused']}")
    layer.close()


def test_mxfp4_extreme_scales_and_activations(torch_cuda):
    """E8M0 bytes far from the generator's range (2^-40 .. 2^-20 and 2^+10 ..
    2^+20 per group) with activations of std 1e-3 and 300: the fp16
    activation pairs and the scale decoding keep the outputs within
    tolerance."""
    cfg = with_codec(MID_A)
    say("[gpu] mxfp4 extreme scales")
    base = synth.gen_layer(cfg, seed=2)
    rng = np.random.default_rng(7)
    for lo, hi in ((127 - 40, 127 - 20), (127 + 10, 127 + 20)):
        arrs = {n: rng.integers(lo, hi, size=getattr(base, n).shape).astype(np.uint8)
                for n in ("gate_s", "up_s", "down_s")}
        weights = dataclasses.replace(base, **arrs)
        for std in (1e-3, 300.0):
            x = synth.gen_tokens(cfg, 3, seed=8, std=std)
            layer, y, ids, w = run_layer(torch_cuda, weights, x)
            res = check_layer(weights, x, y, ids, w)
            say(f"[gpu] mxfp4 scales [{lo}, {hi}) std {std}: worst rel err {res['worst_rel']:.3g}")
            layer.close()


@pytest.mark.parametrize("codec", ["int2"])
def test_codec_batched_call_runs_per_token(torch_cuda, codec):
    """A T > 1 call of an int2 layer whose inter is not a multiple of 256
    runs as T one-token passes: bit-identical to T separate calls, and
    within the oracle's tolerance."""
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = with_codec(synth.TINY, codec)
    weights = synth.gen_layer(cfg, seed=0)
    layer = DeviceLayer(weights, max_T=5)
    xb = synth.gen_tokens(cfg, 5, seed=1)
    x = DeviceLayer.to_device_bf16(xb)
    y, ids, w = layer.forward(x)
    y1, ids1, w1 = layer.forward_each(x)
    torch_cuda.cuda.synchronize()
    assert torch_cuda.equal(y, y1) and torch_cuda.equal(ids, ids1) and torch_cuda.equal(w, w1)
    check_layer(weights, xb, y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy())
    layer.close()


def test_glm_mxfp4_decode(torch_cuda):
    """GLM-shaped MXFP4 layer (19.125 MiB per expert), 300 one-token calls:
    routing of every token against the oracle, outputs on a sample; then the
    same layer with top_p 0.7."""
    cfg = with_codec(synth.GLM)
    say("[gpu] generating the GLM-shaped MXFP4 layer (seed 0)")
    weights = synth.gen_layer(cfg, seed=0)
    from routed_expert_int4_amd.layer import DeviceLayer
    assert B.moe_expert_bytes(cfg) == 20_054_016
    layer = DeviceLayer(weights, max_T=1)
    x = synth.gen_tokens(cfg, 300, seed=1)
    y, ids, w = layer.forward_each(DeviceLayer.to_device_bf16(x))
    torch_cuda.cuda.synchronize()
    y, ids, w = y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    ids_ref, w_ref, gap = oracle.route(weights, x)
    excused = check_routing(cfg, ids, w, ids_ref, w_ref, gap)
    rows = sorted(set([0, 1, 150, 299] + list(np.argsort(gap)[:2])))
    res = check_layer(weights, x, y, ids, w, rows=rows)
    say(f"[gpu] GLM mxfp4: {len(excused)} excused, sampled worst rel err {res['worst_rel']:.3g}")
    layer.close()
    wp = with_top_p(weights, 0.7)
    layer = DeviceLayer(wp, max_T=1)
    y, ids, w = layer.forward_each(DeviceLayer.to_device_bf16(x[:40]))
    torch_cuda.cuda.synchronize()
    res = check_layer(wp, x[:40], y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), rows=[0, 7, 39])
    say(f"[gpu] GLM mxfp4 top-p 0.7: worst rel err {res['worst_rel']:.3g}")
    layer.close()


def test_int8_extreme_codes_and_activations(torch_cuda):
    """Int8 codes at -128 and 127 over whole rows and activations of std 1e-3
    and 300 stay within tolerance (the two nibble planes recombine exactly)."""
    cfg = with_codec(MID_A, "int8")
    say("[gpu] int8 extreme codes")
    base = synth.gen_layer(cfg, seed=3)
    gq = base.gate_q.copy()
    gq[:, 0::3, :] = 0x80  # -128
    gq[:, 1::3, :] = 0x7F  # 127
    dq = base.down_q.copy()
    dq[:, 0::2, :] = 0x80
    weights = dataclasses.replace(base, gate_q=gq, down_q=dq)
    for std in (1e-3, 300.0):
        x = synth.gen_tokens(cfg, 3, seed=11, std=std)
        layer, y, ids, w = run_layer(torch_cuda, weights, x)
        res = check_layer(weights, x, y, ids, w)
        say(f"[gpu] int8 extremes std {std}: worst rel err {res['worst_rel']:.3g}")
        layer.close()


def test_glm_int8_decode(torch_cuda):
    """GLM-shaped int8 layer (twice the int4 code bytes), 200 one-token
    calls: routing of every token and sampled outputs against the oracle."""
    cfg = with_codec(synth.GLM, "int8")
    say("[gpu] generating the GLM-shaped int8 layer (seed 0)")
    weights = synth.gen_layer(cfg, seed=0)
    from routed_expert_int4_amd.layer import DeviceLayer
    layer = DeviceLayer(weights, max_T=1)
    x = synth.gen_tokens(cfg, 200, seed=1)
    y, ids, w = layer.forward_each(DeviceLayer.to_device_bf16(x))
    torch_cuda.cuda.synchronize()
    y, ids, w = y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    ids_ref, w_ref, gap = oracle.route(weights, x)
    excused = check_routing(cfg, ids, w, ids_ref, w_ref, gap)
    rows = sorted(set([0, 1, 100, 199] + list(np.argsort(gap)[:2])))
    res = check_layer(weights, x, y, ids, w, rows=rows)
    say(f"[gpu] GLM int8: {len(excused)} excused, sampled worst rel err {res['worst_rel']:.3g}")
    layer.close()


def test_glm_int2_decode(torch_cuda):
    """GLM-shaped int2 layer (half the int4 code bytes, two rows per stored
    row), 200 one-token calls: routing and sampled outputs against the oracle;
    then top_p 0.7 on the same layer."""
    cfg = with_codec(synth.GLM, "int2")
    say("[gpu] generating the GLM-shaped int2 layer (seed 0)")
    weights = synth.gen_layer(cfg, seed=0)
    from routed_expert_int4_amd.layer import DeviceLayer
    layer = DeviceLayer(weights, max_T=1)
    x = synth.gen_tokens(cfg, 200, seed=1)
    y, ids, w = layer.forward_each(DeviceLayer.to_device_bf16(x))
    torch_cuda.cuda.synchronize()
    y, ids, w = y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    ids_ref, w_ref, gap = oracle.route(weights, x)
    excused = check_routing(cfg, ids, w, ids_ref, w_ref, gap)
    rows = sorted(set([0, 1, 100, 199] + list(np.argsort(gap)[:2])))
    res = check_layer(weights, x, y, ids, w, rows=rows)
    say(f"[gpu] GLM int2: {len(excused)} excused, sampled worst rel err {res['worst_rel']:.3g}")
    layer.close()
    wp = with_top_p(weights, 0.7)
    layer = DeviceLayer(wp, max_T=1)
    y, ids, w = layer.forward_each(DeviceLayer.to_device_bf16(x[:30]))
    torch_cuda.cuda.synchronize()
    res = check_layer(wp, x[:30], y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy(), rows=[0, 29])
    say(f"[gpu] GLM int2 top-p 0.7: worst rel err {res['worst_rel']:.3g}")
    layer.close()


# ---------------------------------------------------------------- degenerate configurations
DEGENERATE = {
    # no shared expert
    "no_shared": synth.LayerConfig(hidden=1024, inter=256, n_experts=64, n_groups=8, topk_group=4, top_k=6,
                                   n_shared=0, routed_scaling_factor=1.5),
    # one group, one expert per token, no shared expert
    "top1_one_group": synth.LayerConfig(hidden=256, inter=128, n_experts=16, n_groups=1, topk_group=1, top_k=1,
                                        n_shared=0),
    # every group kept (group limit inactive), top-8 of 32
    "all_groups": synth.LayerConfig(hidden=512, inter=128, n_experts=32, n_groups=4, topk_group=4, top_k=8),
}


@pytest.mark.parametrize("name", sorted(DEGENERATE))
def test_degenerate_configs_decode(torch_cuda, name):
    cfg = DEGENERATE[name]
    say(f"[gpu] degenerate decode {name}")
    weights = synth.gen_layer(cfg, seed=5)
    x = synth.gen_tokens(cfg, 9, seed=6)
    layer, y, ids, w = run_layer(torch_cuda, weights, x)
    res = check_layer(weights, x, y, ids, w)
    np.testing.assert_allclose(w.sum(axis=1), cfg.routed_scaling_factor, rtol=1e-6)
    say(f"[gpu] {name}: worst rel err {res['worst_rel']:.3g}")
    layer.close()


# ---------------------------------------------------------------- outliers inside a scale group
def with_group_outliers(cfg, x_bits, seed, lo=1e3, hi=1e4):
    """x with one element of every 32-input group set to a factor drawn
    log-uniformly from [lo, hi] times the group's largest magnitude (sign
    kept), rounded to bf16: the
    decode kernels round each group to 16-bit integers relative to the
    group's largest element, so the other 31 lose the most bits here."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = synth.bf16_bits_to_f32(x_bits).copy()
    T, H = x.shape
    pos = rng.integers(0, 32, size=(T, H // 32)) + 32 * np.arange(H // 32)[None, :]
    fac = np.exp(rng.uniform(np.log(lo), np.log(hi), size=(T, H // 32))).astype(np.float32)
    rows = np.arange(T)[:, None]
    gmax = np.abs(x).reshape(T, H // 32, 32).max(axis=2)
    x[rows, pos] = np.where(x[rows, pos] < 0, -1.0, 1.0) * fac * gmax
    return synth.round_to_bf16_bits(x)


def with_heavy_tailed_h(weights, factor=1000.0, seed=0):
    """Up-projection scales of one row in every 32 rows (per expert) raised by
    `factor`, so that h = silu(g) * u has one element per 32-group of the
    down projection's input about `factor` times the others."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cfg = weights.cfg
    us = weights.up_s.copy()
    f = us.view(np.float16).astype(np.float32)
    n_all, I = f.shape[0], f.shape[1]
    rows = rng.integers(0, 32, size=(n_all, I // 32)) + 32 * np.arange(I // 32)[None, :]
    for e in range(n_all):
        f[e, rows[e], :] *= factor
    assert np.all(np.isfinite(f.astype(np.float16)))
    return dataclasses.replace(weights, up_s=f.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("cfg_name", ["TINY", "MID_A", "MID_C"])
def test_activation_outlier_in_every_group(torch_cuda, cfg_name):
    """One activation per 32-group 1e3..1e4 times the others: decode and
    batched outputs within 2e-3 of the oracle per token."""
    cfg = {"TINY": synth.TINY, "MID_A": MID_A, "MID_C": MID_C}[cfg_name]
    say(f"[gpu] activation outliers in every group, {cfg_name}")
    weights = synth.gen_layer(cfg, seed=0)
    T = 4 if cfg.hidden * cfg.inter > 2 ** 24 else 12
    x = with_group_outliers(cfg, synth.gen_tokens(cfg, T, seed=11), seed=12)
    layer, y, ids, w = run_layer(torch_cuda, weights, x)
    res = check_layer(weights, x, y, ids, w)
    from routed_expert_int4_amd.layer import DeviceLayer
    yb, idb, wb = layer.forward(DeviceLayer.to_device_bf16(x))
    torch_cuda.cuda.synchronize()
    resb = check_layer(weights, x, yb.cpu().numpy(), idb.cpu().numpy(), wb.cpu().numpy())
    say(f"[gpu] {cfg_name} outliers: decode worst rel err {res['worst_rel']:.3g}, batched {resb['worst_rel']:.3g}")
    layer.close()


@pytest.mark.parametrize("cfg_name", ["TINY", "MID_A", "MID_B"])
def test_heavy_tailed_h(torch_cuda, cfg_name):
    """Expert weights that make h heavy-tailed (one element per 32-group of
    the down projection's input ~1000 times the rest): decode and batched
    outputs within 2e-3 of the oracle per token."""
    cfg = {"TINY": synth.TINY, "MID_A": MID_A, "MID_B": MID_B}[cfg_name]
    say(f"[gpu] heavy-tailed h, {cfg_name}")
    weights = with_heavy_tailed_h(synth.gen_layer(cfg, seed=0), seed=13)
    x = synth.gen_tokens(cfg, 10, seed=14)
    layer, y, ids, w = run_layer(torch_cuda, weights, x)
    res = check_layer(weights, x, y, ids, w)
    from routed_expert_int4_amd.layer import DeviceLayer
    yb, idb, wb = layer.forward(DeviceLayer.to_device_bf16(x))
    torch_cuda.cuda.synchronize()
    resb = check_layer(weights, x, yb.cpu().numpy(), idb.cpu().numpy(), wb.cpu().numpy())
    say(f"[gpu] {cfg_name} heavy-tailed h: decode worst rel err {res['worst_rel']:.3g}, "
        f"batched {resb['worst_rel']:.3g}")
    layer.close()


def test_glm_activation_outliers(torch_cuda, glm):
    """GLM-shaped layer, outliers in every activation group, 3 tokens."""
    weights, layer = glm
    say("[gpu] GLM activation outliers")
    x = with_group_outliers(synth.GLM, synth.gen_tokens(synth.GLM, 3, seed=15), seed=16)
    from routed_expert_int4_amd.layer import DeviceLayer
    y, ids, w = layer.forward_each(DeviceLayer.to_device_bf16(x))
    torch_cuda.cuda.synchronize()
    res = check_layer(weights, x, y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy())
    say(f"[gpu] GLM outliers: worst rel err {res['worst_rel']:.3g}")
