"""GPU tests of the one-token decode launches with in-kernel hand-offs:
the fused launch (moe_layer_set_decode(layer, 1)) and the router launch
followed by one gate/up + down launch (moe_layer_set_decode(layer, 2)).

The fused launch runs the router, the group-limited top-k, the shared and
routed gate/up, the down projections and the combine of one token in one
kernel on co-resident workgroups (hand-offs inside the kernel).  It computes
every step exactly as the three-launch path does, so through the C ABI:
  * outputs, ids and weights bit-identical to the three launches
    (the default) on every shape with a fused instance,
    and within tolerance of the fp64 oracle;
  * the per-kind launch counts show which path ran (kind 3 = fused);
  * the top-p cut (dropped slots read nothing) and zero inputs;
  * a wait that gives up (forced from the host with a spin limit of one
    poll) is reported as MOE_EHIP by the next call, every kernel having
    finished normally, and binding the workspace again clears it.
"""
import dataclasses
import sys

import numpy as np
import pytest

from routed_expert_int4_amd import binding as B
from routed_expert_int4_amd import synth
from tests.helpers import MID_A, MID_B, MID_C, MID_D, check_layer

pytestmark = pytest.mark.gpu

SHAPES = {"TINY": synth.TINY, "MID_A": MID_A, "MID_B": MID_B, "MID_D": MID_D, "GLM": synth.GLM}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    return torch


def run_both(torch, layer, x):
    """One-token calls with the fused launch and with three launches (the
    default); returns both results and the launch counts per kind."""
    B.moe_layer_set_decode(layer.handle, 1)
    B.moe_layer_profile(layer.handle, True)
    y1, ids1, w1 = layer.forward_each(x)
    torch.cuda.synchronize()
    _, n1 = B.moe_layer_profile_read(layer.handle)
    B.moe_layer_profile(layer.handle, False)
    B.moe_layer_set_decode(layer.handle, 3)
    B.moe_layer_profile(layer.handle, True)
    y3, ids3, w3 = layer.forward_each(x)
    torch.cuda.synchronize()
    _, n3 = B.moe_layer_profile_read(layer.handle)
    B.moe_layer_profile(layer.handle, False)
    return (y1, ids1, w1, n1), (y3, ids3, w3, n3)


@pytest.mark.parametrize("cfg_name", list(SHAPES))
def test_fused_matches_three_launches(torch_cuda, cfg_name):
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = SHAPES[cfg_name]
    say(f"[gpu] fused decode vs three launches, {cfg_name}")
    weights = synth.gen_layer(cfg, seed=0)
    T = 24
    x_bits = synth.gen_tokens(cfg, T, seed=31)
    x_bits[5] = 0  # a zero token: routing on the bias alone, y = 0
    layer = DeviceLayer(weights, max_T=1)
    x = DeviceLayer.to_device_bf16(x_bits)
    (y1, ids1, w1, n1), (y3, ids3, w3, n3) = run_both(torch, layer, x)
    say(f"[gpu] {cfg_name}: launches fused path {n1}, three-launch path {n3}")
    assert n1[3] == T and n1[:3] == [0, 0, 0], "the fused launch did not run"
    assert n3[3] == 0 and n3[:3] == [T, T, T] and n1[4:] == n3[4:] == [0, 0, 0, 0, 0]
    assert torch.equal(ids1, ids3) and torch.equal(w1, w3), "routing differs between the paths"
    assert torch.equal(y1, y3), "outputs differ between the fused and the three-launch path"
    assert torch.all(y1[5] == 0.0)
    rows = list(range(T)) if cfg.hidden * cfg.inter <= 2 ** 24 else [0, 1, 5, 11, 23]
    res = check_layer(weights, x_bits, y1.cpu().numpy(), ids1.cpu().numpy(), w1.cpu().numpy(), rows=rows)
    say(f"[gpu] {cfg_name}: bit-identical, oracle worst rel err {res['worst_rel']:.3g}")
    layer.close()


@pytest.mark.parametrize("cfg_name,top_p", [("MID_A", 0.6), ("GLM", 0.7)])
def test_fused_top_p(torch_cuda, cfg_name, top_p):
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = dataclasses.replace(SHAPES[cfg_name], top_p=top_p)
    say(f"[gpu] fused decode with top-p {top_p}, {cfg_name}")
    weights = synth.gen_layer(cfg, seed=0)
    T = 16
    x_bits = synth.gen_tokens(cfg, T, seed=32)
    layer = DeviceLayer(weights, max_T=1)
    x = DeviceLayer.to_device_bf16(x_bits)
    (y1, ids1, w1, n1), (y3, ids3, w3, n3) = run_both(torch, layer, x)
    assert n1[3] == T
    assert torch.equal(ids1, ids3) and torch.equal(w1, w3) and torch.equal(y1, y3)
    idh = ids1.cpu().numpy()
    assert (idh < 0).any(), "the cut dropped nothing"
    rows = list(range(T)) if cfg.hidden * cfg.inter <= 2 ** 24 else [0, 7, 15]
    res = check_layer(weights, x_bits, y1.cpu().numpy(), idh, w1.cpu().numpy(), rows=rows)
    say(f"[gpu] {cfg_name} top-p: kept {(idh >= 0).sum(1).mean():.2f} per token, rel err {res['worst_rel']:.3g}")
    layer.close()


def test_fused_falls_back_without_instance(torch_cuda):
    """A shape without a fused instance runs the three launches even when
    the fused launch is asked for."""
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    weights = synth.gen_layer(MID_C, seed=0)
    x_bits = synth.gen_tokens(MID_C, 2, seed=33)
    layer = DeviceLayer(weights, max_T=1)
    B.moe_layer_set_decode(layer.handle, 1)
    B.moe_layer_profile(layer.handle, True)
    y, ids, w = layer.forward_each(DeviceLayer.to_device_bf16(x_bits))
    torch.cuda.synchronize()
    _, n = B.moe_layer_profile_read(layer.handle)
    B.moe_layer_profile(layer.handle, False)
    assert n == [2, 2, 2, 0, 0, 0, 0, 0, 0]
    check_layer(weights, x_bits, y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy())
    layer.close()


def test_fused_wait_that_gives_up_is_reported(torch_cuda):
    """With a spin limit of one poll the in-kernel waits give up (the kernel
    still finishes); the next call returns MOE_EHIP, and binding the
    workspace again restores results bit-identical to the three launches'."""
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = MID_B
    say("[gpu] fused decode: a wait that gives up")
    weights = synth.gen_layer(cfg, seed=0)
    x_bits = synth.gen_tokens(cfg, 4, seed=34)
    layer = DeviceLayer(weights, max_T=1)
    x = DeviceLayer.to_device_bf16(x_bits)
    y_ref, ids_ref, w_ref = layer.forward_each(x)
    torch.cuda.synchronize()
    B.moe_layer_set_decode(layer.handle, 1, 1)
    y = torch.empty_like(y_ref)
    ids = torch.empty_like(ids_ref)
    w = torch.empty_like(w_ref)
    B.moe_layer_forward(layer.handle, x[0:1], 1, y[0:1], ids[0:1], w[0:1])
    torch.cuda.synchronize()
    with pytest.raises(B.MoeError) as err:
        B.moe_layer_forward(layer.handle, x[1:2], 1, y[1:2], ids[1:2], w[1:2])
    assert err.value.code == B.MOE_EHIP and "gave up" in B.last_error()
    # rebinding the workspace clears the counters and the status word
    B.moe_layer_set_decode(layer.handle, 1, 0)
    B.moe_layer_set_workspace(layer.handle, layer.ws, layer.ws_bytes, 1)
    y2, ids2, w2 = layer.forward_each(x)
    torch.cuda.synchronize()
    assert torch.equal(y2, y_ref) and torch.equal(ids2, ids_ref) and torch.equal(w2, w_ref)
    layer.close()


def run_mode(torch, layer, x, launches, spin_limit=0):
    """One-token calls of every token of x with the given decode mode;
    returns y, ids, w and the launch counts per kind."""
    B.moe_layer_set_decode(layer.handle, launches, spin_limit)
    B.moe_layer_profile(layer.handle, True)
    y, ids, w = layer.forward_each(x)
    torch.cuda.synchronize()
    _, n = B.moe_layer_profile_read(layer.handle)
    B.moe_layer_profile(layer.handle, False)
    return y, ids, w, n


@pytest.mark.parametrize("cfg_name", list(SHAPES))
def test_gateup_down_matches_three_launches(torch_cuda, cfg_name):
    """The router launch plus one gate/up + down launch gives outputs, ids
    and weights bit-identical to the three launches, within tolerance of the
    oracle; switching between the modes keeps the in-kernel counters
    consistent."""
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = SHAPES[cfg_name]
    say(f"[gpu] gate/up + down launch vs three launches, {cfg_name}")
    weights = synth.gen_layer(cfg, seed=0)
    T = 24
    x_bits = synth.gen_tokens(cfg, T, seed=35)
    x_bits[7] = 0  # a zero token: routing on the bias alone, y = 0
    layer = DeviceLayer(weights, max_T=1)
    x = DeviceLayer.to_device_bf16(x_bits)
    y2, ids2, w2, n2 = run_mode(torch, layer, x, 2)
    y3, ids3, w3, n3 = run_mode(torch, layer, x, 3)
    y2b, ids2b, w2b, n2b = run_mode(torch, layer, x, 2)
    say(f"[gpu] {cfg_name}: launches two-launch path {n2}, three-launch path {n3}")
    assert n2 == n2b == [T, 0, 0, 0, 0, 0, 0, 0, T], "the gate/up + down launch did not run"
    assert n3 == [T, T, T, 0, 0, 0, 0, 0, 0]
    assert torch.equal(ids2, ids3) and torch.equal(w2, w3), "routing differs between the paths"
    assert torch.equal(y2, y3), "outputs differ between the two-launch and the three-launch path"
    assert torch.equal(y2b, y2) and torch.equal(ids2b, ids2) and torch.equal(w2b, w2)
    assert torch.all(y2[7] == 0.0)
    rows = list(range(T)) if cfg.hidden * cfg.inter <= 2 ** 24 else [0, 1, 7, 12, 23]
    res = check_layer(weights, x_bits, y2.cpu().numpy(), ids2.cpu().numpy(), w2.cpu().numpy(), rows=rows)
    say(f"[gpu] {cfg_name}: bit-identical, oracle worst rel err {res['worst_rel']:.3g}")
    layer.close()


@pytest.mark.parametrize("cfg_name,top_p", [("MID_A", 0.6), ("GLM", 0.7)])
def test_gateup_down_top_p(torch_cuda, cfg_name, top_p):
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = dataclasses.replace(SHAPES[cfg_name], top_p=top_p)
    say(f"[gpu] gate/up + down launch with top-p {top_p}, {cfg_name}")
    weights = synth.gen_layer(cfg, seed=0)
    T = 16
    x_bits = synth.gen_tokens(cfg, T, seed=36)
    layer = DeviceLayer(weights, max_T=1)
    x = DeviceLayer.to_device_bf16(x_bits)
    y2, ids2, w2, n2 = run_mode(torch, layer, x, 2)
    y3, ids3, w3, n3 = run_mode(torch, layer, x, 3)
    assert n2[8] == T and n2[1:3] == [0, 0]
    assert torch.equal(ids2, ids3) and torch.equal(w2, w3) and torch.equal(y2, y3)
    idh = ids2.cpu().numpy()
    assert (idh < 0).any(), "the cut dropped nothing"
    rows = list(range(T)) if cfg.hidden * cfg.inter <= 2 ** 24 else [0, 7, 15]
    res = check_layer(weights, x_bits, y2.cpu().numpy(), idh, w2.cpu().numpy(), rows=rows)
    say(f"[gpu] {cfg_name} top-p: kept {(idh >= 0).sum(1).mean():.2f} per token, rel err {res['worst_rel']:.3g}")
    layer.close()


def test_gateup_down_falls_back_without_instance(torch_cuda):
    """A shape or codec without a gate/up + down instance runs the three
    launches when the two are asked for."""
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    for cfg in (MID_C, dataclasses.replace(MID_A, codec="int8")):
        weights = synth.gen_layer(cfg, seed=0)
        x_bits = synth.gen_tokens(cfg, 2, seed=37)
        layer = DeviceLayer(weights, max_T=1)
        y, ids, w, n = run_mode(torch, layer, DeviceLayer.to_device_bf16(x_bits), 2)
        assert n == [2, 2, 2, 0, 0, 0, 0, 0, 0]
        check_layer(weights, x_bits, y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy())
        layer.close()


def test_gateup_down_wait_that_gives_up_is_reported(torch_cuda):
    """With a spin limit of one poll the in-kernel wait of the gate/up +
    down launch gives up (every kernel still finishes); the next call
    returns MOE_EHIP, and binding the workspace again restores results
    bit-identical to the three launches'."""
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = MID_B
    say("[gpu] gate/up + down launch: a wait that gives up")
    weights = synth.gen_layer(cfg, seed=0)
    x_bits = synth.gen_tokens(cfg, 4, seed=38)
    layer = DeviceLayer(weights, max_T=1)
    x = DeviceLayer.to_device_bf16(x_bits)
    y_ref, ids_ref, w_ref, _ = run_mode(torch, layer, x, 3)
    B.moe_layer_set_decode(layer.handle, 2, 1)
    y = torch.empty_like(y_ref)
    ids = torch.empty_like(ids_ref)
    w = torch.empty_like(w_ref)
    B.moe_layer_forward(layer.handle, x[0:1], 1, y[0:1], ids[0:1], w[0:1])
    torch.cuda.synchronize()
    with pytest.raises(B.MoeError) as err:
        B.moe_layer_forward(layer.handle, x[1:2], 1, y[1:2], ids[1:2], w[1:2])
    assert err.value.code == B.MOE_EHIP and "gave up" in B.last_error()
    B.moe_layer_set_decode(layer.handle, 2, 0)
    B.moe_layer_set_workspace(layer.handle, layer.ws, layer.ws_bytes, 1)
    y2, ids2, w2 = layer.forward_each(x)
    torch.cuda.synchronize()
    assert torch.equal(y2, y_ref) and torch.equal(ids2, ids_ref) and torch.equal(w2, w_ref)
    layer.close()
