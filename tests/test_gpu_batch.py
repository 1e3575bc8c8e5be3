"""GPU parity of the batched (batch-union) path with the oracle.

Calls with T > 1 tokens route every token, dispatch the (token, slot)
entries by expert (each distinct expert is read once per call, the colibrì
summary's batch-union rule, fr.news.hada.io topic 31297, "Principales
fonctionnalités implémentées") and run grouped gate/up and down projections
on the matrix cores.  Checked through the C ABI against the oracle:
  * the dispatch (counts, offsets, permutation, distinct experts) bit-exact
    against oracle/dispatch.py, up to the largest sort (8192 entries) and
    degenerate routings;
  * layer outputs element by element (ids bit-exact unless the oracle's gap
    is below 1e-6; outputs within 2e-3 * max|ref| per token) on every shape,
    ragged tiles, an expert taking more than one tile, zero and repeated
    tokens, launch sequences split by the sort capacity;
  * GLM-shaped calls: batch 32 under Zipf-skewed routing and a 512-token
    prefill chunk (routing of every token, outputs on samples).
"""
import sys

import numpy as np
import pytest

from oracle import oracle
from oracle.dispatch import dispatch as oracle_dispatch
from routed_expert_int4_amd import binding as B
from routed_expert_int4_amd import synth
from tests.helpers import MID_A, MID_B, MID_C, MID_D, MID_E, check_layer, check_routing, zipf_glm_weights

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    return torch


def run_batch(torch, layer, x_bits):
    from routed_expert_int4_amd.layer import DeviceLayer
    y, ids, w = layer.forward(DeviceLayer.to_device_bf16(x_bits))
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


# ---------------------------------------------------------------- dispatch
def gpu_dispatch(torch, layer, ids_np):
    T, k = ids_np.shape
    E = layer.cfg.n_experts
    dev = "cuda:0"
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(dev)
    counts = torch.full((E,), -1, dtype=torch.int32, device=dev)
    offsets = torch.full((E + 1,), -1, dtype=torch.int32, device=dev)
    perm = torch.full((max(T * k, 1),), -1, dtype=torch.int32, device=dev)
    distinct = torch.full((E,), -1, dtype=torch.int32, device=dev)
    nd = torch.full((1,), -1, dtype=torch.int32, device=dev)
    B.moe_dispatch(layer.handle, ids, T, counts, offsets, perm, distinct, nd)
    torch.cuda.synchronize()
    n = int(nd.item())
    return {"counts": counts.cpu().numpy(), "offsets": offsets.cpu().numpy(), "perm": perm.cpu().numpy()[:T * k],
            "distinct": distinct.cpu().numpy()[:n]}


@pytest.fixture(scope="module")
def dispatch_layer(torch_cuda):
    from routed_expert_int4_amd.layer import DeviceLayer
    layer = DeviceLayer(synth.gen_layer(MID_D, seed=0), max_T=1024)
    yield layer
    layer.close()


@pytest.mark.parametrize("T,kind", [(1, "uniform"), (2, "uniform"), (32, "zipf"), (37, "uniform"), (512, "uniform"),
                                    (1024, "uniform"), (1024, "zipf"), (300, "same"), (200, "dropped"),
                                    (3, "all_dropped_but_one"), (64, "out_of_range")])
def test_dispatch_matches_oracle(torch_cuda, dispatch_layer, T, kind):
    say(f"[gpu] dispatch T={T} {kind}")
    E, k = MID_D.n_experts, MID_D.top_k
    rng = np.random.default_rng(T)
    if kind == "same":
        ids = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    elif kind == "zipf":
        p = np.arange(1, E + 1, dtype=np.float64) ** -1.1
        ids = np.stack([rng.choice(E, k, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    else:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    if kind == "dropped":  # choices dropped by a top-p cut carry id -1
        ids[rng.random(ids.shape) < 0.3] = -1
    if kind == "all_dropped_but_one":
        ids[:, 1:] = -1
    ref_ids = ids
    if kind == "out_of_range":  # ids outside [-1, E) take no entry, as -1 does
        ids = ids.copy()
        ids[rng.random(ids.shape) < 0.2] = E
        ids[rng.random(ids.shape) < 0.1] = -7
        ref_ids = np.where((ids >= 0) & (ids < E), ids, -1).astype(np.int32)
    got = gpu_dispatch(torch_cuda, dispatch_layer, ids)
    ref = oracle_dispatch(ref_ids, E)
    for key in ("counts", "offsets", "perm", "distinct"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)


def test_dispatch_errors(torch_cuda, dispatch_layer):
    ids = torch_cuda.zeros((2000, MID_D.top_k), dtype=torch_cuda.int32, device="cuda:0")
    z = torch_cuda.zeros(300, dtype=torch_cuda.int32, device="cuda:0")
    with pytest.raises(B.MoeError):  # above the workspace's batch
        B.moe_dispatch(dispatch_layer.handle, ids, 2000, z, z, z, z, z)
    with pytest.raises(B.MoeError):
        B.moe_dispatch(dispatch_layer.handle, ids, 4, None, z, z, z, z)
    B.moe_dispatch(dispatch_layer.handle, ids, 0, z, z, z, z, z)  # T = 0: no-op


# ---------------------------------------------------------------- layer
@pytest.mark.parametrize("cfg_name,T", [("TINY", 4), ("TINY", 2), ("MID_A", 37), ("MID_B", 16), ("MID_C", 5),
                                        ("MID_D", 100), ("MID_E", 70), ("MID_E", 130)])
def test_batch_layer_parity(torch_cuda, cfg_name, T):
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = {"TINY": synth.TINY, "MID_A": MID_A, "MID_B": MID_B, "MID_C": MID_C, "MID_D": MID_D,
           "MID_E": MID_E}[cfg_name]
    say(f"[gpu] batched parity {cfg_name} T={T}")
    weights = synth.gen_layer(cfg, seed=0)
    x = synth.gen_tokens(cfg, T, seed=11)
    layer = DeviceLayer(weights, max_T=T)
    y, ids, w = run_batch(torch_cuda, layer, x)
    res = check_layer(weights, x, y, ids, w)
    say(f"[gpu] {cfg_name} T={T}: worst rel err {res['worst_rel']:.3g}, excused {res['excused']}")
    layer.close()


def test_batch_repeated_zero_and_scaled_tokens(torch_cuda):
    """20 copies of one token (its experts get 20 entries: two tiles), zero
    tokens, tokens far from unit scale; repeated calls are bit-identical."""
    from routed_expert_int4_amd.layer import DeviceLayer
    say("[gpu] batched repeated / zero / scaled tokens")
    weights = synth.gen_layer(MID_A, seed=0)
    x = synth.gen_tokens(MID_A, 33, seed=12)
    x[1:20] = x[0]
    x[25] = 0
    x[26:29] = synth.gen_tokens(MID_A, 3, seed=13, std=300.0)
    x[29:32] = synth.gen_tokens(MID_A, 3, seed=14, std=1e-3)
    layer = DeviceLayer(weights, max_T=33)
    y, ids, w = run_batch(torch_cuda, layer, x)
    check_layer(weights, x, y, ids, w)
    assert np.all(y[25] == 0.0)
    for t in range(1, 20):
        np.testing.assert_array_equal(y[t], y[0])
    y2, ids2, _ = run_batch(torch_cuda, layer, x)
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(ids, ids2)
    layer.close()


def test_batch_split_by_sort_capacity(torch_cuda):
    """T * top_k above the dispatch sort's 8192 entries: two launch sequences."""
    from routed_expert_int4_amd.layer import DeviceLayer
    say("[gpu] batched T=1100 (two launch sequences)")
    weights = synth.gen_layer(MID_D, seed=1)
    x = synth.gen_tokens(MID_D, 1100, seed=15)
    layer = DeviceLayer(weights, max_T=1100)
    y, ids, w = run_batch(torch_cuda, layer, x)
    check_layer(weights, x, y, ids, w)
    layer.close()


def test_batch_router_topk(torch_cuda):
    from routed_expert_int4_amd.layer import DeviceLayer
    say("[gpu] batched router_topk MID_B T=64")
    weights = synth.gen_layer(MID_B, seed=2)
    x = synth.gen_tokens(MID_B, 64, seed=16)
    layer = DeviceLayer(weights, max_T=64)
    ids, w = layer.router_topk(DeviceLayer.to_device_bf16(x))
    torch_cuda.cuda.synchronize()
    ids_ref, w_ref, gap = oracle.route(weights, x)
    check_routing(MID_B, ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, gap)
    layer.close()


# ---------------------------------------------------------------- GLM shape
@pytest.fixture(scope="module")
def glm_zipf(torch_cuda):
    from routed_expert_int4_amd.layer import DeviceLayer
    say("[gpu] generating the GLM-shaped layer (seed 0) with the Zipf bias")
    weights, rec = zipf_glm_weights()
    layer = DeviceLayer(weights, max_T=512)
    yield weights, layer
    layer.close()


def test_glm_batch32_zipf(torch_cuda, glm_zipf):
    """Speculative-verify-sized calls: 4 calls of 32 tokens (x seed 4) with
    Zipf-skewed routing; every token's routing, all outputs of the first call
    and 4 tokens of each other call."""
    weights, layer = glm_zipf
    x_all = synth.gen_tokens(synth.GLM, 128, seed=4)
    for c in range(4):
        x = x_all[32 * c:32 * (c + 1)]
        y, ids, w = run_batch(torch_cuda, layer, x)
        ids_ref, w_ref, gap = oracle.route(weights, x)
        check_routing(synth.GLM, ids, w, ids_ref, w_ref, gap)
        rows = range(32) if c == 0 else [0, 9, 17, 31]
        res = check_layer(weights, x, y, ids, w, rows=rows)
        say(f"[gpu] GLM batch-32 call {c}: {len(set(ids.reshape(-1).tolist()))} distinct experts, "
            f"worst rel err {res['worst_rel']:.3g}")


def test_glm_prefill512(torch_cuda, glm_zipf):
    """A 512-token prefill chunk (x seed 5) on the GLM-shaped layer with
    uniform routing (bias N(0, 0.01)): routing of all 512 tokens, outputs of
    a spread of tokens and the smallest-gap ones."""
    from routed_expert_int4_amd.layer import DeviceLayer
    weights_z, _ = glm_zipf
    weights = synth.gen_layer(synth.GLM, seed=0)
    say("[gpu] GLM prefill 512")
    layer = DeviceLayer(weights, max_T=512)
    x = synth.gen_tokens(synth.GLM, 512, seed=5)
    y, ids, w = run_batch(torch_cuda, layer, x)
    ids_ref, w_ref, gap = oracle.route(weights, x)
    excused = check_routing(synth.GLM, ids, w, ids_ref, w_ref, gap)
    rows = sorted(set([0, 1, 100, 255, 256, 400, 510, 511] + list(np.argsort(gap)[:2])))
    res = check_layer(weights, x, y, ids, w, rows=rows)
    counts = np.bincount(ids.reshape(-1), minlength=256)
    say(f"[gpu] GLM prefill: {int((counts > 0).sum())} distinct experts, max {counts.max()} tokens/expert, "
        f"{len(excused)} excused, worst rel err {res['worst_rel']:.3g}")
    layer.close()


# ---------------------------------------------------------------- adaptive top-p
@pytest.mark.parametrize("cfg_name,T,top_p", [("TINY", 13, 0.5), ("MID_A", 37, 0.8), ("MID_B", 16, 0.6),
                                              ("MID_D", 100, 0.3)])
def test_batch_top_p_parity(torch_cuda, cfg_name, T, top_p):
    """Batch-union calls with the top-p cut: ids (-1 where dropped), weights
    and outputs against the oracle (tokens whose top-p margin is below 1e-6
    excused and re-checked on the GPU's ids); router_topk gives the same
    routing as the layer call."""
    import dataclasses
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = {"TINY": synth.TINY, "MID_A": MID_A, "MID_B": MID_B, "MID_D": MID_D}[cfg_name]
    cfg = dataclasses.replace(cfg, top_p=top_p)
    say(f"[gpu] batched top-p {top_p} {cfg_name} T={T}")
    weights = synth.gen_layer(cfg, seed=0)
    layer = DeviceLayer(weights, max_T=T)
    x = synth.gen_tokens(cfg, T, seed=3)
    y, ids, w = run_batch(torch_cuda, layer, x)
    res = check_layer(weights, x, y, ids, w)
    ids_r, w_r = layer.router_topk(DeviceLayer.to_device_bf16(x))
    torch_cuda.cuda.synchronize()
    np.testing.assert_array_equal(ids_r.cpu().numpy(), ids)
    np.testing.assert_array_equal(w_r.cpu().numpy(), w)
    dropped = int((ids < 0).sum())
    say(f"[gpu] batched top-p {cfg_name}: dropped {dropped}/{ids.size}, worst rel err {res['worst_rel']:.3g}, "
        f"excused {res['excused']}")
    assert dropped > 0
    layer.close()


# ---------------------------------------------------------------- MXFP4 experts
@pytest.mark.parametrize("cfg_name,T,top_p", [("TINY", 4, 1.0), ("MID_A", 37, 1.0), ("MID_B", 16, 1.0),
                                              ("MID_C", 5, 1.0), ("MID_D", 100, 1.0), ("MID_A", 21, 0.7)])
def test_batch_mxfp4_parity(torch_cuda, cfg_name, T, top_p):
    """Batch-union calls of MXFP4 layers (E2M1 codes turned into fp16 pairs
    for the matrix cores, E8M0 scales) against the oracle."""
    import dataclasses
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = {"TINY": synth.TINY, "MID_A": MID_A, "MID_B": MID_B, "MID_C": MID_C, "MID_D": MID_D}[cfg_name]
    cfg = dataclasses.replace(cfg, codec="mxfp4", top_p=top_p)
    say(f"[gpu] batched mxfp4 {cfg_name} T={T} top_p={top_p}")
    weights = synth.gen_layer(cfg, seed=0)
    layer = DeviceLayer(weights, max_T=T)
    x = synth.gen_tokens(cfg, T, seed=4)
    y, ids, w = run_batch(torch_cuda, layer, x)
    res = check_layer(weights, x, y, ids, w)
    say(f"[gpu] batched mxfp4 {cfg_name}: worst rel err {res['worst_rel']:.3g}, excused {res['excused']}")
    layer.close()


# ---------------------------------------------------------------- 32-entry tiles
@pytest.mark.parametrize("cfg_name,T,codec,top_p", [("TINY", 128, "int4", 1.0), ("MID_A", 100, "int4", 1.0),
                                                    ("MID_A", 100, "mxfp4", 1.0), ("MID_D", 300, "int4", 1.0),
                                                    ("TINY", 77, "int4", 0.7)])
def test_batch_wide_tiles_parity(torch_cuda, cfg_name, T, codec, top_p):
    """Calls averaging at least 8 entries per expert take tiles of up to 32
    entries (two MFMA row blocks per weight fragment): experts with more
    than 32 entries, ragged last tiles and the shared expert's tiles,
    against the oracle on every output."""
    import dataclasses
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = {"TINY": synth.TINY, "MID_A": MID_A, "MID_D": MID_D}[cfg_name]
    cfg = dataclasses.replace(cfg, codec=codec, top_p=top_p)
    assert T * cfg.top_k >= 8 * cfg.n_experts
    say(f"[gpu] wide tiles {cfg_name} T={T} {codec} top_p={top_p}")
    weights = synth.gen_layer(cfg, seed=2)
    layer = DeviceLayer(weights, max_T=T)
    x = synth.gen_tokens(cfg, T, seed=6)
    y, ids, w = run_batch(torch_cuda, layer, x)
    counts = np.bincount(ids[ids >= 0].ravel(), minlength=cfg.n_experts)
    if cfg_name == "TINY" and top_p == 1.0:
        assert counts.max() > 32  # several tiles for one expert
    res = check_layer(weights, x, y, ids, w)
    say(f"[gpu] wide tiles {cfg_name}: worst rel err {res['worst_rel']:.3g}, max entries {counts.max()}")
    layer.close()


# ---------------------------------------------------------------- int8 experts
@pytest.mark.parametrize("cfg_name,T,top_p", [("TINY", 4, 1.0), ("MID_A", 37, 1.0), ("MID_B", 16, 1.0),
                                              ("MID_C", 5, 1.0), ("MID_D", 100, 1.0), ("MID_A", 21, 0.7)])
def test_batch_int8_parity(torch_cuda, cfg_name, T, top_p):
    """Batch-union calls of int8 layers (each group step once per nibble
    plane on the matrix cores, under the group's one scale) against the
    oracle."""
    import dataclasses
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = {"TINY": synth.TINY, "MID_A": MID_A, "MID_B": MID_B, "MID_C": MID_C, "MID_D": MID_D}[cfg_name]
    cfg = dataclasses.replace(cfg, codec="int8", top_p=top_p)
    say(f"[gpu] batched int8 {cfg_name} T={T} top_p={top_p}")
    weights = synth.gen_layer(cfg, seed=0)
    layer = DeviceLayer(weights, max_T=T)
    x = synth.gen_tokens(cfg, T, seed=4)
    y, ids, w = run_batch(torch_cuda, layer, x)
    res = check_layer(weights, x, y, ids, w)
    say(f"[gpu] batched int8 {cfg_name}: worst rel err {res['worst_rel']:.3g}, excused {res['excused']}")
    layer.close()


def test_batch_int8_extreme_codes(torch_cuda):
    """Batched int8 calls with codes -128 and 127 over whole rows and
    activations of std 1e-3 and 300: the high plane's 16 (c - 8) and the low
    plane's c recombine exactly in the matrix-core sums."""
    import dataclasses
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = dataclasses.replace(MID_A, codec="int8")
    say("[gpu] batched int8 extreme codes")
    base = synth.gen_layer(cfg, seed=3)
    gq = base.gate_q.copy()
    gq[:, 0::3, :] = 0x80  # -128
    gq[:, 1::3, :] = 0x7F  # 127
    dq = base.down_q.copy()
    dq[:, 0::2, :] = 0x80
    uq = base.up_q.copy()
    uq[:, 1::2, :] = 0x7F
    weights = dataclasses.replace(base, gate_q=gq, up_q=uq, down_q=dq)
    layer = DeviceLayer(weights, max_T=19)
    for std in (1e-3, 300.0):
        x = synth.gen_tokens(cfg, 19, seed=11, std=std)
        y, ids, w = run_batch(torch_cuda, layer, x)
        res = check_layer(weights, x, y, ids, w)
        say(f"[gpu] batched int8 extremes std {std}: worst rel err {res['worst_rel']:.3g}")
    layer.close()


def test_glm_int8_prefill_chunk(torch_cuda):
    """GLM-shaped int8 layer, one 256-token prefill chunk: routing of every
    token against the oracle, outputs on a sample."""
    import dataclasses
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = dataclasses.replace(synth.GLM, codec="int8")
    say("[gpu] GLM int8 prefill chunk of 256")
    weights = synth.gen_layer(cfg, seed=0)
    layer = DeviceLayer(weights, max_T=256)
    x = synth.gen_tokens(cfg, 256, seed=5)
    y, ids, w = run_batch(torch_cuda, layer, x)
    ids_ref, w_ref, gap = oracle.route(weights, x)
    excused = check_routing(cfg, ids, w, ids_ref, w_ref, gap)
    rows = sorted(set([0, 1, 128, 255] + list(np.argsort(gap)[:2])))
    res = check_layer(weights, x, y, ids, w, rows=rows)
    say(f"[gpu] GLM int8 prefill: {len(excused)} excused, sampled worst rel err {res['worst_rel']:.3g}")
    layer.close()


# ---------------------------------------------------------------- int2 experts
@pytest.mark.parametrize("cfg_name,T,top_p", [("MID_A", 37, 1.0), ("MID_B", 16, 1.0), ("MID_C", 5, 1.0),
                                              ("MID_A", 3, 1.0), ("MID_A", 21, 0.7)])
def test_batch_int2_parity(torch_cuda, cfg_name, T, top_p):
    """Batch-union calls of int2 layers (two rows to a stored nibble: two
    fragments per code dword, even and odd rows accumulated apart, each
    under its own scale) against the oracle."""
    import dataclasses
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = {"MID_A": MID_A, "MID_B": MID_B, "MID_C": MID_C}[cfg_name]
    cfg = dataclasses.replace(cfg, codec="int2", top_p=top_p)
    say(f"[gpu] batched int2 {cfg_name} T={T} top_p={top_p}")
    weights = synth.gen_layer(cfg, seed=0)
    layer = DeviceLayer(weights, max_T=T)
    x = synth.gen_tokens(cfg, T, seed=4)
    y, ids, w = run_batch(torch_cuda, layer, x)
    res = check_layer(weights, x, y, ids, w)
    say(f"[gpu] batched int2 {cfg_name}: worst rel err {res['worst_rel']:.3g}, excused {res['excused']}")
    layer.close()


def test_batch_int2_extreme_codes(torch_cuda):
    """Batched int2 calls with whole rows of codes -2 and 1 (every stored
    nibble 0x0 or 0xF) and activations of std 1e-3 and 300."""
    import dataclasses
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = dataclasses.replace(MID_A, codec="int2")
    say("[gpu] batched int2 extreme codes")
    base = synth.gen_layer(cfg, seed=3)
    gq = base.gate_q.copy()
    gq[:, 0::3, :] = 0xAA  # -2 in every 2-bit field
    gq[:, 1::3, :] = 0x55  # 1
    dq = base.down_q.copy()
    dq[:, 0::2, :] = 0xAA
    weights = dataclasses.replace(base, gate_q=gq, down_q=dq)
    layer = DeviceLayer(weights, max_T=19)
    for std in (1e-3, 300.0):
        x = synth.gen_tokens(cfg, 19, seed=11, std=std)
        y, ids, w = run_batch(torch_cuda, layer, x)
        res = check_layer(weights, x, y, ids, w)
        say(f"[gpu] batched int2 extremes std {std}: worst rel err {res['worst_rel']:.3g}")
    layer.close()


def test_glm_int2_prefill_chunk(torch_cuda):
    """GLM-shaped int2 layer, one 256-token prefill chunk: routing of every
    token against the oracle, outputs on a sample."""
    import dataclasses
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = dataclasses.replace(synth.GLM, codec="int2")
    say("[gpu] GLM int2 prefill chunk of 256")
    weights = synth.gen_layer(cfg, seed=0)
    layer = DeviceLayer(weights, max_T=256)
    x = synth.gen_tokens(cfg, 256, seed=5)
    y, ids, w = run_batch(torch_cuda, layer, x)
    ids_ref, w_ref, gap = oracle.route(weights, x)
    excused = check_routing(cfg, ids, w, ids_ref, w_ref, gap)
    rows = sorted(set([0, 1, 128, 255] + list(np.argsort(gap)[:2])))
    res = check_layer(weights, x, y, ids, w, rows=rows)
    say(f"[gpu] GLM int2 prefill: {len(excused)} excused, sampled worst rel err {res['worst_rel']:.3g}")
    layer.close()


def test_glm_mxfp4_prefill_chunk(torch_cuda):
    """GLM-shaped MXFP4 layer, one 512-token prefill chunk: routing of every
    token against the oracle, outputs on a sample."""
    import dataclasses
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = dataclasses.replace(synth.GLM, codec="mxfp4")
    say("[gpu] GLM mxfp4 prefill chunk of 512")
    weights = synth.gen_layer(cfg, seed=0)
    layer = DeviceLayer(weights, max_T=512)
    x = synth.gen_tokens(cfg, 512, seed=5)
    y, ids, w = run_batch(torch_cuda, layer, x)
    ids_ref, w_ref, gap = oracle.route(weights, x)
    excused = check_routing(cfg, ids, w, ids_ref, w_ref, gap)
    rows = sorted(set([0, 1, 255, 511] + list(np.argsort(gap)[:2])))
    res = check_layer(weights, x, y, ids, w, rows=rows)
    say(f"[gpu] GLM mxfp4 prefill: {len(excused)} excused, sampled worst rel err {res['worst_rel']:.3g}")
    layer.close()


@pytest.mark.parametrize("name", ["no_shared", "top1_one_group", "all_groups"])
def test_degenerate_configs_batched(torch_cuda, name):
    from routed_expert_int4_amd.layer import DeviceLayer
    from tests.test_gpu_decode import DEGENERATE
    cfg = DEGENERATE[name]
    say(f"[gpu] degenerate batched {name}")
    weights = synth.gen_layer(cfg, seed=5)
    layer = DeviceLayer(weights, max_T=33)
    x = synth.gen_tokens(cfg, 33, seed=7)
    y, ids, w = run_batch(torch_cuda, layer, x)
    res = check_layer(weights, x, y, ids, w)
    say(f"[gpu] batched {name}: worst rel err {res['worst_rel']:.3g}")
    layer.close()
