"""GPU tests of the HBM expert cache in front of a pinned host store.

The cache follows the per-layer LRU expert cache of the colibri summary
(fr.news.hada.io topic 31297, "Execution d'un MoE basee sur le streaming
disque"), with pinned host RAM in place of the disk.  Checked here, through
the C ABI:
  * every layer's outputs against the fp64 oracle on the GPU's own input to
    that layer (a stack of layers chained as in the 12-layer workload:
    next input = bf16(y / rms(y) + N(0, 0.1) noise));
  * outputs bit-identical to the same layer with every expert resident,
    called one token at a time (the cache changes where a blob is read from,
    not the arithmetic);
  * hit / miss / eviction counts equal to a plain LRU replay of the GPU's
    routing trace (oracle/lru.py), and h2d_bytes = misses x blob bytes;
  * copy/compute ordering with the minimum slot count (every token evicts
    experts the previous token read);
  * prefetch and evict semantics and their errors.
"""
import sys

import numpy as np
import pytest

from oracle import lru
from routed_expert_int4_amd import binding as B
from routed_expert_int4_amd import synth
from tests.helpers import check_layer

pytestmark = pytest.mark.gpu

CFG = synth.LayerConfig(hidden=1024, inter=256, n_experts=64, n_groups=8, topk_group=4, top_k=6)
N_LAYERS = 3
N_TOKENS = 40


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    return torch


def chain_input(y: np.ndarray, noise: np.ndarray) -> np.ndarray:
    """Next layer's bf16 input: weightless RMS normalisation of y plus noise."""
    rms = np.sqrt(np.mean(y.astype(np.float64) ** 2, axis=1, keepdims=True))
    return synth.round_to_bf16_bits((y / rms + noise).astype(np.float32))


def make_stack(torch, slots, n_layers=N_LAYERS, max_T=N_TOKENS, cfg=CFG):
    from routed_expert_int4_amd.layer import DeviceLayer, ExpertCache, HostExpertStore
    cache = ExpertCache(cfg, n_layers, slots)
    weights, cached, resident = [], [], []
    for l in range(n_layers):
        wl = synth.gen_layer(cfg, seed=10 + l)
        weights.append(wl)
        cache.register(l, HostExpertStore(wl))
        lay = DeviceLayer(wl, max_T=max_T, resident=False)
        lay.attach_cache(cache, l)
        cached.append(lay)
        resident.append(DeviceLayer(wl, max_T=max_T))
    torch.cuda.synchronize()
    return cache, weights, cached, resident


@pytest.mark.parametrize("slots", [16, CFG.top_k])
def test_cache_stack_parity_and_lru(torch_cuda, slots):
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    say(f"[gpu] cache stack: {N_LAYERS} layers, {slots} slots, {N_TOKENS} tokens")
    cache, weights, cached, resident = make_stack(torch, slots)
    x_bits = synth.gen_tokens(CFG, N_TOKENS, seed=30)
    for l in range(N_LAYERS):
        x = DeviceLayer.to_device_bf16(x_bits)
        y, ids, w = cached[l].forward(x)
        y_res, ids_res, w_res = resident[l].forward_each(x)
        torch.cuda.synchronize()
        yh, idh, wh = y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
        res = check_layer(weights[l], x_bits, yh, idh, wh)
        assert torch.equal(ids, ids_res) and torch.equal(w, w_res)
        assert torch.equal(y, y_res), "cached and resident outputs differ"
        st = cache.stats(l)
        hits, misses, evictions = lru.replay(idh, slots)
        say(f"[gpu] layer {l}: rel err {res['worst_rel']:.3g}, stats {st}, replay {(hits, misses, evictions)}")
        assert (st["hits"], st["misses"], st["evictions"]) == (hits, misses, evictions)
        assert st["h2d_bytes"] == misses * cache.nb
        assert st["prefetches"] == 0
        x_bits = chain_input(yh, synth.gen_noise(CFG, N_TOKENS, seed=40 + l, std=0.1))
    for lay in cached + resident:
        lay.close()
    cache.close()


def test_cache_prefetch_and_evict(torch_cuda):
    torch = torch_cuda
    from oracle import oracle
    from routed_expert_int4_amd.layer import DeviceLayer
    say("[gpu] cache prefetch/evict")
    cache, weights, cached, resident = make_stack(torch, slots=8, n_layers=1, max_T=2)
    x_bits = synth.gen_tokens(CFG, 1, seed=31)
    ids_ref, _, _ = oracle.route(weights[0], x_bits)
    need = [int(e) for e in ids_ref[0]]
    cache.prefetch(0, need)
    st = cache.stats(0)
    assert st["prefetches"] == CFG.top_k and st["h2d_bytes"] == CFG.top_k * cache.nb
    cache.prefetch(0, need)  # resident already: no new copies
    assert cache.stats(0)["prefetches"] == CFG.top_k
    x = DeviceLayer.to_device_bf16(x_bits)
    y, ids, w = cached[0].forward(x)
    torch.cuda.synchronize()
    check_layer(weights[0], x_bits, y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy())
    st = cache.stats(0)
    assert (st["hits"], st["misses"]) == (CFG.top_k, 0)
    cache.evict(0, need[2])
    cache.evict(0, need[2])  # not resident any more: no-op
    assert cache.stats(0)["evictions"] == 1
    y2, _, _ = cached[0].forward(x)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    st = cache.stats(0)
    assert (st["hits"], st["misses"]) == (2 * CFG.top_k - 1, 1)
    with pytest.raises(B.MoeError) as err:
        cache.prefetch(0, list(range(9)))
    assert err.value.code == B.MOE_ENOSLOT
    with pytest.raises(B.MoeError) as err:
        cache.prefetch(0, [CFG.n_experts])
    assert err.value.code == B.MOE_EINVAL
    with pytest.raises(B.MoeError):
        cache.evict(0, -1)
    for lay in cached + resident:
        lay.close()
    cache.close()


def test_cache_register_errors(torch_cuda):
    from routed_expert_int4_amd.layer import ExpertCache
    cache = ExpertCache(CFG, 1, CFG.top_k)
    buf = np.zeros(16, np.uint8)
    with pytest.raises(B.MoeError):
        B.expert_cache_register(cache.handle, 0, 0, buf.ctypes.data, 16)  # wrong size
    with pytest.raises(B.MoeError):
        B.expert_cache_register(cache.handle, 1, 0, buf.ctypes.data, cache.nb)  # bad layer
    with pytest.raises(B.MoeError):
        B.expert_cache_create(CFG, 1, CFG.top_k - 1, cache.pool, cache.pool.numel(), cache.copy_stream)
    cache.close()


def test_cache_learning_autopin(torch_cuda):
    """Learning cache: usage counts equal the routing trace's histogram; after
    autopin the n most used experts stay resident, and a run from an empty
    LRU part records exactly the hits, misses and evictions of the oracle's
    pinned replay, with outputs unchanged."""
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    slots, n_pin = 16, 8
    say(f"[gpu] learning cache: {slots} slots, autopin {n_pin}")
    cache, weights, cached, resident = make_stack(torch, slots, n_layers=1)
    x1 = synth.gen_tokens(CFG, N_TOKENS, seed=50)
    _, ids1, _ = cached[0].forward(DeviceLayer.to_device_bf16(x1))
    torch.cuda.synchronize()
    trace1 = ids1.cpu().numpy()
    counts = cache.usage(0)
    assert list(counts) == lru.usage(trace1, CFG.n_experts)
    cache.autopin(0, n_pin)
    pins = lru.hottest(lru.usage(trace1, CFG.n_experts), n_pin)
    # empty the LRU part: every unpinned expert leaves its slot
    for e in range(CFG.n_experts):
        if e not in pins:
            cache.evict(0, e)
    st0 = cache.stats(0)
    assert st0["pinned"] == n_pin
    x2 = synth.gen_tokens(CFG, N_TOKENS, seed=51)
    x = DeviceLayer.to_device_bf16(x2)
    y, ids, w = cached[0].forward(x)
    y_res, ids_res, w_res = resident[0].forward_each(x)
    torch.cuda.synchronize()
    idh = ids.cpu().numpy()
    assert torch.equal(ids, ids_res) and torch.equal(y, y_res), "cached and resident outputs differ"
    check_layer(weights[0], x2, y.cpu().numpy(), idh, w.cpu().numpy())
    st = cache.stats(0)
    got = (st["hits"] - st0["hits"], st["misses"] - st0["misses"], st["evictions"] - st0["evictions"])
    want = lru.replay(idh, slots, pinned=pins)
    say(f"[gpu] after autopin: {got}, oracle replay {want}, plain LRU would give {lru.replay(idh, slots)}")
    assert got == want
    assert B.expert_cache_replay(CFG.n_experts, slots, CFG.top_k, idh, pinned=pins) == want
    # pins must leave top_k slots; ids out of range are rejected; unpinning
    # an unpinned expert is a no-op
    with pytest.raises(B.MoeError) as err:
        cache.autopin(0, slots - CFG.top_k + 1)
    assert err.value.code == B.MOE_ENOSLOT
    with pytest.raises(B.MoeError) as err:
        cache.pin(0, [CFG.n_experts])
    assert err.value.code == B.MOE_EINVAL
    cache.unpin(0, [p for p in range(CFG.n_experts) if p not in pins][:3])
    assert cache.stats(0)["pinned"] == n_pin
    cache.unpin(0, pins)
    assert cache.stats(0)["pinned"] == 0
    for lay in cached + resident:
        lay.close()
    cache.close()


def test_cache_top_p(torch_cuda):
    """Adaptive top-p behind the cache: a dropped choice (id -1) is never
    made resident or copied; outputs equal the resident layer's one-token
    calls bit for bit and the oracle's within tolerance; the counts are the
    LRU replay of the kept choices only."""
    import dataclasses
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = dataclasses.replace(CFG, top_p=0.6)
    slots = CFG.top_k
    say(f"[gpu] cache with top-p 0.6, {slots} slots")
    cache, weights, cached, resident = make_stack(torch, slots, n_layers=1, cfg=cfg)
    x_bits = synth.gen_tokens(cfg, N_TOKENS, seed=60)
    x = DeviceLayer.to_device_bf16(x_bits)
    y, ids, w = cached[0].forward(x)
    y_res, ids_res, w_res = resident[0].forward_each(x)
    torch.cuda.synchronize()
    idh = ids.cpu().numpy()
    assert (idh < 0).any(), "the cut dropped nothing"
    assert torch.equal(ids, ids_res) and torch.equal(w, w_res) and torch.equal(y, y_res)
    res = check_layer(weights[0], x_bits, y.cpu().numpy(), idh, w.cpu().numpy())
    kept = [row[row >= 0] for row in idh]
    st = cache.stats(0)
    want = lru.replay(kept, slots)
    say(f"[gpu] top-p cache: rel err {res['worst_rel']:.3g}, stats {st}, replay {want}")
    assert (st["hits"], st["misses"], st["evictions"]) == want
    assert st["h2d_bytes"] == want[1] * cache.nb
    assert list(cache.usage(0)) == lru.usage(kept, CFG.n_experts)
    for lay in cached + resident:
        lay.close()
    cache.close()


@pytest.mark.parametrize("codec", ["mxfp4", "int8", "int2"])
def test_cache_other_codecs(torch_cuda, codec):
    """MXFP4 and int8 experts behind the cache: outputs equal the resident
    layer's one-token calls bit for bit, and the oracle's within tolerance;
    copies move the codec's blobs (h2d_bytes = misses x blob bytes)."""
    import dataclasses
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = dataclasses.replace(CFG, codec=codec)
    slots = CFG.top_k
    say(f"[gpu] {codec} cache, {slots} slots")
    cache, weights, cached, resident = make_stack(torch, slots, n_layers=1, cfg=cfg)
    assert cache.nb == cfg.expert_bytes()
    x_bits = synth.gen_tokens(cfg, N_TOKENS, seed=70)
    x = DeviceLayer.to_device_bf16(x_bits)
    y, ids, w = cached[0].forward(x)
    y_res, ids_res, w_res = resident[0].forward_each(x)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_res) and torch.equal(w, w_res) and torch.equal(y, y_res)
    idh = ids.cpu().numpy()
    res = check_layer(weights[0], x_bits, y.cpu().numpy(), idh, w.cpu().numpy())
    st = cache.stats(0)
    assert (st["hits"], st["misses"], st["evictions"]) == lru.replay(idh, slots)
    assert st["h2d_bytes"] == st["misses"] * cache.nb
    say(f"[gpu] {codec} cache: rel err {res['worst_rel']:.3g}, stats {st}")
    for lay in cached + resident:
        lay.close()
    cache.close()


def glm_stack_layer(l, biases):
    """Layer l of the GLM-shaped stack: weights seed 100 + l with the
    committed Zipf(1.1)-calibrated bias of that layer."""
    wl = synth.gen_layer(synth.GLM, seed=100 + l)
    wl.bias = np.asarray(biases[l], dtype=np.float32)
    return wl


@pytest.mark.parametrize("slots", [64, 12])
def test_glm_cache_stack_parity_and_lru(torch_cuda, slots):
    """The cache-stack workload at full size: two chained GLM-shaped layers
    (hidden 6144, intermediate 2048, 256 experts, top-8) behind an HBM cache
    of `slots` slots per layer fed from pinned host stores, 16 sequential
    tokens.  Every layer's outputs against the oracle on the GPU's own bf16
    input to that layer; hit / miss / eviction counts equal to the LRU replay
    of the GPU's routing trace; h2d_bytes = misses x blob bytes.  With 12
    slots nearly every token evicts experts the previous token read."""
    import json
    import os
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer, ExpertCache, HostExpertStore
    n_layers, n_tok = 2, 16
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "zipf_bias_stack.json")) as f:
        biases = [l["bias"] for l in json.load(f)["layers"]]
    say(f"[gpu] GLM cache stack: {n_layers} layers, {slots} slots, {n_tok} tokens")
    cache = ExpertCache(synth.GLM, n_layers, slots)
    weights, layers = [], []
    for l in range(n_layers):
        wl = glm_stack_layer(l, biases)
        cache.register(l, HostExpertStore(wl))
        lay = DeviceLayer(wl, max_T=n_tok, resident=False)
        lay.attach_cache(cache, l)
        weights.append(wl)
        layers.append(lay)
    torch.cuda.synchronize()
    x_bits = synth.gen_tokens(synth.GLM, n_tok, seed=300)
    noise = synth.gen_noise(synth.GLM, n_tok * n_layers, seed=400, std=0.1)
    for l in range(n_layers):
        y, ids, w = layers[l].forward(DeviceLayer.to_device_bf16(x_bits))
        torch.cuda.synchronize()
        yh, idh, wh = y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
        res = check_layer(weights[l], x_bits, yh, idh, wh)
        st = cache.stats(l)
        want = lru.replay(idh, slots)
        say(f"[gpu] GLM layer {l}: rel err {res['worst_rel']:.3g}, excused {res['excused']}, stats {st}, "
            f"replay {want}")
        assert (st["hits"], st["misses"], st["evictions"]) == want
        assert st["h2d_bytes"] == st["misses"] * cache.nb
        if slots == 12:
            assert st["evictions"] > 0
        x_bits = chain_input(yh, noise[l * n_tok:(l + 1) * n_tok])
    for lay in layers:
        lay.close()
    cache.close()
