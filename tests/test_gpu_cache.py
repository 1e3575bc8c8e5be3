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
  * prefetch and evict semantics and their errors;
  * calls alternating between two streams that the caller orders;
  * batched calls (T > 1) behind the cache: outputs bit-identical to the
    resident batched path run on the same token groups (one group: the whole
    call; groups of one token, which a resident call would run on the decode
    kernels, against the oracle), one lookup per distinct expert and token group,
    the counts equal to the LRU replay of those groups;
  * speculative next-layer prefetch (the next layer's router on the current
    layer's input): outputs unchanged, the predictions equal to the oracle's
    routing, and every count equal to the oracle's prefetching replay; the
    copy/compute timeline sees every copy.
"""
import dataclasses
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
        y, ids, w = cached[l].forward_each(x)
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


def test_cache_calls_on_two_streams(torch_cuda):
    """One-token and batched calls of a cached layer alternating between two
    streams that the caller orders (each call's stream waits for the other
    one first), with as many slots as top_k, so every token evicts experts
    that the previous call, on the other stream, read: outputs bit-identical
    to the resident layer's, counts equal to the LRU replay."""
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    slots, T = CFG.top_k, 12
    say(f"[gpu] cache calls on two streams: {slots} slots, {T} one-token calls, then a batched call")
    cache, weights, cached, resident = make_stack(torch, slots, n_layers=1, max_T=4)
    x_bits = synth.gen_tokens(CFG, T, seed=33)
    x = DeviceLayer.to_device_bf16(x_bits)
    y_res, ids_res, w_res = resident[0].forward_each(x)
    yb_res, idsb_res, _ = resident[0].forward(x[:4])
    y = torch.empty_like(y_res)
    ids = torch.empty_like(ids_res)
    w = torch.empty_like(w_res)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for t in range(T):
        s, other = streams[t % 2], streams[(t + 1) % 2]
        s.wait_stream(other)
        cached[0].forward(x[t:t + 1], y[t:t + 1], ids[t:t + 1], w[t:t + 1], stream=s)
    s = streams[T % 2]
    s.wait_stream(streams[(T + 1) % 2])
    yb, idsb, wb = cached[0].forward(x[:4], stream=s)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_res) and torch.equal(w, w_res)
    assert torch.equal(y, y_res), "cached outputs on two streams differ from the resident layer's"
    assert torch.equal(idsb, idsb_res)
    idh = ids.cpu().numpy()
    groups, spans = token_groups(idsb.cpu().numpy(), slots, [], ranges=True)
    y_g, multi = resident_by_groups(torch, resident[0], x[:4], spans)
    assert torch.equal(yb[multi], y_g[multi])
    check_layer(weights[0], x_bits[:4], yb.cpu().numpy(), idsb.cpu().numpy(), wb.cpu().numpy())
    hits, misses, evictions = lru.replay(list(idh) + groups, slots)
    st = cache.stats(0)
    say(f"[gpu] two streams: stats {st}, replay {(hits, misses, evictions)}")
    assert (st["hits"], st["misses"], st["evictions"]) == (hits, misses, evictions)
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
    _, ids1, _ = cached[0].forward_each(DeviceLayer.to_device_bf16(x1))
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
    y, ids, w = cached[0].forward_each(x)
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
    y, ids, w = cached[0].forward_each(x)
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
    y, ids, w = cached[0].forward_each(x)
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
        y, ids, w = layers[l].forward_each(DeviceLayer.to_device_bf16(x_bits))
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


def run_token_major(torch, cached, x0_bits, noise_seed):
    """Every token through all layers before the next one starts (the order
    in which layer l's prediction is used by layer l + 1's call for the same
    token).  Returns per layer its inputs (bf16 bits) and outputs, ids, w."""
    from routed_expert_int4_amd.layer import DeviceLayer
    n_layers, (T, H), k = len(cached), x0_bits.shape, CFG.top_k
    xs = [np.empty((T, H), np.uint16) for _ in range(n_layers)]
    ys = [np.empty((T, H), np.float32) for _ in range(n_layers)]
    ids = [np.empty((T, k), np.int32) for _ in range(n_layers)]
    ws = [np.empty((T, k), np.float32) for _ in range(n_layers)]
    noise = synth.gen_noise(CFG, T * n_layers, seed=noise_seed, std=0.1)
    for t in range(T):
        xb = x0_bits[t:t + 1]
        for l in range(n_layers):
            xs[l][t] = xb[0]
            y, i, w = cached[l].forward(DeviceLayer.to_device_bf16(xb))
            torch.cuda.synchronize()
            ys[l][t], ids[l][t], ws[l][t] = y.cpu().numpy()[0], i.cpu().numpy()[0], w.cpu().numpy()[0]
            xb = chain_input(ys[l][t:t + 1], noise[t * n_layers + l:t * n_layers + l + 1])
    return xs, ys, ids, ws


@pytest.mark.parametrize("slots,max_prefetch", [(12, 0), (8, 2), (CFG.top_k + 1, 1)])
def test_cache_next_layer_prefetch(torch_cuda, slots, max_prefetch):
    torch = torch_cuda
    from oracle import oracle
    from routed_expert_int4_amd.layer import DeviceLayer
    from tests.helpers import check_routing
    T = 24
    say(f"[gpu] next-layer prefetch: {N_LAYERS} layers, {slots} slots, max_prefetch {max_prefetch}, {T} tokens")
    cache, weights, cached, resident = make_stack(torch, slots, max_T=1)
    for l in range(N_LAYERS - 1):
        cached[l].set_next(cached[l + 1], max_prefetch)
    cache.timeline(True)
    xs, ys, ids, ws = run_token_major(torch, cached, synth.gen_tokens(CFG, T, seed=36), noise_seed=37)
    tl = cache.timeline_read()
    copies = 0
    for l in range(N_LAYERS):
        res = check_layer(weights[l], xs[l], ys[l], ids[l], ws[l])
        y_res, ids_res, _ = resident[l].forward_each(DeviceLayer.to_device_bf16(xs[l]))
        torch.cuda.synchronize()
        assert np.array_equal(ids_res.cpu().numpy(), ids[l]), "prefetching changed the routing"
        assert np.array_equal(y_res.cpu().numpy(), ys[l]), "prefetching changed the outputs"
        predicted = [None] * T
        if l > 0:
            # layer l's router on layer l - 1's input, one token at a time
            # as the predictor runs it, checked against the oracle's routing
            x_prev = DeviceLayer.to_device_bf16(xs[l - 1])
            pr, pw = zip(*(resident[l].router_topk(x_prev[t:t + 1]) for t in range(T)))
            pr = np.concatenate([v.cpu().numpy() for v in pr])
            pw = np.concatenate([v.cpu().numpy() for v in pw])
            ref_ids, ref_w, gap = oracle.route(weights[l], xs[l - 1])
            check_routing(CFG, pr, pw, ref_ids, ref_w, gap)
            predicted = list(pr)
        ref = lru.replay_prefetch(ids[l], predicted, slots, max_prefetch=max_prefetch or CFG.top_k)
        st = cache.stats(l)
        say(f"[gpu] layer {l}: rel err {res['worst_rel']:.3g}, stats {st}")
        assert {k: st[k] for k in ref} == ref
        assert st["h2d_bytes"] == (st["misses"] + st["prefetches"]) * cache.nb
        copies += st["misses"] + st["prefetches"]
    calls, preds = T * N_LAYERS, T * (N_LAYERS - 1)
    say(f"[gpu] timeline {tl}")
    assert not tl["truncated"] and tl["copies"] == copies
    # router + down per call, one or two gate/up launches, one predictor launch per linked call
    assert 3 * calls + preds <= tl["kernels"] <= 4 * calls + preds
    assert 0.0 <= tl["overlap_ms"] <= min(tl["copy_ms"], tl["kernel_ms"]) + 1e-6
    assert tl["span_ms"] >= max(tl["copy_ms"], tl["kernel_ms"]) - 1e-6 and tl["copy_ms"] > 0.0
    for l in range(N_LAYERS - 1):
        cached[l].set_next(None)
    for lay in cached + resident:
        lay.close()
    cache.close()


def test_cache_prefetch_link_errors_and_timeline_limit(torch_cuda):
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    say("[gpu] next-layer link errors and timeline limit")
    cache, weights, cached, resident = make_stack(torch, slots=8, n_layers=2, max_T=1)
    other, _, other_cached, other_resident = make_stack(torch, slots=8, n_layers=1, max_T=1)
    for a, b in [(cached[0], cached[0]), (cached[0], resident[1]), (resident[0], cached[1]),
                 (cached[0], other_cached[0])]:
        with pytest.raises(B.MoeError) as err:
            a.set_next(b)
        assert err.value.code == B.MOE_EINVAL
    with pytest.raises(B.MoeError) as err:
        B.moe_layer_set_next(cached[0].handle, cached[1].handle, -1)
    assert err.value.code == B.MOE_EINVAL
    # a next layer bound to the same workspace is refused, at link time and at call time
    B.moe_layer_set_workspace(cached[1].handle, cached[0].ws, cached[0].ws_bytes, 1)
    with pytest.raises(B.MoeError) as err:
        cached[0].set_next(cached[1])
    assert err.value.code == B.MOE_EINVAL
    B.moe_layer_set_workspace(cached[1].handle, cached[1].ws, cached[1].ws_bytes, 1)
    cached[0].set_next(cached[1])
    x = DeviceLayer.to_device_bf16(synth.gen_tokens(CFG, 2, seed=38))
    B.moe_layer_set_workspace(cached[1].handle, cached[0].ws, cached[0].ws_bytes, 1)
    with pytest.raises(B.MoeError) as err:
        cached[0].forward(x[0:1])
    assert err.value.code == B.MOE_EINVAL and "workspace" in B.last_error()
    torch.cuda.synchronize()
    B.moe_layer_set_workspace(cached[1].handle, cached[1].ws, cached[1].ws_bytes, 1)
    # a timeline limited to three intervals: truncated, and no more recorded
    cache.timeline(True, max_marks=3)
    cached[0].forward(x[1:2])
    torch.cuda.synchronize()
    tl = cache.timeline_read()
    assert tl["truncated"] == 1 and tl["copies"] + tl["kernels"] <= 3
    cache.timeline(False)
    cached[1].forward(x[1:2])
    torch.cuda.synchronize()
    tl = cache.timeline_read()
    assert tl["copies"] == tl["kernels"] == 0 and not tl["truncated"]
    cached[0].set_next(None)
    for lay in cached + resident + other_cached + other_resident:
        lay.close()
    cache.close()
    other.close()


def token_groups(ids, slots, pinned, ranges=False):
    """The consecutive token groups of a batched call behind the cache: as
    many tokens as fit, in order, while the group's distinct experts that are
    not pinned number at most slots - len(pinned); each group is looked up as
    its distinct experts in ascending order.  With ranges, also the groups'
    token ranges [t0, t1)."""
    pinned, room = set(int(e) for e in pinned), slots - len(pinned)
    groups, spans, g0, n = [], [], 0, len(ids)
    while g0 < n:
        seen, used, t = set(), 0, g0
        while t < n:
            row = [int(e) for e in ids[t] if e >= 0]
            add = len({e for e in row if e not in seen and e not in pinned})
            if t > g0 and used + add > room:
                break
            used += add
            seen.update(row)
            t += 1
        groups.append(sorted(seen))
        spans.append((g0, t))
        g0 = t
    return (groups, spans) if ranges else groups


def resident_by_groups(torch, resident, x, spans):
    """The resident layer's batched outputs over each token group on its
    own: the reference of a cached batched call, which runs its groups as
    separate launch sequences (an expert's entries in a group decide its
    kernel, the grouped MFMA or, with a single entry, the GEMV).  A resident
    call of one token takes the decode kernels instead, so one-token groups
    have no bit-exact reference: returns (reference rows, mask of the tokens
    in groups of two or more)."""
    ys, keep = [], []
    for t0, t1 in spans:
        ys.append(resident.forward(x[t0:t1])[0])
        keep += [t1 - t0 > 1] * (t1 - t0)
    return torch.cat(ys), torch.tensor(keep, device=x.device)


@pytest.mark.parametrize("slots,n_pin,top_p", [(64, 0, 1.0), (16, 0, 1.0), (12, 4, 1.0), (16, 0, 0.6)])
def test_cache_batched_call(torch_cuda, slots, n_pin, top_p):
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = dataclasses.replace(CFG, top_p=top_p)
    T = 40
    say(f"[gpu] batched call behind the cache: {slots} slots, {n_pin} pinned, top-p {top_p}, T={T}")
    cache, weights, cached, resident = make_stack(torch, slots, n_layers=1, max_T=T, cfg=cfg)
    x_bits = synth.gen_tokens(cfg, T, seed=39)
    x = DeviceLayer.to_device_bf16(x_bits)
    y_r, ids_r, w_r = resident[0].forward(x)
    torch.cuda.synchronize()
    idh = ids_r.cpu().numpy()
    pins = lru.hottest(lru.usage(idh, cfg.n_experts), n_pin)
    if pins:
        cache.pin(0, pins)
    groups, spans = token_groups(idh, slots, pins, ranges=True)
    y_g, multi = resident_by_groups(torch, resident[0], x, spans)
    if len(spans) == 1:
        assert torch.equal(y_g, y_r)
    for call in range(2):  # the second call finds the last group's experts resident
        y, ids, w = cached[0].forward(x)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_r) and torch.equal(w, w_r), "routing differs from the resident batched path"
        assert torch.equal(y[multi], y_g[multi]), \
            "outputs differ from the resident batched path over the same token groups"
    # every token (one-token groups included) against the oracle
    res = check_layer(weights[0], x_bits, y.cpu().numpy(), idh, w.cpu().numpy())
    hits, misses, evictions = lru.replay(groups + groups, slots, pinned=pins)
    st = cache.stats(0)
    say(f"[gpu] {len(groups)} groups, rel err {res['worst_rel']:.3g}, stats {st}, replay {(hits, misses, evictions)}")
    assert (st["hits"], st["misses"], st["evictions"]) == (hits, misses, evictions)
    assert st["h2d_bytes"] == (misses + len(pins)) * cache.nb
    assert list(cache.usage(0)) == lru.usage(np.concatenate([idh, idh]), cfg.n_experts)
    if slots < cfg.n_experts and top_p == 1.0:
        assert len(groups) > 1, "the call should need several groups"
    for lay in cached + resident:
        lay.close()
    cache.close()


def test_glm_cache_batched_call(torch_cuda):
    """A 32-token call of the GLM-shaped layer with the Zipf(1.1) bias behind
    a 64-slot cache (about 90 distinct experts per call, so several token
    groups): outputs bit-identical to the resident batched path over the
    same token groups, sampled tokens against the oracle, counts equal to the
    LRU replay of the groups."""
    torch = torch_cuda
    from routed_expert_int4_amd.layer import DeviceLayer, ExpertCache, HostExpertStore
    from tests.helpers import zipf_glm_weights
    slots, T = 64, 32
    say(f"[gpu] GLM batched call behind a {slots}-slot cache, T={T}")
    weights, _ = zipf_glm_weights()
    cache = ExpertCache(synth.GLM, 1, slots)
    cache.register(0, HostExpertStore(weights))
    cached = DeviceLayer(weights, max_T=T, resident=False)
    cached.attach_cache(cache, 0)
    resident = DeviceLayer(weights, max_T=T)
    x_bits = synth.gen_tokens(synth.GLM, T, seed=4)
    x = DeviceLayer.to_device_bf16(x_bits)
    y_r, ids_r, w_r = resident.forward(x)
    y, ids, w = cached.forward(x)
    torch.cuda.synchronize()
    idh = ids.cpu().numpy()
    groups, spans = token_groups(idh, slots, [], ranges=True)
    y_g, multi = resident_by_groups(torch, resident, x, spans)
    assert torch.equal(ids, ids_r) and torch.equal(w, w_r) and torch.equal(y[multi], y_g[multi])
    single = [t for t, m in enumerate(multi.cpu().tolist()) if not m]  # one-token groups: the oracle only
    res = check_layer(weights, x_bits, y.cpu().numpy(), idh, w.cpu().numpy(), rows=sorted({0, 9, 31, *single}))
    st = cache.stats(0)
    say(f"[gpu] GLM batched cache: {len(groups)} groups of {[len(g) for g in groups]} experts, "
        f"rel err {res['worst_rel']:.3g}, stats {st}")
    assert len(groups) > 1
    assert (st["hits"], st["misses"], st["evictions"]) == lru.replay(groups, slots)
    assert st["h2d_bytes"] == st["misses"] * cache.nb
    cached.close()
    resident.close()
    cache.close()
