"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every entry point declared in include/moe.h, validates arguments, packs
experts, and its cache slot policy matches a plain LRU replay."""
import os
import re

import numpy as np
import pytest

from oracle import lru
from routed_expert_int4_amd import binding as B
from routed_expert_int4_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 18, names
    L = B.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in moe.h but not exported"


def test_expert_bytes_match_public_layout():
    assert B.moe_expert_bytes(synth.GLM) == 21_233_664
    assert B.moe_expert_bytes(synth.TINY) == 55_296
    assert B.moe_expert_bytes(synth.GLM) == synth.GLM.expert_bytes()


def test_invalid_configs_are_rejected():
    import dataclasses
    bad = [
        dataclasses.replace(synth.TINY, hidden=250),
        dataclasses.replace(synth.TINY, n_groups=3),
        dataclasses.replace(synth.TINY, topk_group=5),
        dataclasses.replace(synth.TINY, top_k=9),
        dataclasses.replace(synth.TINY, top_p=0.0),
        dataclasses.replace(synth.TINY, top_p=1.5),
        dataclasses.replace(synth.TINY, top_p=float("nan")),
    ]
    for cfg in bad:
        assert B.moe_expert_bytes(cfg) == 0
        with pytest.raises(B.MoeError) as e:
            B.moe_layer_create(cfg, None, None, [])
        assert e.value.code == B.MOE_EINVAL
    with pytest.raises(B.MoeError) as e:
        B.moe_layer_create(dataclasses.replace(synth.TINY, hidden=96 * 32), None, None, [])
    assert e.value.code == B.MOE_EUNSUPPORTED
    with pytest.raises(B.MoeError) as e:  # valid shape, but the expert count is not a multiple of 16
        B.moe_layer_create(dataclasses.replace(synth.TINY, n_experts=24, n_groups=3, topk_group=2), None, None, [])
    assert e.value.code == B.MOE_EUNSUPPORTED
    with pytest.raises(B.MoeError) as e:
        B.moe_layer_create(synth.TINY, None, None, [])
    assert e.value.code == B.MOE_EINVAL and "NULL" in B.last_error()


def test_pack_keeps_codes_and_permutes_scales():
    w = synth.gen_layer(synth.TINY, seed=0)
    cfg = synth.TINY
    nb = B.moe_expert_bytes(cfg)
    blob = np.empty(nb, np.uint8)
    B.moe_expert_pack(cfg, *w.expert_arrays(3), blob)
    n = cfg.hidden * cfg.inter // 2
    gq, gs, uq, us, dq, ds = w.expert_arrays(3)
    # codes: same bytes with each nibble in offset binary (q + 8)
    np.testing.assert_array_equal(blob[:n], gq.ravel() ^ 0x88)
    np.testing.assert_array_equal(blob[n:2 * n], uq.ravel() ^ 0x88)
    np.testing.assert_array_equal(blob[2 * n:3 * n], dq.ravel() ^ 0x88)
    # scales: gate and up scales (interleaved) are a permutation of the
    # public ones, and so are the down scales
    sc = blob[3 * n:].view(np.uint16)
    m = sc.size // 3
    np.testing.assert_array_equal(np.sort(sc[:2 * m]), np.sort(np.concatenate([gs.ravel(), us.ravel()])))
    np.testing.assert_array_equal(np.sort(sc[2 * m:]), np.sort(ds.ravel()))


def test_pack_mxfp4_keeps_codes_and_permutes_e8m0_scales():
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, codec="mxfp4")
    w = synth.gen_layer(cfg, seed=0)
    nb = B.moe_expert_bytes(cfg)
    assert nb == cfg.expert_bytes() == 3 * cfg.hidden * cfg.inter // 2 + 3 * cfg.hidden * cfg.inter // 32
    assert B.moe_expert_bytes(dataclasses.replace(synth.GLM, codec="mxfp4")) == 20_054_016  # 19.125 MiB
    blob = np.empty(nb, np.uint8)
    B.moe_expert_pack(cfg, *w.expert_arrays(5), blob)
    n = cfg.hidden * cfg.inter // 2
    gq, gs, uq, us, dq, ds = w.expert_arrays(5)
    # E2M1 codes are kept as they are
    np.testing.assert_array_equal(blob[:n], gq.ravel())
    np.testing.assert_array_equal(blob[n:2 * n], uq.ravel())
    np.testing.assert_array_equal(blob[2 * n:3 * n], dq.ravel())
    sc = blob[3 * n:]
    m = sc.size // 3
    np.testing.assert_array_equal(np.sort(sc[:2 * m]), np.sort(np.concatenate([gs.ravel(), us.ravel()])))
    np.testing.assert_array_equal(np.sort(sc[2 * m:]), np.sort(ds.ravel()))
    # the NaN scale byte is refused
    bad = ds.copy()
    bad[0, 0] = 255
    with pytest.raises(B.MoeError) as e:
        B.moe_expert_pack(cfg, gq, gs, uq, us, dq, bad, blob)
    assert e.value.code == B.MOE_EINVAL
    # an unknown codec value is an invalid config
    import ctypes
    c = B.MoeConfig.from_cfg(cfg)
    c.codec = 7
    assert B.lib().moe_expert_bytes(ctypes.byref(c)) == 0


def test_pack_int8_splits_codes_into_nibble_planes():
    """Int8 blob: high nibbles (offset + 8) where the int4 codes go, low
    nibbles in planes after the scales; q = 16 hi + lo for every code."""
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, codec="int8")
    w = synth.gen_layer(cfg, seed=0)
    nb = B.moe_expert_bytes(cfg)
    assert nb == cfg.expert_bytes() == 3 * cfg.hidden * cfg.inter + 3 * cfg.hidden * cfg.inter // 16
    blob = np.empty(nb, np.uint8)
    B.moe_expert_pack(cfg, *w.expert_arrays(2), blob)
    n = cfg.hidden * cfg.inter // 2
    s_bytes = 3 * cfg.hidden * cfg.inter // 16
    for m, q in enumerate((w.gate_q[2], w.up_q[2], w.down_q[2])):
        hi = blob[m * n:(m + 1) * n]
        lo = blob[3 * n + s_bytes + m * n:3 * n + s_bytes + (m + 1) * n]
        hi_n = np.stack([hi & 15, hi >> 4], axis=-1).reshape(-1).astype(np.int64) - 8
        lo_n = np.stack([lo & 15, lo >> 4], axis=-1).reshape(-1).astype(np.int64)
        np.testing.assert_array_equal(16 * hi_n + lo_n, q.ravel().view(np.int8).astype(np.int64))
    sc = blob[3 * n:3 * n + s_bytes].view(np.uint16)
    m = sc.size // 3
    gs, us, ds = w.gate_s[2], w.up_s[2], w.down_s[2]
    np.testing.assert_array_equal(np.sort(sc[:2 * m]), np.sort(np.concatenate([gs.ravel(), us.ravel()])))
    np.testing.assert_array_equal(np.sort(sc[2 * m:]), np.sort(ds.ravel()))


def test_pack_int2_pairs_rows_in_nibbles():
    """Int2 blob: stored row v holds rows 2v (bits 0-1) and 2v + 1 (bits 2-3)
    of every column, each code + 2; the even and odd rows' scales are each a
    permutation of the public ones."""
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, codec="int2")
    w = synth.gen_layer(cfg, seed=0)
    nb = B.moe_expert_bytes(cfg)
    assert nb == cfg.expert_bytes() == 3 * cfg.hidden * cfg.inter // 4 + 3 * cfg.hidden * cfg.inter // 16
    blob = np.empty(nb, np.uint8)
    B.moe_expert_pack(cfg, *w.expert_arrays(1), blob)
    H, I = cfg.hidden, cfg.inter
    n = H * I // 4
    for m, (q, rows, cols) in enumerate(((w.gate_q[1], I, H), (w.up_q[1], I, H), (w.down_q[1], H, I))):
        plane = blob[m * n:(m + 1) * n].reshape(rows // 2, cols // 2)
        nib = np.stack([plane & 15, plane >> 4], axis=-1).reshape(rows // 2, cols).astype(np.int64)
        f = np.stack([(q >> (2 * t)) & 3 for t in range(4)], axis=-1).reshape(rows, cols).astype(np.int64)
        codes = np.where(f >= 2, f - 4, f)
        np.testing.assert_array_equal((nib & 3) - 2, codes[0::2])
        np.testing.assert_array_equal((nib >> 2) - 2, codes[1::2])
    sc = blob[3 * n:].view(np.uint16)
    gs, us, ds = w.gate_s[1], w.up_s[1], w.down_s[1]
    g_ev, g_od = np.concatenate([gs[0::2].ravel(), us[0::2].ravel()]), np.concatenate([gs[1::2].ravel(), us[1::2].ravel()])
    k = g_ev.size
    d = ds.size // 2
    np.testing.assert_array_equal(np.sort(sc[:k]), np.sort(g_ev))
    np.testing.assert_array_equal(np.sort(sc[k:k + d]), np.sort(ds[0::2].ravel()))
    np.testing.assert_array_equal(np.sort(sc[k + d:2 * k + d]), np.sort(g_od))
    np.testing.assert_array_equal(np.sort(sc[2 * k + d:]), np.sort(ds[1::2].ravel()))


def test_pack_rejects_null():
    code = B.lib().moe_expert_pack(B.MoeConfig.from_cfg(synth.TINY), None, None, None, None, None, None, None)
    assert code == B.MOE_EINVAL


def test_lru_oracle_textbook_pins():
    # Textbook LRU example: reference string 1 2 3 4 1 2 5 1 2 3 4 5 gives
    # 10 faults with 3 frames and 8 with 4 frames (one expert per token).
    ref = [[v] for v in (1, 2, 3, 4, 1, 2, 5, 1, 2, 3, 4, 5)]
    assert lru.replay(ref, 3)[1] == 10
    assert lru.replay(ref, 4)[1] == 8
    # enough slots for every expert: only compulsory misses
    rng = np.random.default_rng(0)
    tr = np.array([rng.choice(32, 4, replace=False) for _ in range(100)])
    h, m, e = lru.replay(tr, 32)
    assert m == len(np.unique(tr)) and e == 0 and h + m == tr.size


def test_lru_oracle_pinned_hand_worked():
    # Worked by hand: 3 slots, top-2 routing, expert 0 pinned (LRU keeps 2).
    #   t0 [0,1]: 0 pinned hit, 1 miss            LRU [1]
    #   t1 [2,0]: 2 miss, 0 hit                    LRU [1,2]
    #   t2 [1,3]: 1 hit; 3 miss evicts 2           LRU [1,3]
    #   t3 [2,1]: 2 miss evicts 3 (1 is needed); 1 hit
    tr = [[0, 1], [2, 0], [1, 3], [2, 1]]
    assert lru.replay(tr, 3, pinned=[0]) == (4, 4, 2)
    # the same trace without the pin: 3 hits, 5 misses, 2 evictions
    assert lru.replay(tr, 3) == (3, 5, 2)
    # every expert of the trace pinned: no miss at all
    assert lru.replay(tr, 4, pinned=[0, 1, 2, 3]) == (8, 0, 0)
    # usage counts and the hottest experts (ties to the lower index)
    assert lru.usage(tr, 5) == [2, 3, 2, 1, 0]
    assert lru.hottest(lru.usage(tr, 5), 3) == [1, 0, 2]


def test_lru_prefetch_oracle_hand_worked():
    # Worked by hand: 3 slots, top-2 routing, at most 2 prefetch copies.
    #   t0 [0,1], no prediction: 0 miss, 1 miss              LRU [0,1]
    #   t1 predicted [2,4]: 2 in; 4 in evicts 0              LRU [1,2,4]
    #      [2,3]: 2 hit (prefetched); 3 miss evicts 1         LRU [4,2,3]
    #   t2 predicted [0,1]: 0 in evicts 4 (never used); 1 in evicts 2
    #      [0,2]: 0 hit (prefetched); 2 miss evicts 3         LRU [1,0,2]
    r = lru.replay_prefetch([[0, 1], [2, 3], [0, 2]], [None, [2, 4], [0, 1]], 3, max_prefetch=2)
    assert r == dict(hits=2, misses=4, evictions=5, prefetches=4, prefetch_hits=2, predicted_uses=4,
                     predicted_hits=2)
    # a limit of one copy per token:
    #   t1 predicted [2,4]: 2 in (free slot), 4 over the limit     LRU [0,1,2]
    #      [2,3]: 2 hit (prefetched); 3 miss evicts 0               LRU [1,2,3]
    #   t2 predicted [0,1]: 0 in evicts 2 (1 is predicted itself); 1 resident
    #                                                               LRU [1,3,0]
    #      [0,2]: 0 hit (prefetched); 2 miss evicts 1               LRU [3,0,2]
    r = lru.replay_prefetch([[0, 1], [2, 3], [0, 2]], [None, [2, 4], [0, 1]], 3, max_prefetch=1)
    assert r == dict(hits=2, misses=4, evictions=3, prefetches=2, prefetch_hits=2, predicted_uses=4,
                     predicted_hits=2)


@pytest.mark.parametrize("slots,n_pin", [(8, 0), (16, 0), (16, 6), (64, 56)])
def test_lru_prefetch_oracle_reductions(slots, n_pin):
    """No prediction, or a limit of zero copies, reduces to plain replay; a
    perfect prediction leaves no miss; the counts stay consistent."""
    rng = np.random.default_rng(slots + n_pin)
    E, k = 256, 8
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    trace = np.array([rng.choice(E, k, replace=False, p=p) for _ in range(300)], np.int32)
    pins = lru.hottest(lru.usage(trace[:100], E), n_pin)
    base = lru.replay(trace, slots, pinned=pins)
    none = lru.replay_prefetch(trace, [None] * len(trace), slots, pinned=pins)
    assert (none["hits"], none["misses"], none["evictions"]) == base and none["prefetches"] == 0
    guess = [rng.choice(E, k, replace=False, p=p) for _ in range(len(trace))]
    zero = lru.replay_prefetch(trace, guess, slots, pinned=pins, max_prefetch=0)
    assert (zero["hits"], zero["misses"], zero["evictions"]) == base and zero["prefetches"] == 0
    perfect = lru.replay_prefetch(trace, trace, slots, pinned=pins)
    assert perfect["misses"] == 0 and perfect["hits"] == trace.size
    assert perfect["predicted_hits"] == perfect["predicted_uses"] == trace.size
    r = lru.replay_prefetch(trace, guess, slots, pinned=pins, max_prefetch=4)
    assert r["hits"] + r["misses"] == trace.size
    assert r["prefetch_hits"] <= r["prefetches"] and r["predicted_hits"] <= r["predicted_uses"] == trace.size
    overlap = sum(len(set(a) & set(b)) for a, b in zip(trace, guess))
    assert r["predicted_hits"] == overlap


@pytest.mark.parametrize("slots,skew", [(8, 0.0), (16, 1.1), (64, 1.1), (64, 0.0)])
def test_cache_policy_matches_lru_replay(slots, skew):
    rng = np.random.default_rng(slots)
    E, k = 256, 8
    p = 1.0 / np.arange(1, E + 1) ** skew
    p /= p.sum()
    trace = np.array([rng.choice(E, k, replace=False, p=p) for _ in range(400)], np.int32)
    assert B.expert_cache_replay(E, slots, k, trace) == lru.replay(trace, slots)
    # with the hottest experts of a separate learning trace pinned
    learn = np.array([rng.choice(E, k, replace=False, p=p) for _ in range(200)], np.int32)
    for n_pin in sorted({1, (slots - k) // 2, slots - k}):
        if n_pin > slots - k:
            continue  # pins must leave top_k slots
        pins = lru.hottest(lru.usage(learn, E), n_pin)
        assert B.expert_cache_replay(E, slots, k, trace, pinned=pins) == lru.replay(trace, slots, pinned=pins)


@pytest.mark.parametrize("slots,n_pin,max_prefetch", [(16, 0, 0), (16, 6, 3), (64, 56, 8), (12, 4, 1), (8, 0, 2)])
def test_cache_replay_prefetch_matches_oracle(slots, n_pin, max_prefetch):
    """The library's host replay of the prefetching cache equals the oracle's
    on Zipf traces, with predictions drawn from the same prior, rows without a
    prediction and top-p drops (id -1) in both."""
    rng = np.random.default_rng(100 + slots + n_pin)
    E, k = 256, 8
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    trace = np.array([rng.choice(E, k, replace=False, p=p) for _ in range(300)], np.int32)
    guess = np.array([rng.choice(E, k, replace=False, p=p) for _ in range(300)], np.int32)
    trace[rng.random(trace.shape) < 0.1] = -1
    guess[rng.random(guess.shape) < 0.1] = -1
    guess[::7] = -1  # no prediction for these tokens
    pins = lru.hottest(lru.usage(trace[:100], E), n_pin)
    got = B.expert_cache_replay_prefetch(E, slots, k, trace, guess, max_prefetch, pins)
    predicted = [None if (row == -1).all() else row for row in guess]
    ref = lru.replay_prefetch(trace, predicted, slots, pinned=pins, max_prefetch=max_prefetch or k)
    assert got == ref
    assert ref["prefetches"] > 0 and ref["predicted_uses"] > 0


def test_cache_replay_prefetch_rejects_bad_arguments():
    trace = np.zeros((2, 4), np.int32)
    guess = np.full((2, 4), -1, np.int32)
    for bad in (dict(slots=3), dict(max_prefetch=-1)):
        kw = dict(slots=8, max_prefetch=0)
        kw.update(bad)
        with pytest.raises(B.MoeError) as e:
            B.expert_cache_replay_prefetch(16, kw["slots"], 4, trace, guess, kw["max_prefetch"])
        assert e.value.code == B.MOE_EINVAL
    g = guess.copy()
    g[1, 2] = 16
    with pytest.raises(B.MoeError) as e:
        B.expert_cache_replay_prefetch(16, 8, 4, trace, g)
    assert e.value.code == B.MOE_EINVAL
    with pytest.raises(B.MoeError) as e:
        B.moe_layer_set_next(None, None, 0)
    assert e.value.code == B.MOE_EINVAL
    with pytest.raises(B.MoeError) as e:
        B.expert_cache_timeline(None, True)
    assert e.value.code == B.MOE_EINVAL


def test_cache_replay_skips_dropped_choices():
    """Traces with top-p drops (id -1): the library's replay and the oracle's
    both skip them, and equal the replay of the trace with them removed."""
    rng = np.random.default_rng(17)
    E, slots, k = 32, 10, 4
    trace = np.stack([rng.choice(E, k, replace=False) for _ in range(200)]).astype(np.int32)
    trace[rng.random(trace.shape) < 0.35] = -1
    got = B.expert_cache_replay(E, slots, k, trace)
    assert got == lru.replay(trace, slots)
    kept = [row[row >= 0] for row in trace]
    assert lru.replay(kept, slots) == got
    assert lru.usage(trace, E) == lru.usage(kept, E)
    bad = trace.copy()
    bad[0, 0] = -2
    with pytest.raises(B.MoeError) as e:
        B.expert_cache_replay(E, slots, k, bad)
    assert e.value.code == B.MOE_EINVAL


def test_cache_replay_rejects_too_many_pins():
    tr = np.zeros((1, 4), np.int32) + np.arange(4, dtype=np.int32)
    with pytest.raises(B.MoeError):
        B.expert_cache_replay(16, 8, 4, tr, pinned=list(range(5)))


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_more_than_one_gpu(n):
    # one GPU only: asking for more exits with status 2 and says why, before
    # any device is touched
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", str(n), "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert f"--gpus {n} is not supported" in r.stderr
    assert r.stdout.strip() == ""
