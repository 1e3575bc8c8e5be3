"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle against a closed form, an invariant, a brute-force
enumeration, a library routine (numpy sort / matmul) on weights the test packs
itself, or byte figures printed on the pages.  The checks are chosen so that a
plausible mistake (wrong nibble order or sign, wrong scale group, a dropped
bias, masked experts treated as 0 instead of ineligible, unnormalised weights,
a missing shared expert, a transposed operand) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle
from routed_expert_int4_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers
def pack_int4(q: np.ndarray) -> np.ndarray:
    """Test-side packer: integer matrix [R, C] in [-8, 7] -> public bytes [R, C/2]
    (two's complement nibbles, even column in the low nibble)."""
    q = np.asarray(q, dtype=np.int64)
    assert q.min() >= -8 and q.max() <= 7 and q.shape[1] % 2 == 0
    nib = (q & 15).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def f16_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def dense(q, s_bits):
    """Dense fp64 matrix from integer codes [R, C] and fp16 scale bits [R, C/32]."""
    s = s_bits.view(np.float16).astype(np.float64)
    return np.asarray(q, np.float64) * np.repeat(s, 32, axis=1)


def silu(z):
    return z / (1.0 + np.exp(-z))


def brute_force_select(s, sb, n_groups, topk_group, top_k, rsf):
    """Exhaustive reading of group-limited top-k on tiny shapes.

    Group score = max over pairs in the group of sb_a + sb_b (the sum of the
    two largest).  Kept groups = the topk_group-subset with the largest total
    group score.  Chosen experts = the top_k-subset of eligible experts with
    the largest total sb.  Ties are not handled (inputs are continuous)."""
    E = len(sb)
    gsz = E // n_groups
    gscore = [max(sb[a] + sb[b] for a, b in itertools.combinations(range(g * gsz, (g + 1) * gsz), 2))
              for g in range(n_groups)]
    best_groups = max(itertools.combinations(range(n_groups), topk_group), key=lambda c: sum(gscore[g] for g in c))
    elig = [e for g in best_groups for e in range(g * gsz, (g + 1) * gsz)]
    best = max(itertools.combinations(elig, top_k), key=lambda c: sum(sb[e] for e in c))
    chosen = sorted(best, key=lambda e: -sb[e])
    w = np.array([rsf * s[e] for e in chosen]) / sum(s[e] for e in chosen)
    return np.array(chosen), w


def dense_layer(wts, x_f64):
    """Independent recomputation of one token with numpy matmuls on densely
    dequantised weights and brute-force routing (tiny shapes only)."""
    cfg = wts.cfg
    logit = wts.router_w.astype(np.float64) @ x_f64
    s = 1.0 / (1.0 + np.exp(-logit))
    sb = s + wts.bias.astype(np.float64)
    ids, w = brute_force_select(s, sb, cfg.n_groups, cfg.topk_group, cfg.top_k, cfg.routed_scaling_factor)

    def unpack(b):
        lo = (b & 15).astype(np.int64)
        hi = (b >> 4).astype(np.int64)
        q = np.empty((b.shape[0], b.shape[1] * 2), np.int64)
        q[:, 0::2], q[:, 1::2] = lo, hi
        return np.where(q >= 8, q - 16, q)

    def ffn(e):
        G = dense(unpack(wts.gate_q[e]), wts.gate_s[e])
        U = dense(unpack(wts.up_q[e]), wts.up_s[e])
        D = dense(unpack(wts.down_q[e]), wts.down_s[e])
        g = G @ x_f64
        return D @ (silu(g) * (U @ x_f64))

    y = sum(wj * ffn(e) for wj, e in zip(w, ids))
    for sh in range(cfg.n_shared):
        y = y + ffn(cfg.n_experts + sh)
    return y, ids, w


@pytest.fixture(scope="module")
def tiny():
    return synth.gen_layer(synth.TINY, seed=0)


@pytest.fixture(scope="module")
def tiny_x():
    return synth.gen_tokens(synth.TINY, 4, seed=1)


# ----------------------------------------------------------------- P1/P2: dequant + expert FFN
def test_expert_unit_vector_pins_nibbles_and_scale_groups():
    """x = e_c gives g_i = W_g[i, c] and u_i = W_u[i, c]: pins nibble order,
    two's complement and which 32-column group a scale covers."""
    rng = np.random.default_rng(11)
    H, I = 64, 32
    Qg = rng.integers(-8, 8, size=(I, H))
    Qu = rng.integers(-8, 8, size=(I, H))
    Qd = rng.integers(-8, 8, size=(H, I))
    Qg[0, :] = -8
    Qg[1, :] = 7
    Sg = f16_bits(np.exp(rng.normal(-1, 0.5, size=(I, H // 32))))
    Su = f16_bits(np.exp(rng.normal(-1, 0.5, size=(I, H // 32))))
    Sd = f16_bits(np.exp(rng.normal(-1, 0.5, size=(H, I // 32))))
    args = (pack_int4(Qg), Sg, pack_int4(Qu), Su, pack_int4(Qd), Sd)
    for c in (0, 1, 2, 31, 32, 33, 63):
        x = np.zeros(H)
        x[c] = 1.0
        d, h = oracle.expert_ffn(H, I, *args, x)
        g = Qg[:, c] * Sg.view(np.float16).astype(np.float64)[:, c // 32]
        u = Qu[:, c] * Su.view(np.float16).astype(np.float64)[:, c // 32]
        np.testing.assert_allclose(h, silu(g) * u, rtol=1e-14, atol=0)
        # down projection against numpy's matmul on the test's own dense matrix
        np.testing.assert_allclose(d, dense(Qd, Sd) @ h, rtol=1e-12, atol=1e-14)


def test_expert_hand_computed_toy():
    """32x32 toy with every code 1 and every scale 1: g = u = sum(x),
    h = silu(sum x) * sum x, d_r = 32 h."""
    H = I = 32
    ones = np.ones((I, H), np.int64)
    S = f16_bits(np.ones((I, 1)))
    x = np.full(H, 0.5)
    d, h = oracle.expert_ffn(H, I, pack_int4(ones), S, pack_int4(ones), S, pack_int4(ones), S, x)
    sx = 16.0
    h_ref = sx / (1.0 + math.exp(-sx)) * sx
    assert np.allclose(h, h_ref, rtol=1e-15)
    assert np.allclose(d, 32.0 * h_ref, rtol=1e-15)


def test_expert_zero_input_and_extreme_codes():
    rng = np.random.default_rng(3)
    H, I = 64, 64
    args = []
    for shape in ((I, H), (I, H), (H, I)):
        args += [pack_int4(rng.integers(-8, 8, size=shape)), f16_bits(np.full((shape[0], shape[1] // 32), 0.25))]
    d, h = oracle.expert_ffn(H, I, *args, np.zeros(H))
    assert np.all(h == 0) and np.all(d == 0)
    # fp16 scale at the top of its range and subnormal scales decode exactly
    S = f16_bits(np.array([[65504.0, 2.0 ** -24]]))
    q = np.zeros((1, 64), np.int64)
    q[0, 0], q[0, 40] = 7, -8
    x = np.zeros(64)
    x[0], x[40] = 1.0, 1.0
    Sd = f16_bits(np.ones((64, 1)))
    qd = np.zeros((64, 1 * 32 // 1), np.int64)[:, :32]
    d, h = oracle.expert_ffn(64, 32, pack_int4(np.vstack([q] * 32)), np.vstack([S] * 32),
                             pack_int4(np.vstack([q] * 32)), np.vstack([S] * 32),
                             pack_int4(qd), Sd, x)
    g = 7 * 65504.0 + (-8) * 2.0 ** -24
    assert np.allclose(h, silu(g) * g, rtol=1e-15)


# ----------------------------------------------------------------- P3-P6: routing
def test_weights_sum_to_rsf_and_are_positive(tiny, tiny_x):
    out = oracle.layer_forward(tiny, tiny_x)
    rsf = tiny.cfg.routed_scaling_factor
    assert np.allclose(out["w"].sum(axis=1), rsf, rtol=0, atol=1e-12)
    assert np.all(out["w"] > 0) and np.all(out["w"] < rsf)


def test_selection_matches_brute_force_tiny():
    """Exhaustive enumeration over group pairs and expert subsets (tiny shape),
    many random score vectors, including negative biased scores (where a
    zero-fill of masked experts would differ from treating them as ineligible)."""
    rng = np.random.default_rng(5)
    cfg = synth.TINY
    for trial in range(300):
        s = 1 / (1 + np.exp(-rng.normal(0, 2, size=cfg.n_experts)))
        bias = rng.normal(0, 0.01 if trial % 2 else 1.0, size=cfg.n_experts)
        sb = s + bias
        ids, w, gap = oracle.select(cfg.n_groups, cfg.topk_group, cfg.top_k, cfg.routed_scaling_factor, s, sb)
        ref_ids, ref_w = brute_force_select(s, sb, cfg.n_groups, cfg.topk_group, cfg.top_k, cfg.routed_scaling_factor)
        assert list(ids) == list(ref_ids), trial
        np.testing.assert_allclose(w, ref_w, rtol=1e-13)
        assert gap > 0


def test_selection_glm_shape_against_argsort():
    """GLM shape: all C(8,4)=70 group subsets enumerated, experts by numpy argsort."""
    rng = np.random.default_rng(6)
    cfg = synth.GLM
    gsz = cfg.n_experts // cfg.n_groups
    for trial in range(50):
        s = 1 / (1 + np.exp(-rng.normal(0, 1.6, size=cfg.n_experts)))
        sb = s + rng.normal(0, 0.01 if trial % 2 else 0.5, size=cfg.n_experts)
        gscore = [np.sort(sb[g * gsz:(g + 1) * gsz])[-2:].sum() for g in range(cfg.n_groups)]
        groups = max(itertools.combinations(range(cfg.n_groups), cfg.topk_group), key=lambda c: sum(gscore[g] for g in c))
        elig = np.array([e for g in groups for e in range(g * gsz, (g + 1) * gsz)])
        ref = elig[np.argsort(-sb[elig], kind="stable")[: cfg.top_k]]
        ids, w, _ = oracle.select(cfg.n_groups, cfg.topk_group, cfg.top_k, cfg.routed_scaling_factor, s, sb)
        assert list(ids) == list(ref)


@pytest.mark.parametrize("n_groups,topk_group", [(4, 4), (1, 1)])
def test_selection_reduces_to_plain_topk(n_groups, topk_group):
    rng = np.random.default_rng(7)
    for _ in range(100):
        s = rng.uniform(0.01, 0.99, size=16)
        sb = s + rng.normal(0, 0.3, size=16)
        ids, w, _ = oracle.select(n_groups, topk_group, 4, 1.0, s, sb)
        assert list(ids) == list(np.argsort(-sb, kind="stable")[:4])
        np.testing.assert_allclose(w, s[ids] / s[ids].sum(), rtol=1e-14)


def test_selection_ties_go_to_lower_index():
    s = np.full(16, 0.5)
    sb = np.full(16, 0.5)
    ids, w, gap = oracle.select(4, 2, 4, 2.5, s, sb)
    assert list(ids) == [0, 1, 2, 3] and gap == 0.0
    np.testing.assert_allclose(w, 2.5 / 4)


def test_gap_is_the_selection_margin():
    s = np.full(16, 0.5)
    sb = np.array([0.9, 0.8, 0.1, 0.0, 0.7, 0.6, 0.05, 0.0, 0.3, 0.2, 0.0, 0.0, 0.1, 0.1, 0.0, 0.0])
    # group scores 1.7, 1.3, 0.5, 0.2 -> groups 0,1 kept (margin 0.8); experts
    # 0.9,0.8,0.7,0.6 chosen, next eligible 0.1 -> margin 0.5
    ids, _, gap = oracle.select(4, 2, 4, 1.0, s, sb)
    assert list(ids) == [0, 1, 4, 5]
    assert abs(gap - 0.5) < 1e-15


def test_zero_input_routes_on_bias_and_returns_shared_only_output(tiny):
    """x = 0: every s = 1/2, selection is group-limited top-k of the bias alone,
    each weight is rsf/k and y = the shared expert's output = 0."""
    cfg = tiny.cfg
    x = np.zeros((2, cfg.hidden), np.uint16)
    out = oracle.layer_forward(tiny, x)
    ref_ids, _ = brute_force_select(np.full(cfg.n_experts, 0.5), 0.5 + tiny.bias.astype(np.float64),
                                    cfg.n_groups, cfg.topk_group, cfg.top_k, cfg.routed_scaling_factor)
    assert list(out["ids"][0]) == list(ref_ids)
    np.testing.assert_array_equal(out["w"], np.full_like(out["w"], cfg.routed_scaling_factor / cfg.top_k))
    assert np.all(out["y"] == 0.0)


# ----------------------------------------------------------------- whole layer
def test_layer_matches_dense_numpy_with_brute_force_routing(tiny, tiny_x):
    out = oracle.layer_forward(tiny, tiny_x)
    xf = synth.bf16_bits_to_f32(tiny_x).astype(np.float64)
    for t in range(tiny_x.shape[0]):
        y, ids, w = dense_layer(tiny, xf[t])
        assert list(out["ids"][t]) == list(ids)
        np.testing.assert_allclose(out["w"][t], w, rtol=1e-13)
        np.testing.assert_allclose(out["y"][t], y, rtol=1e-11, atol=1e-12 * np.abs(y).max())


def test_routed_off_gives_shared_expert_output(tiny, tiny_x):
    import dataclasses
    wts = dataclasses.replace(tiny, gate_q=tiny.gate_q.copy(), up_q=tiny.up_q.copy(), down_q=tiny.down_q.copy())
    E = tiny.cfg.n_experts
    wts.gate_q[:E] = 0
    wts.up_q[:E] = 0
    wts.down_q[:E] = 0
    out = oracle.layer_forward(wts, tiny_x)
    xf = synth.bf16_bits_to_f32(tiny_x).astype(np.float64)
    for t in range(tiny_x.shape[0]):
        d, _ = oracle.expert_ffn(tiny.cfg.hidden, tiny.cfg.inter, *tiny.expert_arrays(E), xf[t])
        np.testing.assert_array_equal(out["y"][t], d)
        assert np.any(d != 0)


def test_rsf_scales_routed_part_linearly(tiny, tiny_x):
    import dataclasses
    base = oracle.layer_forward(tiny, tiny_x)
    cfg2 = dataclasses.replace(tiny.cfg, routed_scaling_factor=2 * tiny.cfg.routed_scaling_factor)
    out2 = oracle.layer_forward(dataclasses.replace(tiny, cfg=cfg2), tiny_x)
    xf = synth.bf16_bits_to_f32(tiny_x).astype(np.float64)
    E = tiny.cfg.n_experts
    for t in range(tiny_x.shape[0]):
        ds, _ = oracle.expert_ffn(tiny.cfg.hidden, tiny.cfg.inter, *tiny.expert_arrays(E), xf[t])
        np.testing.assert_allclose(out2["y"][t] - ds, 2 * (base["y"][t] - ds), rtol=1e-12, atol=1e-12)


def test_permuting_experts_within_a_group_maps_ids(tiny, tiny_x):
    import dataclasses
    cfg = tiny.cfg
    gsz = cfg.n_experts // cfg.n_groups
    perm = np.arange(cfg.n_experts)
    rng = np.random.default_rng(9)
    for g in range(cfg.n_groups):
        perm[g * gsz:(g + 1) * gsz] = rng.permutation(np.arange(g * gsz, (g + 1) * gsz))
    full = np.concatenate([perm, np.arange(cfg.n_experts, cfg.n_total_experts)])
    wp = dataclasses.replace(
        tiny, router_w=tiny.router_w[perm].copy(), bias=tiny.bias[perm].copy(),
        gate_q=tiny.gate_q[full].copy(), gate_s=tiny.gate_s[full].copy(), up_q=tiny.up_q[full].copy(),
        up_s=tiny.up_s[full].copy(), down_q=tiny.down_q[full].copy(), down_s=tiny.down_s[full].copy())
    a = oracle.layer_forward(tiny, tiny_x)
    b = oracle.layer_forward(wp, tiny_x)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(inv[a["ids"]], b["ids"])
    np.testing.assert_array_equal(a["y"], b["y"])


def test_tokens_are_independent(tiny):
    x = synth.gen_tokens(tiny.cfg, 6, seed=4)
    full = oracle.layer_forward(tiny, x)
    for t in range(6):
        one = oracle.layer_forward(tiny, x[t:t + 1])
        np.testing.assert_array_equal(one["y"][0], full["y"][t])
        np.testing.assert_array_equal(one["ids"][0], full["ids"][t])


def test_forced_ids_reweight_over_the_forced_set(tiny, tiny_x):
    out = oracle.layer_forward(tiny, tiny_x, want_logits=True)
    forced = np.tile(np.array([[3, 0, 9, 12]], np.int32), (tiny_x.shape[0], 1))
    f = oracle.layer_forward(tiny, tiny_x, forced_ids=forced)
    s = 1 / (1 + np.exp(-out["logits"]))
    ref_w = tiny.cfg.routed_scaling_factor * s[:, [3, 0, 9, 12]] / s[:, [3, 0, 9, 12]].sum(axis=1, keepdims=True)
    np.testing.assert_allclose(f["w"], ref_w, rtol=1e-13)
    np.testing.assert_array_equal(f["ids"], forced)


def test_router_logits_against_numpy(tiny, tiny_x):
    out = oracle.layer_forward(tiny, tiny_x, want_logits=True)
    xf = synth.bf16_bits_to_f32(tiny_x).astype(np.float64)
    np.testing.assert_allclose(out["logits"], xf @ tiny.router_w.astype(np.float64).T, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------- P10: bytes vs the pages
def test_byte_accounting_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "byte_accounting.json")))
    H, I, E, K, L = 6144, 2048, 256, 8, 75
    n = 3 * H * I  # weights per expert

    def close(key, v):
        ref = g[key]
        assert abs(v - ref["value"]) <= ref["rtol"] * ref["value"], (key, v, ref)

    close("int4_codes_per_expert_bytes", n // 2)
    close("int4_routed_bytes_per_token", K * L * n // 2)
    close("int4_routed_experts_on_disk_bytes", (L + 1) * E * n // 2)
    mxfp4 = n * 4.25 / 8
    close("mxfp4_routed_gib_per_token", K * L * mxfp4 / 2 ** 30)
    close("mxfp4_gib_per_s_for_5_tok_s", 5 * K * L * mxfp4 / 2 ** 30)
    close("bf16_active_bytes_per_token", K * L * n * 2)
    close("bf16_bytes_per_layer", E * n * 2)
    close("bf16_whole_layer_bytes_per_token", L * E * n * 2)
    close("int4_all_experts_bytes", L * E * synth.GLM.expert_bytes())
    assert synth.GLM.expert_bytes() == 21_233_664
    assert synth.TINY.expert_bytes() == 55_296


def test_generator_is_deterministic_and_codes_uniform():
    a = synth.gen_layer(synth.TINY, seed=0)
    b = synth.gen_layer(synth.TINY, seed=0)
    np.testing.assert_array_equal(a.gate_q, b.gate_q)
    np.testing.assert_array_equal(a.router_w, b.router_w)
    nib = np.concatenate([(a.gate_q & 15).ravel(), (a.gate_q >> 4).ravel()])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.8 * counts.mean()


# ---------------------------------------------------------------- dispatch
def test_dispatch_hand_example():
    from oracle.dispatch import dispatch
    # 3 tokens, top-2, 4 experts: entries 0..5 = (0,0) (0,1) (1,0) (1,1) (2,0) (2,1)
    ids = np.array([[2, 0], [0, 3], [2, 0]])
    r = dispatch(ids, 4)
    assert r["counts"].tolist() == [3, 0, 2, 1]
    assert r["offsets"].tolist() == [0, 3, 3, 5, 6]
    assert r["perm"].tolist() == [1, 2, 5, 0, 4, 3]
    assert r["distinct"].tolist() == [0, 2, 3]


def test_dispatch_hand_example_with_dropped_choices():
    from oracle.dispatch import dispatch
    # the same routing with entries (0,1) and (2,0) dropped by a top-p cut
    ids = np.array([[2, -1], [0, 3], [-1, 0]])
    r = dispatch(ids, 4)
    assert r["counts"].tolist() == [2, 0, 1, 1]
    assert r["offsets"].tolist() == [0, 2, 2, 3, 4]
    assert r["perm"].tolist() == [2, 5, 0, 3, -1, -1]
    assert r["distinct"].tolist() == [0, 2, 3]


def test_dispatch_invariants_random():
    from oracle.dispatch import dispatch
    rng = np.random.default_rng(5)
    for T, K, E in [(1, 8, 256), (32, 8, 256), (7, 4, 16), (100, 6, 64)]:
        ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
        r = dispatch(ids, E)
        flat = ids.reshape(-1)
        perm = r["perm"]
        assert sorted(perm.tolist()) == list(range(T * K))           # a permutation
        keys = [(flat[p], p) for p in perm]
        assert keys == sorted(keys)                                    # expert, then entry order
        for e in range(E):                                             # offsets delimit each expert
            seg = perm[r["offsets"][e]:r["offsets"][e + 1]]
            assert all(flat[p] == e for p in seg) and len(seg) == r["counts"][e]
        assert r["distinct"].tolist() == sorted(set(flat.tolist()))
        assert r["offsets"][-1] == T * K


def test_dispatch_degenerate():
    from oracle.dispatch import dispatch
    r = dispatch(np.full((5, 1), 7), 8)                                # one expert takes everything
    assert r["counts"].tolist() == [0] * 7 + [5] and r["perm"].tolist() == [0, 1, 2, 3, 4]
    assert r["distinct"].tolist() == [7]
    r = dispatch(np.zeros((0, 4), np.int32), 8)                        # empty routing
    assert r["counts"].sum() == 0 and len(r["perm"]) == 0 and len(r["distinct"]) == 0


def test_top_p_hand_worked():
    # Selection of 4 of 8 experts (two groups, both kept), zero bias:
    # ids by sb = [0, 6, 2, 7], shares by s = 0.9, 0.8, 0.6, 0.4 over 2.7.
    s = np.array([0.9, 0.1, 0.6, 0.3, 0.2, 0.05, 0.8, 0.4])
    ids, w, _, pgap = oracle.select(2, 2, 4, 2.5, s, s.copy(), top_p=0.6, with_pgap=True)
    # shares before each: 0, 1/3 (kept), 0.6296 (>= 0.6: dropped), 0.8519 (dropped)
    assert list(ids) == [0, 6, -1, -1]
    assert np.allclose(w, [2.5 * 0.9 / 1.7, 2.5 * 0.8 / 1.7, 0.0, 0.0], rtol=0, atol=1e-15)
    assert abs(pgap - (1.7 / 2.7 - 0.6)) < 1e-15
    # a bias that moves expert 7 first in the selection order does not change
    # which experts top-p keeps (it ranks by s), only their slots
    sb = s.copy()
    sb[7] += 1.0
    ids, w, _ = oracle.select(2, 2, 4, 2.5, s, sb, top_p=0.6)
    assert list(ids) == [-1, 0, 6, -1]
    assert np.allclose(w, [0.0, 2.5 * 0.9 / 1.7, 2.5 * 0.8 / 1.7, 0.0], rtol=0, atol=1e-15)
    # a tiny top_p keeps the single largest share; top_p = 1 is plain top-k
    ids, w, _ = oracle.select(2, 2, 4, 2.5, s, sb, top_p=1e-9)
    assert list(ids) == [-1, 0, -1, -1] and abs(w[1] - 2.5) < 1e-15
    ids1, w1, g1 = oracle.select(2, 2, 4, 2.5, s, sb, top_p=1.0)
    ids0, w0, g0 = oracle.select(2, 2, 4, 2.5, s, sb)
    assert list(ids1) == list(ids0) == [7, 0, 6, 2] and np.array_equal(w1, w0)


def test_top_p_layer_matches_forced_kept_experts(tiny, tiny_x):
    import dataclasses
    # the layer with top-p equals the layer forced onto the kept experts
    # (empty slots skipped, weights renormalised over the kept ones)
    cfg = dataclasses.replace(tiny.cfg, top_p=0.7)
    wp = dataclasses.replace(tiny, cfg=cfg)
    out = oracle.layer_forward(wp, tiny_x)
    assert (out["ids"] < 0).any(), "top_p = 0.7 should drop some slot on the tiny tokens"
    forced = oracle.layer_forward(tiny, tiny_x, forced_ids=out["ids"])
    assert np.array_equal(out["y"], forced["y"])
    assert np.allclose(out["w"], forced["w"], rtol=0, atol=1e-15)
    # kept weights sum to rsf for every token; at least one expert is kept
    assert np.allclose(out["w"].sum(axis=1), cfg.routed_scaling_factor, rtol=0, atol=1e-12)
    assert ((out["ids"] >= 0).sum(axis=1) >= 1).all()


# ----------------------------------------------------------------- MXFP4 codec
# The OCP Microscaling (MX) v1.0 FP4 (E2M1) value set, listed as the standard's
# table gives it (the oracle computes it from the bit fields instead), and the
# E8M0 scale 2^(b - 127).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def pack_nibbles(n: np.ndarray) -> np.ndarray:
    """Nibble matrix [R, C] (0..15) -> bytes [R, C/2], even column in the low nibble."""
    n = np.asarray(n, dtype=np.uint8)
    return (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)


def test_mxfp4_every_code_and_scale_decodes_to_the_standard_value():
    """Row r holds code r in every column; with x = e_c the matvec returns
    the weight W[r, c]: every E2M1 code, both nibble positions, several E8M0
    scale bytes including the extremes 0 (2^-127) and 254 (2^127)."""
    rows, cols = 16, 64
    codes = np.repeat(np.arange(16, dtype=np.uint8)[:, None], cols, axis=1)
    for b0, b1 in ((127, 127), (126, 130), (0, 254), (100, 1)):
        s = np.array([[b0, b1]] * rows, np.uint8)
        for c in (0, 1, 30, 31, 32, 33, 62, 63):
            x = np.zeros(cols)
            x[c] = 1.0
            y = oracle.matvec(pack_nibbles(codes), s, x, codec="mxfp4")
            b = b0 if c < 32 else b1
            want = np.array([E2M1_TABLE[r] * 2.0 ** (b - 127) for r in range(16)])
            np.testing.assert_array_equal(y, want)
    # scale byte 255 is NaN: it poisons its row (NaN * 0 is NaN), not the others
    s = np.array([[127, 127]] * rows, np.uint8)
    s[5, 1] = 255
    x = np.zeros(cols)
    x[40] = 1.0
    y = oracle.matvec(pack_nibbles(codes), s, x, codec="mxfp4")
    assert np.isnan(y[5])
    np.testing.assert_array_equal(np.delete(y, 5), np.delete(np.array(E2M1_TABLE), 5))


def test_mxfp4_mixed_nibbles_against_numpy():
    """Random codes and scales: the oracle's matvec equals numpy's product of
    x with the test's own dense matrix (table lookup, low nibble first)."""
    rng = np.random.default_rng(21)
    rows, cols = 24, 96
    nib = rng.integers(0, 16, size=(rows, cols))
    s = rng.integers(110, 140, size=(rows, cols // 32)).astype(np.uint8)
    W = np.array(E2M1_TABLE)[nib] * np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    x = rng.normal(size=cols)
    np.testing.assert_allclose(oracle.matvec(pack_nibbles(nib), s, x, codec="mxfp4"), W @ x, rtol=1e-13, atol=1e-15)


def test_mxfp4_layer_equals_int4_layer_on_shared_values():
    """An MXFP4 layer whose codes take only integer values {0, +-1, +-2, +-3,
    +-4, +-6} and whose scales are powers of two within fp16's range is the
    same layer as the int4 one with q = value and fp16 scale = 2^(b - 127):
    the oracle gives bit-identical routing and outputs for both codecs."""
    import dataclasses
    cfg4 = synth.TINY
    cfg_fp4 = dataclasses.replace(cfg4, codec="mxfp4")
    base = synth.gen_layer(cfg4, seed=3)
    rng = np.random.default_rng(5)
    int_codes = np.array([0, 2, 4, 5, 6, 7, 8, 10, 12, 13, 14, 15])  # E2M1 codes with integer values
    int_vals = np.array([E2M1_TABLE[c] for c in int_codes]).astype(np.int64)

    def make(shape_q):
        n = int_codes[rng.integers(0, len(int_codes), size=(shape_q[0], shape_q[1] * 2))]
        q = np.array([int_vals[list(int_codes).index(c)] for c in n.ravel()]).reshape(n.shape)
        b = rng.integers(127 - 12, 127 + 8, size=(shape_q[0], shape_q[1] * 2 // 32)).astype(np.uint8)
        return pack_nibbles(n), b, pack_int4(q), f16_bits(2.0 ** (b.astype(np.float64) - 127))

    fp4, i4 = {}, {}
    for name in ("gate", "up", "down"):
        qs = getattr(base, name + "_q")
        parts = [make(qs.shape[1:]) for _ in range(qs.shape[0])]
        fp4[name + "_q"] = np.stack([p[0] for p in parts])
        fp4[name + "_s"] = np.stack([p[1] for p in parts])
        i4[name + "_q"] = np.stack([p[2] for p in parts])
        i4[name + "_s"] = np.stack([p[3] for p in parts])
    w4 = dataclasses.replace(base, **i4)
    wf = dataclasses.replace(base, cfg=cfg_fp4, **fp4)
    x = synth.gen_tokens(cfg4, 5, seed=6)
    a, b = oracle.layer_forward(w4, x), oracle.layer_forward(wf, x)
    np.testing.assert_array_equal(a["ids"], b["ids"])
    np.testing.assert_array_equal(a["w"], b["w"])
    np.testing.assert_array_equal(a["y"], b["y"])
    assert np.abs(a["y"]).max() > 0


def test_mxfp4_byte_accounting_matches_largerlm():
    """19.125 MiB per GLM-shaped MXFP4 expert (codes + one E8M0 byte per 32
    weights), and 8 experts x 75 layers of it = the 11.206 GiB per token the
    LargerLM README prints."""
    import dataclasses
    g = json.load(open(os.path.join(GOLDEN, "byte_accounting.json")))
    eb = dataclasses.replace(synth.GLM, codec="mxfp4").expert_bytes()
    assert eb == 20_054_016 and eb / 2 ** 20 == 19.125
    ref = g["mxfp4_routed_gib_per_token"]
    assert abs(8 * 75 * eb / 2 ** 30 - ref["value"]) <= ref["rtol"] * ref["value"]


def test_mxfp4_generator_dtypes_and_scale_range():
    import dataclasses
    w = synth.gen_layer(dataclasses.replace(synth.TINY, codec="mxfp4"), seed=0)
    assert w.gate_s.dtype == np.uint8 and w.down_s.dtype == np.uint8
    assert 110 <= int(w.gate_s.min()) and int(w.gate_s.max()) <= 135
    out = oracle.layer_forward(w, synth.gen_tokens(synth.TINY, 3, seed=1))
    assert np.all(np.isfinite(out["y"]))


# ----------------------------------------------------------------- int8 codec
def test_int8_unit_vectors_and_extreme_codes():
    """x = e_c returns column c of W = scale * q for int8 codes, including
    -128 and 127, and the scale group each column falls in."""
    rng = np.random.default_rng(31)
    rows, cols = 8, 96
    q = rng.integers(-128, 128, size=(rows, cols))
    q[0, :] = -128
    q[1, :] = 127
    s = f16_bits(np.exp(rng.normal(-3, 0.5, size=(rows, cols // 32))))
    sc = s.view(np.float16).astype(np.float64)
    for c in (0, 1, 31, 32, 63, 64, 95):
        x = np.zeros(cols)
        x[c] = 1.0
        y = oracle.matvec(q.astype(np.int8).view(np.uint8), s, x, codec="int8")
        np.testing.assert_array_equal(y, q[:, c] * sc[:, c // 32])
    x = rng.normal(size=cols)
    np.testing.assert_allclose(oracle.matvec(q.astype(np.int8).view(np.uint8), s, x, codec="int8"),
                               (q * np.repeat(sc, 32, axis=1)) @ x, rtol=1e-13)


def test_int8_layer_equals_int4_layer_on_shared_codes():
    """An int8 layer whose codes lie in [-8, 7] is the int4 layer with the
    same codes and scales: bit-identical routing and outputs."""
    import dataclasses
    base = synth.gen_layer(synth.TINY, seed=4)
    rng = np.random.default_rng(9)
    i4, i8 = {}, {}
    for name in ("gate", "up", "down"):
        qs = getattr(base, name + "_q")
        q = rng.integers(-8, 8, size=(qs.shape[0], qs.shape[1], qs.shape[2] * 2))
        i4[name + "_q"] = np.stack([pack_int4(m) for m in q])
        i8[name + "_q"] = q.astype(np.int8).view(np.uint8)
    w4 = dataclasses.replace(base, **i4)
    w8 = dataclasses.replace(base, cfg=dataclasses.replace(base.cfg, codec="int8"), **i8)
    x = synth.gen_tokens(synth.TINY, 5, seed=10)
    a, b = oracle.layer_forward(w4, x), oracle.layer_forward(w8, x)
    np.testing.assert_array_equal(a["ids"], b["ids"])
    np.testing.assert_array_equal(a["y"], b["y"])
    assert np.abs(a["y"]).max() > 0


def test_int8_generator_layout():
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, codec="int8")
    w = synth.gen_layer(cfg, seed=0)
    assert w.gate_q.shape == (cfg.n_total_experts, cfg.inter, cfg.hidden)
    assert w.down_q.shape == (cfg.n_total_experts, cfg.hidden, cfg.inter)
    assert cfg.expert_bytes() == 3 * cfg.hidden * cfg.inter + 3 * cfg.hidden * cfg.inter // 16
    y = oracle.layer_forward(w, synth.gen_tokens(cfg, 2, seed=1))["y"]
    assert np.all(np.isfinite(y)) and 0.05 < np.abs(y).max() < 1e3


# ----------------------------------------------------------------- int2 codec
def pack_int2(q: np.ndarray) -> np.ndarray:
    """Test-side packer: integers [R, C] in [-2, 1] -> bytes [R, C/4], column
    4j + t in bits [2t, 2t + 2) of byte j, two's complement."""
    q = np.asarray(q, dtype=np.int64)
    assert q.min() >= -2 and q.max() <= 1 and q.shape[1] % 4 == 0
    f = (q & 3).astype(np.uint8)
    return (f[:, 0::4] | (f[:, 1::4] << 2) | (f[:, 2::4] << 4) | (f[:, 3::4] << 6)).astype(np.uint8)


def test_int2_unit_vectors_every_field_position():
    """x = e_c returns column c of W = scale * q: each of the four 2-bit
    fields of a byte, every code value (-2, -1, 0, 1) and the scale group."""
    rng = np.random.default_rng(41)
    rows, cols = 8, 64
    q = rng.integers(-2, 2, size=(rows, cols))
    q[0, :] = -2
    q[1, :] = 1
    q[2, 0:4] = [-2, -1, 0, 1]
    q[3, 0:4] = [1, 0, -1, -2]
    s = f16_bits(np.exp(rng.normal(-1, 0.5, size=(rows, cols // 32))))
    sc = s.view(np.float16).astype(np.float64)
    for c in (0, 1, 2, 3, 4, 31, 32, 35, 63):
        x = np.zeros(cols)
        x[c] = 1.0
        np.testing.assert_array_equal(oracle.matvec(pack_int2(q), s, x, codec="int2"), q[:, c] * sc[:, c // 32])
    x = rng.normal(size=cols)
    np.testing.assert_allclose(oracle.matvec(pack_int2(q), s, x, codec="int2"),
                               (q * np.repeat(sc, 32, axis=1)) @ x, rtol=1e-13)


def test_int2_layer_equals_int4_layer_on_shared_codes():
    """An int2 layer is the int4 layer with the same codes (in [-2, 1]) and
    scales: bit-identical routing and outputs."""
    import dataclasses
    base = synth.gen_layer(synth.TINY, seed=6)
    rng = np.random.default_rng(12)
    i4, i2 = {}, {}
    for name in ("gate", "up", "down"):
        qs = getattr(base, name + "_q")
        q = rng.integers(-2, 2, size=(qs.shape[0], qs.shape[1], qs.shape[2] * 2))
        i4[name + "_q"] = np.stack([pack_int4(m) for m in q])
        i2[name + "_q"] = np.stack([pack_int2(m) for m in q])
    w4 = dataclasses.replace(base, **i4)
    w2 = dataclasses.replace(base, cfg=dataclasses.replace(base.cfg, codec="int2"), **i2)
    x = synth.gen_tokens(synth.TINY, 5, seed=13)
    a, b = oracle.layer_forward(w4, x), oracle.layer_forward(w2, x)
    np.testing.assert_array_equal(a["ids"], b["ids"])
    np.testing.assert_array_equal(a["y"], b["y"])
    assert np.abs(a["y"]).max() > 0


def test_int2_generator_layout():
    import dataclasses
    cfg = dataclasses.replace(synth.TINY, codec="int2")
    w = synth.gen_layer(cfg, seed=0)
    assert w.gate_q.shape == (cfg.n_total_experts, cfg.inter, cfg.hidden // 4)
    assert w.down_q.shape == (cfg.n_total_experts, cfg.hidden, cfg.inter // 4)
    assert cfg.expert_bytes() == 3 * cfg.hidden * cfg.inter // 4 + 3 * cfg.hidden * cfg.inter // 16
    y = oracle.layer_forward(w, synth.gen_tokens(cfg, 2, seed=1))["y"]
    assert np.all(np.isfinite(y)) and 0.05 < np.abs(y).max() < 1e3
