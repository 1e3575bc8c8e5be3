"""Shared helpers of the tests: parity comparison of the GPU path with the oracle."""
import numpy as np

from oracle import oracle
from routed_expert_int4_amd import synth

GAP_EXCUSE = 1e-6      # selection margin below which differing ids are excused
Y_RTOL = 2e-3          # max |y_gpu - y_ref| <= Y_RTOL * max |y_ref| per token
W_ATOL_PER_RSF = 1e-6  # |w_gpu - w_ref| <= W_ATOL_PER_RSF * rsf


def check_routing(cfg, ids_gpu, w_gpu, ids_ref, w_ref, gap_ref, pgap_ref=None):
    """ids: equal (as sets and in order, -1 for a choice the top-p cut
    dropped) unless the oracle's selection gap, or its top-p decision margin
    (pgap_ref), is below GAP_EXCUSE; weights within W_ATOL_PER_RSF * rsf where
    ids agree.  Returns the indices of excused tokens."""
    excused = []
    for t in range(ids_ref.shape[0]):
        same = list(ids_gpu[t]) == list(ids_ref[t])
        if not same:
            margin = gap_ref[t] if pgap_ref is None else min(gap_ref[t], pgap_ref[t])
            assert margin < GAP_EXCUSE, (
                f"token {t}: ids {list(ids_gpu[t])} != oracle {list(ids_ref[t])} with margin {margin:.3g}")
            excused.append(t)
            continue
        err = np.abs(w_gpu[t].astype(np.float64) - w_ref[t]).max()
        assert err <= W_ATOL_PER_RSF * cfg.routed_scaling_factor, f"token {t}: weight error {err:.3g}"
    return excused


def check_outputs(y_gpu, y_ref, tokens=None):
    tokens = range(y_ref.shape[0]) if tokens is None else tokens
    worst = 0.0
    for t in tokens:
        ref = y_ref[t]
        err = np.abs(y_gpu[t].astype(np.float64) - ref).max()
        bound = Y_RTOL * np.abs(ref).max()
        assert np.all(np.isfinite(y_gpu[t])), f"token {t}: non-finite output"
        assert err <= bound, f"token {t}: max|dy| {err:.4g} > {bound:.4g}"
        worst = max(worst, err / max(np.abs(ref).max(), 1e-300))
    return worst


def check_layer(weights, x_bits, y_gpu, ids_gpu, w_gpu, rows=None):
    """Full parity of some tokens (rows) of a GPU forward with the oracle.
    Tokens whose ids were excused are re-checked with the oracle forced onto
    the GPU's ids, so the expert math is still verified."""
    rows = np.arange(x_bits.shape[0]) if rows is None else np.asarray(rows)
    ref = oracle.layer_forward(weights, x_bits[rows])
    excused = check_routing(weights.cfg, ids_gpu[rows], w_gpu[rows], ref["ids"], ref["w"], ref["gap"], ref["pgap"])
    good = [i for i in range(len(rows)) if i not in excused]
    worst = check_outputs(y_gpu[rows], ref["y"], good)
    if excused:
        forced = oracle.layer_forward(weights, x_bits[rows[excused]], forced_ids=ids_gpu[rows[excused]])
        worst = max(worst, check_outputs(y_gpu[rows[excused]], forced["y"]))
    return {"excused": len(excused), "worst_rel": worst}


# Shapes that exercise every lane mapping of the kernels: rows narrower and
# wider than a wave load, 1/2/4 experts per router lane, odd top_k.
MID_A = synth.LayerConfig(hidden=1024, inter=256, n_experts=64, n_groups=8, topk_group=4, top_k=6,
                          routed_scaling_factor=1.5)
MID_B = synth.LayerConfig(hidden=4096, inter=1024, n_experts=128, n_groups=4, topk_group=2, top_k=8)
MID_C = synth.LayerConfig(hidden=8192, inter=4096, n_experts=16, n_groups=4, topk_group=2, top_k=4)
MID_D = synth.LayerConfig(hidden=512, inter=128, n_experts=256, n_groups=8, topk_group=4, top_k=8)
# 96 experts (the batched router's two-block expert tiles) in 3 groups,
# hidden 2048 (8 steps of 16 columns per router split)
MID_E = synth.LayerConfig(hidden=2048, inter=512, n_experts=96, n_groups=3, topk_group=2, top_k=6)


def zipf_glm_weights():
    """GLM-shaped layer (weights seed 0) with the committed Zipf-calibrated
    correction bias (tests/golden/zipf_bias_glm.json, written by
    tests/golden/make_zipf_bias.py from the oracle)."""
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "zipf_bias_glm.json")
    with open(path) as f:
        rec = json.load(f)
    weights = synth.gen_layer(synth.GLM, seed=0)
    weights.bias = np.asarray(rec["bias"], dtype=np.float32)
    return weights, rec
