"""Writes the Zipf-skewed correction bias of the GLM-shaped layer (weights seed 0).

Batched workloads route with a correction bias chosen so that expert selection
frequencies follow a Zipf(s = 1.1) law over expert ranks.  A literal Zipf law
cannot be met with top-8 of 256 experts (rank 1 would need a frequency above
1 per token), so the target is capped: p_e = min(1, c * r_e^-1.1) with c set so
that the frequencies sum to top_k; r_e is expert e's rank in a seeded random
permutation (seed 2).  The bias is calibrated by the fixed-point iteration
b_e += eta * (p_e - phat_e) on 4096 calibration tokens (N(0,1) bf16, seed 3),
where phat_e is expert e's realised selection frequency.  Router scores are
computed once by the oracle; only the selection is repeated per iteration, by
the oracle's selection routine.  Only oracle/ and the input generators are
used.

Run: python tests/golden/make_zipf_bias.py           (zipf_bias_glm.json: the
     GLM-shaped layer of weights seed 0, permutation seed 2, tokens seed 3)
     python tests/golden/make_zipf_bias.py --stack   (zipf_bias_stack.json:
     12 stacked layers, layer l of weights seed 100 + l, permutation seed
     200 + l, calibration tokens seed 250 + l)
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import oracle  # noqa: E402
from routed_expert_int4_amd import synth  # noqa: E402

ZIPF_S = 1.1
PERM_SEED = 2
CAL_SEED = 3
N_CAL = 4096
ITERS = 300
ETA = 0.5


def capped_zipf_targets(n_experts, top_k, s, perm_seed):
    ranks = np.empty(n_experts, np.int64)
    ranks[np.random.Generator(np.random.PCG64(perm_seed)).permutation(n_experts)] = np.arange(1, n_experts + 1)
    base = ranks.astype(np.float64) ** -s
    lo, hi = 0.0, float(top_k) / base.min()
    for _ in range(200):  # bisection on c: sum(min(1, c * base)) = top_k
        c = 0.5 * (lo + hi)
        if np.minimum(1.0, c * base).sum() < top_k:
            lo = c
        else:
            hi = c
    return ranks, np.minimum(1.0, c * base), c


def calibrate(weights_seed, perm_seed, cal_seed, verbose=True):
    cfg = synth.GLM
    router_w, _ = synth.gen_router(cfg, weights_seed)
    ranks, target, c = capped_zipf_targets(cfg.n_experts, cfg.top_k, ZIPF_S, perm_seed)
    x = synth.gen_tokens(cfg, N_CAL, seed=cal_seed)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    zero_bias = np.zeros(cfg.n_experts, np.float32)
    s_all = np.empty((N_CAL, cfg.n_experts), np.float64)
    for t in range(N_CAL):
        _, s_all[t], _ = oracle.router_scores(router_w, zero_bias, xf[t])
    b = np.zeros(cfg.n_experts, np.float64)
    best = None
    for it in range(ITERS):
        b32 = b.astype(np.float32).astype(np.float64)
        freq = np.zeros(cfg.n_experts, np.float64)
        for t in range(N_CAL):
            ids, _, _ = oracle.select(cfg.n_groups, cfg.topk_group, cfg.top_k, cfg.routed_scaling_factor,
                                      s_all[t], s_all[t] + b32)
            freq[ids] += 1.0
        freq /= N_CAL
        err = float(np.abs(freq - target).max())
        if best is None or err < best[0]:
            best = (err, b32.copy(), freq.copy())
        if verbose and it % 20 == 0:
            print(f"seed {weights_seed} iter {it}: max |freq - target| = {err:.4f}", flush=True)
        b = b + ETA * (target - freq)
    err, b_best, freq = best
    order = np.argsort(ranks)
    live = freq[order] > 0
    r = np.arange(1, cfg.n_experts + 1)[live]
    slope = float(np.polyfit(np.log(r[1:]), np.log(freq[order][live][1:]), 1)[0])
    return {
        "weights_seed": weights_seed, "perm_seed": perm_seed, "calibration_seed": cal_seed,
        "zipf_s": ZIPF_S, "calibration_tokens": N_CAL, "iterations": ITERS, "eta": ETA, "c": c,
        "max_abs_freq_error": err, "realised_loglog_slope_ranks_2_up": slope,
        "ranks": ranks.tolist(), "bias": [float(v) for v in b_best.astype(np.float32)],
    }


def _stack_layer(l):
    return calibrate(100 + l, 200 + l, 250 + l, verbose=False)


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    if "--stack" in sys.argv:
        import multiprocessing
        with multiprocessing.Pool(4) as pool:
            layers = pool.map(_stack_layer, range(12))
        out = {"what": "correction biases of 12 stacked GLM-shaped layers for capped Zipf(1.1) routing",
               "layers": layers}
        path = os.path.join(here, "zipf_bias_stack.json")
        with open(path, "w") as f:
            json.dump(out, f)
        print(f"wrote {path}: max errors {[round(l['max_abs_freq_error'], 4) for l in layers]}")
        return
    rec = calibrate(0, PERM_SEED, CAL_SEED)
    out = {"what": "correction bias of the GLM-shaped layer (weights seed 0) for capped Zipf(1.1) routing"}
    out.update(rec)
    path = os.path.join(here, "zipf_bias_glm.json")
    with open(path, "w") as f:
        json.dump(out, f)
    print(f"wrote {path}: max error {rec['max_abs_freq_error']:.4f}, slope "
          f"{rec['realised_loglog_slope_ranks_2_up']:.3f}, c {rec['c']:.4f}")


if __name__ == "__main__":
    main()
