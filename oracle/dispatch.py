"""Batch-union dispatch of a routing (TEST INFRASTRUCTURE ONLY).

The colibrì summary (fr.news.hada.io topic 31297, "Principales
fonctionnalités implémentées") describes batch-union MoE for prefill and
batched verification: the distinct experts of a batch are read once and
applied to every position routed to them.  Reading used here: the T*K
(token, slot) entries of a routing ids[T][K] are grouped by expert in
ascending expert order and, inside an expert, in entry order (token, then
slot).  Written as plain loops.

dispatch(ids, n_experts) -> dict(counts [E], offsets [E+1], perm [T*K],
distinct [D]) with perm[p] = token*K + slot of the p-th entry.  A choice
dropped by the adaptive top-p cut (id -1) takes no place: the kept entries
fill perm[0 .. offsets[E]) and the rest of perm is -1.
"""
import numpy as np


def dispatch(ids, n_experts: int):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    counts = [0] * n_experts
    for e in flat:
        if e >= 0:
            counts[e] += 1
    offsets = [0] * (n_experts + 1)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = list(offsets[:n_experts])
    perm = [-1] * len(flat)
    for entry, e in enumerate(flat):  # entries visited in order: stable
        if e < 0:
            continue
        perm[fill[e]] = entry
        fill[e] += 1
    distinct = [e for e in range(n_experts) if counts[e] > 0]
    return {
        "counts": np.array(counts, np.int32),
        "offsets": np.array(offsets, np.int32),
        "perm": np.array(perm, np.int32),
        "distinct": np.array(distinct, np.int32),
    }
