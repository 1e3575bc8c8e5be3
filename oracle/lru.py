"""Plain replay of one layer's expert cache (TEST INFRASTRUCTURE ONLY).

The cache is the per-layer LRU expert cache of the colibri summary
(fr.news.hada.io topic 31297, "Execution d'un MoE basee sur le streaming
disque") over a fixed number of slots, with the pinned hot store of its
learning cache ("Learning cache et attentes selon le materiel": routed
experts are counted as they are used, and the hottest ones are pinned).
Reading used here: a token's experts are looked up in routing order; a hit
refreshes the expert's recency; a miss takes a free slot, else evicts the
least recently used expert that the same token does not need.  Pinned
experts are resident from the start, are never evicted, and leave
slots - len(pinned) slots to the LRU.  A choice dropped by the adaptive
top-p cut (id -1) is not looked up.  Returns the hit, miss and eviction
counts from a cold start (pinned experts loaded beforehand).
"""
from collections import OrderedDict


def replay(trace, slots: int, pinned=()):
    pinned = set(int(e) for e in pinned)
    capacity = slots - len(pinned)
    resident = OrderedDict()  # unpinned expert -> None, least recently used first
    hits = misses = evictions = 0
    for token in trace:
        token = [int(e) for e in token if int(e) >= 0]
        need = set(token)
        for e in token:
            if e in pinned:
                hits += 1
                continue
            if e in resident:
                hits += 1
                resident.move_to_end(e)
                continue
            misses += 1
            if len(resident) >= capacity:
                victim = next(v for v in resident if v not in need)
                del resident[victim]
                evictions += 1
            resident[e] = None
    return hits, misses, evictions


def usage(trace, n_experts: int):
    """Routed uses of every expert in a trace (the learning cache's counts)."""
    counts = [0] * n_experts
    for token in trace:
        for e in token:
            if int(e) >= 0:
                counts[int(e)] += 1
    return counts


def hottest(counts, n: int):
    """The n most used experts, most used first, ties to the lower index."""
    order = sorted(range(len(counts)), key=lambda e: (-counts[e], e))
    return order[:n]
