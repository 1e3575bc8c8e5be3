"""Plain LRU replay of one layer's expert cache (TEST INFRASTRUCTURE ONLY).

The cache is the per-layer LRU expert cache of the colibri summary
(fr.news.hada.io topic 31297, "Execution d'un MoE basee sur le streaming
disque") over a fixed number of slots.  Reading used here: a token's experts
are looked up in routing order; a hit refreshes the expert's recency; a miss
takes a free slot, else evicts the least recently used expert that the same
token does not need.  Returns the hit, miss and eviction counts from a cold
start.
"""
from collections import OrderedDict


def replay(trace, slots: int):
    resident = OrderedDict()  # expert -> None, least recently used first
    hits = misses = evictions = 0
    for token in trace:
        need = set(int(e) for e in token)
        for e in token:
            e = int(e)
            if e in resident:
                hits += 1
                resident.move_to_end(e)
                continue
            misses += 1
            if len(resident) >= slots:
                victim = next(v for v in resident if v not in need)
                del resident[victim]
                evictions += 1
            resident[e] = None
    return hits, misses, evictions
