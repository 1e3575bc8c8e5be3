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
replay_prefetch adds a speculative prefetch of each token's predicted
experts before its lookup (the expert readahead of the same summary).
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


def replay_prefetch(trace, predicted, slots: int, pinned=(), max_prefetch=None):
    """Replay with speculative next-layer prefetch before every lookup.

    Reading of the colibri summary's expert readahead ("Principales
    fonctionnalites implementees": the next expert block is fetched while the
    current one is being multiplied), with the prediction of a layer's experts
    taken from the next layer's router applied to the current layer's input:
    predicted[t] is the expert list predicted for token t of this layer (None:
    no prediction for that token).  Before token t is looked up, its predicted
    experts are visited in order; one that is resident (pinned or in the LRU)
    is left as it is (no recency change), one that is not is brought in like a
    miss (a free slot, else the least recently used unpinned expert that is not
    itself predicted for t), until max_prefetch experts have been brought in
    (None: no limit).  Ids -1 are skipped.  Then token t is looked up as in
    replay().

    Returns a dict of counts: hits, misses, evictions (by lookups and
    prefetches alike), prefetches (experts brought in by prefetch),
    prefetch_hits (uses that found an expert a prefetch brought in and that
    nothing had used since), predicted_uses (uses of tokens with a prediction)
    and predicted_hits (those uses whose expert was predicted).
    """
    pinned = set(int(e) for e in pinned)
    capacity = slots - len(pinned)
    resident = OrderedDict()
    fresh = set()  # brought in by a prefetch, not used since
    n = dict(hits=0, misses=0, evictions=0, prefetches=0, prefetch_hits=0, predicted_uses=0, predicted_hits=0)

    def bring_in(e, keep):
        if len(resident) >= capacity:
            victim = next(v for v in resident if v not in keep)
            del resident[victim]
            fresh.discard(victim)
            n["evictions"] += 1
        resident[e] = None

    for t, token in enumerate(trace):
        token = [int(e) for e in token if int(e) >= 0]
        guess = None if predicted[t] is None else [int(e) for e in predicted[t] if int(e) >= 0]
        if guess is not None:
            keep = set(guess)
            copies = 0
            for e in guess:
                if e in pinned or e in resident:
                    continue
                if max_prefetch is not None and copies >= max_prefetch:
                    break
                bring_in(e, keep)
                fresh.add(e)
                n["prefetches"] += 1
                copies += 1
            n["predicted_uses"] += len(token)
            n["predicted_hits"] += sum(1 for e in token if e in keep)
        need = set(token)
        for e in token:
            if e in pinned or e in resident:
                n["hits"] += 1
                if e in resident:
                    resident.move_to_end(e)
                if e in fresh:
                    n["prefetch_hits"] += 1
                    fresh.discard(e)
                continue
            n["misses"] += 1
            bring_in(e, need)
    return n
