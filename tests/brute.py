"""Brute-force attention in pure Python loops, written separately from the oracle, for tiny inputs.

It pins the fp64 oracle: no shared code, a different formulation (whole score lists instead of online
softmax; skip-softmax as "decide the kept tiles first, then one softmax over the kept keys").
"""
import math


def scores(q, keys, scale):
    return [scale * sum(a * b for a, b in zip(q, k)) for k in keys]


def softmax_attend(s, values):
    """o = sum_j softmax(s)_j v_j, lse; empty -> zeros, -inf."""
    D = len(values[0]) if values else 0
    if not s:
        return None, -math.inf, []
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = sum(e)
    p = [x / z for x in e]
    o = [sum(p[j] * values[j][d] for j in range(len(s))) for d in range(D)]
    return o, m + math.log(z), p


def skip_attend(s, values, tile, thr):
    """Skip-softmax by first deciding which tiles survive, then one softmax over the survivors.

    Walks the tiles in order keeping the running max of the tiles kept so far; a tile is dropped when
    that max exists and exp(tile max - running max) < thr.  Returns (o, lse, decisions)."""
    n = len(s)
    kept, decisions, run = [], [], None
    for t0 in range(0, n, tile):
        idx = list(range(t0, min(t0 + tile, n)))
        tmax = max(s[j] for j in idx)
        drop = thr > 0 and run is not None and math.exp(tmax - run) < thr
        decisions.append(1 if drop else 0)
        if not drop:
            kept += idx
            run = tmax if run is None else max(run, tmax)
    if not kept:
        return None, -math.inf, decisions
    o, lse, _ = softmax_attend([s[j] for j in kept], [values[j] for j in kept])
    return o, lse, decisions
