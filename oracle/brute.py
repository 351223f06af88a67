"""Pure-Python decode attention for tiny inputs (test infrastructure).

Softmax attention of one query row over an explicit list of key / value rows,
written with ``math.exp`` loops and no library routine, so that it can serve
as an independent check of the C oracle on small cases.  The definition is
the plain one the pages assume (attention over each head's retained entries,
Tangram abstract; over selected critical entries, KVDrive Fig 1).
"""
import math


def attend(q, keys, values, scale):
    """q: list of floats; keys/values: lists of rows.  Returns (out, lse)."""
    if not keys:
        return [0.0] * len(q), float("-inf")
    z = [scale * sum(a * b for a, b in zip(q, k)) for k in keys]
    m = max(z)
    w = [math.exp(x - m) for x in z]
    l = sum(w)
    out = [sum(w[t] * values[t][d] for t in range(len(values))) / l
           for d in range(len(q))]
    return out, m + math.log(l)
