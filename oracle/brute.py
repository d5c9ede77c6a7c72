"""Contiguous, unpaged brute force — TEST INFRASTRUCTURE ONLY.

Before paging, each sequence's cache was one contiguous region reserved for
its longest possible length [F55 §先占好最长的位置].  This module keeps that
layout: a sequence's keys and values are plain Python lists in token order,
and attention is the textbook scaled dot-product softmax, written with
Python floats (IEEE double) and loops.  It reads no pool and no block table,
so it checks the paged oracle independently on tiny inputs.
"""
import math


def softmax(xs):
    m = max(xs)
    e = [math.exp(x - m) for x in xs]
    z = sum(e)
    return [v / z for v in e]


def attend(q, keys, values, scale):
    """One query vector over lists of key and value vectors."""
    if not keys:
        return [0.0] * len(q)
    scores = [scale * sum(a * b for a, b in zip(q, k)) for k in keys]
    w = softmax(scores)
    d = len(values[0])
    return [sum(w[t] * values[t][i] for t in range(len(values))) for i in range(d)]


def decode_contiguous(q, keys, values, scale, group):
    """q: [B][Hq][d] nested lists; keys/values: [B][T_b][Hkv][d] nested lists.

    Query head h reads KV head h // group.  Returns [B][Hq][d].
    """
    out = []
    for b in range(len(q)):
        rows = []
        for h in range(len(q[b])):
            g = h // group
            ks = [tok[g] for tok in keys[b]]
            vs = [tok[g] for tok in values[b]]
            rows.append(attend(q[b][h], ks, vs, scale))
        out.append(rows)
    return out
