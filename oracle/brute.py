"""Scalar pure-Python brute force of the WAITS score, for tiny prompts.

TEST INFRASTRUCTURE ONLY.  Written independently of ``waits_oracle`` (plain
loops, ``math.exp`` and ``math.fsum``; no numpy arithmetic) so that the two
pin each other on N <= 64.  Definition: WAITS README, introduction (sigmoid
forgetting curve times causal softmax attention, summed over query rows),
with the readings listed in ``waits_oracle``.
"""
from __future__ import annotations

import math


def weight(q: int, n: int, a: float, b: int) -> float:
    """Forgetting-curve weight of query row q (0-based) in a prompt of n."""
    x = q - (n - b - 0.5)
    if math.isinf(a):
        return 1.0 if x > 0 else 0.0
    try:
        return 1.0 / (1.0 + math.exp(-a * x))
    except OverflowError:      # exp overflows float64: the weight is 0
        return 0.0


def scores(q, k, n_q_heads: int, n_kv_heads: int, a: float, b: int,
           scale: float):
    """``q[n][Hq][d]``, ``k[n][Hkv][d]`` nested lists of floats (one prompt).

    Returns ``s[h][key]`` as nested lists.
    """
    n = len(q)
    group = n_q_heads // n_kv_heads
    terms = [[[] for _ in range(n)] for _ in range(n_kv_heads)]
    for g in range(n_q_heads):
        h = g // group
        for row in range(n):
            wq = weight(row, n, a, b)
            if wq == 0.0:
                continue
            logits = []
            for key in range(row + 1):
                dot = math.fsum(q[row][g][i] * k[key][h][i]
                                for i in range(len(q[row][g])))
                logits.append(scale * dot)
            top = max(logits)
            ex = [math.exp(x - top) for x in logits]
            z = math.fsum(ex)
            for key in range(row + 1):
                terms[h][key].append(wq * ex[key] / z)
    return [[math.fsum(t) for t in terms[h]] for h in range(n_kv_heads)]


def topk(s, budget: int):
    """Positions of the ``budget`` largest scores, ties to the lower
    position, ascending, padded with -1."""
    ranked = sorted(range(len(s)), key=lambda i: (-s[i], i))
    kept = sorted(ranked[:budget])
    return kept + [-1] * (budget - len(kept))


def decode(qv, kc, vc, scale: float):
    """Decode attention of one query vector ``qv[d]`` over cache rows
    ``kc[n][d]``, ``vc[n][d]`` (nested lists of floats), written as scalar
    loops: softmax over the rows of ``scale * <q, k_j>``, then the weighted
    sum of the ``v_j``.  Returns ``(out[d], lse)``; an empty cache gives
    zeros and -inf.  (README "Quickstart": generation after init_cache
    attends over the kept rows.)"""
    d = len(qv)
    if not kc:
        return [0.0] * d, -math.inf
    logits = [scale * math.fsum(qv[i] * row[i] for i in range(d)) for row in kc]
    top = max(logits)
    ex = [math.exp(x - top) for x in logits]
    z = math.fsum(ex)
    out = [math.fsum(ex[j] * vc[j][i] for j in range(len(kc))) / z for i in range(d)]
    return out, top + math.log(z)


def attention(q, k, v, group: int, scale: float):
    """Causal attention of one prompt in scalar loops: ``q[n][Hq][d]``,
    ``k / v[n][Hkv][d]`` nested lists.  Returns ``out[n][Hq][d]`` and
    ``lse[Hq][n]``.  (Row ``r`` is decode attention over the keys ``<= r``.)"""
    n, hq = len(q), len(q[0])
    out = [[None] * hq for _ in range(n)]
    lse = [[0.0] * n for _ in range(hq)]
    for g in range(hq):
        h = g // group
        for r in range(n):
            o, z = decode(q[r][g], [k[j][h] for j in range(r + 1)],
                          [v[j][h] for j in range(r + 1)], scale)
            out[r][g] = o
            lse[g][r] = z
    return out, lse
