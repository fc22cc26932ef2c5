"""Plain float64 oracle of decode attention over a compacted KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Source: the WAITS README (page "Dirac-Notation/A2SF").  Its introduction
states the purpose of the method, a smaller inference cache that keeps only
selected key-value pairs; its "Quickstart" compresses the cache with
``init_cache`` and then generates, so every decoding step attends over the
kept rows (and the rows generation appends after them).

Readings taken where the page is silent:

* the attention of a decoding step is the model's ordinary scaled
  dot-product attention: for query head ``g`` of sequence ``i``,
  ``out = sum_j softmax_j(scale * <q[i, g], K[i, h, j]>) * V[i, h, j]`` over
  the cache rows ``j < len[i]`` of KV head ``h = g // G`` (contiguous GQA
  groups), with no mask inside the cache (every kept row precedes the new
  token) and no position change (the cached keys already carry theirs);
* the cache of sequence ``i`` is ``[n_kv_heads, capacity, head_dim]``; rows
  ``j >= len[i]`` (compaction padding, unused capacity) are not attended;
* ``lse = ln sum_j exp(scale * <q, K_j>)``; an empty cache (``len = 0``)
  gives ``out = 0`` and ``lse = -inf``;
* the scale is taken as the float32 value a caller passes, promoted to
  float64.
"""
from __future__ import annotations

import numpy as np


def decode_head(q: np.ndarray, kc: np.ndarray, vc: np.ndarray, scale: float):
    """One query vector ``q[d]`` over cache rows ``kc[n, d]``, ``vc[n, d]``:
    returns ``(out[d], lse)`` in float64.  ``n = 0`` gives zeros and -inf."""
    d = q.shape[0]
    if kc.shape[0] == 0:
        return np.zeros(d), -np.inf
    s = float(np.float32(scale)) * (np.asarray(kc, np.float64) @ np.asarray(q, np.float64))
    m = s.max()
    e = np.exp(s - m)
    tot = e.sum()
    return (e / tot) @ np.asarray(vc, np.float64), m + np.log(tot)


def waits_decode(q, k_cache, v_cache, lens, scale):
    """Decode attention for a batch.

    ``q[B, Hq, d]``, ``k_cache`` / ``v_cache`` ``[B, Hkv, capacity, d]``,
    ``lens[B]`` (rows attended per sequence, ``0 <= lens <= capacity``).
    Returns ``out[B, Hq, d]`` and ``lse[B, Hq]`` in float64.
    """
    bsz, hq, d = q.shape
    hkv = k_cache.shape[1]
    if hq % hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != bsz or k_cache.shape[3] != d:
        raise ValueError("cache shapes do not match q")
    group = hq // hkv
    out = np.zeros((bsz, hq, d))
    lse = np.zeros((bsz, hq))
    for i in range(bsz):
        n = int(lens[i])
        if not 0 <= n <= k_cache.shape[2]:
            raise ValueError("lens must lie in [0, capacity]")
        for g in range(hq):
            h = g // group
            out[i, g], lse[i, g] = decode_head(q[i, g], k_cache[i, h, :n], v_cache[i, h, :n],
                                               scale)
    return out, lse
