"""Plain float64 oracle of the prefill attention forward with its per-row
log-sum-exp, the kernel WAITS pass 1 can ride on.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Source: the WAITS README (page "Dirac-Notation/A2SF").  Its "Quickstart"
describes the method as a plugin inside the model's attention call, and its
introduction defines the score through the causal softmax attention of every
prompt row; the softmax normaliser of each row is what WAITS pass 1 needs.
The attention itself is the model's ordinary causal scaled dot-product
attention.

Readings taken where the page is silent:

* ``out[t0 + q, g] = sum_{k <= q} softmax_k(scale <Q[q, g], K[k, h]>) V[k, h]``
  for every query row ``q`` of every prompt (0-based positions restarting per
  prompt, keys ``k <= q``, diagonal included), ``h = g // G`` (contiguous GQA
  groups);
* ``lse[g, t0 + q] = ln sum_{k <= q} exp(scale <Q[q, g], K[k, h]>)``, the same
  quantity as WAITS pass 1's row normaliser;
* the scale is taken as the float32 value a caller passes, promoted to
  float64.
"""
from __future__ import annotations

import numpy as np


def prefill_attention(q, k, v, cu_seqlens, n_q_heads: int, n_kv_heads: int, scale: float,
                      row_block: int = 256):
    """Causal attention of a packed batch: returns ``out[T, Hq, d]`` and
    ``lse[Hq, T]`` in float64.  ``q[T, Hq, d]``, ``k / v[T, Hkv, d]``."""
    if n_q_heads % n_kv_heads:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    tot, _, d = q.shape
    if k.shape != v.shape or k.shape[0] != tot or k.shape[1] != n_kv_heads:
        raise ValueError("K/V do not match Q")
    group = n_q_heads // n_kv_heads
    sc = float(np.float32(scale))
    out = np.zeros((tot, n_q_heads, d))
    lse = np.zeros((n_q_heads, tot))
    for p in range(len(cu_seqlens) - 1):
        lo, hi = int(cu_seqlens[p]), int(cu_seqlens[p + 1])
        n = hi - lo
        for g in range(n_q_heads):
            h = g // group
            qg = np.asarray(q[lo:hi, g], np.float64)
            kh = np.asarray(k[lo:hi, h], np.float64)
            vh = np.asarray(v[lo:hi, h], np.float64)
            for r0 in range(0, n, row_block):
                rows = np.arange(r0, min(n, r0 + row_block))
                span = int(rows[-1]) + 1                  # keys any of these rows sees
                s = sc * (qg[rows] @ kh[:span].T)
                s[np.arange(span)[None, :] > rows[:, None]] = -np.inf
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                z = e.sum(axis=1, keepdims=True)
                out[lo + rows, g] = (e / z) @ vh[:span]
                lse[g, lo + rows] = (m + np.log(z))[:, 0]
    return out, lse
