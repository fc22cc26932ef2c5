"""Plain float64 oracle of WAITS score -> select -> compact.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Source: the WAITS README (page "Dirac-Notation/A2SF"), introduction.  WAITS
keeps, per KV head, the prompt keys with the largest accumulated attention,
where the attention that query row ``q`` pays to key ``k`` is weighted by a
sigmoid forgetting curve ``w[q] = 1 / (1 + exp(-a (q - (N - b - 0.5))))``.
The README's "Quickstart" names the knobs (``sigmoid_a`` = a,
``recent_budget`` = b, ``select_budget`` = number of keys kept) and its
"Repository layout" names the selector (top-k).

Readings taken where the page is silent:

* query and key positions are 0-based (with b = 1 and a -> inf only the last
  row keeps weight, which is the TOVA limit the introduction names);
* ``A[q, .]`` is the causal softmax of ``scale * <Q[g, q], K[h, .]>`` over
  keys ``k <= q`` (diagonal included);
* query head ``g`` reads KV head ``g // G`` (contiguous GQA groups) and a KV
  head's score is the *sum* over its G query heads;
* every key competes for the budget (b only shapes the curve); ties go to
  the lower position; the kept positions are returned in ascending order and
  padded with -1 when the prompt is shorter than the budget;
* ``a`` and the softmax scale are taken as the float32 values a caller
  passes, promoted to float64; a = +inf uses IEEE arithmetic literally
  (``q - c`` is never 0 because ``c`` is a half-integer), giving a 0/1 step.
"""
from __future__ import annotations

import numpy as np


def sigmoid_weights(n: int, a: float, b: int) -> np.ndarray:
    """``w[q]`` for ``q = 0..n-1`` in float64 (the forgetting curve)."""
    a64 = float(np.float32(a))
    q = np.arange(n, dtype=np.float64)
    c = float(n) - float(b) - 0.5
    with np.errstate(over="ignore", invalid="raise"):
        return 1.0 / (1.0 + np.exp(-a64 * (q - c)))


def live_rows(w: np.ndarray) -> np.ndarray:
    """Rows whose weight is nonzero.  Rows with w == 0 add exact zeros, so
    leaving them out changes no sum."""
    return np.nonzero(w != 0.0)[0]


def _row_softmax(qg: np.ndarray, kh: np.ndarray, rows: np.ndarray,
                 scale: float):
    """Causal softmax rows ``A[rows, :kmax]`` (float64) and their keys' span."""
    kmax = int(rows[-1]) + 1
    logits = scale * (qg[rows] @ kh[:kmax].T)
    future = np.arange(kmax)[None, :] > rows[:, None]
    logits[future] = -np.inf
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=1, keepdims=True), kmax


def head_scores(qg: np.ndarray, kh: np.ndarray, w: np.ndarray, scale: float,
                row_block: int = 256, weight_floor: float = 0.0,
                row_min: int = 0) -> np.ndarray:
    """Accumulated weighted attention of one KV head.

    ``qg[G, N, d]`` are the query heads of the group, ``kh[N, d]`` the keys.
    Returns ``s[k] = sum_g sum_q w[q] A_g[q, k]`` in float64.

    The defaults compute the definition exactly.  For sampled checks at full
    size two restrictions are available, each with a stated effect:
    ``weight_floor`` drops rows with ``w[q] <= weight_floor``; since
    ``A[q, k] <= 1`` the dropped part of any ``s[k]`` is at most
    ``G * N * weight_floor``.  ``row_min`` drops rows ``q < row_min``; rows
    only reach keys ``k <= q``, so ``s[k]`` stays exact for ``k >= row_min``.
    """
    n = kh.shape[0]
    s = np.zeros(n, dtype=np.float64)
    rows_all = live_rows(w)
    rows_all = rows_all[(w[rows_all] > weight_floor) & (rows_all >= row_min)]
    kh = np.asarray(kh, dtype=np.float64)
    for g in range(qg.shape[0]):
        qf = np.asarray(qg[g], dtype=np.float64)
        for r0 in range(0, len(rows_all), row_block):
            rows = rows_all[r0:r0 + row_block]
            attn, kmax = _row_softmax(qf, kh, rows, scale)
            s[:kmax] += w[rows] @ attn
    return s


def _check_packed(q, k, cu_seqlens, n_q_heads, n_kv_heads):
    if n_q_heads % n_kv_heads:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if q.shape[1] != n_q_heads or k.shape[1] != n_kv_heads:
        raise ValueError("head counts do not match the arrays")
    if int(cu_seqlens[-1]) != q.shape[0] or k.shape[0] != q.shape[0]:
        raise ValueError("cu_seqlens does not cover the packed tokens")


def waits_scores(q, k, cu_seqlens, n_q_heads, n_kv_heads, a, b, scale,
                 row_block: int = 256, weight_floor: float = 0.0,
                 row_min=None) -> np.ndarray:
    """Scores ``[Hkv, T]`` for a packed batch.

    ``q[T, Hq, d]``, ``k[T, Hkv, d]`` token-major; ``a[i]``, ``b[i]`` per
    prompt; positions restart at 0 in every prompt.  ``weight_floor`` and
    ``row_min`` (one value per prompt) restrict rows as in ``head_scores``.
    """
    _check_packed(q, k, cu_seqlens, n_q_heads, n_kv_heads)
    group = n_q_heads // n_kv_heads
    scale64 = float(np.float32(scale))
    out = np.zeros((n_kv_heads, q.shape[0]), dtype=np.float64)
    for p in range(len(cu_seqlens) - 1):
        lo, hi = int(cu_seqlens[p]), int(cu_seqlens[p + 1])
        if hi == lo:
            continue
        w = sigmoid_weights(hi - lo, a[p], b[p])
        for h in range(n_kv_heads):
            qg = np.stack([q[lo:hi, h * group + j] for j in range(group)])
            out[h, lo:hi] = head_scores(
                qg, k[lo:hi, h], w, scale64, row_block, weight_floor,
                0 if row_min is None else int(row_min[p]))
    return out


def waits_lse(q, k, cu_seqlens, n_q_heads, n_kv_heads, scale,
              rows_per_prompt=None) -> np.ndarray:
    """Natural-log row normaliser ``ln sum_{k<=q} exp(scale <Q[g,q], K[h,k]>)``.

    Returns ``[Hq, T]`` float64; rows not asked for (``rows_per_prompt[p]``
    lists the 0-based rows of prompt p; ``None`` = all) are NaN.
    """
    _check_packed(q, k, cu_seqlens, n_q_heads, n_kv_heads)
    group = n_q_heads // n_kv_heads
    scale64 = float(np.float32(scale))
    out = np.full((n_q_heads, q.shape[0]), np.nan)
    for p in range(len(cu_seqlens) - 1):
        lo, hi = int(cu_seqlens[p]), int(cu_seqlens[p + 1])
        if hi == lo:
            continue
        rows = (np.arange(hi - lo) if rows_per_prompt is None
                else np.asarray(rows_per_prompt[p], dtype=np.int64))
        for g in range(n_q_heads):
            qf = np.asarray(q[lo:hi, g], dtype=np.float64)
            kf = np.asarray(k[lo:hi, g // group], dtype=np.float64)
            for r0 in range(0, len(rows), 256):
                rr = rows[r0:r0 + 256]
                kmax = int(rr.max()) + 1
                logits = scale64 * (qf[rr] @ kf[:kmax].T)
                logits[np.arange(kmax)[None, :] > rr[:, None]] = -np.inf
                m = logits.max(axis=1)
                out[g, lo + rr] = m + np.log(np.exp(logits - m[:, None]).sum(axis=1))
    return out


def select_topk(s: np.ndarray, budget: int) -> np.ndarray:
    """Top-``budget`` positions by (score descending, position ascending),
    returned ascending and padded with -1 to length ``budget``."""
    n = len(s)
    keep = min(int(budget), n)
    order = np.lexsort((np.arange(n), -np.asarray(s, dtype=np.float64)))
    out = np.full(int(budget), -1, dtype=np.int32)
    out[:keep] = np.sort(order[:keep])
    return out


def waits_select(scores: np.ndarray, cu_seqlens, n_kv_heads: int,
                 budget: int) -> np.ndarray:
    """``idx[B, Hkv, budget]`` (int32, prompt-relative positions)."""
    nb = len(cu_seqlens) - 1
    out = np.full((nb, n_kv_heads, int(budget)), -1, dtype=np.int32)
    for p in range(nb):
        lo, hi = int(cu_seqlens[p]), int(cu_seqlens[p + 1])
        for h in range(n_kv_heads):
            out[p, h] = select_topk(scores[h, lo:hi], budget)
    return out


def waits_compact(k: np.ndarray, v: np.ndarray, cu_seqlens,
                  idx: np.ndarray):
    """Gather the kept rows: ``kc[p, h, j] = k[cu[p] + idx[p, h, j], h]``.

    Works on any element type (bit patterns included); slots with idx == -1
    are zero.
    """
    nb, hkv, budget = idx.shape
    d = k.shape[-1]
    kc = np.zeros((nb, hkv, budget, d), dtype=k.dtype)
    vc = np.zeros((nb, hkv, budget, d), dtype=v.dtype)
    for p in range(nb):
        lo = int(cu_seqlens[p])
        for h in range(hkv):
            sel = idx[p, h]
            ok = sel >= 0
            kc[p, h, ok] = k[lo + sel[ok], h]
            vc[p, h, ok] = v[lo + sel[ok], h]
    return kc, vc
