"""Seeded synthetic prompts shaped like the WAITS evaluation workloads.

Recipe (one prompt = one sequence of one layer):

* ``rng = numpy.random.default_rng(seed)``.
* Draw, in this order and in float32, ``Q[N, Hq, d]``, ``K[N, Hkv, d]`` and
  ``V[N, Hkv, d]`` from the standard normal distribution (token-major, the
  packed layout of a prefill batch).
* With heavy hitters on: draw ``u`` (d standard normals, normalised to unit
  length in float64, then rounded to float32), then the heavy positions
  ``{0} U rng.choice(N, round(0.01 N), replace=False)``.  Every heavy key
  gets ``+3 u``; every query gets ``+3 u`` (the direction is shared with the
  queries), which gives those keys a large accumulated attention mass.
* Round to bfloat16 with round-to-nearest-even when the dtype is bf16.

The stored bf16 (or fp32) values are *the* inputs: the oracle promotes the
same values to float64 and the GPU reads the same bits.

Nothing here computes anything the method computes.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

# The five regime-representative (a, b) actions the WAITS router chooses
# from (WAITS README, "Training the routing policy", the --actions list).
ACTIONS = ((0.0, 1), (0.01, 128), (1.0, 16), (10.0, 1), (10.0, 16))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the float32 values they encode (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


@dataclass
class Batch:
    """A packed batch of prompts, token-major: ``q[T, Hq, d]``, ``k/v[T, Hkv, d]``.

    ``q``, ``k``, ``v`` hold the exact input values as float32 (``None`` when
    the caller asked for bits only); ``*_bits`` hold the bf16 bit patterns
    (``None`` for fp32 inputs).  ``cu_seqlens[i]`` is the first token of
    prompt ``i``; ``cu_seqlens[-1] == T``.
    """

    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    cu_seqlens: np.ndarray
    q: Optional[np.ndarray] = None
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None
    seeds: Sequence[int] = field(default_factory=list)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens)

    @property
    def batch(self) -> int:
        return len(self.cu_seqlens) - 1


def _draw(seed: int, n: int, n_q_heads: int, n_kv_heads: int, d: int,
          heavy: bool):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, n_q_heads, d), dtype=np.float32)
    k = rng.standard_normal((n, n_kv_heads, d), dtype=np.float32)
    v = rng.standard_normal((n, n_kv_heads, d), dtype=np.float32)
    if heavy and n > 0:
        u64 = rng.standard_normal(d, dtype=np.float32).astype(np.float64)
        u = (u64 / np.linalg.norm(u64)).astype(np.float32)
        extra = rng.choice(n, int(round(0.01 * n)), replace=False)
        pos = np.union1d(np.array([0]), extra)
        k[pos] += np.float32(3.0) * u
        q += np.float32(3.0) * u
    return q, k, v


def make_prompt(seed: int, n: int, n_q_heads: int, n_kv_heads: int,
                head_dim: int, heavy: bool = True, dtype: str = "bf16",
                values: bool = True) -> Batch:
    """One prompt of ``n`` tokens (a batch of one)."""
    return make_batch([seed], [n], n_q_heads, n_kv_heads, head_dim,
                      heavy=heavy, dtype=dtype, values=values)


def make_batch(seeds: Sequence[int], lengths: Sequence[int], n_q_heads: int,
               n_kv_heads: int, head_dim: int, heavy: bool = True,
               dtype: str = "bf16", values: bool = True) -> Batch:
    """Independent prompts (or layers), one seed each, packed token-major."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    if len(seeds) != len(lengths):
        raise ValueError("one seed per prompt")
    lengths = [int(x) for x in lengths]
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    total = int(cu[-1])
    shapes = ((n_q_heads,), (n_kv_heads,), (n_kv_heads,))
    if dtype == "bf16":
        bits = [np.empty((total,) + s + (head_dim,), np.uint16) for s in shapes]
    vals = ([np.empty((total,) + s + (head_dim,), np.float32) for s in shapes]
            if (values or dtype == "f32") else None)
    for i, (seed, n) in enumerate(zip(seeds, lengths)):
        drawn = _draw(int(seed), n, n_q_heads, n_kv_heads, head_dim, heavy)
        lo, hi = int(cu[i]), int(cu[i + 1])
        for j, x in enumerate(drawn):
            if dtype == "bf16":
                b = bf16_bits(x)
                bits[j][lo:hi] = b
                if vals is not None:
                    vals[j][lo:hi] = bf16_bits_to_f32(b)
            else:
                vals[j][lo:hi] = x
    out = Batch(n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                head_dim=head_dim, dtype=dtype, cu_seqlens=cu,
                seeds=[int(s) for s in seeds])
    if vals is not None:
        out.q, out.k, out.v = vals
    if dtype == "bf16":
        out.q_bits, out.k_bits, out.v_bits = bits
    return out


@dataclass
class DecodeInputs:
    """One decoding step's inputs: ``q[B, Hq, d]`` and a dense cache
    ``k/v[B, Hkv, capacity, d]`` (the layout the compaction writes), as
    float32 values (exact bf16 values for bf16) plus bf16 bit patterns."""

    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None


def make_decode(seed: int, batch: int, n_q_heads: int, n_kv_heads: int, capacity: int,
                head_dim: int, dtype: str = "bf16", heavy: bool = True) -> DecodeInputs:
    """Seeded decode inputs.  Recipe: ``rng = default_rng(seed)``; draw
    float32 standard normals ``q[B, Hq, d]``, then ``k[B, Hkv, capacity, d]``,
    then ``v`` of the same shape; with ``heavy``, draw a unit direction ``u``
    (as for prompts) and the positions ``rng.choice(capacity,
    max(1, round(0.05 capacity)))`` of every (sequence, KV head), add
    ``+3 u`` to those keys and to every query; round to bf16 (nearest even)
    for ``dtype == "bf16"``."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((batch, n_q_heads, head_dim), dtype=np.float32)
    k = rng.standard_normal((batch, n_kv_heads, capacity, head_dim), dtype=np.float32)
    v = rng.standard_normal((batch, n_kv_heads, capacity, head_dim), dtype=np.float32)
    if heavy:
        u64 = rng.standard_normal(head_dim, dtype=np.float32).astype(np.float64)
        u = (u64 / np.linalg.norm(u64)).astype(np.float32)
        cnt = max(1, int(round(0.05 * capacity)))
        for i in range(batch):
            for h in range(n_kv_heads):
                k[i, h, rng.choice(capacity, cnt, replace=False)] += np.float32(3.0) * u
        q += np.float32(3.0) * u
    out = DecodeInputs(dtype=dtype, q=q, k=k, v=v)
    if dtype == "bf16":
        out.q_bits, out.k_bits, out.v_bits = (bf16_bits(x) for x in (q, k, v))
        out.q, out.k, out.v = (bf16_bits_to_f32(b) for b in (out.q_bits, out.k_bits, out.v_bits))
    return out
