"""Pins for the CPU oracle (no GPU).

Each test fixes the oracle against something other than itself: closed forms
(harmonic numbers for uniform attention), the limits the WAITS README's
introduction names (H2O at a=0, TOVA at a->inf with b=1, SnapKV at a->inf
with b=window) checked through ``scipy.special.softmax``, the README's snap
aliases (window >= N reproduces H2O's plain column sums), invariants that any
correct implementation keeps, and a scalar brute force on tiny prompts.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

from oracle import brute
from oracle import waits_oracle as orc
from synth import make_prompt

F32 = lambda x: float(np.float32(x))  # noqa: E731


def _prompt(n, hq, hkv, d, seed, heavy=False, dtype="f32"):
    bt = make_prompt(seed, n, hq, hkv, d, heavy=heavy, dtype=dtype)
    return bt.q.astype(np.float64), bt.k.astype(np.float64), bt.cu_seqlens


def _softmax_rows(q, k, g, h, scale):
    """Causal attention rows of one head via scipy (a library routine)."""
    n = q.shape[0]
    logits = scale * (q[:, g, :] @ k[:, h, :].T)
    logits[np.triu_indices(n, 1)] = -np.inf
    return softmax(logits, axis=1)


# ---------------------------------------------------------------- weights ---

@pytest.mark.parametrize("n,b", [(1, 1), (7, 1), (64, 16), (512, 16), (40, 128)])
def test_weights_a0_is_half(n, b):
    w = orc.sigmoid_weights(n, 0.0, b)
    assert np.all(w == 0.5)


@pytest.mark.parametrize("n,b", [(1, 1), (9, 1), (64, 16), (512, 128), (10, 32768)])
def test_weights_ainf_is_step(n, b):
    # 0-based positions: exactly the last min(b, n) rows keep weight 1
    w = orc.sigmoid_weights(n, math.inf, b)
    expect = np.zeros(n)
    expect[max(0, n - b):] = 1.0
    assert np.array_equal(w, expect)
    assert w.sum() == min(b, n)


@pytest.mark.parametrize("a", [0.01, 1.0, 10.0])
def test_weights_sigmoid_symmetry(a):
    # w(c + x) + w(c - x) = 1 around the half-integer centre c = N - b - 0.5
    n, b = 300, 137
    w = orc.sigmoid_weights(n, a, b)
    c = n - b - 0.5
    for x in (0.5, 1.5, 10.5, 100.5):
        lo, hi = int(c - x), int(c + x)
        assert abs(w[lo] + w[hi] - 1.0) < 1e-15
        assert w[hi] > 0.5 > w[lo]
    assert np.all(np.diff(w) >= 0)


def test_weights_take_float32_a():
    # a crosses the boundary as float32; 0.01 becomes 0.0099999998
    w = orc.sigmoid_weights(10, 0.01, 3)
    a32 = float(np.float32(0.01))
    assert a32 != 0.01
    assert w[0] == 1.0 / (1.0 + math.exp(-a32 * (0 - 6.5)))


# ---------------------------------------------------- uniform attention ---

def _harmonic(n):
    return sum((Fraction(1, i) for i in range(1, n + 1)), Fraction(0))


@pytest.mark.parametrize("n,group", [(1, 1), (8, 1), (33, 2), (100, 4)])
def test_uniform_attention_h2o_closed_form(n, group):
    # Q = 0 => every causal row is uniform: A[q, k] = 1/(q+1).  At a = 0,
    # w = 1/2, so s[k] = (G/2) (H_N - H_k) with H the harmonic numbers.
    d = 8
    q = np.zeros((n, group, d))
    k = np.random.default_rng(5).standard_normal((n, 1, d))
    s = orc.waits_scores(q, k, np.array([0, n]), group, 1, [0.0], [1], 0.125)[0]
    hn = _harmonic(n)
    for key in range(n):
        exact = Fraction(group, 2) * (hn - _harmonic(key))
        assert abs(s[key] - float(exact)) <= 1e-13 * float(exact)


@pytest.mark.parametrize("n,window", [(16, 1), (16, 5), (50, 16), (12, 40)])
def test_uniform_attention_snap_window_closed_form(n, window):
    # a = inf, b = W: s[k] = sum over the last W rows q >= k of 1/(q+1)
    q = np.zeros((n, 1, 4))
    k = np.ones((n, 1, 4))
    s = orc.waits_scores(q, k, np.array([0, n]), 1, 1, [math.inf], [window], 0.5)[0]
    for key in range(n):
        exact = sum((Fraction(1, r + 1) for r in range(max(key, n - window), n)),
                    Fraction(0))
        assert abs(s[key] - float(exact)) <= 1e-14


# --------------------------------------------------------------- limits ---

@pytest.mark.parametrize("seed,n,hq,hkv,d", [(1, 40, 2, 1, 16), (2, 65, 4, 2, 8),
                                             (3, 128, 1, 1, 64)])
def test_tova_limit_is_last_row(seed, n, hq, hkv, d):
    q, k, cu = _prompt(n, hq, hkv, d, seed)
    scale = F32(1 / math.sqrt(d))
    s = orc.waits_scores(q, k, cu, hq, hkv, [math.inf], [1], scale)
    g = hq // hkv
    for h in range(hkv):
        ref = sum(_softmax_rows(q, k, h * g + j, h, scale)[-1] for j in range(g))
        np.testing.assert_allclose(s[h], ref, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("window", [2, 16, 31])
def test_snapkv_limit_is_last_window_rows(window):
    n, hq, hkv, d = 48, 4, 2, 16
    q, k, cu = _prompt(n, hq, hkv, d, 11, heavy=True)
    scale = F32(1 / math.sqrt(d))
    s = orc.waits_scores(q, k, cu, hq, hkv, [math.inf], [window], scale)
    g = hq // hkv
    for h in range(hkv):
        ref = sum(_softmax_rows(q, k, h * g + j, h, scale)[n - window:].sum(axis=0)
                  for j in range(g))
        np.testing.assert_allclose(s[h], ref, rtol=1e-12)


@pytest.mark.parametrize("window", [48, 32768])
def test_h2o_alias_window_covers_prompt(window):
    # the README's H2O alias is the snap scorer with a window >= N: plain sums
    n, hq, hkv, d = 48, 2, 1, 16
    q, k, cu = _prompt(n, hq, hkv, d, 12)
    scale = F32(0.25)
    s = orc.waits_scores(q, k, cu, hq, hkv, [math.inf], [window], scale)[0]
    ref = sum(_softmax_rows(q, k, j, 0, scale).sum(axis=0) for j in range(hq))
    np.testing.assert_allclose(s, ref, rtol=1e-12)


def test_h2o_a0_is_half_the_column_sums():
    n, hq, hkv, d = 64, 4, 1, 32
    q, k, cu = _prompt(n, hq, hkv, d, 13, heavy=True)
    scale = F32(1 / math.sqrt(d))
    s = orc.waits_scores(q, k, cu, hq, hkv, [0.0], [16], scale)[0]
    ref = 0.5 * sum(_softmax_rows(q, k, j, 0, scale).sum(axis=0) for j in range(hq))
    np.testing.assert_allclose(s, ref, rtol=1e-12)


# ----------------------------------------------------------- invariants ---

@pytest.mark.parametrize("a,b", [(0.0, 1), (0.01, 128), (1.0, 16), (10.0, 1),
                                 (10.0, 16), (math.inf, 7), (3.0, 500)])
def test_attention_mass(a, b):
    # every softmax row sums to one: sum_k s[h, k] = G * sum_q w[q]
    n, hq, hkv, d = 200, 4, 2, 16
    q, k, cu = _prompt(n, hq, hkv, d, 21, heavy=True)
    s = orc.waits_scores(q, k, cu, hq, hkv, [a], [b], F32(0.25))
    w = orc.sigmoid_weights(n, a, b)
    for h in range(hkv):
        assert abs(s[h].sum() - 2 * w.sum()) <= 1e-12 * max(1.0, w.sum())


def test_causal_support():
    # s[k] depends only on query rows q >= k: perturb rows < k0, keys >= k0 stay
    n, hq, hkv, d, k0 = 96, 2, 1, 16, 40
    q, k, cu = _prompt(n, hq, hkv, d, 31)
    s1 = orc.waits_scores(q, k, cu, hq, hkv, [0.05], [16], F32(0.25))
    q2 = q.copy()
    q2[:k0] += np.random.default_rng(0).standard_normal(q2[:k0].shape)
    s2 = orc.waits_scores(q2, k, cu, hq, hkv, [0.05], [16], F32(0.25))
    np.testing.assert_array_equal(s1[:, k0:], s2[:, k0:])
    assert not np.allclose(s1[:, :k0], s2[:, :k0])


def test_gqa_group_is_a_sum_and_order_free():
    n, d = 50, 8
    q, k, cu = _prompt(n, 4, 2, d, 41)
    s = orc.waits_scores(q, k, cu, 4, 2, [1.0], [5], F32(0.3))
    # head h sums query heads 2h and 2h+1, each seen as a 1:1 problem
    for h in range(2):
        parts = [orc.waits_scores(q[:, [2 * h + j]], k[:, [h]], cu, 1, 1, [1.0], [5],
                                  F32(0.3))[0] for j in range(2)]
        np.testing.assert_allclose(s[h], parts[0] + parts[1], rtol=1e-13)
    swapped = q[:, [1, 0, 3, 2]]
    s2 = orc.waits_scores(swapped, k, cu, 4, 2, [1.0], [5], F32(0.3))
    np.testing.assert_allclose(s, s2, rtol=1e-13)


def test_packed_prompts_are_independent():
    # positions restart in every prompt; a prompt's scores ignore its neighbours
    a = make_prompt(51, 30, 2, 1, 8, heavy=False, dtype="f32")
    b = make_prompt(52, 45, 2, 1, 8, heavy=False, dtype="f32")
    q = np.concatenate([a.q, b.q]).astype(np.float64)
    k = np.concatenate([a.k, b.k]).astype(np.float64)
    cu = np.array([0, 30, 75])
    s = orc.waits_scores(q, k, cu, 2, 1, [1.0, 10.0], [4, 9], F32(0.35))
    sa = orc.waits_scores(a.q.astype(np.float64), a.k.astype(np.float64), a.cu_seqlens,
                          2, 1, [1.0], [4], F32(0.35))
    sb = orc.waits_scores(b.q.astype(np.float64), b.k.astype(np.float64), b.cu_seqlens,
                          2, 1, [10.0], [9], F32(0.35))
    np.testing.assert_array_equal(s[:, :30], sa)
    np.testing.assert_array_equal(s[:, 30:], sb)


def test_lse_closed_form_and_consistency():
    # Q = 0: lse[q] = ln(q + 1) exactly (uniform rows)
    n = 37
    q = np.zeros((n, 1, 4))
    k = np.random.default_rng(3).standard_normal((n, 1, 4))
    lse = orc.waits_lse(q, k, np.array([0, n]), 1, 1, 0.5)[0]
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), rtol=1e-15, atol=1e-15)
    # random Q: softmax rows rebuilt from lse sum to 1
    q, k, cu = _prompt(60, 2, 1, 16, 61)
    lse = orc.waits_lse(q, k, cu, 2, 1, F32(0.25))
    for g in range(2):
        logits = F32(0.25) * (q[:, g] @ k[:, 0].T)
        logits[np.triu_indices(60, 1)] = -np.inf
        np.testing.assert_allclose(np.exp(logits - lse[g][:, None]).sum(axis=1), 1.0,
                                   rtol=1e-13)


# ---------------------------------------------------------- brute force ---

CASES = [
    # n, hq, hkv, d, a, b
    (1, 1, 1, 4, 1.0, 16),
    (2, 1, 1, 4, 0.0, 1),
    (17, 4, 1, 8, 1.0, 2),
    (33, 8, 2, 4, 10.0, 16),
    (64, 1, 1, 64, 0.01, 128),
    (48, 4, 2, 8, math.inf, 1),
    (40, 2, 2, 8, math.inf, 45),
    (63, 2, 1, 16, 3.0, 64),
]


@pytest.mark.parametrize("n,hq,hkv,d,a,b", CASES)
def test_numpy_oracle_matches_brute_force(n, hq, hkv, d, a, b):
    bt = make_prompt(70 + n, n, hq, hkv, d, heavy=True, dtype="bf16")
    scale = F32(1 / math.sqrt(d))
    a32 = F32(a)
    got = orc.waits_scores(bt.q, bt.k, bt.cu_seqlens, hq, hkv, [a32], [b], scale)
    ref = brute.scores(bt.q.astype(float).tolist(), bt.k.astype(float).tolist(),
                       hq, hkv, a32, b, scale)
    for h in range(hkv):
        np.testing.assert_allclose(got[h], ref[h], rtol=1e-12, atol=1e-300)


# ----------------------------------------------------------------- top-k ---

def test_topk_matches_full_sort():
    rng = np.random.default_rng(7)
    for n, budget in [(1, 1), (10, 3), (100, 100), (100, 128), (257, 64)]:
        s = rng.random(n)
        s[rng.integers(0, n, n // 4)] = 0.5      # plenty of exact ties
        got = orc.select_topk(s, budget)
        assert got.tolist() == brute.topk(s.tolist(), budget)


def test_topk_ties_go_to_lower_position():
    assert orc.select_topk(np.ones(10), 4).tolist() == [0, 1, 2, 3]
    s = np.array([1.0, 3.0, 2.0, 2.0, 2.0, 0.5, 2.0])
    assert orc.select_topk(s, 3).tolist() == [1, 2, 3]
    assert orc.select_topk(s, 5).tolist() == [1, 2, 3, 4, 6]
    assert orc.select_topk(np.array([5.0, 4.0]), 4).tolist() == [0, 1, -1, -1]


def test_topk_tie_pins_from_uniform_attention():
    # Q = 0, a = inf, b = 1: every score is 1/N -> the first `budget` keys.
    # Q = 0, a = 0: scores strictly decrease with k -> also the first keys.
    n = 300
    q = np.zeros((n, 1, 4))
    k = np.random.default_rng(9).standard_normal((n, 1, 4))
    cu = np.array([0, n])
    for a, b in [(math.inf, 1), (0.0, 1)]:
        s = orc.waits_scores(q, k, cu, 1, 1, [a], [b], 0.5)
        idx = orc.waits_select(s, cu, 1, 128)
        assert idx[0, 0].tolist() == list(range(128))


def test_compact_gathers_exact_bits():
    bt = make_prompt(3, 50, 2, 2, 8, heavy=True, dtype="bf16")
    idx = np.array([[[0, 7, 49, -1], [3, 4, 5, 6]]], dtype=np.int32)
    kc, vc = orc.waits_compact(bt.k_bits, bt.v_bits, bt.cu_seqlens, idx)
    assert kc.dtype == np.uint16
    assert np.array_equal(kc[0, 0, 1], bt.k_bits[7, 0])
    assert np.array_equal(vc[0, 1, 3], bt.v_bits[6, 1])
    assert not kc[0, 0, 3].any() and not vc[0, 0, 3].any()


def test_sampling_restrictions_keep_their_stated_bounds():
    # row_min: exact for keys >= row_min; weight_floor: error <= G * N * floor
    n, hq, hkv, d = 160, 4, 2, 16
    q, k, cu = _prompt(n, hq, hkv, d, 81, heavy=True)
    full = orc.waits_scores(q, k, cu, hq, hkv, [0.3], [9], F32(0.25))
    tail = orc.waits_scores(q, k, cu, hq, hkv, [0.3], [9], F32(0.25), row_min=[100])
    np.testing.assert_array_equal(tail[:, 100:], full[:, 100:])
    floor = 1e-12
    cut = orc.waits_scores(q, k, cu, hq, hkv, [0.3], [9], F32(0.25), weight_floor=floor)
    assert np.all(np.abs(cut - full) <= 2 * n * floor)
    assert np.any(cut != full)


@pytest.mark.parametrize("a,b,floor", [(0.0, 1, 0.0), (0.05, 7, 0.0), (1.0, 16, 1e-30),
                                       (math.inf, 40, 0.0)])
def test_pooled_kv_head_scores_equal_the_oracle(a, b, floor):
    # the full-size GPU checks add per-(query head, row range) oracle pieces
    # computed in worker processes; on a small prompt that sum must equal
    # waits_scores of the whole KV head to rounding
    import oracle_pool
    n, hq, hkv, d = 700, 6, 2, 64
    bt = make_prompt(77, n, hq, hkv, d, heavy=True, dtype="bf16")
    scale = float(np.float32(1 / math.sqrt(d)))
    ref = orc.waits_scores(bt.q, bt.k, bt.cu_seqlens, hq, hkv, [a], [b], scale, weight_floor=floor)
    with oracle_pool.make_pool() as pool:
        for h in range(hkv):
            got = oracle_pool.kv_head_scores(bt.q, bt.k, h, hq // hkv, a, b, scale,
                                             weight_floor=floor, pool=pool)
            np.testing.assert_allclose(got, ref[h], rtol=1e-12, atol=0)
