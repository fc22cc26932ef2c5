"""Pins for the decode-attention oracle (no GPU).

The oracle of decode attention over a compacted cache is fixed against
closed forms (uniform attention, one row, two rows), the prefill oracle's
last causal row (the TOVA limit of the WAITS README's introduction picks
exactly that row), a scalar brute force, and invariants of softmax attention
(row permutation, padding rows, the GQA head map, shifts of V).
"""
import math

import numpy as np
import pytest

from oracle import brute
from oracle import decode_oracle as dec
from oracle import waits_oracle as orc
from synth import make_prompt

F32 = lambda x: float(np.float32(x))  # noqa: E731


def _cache(seed, bsz, hq, hkv, cap, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((bsz, hq, d))
    kc = rng.standard_normal((bsz, hkv, cap, d))
    vc = rng.standard_normal((bsz, hkv, cap, d))
    return q, kc, vc


def test_uniform_attention_is_the_mean_of_v():
    # q = 0: every row gets weight 1/len, lse = ln(len)
    q, kc, vc = _cache(1, 3, 4, 2, 20, 8)
    q[:] = 0.0
    lens = [20, 7, 1]
    out, lse = dec.waits_decode(q, kc, vc, lens, 0.125)
    for i, n in enumerate(lens):
        for g in range(4):
            np.testing.assert_allclose(out[i, g], vc[i, g // 2, :n].mean(axis=0), rtol=1e-13)
            assert lse[i, g] == pytest.approx(math.log(n), rel=1e-14)


def test_one_row_returns_that_row():
    q, kc, vc = _cache(2, 1, 2, 1, 5, 16)
    out, lse = dec.waits_decode(q, kc, vc, [1], 0.3)
    for g in range(2):
        assert np.array_equal(out[0, g], vc[0, 0, 0])
        assert lse[0, g] == pytest.approx(F32(0.3) * float(q[0, g] @ kc[0, 0, 0]), rel=1e-14)


def test_two_rows_closed_form_depends_on_the_scale():
    # out = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1 with s_j = scale <q, k_j>
    q = np.array([[[1.0, 2.0]]])
    kc = np.array([[[[1.0, 0.0], [0.0, 1.0], [9.0, 9.0]]]])
    vc = np.array([[[[1.0, 0.0], [0.0, 1.0], [5.0, 5.0]]]])
    scale = 0.75
    out, lse = dec.waits_decode(q, kc, vc, [2], scale)
    s0, s1 = F32(scale) * 1.0, F32(scale) * 2.0
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(out[0, 0], [p0, 1.0 - p0], rtol=1e-14)
    assert lse[0, 0] == pytest.approx(math.log(math.exp(s0) + math.exp(s1)), rel=1e-14)


def test_empty_cache_gives_zero_and_minus_inf():
    q, kc, vc = _cache(3, 2, 2, 2, 4, 8)
    out, lse = dec.waits_decode(q, kc, vc, [0, 4], 0.5)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


@pytest.mark.parametrize("hq,hkv,n,d", [(1, 1, 9, 4), (4, 2, 13, 8), (6, 3, 3, 5)])
def test_matches_scalar_brute_force(hq, hkv, n, d):
    q, kc, vc = _cache(10 + n, 2, hq, hkv, n + 2, d)
    lens = [n, 1]
    scale = 1 / math.sqrt(d)
    out, lse = dec.waits_decode(q, kc, vc, lens, scale)
    for i, ln in enumerate(lens):
        for g in range(hq):
            h = g // (hq // hkv)
            bo, bl = brute.decode(q[i, g].tolist(), kc[i, h, :ln].tolist(),
                                  vc[i, h, :ln].tolist(), F32(scale))
            np.testing.assert_allclose(out[i, g], bo, rtol=1e-12, atol=1e-14)
            assert lse[i, g] == pytest.approx(bl, rel=1e-13)


def test_last_prompt_row_matches_the_prefill_oracle():
    # Decoding the prompt's last token over its full, uncompacted cache is the
    # last causal row of prefill attention: its normaliser is waits_lse's last
    # row, and with a = inf, b = 1 (TOVA) the WAITS score of each key is exactly
    # that row's attention (one query head per KV head here), so the output is
    # scores @ V.
    n, hq, hkv, d = 48, 2, 2, 16
    bt = make_prompt(5, n, hq, hkv, d, heavy=True, dtype="f32")
    qf, kf = bt.q.astype(np.float64), bt.k.astype(np.float64)
    vf = bt.v.astype(np.float64)
    scale = 1 / math.sqrt(d)
    qd = qf[n - 1][None]                               # [1, Hq, d]
    kc = kf.transpose(1, 0, 2)[None]                   # [1, Hkv, N, d]
    vc = vf.transpose(1, 0, 2)[None]
    out, lse = dec.waits_decode(qd, kc, vc, [n], scale)
    lse_ref = orc.waits_lse(qf, kf, bt.cu_seqlens, hq, hkv, scale, rows_per_prompt=[[n - 1]])
    s_tova = orc.waits_scores(qf, kf, bt.cu_seqlens, hq, hkv, [math.inf], [1], scale)
    for g in range(hq):
        assert lse[0, g] == pytest.approx(lse_ref[g, n - 1], rel=1e-13)
        np.testing.assert_allclose(out[0, g], s_tova[g] @ vf[:, g], rtol=1e-12, atol=1e-14)


def test_gqa_map_reads_head_g_over_group():
    # V rows of KV head h all equal h: out[g] is exactly g // G for any weights
    q, kc, vc = _cache(4, 2, 8, 2, 11, 4)
    for h in range(2):
        vc[:, h] = float(h)
    out, _ = dec.waits_decode(q, kc, vc, [11, 6], 0.4)
    for g in range(8):
        np.testing.assert_allclose(out[:, g], float(g // 4), rtol=0, atol=1e-14)


def test_rows_past_len_are_not_read():
    q, kc, vc = _cache(6, 1, 2, 1, 10, 8)
    out, lse = dec.waits_decode(q, kc, vc, [6], 0.5)
    kc[0, 0, 6:] = np.nan
    vc[0, 0, 6:] = np.nan
    out2, lse2 = dec.waits_decode(q, kc, vc, [6], 0.5)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_row_order_and_v_shift_invariance():
    q, kc, vc = _cache(7, 1, 4, 2, 17, 8)
    out, lse = dec.waits_decode(q, kc, vc, [17], 0.3)
    perm = np.random.default_rng(0).permutation(17)
    out_p, lse_p = dec.waits_decode(q, kc[:, :, perm], vc[:, :, perm], [17], 0.3)
    np.testing.assert_allclose(out_p, out, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse_p, lse, rtol=1e-14)
    shift = np.arange(8) * 0.5
    out_s, _ = dec.waits_decode(q, kc, vc + shift, [17], 0.3)
    np.testing.assert_allclose(out_s, out + shift, rtol=1e-13, atol=1e-13)
