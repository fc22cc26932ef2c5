"""Pins for the prefill-attention oracle (no GPU).

The oracle of causal attention with its row log-sum-exp is fixed against the
WAITS oracle's own row normaliser (written separately), the closed form of
uniform attention (a running mean of V, lse = ln(q+1)), the decode oracle at
the last row, a scalar brute force, causality and the GQA head map.
"""
import math

import numpy as np
import pytest

from oracle import attention_oracle as att
from oracle import brute
from oracle import decode_oracle as dec
from oracle import waits_oracle as orc
from synth import make_batch, make_prompt

F32 = lambda x: float(np.float32(x))  # noqa: E731


def _batch(lengths, hq, hkv, d, seed=3):
    bt = make_batch([seed + i for i in range(len(lengths))], lengths, hq, hkv, d, heavy=True,
                    dtype="f32")
    return bt.q.astype(np.float64), bt.k.astype(np.float64), bt.v.astype(np.float64), bt.cu_seqlens


def test_lse_equals_the_waits_row_normaliser():
    q, k, v, cu = _batch([300, 40, 1], 8, 2, 16)
    scale = 0.25
    _, lse = att.prefill_attention(q, k, v, cu, 8, 2, scale, row_block=64)
    ref = orc.waits_lse(q, k, cu, 8, 2, scale)
    np.testing.assert_allclose(lse, ref, rtol=1e-13, atol=1e-13)


def test_uniform_attention_is_the_running_mean():
    q, k, v, cu = _batch([70, 9], 4, 2, 8)
    q[:] = 0.0
    out, lse = att.prefill_attention(q, k, v, cu, 4, 2, 0.5, row_block=16)
    for p in range(2):
        lo, hi = int(cu[p]), int(cu[p + 1])
        for g in range(4):
            csum = np.cumsum(v[lo:hi, g // 2], axis=0)
            cnt = np.arange(1, hi - lo + 1)[:, None]
            np.testing.assert_allclose(out[lo:hi, g], csum / cnt, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(lse[g, lo:hi], np.log(cnt[:, 0]), rtol=1e-14)


def test_first_row_is_v0_and_last_row_is_decode():
    q, k, v, cu = _batch([50], 4, 1, 16)
    scale = 1 / math.sqrt(16)
    out, lse = att.prefill_attention(q, k, v, cu, 4, 1, scale)
    for g in range(4):
        assert np.array_equal(out[0, g], v[0, 0])
        assert lse[g, 0] == pytest.approx(F32(scale) * float(q[0, g] @ k[0, 0]), rel=1e-14)
    od, ld = dec.waits_decode(q[49][None], k.transpose(1, 0, 2)[None], v.transpose(1, 0, 2)[None],
                              [50], scale)
    np.testing.assert_allclose(out[49], od[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[:, 49], ld[0], rtol=1e-13)


@pytest.mark.parametrize("n,hq,hkv,d", [(13, 2, 1, 4), (9, 3, 3, 6), (20, 4, 2, 5)])
def test_matches_scalar_brute_force(n, hq, hkv, d):
    bt = make_prompt(n + 100, n, hq, hkv, d, heavy=False, dtype="f32")
    q, k, v = (x.astype(np.float64) for x in (bt.q, bt.k, bt.v))
    scale = 0.3
    out, lse = att.prefill_attention(q, k, v, bt.cu_seqlens, hq, hkv, scale, row_block=4)
    bo, bl = brute.attention(q.tolist(), k.tolist(), v.tolist(), hq // hkv, F32(scale))
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(bl), rtol=1e-13)


def test_causality_and_gqa_map():
    q, k, v, cu = _batch([64], 8, 2, 8)
    out, lse = att.prefill_attention(q, k, v, cu, 8, 2, 0.4)
    k2, v2 = k.copy(), v.copy()
    k2[40:] = np.random.default_rng(0).standard_normal(k2[40:].shape)
    v2[40:] = 7.0
    out2, lse2 = att.prefill_attention(q, k2, v2, cu, 8, 2, 0.4)
    assert np.array_equal(out[:40], out2[:40]) and np.array_equal(lse[:, :40], lse2[:, :40])
    v3 = v.copy()
    for h in range(2):
        v3[:, h] = float(h)
    out3, _ = att.prefill_attention(q, k, v3, cu, 8, 2, 0.4)
    for g in range(8):
        np.testing.assert_allclose(out3[:, g], float(g // 4), rtol=0, atol=1e-14)
