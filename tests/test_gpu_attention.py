"""GPU parity: the prefill attention forward with its row log-sum-exp, and the
WAITS scores computed from that lse (pass 1 taken from the attention call),
through the C ABI, against the float64 oracles.

Bar for out, derived from the arithmetic: P is rounded to bf16 for the P V
product (each weight moves by at most 2^-9 relative, so out by at most
2^-9 max|V|), out is rounded to bf16 (2^-9 relative), and the scores carry
the fp32 dot-product error (~3e-4 max|V| at most); so
|out - ref| <= 2.5e-3 max|V| + 2^-8 |ref|.  lse is fp32 throughout:
|lse - ref| <= 2e-4.  Sampled rows at full size use the decode oracle (row q
of causal attention is decode attention over keys 0..q).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import attention_score_eviction_amd as W
from oracle import attention_oracle as att
from oracle import decode_oracle as dec
from oracle import waits_oracle as orc
from synth import make_batch, make_prompt

from parity import DEV, check_scores, check_select_exact, check_select_vs_oracle, to_device

pytestmark = pytest.mark.gpu

OUT_ATOL = 2.5e-3   # times max |V| of the prompt's head
OUT_RTOL = 2.0 ** -8
LSE_TOL = 2e-4


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    W.waits.lib()
    yield


def _bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def _check_rows(out_gpu, lse_gpu, ref_out, ref_lse, vmax, rows=None):
    """out_gpu [T, Hq, d] / lse_gpu [Hq, T] (numpy) against the oracle at the
    given token rows (all when None); vmax[t, g]: max |V| the row can see."""
    sel = slice(None) if rows is None else rows
    o, r = out_gpu[sel], ref_out[sel]
    lim = OUT_ATOL * vmax[sel][..., None] + OUT_RTOL * np.abs(r)
    bad = np.abs(o - r) > lim
    assert not bad.any(), f"out mismatch at {np.argwhere(bad)[:5]}: gpu {o[bad][:5]} ref {r[bad][:5]}"
    dl = np.abs(lse_gpu[:, sel] - ref_lse[:, sel])
    assert dl.max() <= LSE_TOL, f"lse max err {dl.max():.3e}"


def _vmax(bt, group):
    """max |V| per (token, query head) over the whole prompt of that token."""
    tot, hq = bt.q.shape[0], bt.q.shape[1]
    vm = np.zeros((tot, hq))
    for p in range(bt.batch):
        lo, hi = int(bt.cu_seqlens[p]), int(bt.cu_seqlens[p + 1])
        if hi == lo:
            continue
        m = np.abs(bt.v[lo:hi]).max(axis=(0, 2))        # per KV head
        for g in range(hq):
            vm[lo:hi, g] = m[g // group]
    return vm


def _run(bt, scale):
    q, k, v = to_device(bt)
    out, lse = W.attention(q, k, v, bt.cu_seqlens, scale)
    torch.cuda.synchronize()
    return _bf16_to_f64(out), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("hq,hkv,d", [(1, 1, 64), (2, 1, 128), (6, 2, 64), (8, 2, 128), (32, 8, 64),
                                      (8, 1, 128)])
def test_attention_small_ragged_batch(hq, hkv, d):
    # lengths cover one row, partial row tiles and blocks, and several blocks
    lengths = [1, 2, 31, 33, 64, 65, 200, 257, 0, 700]
    _say(f"attention small hq={hq} hkv={hkv} d={d}")
    bt = make_batch([40 + i for i in range(len(lengths))], lengths, hq, hkv, d, heavy=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    out, lse = _run(bt, scale)
    ref_out, ref_lse = att.prefill_attention(bt.q, bt.k, bt.v, bt.cu_seqlens, hq, hkv, scale)
    _check_rows(out, lse, ref_out, ref_lse, _vmax(bt, hq // hkv))


def test_attention_scale_other_than_default():
    # a sharp softmax (scale 0.3, logits in the tens) over ragged prompts
    _say("attention scale 0.3")
    bt = make_batch([51, 52], [1500, 333], 8, 2, 128, heavy=True)
    scale = 0.3
    out, lse = _run(bt, scale)
    ref_out, ref_lse = att.prefill_attention(bt.q, bt.k, bt.v, bt.cu_seqlens, 8, 2, float(np.float32(scale)))
    _check_rows(out, lse, ref_out, ref_lse, _vmax(bt, 4))


def test_attention_llama32_1b_full():
    # 32/8/64 at N = 2048, every row against the oracle
    _say("attention 1b shape N=2048")
    bt = make_prompt(1, 2048, 32, 8, 64, heavy=True)
    scale = float(np.float32(1 / 8))
    out, lse = _run(bt, scale)
    ref_out, ref_lse = att.prefill_attention(bt.q, bt.k, bt.v, bt.cu_seqlens, 32, 8, scale)
    _check_rows(out, lse, ref_out, ref_lse, _vmax(bt, 4))


def test_attention_llama31_8b_sampled_rows():
    # one 8B layer at N = 16384: sampled rows through the decode oracle, lse
    # of every row through the WAITS oracle's normaliser on a subset of rows
    _say("attention 8b N=16384 sampled")
    n = 16384
    bt = make_prompt(1000, n, 32, 8, 128, heavy=True)
    scale = float(np.float32(1 / math.sqrt(128)))
    out, lse = _run(bt, scale)
    rows = np.concatenate([np.arange(0, 40), np.array([255, 256, 4095, 8191, 8192]),
                           np.arange(n - 40, n)])
    ref_out = np.zeros((n, 32, 128))
    ref_lse = np.zeros((32, n))
    for r in rows:
        for g in range(32):
            o, l = dec.decode_head(bt.q[r, g], bt.k[:r + 1, g // 4], bt.v[:r + 1, g // 4], scale)
            ref_out[r, g], ref_lse[g, r] = o, l
    _check_rows(out, lse, ref_out, ref_lse, _vmax(bt, 4), rows=rows)


def test_attention_long_context_sampled_rows():
    # one layer of the long-context shape, N = 131072 (2048 row blocks per KV
    # head, key ranges up to the whole prompt): sampled rows through the
    # decode oracle, including both ends and row-block boundaries
    _say("attention long N=131072 sampled")
    n = 131072
    bt = make_prompt(2, n, 32, 8, 128, heavy=True)
    scale = float(np.float32(1 / math.sqrt(128)))
    out, lse = _run(bt, scale)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([np.array([0, 1, 63, 64, 65, 16383, 16384, 65535, 65536, n - 2, n - 1]),
                                     rng.integers(0, n, size=13)]))
    ref_out = np.zeros((n, 32, 128))
    ref_lse = np.zeros((32, n))
    for r in rows:
        for g in range(32):
            o, l = dec.decode_head(bt.q[r, g], bt.k[:r + 1, g // 4], bt.v[:r + 1, g // 4], scale)
            ref_out[r, g], ref_lse[g, r] = o, l
    _check_rows(out, lse, ref_out, ref_lse, _vmax(bt, 4), rows=rows)


def test_attention_lse_feeds_waits_pass2():
    # The fused flow: lse from the attention call replaces pass 1; the scores,
    # selection and compaction then meet the WAITS bar against the oracle.
    _say("attention lse -> colsum -> select")
    lengths = [3000, 700, 1]
    bt = make_batch([7, 8, 9], lengths, 32, 8, 128, heavy=True)
    a, b, budget = [1.0, 0.0, 1.0], [16, 1, 16], 128
    q, k, v = to_device(bt)
    out, lse = W.attention(q, k, v, bt.cu_seqlens)
    s = W.colsum(q, k, lse, bt.cu_seqlens, a, b)
    idx, kc, vc = W.select_compact(s, k, v, bt.cu_seqlens, budget)
    lse_ref = W.lse(q, k, bt.cu_seqlens, a, b)       # the library's own pass 1, processed rows
    torch.cuda.synchronize()
    scale = float(np.float32(1 / math.sqrt(128)))
    s_ref = orc.waits_scores(bt.q, bt.k, bt.cu_seqlens, 32, 8, a, b, scale)
    s_gpu = s.cpu().numpy()
    check_scores(s_gpu, s_ref)
    check_select_exact(idx.cpu().numpy(), s_gpu, bt.cu_seqlens, budget)
    check_select_vs_oracle(idx.cpu().numpy(), s_ref, bt.cu_seqlens, budget)
    # at the rows pass 1 processes, the two lse agree to fp32 rounding
    fr = W.waits.first_rows(bt.cu_seqlens, a, b)
    lg, lr = lse.cpu().numpy(), lse_ref.cpu().numpy()
    for p in range(3):
        lo, hi = int(bt.cu_seqlens[p]), int(bt.cu_seqlens[p + 1])
        sl = slice(lo + int(fr[p]), hi)
        np.testing.assert_allclose(lg[:, sl], lr[:, sl], rtol=0, atol=LSE_TOL)


def test_attention_head_major_strides_and_determinism():
    _say("attention head-major views, repeatability")
    bt = make_prompt(5, 777, 8, 2, 128, heavy=True)
    q, k, v = to_device(bt)
    qh = q.permute(1, 0, 2).contiguous().permute(1, 0, 2)     # [T, H, d] views of head-major storage
    kh = k.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    vh = v.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    o1, l1 = W.attention(q, k, v, bt.cu_seqlens)
    o2, l2 = W.attention(qh, kh, vh, bt.cu_seqlens)
    o3, l3 = W.attention(q, k, v, bt.cu_seqlens)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_attention_packed_qkv_views():
    # Q, K and V as views into one [T, Hq + 2 Hkv, d] buffer
    _say("attention packed qkv views")
    bt = make_batch([25, 26], [900, 400], 8, 2, 128, heavy=True)
    q, k, v = to_device(bt)
    qkv = torch.cat([q, k, v], dim=1).contiguous()
    o1, l1 = W.attention(q, k, v, bt.cu_seqlens)
    o2, l2 = W.attention(qkv[:, :8], qkv[:, 8:10], qkv[:, 10:12], bt.cu_seqlens)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_attention_rejects_fp32():
    bt = make_prompt(2, 64, 2, 1, 64, heavy=False, dtype="f32")
    q, k, v = to_device(bt)
    with pytest.raises(W.WaitsError) as e:
        W.attention(q, k, v, bt.cu_seqlens)
    assert e.value.code == W.waits.WAITS_EUNSUPPORTED
