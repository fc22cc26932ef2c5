"""GPU parity: decode attention over the compacted cache, through the C ABI,
against the float64 oracle (oracle/decode_oracle.py).

Bar, derived from the arithmetic: a score is a fp32-accumulated dot product
of at most 128 exact bf16 (or rounded fp32) products, so its error is below
about d * 2^-24 * |q| |k| * scale (~1.4e-4 here) and moves each probability
by that relative amount; the output, a convex combination of V rows, moves
by at most twice that times max |V|; fp32 sums add ~1e-5.  So
|out - ref| <= 3e-4 * max|V| (over the attended rows) and |lse - ref| <= 2e-4.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import attention_score_eviction_amd as W
from oracle import decode_oracle as dec
from synth import make_batch, make_decode

from parity import DEV, to_device

pytestmark = pytest.mark.gpu

OUT_TOL = 3e-4   # times max |V| of the attended rows
LSE_TOL = 2e-4


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    W.waits.lib()
    yield


def _to_dev(x):
    if x.dtype == "bf16":
        conv = lambda b: torch.from_numpy(np.ascontiguousarray(b)).view(torch.bfloat16).to(DEV)  # noqa: E731
        return conv(x.q_bits), conv(x.k_bits), conv(x.v_bits)
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (x.q, x.k, x.v))


def _check(out, lse, q, k, v, lens, scale):
    """Compare device results with the oracle over host values q, k, v."""
    ref_out, ref_lse = dec.waits_decode(q, k, v, lens, scale)
    out = out.cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    group = q.shape[1] // k.shape[1]
    worst = 0.0
    for i, n in enumerate(lens):
        n = min(max(int(n), 0), k.shape[2])
        for g in range(q.shape[1]):
            if n == 0:
                assert np.all(out[i, g] == 0.0) and np.isneginf(lse[i, g]), (i, g)
                continue
            vmax = float(np.abs(v[i, g // group, :n]).max())
            err = float(np.abs(out[i, g] - ref_out[i, g]).max())
            assert err <= OUT_TOL * vmax, (i, g, err, vmax)
            assert abs(lse[i, g] - ref_lse[i, g]) <= LSE_TOL, (i, g, lse[i, g], ref_lse[i, g])
            worst = max(worst, err / vmax)
    return worst


def _run(x, lens, scale=None):
    q, k, v = _to_dev(x)
    ln = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, lse = W.decode(q, k, v, ln, scale)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 1), (3, 1), (4, 1), (6, 1), (8, 2), (8, 1),
                                    (12, 1), (32, 8)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "bf16"), (64, "f32"), (128, "f32")])
def test_decode_small_shapes(hq, hkv, d, dtype):
    # capacity 70 (a ragged 16-row tail), lengths full, partial and empty;
    # group sizes cover every query-head chunking (1, 2, 4, 8, and 12 = 8 + 4)
    _say(f"decode small hq={hq} hkv={hkv} d={d} {dtype}")
    x = make_decode(hq * 10 + d, 3, hq, hkv, 70, d, dtype)
    lens = [70, 33, 0]
    scale = 1 / math.sqrt(d)
    out, lse = _run(x, lens, scale)
    _check(out, lse, x.q, x.k, x.v, lens, float(np.float32(scale)))


@pytest.mark.parametrize("cap,lens", [(64, [64]), (65, [65]), (1000, [999]), (4097, [4097]),
                                      (65536, [65536]), (65536, [40001]), (2048, [1]),
                                      (1 << 20, [1 << 20]), (1 << 20, [777777])])
def test_decode_split_and_combine(cap, lens):
    # one sequence, one KV head: the cache is cut into up to 1024 splits that
    # the combine kernel merges (2^20 rows: the largest capacity accepted,
    # every split at its longest)
    _say(f"decode splits cap={cap} lens={lens}")
    x = make_decode(cap % 977, 1, 4, 1, cap, 128, "bf16")
    out, lse = _run(x, lens)
    _check(out, lse, x.q, x.k, x.v, lens, float(np.float32(1 / math.sqrt(128))))


@pytest.mark.parametrize("scale", [0.02, 0.3])
def test_decode_scale_other_than_default(scale):
    _say(f"decode scale {scale}")
    x = make_decode(31, 4, 32, 8, 3000, 128, "bf16")
    lens = [3000, 1234, 1, 2999]
    out, lse = _run(x, lens, scale)
    _check(out, lse, x.q, x.k, x.v, lens, float(np.float32(scale)))


def test_decode_lengths_are_clamped():
    _say("decode clamped lengths")
    x = make_decode(5, 3, 8, 2, 40, 64, "bf16")
    out, lse = _run(x, [1000, -7, 40])
    _check(out, lse, x.q, x.k, x.v, [40, 0, 40], float(np.float32(1 / 8)))


def test_decode_full_size_and_deterministic():
    # 64 sequences of the Llama-3.1-8B shape (32/8/128) over a 2048-row cache,
    # some sequences shorter; two calls agree bit for bit
    _say("decode 64 x 32/8/128 cap 2048")
    x = make_decode(2024, 64, 32, 8, 2048, 128, "bf16")
    rng = np.random.default_rng(7)
    lens = [2048] * 48 + [int(v) for v in rng.integers(1, 2048, size=16)]
    q, k, v = _to_dev(x)
    ln = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, lse = W.decode(q, k, v, ln)
    out2, lse2 = W.decode(q, k, v, ln)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    _check(out, lse, x.q, x.k, x.v, lens, float(np.float32(1 / math.sqrt(128))))


@pytest.mark.parametrize("lengths", [[4096, 100], [700]])
def test_decode_after_prefill_compaction(lengths):
    # The whole flow: WAITS scores, selection and compaction of each prompt on
    # the GPU, then new tokens appended after the kept rows, then one decoding
    # step.  The oracle decodes over the same rows gathered on the host with
    # the GPU's kept positions (the compaction itself is checked bit for bit
    # elsewhere); a prompt shorter than the budget leaves padding rows that
    # must not be attended.
    _say(f"decode after prefill {lengths}")
    hq, hkv, d, budget, new = 32, 8, 64, 128, 8
    bt = make_batch([11 + i for i in range(len(lengths))], lengths, hq, hkv, d, heavy=True,
                    dtype="bf16")
    q, k, v = to_device(bt)
    _, idx, kc, vc = W.score_select_compact(q, k, v, bt.cu_seqlens, [1.0] * len(lengths),
                                            [16] * len(lengths), budget)
    nb = len(lengths)
    cap = budget + new
    x = make_decode(99, nb, hq, hkv, cap, d, "bf16")          # new queries and appended rows
    kcache = torch.from_numpy(x.k_bits).view(torch.bfloat16).to(DEV)
    vcache = torch.from_numpy(x.v_bits).view(torch.bfloat16).to(DEV)
    kept = [min(n, budget) for n in lengths]
    for i in range(nb):
        kcache[i, :, :budget] = kc[i]
        vcache[i, :, :budget] = vc[i]
        # new rows right after the kept ones (a short prompt's padding is overwritten)
        kcache[i, :, kept[i]:kept[i] + new] = torch.from_numpy(x.k_bits[i, :, budget:]).view(torch.bfloat16).to(DEV)
        vcache[i, :, kept[i]:kept[i] + new] = torch.from_numpy(x.v_bits[i, :, budget:]).view(torch.bfloat16).to(DEV)
    lens = [kept[i] + new for i in range(nb)]
    qd = torch.from_numpy(x.q_bits).view(torch.bfloat16).to(DEV)
    out, lse = W.decode(qd, kcache, vcache, torch.tensor(lens, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    # host cache from the prompt's own rows at the GPU's kept positions
    idx_h = idx.cpu().numpy()
    kh = np.zeros((nb, hkv, cap, d))
    vh = np.zeros((nb, hkv, cap, d))
    for i in range(nb):
        lo = int(bt.cu_seqlens[i])
        for h in range(hkv):
            pos = idx_h[i, h, :kept[i]]
            assert np.all(pos >= 0)
            kh[i, h, :kept[i]] = bt.k[lo + pos, h]
            vh[i, h, :kept[i]] = bt.v[lo + pos, h]
            kh[i, h, kept[i]:kept[i] + new] = x.k[i, h, budget:]
            vh[i, h, kept[i]:kept[i] + new] = x.v[i, h, budget:]
    _check(out, lse, x.q, kh, vh, lens, float(np.float32(1 / 8)))
