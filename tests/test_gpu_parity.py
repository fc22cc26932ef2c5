"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Sizes: the oracle runs the full definition where it finishes in seconds
(several tiles plus ragged tails); at the workloads' full sizes it checks
sampled outputs it can compute exactly (tail keys, or rows above a weight
floor with a stated bound) plus properties that hold at any size.
"""
import math
import sys

import numpy as np
import pytest
import torch

import attention_score_eviction_amd as W
from oracle import waits_oracle as orc
from synth import ACTIONS, make_batch, make_prompt

from parity import (DEV, check_compact, check_scores, check_select_exact,
                    check_select_vs_oracle, host_bits, to_device)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _run_all(bt, a, b, budget, scale=None):
    q, k, v = to_device(bt)
    cu = bt.cu_seqlens
    s, idx, kc, vc = W.score_select_compact(q, k, v, cu, a, b, budget, scale)
    torch.cuda.synchronize()
    return s.cpu().numpy(), idx.cpu().numpy(), kc, vc


def _full_check(bt, a, b, budget, scale=None, weight_floor=0.0):
    d = bt.head_dim
    scale = np.float32(1 / math.sqrt(d)) if scale is None else np.float32(scale)
    s_gpu, idx, kc, vc = _run_all(bt, a, b, budget, float(scale))
    s_ref = orc.waits_scores(bt.q, bt.k, bt.cu_seqlens, bt.n_q_heads, bt.n_kv_heads,
                             a, b, float(scale), weight_floor=weight_floor)
    err = check_scores(s_gpu, s_ref)
    check_select_exact(idx, s_gpu, bt.cu_seqlens, budget)
    check_select_vs_oracle(idx, s_ref, bt.cu_seqlens, budget)
    src_k = bt.k_bits if bt.dtype == "bf16" else bt.k
    src_v = bt.v_bits if bt.dtype == "bf16" else bt.v
    check_compact(kc, vc, src_k, src_v, idx, bt.cu_seqlens)
    return err


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    W.waits.lib()
    yield


# ------------------------------------------------------- the five configs ---

@pytest.mark.parametrize("a,b", [(1.0, 16), (0.0, 1), (0.0, 16), (math.inf, 1), (math.inf, 16)])
def test_tiny_fp32(a, b):
    # 1 layer, 1 query head, 1 KV head, d=64, N=512, fp32 N(0,1), budget 128
    _say(f"tiny fp32 a={a} b={b}")
    bt = make_prompt(0, 512, 1, 1, 64, heavy=False, dtype="f32")
    _full_check(bt, [a], [b], 128)


@pytest.fixture(scope="module")
def llama1b():
    return make_prompt(1, 4096, 32, 8, 64, heavy=True, dtype="bf16")


@pytest.mark.parametrize("a,b", list(ACTIONS))
def test_llama32_1b_layer(llama1b, a, b):
    # 32 query heads, 8 KV heads, d=64, N=4096, heavy hitters, budget 128
    _say(f"llama3.2-1b a={a} b={b}")
    _full_check(llama1b, [a], [b], 128)


def test_llama31_8b_layer_full_size():
    # one layer of the 8B shape at full size: 32/8/128, N=16384, a=1, b=16
    _say("llama3.1-8b layer N=16384")
    bt = make_prompt(1000, 16384, 32, 8, 128, heavy=True, dtype="bf16")
    # rows with w <= 1e-30 are left out of the oracle: |error| <= G*N*1e-30
    _full_check(bt, [1.0], [16], 128, weight_floor=1e-30)


def test_llama31_8b_layers_batched():
    # layers are independent sequences of one launch (reduced N)
    _say("8b-shape 3 layers N=2048 batched")
    bt = make_batch([1000, 1001, 1002], [2048, 2048, 2048], 32, 8, 128, heavy=True)
    _full_check(bt, [1.0] * 3, [16] * 3, 128)


@pytest.fixture(scope="module")
def long_prompt():
    return make_prompt(2, 131072, 32, 8, 128, heavy=True, dtype="bf16")


@pytest.mark.parametrize("a,b", [(math.inf, 16), (1.0, 16), (math.inf, 1), (1.0, 1), (1.0, 128),
                                 (math.inf, 128)])
def test_long_context_full_size(long_prompt, a, b):
    # one layer, N=131072, 32/8/128, budget 2048: the a in {1, inf} x b in
    # {1, 16, 128} sweep of this shape (a = 0 below).  The processed rows are
    # few (b at a = inf, about b + 70 at a = 1), so the oracle runs in full;
    # the sweep spans the 16-row kernel (1:1), the 512-row few-rows shape
    # (inf:128), the smallest shapes (inf:1, inf:16) and row blocks with key
    # blocks (1:128).
    _say(f"long N=131072 a={a} b={b}")
    _full_check(long_prompt, [a], [b], 2048, weight_floor=1e-30)


def test_long_context_h2o_sampled(long_prompt):
    # a=0 at N=131072: every row is live; the oracle checks the last 48 keys
    # exactly (they only see the last 48 rows) and the mass invariant holds
    # for every key
    _say("long N=131072 a=0 sampled")
    n = 131072
    bt = long_prompt
    s_gpu, idx, kc, vc = _run_all(bt, [0.0], [1], 2048)
    tail = n - 48
    s_ref = orc.waits_scores(bt.q, bt.k, bt.cu_seqlens, 32, 8, [0.0], [1],
                             float(np.float32(1 / math.sqrt(128))), row_min=[tail])
    check_scores(s_gpu[:, tail:], s_ref[:, tail:])
    # sum_k s[h, k] = G * sum_q w[q] = 4 * N / 2
    np.testing.assert_allclose(s_gpu.astype(np.float64).sum(axis=1), 2.0 * n, rtol=1e-4)
    check_select_exact(idx, s_gpu, bt.cu_seqlens, 2048)
    check_compact(kc, vc, bt.k_bits, bt.v_bits, idx, bt.cu_seqlens)


def test_row_block_and_key_block_pass2_in_one_launch():
    # a=0 everywhere: the 70000-token prompt's row-block partials (547 blocks x
    # 8 heads x 70000 keys, 1.2 GB) exceed the per-sequence cap, so its pass 2
    # runs on key blocks; the 1500-token prompt's runs on row blocks with a
    # block-order reduce.  Both share one launch group and one workspace.
    _say("pass 2 on key blocks and row blocks in one batch")
    lens = [70000, 1500]
    bt = make_batch([91, 92], lens, 32, 8, 128, heavy=True)
    s_gpu, idx, kc, vc = _run_all(bt, [0.0, 0.0], [1, 1], 256)
    cu = bt.cu_seqlens
    tail = lens[0] - 48
    s_ref = orc.waits_scores(bt.q, bt.k, cu, 32, 8, [0.0, 0.0], [1, 1],
                             float(np.float32(1 / math.sqrt(128))), row_min=[tail, 0])
    # the long prompt: exact on its last 48 keys (they see only the last 48
    # rows) and the mass invariant sum_k s[h, k] = G * N / 2 on every head
    check_scores(s_gpu[:, tail:lens[0]], s_ref[:, tail:lens[0]])
    np.testing.assert_allclose(s_gpu[:, :lens[0]].astype(np.float64).sum(axis=1), 2.0 * lens[0], rtol=1e-4)
    # the short prompt: every key
    check_scores(s_gpu[:, lens[0]:], s_ref[:, lens[0]:])
    check_select_exact(idx, s_gpu, cu, 256)
    check_compact(kc, vc, bt.k_bits, bt.v_bits, idx, cu)


@pytest.fixture(scope="module")
def longest_prompt():
    return make_prompt(9, (1 << 22) - 1, 1, 1, 64, heavy=True, dtype="bf16")


@pytest.mark.parametrize("a,b", [(math.inf, 16), (1.0, 16)])
def test_longest_accepted_sequence(longest_prompt, a, b):
    # N = 2^22 - 1, the longest sequence the boundary accepts (one head,
    # head_dim 64): key ranges cut over many workgroups and merged, chunk
    # buffer spans near their 2^31-byte bound, and the select over 4M keys in
    # 4096-key chunks; the processed rows are few, so the oracle runs in full
    _say(f"longest N=2^22-1 a={a} b={b}")
    _full_check(longest_prompt, [a], [b], 2048, weight_floor=1e-30)


def _mistral_batch(lo, hi, seed=3):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi, endpoint=True, size=8)
    acts = rng.integers(0, 5, size=8)
    bt = make_batch([3000 + i for i in range(8)], lengths, 32, 8, 128, heavy=True)
    a = [ACTIONS[j][0] for j in acts]
    b = [ACTIONS[j][1] for j in acts]
    return bt, a, b


def test_mistral_ragged_batch_reduced():
    # 8 prompts, ragged lengths, per-prompt (a, b) from the five actions,
    # budget 256, one launch; lengths cut to [300, 1500] so the oracle is exact
    _say("mistral ragged reduced")
    bt, a, b = _mistral_batch(300, 1500)
    _full_check(bt, a, b, 256)


def test_mistral_ragged_batch_full_size():
    # lengths in [8192, 32768]; tail keys exact, selection and gather exact
    _say("mistral ragged full size")
    bt, a, b = _mistral_batch(8192, 32768)
    s_gpu, idx, kc, vc = _run_all(bt, a, b, 256)
    cu = bt.cu_seqlens
    tails = [int(n) - 32 for n in bt.lengths]
    s_ref = orc.waits_scores(bt.q, bt.k, cu, 32, 8, a, b,
                             float(np.float32(1 / math.sqrt(128))), row_min=tails)
    mask = np.zeros(s_gpu.shape, dtype=bool)
    for p in range(8):
        mask[:, int(cu[p]) + tails[p]:int(cu[p + 1])] = True
    check_scores(s_gpu, s_ref, mask=mask)
    for p in range(8):
        w = orc.sigmoid_weights(int(bt.lengths[p]), a[p], b[p])
        got = s_gpu[:, int(cu[p]):int(cu[p + 1])].astype(np.float64).sum(axis=1)
        np.testing.assert_allclose(got, 4 * w.sum(), rtol=1e-4)
    check_select_exact(idx, s_gpu, cu, 256)
    check_compact(kc, vc, bt.k_bits, bt.v_bits, idx, cu)


# ------------------------------------------------------------ edge cases ---

@pytest.mark.parametrize("n", [1, 2, 31, 33, 63, 65, 129, 257, 300])
@pytest.mark.parametrize("hq,hkv,d", [(1, 1, 64), (2, 1, 128), (8, 1, 64), (16, 2, 128)])
def test_ragged_small_sizes(n, hq, hkv, d):
    _say(f"small n={n} hq={hq} hkv={hkv} d={d}")
    bt = make_prompt(n * 7 + hq, n, hq, hkv, d, heavy=True, dtype="bf16")
    for a, b in [(1.0, 16), (0.0, 1), (math.inf, 5), (10.0, 1)]:
        _full_check(bt, [a], [b], 64)


@pytest.mark.parametrize("scale", [0.05, 0.3])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_softmax_scale_other_than_default(scale, dtype):
    # the scale is an argument, not 1/sqrt(d) baked in: a flat (0.05) and a
    # sharp (0.3, logits in the tens) softmax, every regime of a small batch
    _say(f"scale {scale} {dtype}")
    bt = make_batch([91, 92], [2000, 700], 8, 2, 128, heavy=True, dtype=dtype)
    for a, b in [(1.0, 16), (0.0, 1), (math.inf, 40)]:
        _full_check(bt, [a, a], [b, b], 128, scale=scale)


@pytest.mark.parametrize("hq,hkv,d", [(3, 1, 64), (6, 2, 128), (10, 2, 64), (14, 2, 128)])
def test_group_sizes_not_powers_of_two(hq, hkv, d):
    # G = 3, 3, 5, 7: packed rows interleave the G query heads of a position,
    # so row tiles, row blocks and key-block row stages start mid-position;
    # a = 1 runs the few-rows shapes, a = 0 row blocks and key blocks, a = inf
    # with b = 40 the few-rows shapes at 120..280 packed rows
    _say(f"group sizes hq={hq} hkv={hkv} d={d}")
    bt = make_batch([81 + hq, 82 + hq], [3000, 1500], hq, hkv, d, heavy=True)
    for a, b in [(1.0, 16), (0.0, 1), (math.inf, 40)]:
        _full_check(bt, [a, a], [b, b], 128)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("a,b", [(math.inf, 65), (math.inf, 96), (math.inf, 97), (1.0, 16),
                                 (math.inf, 112), (math.inf, 113), (math.inf, 128)])
def test_mid_size_heads_split_keys(d, a, b):
    # G = 4 and a = inf keep the last b rows: 4 b packed rows per KV head, here
    # 260..512: the 16-row-tile shapes (partly filled and full, up to 448 rows)
    # and the 32-row shape just past them; a = 1, b = 16 keeps about 105 rows.  N = 6000 cuts each head's keys into chunks
    # that the combine merges.
    _say(f"mid-size heads d={d} a={a} b={b}")
    bt = make_prompt(60 + b + d, 6000, 8, 2, d, heavy=True, dtype="bf16")
    _full_check(bt, [a], [b], 256)
    bt = make_batch([70, 71, 72], [700, 6000, 2500], 8, 2, d, heavy=True)
    _full_check(bt, [a, 0.0, a], [b, 1, b], 256)


def test_batch_with_empty_and_tiny_sequences():
    _say("batch with empty sequences")
    bt = make_batch([5, 6, 7, 8, 9], [0, 1, 700, 0, 45], 8, 2, 64, heavy=True)
    a, b = [1.0, 0.0, 0.01, 1.0, math.inf], [16, 1, 128, 4, 3]
    _full_check(bt, a, b, 40)


def test_b_larger_than_n_and_budget_at_least_n():
    _say("b > N, budget >= N")
    bt = make_prompt(11, 200, 4, 2, 64, heavy=True)
    _full_check(bt, [0.5], [1000], 256)
    _full_check(bt, [math.inf], [32768], 200)


def test_many_sequences_span_launch_groups():
    # more sequences than one launch's table holds
    _say("40 sequences")
    lens = [int(x) for x in np.random.default_rng(4).integers(1, 200, size=40)]
    bt = make_batch(list(range(100, 140)), lens, 4, 2, 64, heavy=True)
    acts = [ACTIONS[i % 5] for i in range(40)]
    _full_check(bt, [x[0] for x in acts], [x[1] for x in acts], 16)


def test_all_tied_scores_keep_lowest_positions():
    # Q = 0 and a = inf, b = 1: the last row is uniform, every score is 1/N
    _say("all tied")
    n = 1000
    q = torch.zeros((n, 4, 64), dtype=torch.bfloat16, device=DEV)
    k = torch.randn((n, 1, 64), device=DEV).to(torch.bfloat16)
    s = W.score(q, k, [0, n], [math.inf], [1])
    sc = s.cpu().numpy()
    assert np.all(sc == sc[0, 0])
    np.testing.assert_allclose(sc, 4.0 / n, rtol=1e-5)
    idx = W.select(s, [0, n], 128).cpu().numpy()
    assert idx[0, 0].tolist() == list(range(128))


def test_uniform_attention_closed_form_on_gpu():
    # Q = 0 at a = 0: s[k] = (G/2)(H_N - H_k) (harmonic numbers)
    _say("uniform closed form")
    n, g = 777, 4
    q = torch.zeros((n, g, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.randn((n, 1, 128), device=DEV).to(torch.bfloat16)
    s = W.score(q, k, [0, n], [0.0], [1]).cpu().numpy()[0].astype(np.float64)
    harm = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    np.testing.assert_allclose(s, g / 2 * (harm[n] - harm[:n]), rtol=2e-5)


@pytest.mark.parametrize("a,b", [(1.0, 16), (0.0, 1)])
def test_head_major_strides_match_token_major(a, b):
    # a=1: one workgroup holds all rows; a=0: row blocks and key blocks
    _say(f"head-major strides a={a}")
    bt = make_prompt(21, 999, 8, 2, 128, heavy=True)
    q, k, v = to_device(bt)
    qh = q.permute(1, 0, 2).contiguous().permute(1, 0, 2)   # [T, H, d] view of [H, T, d]
    kh = k.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    assert qh.stride(0) == 128 and kh.stride(1) == 999 * 128
    s1 = W.score(q, k, bt.cu_seqlens, [a], [b])
    s2 = W.score(qh, kh, bt.cu_seqlens, [a], [b])
    assert torch.equal(s1, s2)


@pytest.mark.parametrize("a,b", [(1.0, 16), (0.0, 1), (math.inf, 40)])
def test_packed_qkv_views_match_separate_tensors(a, b):
    # a model's fused projection: one [T, Hq + 2 Hkv, d] buffer, Q, K and V as
    # views into it (token stride (Hq + 2 Hkv) d); scores, kept positions
    # and the compacted cache equal those of separate contiguous tensors
    _say(f"packed qkv a={a} b={b}")
    bt = make_batch([23, 24], [1700, 600], 8, 2, 128, heavy=True)
    q, k, v = to_device(bt)
    qkv = torch.cat([q, k, v], dim=1).contiguous()
    qv, kv_, vv = qkv[:, :8], qkv[:, 8:10], qkv[:, 10:12]
    assert qv.stride(0) == 12 * 128 and kv_.stride() == vv.stride()
    r1 = W.score_select_compact(q, k, v, bt.cu_seqlens, [a, a], [b, b], 128)
    r2 = W.score_select_compact(qv, kv_, vv, bt.cu_seqlens, [a, a], [b, b], 128)
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("a,b", [(1.0, 16), (0.0, 1), (0.01, 128)])
def test_fp32_head_dim_128(a, b):
    # fp32 rows of 512 bytes take the row-group / key-group kernels
    _say(f"fp32 d=128 a={a} b={b}")
    bt = make_batch([41, 42], [700, 1500], 4, 2, 128, heavy=True, dtype="f32")
    _full_check(bt, [a, a], [b, b], 128)


def test_deterministic_and_causal_support():
    # bitwise reproducible; perturbing query rows < k0 leaves scores of keys
    # >= k0 bitwise unchanged (rows only reach keys at or before them)
    _say("determinism + causal support")
    bt = make_prompt(31, 3000, 16, 4, 64, heavy=True)
    q, k, _ = to_device(bt)
    s1 = W.score(q, k, bt.cu_seqlens, [0.002], [64])
    s2 = W.score(q, k, bt.cu_seqlens, [0.002], [64])
    assert torch.equal(s1, s2)
    k0 = 1234
    q2 = q.clone()
    q2[:k0] = torch.randn_like(q2[:k0], dtype=torch.float32).to(torch.bfloat16)
    s3 = W.score(q2, k, bt.cu_seqlens, [0.002], [64])
    assert torch.equal(s1[:, k0:], s3[:, k0:])
    assert not torch.equal(s1[:, :k0], s3[:, :k0])


def test_lse_matches_oracle_on_processed_rows():
    _say("lse parity")
    bt = make_batch([41, 42], [1500, 600], 8, 2, 128, heavy=True)
    q, k, _ = to_device(bt)
    a, b = [1.0, 0.0], [16, 1]
    first = W.waits.first_rows(bt.cu_seqlens, a, b)
    out = torch.full((8, bt.total_tokens), float("nan"), device=DEV)
    W.lse(q, k, bt.cu_seqlens, a, b, out=out)
    got = out.cpu().numpy()
    rows = [np.arange(int(f), int(n)) for f, n in zip(first, bt.lengths)]
    ref = orc.waits_lse(bt.q, bt.k, bt.cu_seqlens, 8, 2, float(np.float32(1 / math.sqrt(128))),
                        rows_per_prompt=rows)
    done = ~np.isnan(ref)
    assert np.array_equal(~np.isnan(got), done)   # exactly the processed rows are written
    np.testing.assert_allclose(got[done], ref[done], rtol=0, atol=2e-5 * np.abs(ref[done]).max())


# ------------------------------------------------------- select / compact ---

@pytest.mark.parametrize("n,budget", [(5000, 128), (20000, 256), (131072, 2048), (70, 128)])
def test_select_on_arbitrary_scores(n, budget):
    _say(f"select n={n}")
    rng = np.random.default_rng(n)
    s = rng.random((3, n)).astype(np.float32)
    s[:, rng.integers(0, n, n // 3)] = np.float32(0.75)   # many exact ties
    s[1] = np.float32(0.5)                                 # a head of all ties
    s[2, :n // 2] = 0.0
    idx = W.select(torch.from_numpy(s).to(DEV), [0, n], budget).cpu().numpy()
    for h in range(3):
        np.testing.assert_array_equal(idx[0, h], orc.select_topk(s[h].astype(np.float64), budget))


@pytest.mark.parametrize("n", [1, 63, 64, 1023, 1024, 1025, 16384, 16385, 32768, 32769, 65600])
def test_select_segment_boundaries(n):
    # key counts around the per-wave segment sizes and the register-cache limits
    _say(f"select boundaries n={n}")
    rng = np.random.default_rng(1000 + n)
    s = (rng.random((2, n)) ** 6).astype(np.float32)
    s[1, rng.integers(0, n, max(1, n // 4))] = np.float32(0.25)
    for budget in (1, 128, min(n, 3000)):
        idx = W.select(torch.from_numpy(s).to(DEV), [0, n], budget).cpu().numpy()
        for h in range(2):
            np.testing.assert_array_equal(idx[0, h], orc.select_topk(s[h].astype(np.float64), budget))


@pytest.mark.parametrize("n", [129, 1000, 5000, 16383, 20001, 32767])
def test_select_threshold_zero(n):
    # fewer positive scores than the budget: the kept zeros are the
    # lowest-positioned ones (the kernel's slots past N also read as 0 and
    # must never be kept); one head all zeros, one with 40 positives
    _say(f"select threshold 0 n={n}")
    rng = np.random.default_rng(2000 + n)
    s = np.zeros((2, n), dtype=np.float32)
    s[1, rng.choice(n, 40, replace=False)] = rng.random(40).astype(np.float32) + np.float32(0.5)
    sd = torch.from_numpy(s).to(DEV)
    idx = W.select(sd, [0, n], 128).cpu().numpy()
    for h in range(2):
        np.testing.assert_array_equal(idx[0, h], orc.select_topk(s[h].astype(np.float64), 128))
    assert idx[0, 0].tolist() == list(range(128))
    # the fused gather keeps the same rows, bit for bit
    k = torch.randn((n, 2, 64), device=DEV).to(torch.bfloat16)
    v = torch.randn((n, 2, 64), device=DEV).to(torch.bfloat16)
    idx2, kc, vc = W.select_compact(sd, k, v, [0, n], 128)
    assert np.array_equal(idx2.cpu().numpy(), idx)
    for h in range(2):
        rows = torch.from_numpy(idx[0, h].astype(np.int64)).to(DEV)
        assert torch.equal(kc[0, h].view(torch.int16), k[rows, h].view(torch.int16))
        assert torch.equal(vc[0, h].view(torch.int16), v[rows, h].view(torch.int16))


@pytest.mark.parametrize("lengths,budget", [([3000, 17000, 40, 0, 33000], 256), ([5000, 9000], 10000),
                                            ([700] * 40, 64), ([128, 127, 129], 128)])
def test_select_compact_fused_matches_separate(lengths, budget):
    # one launch (select + gather) against waits_select then waits_compact, bit for bit
    _say(f"fused select+compact lengths={lengths[:5]} budget={budget}")
    bt = make_batch(list(range(60, 60 + len(lengths))), lengths, 4, 2, 128, heavy=True, values=True)
    _, k, v = to_device(bt)
    rng = np.random.default_rng(7)
    T = int(bt.cu_seqlens[-1])
    s = torch.from_numpy((rng.random((2, T)) ** 4).astype(np.float32)).to(DEV)
    idx1 = W.select(s, bt.cu_seqlens, budget)
    kc1, vc1 = W.compact(k, v, idx1, bt.cu_seqlens, budget)
    idx2, kc2, vc2 = W.select_compact(s, k, v, bt.cu_seqlens, budget)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16))
    check_compact(kc2, vc2, bt.k_bits, bt.v_bits, idx2.cpu().numpy(), bt.cu_seqlens)


def test_compact_with_padding_slots():
    _say("compact padding")
    bt = make_batch([51, 52], [10, 300], 4, 2, 128, heavy=True)
    _, k, v = to_device(bt)
    idx = np.full((2, 2, 16), -1, dtype=np.int32)
    idx[0, :, :10] = np.arange(10)
    idx[1, 0] = np.sort(np.random.default_rng(0).choice(300, 16, replace=False))
    idx[1, 1, :5] = [0, 1, 2, 298, 299]
    kc, vc = W.compact(k, v, torch.from_numpy(idx).to(DEV), bt.cu_seqlens, 16)
    check_compact(kc, vc, bt.k_bits, bt.v_bits, idx, bt.cu_seqlens)
