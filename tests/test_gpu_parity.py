"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Sizes: the oracle runs the full definition where it finishes in seconds
(several tiles plus ragged tails).  At the workloads' full sizes it runs in
full where the processed rows are few (rows above a weight floor with a
stated bound), and elsewhere on whole KV heads, computed in worker processes
(tests/oracle_pool.py), plus properties that hold at any size.
"""
import math
import sys

import numpy as np
import pytest
import torch

import attention_score_eviction_amd as W
from oracle import waits_oracle as orc
from synth import ACTIONS, make_batch, make_prompt

import oracle_pool
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


def _full_check(bt, a, b, budget, scale=None, weight_floor=0.0, s_ref=None):
    d = bt.head_dim
    scale = np.float32(1 / math.sqrt(d)) if scale is None else np.float32(scale)
    s_gpu, idx, kc, vc = _run_all(bt, a, b, budget, float(scale))
    if s_ref is None:
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


@pytest.fixture(scope="module")
def llama1b_refs(llama1b):
    """The oracle's scores of the 1B prompt, per action, computed once."""
    scale = float(np.float32(1 / math.sqrt(64)))
    refs = {}

    def ref(a, b):
        if (a, b) not in refs:
            refs[(a, b)] = orc.waits_scores(llama1b.q, llama1b.k, llama1b.cu_seqlens, 32, 8, [a], [b], scale)
        return refs[(a, b)]
    return ref


@pytest.mark.parametrize("a,b", list(ACTIONS))
def test_llama32_1b_layer(llama1b, llama1b_refs, a, b):
    # 32 query heads, 8 KV heads, d=64, N=4096, heavy hitters, budget 128
    _say(f"llama3.2-1b a={a} b={b}")
    _full_check(llama1b, [a], [b], 128, s_ref=llama1b_refs(a, b))


@pytest.mark.timeout(300)
def test_1b_batch_as_benchmarked(llama1b, llama1b_refs):
    # bench.py's 1b step, with its buffers and calls: the five actions as five
    # sequences of one batch, all on the 1B prompt.  The batch mixes the
    # few-rows workgroup shapes (row blocks at a = 0 and a = 0.01, the 16-row
    # kernel at a = 1, the 2- and 4-wave shapes at a = 10), whose launches run
    # side by side on separate streams.  Every key of every sequence against
    # the oracle; a second step gives the same bits.
    import bench
    _say("1b batch as benchmarked: five actions x 4096")
    wl = bench.workload("1b")
    assert [(a, b) for a, b in zip(wl["a"], wl["b"])] == list(ACTIONS)
    q, k, v, cu = bench.make_inputs(wl, DEV)
    bufs = bench.step_buffers(wl, q, k, cu)
    calls = bench.step_calls(wl, q, k, v, cu, bufs)
    outs = []
    for _ in range(2):
        for call in calls:
            call()
        torch.cuda.synchronize()
        outs.append({n: bufs[n].cpu() for n in ("lse", "scores", "idx", "kc", "vc")})
    for n in outs[0]:
        assert torch.equal(outs[0][n], outs[1][n]), f"{n} differs between two steps"
    s_gpu = outs[0]["scores"].numpy()
    idx = outs[0]["idx"].numpy()
    check_select_exact(idx, s_gpu, cu, wl["budget"])
    for p, (a, b) in enumerate(ACTIONS):
        lo, hi = int(cu[p]), int(cu[p + 1])
        s_ref = llama1b_refs(a, b)
        err = check_scores(s_gpu[:, lo:hi], s_ref)
        check_select_vs_oracle(idx[p:p + 1], s_ref, llama1b.cu_seqlens, wl["budget"])
        check_compact(bufs["kc"][p:p + 1], bufs["vc"][p:p + 1], llama1b.k_bits, llama1b.v_bits,
                      idx[p:p + 1], llama1b.cu_seqlens)
        _say(f"  a={a} b={b}: every key within {err:.2e}")


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


@pytest.mark.timeout(600)
def test_headline_batch_as_benchmarked():
    # bench.py's default step, with its buffers and calls: 32 layers x
    # N=16384 in one batch (a = 1, b = 16, budget 128).  Every KV head has 420
    # packed rows, and the batch gives one workgroup per head, so both passes
    # run whole key ranges in the 16-row-tile kernel: pass 1 writes lse
    # directly (no key split, no combine, no pass-1 workspace).  The first
    # and the last layer against the oracle in full; selection on every layer.
    import bench
    _say("headline batch as benchmarked: 32 x 16384")
    wl = bench.workload("8b")
    q, k, v, cu = bench.make_inputs(wl, DEV)
    assert W.waits.lse_workspace_bytes(q, k, cu, wl["a"], wl["b"]) == 0
    bufs = bench.step_buffers(wl, q, k, cu)
    for call in bench.step_calls(wl, q, k, v, cu, bufs):
        call()
    torch.cuda.synchronize()
    s_gpu = bufs["scores"].cpu().numpy()
    idx = bufs["idx"].cpu().numpy()
    check_select_exact(idx, s_gpu, cu, wl["budget"])
    scale = float(np.float32(1 / math.sqrt(128)))
    for layer in (0, 31):
        bt = make_prompt(wl["seeds"][layer], 16384, 32, 8, 128, heavy=True, dtype="bf16")
        lo, hi = int(cu[layer]), int(cu[layer + 1])
        # rows with w <= 1e-30 are left out of the oracle: |error| <= G*N*1e-30
        s_ref = orc.waits_scores(bt.q, bt.k, bt.cu_seqlens, 32, 8, [1.0], [16], scale,
                                 weight_floor=1e-30)
        err = check_scores(s_gpu[:, lo:hi], s_ref)
        check_select_vs_oracle(idx[layer:layer + 1], s_ref, bt.cu_seqlens, wl["budget"])
        check_compact(bufs["kc"][layer:layer + 1], bufs["vc"][layer:layer + 1], bt.k_bits, bt.v_bits,
                      idx[layer:layer + 1], bt.cu_seqlens)
        _say(f"  layer {layer}: every key within {err:.2e}")


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


def _check_full_heads(s_gpu, idx, bt, p, heads, a, b, budget, pool, weight_floor=0.0):
    """Every key of the given KV heads of prompt p against the oracle (the
    per-key bar), and those heads' kept sets (the index-set rule)."""
    lo, hi = int(bt.cu_seqlens[p]), int(bt.cu_seqlens[p + 1])
    g = bt.n_q_heads // bt.n_kv_heads
    scale = float(np.float32(1 / math.sqrt(bt.head_dim)))
    for h in heads:
        ref = oracle_pool.kv_head_scores(bt.q[lo:hi], bt.k[lo:hi], h, g, a, b, scale,
                                         weight_floor=weight_floor, pool=pool)
        err = check_scores(s_gpu[h, lo:hi], ref)
        check_select_vs_oracle(idx[p:p + 1, h:h + 1], ref[None], [0, hi - lo], budget)
        _say(f"  prompt {p} head {h}: every key within {err:.2e}")


H2O_HEADS = (0, 5)


@pytest.fixture(scope="module")
def long_h2o_ref(long_prompt):
    """Oracle scores of two whole KV heads of the long prompt at a = 0."""
    bt = long_prompt
    scale = float(np.float32(1 / math.sqrt(128)))
    with oracle_pool.make_pool() as pool:
        return {h: oracle_pool.kv_head_scores(bt.q, bt.k, h, 4, 0.0, 1, scale, pool=pool)
                for h in H2O_HEADS}


def _check_h2o_heads(s_gpu, idx, ref, lo, n, budget, what):
    for h, r in ref.items():
        err = check_scores(s_gpu[h, lo:lo + n], r)
        check_select_vs_oracle(idx[:, h:h + 1], r[None], [0, n], budget)
        _say(f"  {what} head {h}: every key within {err:.2e}")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("plan", ["auto", "key_blocks"])
def test_long_context_h2o_full_heads(long_prompt, long_h2o_ref, plan):
    # a=0 at N=131072 (the H2O limit): every row is live; pass 2 runs on row
    # blocks (4 GiB of per-block partials) in the automatic plan, on key
    # blocks in the key-block plan.  Two whole KV heads against the oracle,
    # key by key, with their kept sets; on every head the last 48 keys (they
    # see only the last 48 rows) and the mass invariant
    _say(f"long N=131072 a=0, plan {plan}, two full KV heads")
    n = 131072
    bt = long_prompt
    q, k, v = to_device(bt)
    s = W.score(q, k, bt.cu_seqlens, [0.0], [1], pass2=plan)
    idx, kc, vc = W.select_compact(s, k, v, bt.cu_seqlens, 2048)
    torch.cuda.synchronize()
    s_gpu, idx = s.cpu().numpy(), idx.cpu().numpy()
    _check_h2o_heads(s_gpu, idx, long_h2o_ref, 0, n, 2048, plan)
    tail = n - 48
    s_ref = orc.waits_scores(bt.q, bt.k, bt.cu_seqlens, 32, 8, [0.0], [1],
                             float(np.float32(1 / math.sqrt(128))), row_min=[tail])
    check_scores(s_gpu[:, tail:], s_ref[:, tail:])
    # sum_k s[h, k] = G * sum_q w[q] = 4 * N / 2
    np.testing.assert_allclose(s_gpu.astype(np.float64).sum(axis=1), 2.0 * n, rtol=1e-4)
    check_select_exact(idx, s_gpu, bt.cu_seqlens, 2048)
    check_compact(kc, vc, bt.k_bits, bt.v_bits, idx, bt.cu_seqlens)


@pytest.mark.timeout(900)
def test_row_block_and_key_block_pass2_in_one_launch(long_prompt, long_h2o_ref):
    # the long prompt twice in one batch at a = 0: the first sequence's
    # row-block partials (4 GiB) fit the automatic plan's 6 GiB per launch
    # group, the second's would pass it, so the second runs pass 2 on key
    # blocks in the same launch group and workspace.  Both copies against the
    # oracle on two whole KV heads, and against each other on every key.
    _say("pass 2 on row blocks and key blocks in one batch: the long prompt twice")
    n = 131072
    bt = long_prompt
    q1, k1, v1 = to_device(bt)
    q, k, v = (torch.cat([x, x]) for x in (q1, k1, v1))
    del q1, k1, v1
    cu = np.array([0, n, 2 * n], dtype=np.int64)
    ws = W.waits.colsum_workspace_bytes(q, k, cu, [0.0, 0.0], [1, 1])
    rb_one = 1024 * 8 * n * 4          # one copy's row-block partials: 1024 blocks x 8 heads x N
    assert rb_one <= ws < 2 * rb_one   # the other copy's key-block chunks are far smaller
    s = W.score(q, k, cu, [0.0, 0.0], [1, 1])
    idx, kc, vc = W.select_compact(s, k, v, cu, 2048)
    torch.cuda.synchronize()
    s_gpu, idx = s.cpu().numpy(), idx.cpu().numpy()
    for p in range(2):
        _check_h2o_heads(s_gpu, idx[p:p + 1], long_h2o_ref, p * n, n, 2048, f"copy {p}")
    # the same sums in two orders: equal to fp32 rounding
    np.testing.assert_allclose(s_gpu[:, n:], s_gpu[:, :n], rtol=2e-5, atol=0)
    check_select_exact(idx, s_gpu, cu, 2048)
    kb = np.concatenate([bt.k_bits, bt.k_bits])
    vb = np.concatenate([bt.v_bits, bt.v_bits])
    check_compact(kc, vc, kb, vb, idx, cu)


@pytest.mark.parametrize("hq,hkv,d,dtype", [(12, 4, 128, "bf16"), (6, 2, 64, "bf16"),
                                             (3, 1, 128, "bf16"), (14, 2, 64, "bf16"),
                                             (7, 1, 128, "bf16"), (8, 2, 64, "f32")])
def test_key_block_plan_full_definition(hq, hkv, d, dtype):
    # pass 2 forced onto key blocks (the plan the longest a = 0 prompts take)
    # at sizes the oracle finishes: G in {3, 4, 7}, head_dim 64 and 128, bf16
    # and fp32; every row live (a = 0, a = 0.01) or about 1800 of 3000 (a =
    # 0.05), so each KV head has 4K..21K packed rows cut into row chunks,
    # whose partial sums colsum_reduce_kernel adds in chunk order
    _say(f"key-block plan hq={hq} hkv={hkv} d={d} {dtype}")
    bt = make_batch([41 + hq, 42 + hq], [3000, 1500], hq, hkv, d, heavy=True, dtype=dtype)
    q, k, _ = to_device(bt)
    cu = bt.cu_seqlens
    for a, b in [(0.0, 1), (0.01, 128), (0.05, 16)]:
        assert W.waits.colsum_workspace_bytes(q, k, cu, [a, a], [b, b], pass2="key_blocks") > 0
        scale = float(np.float32(1 / math.sqrt(d)))
        s = W.score(q, k, cu, [a, a], [b, b], pass2="key_blocks").cpu().numpy()
        s_ref = orc.waits_scores(bt.q, bt.k, cu, hq, hkv, [a, a], [b, b], scale)
        check_scores(s, s_ref)
        # the automatic plan (row blocks here) computes the same sums in
        # another order: equal to fp32 rounding
        s_auto = W.score(q, k, cu, [a, a], [b, b]).cpu().numpy()
        np.testing.assert_allclose(s, s_auto, rtol=2e-5, atol=0)
        idx = W.select(torch.from_numpy(s).to(DEV), cu, 128).cpu().numpy()
        check_select_exact(idx, s, cu, 128)
        check_select_vs_oracle(idx, s_ref, cu, 128)


def test_key_block_plan_one_row_chunk_per_block():
    # enough key blocks over the batch (8 KV heads x 256 blocks) that every
    # block's rows form one chunk: the kernel writes the scores directly and
    # the plan needs no workspace.  G = 1; about 590 processed rows per head
    # (a = 0.15), so the oracle runs every key of every head.
    n, h, d = 131072, 8, 64
    _say(f"key-block plan, one row chunk per block, N={n}")
    bt = make_prompt(57, n, h, h, d, heavy=True, dtype="bf16")
    q, k, _ = to_device(bt)
    cu = bt.cu_seqlens
    a, b = [0.15], [1]
    assert 512 < n - int(W.waits.first_rows(cu, a, b)[0]) <= 1024
    assert W.waits.colsum_workspace_bytes(q, k, cu, a, b, pass2="key_blocks") == 0
    s = W.score(q, k, cu, a, b, pass2="key_blocks").cpu().numpy()
    s_ref = orc.waits_scores(bt.q, bt.k, cu, h, h, a, b, float(np.float32(1 / math.sqrt(d))))
    check_scores(s, s_ref)
    idx = W.select(torch.from_numpy(s).to(DEV), cu, 2048).cpu().numpy()
    check_select_exact(idx, s, cu, 2048)
    check_select_vs_oracle(idx, s_ref, cu, 2048)


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


@pytest.mark.timeout(900)
def test_mistral_ragged_batch_full_size():
    # lengths in [8192, 32768], one launch; two whole KV heads of every
    # prompt key by key with their kept sets, the tail keys of every head,
    # the mass invariant, and the selection and gather exactly
    _say("mistral ragged full size")
    bt, a, b = _mistral_batch(8192, 32768)
    s_gpu, idx, kc, vc = _run_all(bt, a, b, 256)
    cu = bt.cu_seqlens
    with oracle_pool.make_pool() as pool:
        for p in range(8):
            _check_full_heads(s_gpu, idx, bt, p, [p % 8, (p + 4) % 8], a[p], b[p], 256, pool)
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


@pytest.mark.parametrize("d", [64, 128])
def test_every_workgroup_shape_in_one_batch(d):
    # packed rows per KV head (G = 4): a = 0 -> 12000 (row blocks), a = 10
    # with b = 1 / 16 / 40 -> 40 / 100 / 196 (the 2-, 4- and 8-wave one-tile
    # shapes), a = 1 with b = 16 / 1 -> 420 / 360 (the 16-row-tile bodies with
    # 4 and 3 tiles per wave), a = inf with b = 128 -> 512 (the two-tile
    # shape).  Each pass runs all of them in one launch; at head_dim 64 pass
    # 1's 256-row blocks share a segment with the 196-row heads.
    lengths = [3000, 1800, 2200, 2500, 2600, 2100, 1900]
    a = [0.0, 10.0, 10.0, 10.0, 1.0, 1.0, math.inf]
    b = [1, 1, 16, 40, 16, 1, 128]
    _say(f"every shape in one batch d={d}")
    bt = make_batch([140 + i for i in range(len(lengths))], lengths, 8, 2, d, heavy=True)
    first = W.waits.first_rows(bt.cu_seqlens, a, b)
    assert [4 * (n - int(f)) for n, f in zip(lengths, first)] == [12000, 40, 100, 196, 420, 360, 512]
    _full_check(bt, a, b, 128)


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
    # so row tiles and row blocks start mid-position; a = 1 runs the few-rows
    # shapes, a = 0 row blocks for both passes (key blocks: the key-block
    # plan test), a = inf with b = 40 the few-rows shapes at 120..280 packed rows
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


@pytest.mark.parametrize("a,b,plan", [(1.0, 16, "auto"), (0.0, 1, "auto"), (0.0, 1, "key_blocks")])
def test_head_major_strides_match_token_major(a, b, plan):
    # a=1: one workgroup holds all rows; a=0: pass 2 on row blocks (the
    # automatic plan) or on key blocks, whose row stages address the G heads
    # of a group from one base
    _say(f"head-major strides a={a} plan {plan}")
    bt = make_prompt(21, 999, 8, 2, 128, heavy=True)
    q, k, v = to_device(bt)
    qh = q.permute(1, 0, 2).contiguous().permute(1, 0, 2)   # [T, H, d] view of [H, T, d]
    kh = k.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    assert qh.stride(0) == 128 and kh.stride(1) == 999 * 128
    s1 = W.score(q, k, bt.cu_seqlens, [a], [b], pass2=plan)
    s2 = W.score(qh, kh, bt.cu_seqlens, [a], [b], pass2=plan)
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


@pytest.mark.parametrize("n", [1, 63, 64, 1023, 1024, 1025, 4096, 4097, 8192, 8193, 16384, 16385, 32768, 32769, 65600])
def test_select_segment_boundaries(n):
    # key counts around the per-wave segment sizes and the register-cache limits
    # (4, 8, 16 and 32 slots per lane up to 4096, 8192, 16384 and 32768 keys)
    _say(f"select boundaries n={n}")
    rng = np.random.default_rng(1000 + n)
    s = (rng.random((2, n)) ** 6).astype(np.float32)
    s[1, rng.integers(0, n, max(1, n // 4))] = np.float32(0.25)
    for budget in (1, 128, min(n, 3000)):
        idx = W.select(torch.from_numpy(s).to(DEV), [0, n], budget).cpu().numpy()
        for h in range(2):
            np.testing.assert_array_equal(idx[0, h], orc.select_topk(s[h].astype(np.float64), budget))


@pytest.mark.parametrize("n", [129, 1000, 5000, 16383, 20001, 32767, 40001, 70000])
def test_select_threshold_zero(n):
    # fewer positive scores than the budget: the kept zeros are the
    # lowest-positioned ones (the kernel's slots past N also read as 0 and
    # must never be kept); one head all zeros, one with 40 positives.  Past
    # 32768 keys the select runs over several workgroups, where the kept
    # zeros come from the first chunk and the positives from any
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


@pytest.mark.parametrize("n,budget", [(300000, 2048), (70000, 4000)])
def test_wide_select_long_heads_and_crowded_chunks(n, budget):
    # heads past 64 chunks of 4096 keys (300000 keys: the bin offsets are read
    # again rather than held in LDS), and scores falling with position as at
    # a = 0, so the first chunk keeps almost every kept row (4000 of its
    # 4096: the fused gather runs several trips in one workgroup); kept
    # positions against the oracle's top-k, rows bit for bit
    _say(f"wide select n={n} budget={budget}")
    rng = np.random.default_rng(3000 + n)
    s = np.empty((2, n), dtype=np.float32)
    s[0] = (rng.random(n) ** 3).astype(np.float32)
    s[1] = (1.0 / (1.0 + np.arange(n) / 8.0)).astype(np.float32) * np.float32(1 + 0.01 * rng.random())
    s[1, rng.integers(0, n, n // 100)] *= np.float32(3.0)
    sd = torch.from_numpy(s).to(DEV)
    k = torch.randn((n, 2, 64), device=DEV).to(torch.bfloat16)
    v = torch.randn((n, 2, 64), device=DEV).to(torch.bfloat16)
    idx, kc, vc = W.select_compact(sd, k, v, [0, n], budget)
    got = idx.cpu().numpy()
    for h in range(2):
        np.testing.assert_array_equal(got[0, h], orc.select_topk(s[h].astype(np.float64), budget))
        rows = torch.from_numpy(got[0, h].astype(np.int64)).to(DEV)
        assert torch.equal(kc[0, h].view(torch.int16), k[rows, h].view(torch.int16))
        assert torch.equal(vc[0, h].view(torch.int16), v[rows, h].view(torch.int16))
    if n == 70000:
        assert int((got[0, 1] < 4096).sum()) > 3500   # the first chunk keeps most rows


def test_wide_select_ignores_workspace_contents():
    # the several-workgroup select reads only workspace words it wrote in the
    # same call: a workspace full of 0xff bytes, or one left by a call on
    # other inputs, gives the same kept positions and rows bit for bit
    _say("wide select, workspace contents")
    rng = np.random.default_rng(77)
    lengths = [40000, 131072, 0, 33000]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1])
    s = (rng.random((2, T)) ** 5).astype(np.float32)
    s[:, rng.integers(0, T, T // 7)] = np.float32(0.5)
    sd = torch.from_numpy(s).to(DEV)
    k = torch.randn((T, 2, 64), device=DEV).to(torch.bfloat16)
    v = torch.randn((T, 2, 64), device=DEV).to(torch.bfloat16)
    budget = 1500
    nbytes = W.waits.select_workspace_bytes(cu, 2, budget)
    assert nbytes > 0
    want = W.select_compact(sd, k, v, cu, budget, workspace=torch.zeros(nbytes, dtype=torch.uint8, device=DEV))
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
    got1 = W.select_compact(sd, k, v, cu, budget, workspace=ws)
    other = torch.from_numpy((rng.random((2, T)) ** 2).astype(np.float32)).to(DEV)
    W.select_compact(other, k, v, cu, budget, workspace=ws)          # leaves its own records behind
    got2 = W.select_compact(sd, k, v, cu, budget, workspace=ws)
    torch.cuda.synchronize()
    for got in (got1, got2):
        assert torch.equal(got[0], want[0])
        assert torch.equal(got[1].view(torch.int16), want[1].view(torch.int16))
        assert torch.equal(got[2].view(torch.int16), want[2].view(torch.int16))
    for p_ in range(len(lengths)):
        lo, hi = int(cu[p_]), int(cu[p_ + 1])
        for h in range(2):
            np.testing.assert_array_equal(want[0][p_, h].cpu().numpy(),
                                          orc.select_topk(s[h, lo:hi].astype(np.float64), budget))


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
