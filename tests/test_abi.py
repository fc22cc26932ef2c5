"""C ABI checks that need no GPU: the library loads, exports every entry
point include/waits.h declares, and rejects bad arguments on the host
before enqueuing anything (no call here reaches a kernel launch)."""
import ctypes
import math
import subprocess

import numpy as np
import pytest
import torch

from attention_score_eviction_amd import waits as W

FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: every call below fails validation


def _shape(batch=1, n=64, hq=4, hkv=2, d=64, dtype=W.WAITS_BF16, scale=0.125, cu=None):
    cu = np.ascontiguousarray(np.asarray(cu if cu is not None else [0, n], np.int64))
    s = W.WaitsShape()
    s.batch = batch if cu is None else len(cu) - 1
    s.cu_seqlens = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    s.n_q_heads, s.n_kv_heads, s.head_dim, s.dtype = hq, hkv, d, dtype
    s.q_stride_tok, s.q_stride_head = hq * d, d
    s.kv_stride_tok, s.kv_stride_head = hkv * d, d
    s.scale = scale
    s._keep = cu
    return s


def _ab(a=1.0, b=16, n=1):
    return (np.full(n, a, np.float32), np.full(n, b, np.int32))


def _score(shape, a, b, ws_bytes=1 << 30, ws=FAKE):
    return W.lib().waits_score(ctypes.byref(shape), FAKE, FAKE, a.ctypes.data_as(W._FP),
                               b.ctypes.data_as(W._IP), FAKE, ws, ws_bytes, None)


def test_library_exports_every_declared_symbol():
    declared = W.header_symbols()
    assert len(declared) >= 9
    out = subprocess.run(["nm", "-D", "--defined-only", W.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in declared:
        assert name in exported, name
        assert getattr(W.lib(), name) is not None


def test_strerror_codes():
    assert W.strerror(0) == "ok"
    for code in (1, 2, 3, 4):
        assert W.strerror(code) and W.strerror(code) != "ok"
    assert "unknown" in W.strerror(99)


@pytest.mark.parametrize("field,value,code", [
    ("n_q_heads", 3, W.WAITS_EINVAL),        # not a multiple of n_kv_heads
    ("n_kv_heads", 0, W.WAITS_EINVAL),
    ("head_dim", 96, W.WAITS_EUNSUPPORTED),
    ("head_dim", 0, W.WAITS_EINVAL),
    ("dtype", 7, W.WAITS_EINVAL),
    ("scale", float("nan"), W.WAITS_EINVAL),
    ("scale", 0.0, W.WAITS_EINVAL),
    ("scale", float("inf"), W.WAITS_EINVAL),
    ("q_stride_tok", 3, W.WAITS_EINVAL),      # row start not 16-byte aligned
    ("kv_stride_head", -64, W.WAITS_EINVAL),
])
def test_shape_validation(field, value, code):
    s = _shape()
    setattr(s, field, value)
    a, b = _ab()
    assert _score(s, a, b) == code


@pytest.mark.parametrize("a,b", [(float("nan"), 16), (-1.0, 16), (1.0, 0), (1.0, -3),
                                 (1.0, (1 << 22) + 1)])
def test_curve_validation(a, b):
    s = _shape()
    aa, bb = np.array([a], np.float32), np.array([b], np.int32)
    assert _score(s, aa, bb) == W.WAITS_EINVAL
    out = ctypes.c_size_t(0)
    assert W.lib().waits_score_workspace_bytes(ctypes.byref(s), aa.ctypes.data_as(W._FP),
                                               bb.ctypes.data_as(W._IP),
                                               ctypes.byref(out)) == W.WAITS_EINVAL


def test_cu_seqlens_validation():
    a, b = _ab(n=2)
    assert _score(_shape(cu=[1, 5, 9]), a, b) == W.WAITS_EINVAL      # must start at 0
    assert _score(_shape(cu=[0, 9, 5]), a, b) == W.WAITS_EINVAL      # descending
    assert _score(_shape(cu=[0, 1 << 22, (1 << 22) + 1]), a, b) == W.WAITS_EINVAL  # too long


def test_null_pointers_and_workspace():
    s = _shape()
    a, b = _ab()
    assert W.lib().waits_score(ctypes.byref(s), None, FAKE, a.ctypes.data_as(W._FP),
                               b.ctypes.data_as(W._IP), FAKE, FAKE, 1 << 30, None) == W.WAITS_EINVAL
    assert W.lib().waits_score(None, FAKE, FAKE, a.ctypes.data_as(W._FP),
                               b.ctypes.data_as(W._IP), FAKE, FAKE, 1 << 30, None) == W.WAITS_EINVAL
    need = ctypes.c_size_t(0)
    assert W.lib().waits_score_workspace_bytes(ctypes.byref(s), a.ctypes.data_as(W._FP),
                                               b.ctypes.data_as(W._IP), ctypes.byref(need)) == 0
    assert need.value >= 4 * 64 * 4
    assert _score(s, a, b, ws_bytes=need.value - 1) == W.WAITS_EWORKSPACE
    assert _score(s, a, b, ws=None) == W.WAITS_EWORKSPACE
    assert _score(s, a, b, ws=ctypes.c_void_p(0x100010)) == W.WAITS_EWORKSPACE  # not 256-aligned
    assert W.lib().waits_score(ctypes.byref(s), ctypes.c_void_p(0x100002), FAKE,
                               a.ctypes.data_as(W._FP), b.ctypes.data_as(W._IP), FAKE, FAKE,
                               1 << 30, None) == W.WAITS_EINVAL   # misaligned Q


def test_select_and_compact_validation():
    s = _shape()
    lib = W.lib()
    assert lib.waits_select(ctypes.byref(s), FAKE, 0, FAKE, None, 0, None) == W.WAITS_EINVAL
    assert lib.waits_select(ctypes.byref(s), FAKE, 128, None, None, 0, None) == W.WAITS_EINVAL
    assert lib.waits_select(ctypes.byref(_shape(cu=[0, -1])), FAKE, 8, FAKE, None, 0,
                            None) == W.WAITS_EINVAL
    assert lib.waits_compact(ctypes.byref(s), FAKE, FAKE, FAKE, 0, FAKE, FAKE, None) == W.WAITS_EINVAL
    assert lib.waits_compact(ctypes.byref(s), FAKE, FAKE, FAKE, 8, None, FAKE, None) == W.WAITS_EINVAL
    bad = _shape(d=80)
    assert lib.waits_compact(ctypes.byref(bad), FAKE, FAKE, FAKE, 8, FAKE, FAKE,
                             None) == W.WAITS_EUNSUPPORTED


@pytest.mark.parametrize("n,a,b", [(4096, 1.0, 16), (16384, 1.0, 16), (16384, 10.0, 1),
                                   (16384, 10.0, 16), (4096, 0.01, 128), (32768, 0.01, 128),
                                   (131072, 1.0, 128), (100, 3.5, 200), (1, 10.0, 1),
                                   (513, 0.0, 1), (2000, math.inf, 16), (2000, math.inf, 5000)])
def test_first_rows_skip_only_zero_weight_rows(n, a, b):
    q0 = int(W.first_rows([0, n], [a], [b])[0])
    a32 = np.float32(a)
    c = np.float32(n) - np.float32(b) - np.float32(0.5)
    with np.errstate(over="ignore", invalid="ignore"):
        x = a32 * (c - np.arange(n, dtype=np.float32))      # fp32, as on the device
        w = np.float32(1) / (np.float32(1) + np.exp(x))      # fp32 weight
    # every skipped row overflows expf (ln FLT_MAX = 88.7228...) -> weight exactly 0
    assert np.all(x[:q0] > np.float32(88.7229))
    assert np.all(w[:q0] == 0)
    # and the range is tight: the first processed row is within the 89 margin
    assert q0 == 0 or x[q0] <= np.float32(89.0)
    assert q0 <= n - 1


def test_first_rows_match_survey_live_counts():
    # fp32 live-row counts for N = 16384 at the README's five actions
    n = 16384
    got = {ab: n - int(W.first_rows([0, n], [ab[0]], [ab[1]])[0])
           for ab in [(0.0, 1), (1.0, 16), (10.0, 1), (10.0, 16), (math.inf, 16)]}
    assert got == {(0.0, 1): n, (1.0, 16): 105, (10.0, 1): 10, (10.0, 16): 25,
                   (math.inf, 16): 16}


def test_workspace_sizes():
    q = torch.empty((4096, 32, 64), dtype=torch.bfloat16)
    k = torch.empty((4096, 8, 64), dtype=torch.bfloat16)
    # 105 live rows (one workgroup per KV head): key range split into chunks
    # with (max, sum) partials; pass 2 writes its scores directly
    assert W.lse_workspace_bytes(q, k, [0, 4096], [1.0], [16]) > 0
    assert W.colsum_workspace_bytes(q, k, [0, 4096], [1.0], [16]) == 0
    # all rows live, one short sequence: too few row blocks for the chip, so
    # pass 1 splits keys and pass 2 writes one partial column sum per row
    # block ([row block][Hkv][N] fp32)
    lse_ws = W.lse_workspace_bytes(q, k, [0, 4096], [0.0], [1])
    col_ws = W.colsum_workspace_bytes(q, k, [0, 4096], [0.0], [1])
    assert lse_ws > 0 and col_ws == 32 * 8 * 4096 * 4
    assert (W.score_workspace_bytes(q, k, [0, 4096], [0.0], [1])
            >= 32 * 4096 * 4 + max(lse_ws, col_ws))


def test_select_workspace():
    # one workgroup per (sequence, head) up to 32768 keys: no workspace
    assert W.select_workspace_bytes([0, 32768], 8, 128) == 0
    assert W.select_workspace_bytes([0, 0], 8, 128) == 0
    # longer: 4096-key chunks, each with its counting-sort record: 65 coarse
    # offsets (u32, padded to 272 bytes), 4097 bin offsets (u16, padded to
    # 4104) and 4096 order keys (u32)
    need = W.select_workspace_bytes([0, 131072, 131072 + 5000], 8, 2048)
    assert need == 8 * (32 + 2) * (272 + 2 * 4104 + 4 * 4096)
    s = _shape(cu=[0, 40000], hkv=2)
    lib = W.lib()
    assert lib.waits_select(ctypes.byref(s), FAKE, 64, FAKE, None, 0, None) == W.WAITS_EWORKSPACE
    assert lib.waits_select(ctypes.byref(s), FAKE, 64, FAKE, ctypes.c_void_p(0x100008), 1 << 20,
                            None) == W.WAITS_EWORKSPACE   # not 16-byte aligned


def test_colsum_workspace_validation():
    s = _shape(n=4096, hq=32, hkv=8)
    a, b = _ab(a=0.0, b=1)
    need = ctypes.c_size_t(0)
    assert W.lib().waits_colsum_workspace_bytes(ctypes.byref(s), a.ctypes.data_as(W._FP),
                                                b.ctypes.data_as(W._IP), ctypes.byref(need)) == 0
    assert need.value > 0

    def colsum(ws, nbytes):
        return W.lib().waits_colsum(ctypes.byref(s), FAKE, FAKE, FAKE, a.ctypes.data_as(W._FP),
                                    b.ctypes.data_as(W._IP), FAKE, ws, nbytes, None)
    assert colsum(None, 0) == W.WAITS_EWORKSPACE
    assert colsum(FAKE, need.value - 1) == W.WAITS_EWORKSPACE
    assert colsum(ctypes.c_void_p(0x100002), need.value) == W.WAITS_EWORKSPACE  # misaligned


def test_lse_workspace_validation():
    # a = 0 at N = 4096 on 32/8 heads: pass 1 splits keys, so it needs room
    # for its (max, sum) partials, 8-byte aligned
    s = _shape(n=4096, hq=32, hkv=8)
    a, b = _ab(a=0.0, b=1)
    need = ctypes.c_size_t(0)
    assert W.lib().waits_lse_workspace_bytes(ctypes.byref(s), a.ctypes.data_as(W._FP),
                                             b.ctypes.data_as(W._IP), ctypes.byref(need)) == 0
    if need.value == 0:
        pytest.skip("this plan splits no keys")

    def lse(ws, nbytes):
        return W.lib().waits_lse(ctypes.byref(s), FAKE, FAKE, a.ctypes.data_as(W._FP),
                                 b.ctypes.data_as(W._IP), FAKE, ws, nbytes, None)
    assert lse(None, need.value) == W.WAITS_EWORKSPACE
    assert lse(FAKE, need.value - 1) == W.WAITS_EWORKSPACE
    assert lse(ctypes.c_void_p(0x100004), need.value) == W.WAITS_EWORKSPACE  # not 8-byte aligned


def test_pass2_plan_validation_and_workspace():
    # the plan field is checked by every call that takes Q
    s = _shape(n=4096, hq=32, hkv=8)
    a, b = _ab(a=0.0, b=1)
    s.pass2 = 2
    assert _score(s, a, b) == W.WAITS_EINVAL
    need = ctypes.c_size_t(0)
    assert W.lib().waits_colsum_workspace_bytes(ctypes.byref(s), a.ctypes.data_as(W._FP),
                                                b.ctypes.data_as(W._IP),
                                                ctypes.byref(need)) == W.WAITS_EINVAL
    # all rows live at N = 4096: the automatic plan reuses pass 1's 512-row
    # blocks ([row block][Hkv][N] partials); the key-block plan cuts each
    # 512-key block's rows into chunks ([chunk][Hkv][T] partials)
    q = torch.empty((4096, 32, 64), dtype=torch.bfloat16)
    k = torch.empty((4096, 8, 64), dtype=torch.bfloat16)
    auto = W.colsum_workspace_bytes(q, k, [0, 4096], [0.0], [1])
    kb = W.colsum_workspace_bytes(q, k, [0, 4096], [0.0], [1], pass2="key_blocks")
    assert auto == (4 * 4096 // 512) * 8 * 4096 * 4
    assert kb > 0 and kb % (8 * 4096 * 4) == 0
    # pass 1 does not depend on the pass-2 plan
    assert (W.lse_workspace_bytes(q, k, [0, 4096], [0.0], [1])
            == W.lse_workspace_bytes(q, k, [0, 4096], [0.0], [1], pass2="key_blocks"))
    # few rows per KV head: one workgroup holds them all, no partials either way
    assert W.colsum_workspace_bytes(q, k, [0, 4096], [1.0], [16], pass2="key_blocks") == 0
    with pytest.raises(ValueError):
        W.colsum_workspace_bytes(q, k, [0, 4096], [0.0], [1], pass2="rows")


def test_head_major_group_span_only_limits_key_blocks():
    # head-major Q of a 2^20-token prompt: one token's rows of a 4-head group
    # span 3 T d + d elements (> 2^29 bytes), which only the key-block kernel
    # addresses from one buffer base.  About 200 processed rows per query
    # head (800 packed rows per KV head) run pass 2 on row blocks in the
    # automatic plan, so the call gets as far as the workspace check; the
    # key-block plan refuses the layout.  No call here reaches a launch.
    n, hq, d = 1 << 20, 4, 128
    s = _shape(n=n, hq=hq, hkv=1, d=d)
    s.q_stride_tok, s.q_stride_head = d, n * d
    s.kv_stride_tok, s.kv_stride_head = d, n * d
    a, b = _ab(a=89.0 / 200, b=1)
    q0 = int(W.first_rows([0, n], a, b)[0])
    assert 512 < hq * (n - q0) <= 1024

    def colsum(plan):
        s.pass2 = plan
        return W.lib().waits_colsum(ctypes.byref(s), FAKE, FAKE, FAKE, a.ctypes.data_as(W._FP),
                                    b.ctypes.data_as(W._IP), FAKE, None, 0, None)
    assert colsum(W.WAITS_PASS2_AUTO) == W.WAITS_EWORKSPACE
    assert colsum(W.WAITS_PASS2_KEY_BLOCKS) == W.WAITS_EUNSUPPORTED


def test_binding_raises_without_library(monkeypatch):
    monkeypatch.setattr(W, "_lib", None)
    monkeypatch.setattr(W, "LIB_PATH", W.LIB_PATH + ".missing")
    with pytest.raises(RuntimeError, match="missing"):
        W.lib()


# ------------------------------------------------------------------ decode ---

def _dshape(batch=2, hq=8, hkv=2, d=128, dtype=W.WAITS_BF16, cap=128, scale=0.088):
    s = W.WaitsDecodeShape()
    s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim = batch, hq, hkv, d
    s.dtype, s.capacity, s.scale = dtype, cap, scale
    return s


def _decode(s, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, out=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return W.lib().waits_decode(ctypes.byref(s) if s is not None else None, q, k, v, lens, out, lse,
                                ws, ws_bytes, None)


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, W.WAITS_EINVAL),
    ("n_q_heads", 3, W.WAITS_EINVAL),         # not a multiple of n_kv_heads
    ("n_kv_heads", 0, W.WAITS_EINVAL),
    ("head_dim", 96, W.WAITS_EUNSUPPORTED),
    ("dtype", 5, W.WAITS_EINVAL),
    ("capacity", 0, W.WAITS_EINVAL),
    ("capacity", (1 << 20) + 1, W.WAITS_EUNSUPPORTED),
    ("scale", float("nan"), W.WAITS_EINVAL),
    ("scale", -1.0, W.WAITS_EINVAL),
])
def test_decode_shape_validation(field, value, code):
    s = _dshape()
    setattr(s, field, value)
    assert _decode(s) == code
    n = ctypes.c_size_t(0)
    assert W.lib().waits_decode_workspace_bytes(ctypes.byref(s), ctypes.byref(n)) == code


def test_decode_pointer_and_workspace_validation():
    s = _dshape()
    assert _decode(None) == W.WAITS_EINVAL
    for kw in ("q", "k", "v", "lens", "out"):
        assert _decode(s, **{kw: None}) == W.WAITS_EINVAL, kw
    assert _decode(s, q=ctypes.c_void_p(0x100008)) == W.WAITS_EINVAL    # q not 16-byte aligned
    assert _decode(s, v=ctypes.c_void_p(0x100004)) == W.WAITS_EINVAL    # cache not 16-byte aligned
    assert _decode(s, out=ctypes.c_void_p(0x100002)) == W.WAITS_EINVAL  # out not 4-byte aligned
    # a long cache over few sequences is split: the partials need room
    big = _dshape(batch=1, hkv=1, hq=4, cap=65536)
    n = ctypes.c_size_t(0)
    assert W.lib().waits_decode_workspace_bytes(ctypes.byref(big), ctypes.byref(n)) == W.WAITS_OK
    assert n.value > 0
    assert _decode(big, ws_bytes=n.value - 1) == W.WAITS_EWORKSPACE
    assert _decode(big, ws=None) == W.WAITS_EWORKSPACE
    assert _decode(big, ws=ctypes.c_void_p(0x100008)) == W.WAITS_EWORKSPACE  # not 16-byte aligned


@pytest.mark.parametrize("batch,hq,hkv,cap,expect_zero", [
    (32, 32, 8, 128, True),      # a 128-row cache is one split (no combine)
    (256, 32, 8, 128, True),     # many sequences: one item per (sequence, head)
    (4, 32, 8, 1024, False),     # few sequences, longer caches: split for parallelism
    (1, 32, 8, 2048, False),
    (64, 32, 8, 2048, False),
])
def test_decode_workspace_sizes(batch, hq, hkv, cap, expect_zero):
    s = _dshape(batch=batch, hq=hq, hkv=hkv, cap=cap)
    n = ctypes.c_size_t(0)
    assert W.lib().waits_decode_workspace_bytes(ctypes.byref(s), ctypes.byref(n)) == W.WAITS_OK
    assert (n.value == 0) == expect_zero
    if n.value:
        # at least two splits' (max, sum) and head_dim vector per (sequence, query head)
        assert n.value >= batch * hq * 2 * (8 + 4 * 128)


def test_decode_binding_checks_layouts():
    q = torch.zeros((2, 8, 64), dtype=torch.bfloat16)
    kc = torch.zeros((2, 2, 16, 64), dtype=torch.bfloat16)
    lens = torch.full((2,), 16, dtype=torch.int32)
    with pytest.raises(ValueError):
        W.decode(q, kc.transpose(2, 3), kc, lens)                 # not dense
    with pytest.raises(ValueError):
        W.decode(q, kc, kc, lens.to(torch.int64))                 # lens dtype
    with pytest.raises(TypeError):
        W.decode(q.float(), kc, kc, lens)                         # mixed dtypes
    with pytest.raises(ValueError):
        W.decode(q[:, :, :32].contiguous(), kc, kc, lens)         # head_dim mismatch


def test_noalloc_select_compact_rejects_batches_beyond_its_scratch():
    # 32 sequences x 32 KV heads of 80000 keys: 20 chunks per head of 1040
    # bytes each (21 MB) pass the 16 MiB static scratch; refused before any launch
    lib = W.lib()
    assert "scratch" in W.strerror(W.WAITS_ESCRATCH)
    s = _shape(cu=[80000 * i for i in range(33)], hkv=32, hq=32)
    need = ctypes.c_size_t(0)
    assert lib.waits_select_workspace_bytes(ctypes.byref(s), 256, ctypes.byref(need)) == 0
    assert need.value > W.STATIC_SCRATCH_BYTES
    assert lib.waits_select_compact_noalloc(ctypes.byref(s), FAKE, FAKE, FAKE, 256, FAKE, FAKE, FAKE,
                                            None) == W.WAITS_ESCRATCH
    # argument checks come first, as in waits_select_compact
    assert lib.waits_select_compact_noalloc(ctypes.byref(s), FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE,
                                            None) == W.WAITS_EINVAL
