"""GPU: waits_select_compact_noalloc, the select+compact call that takes its
scratch from the library's static per-GPU array instead of a workspace,
against waits_select_compact with a caller workspace: kept positions and
compacted K/V bit for bit, on calls in a row whose inputs shrink (the
static array keeps the earlier call's contents), through the C ABI."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import attention_score_eviction_amd as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def _inputs(seed, lengths, hkv, d):
    """Scores with many exact ties, and K/V rows, for a packed batch."""
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    s = (rng.random((hkv, T)) ** 4).astype(np.float32)
    s[:, rng.integers(0, T, max(1, T // 5))] = np.float32(0.125)
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((T, hkv, d), generator=g).to(torch.bfloat16)
    v = torch.randn((T, hkv, d), generator=g).to(torch.bfloat16)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return torch.from_numpy(s).to(DEV), k.to(DEV), v.to(DEV), cu


def _outputs(nb, hkv, budget, d):
    return (torch.full((nb, hkv, budget), -7, dtype=torch.int32, device=DEV),
            torch.full((nb, hkv, budget, d), 3.0, dtype=torch.bfloat16, device=DEV),
            torch.full((nb, hkv, budget, d), -3.0, dtype=torch.bfloat16, device=DEV))


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    W.waits.lib()
    yield


def test_noalloc_matches_workspace_call_on_shrinking_inputs():
    cases = [  # (seed, lengths, KV heads, head_dim, budget)
        (1, [40000, 131072, 700], 8, 128, 2048),   # several-workgroup select: scratch in use
        (2, [33000, 5000], 2, 64, 256),            # smaller: less scratch, earlier contents left
        (3, [3000, 17000, 40, 0], 4, 128, 128),    # short heads only: no scratch
        (4, [32769], 1, 128, 9000),                # budget past the fused gather: select, then compact
    ]
    for seed, lengths, hkv, d, budget in cases:
        _say(f"noalloc vs workspace: lengths {lengths} hkv {hkv} d {d} budget {budget}")
        s, k, v, cu = _inputs(seed, lengths, hkv, d)
        nb = len(lengths)
        want = W.select_compact(s, k, v, cu, budget)
        idx, kc, vc = _outputs(nb, hkv, budget, d)
        W.waits.select_compact_noalloc(s, k, v, cu, budget, idx, kc, vc)
        torch.cuda.synchronize()
        assert torch.equal(idx, want[0])
        assert torch.equal(kc.view(torch.int16), want[1].view(torch.int16))
        assert torch.equal(vc.view(torch.int16), want[2].view(torch.int16))
