"""GPU: the path captured into HIP graphs, as bench.py replays it, gives on
every replay bit for bit what eager library calls give.

Each test captures its calls once, then replays the graph several times.
Between replays the program runs its own eager work (another eager pass
into separate buffers) and synchronises.  Before each replay the graph's
output buffers are poisoned, so a replay that skipped a kernel shows up.
The batches cover every launch shape of a step: few-rows passes with their
lse combine, row-block pass 1 with pass 2 on the same row blocks and their
block-order reduce (the automatic plan) or on key blocks with the row-chunk
reduce (the key-block plan), and the select+compact of short heads (one
launch) and of heads of more than 32768 keys (several launches).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import attention_score_eviction_amd as W
from synth import make_batch, make_decode

from parity import DEV, to_device

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _say(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    W.waits.lib()
    yield


def _capture(fn):
    """Warm fn on a side stream, then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, graph_bufs, eager_bufs, poison, eager_again):
    for rep in range(REPLAYS):
        for name, t in graph_bufs.items():
            poison(name, t)
        eager_again()                   # the program's own eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in graph_bufs.items():
            assert torch.equal(t, eager_bufs[name]), f"replay {rep}: {name} differs from the eager result"


@pytest.mark.parametrize("plan", ["auto", "key_blocks"])
def test_graph_replays_match_eager_scores_select_compact(plan):
    lengths = [3000, 40000, 700, 1, 5000]
    a = [1.0, math.inf, 0.0, 1.0, 0.01]
    b = [16, 16, 1, 1, 128]
    hq, hkv, d, budget = 8, 2, 128, 256
    _say(f"graph: score + select + compact, pass-2 plan {plan}, lengths {lengths}")
    bt = make_batch([61 + i for i in range(len(lengths))], lengths, hq, hkv, d, heavy=True)
    q, k, v = to_device(bt)
    cu = bt.cu_seqlens
    T, nb = int(cu[-1]), len(lengths)
    ws = torch.empty(max(W.waits.lse_workspace_bytes(q, k, cu, a, b),
                         W.waits.colsum_workspace_bytes(q, k, cu, a, b, pass2=plan), 256),
                     dtype=torch.uint8, device=DEV)
    sel_ws = torch.empty(max(W.waits.select_workspace_bytes(cu, hkv, budget), 256), dtype=torch.uint8,
                         device=DEV)

    def bufs():
        return {"lse": torch.zeros((hq, T), device=DEV),
                "scores": torch.empty((hkv, T), device=DEV),
                "idx": torch.empty((nb, hkv, budget), dtype=torch.int32, device=DEV),
                "k_out": torch.empty((nb, hkv, budget, d), dtype=torch.bfloat16, device=DEV),
                "v_out": torch.empty((nb, hkv, budget, d), dtype=torch.bfloat16, device=DEV)}

    def run(bf):
        W.lse(q, k, cu, a, b, out=bf["lse"], workspace=ws)
        W.colsum(q, k, bf["lse"], cu, a, b, out=bf["scores"], workspace=ws, pass2=plan)
        W.select_compact(bf["scores"], k, v, cu, budget, idx=bf["idx"], k_out=bf["k_out"], v_out=bf["v_out"],
                         workspace=sel_ws)

    eager, other, graph = bufs(), bufs(), bufs()
    run(eager)
    torch.cuda.synchronize()
    g = _capture(lambda: run(graph))

    def poison(name, t):
        if name == "lse":
            t.zero_()                   # rows pass 1 does not process stay 0, as in the eager buffer
        elif name == "idx":
            t.fill_(-7)
        else:
            t.fill_(-1.0)

    _replay_and_check(g, graph, eager, poison, lambda: run(other))
    # the eager pass between replays agrees too
    for name in eager:
        assert torch.equal(other[name], eager[name]), name


def test_graph_replays_match_eager_attention():
    lengths = [700, 257, 2000]
    hq, hkv, d = 8, 2, 128
    _say(f"graph: attention forward, lengths {lengths}")
    bt = make_batch([71, 72, 73], lengths, hq, hkv, d, heavy=True)
    q, k, v = to_device(bt)
    cu = bt.cu_seqlens
    T = int(cu[-1])

    def bufs():
        return {"out": torch.empty_like(q), "lse": torch.empty((hq, T), device=DEV)}

    def run(bf):
        W.attention(q, k, v, cu, out=bf["out"], lse=bf["lse"])

    eager, other, graph = bufs(), bufs(), bufs()
    run(eager)
    torch.cuda.synchronize()
    g = _capture(lambda: run(graph))
    _replay_and_check(g, graph, eager, lambda name, t: t.fill_(-1.0), lambda: run(other))


def test_graph_replays_match_eager_decode():
    bsz, hq, hkv, d, cap = 16, 32, 8, 128, 4097
    _say(f"graph: decode, {bsz} sequences, capacity {cap}")
    x = make_decode(81, bsz, hq, hkv, cap, d, "bf16")
    q, k, v = (torch.from_numpy(np.ascontiguousarray(t)).view(torch.bfloat16).to(DEV)
               for t in (x.q_bits, x.k_bits, x.v_bits))
    lens = torch.tensor([cap, 1, 0, 2048] + [cap - 7 * i for i in range(bsz - 4)], dtype=torch.int32,
                        device=DEV)
    ws = torch.empty(max(W.waits.decode_workspace_bytes(q, k), 256), dtype=torch.uint8, device=DEV)

    def bufs():
        return {"out": torch.empty((bsz, hq, d), device=DEV), "lse": torch.empty((bsz, hq), device=DEV)}

    def run(bf):
        W.decode(q, k, v, lens, out=bf["out"], lse=bf["lse"], workspace=ws)

    eager, other, graph = bufs(), bufs(), bufs()
    run(eager)
    torch.cuda.synchronize()
    g = _capture(lambda: run(graph))
    _replay_and_check(g, graph, eager, lambda name, t: t.fill_(7.0), lambda: run(other))
