"""Benchmark of the WAITS prefill KV-selection path on one MI355X.

One step = the whole path (pass-1 row log-sum-exp, pass-2 weighted column
sums, top-k select, K/V compaction) over one batch of synthetic inputs that
are already resident in HBM.  Default workload: the Llama-3.1-8B layer shape
(32 query heads, 8 KV heads, head_dim 128), 32 independently generated
layers of N = 16384 prompt tokens, a = 1, b = 16, select_budget = 128, bf16.

Prints one JSON line: prompt tokens/s per layer (= layers x tokens / step
time), the dominant kernel's roofline fraction (per-kernel times from HIP
events on the stream the library launches on), and the CPU oracle timed on
a bounded sample of the same workload.

Each stage of a step (pass 1, pass 2, select+compact) is one library call
per step; ``--graph`` instead captures each stage once into a HIP graph and
replays it (the library is capture-safe: no allocation, memset or host sync
inside its calls).  On ROCm 7.2 a replay costs about 1 us more per kernel node
than direct launches, so the default is direct calls.

    python bench.py [--steps K] [--warmup W] [--graph]
                    [--workload 8b|1b|long|long_snap|long_tova|long_a<A>_b<B>|mistral|decode|fused]

``long_a<A>_b<B>`` is one point of the long-context sweep (N = 131072, A in
{0, 1, inf}, B in {1, 16, 128}; ``long_a0`` stands for every B); ``long``,
``long_snap`` and ``long_tova`` are a=1 b=16, a=inf b=16 and a=inf b=1.

``--workload decode`` measures the step after the path instead: one decoding
step's attention over the compacted cache (64 sequences of the Llama-3.1-8B
shape, 2048 kept rows each), against the HBM roofline.

``--workload fused`` runs the headline batch the way a model's attention call
would: the prefill attention forward writes out and the row lse, and the
WAITS scores take that lse (pass 2 only), then select+compact.  The line
reports the attention kernel against the MFMA roofline, the WAITS marginal
cost (pass 2 + select/compact) and pass 1's time, which the fusion saves.
"""
from __future__ import annotations

import argparse
import contextlib
import gc
import json
import math
import os
import platform
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synth import ACTIONS, make_batch, make_decode, make_prompt  # noqa: E402

METRIC = "prompt tokens/s per layer for WAITS score+select+compact; % bf16 MFMA peak"
UNIT = "tokens/s/layer"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


# The long-context sweep a in {0, 1, inf} x b in {1, 16, 128} at N = 131072:
# at a = 0 every weight is 1/2 whatever b is, so one run stands for all three.
LONG_SWEEP = {f"long_a{'inf' if a == math.inf else int(a)}_b{b}": (a, b)
              for a in (1.0, math.inf) for b in (1, 16, 128)}
LONG_SWEEP["long_a0"] = (0.0, 1)
WORKLOADS = ["8b", "1b", "long", "long_snap", "long_tova", *sorted(LONG_SWEEP), "mistral", "decode", "fused"]


def workload(name: str):
    """(description, heads, d, lengths, seeds, a, b, budget)."""
    if name == "8b":
        L, n = 32, 16384
        return dict(desc="Llama-3.1-8B layer shape, 32 layers x N=16384, a=1 b=16, budget 128",
                    hq=32, hkv=8, d=128, lengths=[n] * L, seeds=[1000 + i for i in range(L)],
                    a=[1.0] * L, b=[16] * L, budget=128, layers=L)
    if name == "1b":
        return dict(desc="Llama-3.2-1B layer shape, N=4096, five actions as five sequences, budget 128",
                    hq=32, hkv=8, d=64, lengths=[4096] * 5, seeds=[1] * 5,
                    a=[x[0] for x in ACTIONS], b=[x[1] for x in ACTIONS], budget=128, layers=5)
    long_alias = {"long": "long_a1_b16", "long_snap": "long_ainf_b16", "long_tova": "long_ainf_b1"}
    name = long_alias.get(name, name)
    if name in LONG_SWEEP:
        a, b = LONG_SWEEP[name]
        limit = {0.0: " (H2O limit: w = 1/2 for every row, the same computation for every b)",
                 math.inf: " (TOVA limit)" if b == 1 else " (SnapKV limit)"}.get(a, "")
        return dict(desc=f"Llama-3.1-8B layer shape, one layer N=131072, a={a:g} b={b}{limit}, budget 2048",
                    hq=32, hkv=8, d=128, lengths=[131072], seeds=[2], a=[a], b=[b],
                    budget=2048, layers=1)
    if name == "mistral":
        rng = np.random.default_rng(3)
        lengths = [int(x) for x in rng.integers(8192, 32768, endpoint=True, size=8)]
        acts = rng.integers(0, 5, size=8)
        return dict(desc="Mistral-7B shape, 8 ragged prompts in [8192, 32768], per-prompt actions, budget 256",
                    hq=32, hkv=8, d=128, lengths=lengths, seeds=[3000 + i for i in range(8)],
                    a=[ACTIONS[j][0] for j in acts], b=[ACTIONS[j][1] for j in acts],
                    budget=256, layers=1)
    raise SystemExit(f"unknown workload {name!r}")


def live_rows_fp32(n: int, a: float, b: int) -> np.ndarray:
    """Rows whose fp32 forgetting-curve weight is nonzero (the work the
    method must do; rows with weight exactly 0 add nothing)."""
    a32 = np.float32(a)
    c = np.float32(n) - np.float32(b) - np.float32(0.5)
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.float32(1) / (np.float32(1) + np.exp(a32 * (c - np.arange(n, dtype=np.float32))))
    return np.nonzero(w != 0)[0]


def algorithmic_work(wl):
    """Per-launch algorithmic flops and bytes of one QK^T pass, and bytes of
    select/compact.  Pass bytes: K read once, the live Q rows, lse (pass 1
    writes it, pass 2 reads it); pass 2 also writes the scores."""
    flops_pass, live = 0.0, 0
    for n, a, b in zip(wl["lengths"], wl["a"], wl["b"]):
        rows = live_rows_fp32(n, a, b)
        flops_pass += 2.0 * wl["d"] * wl["hq"] * float(np.sum(rows + 1))
        live += len(rows)
    hkv, hq, d, budget, B = wl["hkv"], wl["hq"], wl["d"], wl["budget"], len(wl["lengths"])
    T = sum(wl["lengths"])
    bytes_pass = hkv * T * d * 2 + hq * live * d * 2 + hq * live * 4
    select_bytes = hkv * T * 4 + B * hkv * budget * 4
    compact_bytes = 2 * 2 * B * hkv * budget * d * 2 + B * hkv * budget * 4
    return flops_pass, bytes_pass, select_bytes, compact_bytes


def make_inputs(wl, device):
    import torch

    hq, hkv, d = wl["hq"], wl["hkv"], wl["d"]
    T = sum(wl["lengths"])
    q = torch.empty((T, hq, d), dtype=torch.bfloat16, device=device)
    k = torch.empty((T, hkv, d), dtype=torch.bfloat16, device=device)
    v = torch.empty((T, hkv, d), dtype=torch.bfloat16, device=device)
    cu = np.zeros(len(wl["lengths"]) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(wl["lengths"])

    def one(i):
        return i, make_prompt(wl["seeds"][i], wl["lengths"][i], hq, hkv, d,
                              heavy=True, dtype="bf16", values=False)

    workers = min(16, len(wl["lengths"]), os.cpu_count() or 1)
    with ThreadPoolExecutor(workers) as ex:
        for i, bt in ex.map(one, range(len(wl["lengths"]))):
            lo, hi = int(cu[i]), int(cu[i + 1])
            for dst, src in ((q, bt.q_bits), (k, bt.k_bits), (v, bt.v_bits)):
                dst[lo:hi].copy_(torch.from_numpy(src).view(torch.bfloat16))
    return q, k, v, cu


def _host_info():
    """(BLAS threads, BLAS description, CPU model) of this host."""
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([x.get("num_threads", 1) for x in info] or [1])
        blas = ",".join(sorted({f"{x.get('internal_api', '?')}x{x.get('num_threads', '?')}"
                                for x in info}))
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads, blas = 1, "unknown"
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return threads, blas, cpu


def _oracle_work(n: int, a: float, b: int, hq: int) -> float:
    """Score elements the oracle computes for one sequence (every live row
    against every key it sees, for every query head)."""
    return float(hq) * float(np.sum(live_rows_fp32(n, a, b) + 1))


def cpu_baseline(wl, budget_s: float):
    """The float64 oracle, as it stands, on a bounded sample of the workload,
    timed on this host's cores, in the GPU's unit (sequence tokens per second;
    one sequence = one layer of one prompt).  Whole sequences (all KV heads,
    with select+compact) are taken in order until about ``budget_s`` seconds
    have run.  A sequence too large for the budget (e.g. every row live at
    N = 131072) is sampled instead: the oracle runs on its last rows only
    (``row_min``), sized to about ``budget_s``, and the rate is scaled by the
    share of the sequence's score elements those rows hold."""
    from oracle import waits_oracle as orc

    scale = float(np.float32(1 / math.sqrt(wl["d"])))
    hq, hkv, d = wl["hq"], wl["hkv"], wl["d"]
    rate_guess = 1e8   # oracle score elements per second on 16 cores (measured order)
    done_tokens, spent, used, sampled = 0.0, 0.0, 0, ""
    for i in range(len(wl["lengths"])):
        n, a, b = wl["lengths"][i], wl["a"][i], wl["b"][i]
        work = _oracle_work(n, a, b, hq)
        if used and (spent + work / rate_guess > 1.5 * budget_s):
            break
        bt = make_prompt(wl["seeds"][i], n, hq, hkv, d, heavy=True, dtype="bf16")
        if work / rate_guess <= 1.5 * budget_s:
            t0 = time.perf_counter()
            s = orc.waits_scores(bt.q, bt.k, bt.cu_seqlens, hq, hkv, [a], [b], scale)
            idx = orc.waits_select(s, bt.cu_seqlens, hkv, wl["budget"])
            orc.waits_compact(bt.k_bits, bt.v_bits, bt.cu_seqlens, idx)
            spent += time.perf_counter() - t0
            done_tokens += n
        else:
            # the last rows, about budget_s of work (each sees about n keys)
            rows = max(1, int(budget_s * rate_guess / (hq * n)))
            row_min = n - rows
            t0 = time.perf_counter()
            s = orc.waits_scores(bt.q, bt.k, bt.cu_seqlens, hq, hkv, [a], [b], scale,
                                 row_min=[row_min])
            idx = orc.waits_select(s, bt.cu_seqlens, hkv, wl["budget"])
            orc.waits_compact(bt.k_bits, bt.v_bits, bt.cu_seqlens, idx)
            dt = time.perf_counter() - t0
            w = orc.sigmoid_weights(n, a, b)
            live = np.nonzero(w != 0.0)[0]
            share = float(np.sum(live[live >= row_min] + 1)) / float(np.sum(live + 1))
            spent += dt / share
            done_tokens += n
            sampled = (f"; sequence {i} sampled on its last {rows} rows ({share:.2e} of its score "
                       f"elements, {dt:.1f} s), time scaled by 1/share")
        used += 1
        if spent >= budget_s:
            break
    threads, blas, cpu = _host_info()
    return {"value": done_tokens / spent, "unit": UNIT, "cores": threads, "kind": "oracle",
            "sample": f"first {used} of {len(wl['lengths'])} sequences of the workload "
                      f"({int(done_tokens)} tokens, all {hkv} KV heads), float64 numpy oracle "
                      f"incl. select+compact, {spent:.1f} s{sampled}; BLAS {blas}; "
                      f"{len(os.sched_getaffinity(0))} cpus in affinity; {cpu}"}


KERNEL_SOURCES = ("attention_score_eviction_amd/build.py",  # compile flags shape the kernels too
                  "attention_score_eviction_amd/csrc/few_rows.hpp",
                  "attention_score_eviction_amd/csrc/few_rows16.hpp",
                  "attention_score_eviction_amd/csrc/few_rows_multi.hpp",
                  "attention_score_eviction_amd/csrc/key_blocks.hpp",
                  "attention_score_eviction_amd/csrc/select_compact.hpp",
                  "attention_score_eviction_amd/csrc/device_common.hpp",
                  "attention_score_eviction_amd/csrc/kernel_args.hpp")

# Bench kernel names and a substring of the device symbol each launches (the
# timed kernel: few_rows_kernel, few_rows16_kernel or, for a batch mixing
# workgroup shapes, few_rows_multi_kernel; pass 1 may add the small combine
# kernel, which is not counted).
KERNEL_SYMBOLS = {"pass1_lse": ("few_rows", "false"),
                  "pass2_colsum": ("few_rows", "true"),
                  "select_compact": ("select_kernel", "true")}

# the same for the decode step (one kernel; the split merge is not counted)
DECODE_SOURCES = ("attention_score_eviction_amd/build.py",
                  "attention_score_eviction_amd/csrc/decode.hpp",
                  "attention_score_eviction_amd/csrc/decode_api.hip",
                  "attention_score_eviction_amd/csrc/device_common.hpp")
DECODE_SYMBOLS = {"decode": ("decode_kernel", None)}


def _traffic_spec(workload_name: str):
    """(kernel sources, bench kernel -> symbol match, description) of a workload's counter record."""
    if workload_name == "decode":
        return DECODE_SOURCES, DECODE_SYMBOLS, DECODE_WL["desc"]
    return KERNEL_SOURCES, KERNEL_SYMBOLS, workload(workload_name)["desc"]


def kernel_source_hash(workload_name: str = "8b") -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in _traffic_spec(workload_name)[0]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload_name: str):
    """HBM bytes per launch of ``kernel`` from the committed counter record
    (profiles/traffic_<workload>.json), or None when there is none or the
    kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash(workload_name):
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def copy_calibration(nbytes: int, reps: int = 3):
    """A plain device-to-device copy of a known size, for scaling the HBM
    byte counters (each launch reads and writes ``nbytes``)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def _counter_means(run_dir: str, counter: str):
    """Mean counter value per dispatch, by kernel symbol, from a rocprofv3
    --pmc csv run directory."""
    import csv
    import glob
    sums, counts = {}, {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                k = row["Kernel_Name"]
                sums[k] = sums.get(k, 0.0) + float(row["Counter_Value"])
                counts[k] = counts.get(k, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def _trace_means(run_dir: str):
    """Mean duration (ns) per kernel symbol from a rocprofv3 kernel-trace csv."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                out[row["Name"]] = float(row["AverageNs"])
    return out


def counters_from(prof_dir: str, workload_name: str, copy_bytes: int):
    """Write profiles/traffic_<workload>.json from rocprofv3 runs under
    prof_dir: fetch/ and write/ (FETCH_SIZE, WRITE_SIZE over bench.py),
    cfetch/ and cwrite/ (the same over --copy-calibration copy_bytes), trace/
    (kernel trace).  The counters, in KiB per dispatch, are scaled by what
    they read for the copy, whose bytes are known."""
    _, symbols, desc = _traffic_spec(workload_name)

    def pick(means, name):
        base, flag = symbols[name]
        hits = [k for k in means
                if base in k and (flag is None or f", {flag}," in k or f", {flag}>" in k)]
        return max(hits, key=lambda k: means[k]) if hits else None
    fetch = _counter_means(os.path.join(prof_dir, "fetch"), "FETCH_SIZE")
    write = _counter_means(os.path.join(prof_dir, "write"), "WRITE_SIZE")
    cfetch = max(_counter_means(os.path.join(prof_dir, "cfetch"), "FETCH_SIZE").values())
    cwrite = max(_counter_means(os.path.join(prof_dir, "cwrite"), "WRITE_SIZE").values())
    trace = _trace_means(os.path.join(prof_dir, "trace"))
    ff, wf = copy_bytes / (cfetch * 1024.0), copy_bytes / (cwrite * 1024.0)
    rec = {"workload": desc, "source_hash": kernel_source_hash(workload_name),
           "copy_calibration": {"bytes_read": copy_bytes, "bytes_written": copy_bytes,
                                "fetch_kib": cfetch, "write_kib": cwrite,
                                "fetch_factor": ff, "write_factor": wf},
           "kernels": {}}
    for name in symbols:
        sym = pick(fetch, name)
        if sym is None:
            continue
        rd = fetch[sym] * 1024.0 * ff
        wr = write.get(sym, 0.0) * 1024.0 * wf
        rec["kernels"][name] = {"symbol": sym, "fetch_kib_raw": fetch[sym],
                                "write_kib_raw": write.get(sym), "hbm_read_bytes": rd,
                                "hbm_write_bytes": wr, "hbm_bytes_per_launch": rd + wr,
                                "avg_duration_ns": trace.get(sym)}
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1), flush=True)


def step_buffers(wl, q, k, cu):
    """Device buffers of one step of a workload: lse, pass workspace, scores,
    kept positions, compacted K/V and the select workspace, allocated once."""
    import torch
    import attention_score_eviction_amd as W

    a, b, budget = wl["a"], wl["b"], wl["budget"]
    T, hq, hkv, d = int(cu[-1]), wl["hq"], wl["hkv"], wl["d"]
    B, dev = len(wl["lengths"]), q.device
    ws_bytes = max(W.waits.lse_workspace_bytes(q, k, cu, a, b),
                   W.waits.colsum_workspace_bytes(q, k, cu, a, b))
    kc = torch.empty((B, hkv, budget, d), dtype=torch.bfloat16, device=dev)
    return {"lse": torch.empty((hq, T), dtype=torch.float32, device=dev),
            "ws": torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev),
            "scores": torch.empty((hkv, T), dtype=torch.float32, device=dev),
            "idx": torch.empty((B, hkv, budget), dtype=torch.int32, device=dev),
            "kc": kc, "vc": torch.empty_like(kc),
            "sel_ws": torch.empty(max(W.waits.select_workspace_bytes(cu, hkv, budget), 256),
                                  dtype=torch.uint8, device=dev)}


def step_calls(wl, q, k, v, cu, bf):
    """The three library calls of one step (pass 1, pass 2, select+compact)."""
    import attention_score_eviction_amd as W

    a, b, budget = wl["a"], wl["b"], wl["budget"]
    return [
        lambda: W.lse(q, k, cu, a, b, out=bf["lse"], workspace=bf["ws"]),
        lambda: W.colsum(q, k, bf["lse"], cu, a, b, out=bf["scores"], workspace=bf["ws"]),
        lambda: W.select_compact(bf["scores"], k, v, cu, budget, idx=bf["idx"], k_out=bf["kc"],
                                 v_out=bf["vc"], workspace=bf["sel_ws"]),
    ]


def stage_runners(fns, graph: bool):
    """One callable per stage of a step: the library calls themselves, or,
    with ``graph``, the replay of a HIP graph (torch.cuda.CUDAGraph) captured
    once from them; every replay launches all of the stage's kernels on the
    current stream, with the host-side planning done once at capture."""
    if not graph:
        return list(fns)
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for f in fns:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f()
        graphs.append(g)
    torch.cuda.synchronize()
    return [g.replay for g in graphs]


@contextlib.contextmanager
def no_gc():
    """Python's cyclic collector off for the timed region (collected once
    before it): a full collection of torch's object graph takes 30-40 ms on
    the host, and the GPU drains its queue and idles while one runs."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def launch_mode(args) -> str:
    return "one HIP graph replay per stage" if args.graph else "direct library calls"


DECODE_WL = dict(desc="decode over the compacted cache: 64 sequences, Llama-3.1-8B shape "
                      "(32/8/128), 2048 kept rows per KV head, one new token each",
                 batch=64, hq=32, hkv=8, d=128, cap=2048, seed=4242)


def decode_bench(args):
    """One decoding step's attention for a batch over its compacted cache:
    value = new tokens per second (one per sequence), roofline against HBM
    (K and V rows read once, plus q, out and lse)."""
    import torch
    import attention_score_eviction_amd as W
    from oracle import decode_oracle as dec

    wl = DECODE_WL
    bsz, hq, hkv, d, cap = wl["batch"], wl["hq"], wl["hkv"], wl["d"], wl["cap"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    x = make_decode(wl["seed"], bsz, hq, hkv, cap, d, "bf16")
    t_gen = time.perf_counter() - t_gen
    q, k, v = (torch.from_numpy(b).view(torch.bfloat16).to(dev) for b in (x.q_bits, x.k_bits, x.v_bits))
    lens = torch.full((bsz,), cap, dtype=torch.int32, device=dev)
    out = torch.empty((bsz, hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((bsz, hq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(W.waits.decode_workspace_bytes(q, k), 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    (run,) = stage_runners([lambda: W.decode(q, k, v, lens, out=out, lse=lse, workspace=ws)], args.graph)
    with no_gc():
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            run()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_kernel = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    nbytes = 2 * bsz * hkv * cap * d * 2 + bsz * hq * d * 2 + bsz * hq * (d + 1) * 4
    roof = {"bound": "hbm", "kernel": "decode", "achieved": nbytes / (ms_kernel * 1e-3) / 1e9,
            "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic("decode", "decode")
    res = {
        "metric": "decode tokens/s over the compacted cache (one new token per sequence, one layer)",
        "value": bsz / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl["desc"], "sequences": bsz, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": d, "cache_rows": cap, "parallelism": "single GPU",
                   "launch": launch_mode(args)},
        "roofline": roof, "kernels_us": {"decode": ms_kernel * 1e3},
        "algorithmic": {"bytes_per_step": nbytes}, "input_gen_s": t_gen, "host": platform.node(),
    }
    if not args.no_cpu_baseline:
        scale = float(np.float32(1 / math.sqrt(d)))
        done, spent = 0, 0.0
        lens_h = [cap] * bsz
        while spent < min(args.cpu_budget_s, 10.0) and done < bsz:
            t1 = time.perf_counter()
            dec.waits_decode(x.q[done:done + 1], x.k[done:done + 1], x.v[done:done + 1],
                             lens_h[done:done + 1], scale)
            spent += time.perf_counter() - t1
            done += 1
        threads, blas, cpu = _host_info()
        res["cpu_baseline"] = {"value": done / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"first {done} of {bsz} sequences, float64 numpy decode oracle, "
                                         f"{spent:.1f} s; BLAS {blas}; {cpu}"}
    print(json.dumps(res), flush=True)


def fused_bench(args):
    """Headline batch through the attention forward (out + lse), then pass 2
    and select+compact.  value = layer tokens per second of the whole step."""
    import torch
    import attention_score_eviction_amd as W

    wl = workload("8b")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    q, k, v, cu = make_inputs(wl, dev)
    t_gen = time.perf_counter() - t_gen
    a, b, budget = wl["a"], wl["b"], wl["budget"]
    T, hq, hkv, d = int(cu[-1]), wl["hq"], wl["hkv"], wl["d"]
    B = len(wl["lengths"])
    out = torch.empty_like(q)
    lse = torch.empty((hq, T), dtype=torch.float32, device=dev)
    lse1 = torch.empty_like(lse)
    ws = torch.empty(max(W.waits.lse_workspace_bytes(q, k, cu, a, b),
                         W.waits.colsum_workspace_bytes(q, k, cu, a, b), 256), dtype=torch.uint8, device=dev)
    scores = torch.empty((hkv, T), dtype=torch.float32, device=dev)
    idx = torch.empty((B, hkv, budget), dtype=torch.int32, device=dev)
    kc = torch.empty((B, hkv, budget, d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    sel_ws = torch.empty(max(W.waits.select_workspace_bytes(cu, hkv, budget), 256), dtype=torch.uint8,
                         device=dev)
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]

    runs = stage_runners([
        lambda: W.attention(q, k, v, cu, out=out, lse=lse),
        lambda: W.colsum(q, k, lse, cu, a, b, out=scores, workspace=ws),
        lambda: W.select_compact(scores, k, v, cu, budget, idx=idx, k_out=kc, v_out=vc, workspace=sel_ws),
    ], args.graph)

    def step(e=None):
        for j, run in enumerate(runs):
            if e: e[j].record(stream)
            run()
        if e: e[len(runs)].record(stream)

    with no_gc():
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(ev[i])
        torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    names = ["attention", "pass2_colsum", "select_compact"]
    per = {nm: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
           for j, nm in enumerate(names)}
    # pass 1 on its own, for the saving the fusion brings (not part of the step)
    p1 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    with no_gc():
        W.lse(q, k, cu, a, b, out=lse1, workspace=ws)
        p1[0].record(stream)
        for _ in range(3):
            W.lse(q, k, cu, a, b, out=lse1, workspace=ws)
        p1[1].record(stream)
        torch.cuda.synchronize()
    pass1_ms = p1[0].elapsed_time(p1[1]) / 3
    n = wl["lengths"][0]
    att_flops = 4.0 * d * hq * (n * (n + 1) / 2) * B          # QK^T and PV over the causal triangle
    flops_pass, _, sel_bytes, cmp_bytes = algorithmic_work(wl)
    roof = {"bound": "mfma", "kernel": "attention",
            "achieved": att_flops / (per["attention"] * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    res = {
        "metric": "prompt tokens/s per layer for attention forward + WAITS pass 2 + select+compact",
        "value": float(sum(wl["lengths"])) / (ms_step * 1e-3), "unit": UNIT, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl["desc"] + ", with the prefill attention forward supplying lse",
                   "sequences": B, "tokens_per_step": T, "q_heads": hq, "kv_heads": hkv, "head_dim": d,
                   "select_budget": budget, "parallelism": "single GPU", "launch": launch_mode(args)},
        "roofline": roof,
        "kernels_us": {nm: per[nm] * 1e3 for nm in names},
        "waits_marginal_us": (per["pass2_colsum"] + per["select_compact"]) * 1e3,
        "pass1_saved_us": pass1_ms * 1e3,
        "algorithmic": {"attention_flops": att_flops, "pass2_flops": flops_pass,
                        "select_compact_bytes": sel_bytes + cmp_bytes},
        "input_gen_s": t_gen, "host": platform.node(),
    }
    print(json.dumps(res), flush=True)


UBENCH_MODES = ["mfma: 8 MFMA 16x16x32 bf16", "triple: 8 (fma, exp, add)", "exp: 8 v_exp_f32",
                "fma: 8 v_fma_f32", "add: 8 v_add_f32", "mixed: 8 MFMA + 8 triples, compiler's interleave",
                "clusters: 8 MFMA then 8 triples", "clusters, MFMA at raised wave priority",
                "split: waves 0-3 8 MFMA, waves 4-7 8 triples",
                "split: waves 0-3 8 MFMA, waves 4-7 8 fma", "split: waves 0-3 8 MFMA, waves 4-7 8 exp"]
UBENCH_WAVES = [(512, 4), (768, 4), (768, 3), (1024, 3), (1024, 2)]  # (threads, row tiles per wave)
UBENCH_OPERANDS = ["MFMAs only, all in VGPRs", "MFMAs + epilogue, all in VGPRs",
                   "MFMAs only, multiplicands in AGPRs", "MFMAs + epilogue, multiplicands in AGPRs",
                   "epilogue only, accumulators in AGPRs", "MFMAs + epilogue, accumulators in AGPRs"]
UBENCH_SELECT = ["start to first barrier (loads issued, LDS cleared)", "pass 1 (top byte, waits for the scores)",
                 "pass 2", "pass 3 (and the L2 requests)", "pass 4", "totals", "output placed", "gather",
                 "total"]
UBENCH_TILE = ["MFMAs only", "epilogue only", "one cluster, MFMAs at raised priority",
               "groups of 32 MFMAs", "groups of 16", "groups of 8", "groups of 4", "groups of 2",
               "groups of 1"]


def ubench(args):
    """Instruction-mix microbenchmarks of the QK^T passes (libwaits_ubench.so):
    cycles per loop iteration of the slowest wave of each half of the
    workgroup's waves, per mode, at one and two waves per SIMD."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "attention_score_eviction_amd", "libwaits_ubench.so"))
    n = lib.waits_ubench_modes()
    assert n == len(UBENCH_MODES)
    for threads in (256, 512):
        res = (ctypes.c_double * (3 * n))()
        simd = (ctypes.c_int * 16)()
        rc = lib.waits_ubench_mix(threads, 256, 4000, res, simd)
        if rc:
            raise SystemExit(f"waits_ubench_mix failed ({rc})")
        print(json.dumps({"ubench": "instruction mix", "threads": threads, "workgroups": 256,
                          "waves_per_simd": threads // 256,
                          "simd_of_wave": list(simd[:threads // 64]),
                          "cycles_per_iteration": {m: {"waves_first_half": round(res[3 * i], 1),
                                                       "waves_second_half": round(res[3 * i + 1], 1),
                                                       "clock_ghz": round(res[3 * i + 2], 3)}
                                                   for i, m in enumerate(UBENCH_MODES)}}), flush=True)
    # the passes' own shape: 32 MFMAs and a 32-element epilogue per wave and iteration
    for threads in (256, 512):
        res = (ctypes.c_double * (2 * len(UBENCH_TILE)))()
        rc = lib.waits_ubench_tile(threads, 256, 4000, res)
        if rc:
            raise SystemExit(f"waits_ubench_tile failed ({rc})")
        print(json.dumps({"ubench": "pass shape (32 MFMA + 32 epilogue elements per wave)",
                          "threads": threads, "workgroups": 256, "waves_per_simd": threads // 256,
                          "cycles_per_iteration": {m: {"slowest_wave": round(res[2 * i], 1),
                                                       "clock_ghz": round(res[2 * i + 1], 3)}
                                                   for i, m in enumerate(UBENCH_TILE)}}), flush=True)
    # the headline's select+compact with its phases stamped
    res = (ctypes.c_double * 10)()
    rc = lib.waits_ubench_select(32, 16384, 128, res)
    if rc:
        raise SystemExit(f"waits_ubench_select failed ({rc})")
    print(json.dumps({"ubench": "select_kernel<16, true> phases (32 sequences x 8 KV heads x 16384 keys, "
                                "budget 128, head_dim 128)",
                      "median_cycles_per_workgroup": {nm: round(res[i], 0) for i, nm in enumerate(UBENCH_SELECT)},
                      "us_per_launch": round(res[9], 2)}), flush=True)
    # the kernels' one-cluster order at two to four waves per SIMD
    res = (ctypes.c_double * (2 * len(UBENCH_WAVES)))()
    rc = lib.waits_ubench_tile_waves(256, 4000, res)
    if rc:
        raise SystemExit(f"waits_ubench_tile_waves failed ({rc})")
    print(json.dumps({"ubench": "pass shape, one cluster at raised priority, by waves per SIMD",
                      "workgroups": 256,
                      "simd_cycles_per_mfma": {f"{t} threads ({t // 256} waves/SIMD), {nt} row tiles": {
                          "cycles": round(res[2 * i] / (t // 256 * 8 * nt), 2),
                          "clock_ghz": round(res[2 * i + 1], 3)}
                          for i, (t, nt) in enumerate(UBENCH_WAVES)}}), flush=True)
    # where the MFMA operands and accumulators live (two waves per SIMD)
    res = (ctypes.c_double * (2 * len(UBENCH_OPERANDS)))()
    rc = lib.waits_ubench_operands(256, 4000, res)
    if rc:
        raise SystemExit(f"waits_ubench_operands failed ({rc})")
    print(json.dumps({"ubench": "pass shape, one cluster at raised priority, by operand placement "
                                "(512 threads, 2 waves/SIMD, 4 row tiles)", "workgroups": 256,
                      "cycles_per_iteration": {m: {"slowest_wave": round(res[2 * i], 1),
                                                   "clock_ghz": round(res[2 * i + 1], 3)}
                                               for i, m in enumerate(UBENCH_OPERANDS)}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the clock ramps up over the first ~20 ms of sustained load (about 20
    # headline steps, 1.26 -> 1.01 ms), so the timed steps start after that
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="8b",
                    choices=WORKLOADS)
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each stage from a captured HIP graph instead of calling the library")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES (counter calibration) and exit")
    ap.add_argument("--ubench", action="store_true",
                    help="only run the instruction-mix microbenchmarks (libwaits_ubench.so) and exit")
    ap.add_argument("--counters-from", metavar="DIR",
                    help="only write profiles/traffic_<workload>.json from rocprofv3 runs in DIR "
                         "(fetch/, write/, cfetch/, cwrite/, trace/) and exit; no GPU needed")
    args = ap.parse_args()
    if args.ubench:
        ubench(args)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.counters_from:
        counters_from(args.counters_from, args.workload, 1 << 30)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the WAITS path needs no collectives and this "
              "build runs on a single MI355X; multi-GPU sharding is design-only.",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "decode":
        decode_bench(args)
        return
    if args.workload == "fused":
        fused_bench(args)
        return

    import torch
    import attention_score_eviction_amd as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workload(args.workload)
    t_gen = time.perf_counter()
    q, k, v, cu = make_inputs(wl, dev)
    t_gen = time.perf_counter() - t_gen
    a, b, budget = wl["a"], wl["b"], wl["budget"]
    T, hq, hkv, d = int(cu[-1]), wl["hq"], wl["hkv"], wl["d"]
    B = len(wl["lengths"])

    bufs = step_buffers(wl, q, k, cu)
    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    runs = stage_runners(step_calls(wl, q, k, v, cu, bufs), args.graph)

    def step(e=None):
        for j, run in enumerate(runs):
            if e: e[j].record(stream)
            run()
        if e: e[len(runs)].record(stream)

    with no_gc():
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(ev[i])
        torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    names = ["pass1_lse", "pass2_colsum", "select_compact"]
    per = {nm: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
           for j, nm in enumerate(names)}  # ms per launch (pass 1 includes its combine, if any)

    flops_pass, bytes_pass, sel_bytes, cmp_bytes = algorithmic_work(wl)
    tokens_layers = float(sum(wl["lengths"]))  # every sequence is one layer of one prompt
    value = tokens_layers / (ms_step * 1e-3)

    frac = {
        "pass1_lse": flops_pass / (per["pass1_lse"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "pass2_colsum": flops_pass / (per["pass2_colsum"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "select_compact": (sel_bytes + cmp_bytes) / (per["select_compact"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    dom = max(("pass1_lse", "pass2_colsum"), key=lambda nm: per[nm])
    # the passes are MFMA-bound above the ridge (peak flops / peak bytes), HBM-bound below
    mfma_bound = flops_pass / bytes_pass >= PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "kernel": dom,
                "achieved": flops_pass / (per[dom] * 1e-3) / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "kernel": dom,
                "achieved": bytes_pass / (per[dom] * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom, args.workload)
    passes_ms = per["pass1_lse"] + per["pass2_colsum"]
    sc_ms = per["select_compact"]

    out = {
        "metric": METRIC,
        "value": value,
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl["desc"], "sequences": B, "tokens_per_step": T,
                   "q_heads": hq, "kv_heads": hkv, "head_dim": d, "select_budget": budget,
                   "parallelism": "single GPU", "launch": launch_mode(args)},
        "roofline": roof,
        "passes_mfma_frac": 2 * flops_pass / (passes_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "select_compact_hbm_frac": (sel_bytes + cmp_bytes) / (sc_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "kernels_us": {nm: per[nm] * 1e3 for nm in names},
        "kernel_frac": frac,
        "algorithmic": {"flops_per_pass": flops_pass, "bytes_per_pass": bytes_pass,
                        "select_bytes": sel_bytes,
                        "compact_bytes": cmp_bytes},
        "input_gen_s": t_gen,
        "host": platform.node(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
