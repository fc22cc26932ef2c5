"""Helpers for the GPU parity tests: move synthetic batches to the device and
compare the HIP path with the oracle to the acceptance bar.

Bar (scores fp32 vs the float64 oracle):
  * per key, |s_gpu - s_ref| <= 2e-3 * s_ref;
  * selection: the GPU's kept set equals the oracle's, except keys whose
    oracle score lies within 2e-3 (relative) of the oracle's budget-th largest
    score; in addition the GPU's kept positions must be *exactly* the top-k of
    the GPU's own scores (ties to the lower position, ascending, -1 padded) --
    that selection is unique, so it is compared bit for bit;
  * compaction: bit-exact against host fancy-indexing with the GPU's indices.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import waits_oracle as orc

DEV = "cuda:0"
SCORE_RTOL = 2e-3


def to_device(bt):
    """(q, k, v) device tensors carrying exactly the batch's input values."""
    if bt.dtype == "bf16":
        conv = lambda x: torch.from_numpy(x).view(torch.bfloat16).to(DEV)  # noqa: E731
        return conv(bt.q_bits), conv(bt.k_bits), conv(bt.v_bits)
    return (torch.from_numpy(bt.q).to(DEV), torch.from_numpy(bt.k).to(DEV),
            torch.from_numpy(bt.v).to(DEV))


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> its raw bits as a numpy array (uint16 for bf16)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def check_scores(s_gpu: np.ndarray, s_ref: np.ndarray, mask=None, rtol=SCORE_RTOL):
    s_gpu = np.asarray(s_gpu, dtype=np.float64)
    if mask is not None:
        s_gpu, s_ref = s_gpu[mask], s_ref[mask]
    assert np.all(np.isfinite(s_gpu))
    assert np.all(s_ref > 0), "oracle scores are positive when b >= 1"
    rel = np.abs(s_gpu - s_ref) / s_ref
    worst = int(np.argmax(rel))
    assert rel.max() <= rtol, (
        f"max rel err {rel.max():.3e} at {worst}: gpu {s_gpu.flat[worst]!r} ref {s_ref.flat[worst]!r}")
    return float(rel.max())


def check_select_exact(idx_gpu: np.ndarray, s_gpu: np.ndarray, cu, budget: int):
    """GPU idx == top-k of the GPU's own scores (unique selection)."""
    nb, hkv, _ = idx_gpu.shape
    for p in range(nb):
        lo, hi = int(cu[p]), int(cu[p + 1])
        for h in range(hkv):
            want = orc.select_topk(np.asarray(s_gpu[h, lo:hi], dtype=np.float64), budget)
            np.testing.assert_array_equal(idx_gpu[p, h], want, err_msg=f"seq {p} head {h}")


def check_select_vs_oracle(idx_gpu: np.ndarray, s_ref: np.ndarray, cu, budget: int,
                           rtol=SCORE_RTOL):
    """Kept sets agree with the oracle's except within rtol of its boundary."""
    nb, hkv, _ = idx_gpu.shape
    for p in range(nb):
        lo, hi = int(cu[p]), int(cu[p + 1])
        n = hi - lo
        for h in range(hkv):
            ref = orc.select_topk(s_ref[h, lo:hi], budget)
            keep = min(budget, n)
            got_set = set(idx_gpu[p, h, :keep].tolist())
            ref_set = set(ref[:keep].tolist())
            assert np.all(idx_gpu[p, h, keep:] == -1)
            if keep == 0:
                continue
            t = np.sort(s_ref[h, lo:hi])[::-1][keep - 1]
            for key in got_set ^ ref_set:
                assert abs(s_ref[h, lo + key] - t) <= rtol * t, (
                    f"seq {p} head {h}: key {key} score {s_ref[h, lo + key]} boundary {t}")


def _raw(x: np.ndarray) -> np.ndarray:
    return x.view(np.uint32) if x.dtype == np.float32 else x


def check_compact(kc, vc, k_src, v_src, idx_gpu, cu):
    """k_src / v_src: the host inputs (bf16 bit patterns or float32 values)."""
    kr, vr = orc.waits_compact(k_src, v_src, cu, idx_gpu)
    np.testing.assert_array_equal(_raw(host_bits(kc)), _raw(kr))
    np.testing.assert_array_equal(_raw(host_bits(vc)), _raw(vr))
